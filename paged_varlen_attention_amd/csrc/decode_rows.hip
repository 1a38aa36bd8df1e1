// decode_rows.hip -- paged GQA decode attention for gfx950 that streams whole
// cache rows: one workgroup per (request, partition) serves every KV head, so
// each DMA instruction reads 1 KB of consecutive bytes of a page and the
// heads of a token are fetched together.
//
// What it computes is the same as the other decode kernels (vllm-metal kernel
// walkthrough, "What is Paged Attention"; GQA decode tips 1-4): softmax(q.k *
// scale) v over one request's keys read page by page through its block table,
// all query heads of a GQA group served from one read of each K/V row, the
// softmax online in log2 space, and the key range optionally cut into
// partitions whose (max, exp-sum) statistics and normalised partial outputs
// the reduce kernel merges.
//
// Why whole rows: a cache row of a token holds all KV heads (Hkv x D
// elements).  A workgroup per KV head reads one head's 2D-byte slice of every
// row, so HBM sees short strided pieces of each page; reading the row whole
// lets the memory system move each page as one contiguous run.  On the GQA
// decode batch (random 32 KB pages) a DMA-only skeleton of this order moves
// the batch at about 5.6 TB/s against about 5.0 TB/s for per-head slices.
//
// The design is our own for CDNA4:
//  * grid = (requests, partitions), partitions last-first, so consecutive
//    workgroups (different XCDs) take different requests; NW waves take the
//    chunks of the partition round-robin, each with a private ring of NST LDS
//    stages refilled as soon as the chunk's fragments are in registers;
//  * a chunk is KPB consecutive keys of one page, whole rows of K and of V;
//  * the heads are served in MFMA blocks of HPB heads: S^T of a block is a
//    16x16 product whose 16 rows are (head, key) pairs (HPB heads x KPB keys)
//    and whose 16 columns are the HPB groups' query heads (HPB x group <= 16);
//    only the entries whose row head is the column's head are scores, the
//    others are set to -inf, so P^T is zero there and O^T = V^T P^T of the
//    same block adds each head's values to its own queries only;
//  * LDS row layout: the 16-byte pieces of row (t, head) are XORed with
//    sigma(i) = (2i mod 16) | (i / 8), i = (head mod HPB) KPB + t its row in
//    the block.  sigma is a bijection on 0..15, so the 16 lanes of a K
//    fragment read (one piece of 16 block rows) reach 16 distinct 16-byte
//    slots, and it maps rows 0..7 (and 8..15) to distinct halves sigma/2, so
//    the 32 lanes of a V^T transpose read (pieces 2b and 2b+1 of 8 rows)
//    cover all banks (counted: no conflicts; the K reads still show about one
//    extra cycle each, which does not limit this memory-bound kernel);
//  * the waves' states meet in LDS in the accumulator layout: every wave
//    holds the same (head, dim) at the same lane and register, so each lane
//    merges one float4 position of all waves (its own from registers) and
//    stores 4 consecutive dims; the states are parked in the waves' own rings
//    and the queries sit in per-wave areas, so the kernel has one barrier
//    (one workgroup per CU leaves no other workgroup to hide the start-up and
//    the epilogue, so both are kept short).
#include <cstdlib>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr float ROWS_RESCALE_THRESHOLD = 8.0f;  // log2 units

template <int D, int HPB, int NB, int NW>
struct RowCfg {
    static constexpr int KPB = 16 / HPB;   // keys per chunk = rows of a block per head
    static constexpr int HB = HPB * NB;    // KV heads served (all heads of a cache row)
    static constexpr int R = 2 * D;        // bytes of one head's K (or V) row
    static constexpr int RB = HB * R;      // bytes of a cache row
    static constexpr int TILE = KPB * RB;  // K (or V) bytes of a chunk
    static constexpr int NI = TILE / 1024; // 1 KB DMA instructions per tile
    static constexpr int VM = 2 * NI;      // per chunk: K and V
    static constexpr int NST = 2 * VM < 64 ? 2 : 1;
    static constexpr int SLOT = 2 * TILE;
    static constexpr int KS = D / 32;      // k-steps of S^T (16x16x32)
    static constexpr int DB = D / 16;      // 16-row blocks of O^T
    static constexpr int QHMAX = 16 * NB;  // most query heads (HPB x group <= 16 per block)
    static constexpr int RING = NW * NST * SLOT;
    static constexpr int QBYTES = QHMAX * 2 * D;
    static constexpr int LDS_BYTES = RING + NW * QBYTES;  // a query area per wave
    // a wave's state (O^T accumulators, max and exp-sum per column) fits its ring
    static_assert(NB * DB * 1024 + 2 * NB * 16 * 4 <= NST * SLOT, "state in the ring");
    static_assert(KPB >= 2 && KPB <= 8 && NB >= 1 && NB <= 2, "block shape");
    static_assert(D >= 128, "pieces per head row >= 16 (the swizzle XORs 4 bits)");
    static_assert(TILE % 1024 == 0 && VM < 64, "DMA shape");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int sigma(int i) { return ((2 * i) & 15) | (i >> 3); }

template <int D, int HPB, int NB, int NW>
__global__ __launch_bounds__(NW * 64) void decode_rows_kernel(const AttnParams p) {
    using C = RowCfg<D, HPB, NB, NW>;
    constexpr int KPB = C::KPB;
    constexpr int NST = C::NST;
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];

    const int r = blockIdx.x;
    const int part = gridDim.y - 1 - blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;  // MFMA column: query head `col` of a block
    const int grp = lane >> 4;  // lane group: block rows 4 grp .. 4 grp + 3
    const int tok_begin = p.partition ? part * p.partition : 0;
    const int bs = p.block_size;
    const int lbs = p.log2_bs;
    const int c_begin = tok_begin / KPB;

    // Block-table window: lane i holds the page of the wave's chunk kw0 + i
    // (a chunk never spans two pages: KPB divides the page size).
    const int32_t *bt_row = p.bt + (size_t)r * p.bt_stride;
    auto load_window = [&](int kw0) -> int {
        const int ch = c_begin + wave + (kw0 + lane) * NW;
        const int lp = (ch * KPB) >> lbs;
        const int v = lp < p.bt_stride ? bt_row[lp] : 0;
        return v < 0 ? 0 : (v >= p.num_blocks ? p.num_blocks - 1 : v);
    };
    int win_base = 0;
    int btv = load_window(0);

    const int q0 = p.cu_q[r];
    const int q1 = p.cu_q[r + 1];
    const int seq_len = p.seq_lens[r];
    if (q1 - q0 <= 0) return;
    if (tok_begin >= seq_len || seq_len <= 0) return;
    const int tok_end = p.partition ? min(seq_len, tok_begin + p.partition) : seq_len;
    const int nparts = p.partition ? (seq_len + p.partition - 1) / p.partition : 1;
    const int G = p.group;
    const int QH = C::HB * G;  // query heads of the request (= Hq)
    const int c_end = (tok_end + KPB - 1) / KPB;
    const int nchunks = c_end - c_begin;
    const int nmy = nchunks > wave ? (nchunks - wave + NW - 1) / NW : 0;

    const char *kc = reinterpret_cast<const char *>(p.kc);
    const int64_t v_minus_k = reinterpret_cast<const char *>(p.vc) - kc;
    const uint64_t page_bytes = (uint64_t)bs * C::RB;

    // DMA lane offsets: instruction n fills tile bytes 1024 n + 16 lane, i.e.
    // slot s of head h of row t; it fetches piece s ^ sigma(i) of that row.
    uint32_t voff[C::NI];
#pragma unroll
    for (int n = 0; n < C::NI; ++n) {
        const int pos = n * 1024 + lane * 16;
        const int t = pos / C::RB;
        const int h = (pos % C::RB) / C::R;
        const int s = (pos % C::R) / 16;
        const int i = (h % HPB) * KPB + t;
        voff[n] = (uint32_t)(t * C::RB + h * C::R + ((s ^ sigma(i)) << 4));
    }
    const uint32_t lds_wave = lds_addr(lds) + (uint32_t)(wave * NST * C::SLOT);

    auto issue = [&](int k, int s) {
        if (k - win_base >= 64) {  // slide the window (long unsplit ranges only)
            win_base = k;
            btv = load_window(k);
        }
        const int tok0 = (c_begin + wave + k * NW) * KPB;
        const int phys = __builtin_amdgcn_readlane(btv, k - win_base);
        const uint64_t off = (uint64_t)phys * page_bytes + (uint64_t)(tok0 & (bs - 1)) * C::RB;
        const uint32_t ldsk = lds_wave + (uint32_t)(s * C::SLOT);
#pragma unroll
        for (int n = 0; n < C::NI; ++n) dma_lds<16>(kc + off, voff[n], ldsk + n * 1024);
#pragma unroll
        for (int n = 0; n < C::NI; ++n)
            dma_lds<16>(kc + off + v_minus_k, voff[n], ldsk + C::TILE + n * 1024);
    };

    // Chunk 0, then the request's query rows (all heads, QH x 2D contiguous
    // bytes) into this wave's own query area, then the other ring stage; the
    // wave reads its Q^T once its own DMA has landed (no barrier: the waves
    // start their streams independently).
    const int q_area = C::RING + wave * C::QBYTES;
    if (nmy > 0) issue(0, 0);
    {
        const char *qg = reinterpret_cast<const char *>(p.q) + (size_t)q0 * p.hq * (2 * D);
        const int qbytes = QH * 2 * D;
        for (int j = 0; j * 1024 < qbytes; ++j) {
            const uint32_t off = (uint32_t)(j * 1024 + lane * 16);
            dma_lds<16>(qg, off < (uint32_t)qbytes ? off : 0u, lds_addr(lds) + q_area + j * 1024);
        }
    }
    if (NST > 1 && nmy > 1) issue(1, 1);
    if (NST > 1 && nmy > 1)
        wait_vmcnt<C::VM>();
    else
        wait_vmcnt<0>();

    // Q^T of block X (B operand of S^T): column `col` is query head
    // X HPB G + col (zero past the block's HPB G heads), dims 32 ks + 8 grp ..
    bf16x8_t qb[NB][C::KS];
    const int ncol = HPB * G;
#pragma unroll
    for (int X = 0; X < NB; ++X) {
        const char *qrow = lds + q_area + (X * ncol + col) * (2 * D) + 16 * grp;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            if (col < ncol) {
                qb[X][ks] = *reinterpret_cast<const bf16x8_t *>(qrow + 64 * ks);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) qb[X][ks][e] = (__bf16)0.f;
            }
        }
    }

    // Scores of block row 4 grp + e are kept only where its head is the
    // column's head (unused columns join head 0: zero queries, finite scores).
    const int col_head = col < ncol ? col / G : 0;
    uint32_t keep = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if ((4 * grp + e) / KPB == col_head) keep |= 1u << e;

    // Fragment addresses inside a stage.  K (S^T A operand): block row `col`
    // = (head col / KPB, key col % KPB), pieces 4 ks + grp.  V^T (O^T A
    // operand, transpose read): row 4 grp + col / 4, pieces 2 b + (col % 4) / 2,
    // 8-byte half col % 2.
    const int ki = col;
    const int ksg = sigma(ki);
    const int k_row = (ki % KPB) * C::RB + (ki / KPB) * C::R;
    const int vi = 4 * grp + (col >> 2);
    const int vsg = sigma(vi);
    const int v_row = (vi % KPB) * C::RB + (vi / KPB) * C::R + (col & 1) * 8;
    const int vlo = ((col & 3) >> 1) ^ (vsg & 1);

    struct Frags {
        bf16x8_t k[NB][C::KS];
        s16x4_t v[NB][C::DB];
    };
    auto read = [&](const char *st, Frags &f) {
#pragma unroll
        for (int X = 0; X < NB; ++X) {
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int pc = (((ks ^ (ksg >> 2)) << 2) | (grp ^ (ksg & 3)));
                f.k[X][ks] = *reinterpret_cast<const bf16x8_t *>(st + X * HPB * C::R + k_row +
                                                                 (pc << 4));
            }
#pragma unroll
            for (int b = 0; b < C::DB; ++b) {
                const int pc = (((b ^ (vsg >> 1)) << 1) | vlo);
                f.v[X][b] = lds_read_tr16(st + C::TILE + X * HPB * C::R + v_row + (pc << 4));
            }
        }
    };

    float m[NB], mtrue[NB], l[NB];
    f32x4_t o[NB][C::DB];
#pragma unroll
    for (int X = 0; X < NB; ++X) {
        m[X] = NEG_INF;
        mtrue[X] = NEG_INF;
        l[X] = 0.f;
#pragma unroll
        for (int b = 0; b < C::DB; ++b) o[X][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float scale_log2 = p.scale_log2;

    // One chunk: per block S^T, online softmax, O^T.  MASKED is the chunk
    // holding the end of the key range (keys from tok_end on get -inf and
    // their V entries, possibly NaN page tails, are replaced by zeros).
    auto chunk = [&](Frags &f, auto masked, int key0) {
        constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
        for (int X = 0; X < NB; ++X) {
            f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C::KS; ks += 2) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k[X][ks], qb[X][ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k[X][ks + 1], qb[X][ks + 1], s1, 0,
                                                             0, 0);
            }
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = (keep >> e) & 1 ? (s0[e] + s1[e]) * scale_log2 : NEG_INF;
                if (MASKED && key0 + (4 * grp + e) % KPB >= tok_end) x[e] = NEG_INF;
            }
            const float cm = rows_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
            mtrue[X] = fmaxf(mtrue[X], cm);
            if constexpr (!MASKED) {
                const bool up = cm > m[X] + ROWS_RESCALE_THRESHOLD;
                if (__builtin_amdgcn_ballot_w64(up)) {
                    const float mn = up ? cm : m[X];
                    const float alpha = exp2_diff(m[X], mn);  // m = -inf before the first key
                    m[X] = mn;
                    l[X] *= alpha;
#pragma unroll
                    for (int b = 0; b < C::DB; ++b)
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[X][b][e] *= alpha;
                }
            } else {
                const float mn = fmaxf(m[X], cm);
                const float alpha = exp2_diff(m[X], mn);
                m[X] = mn;
                l[X] *= alpha;
#pragma unroll
                for (int b = 0; b < C::DB; ++b)
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[X][b][e] *= alpha;
            }
            float pr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // m is finite once a chunk has been seen (every column keeps a row)
                pr[e] = MASKED ? exp2_diff(x[e], m[X]) : __builtin_amdgcn_exp2f(x[e] - m[X]);
                l[X] += pr[e];
            }
            const uint2 pw = make_uint2(pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]));
            const s16x4_t pb = __builtin_bit_cast(s16x4_t, pw);
#pragma unroll
            for (int b = 0; b < C::DB; ++b) {
                s16x4_t a = f.v[X][b];
                if constexpr (MASKED) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (key0 + (4 * grp + e) % KPB >= tok_end) a[e] = 0;
                }
                o[X][b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[X][b], 0, 0, 0);
            }
        }
    };

    // Land chunk k, read its fragments, refill its stage with chunk k + NST.
    auto stage = [&](int k, Frags &f) {
        if (NST > 1 && k + 1 < nmy)
            wait_vmcnt<C::VM>();
        else
            wait_vmcnt<0>();
        read(lds + (wave * NST + k % NST) * C::SLOT, f);
        if (k + NST < nmy) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage k is read
            issue(k + NST, k % NST);
        }
    };
    for (int k = 0; k < nmy - 1; ++k) {
        Frags f;
        stage(k, f);
        chunk(f, std::false_type{}, 0);
    }
    if (nmy > 0) {
        Frags f;
        stage(nmy - 1, f);
        chunk(f, std::true_type{}, (c_begin + wave + (nmy - 1) * NW) * KPB);
    }

    // ---- the wave's state: exp-sums over the 4 lane groups, everything
    // rescaled to the true max ----
#pragma unroll
    for (int X = 0; X < NB; ++X) {
        l[X] = rows_sum(l[X]);
        const float f = exp2_diff(m[X], mtrue[X]);
        l[X] *= f;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[X][b][e] *= f;
    }

    // ---- each wave parks its state in its own ring (its DMA has landed and
    // its reads are done, so no barrier is needed first) in the accumulator
    // layout (a lane's float4 at lane-consecutive addresses); after one
    // barrier wave w finishes the 16-dim tiles j = w, w + NW, .. of the
    // NB x DB: every lane merges the same register position of all waves and
    // stores 4 consecutive dims ----
    auto ring_o = [&](int w) {
        return reinterpret_cast<f32x4_t *>(lds + w * NST * C::SLOT);
    };
    auto ring_m = [&](int w) {  // [block][column] max, then exp-sum
        return reinterpret_cast<float *>(lds + w * NST * C::SLOT + NB * C::DB * 1024);
    };
    {
        f32x4_t *mo = ring_o(wave);
        float *mm = ring_m(wave);
#pragma unroll
        for (int X = 0; X < NB; ++X) {
#pragma unroll
            for (int b = 0; b < C::DB; ++b)  // tiles this wave merges stay in registers
                if ((X * C::DB + b) % NW != wave) mo[(X * C::DB + b) * 64 + lane] = o[X][b];
            if (grp == 0) {
                mm[X * 16 + col] = mtrue[X];
                mm[NB * 16 + X * 16 + col] = l[X];
            }
        }
    }
    __syncthreads();

    const bool direct = nparts <= 1;
#pragma unroll
    for (int X = 0; X < NB; ++X) {
        float fw[NW];
        float M = NEG_INF, den = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            fw[w] = ring_m(w)[X * 16 + col];
            M = fmaxf(M, fw[w]);
        }
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            fw[w] = exp2_diff(fw[w], M);
            den += ring_m(w)[NB * 16 + X * 16 + col] * fw[w];
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
            if ((X * C::DB + b) % NW != wave) continue;
            f32x4_t num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < NW; ++w)
                num += (w == wave ? o[X][b] : ring_o(w)[(X * C::DB + b) * 64 + lane]) * fw[w];
            if (col >= ncol) continue;
            const int h = X * ncol + col;
            const int d0 = 16 * b + 4 * grp;
            if (direct) {
                float inv = 1.f / den;
                if (p.sinks) {
                    // the head's sink: one more denominator term, no value (log2 units)
                    const float s2 = p.sinks[h] * LOG2E_F;
                    const float Mx = fmaxf(M, s2);
                    const float a = exp2_diff(M, Mx);
                    inv = a / (den * a + exp2_diff(s2, Mx));
                }
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.out) +
                                           ((size_t)q0 * p.hq + h) * D + d0) =
                    make_uint2(pack_bf16(num[0] * inv, num[1] * inv), pack_bf16(num[2] * inv, num[3] * inv));
            } else {
                const size_t si = ((size_t)q0 * p.hq + h) * p.max_parts + part;
                const float inv = 1.f / den;
                *reinterpret_cast<f32x4_t *>(p.tmp_out + si * D + d0) =
                    f32x4_t{num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv};
                if (b == 0 && grp == 0) {
                    p.max_logits[si] = M;
                    p.exp_sums[si] = den;
                }
            }
        }
    }
}

constexpr int ROWS_NW = 4;

// Heads per MFMA block for a group size: the largest power of two whose
// groups fit the 16 columns, at most 8 and at most the KV head count.
int rows_hpb(int group, int hkv) {
    int h = 8;
    while (h > 1 && (h * group > 16 || h > hkv)) h >>= 1;
    return h;
}

template <int D, int HPB, int NB>
hipError_t launch_rows(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    using C = RowCfg<D, HPB, NB, ROWS_NW>;
    const int parts = p.partition ? (p.max_seq_len + p.partition - 1) / p.partition : 1;
    const dim3 grid(p.num_seqs, parts, 1);
    const dim3 block(ROWS_NW * 64);
    if (li) *li = LaunchInfo{{(int)grid.x, (int)grid.y, 1}, (int)block.x, {C::KPB, ROWS_NW, C::NST}, 0};
    hipLaunchKernelGGL((decode_rows_kernel<D, HPB, NB, ROWS_NW>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int D, int NB>
hipError_t launch_rows_h(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    switch (p.hkv / NB) {
        case 2: return launch_rows<D, 2, NB>(p, stream, li);
        case 4: return launch_rows<D, 4, NB>(p, stream, li);
        case 8: return launch_rows<D, 8, NB>(p, stream, li);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rows_128(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    return p.hkv == rows_hpb(p.group, p.hkv) ? launch_rows_h<128, 1>(p, stream, li)
                                             : launch_rows_h<128, 2>(p, stream, li);
}

}  // namespace

// PA_DECODE_ROWS (read at every call): 0 never uses the whole-row kernels, 2
// uses them whenever the shape allows, otherwise (default) when the launch
// has enough (request, partition) items to occupy most CUs with one
// workgroup each.
// 8-bit caches take the whole-row kernel of decode_rows8.hip where its shape
// rule allows, under the same launch-size rule.
bool decode_rows_supported(const AttnParams &p) {
    if (p.kv8) {
        if (!decode_rows8_shape(p)) return false;
    } else {
        if (p.per_token || p.dtype != 1) return false;
        if (p.head_dim != 128 && p.head_dim != 256) return false;
        if (p.group < 1 || p.group > 8 || p.hkv < 2) return false;
        const int hpb = rows_hpb(p.group, p.hkv);
        if (hpb < 2 || (p.hkv != hpb && p.hkv != 2 * hpb)) return false;
        if (16 / hpb > p.block_size) return false;  // a chunk stays inside one page
        // Two blocks of D = 256 make 16 KB tiles: 32 DMA instructions a chunk
        // leave room for one ring stage only (vmcnt counts to 63), and that form
        // measured slower than the per-head kernel.
        if (p.head_dim == 256 && p.hkv == 2 * hpb) return false;
    }
    const char *e = std::getenv("PA_DECODE_ROWS");
    const int mode = e && e[0] ? std::atoi(e) : 1;
    if (mode == 0) return false;
    if (mode == 2) return true;
    // Launch-size rule: enough (request, partition) items for most CUs.  The
    // grid counts partitions up to the longest request, so short requests
    // leave some empty; 8-bit rows carry half the bytes of a workgroup's
    // chunks and need more items (GQA decode batch: 128 items, 86 of them
    // non-empty, took 52.5 us against 42.7 on the per-head kernel; 256 items,
    // 156 non-empty, 34.5 against 42.4).
    const long parts = p.partition ? (p.max_seq_len + p.partition - 1) / p.partition : 1;
    return (long)p.num_seqs * parts >= (p.kv8 ? 256 : 128);
}

hipError_t launch_decode_rows(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    if (p.kv8) return launch_decode_rows8(p, stream, li);
    switch (p.head_dim) {
        case 128: return launch_rows_128(p, stream, li);
        case 256: return launch_rows_h<256, 1>(p, stream, li);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
