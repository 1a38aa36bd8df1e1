// decode_rows8.hip -- paged GQA decode attention for gfx950 over 8-bit (E4M3)
// caches that streams whole cache rows: one workgroup per (request,
// partition) serves every KV head.
//
// What it computes is the same as the other decode kernels (vllm-metal kernel
// walkthrough, "What is Paged Attention"; GQA decode tips 1-4): softmax(q.k *
// scale) v over one request's keys read page by page through its block table,
// all query heads of a GQA group served from one read of each K/V row, the
// softmax online in log2 space, the key range optionally cut into partitions
// for the reduce kernel.  The caches hold E4M3 codes with one K and one V
// scale per KV head; codes widen exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8),
// the K scale joins the score scale and the V scale the finished output.
//
// Why whole rows: an 8-bit row of a token is Hkv x D bytes (1 KB for 8 heads
// of 128), so per-head slices are 128-byte pieces of every row; on random
// 16 KB pages a DMA-only skeleton moves the GQA decode batch at about
// 5.3 TB/s with whole (or half) rows against about 4.3 TB/s with head slices.
//
// Design (our own for CDNA4):
//  * the KV heads form groups of HG = 16 / group heads, so a group's query
//    heads fill the 16 columns of an MFMA block; wave w of the 4 serves head
//    group w % NG (NG = Hkv / HG groups) and takes the chunks w / NG,
//    w / NG + 4 / NG, .. of the partition, each a 16-key run of one page
//    (its group's HG x D bytes of each row, K and V), through a private ring;
//  * dense scores: the S^T block is 16 keys x 16 query heads, the sum over
//    the group's heads h of K_h Q_h^T where Q_h^T keeps only head h's query
//    columns (zero elsewhere), so every entry is the score of a column's
//    query with a key of the column's own head; the softmax works on 4 live
//    scores per lane, none wasted;
//  * O^T = V^T P^T with 16x16x32 products whose 32 k-slots are 4 keys x a
//    pair of heads per lane group; P^T keeps each column's probabilities in
//    the slots of its own head (zero in the other's), so the sum adds every
//    head's values to its own queries only; the V^T operand comes from one
//    ds_read_b64_tr_b8 (8 rows x 16 dims per 16 lanes);
//  * LDS layout of a tile: row t (key) is its group's HG x D bytes; inside
//    each 256-byte block (a pair of heads at D = 128) the 16-byte piece p of
//    row t sits at slot p ^ t.  The 32 lanes of a K read (piece p of 16 rows)
//    then reach 16 distinct slots of the 256-byte bank window, and so do the
//    32 lanes of a V^T read (pieces p and p ^ 8 of keys 0..7 or 8..15);
//  * the waves of a head group merge their states in LDS in the accumulator
//    layout after one barrier, the query rows come in by DMA to a per-wave
//    area (the waves start without a barrier).
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr float R8_RESCALE_THRESHOLD = 8.0f;  // log2 units

template <int HG>
struct Rows8Cfg {
    static constexpr int D = 128;
    static constexpr int NW = 4;
    static constexpr int KPC = 16;            // keys per chunk
    static constexpr int GR = HG * D;         // bytes of a group's part of an 8-bit row
    static constexpr int NPAIR = HG / 2;      // head pairs (256-byte blocks) of a group
    static constexpr int TILE = KPC * GR;     // K (or V) bytes of a chunk
    static constexpr int NI = TILE / 1024;    // 1 KB DMA instructions per tile
    static constexpr int VM = 2 * NI;         // per chunk: K and V
    static constexpr int NST = HG == 4 ? 2 : 4;
    static constexpr int SLOT = 2 * TILE;
    static constexpr int KS = D / 32;         // k-steps of S^T per head (16x16x32)
    static constexpr int DB = D / 16;         // 16-dim blocks of O^T
    static constexpr int RING = NW * NST * SLOT;
    static constexpr int QBYTES = 16 * 2 * D; // a group's 16 query rows (bf16)
    static constexpr int LDS_BYTES = RING + NW * QBYTES;
    static_assert(HG == 2 || HG == 4, "head groups of 2 or 4 heads");
    static_assert(DB * 1024 + 2 * 16 * 4 <= NST * SLOT, "a wave's state fits its ring");
    static_assert(VM * (NST - 1) < 64, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Wait until at most `ahead` chunks of this wave's DMA are in flight.
template <int VM, int MAXA>
__device__ __forceinline__ void r8_wait_ahead(int ahead) {
    if constexpr (MAXA >= 3) {
        if (ahead >= 3) {
            wait_vmcnt<3 * VM>();
            return;
        }
    }
    if constexpr (MAXA >= 2) {
        if (ahead == 2) {
            wait_vmcnt<2 * VM>();
            return;
        }
    }
    if (ahead >= 1)
        wait_vmcnt<VM>();
    else
        wait_vmcnt<0>();
}

template <int HG, int NG>
__global__ __launch_bounds__(256) void decode_rows8_kernel(const AttnParams p) {
    using C = Rows8Cfg<HG>;
    constexpr int D = C::D;
    constexpr int NW = C::NW;
    constexpr int NST = C::NST;
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];

    const int r = blockIdx.x;
    const int part = gridDim.y - 1 - blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;  // MFMA column: query head g 16 + col
    const int grp = lane >> 4;  // lane group: rows 4 grp .. 4 grp + 3
    const int G = p.group;      // 16 / HG
    constexpr int WPG = NW / NG;  // waves per head group (NG = Hkv / HG head groups)
    const int g = wave % NG;
    const int wi = wave / NG;
    const int tok_begin = p.partition ? part * p.partition : 0;
    const int lbs = p.log2_bs;
    const int c_begin = tok_begin / C::KPC;

    // Block-table window: lane i holds the page of the wave's chunk kw0 + i
    // (a chunk never spans two pages: 16 divides the page size).
    const int32_t *bt_row = p.bt + (size_t)r * p.bt_stride;
    auto load_window = [&](int kw0) -> int {
        const int ch = c_begin + wi + (kw0 + lane) * WPG;
        const int lp = (ch * C::KPC) >> lbs;
        const int v = lp < p.bt_stride ? bt_row[lp] : 0;
        return v < 0 ? 0 : (v >= p.num_blocks ? p.num_blocks - 1 : v);
    };
    // Every load the prologue needs is issued before the first wait: the
    // request's token range and key count, the first block-table window, the
    // group's K and V scales and the column's sink (a load first used at the
    // end would otherwise expose its latency there).
    const int q0 = p.cu_q[r];
    const int q1 = p.cu_q[r + 1];
    const int seq_len = p.seq_lens[r];
    int win_base = 0;
    int btv = load_window(0);
    float ksc[HG], vsc[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) {
        ksc[h] = p.k_scale[g * HG + h];
        vsc[h] = p.v_scale[g * HG + h];
    }
    // (without sinks the load reads a K scale and the value is not used)
    const float sink = *(p.sinks ? p.sinks + g * 16 + col : p.k_scale);
    if ((q1 - q0 <= 0) | (tok_begin >= seq_len) | (seq_len <= 0)) return;
    const int tok_end = p.partition ? min(seq_len, tok_begin + p.partition) : seq_len;
    const int nparts = p.partition ? (seq_len + p.partition - 1) / p.partition : 1;
    const int c_end = (tok_end + C::KPC - 1) / C::KPC;
    const int nchunks = c_end - c_begin;
    const int nmy = nchunks > wi ? (nchunks - wi + WPG - 1) / WPG : 0;

    const int RB = p.hkv * D;  // bytes of an 8-bit cache row
    const char *kc = reinterpret_cast<const char *>(p.kc) + g * C::GR;
    const int64_t v_minus_k = reinterpret_cast<const char *>(p.vc) - reinterpret_cast<const char *>(p.kc);
    const uint64_t page_bytes = (uint64_t)p.block_size * RB;

    // DMA lane offsets: instruction n fills tile bytes 1024 n + 16 lane, i.e.
    // slot s of pair block b of row t; it fetches piece s ^ t of that block.
    uint32_t voff[C::NI];
#pragma unroll
    for (int n = 0; n < C::NI; ++n) {
        const int pos = n * 1024 + lane * 16;
        const int t = pos / C::GR;
        const int b = (pos % C::GR) / 256;
        const int s = (pos % 256) / 16;
        voff[n] = (uint32_t)(t * RB + b * 256 + ((s ^ t) << 4));
    }
    const uint32_t lds_wave = lds_addr(lds) + (uint32_t)(wave * NST * C::SLOT);

    auto issue = [&](int k, int s) {
        if (k - win_base >= 64) {  // slide the window (long unsplit ranges only)
            win_base = k;
            btv = load_window(k);
        }
        const int tok0 = (c_begin + wi + k * WPG) * C::KPC;
        const int phys = __builtin_amdgcn_readlane(btv, k - win_base);
        const uint64_t off = (uint64_t)phys * page_bytes + (uint64_t)(tok0 & (p.block_size - 1)) * RB;
        const uint32_t ldsk = lds_wave + (uint32_t)(s * C::SLOT);
#pragma unroll
        for (int n = 0; n < C::NI; ++n) dma_lds<16>(kc + off, voff[n], ldsk + n * 1024);
#pragma unroll
        for (int n = 0; n < C::NI; ++n)
            dma_lds<16>(kc + off + v_minus_k, voff[n], ldsk + C::TILE + n * 1024);
    };

    // Chunk 0, the group's 16 query rows (4 KB) into this wave's own query
    // area, then the other ring stages.
    const int q_area = C::RING + wave * C::QBYTES;
    if (nmy > 0) issue(0, 0);
    {
        const char *qg = reinterpret_cast<const char *>(p.q) + ((size_t)q0 * p.hq + g * 16) * (2 * D);
#pragma unroll
        for (int j = 0; j < C::QBYTES / 1024; ++j)
            dma_lds<16>(qg, (uint32_t)(j * 1024 + lane * 16), lds_addr(lds) + q_area + j * 1024);
    }
#pragma unroll
    for (int s = 1; s < NST; ++s)
        if (s < nmy) issue(s, s);
    // chunk 0 and the queries have landed when at most the later chunks are in flight
    r8_wait_ahead<C::VM, NST - 1>(min(NST, nmy) - 1);

    // Q_h^T of the group's head h (B operand of S^T): column `col` is query
    // head g 16 + col when col / G == h, else zero; dims 32 ks + 8 grp ..
    const int hl = col / G;  // the column's head inside the group
    bf16x8_t qm[HG][C::KS];
    {
        const char *qrow = lds + q_area + col * (2 * D) + 16 * grp;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const bf16x8_t qv = *reinterpret_cast<const bf16x8_t *>(qrow + 64 * ks);
#pragma unroll
            for (int h = 0; h < HG; ++h) {
#pragma unroll
                for (int e = 0; e < 8; ++e) qm[h][ks][e] = hl == h ? qv[e] : (__bf16)0.f;
            }
        }
    }
    // P^T masks of head pair b: slots 0..3 of a lane group hold head 2b, 4..7 head 2b + 1
    uint32_t pa_mask[C::NPAIR], pb_mask[C::NPAIR];
#pragma unroll
    for (int b = 0; b < C::NPAIR; ++b) {
        pa_mask[b] = hl == 2 * b ? ~0u : 0u;
        pb_mask[b] = hl == 2 * b + 1 ? ~0u : 0u;
    }
    float scale_log2 = p.scale_log2 * ksc[0], vscale = vsc[0];
#pragma unroll
    for (int h = 1; h < HG; ++h)
        if (hl == h) {
            scale_log2 = p.scale_log2 * ksc[h];
            vscale = vsc[h];
        }

    // Fragment addresses inside a stage.  K (S^T A operand) of head h, k-step
    // ks: row `col`, piece 8 (h % 2) + 2 ks + grp / 2 of pair block h / 2,
    // 8-byte half grp % 2.  V^T (O^T A operand, transpose read) of pair b, dim
    // block j: row 4 grp + (col / 2) % 4, piece 8 (col / 8) + j, half col % 2.
    const int k_row = col * C::GR + (grp & 1) * 8;
    const int vt = 4 * grp + ((col >> 1) & 3);
    const int v_row = C::TILE + vt * C::GR + (col & 1) * 8;
    const int v_hi = (col >> 3) << 3;

    struct Frags {
        uint2 k[HG][C::KS];
        uint2 v[C::NPAIR][C::DB];
    };
    auto read = [&](const char *st, Frags &f) {
#pragma unroll
        for (int h = 0; h < HG; ++h)
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int pc = 8 * (h & 1) + 2 * ks + (grp >> 1);
                f.k[h][ks] = *reinterpret_cast<const uint2 *>(st + k_row + (h >> 1) * 256 +
                                                              ((pc ^ col) << 4));
            }
#pragma unroll
        for (int b = 0; b < C::NPAIR; ++b)
#pragma unroll
            for (int j = 0; j < C::DB; ++j) {
                const int pc = v_hi + j;
                f.v[b][j] = lds_read_tr8(st + v_row + b * 256 + ((pc ^ vt) << 4));
            }
    };

    float m = NEG_INF, mtrue = NEG_INF, l = 0.f;
    f32x4_t o[C::DB];
#pragma unroll
    for (int j = 0; j < C::DB; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // One chunk: S^T, online softmax, O^T.  MASKED is a wave's last chunk,
    // which may hold the end of the key range (keys from tok_end on get -inf
    // and their V codes, possibly NaN page tails, are replaced by zeros).
    auto chunk = [&](Frags &f, auto masked, int key0) {
        constexpr bool MASKED = decltype(masked)::value;
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < HG; ++h)
#pragma unroll
            for (int ks = 0; ks < C::KS; ks += 2) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    e4m3x8_to_bf16(f.k[h][ks].x, f.k[h][ks].y), qm[h][ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    e4m3x8_to_bf16(f.k[h][ks + 1].x, f.k[h][ks + 1].y), qm[h][ks + 1], s1, 0, 0, 0);
            }
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = (s0[e] + s1[e]) * scale_log2;
            if (MASKED && key0 + 4 * grp + e >= tok_end) x[e] = NEG_INF;
        }
        const float cm = rows_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        mtrue = fmaxf(mtrue, cm);
        if constexpr (!MASKED) {
            const bool up = cm > m + R8_RESCALE_THRESHOLD;
            if (__builtin_amdgcn_ballot_w64(up)) {
                const float mn = up ? cm : m;
                const float alpha = exp2_diff(m, mn);  // m = -inf before the first key
                m = mn;
                l *= alpha;
#pragma unroll
                for (int j = 0; j < C::DB; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[j][e] *= alpha;
            }
        } else {
            const float mn = fmaxf(m, cm);
            const float alpha = exp2_diff(m, mn);
            m = mn;
            l *= alpha;
#pragma unroll
            for (int j = 0; j < C::DB; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[j][e] *= alpha;
        }
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // m is finite once a chunk has been seen (every chunk has a live key)
            pr[e] = MASKED ? exp2_diff(x[e], m) : __builtin_amdgcn_exp2f(x[e] - m);
            l += pr[e];
        }
        const uint32_t pw0 = pack_bf16(pr[0], pr[1]), pw1 = pack_bf16(pr[2], pr[3]);
        uint32_t vmask = ~0u;
        if constexpr (MASKED) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (key0 + 4 * grp + e >= tok_end) vmask &= ~(0xffu << (8 * e));
        }
#pragma unroll
        for (int b = 0; b < C::NPAIR; ++b) {
            const bf16x8_t pb = __builtin_bit_cast(
                bf16x8_t, make_uint4(pw0 & pa_mask[b], pw1 & pa_mask[b], pw0 & pb_mask[b],
                                     pw1 & pb_mask[b]));
#pragma unroll
            for (int j = 0; j < C::DB; ++j) {
                uint2 w = f.v[b][j];
                if constexpr (MASKED) {
                    w.x &= vmask;
                    w.y &= vmask;
                }
                o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(w.x, w.y), pb, o[j],
                                                               0, 0, 0);
            }
        }
    };

    // Land chunk k, read its fragments, refill its stage with chunk k + NST.
    auto stage = [&](int k, Frags &f) {
        r8_wait_ahead<C::VM, NST - 1>(min(NST - 1, nmy - 1 - k));
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
        chunk(f, std::true_type{}, (c_begin + wi + (nmy - 1) * WPG) * C::KPC);
    }

    // ---- the wave's state: exp-sum over the 4 lane groups, everything
    // rescaled to the true max (a wave without chunks keeps m = -inf: zero) ----
    l = rows_sum(l);
    {
        const float f = exp2_diff(m, mtrue);
        l *= f;
#pragma unroll
        for (int j = 0; j < C::DB; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[j][e] *= f;
    }

    // ---- the waves of a head group meet in LDS: each parks its state in its
    // own ring (its DMA has landed and its reads are done) in the accumulator
    // layout; after one barrier wave wi of the group finishes the 16-dim
    // blocks j = wi, wi + WPG, ..: every lane merges the same register
    // position of the group's waves and stores 4 consecutive dims ----
    auto ring_o = [&](int w) { return reinterpret_cast<f32x4_t *>(lds + w * NST * C::SLOT); };
    auto ring_m = [&](int w) {  // [column] max, then exp-sum
        return reinterpret_cast<float *>(lds + w * NST * C::SLOT + C::DB * 1024);
    };
    if constexpr (WPG > 1) {
        f32x4_t *mo = ring_o(wave);
        float *mm = ring_m(wave);
#pragma unroll
        for (int j = 0; j < C::DB; ++j)
            if (j % WPG != wi) mo[j * 64 + lane] = o[j];
        if (grp == 0) {
            mm[col] = mtrue;
            mm[16 + col] = l;
        }
        __syncthreads();
    }

    const bool direct = nparts <= 1;
    const int h = g * 16 + col;  // query head
    float M = mtrue, den = l;
    float fw[WPG];
    if constexpr (WPG > 1) {
        M = NEG_INF;
        den = 0.f;
#pragma unroll
        for (int u = 0; u < WPG; ++u) {
            fw[u] = ring_m(g + u * NG)[col];
            M = fmaxf(M, fw[u]);
        }
#pragma unroll
        for (int u = 0; u < WPG; ++u) {
            fw[u] = exp2_diff(fw[u], M);
            den += ring_m(g + u * NG)[16 + col] * fw[u];
        }
    }
#pragma unroll
    for (int j = 0; j < C::DB; ++j) {
        if (j % WPG != wi) continue;
        f32x4_t num = o[j];
        if constexpr (WPG > 1) {
            num = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < WPG; ++u)
                num += (u == wi ? o[j] : ring_o(g + u * NG)[j * 64 + lane]) * fw[u];
        }
        num *= vscale;
        const int d0 = 16 * j + 4 * grp;
        if (direct) {
            float inv = 1.f / den;
            if (p.sinks) {
                // the head's sink: one more denominator term, no value (log2 units)
                const float s2 = sink * LOG2E_F;
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
            if (wi == 0 && j == 0 && grp == 0) {
                p.max_logits[si] = M;
                p.exp_sums[si] = den;
            }
        }
    }
}

template <int HG, int NG>
hipError_t launch_rows8(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    using C = Rows8Cfg<HG>;
    const int parts = p.partition ? (p.max_seq_len + p.partition - 1) / p.partition : 1;
    const dim3 grid(p.num_seqs, parts, 1);
    const dim3 block(C::NW * 64);
    if (li) *li = LaunchInfo{{(int)grid.x, (int)grid.y, 1}, (int)block.x, {C::KPC, C::NW, C::NST}, 0};
    hipLaunchKernelGGL((decode_rows8_kernel<HG, NG>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int HG>
hipError_t launch_rows8_g(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    switch (p.hkv / HG) {
        case 1: return launch_rows8<HG, 1>(p, stream, li);
        case 2: return launch_rows8<HG, 2>(p, stream, li);
        case 4: return launch_rows8<HG, 4>(p, stream, li);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// 8-bit caches, bf16 queries, D = 128, groups of 4 or 8 query heads per KV
// head (head groups of 4 or 2 KV heads fill 16 columns), 1, 2 or 4 head
// groups, pages of a multiple of 16 tokens.
bool decode_rows8_shape(const AttnParams &p) {
    if (!p.kv8 || p.per_token || p.dtype != 1 || p.head_dim != 128) return false;
    if (p.group != 4 && p.group != 8) return false;
    const int hg = 16 / p.group;
    if (p.hkv % hg != 0) return false;
    const int ng = p.hkv / hg;
    if (ng != 1 && ng != 2 && ng != 4) return false;
    return p.block_size >= 16 && p.block_size % 16 == 0;
}

hipError_t launch_decode_rows8(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    switch (p.group) {
        case 4: return launch_rows8_g<4>(p, stream, li);
        case 8: return launch_rows8_g<2>(p, stream, li);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
