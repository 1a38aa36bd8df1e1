// prefill.hip -- tiled bf16-MFMA paged attention for prefill and mixed batches.
//
// What it computes follows the pages: packed varlen queries [total_q, Hq, D]
// with request boundaries in cu_seqlens (v0.28.0 release post, "Packed queries
// and paged KV"), keys and values read through each request's block table
// (kernel walkthrough, "What is Paged Attention"), query heads of one GQA group
// sharing a KV head, each request's new tokens causally masked against its
// cached prefix (bottom-right: query j at position ctx + j sees keys 0..ctx+j),
// and a FlashAttention-2 style tiled online softmax (kernel walkthrough, "three
// Metal kernels": the tiled prefill kernel) in log2 space.
//
// The design is our own for CDNA4 (gfx950):
//  * one workgroup = one q-tile of one request x one KV head (x one split-KV
//    partition); 4 waves x 32 rows, the rows being (token, head-of-group)
//    pairs, so every K/V tile loaded serves the whole GQA group;
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: Q^T stays in registers as the
//    B operand for the whole key loop, K tiles are the A operand read from LDS;
//    a lane's accumulator column is one query row, so the softmax statistics
//    are per lane plus one v_permlane32_swap;
//  * O^T += V^T P^T: P^T comes straight from the S^T accumulator registers
//    (the key order of V^T in LDS is chosen to match the accumulator layout);
//  * K tiles move HBM -> LDS by global_load_lds_dwordx4 with an XOR swizzle of
//    the 16-byte pieces (conflict-free A-operand reads); V is transposed in
//    registers (v_perm_b32) into a padded V^T tile; two stages, one barrier per
//    32-key tile;
//  * requests are mapped to workgroups without a host pass: virtual tile x
//    belongs to the last request r with cu[r]/BQ + r <= x (surplus tiles exit).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

template <int D>
struct PrefillCfg {
    static constexpr int NWV = 4;                 // waves per workgroup
    static constexpr int N = 32;                  // keys per tile
    static constexpr int R = D * 2;               // bytes of a K/V row of one head
    static constexpr int KS = D / 16;             // MFMA k-steps of QK^T
    static constexpr int DB = D / 32;             // 32-row blocks of O^T
    static constexpr int K_BYTES = N * R;
    static constexpr int VT_STRIDE = N * 2 + 16;  // bytes per V^T row (padded)
    static constexpr int VT_BYTES = D * VT_STRIDE;
    static constexpr int STAGE = K_BYTES + VT_BYTES;
    static constexpr int NI_K = K_BYTES / 1024;   // DMA instructions per K tile
    static constexpr int NI_W = NI_K / NWV;       // per wave
    static constexpr int RPI = 1024 / R;          // K rows per DMA instruction
    static constexpr int PPR = R / 16;            // 16-byte pieces per row
    static constexpr int SWZ = PPR >= 16 ? 15 : PPR - 1;
    static constexpr int LDS_BYTES = 2 * STAGE;
    static_assert(NI_K % NWV == 0, "K tile split over the waves");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Position of tile key kk (0..31) in a V^T row: the 8 keys that one lane's
// B-operand slots of P^T hold (the S^T accumulator rows of k-step kk/16 and
// lane half h) are made contiguous.
__device__ __forceinline__ int vt_pos(int kk) {
    const int ks = kk >> 4, rem = kk & 15;
    const int a = rem >> 3, h = (rem >> 2) & 1, b = rem & 3;
    return 16 * ks + 8 * h + 4 * a + b;
}

template <int D>
__global__ __launch_bounds__(256) void prefill_kernel(const AttnParams p) {
    using C = PrefillCfg<D>;
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = p.group;
    const int TPW = 32 / G;       // tokens per wave
    const int BQ = C::NWV * TPW;  // tokens per workgroup

    // ---- which request and which q-tile (heaviest virtual tiles first) ----
    const int x = gridDim.x - 1 - blockIdx.x;
    int r;
    {
        int lo = 0, hi = p.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.cu_q[mid] / BQ + mid <= x) lo = mid; else hi = mid - 1;
        }
        r = lo;
    }
    const int q_begin = p.cu_q[r];
    const int q_len = p.cu_q[r + 1] - q_begin;
    const int tile = x - (q_begin / BQ + r);
    const int j0 = tile * BQ;  // first token of the tile within the request
    if (tile < 0 || j0 >= q_len) return;
    const int seq_len = p.seq_lens[r];
    const int ctx = seq_len - q_len;
    const int kvh = blockIdx.y;
    const int part = blockIdx.z;
    const int j_last = min(q_len, j0 + BQ) - 1;
    // keys of this workgroup: the partition, cut at the last token's position
    const int k_lo = p.partition ? part * p.partition : 0;
    const int k_part_end = p.partition ? k_lo + p.partition : seq_len;
    const int k_hi = min(k_part_end, ctx + j_last + 1);
    if (k_lo >= k_hi) return;

    // ---- this lane's query row (column of S^T) ----
    const int q = lane & 31;
    const int h = lane >> 5;
    const int tl = min(wave * TPW + q / G, j_last - j0);  // padding rows repeat the last token
    const int hg = q % G;
    const bool row_valid = q < TPW * G && j0 + wave * TPW + q / G <= j_last;
    const int jq = j0 + tl;          // token index within the request
    const int pos = ctx + jq;        // absolute position: sees keys 0..pos
    const int t_glob = q_begin + jq;
    const int head = kvh * G + hg;

    // Q^T B operand: 8 bf16 of d = 16*ks + 8*h .. +8 of this row, per k-step
    bf16x8_t qb[C::KS];
    {
        const uint4 *qrow = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const uint16_t *>(p.q) + ((size_t)t_glob * p.hq + head) * D);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const uint4 v = qrow[2 * ks + h];
            qb[ks] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    // ---- block-table window: lane i holds page (win_page + i) of the request ----
    const int bs = p.block_size, lbs = p.log2_bs;
    const int seq_pages = (seq_len + bs - 1) >> lbs;
    const int32_t *bt_row = p.bt + (size_t)r * p.bt_stride;
    auto load_window = [&](int page0) {
        const int lp = page0 + lane;
        int v = lp < seq_pages ? bt_row[lp] : 0;
        return v < 0 ? 0 : (v >= p.num_blocks ? p.num_blocks - 1 : v);
    };
    int win_page = k_lo >> lbs;
    int btv = load_window(win_page);
    // physical page of logical page lp (clamped to the last page of the request)
    auto phys_of = [&](int lp) -> int {
        lp = min(lp, seq_pages - 1);
        return __builtin_amdgcn_readlane(btv, lp - win_page);
    };

    const uint32_t row_stride = (uint32_t)p.hkv * C::R;
    const uint64_t page_bytes = (uint64_t)bs * row_stride;
    const uint64_t head_off = (uint64_t)kvh * C::R;
    const char *kc = reinterpret_cast<const char *>(p.kc);
    const char *vc = reinterpret_cast<const char *>(p.vc);

    // K DMA: this wave's instructions ii = wave*NI_W + i; lane offsets with the
    // piece swizzle (LDS slot s of row kk holds global piece s ^ (kk & SWZ))
    uint32_t kvoff[C::NI_W];
#pragma unroll
    for (int i = 0; i < C::NI_W; ++i) {
        const int ii = wave * C::NI_W + i;
        const int row = ii * C::RPI + lane / C::PPR;
        const int slot = lane % C::PPR;
        const int piece = slot ^ (row & C::SWZ);
        kvoff[i] = (uint32_t)(row & (bs - 1)) * row_stride + (uint32_t)piece * 16u;
    }
    const uint32_t lds0 = lds_addr(lds);

    // V load assignment: key quad kq (keys 4kq..4kq+3), 8-element d chunk dblk
    const int vt_id = threadIdx.x;
    const bool v_active = vt_id < D;  // (N/4) * (D/8) = D work units
    const int kq = vt_id & 7;
    const int dblk = vt_id >> 3;

    auto issue_k = [&](int kt, int stage) {
        const int lp0 = kt >> lbs;
        if (lp0 + ((C::N - 1) >> lbs) - win_page >= 64) {
            win_page = lp0;
            btv = load_window(win_page);
        }
#pragma unroll
        for (int i = 0; i < C::NI_W; ++i) {
            const int ii = wave * C::NI_W + i;
            const int phys = phys_of(lp0 + ((ii * C::RPI) >> lbs));
            const char *base = kc + (uint64_t)phys * page_bytes + head_off;
            dma16(base, kvoff[i], lds0 + stage * C::STAGE + ii * 1024);
        }
    };
    auto load_v = [&](int kt, uint4 (&vr)[4]) {
        if (!v_active) return;
        const int key0 = kt + 4 * kq;
        const int lp = key0 >> lbs;
        // the 4 keys of a quad share a page (pages hold a multiple of 4 keys)
        const int lpc = min(lp, seq_pages - 1);
        const int phys = __shfl(btv, lpc - win_page);
        const char *base = vc + (uint64_t)phys * page_bytes + head_off + dblk * 16;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int off = (key0 + b) & (bs - 1);
            vr[b] = *reinterpret_cast<const uint4 *>(base + (uint64_t)off * row_stride);
        }
    };
    auto store_vt = [&](int kt, int stage, uint4 (&vr)[4]) {
        if (!v_active) return;
        // keys past the sequence may hold anything (NaN): zeros, since p = 0
        // does not cancel a NaN in the MFMA
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (kt + 4 * kq + b >= seq_len) vr[b] = make_uint4(0, 0, 0, 0);
        char *vt = lds + stage * C::STAGE + C::K_BYTES;
        const int col = vt_pos(4 * kq) * 2;
        const uint32_t w0[4] = {vr[0].x, vr[0].y, vr[0].z, vr[0].w};
        const uint32_t w1[4] = {vr[1].x, vr[1].y, vr[1].z, vr[1].w};
        const uint32_t w2[4] = {vr[2].x, vr[2].y, vr[2].z, vr[2].w};
        const uint32_t w3[4] = {vr[3].x, vr[3].y, vr[3].z, vr[3].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // d = 8*dblk + 2w (low halves) and 2w+1 (high halves), 4 keys each
            uint2 lo, hi;
            lo.x = perm(w1[w], w0[w], 0x05040100u);
            lo.y = perm(w3[w], w2[w], 0x05040100u);
            hi.x = perm(w1[w], w0[w], 0x07060302u);
            hi.y = perm(w3[w], w2[w], 0x07060302u);
            const int d = 8 * dblk + 2 * w;
            *reinterpret_cast<uint2 *>(vt + d * C::VT_STRIDE + col) = lo;
            *reinterpret_cast<uint2 *>(vt + (d + 1) * C::VT_STRIDE + col) = hi;
        }
    };

    // ---- online softmax state (column q) ----
    f32x16_t o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
    float m = NEG_INF;  // running max of this row's scores (log2 units), shared by the lane pair
    float l = 0.f;      // this lane's half of the exp-sum
    const float sl2 = p.scale_log2;
    const int k_vis_end = min(k_hi, seq_len);  // keys past this are never visible

    const int ntiles = (k_hi - k_lo + C::N - 1) / C::N;
    uint4 vr[4];
    issue_k(k_lo, 0);
    load_v(k_lo, vr);
    wait_vmcnt<0>();
    store_vt(k_lo, 0, vr);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int kt = k_lo + it * C::N;
        const int stage = it & 1;
        const bool more = it + 1 < ntiles;
        if (more) {
            issue_k(kt + C::N, stage ^ 1);
            load_v(kt + C::N, vr);
        }
        const char *ks_base = lds + stage * C::STAGE;
        const char *vt_base = ks_base + C::K_BYTES;

        // ---- S^T = K Q^T (32 keys x 32 rows) ----
        f32x16_t s = {};
        {
            const int kk = lane & 31;
            const char *krow = ks_base + kk * C::R;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int piece = (2 * ks + h) ^ (kk & C::SWZ);
                const uint4 a = *reinterpret_cast<const uint4 *>(krow + piece * 16);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                            qb[ks], s, 0, 0, 0);
            }
        }
        // ---- mask, online softmax ----
        // key of accumulator register j: kt + 8*(j/4) + 4*h + (j%4)
        const bool need_mask = kt + C::N - 1 > ctx + j0 || kt + C::N > k_vis_end;
        float mx = NEG_INF;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float v = s[j] * sl2;
            if (need_mask) {
                const int key = kt + 8 * (j >> 2) + 4 * h + (j & 3);
                v = (key <= pos && key < k_vis_end) ? v : NEG_INF;
            }
            s[j] = v;
            mx = fmaxf(mx, v);
        }
        {
            const RowPair pm = row_pair32(mx);
            mx = fmaxf(pm.a, pm.b);
        }
        const float mn = fmaxf(m, mx);
        const float alpha = exp2_diff(m, mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
        uint32_t pk[8];
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            const float p0 = exp2_diff(s[j], m);
            const float p1 = exp2_diff(s[j + 1], m);
            pk[j / 2] = pack_bf16(p0, p1);
            l += bf16lo(pk[j / 2]) + bf16hi(pk[j / 2]);  // the weights actually applied
        }
        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
            u32x4_t pb = {pk[4 * ks2], pk[4 * ks2 + 1], pk[4 * ks2 + 2], pk[4 * ks2 + 3]};
            const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, pb);
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const int d = db * 32 + (lane & 31);
                const uint4 a = *reinterpret_cast<const uint4 *>(vt_base + d * C::VT_STRIDE +
                                                                 (16 * ks2 + 8 * h) * 2);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                bop, o[db], 0, 0, 0);
            }
        }
        if (more) {
            wait_vmcnt<0>();          // the next K tile's DMA and V rows are in
            store_vt(kt + C::N, stage ^ 1, vr);
        }
        __syncthreads();
    }

    // ---- finish: full exp-sum of the row, normalise, store ----
    {
        const RowPair pl = row_pair32(l);
        l = pl.a + pl.b;
    }
    if (!row_valid) return;
    const int n_parts = p.partition ? pos / p.partition + 1 : 1;
    if (p.partition && part >= n_parts) return;  // no keys of this row here
    const float inv = 1.f / l;
    if (n_parts == 1) {
        uint16_t *orow = reinterpret_cast<uint16_t *>(p.out) + ((size_t)t_glob * p.hq + head) * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d = db * 32 + 8 * a + 4 * h;
                uint2 w;
                w.x = pack_bf16(o[db][4 * a] * inv, o[db][4 * a + 1] * inv);
                w.y = pack_bf16(o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + d) = w;
            }
    } else {
        const size_t si = ((size_t)t_glob * p.hq + head) * p.max_parts + part;
        float *orow = p.tmp_out + si * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d = db * 32 + 8 * a + 4 * h;
                float4 w = {o[db][4 * a] * inv, o[db][4 * a + 1] * inv, o[db][4 * a + 2] * inv,
                            o[db][4 * a + 3] * inv};
                *reinterpret_cast<float4 *>(orow + d) = w;
            }
        if (h == 0) {
            p.max_logits[si] = m;
            p.exp_sums[si] = l;
        }
    }
}

template <int D>
hipError_t launch_d(const AttnParams &p, hipStream_t stream) {
    const int TPW = 32 / p.group;
    const int BQ = PrefillCfg<D>::NWV * TPW;
    const int tiles = p.total_q / BQ + p.num_seqs;
    const int parts = p.partition ? (p.max_seq_len + p.partition - 1) / p.partition : 1;
    hipLaunchKernelGGL((prefill_kernel<D>), dim3(tiles, p.hkv, parts), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int group) {
    return dtype == 1 && (head_dim == 64 || head_dim == 128 || head_dim == 256) && group >= 1 &&
           group <= 8;
}

hipError_t launch_prefill(const AttnParams &p, hipStream_t stream) {
    switch (p.head_dim) {
        case 64: return launch_d<64>(p, stream);
        case 128: return launch_d<128>(p, stream);
        case 256: return launch_d<256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
