// decode_mfma.hip -- paged GQA decode attention for gfx950 with the group's
// scores and PV on bf16 MFMA: decode batches (one query token per request)
// with bf16 queries over bf16 or 8-bit (E4M3) caches.
//
// What it computes is the same as the VALU decode kernel (vllm-metal kernel
// walkthrough, "What is Paged Attention"; GQA decode tips 1-4): softmax(q.k *
// scale) v over one request's keys read page by page through its block table,
// all query heads of a GQA group served together so each K/V page is read
// from HBM once, the softmax online in log2 space, and the key range
// optionally cut into partitions whose (max, exp-sum) statistics and
// normalised partial outputs the reduce kernel merges.
//
// Why MFMA here: per 16-key chunk the VALU form spends about a thousand
// cycles of v_dot2 and cross-lane sums per wave, as long as the chunk's DMA
// takes to land, so the per-chunk arithmetic (not HBM) set the pace.  With the
// group's heads as the 16 columns of a 16x16 block the same chunk costs
// D/32 v_mfma_f32_16x16x32_bf16 for S^T and D/16 v_mfma_f32_16x16x16_bf16 for
// O^T (unused columns are zero queries), and the softmax touches 4 scores a
// lane.
//
// The design is our own for CDNA4:
//  * grid = (kv_heads, requests, partitions), partitions last-first; NW waves
//    take the 16-key chunks of the partition round-robin, each with a private
//    ring of NST LDS stages, so no barrier is needed until the final merge;
//  * K/V rows move HBM -> LDS with global_load_lds_dwordx4 into a
//    piece-major layout: keys in groups of 8, each 16-byte piece of the 8
//    keys one 128-byte line, the key slot XORed with 4 on odd pieces; one
//    instruction fills 8 pieces of one key group, so a lane's source offset
//    within the page is fixed and an instruction never spans two pages;
//  * S^T = K Q^T (16 keys x 16 heads): K fragments by ds_read_b128 (8 lanes
//    read one full line), Q^T in registers for the whole partition;
//  * a lane's accumulator column is one head and its 4 rows are 4 keys, so the
//    chunk max needs two row-pair exchanges; exp2 on 4 values;
//  * O^T += V^T P^T: P^T is the S^T accumulator packed to bf16 in place, V^T
//    fragments come from the row-major V tile through ds_read_b64_tr_b16;
//    the O^T column of a lane is its own head, so rescales are per lane;
//  * the reference max is raised lazily (only when a chunk's max passes it by
//    more than 8 in log2 units), and every wave is rescaled to the true max
//    before the LDS merge, so the statistics stored for the reduce are exact;
//  * 8-bit caches: 32-key chunks land as raw E4M3 rows (16-byte pieces XOR-
//    swizzled by row) and are converted in registers after the fragment reads
//    (v_cvt_scalef32_pk_bf16_fp8, exact).  S^T is two 16-key blocks whose rows
//    are permuted so that a lane's 8 scores are 8 consecutive keys, the B
//    operand of a 32-key v_mfma_f32_16x16x32_bf16 for O^T; its V^T operand
//    (8 keys of one column) comes from ds_read_b64_tr_b8.  The head's K scale
//    joins the softmax scale and its V scale the output.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr float MF_RESCALE_THRESHOLD = 8.0f;  // log2 units

template <int D, bool KV8_, int NW_, int NST_>
struct MfCfg {
    static constexpr bool KV8 = KV8_;            // caches hold E4M3 codes
    static constexpr int CT = KV8 ? 32 : 16;     // keys per chunk (one or two 16-row S^T blocks)
    static constexpr int QR = D * 2;             // bytes of a bf16 query row of one head
    static constexpr int R = KV8 ? D : 2 * D;    // bytes of a cached K/V row of one head
    static constexpr int TILE = CT * R;          // K (or V) tile of one chunk
    static constexpr int SLOT = 2 * TILE;        // one LDS stage: K tile, then V tile
    // bytes one lane moves per DMA instruction: 16, or 4 for 64-byte 8-bit
    // rows (so one instruction never spans more than 8 rows, i.e. one page)
    static constexpr int DW = (KV8 && D < 128) ? 4 : 16;
    static constexpr int NI = TILE / (64 * DW);  // DMA instructions per tile
    static constexpr int RPI = 64 * DW / R;      // rows per instruction (8-bit tiles)
    static constexpr int VM_PER_CHUNK = 2 * NI;  // K and V
    static constexpr int PPR = R / 16;           // 16-byte pieces per row
    static constexpr int GROUP_BYTES = 8 * R;    // one 8-key group of the bf16 layout
    static constexpr int IPG = PPR / 8;          // bf16: DMA instructions per key group (1 KB each)
    static constexpr int KS = D / 32;            // k-steps of S^T (16x16x32)
    static constexpr int DB = D / 16;            // 16-row blocks of O^T
    static constexpr int NW = NW_;
    static constexpr int NST = NST_;
    static constexpr int GMAX = 8;               // largest group served
    static constexpr int STATE_FLOATS = GMAX * D + 2 * GMAX;  // O^T rows of the group, m, l
    static constexpr int STAGE_BYTES = NW * NST * SLOT;
    static constexpr int QI = (GMAX * QR + 1023) / 1024;  // most DMA instructions for a group's queries
    static constexpr int QBYTES = QI * 1024;     // per wave: the group's query rows
    static constexpr int RING_BYTES = STAGE_BYTES + NW * QBYTES;
    static constexpr int MERGE_BYTES = NW * STATE_FLOATS * 4;
    static constexpr int LDS_BYTES = RING_BYTES > MERGE_BYTES ? RING_BYTES : MERGE_BYTES;
    static_assert(KV8 || PPR % 8 == 0, "whole 128-byte lines per row");
    static_assert(!KV8 || (RPI >= 1 && RPI <= 8 && CT % RPI == 0), "8-bit DMA shape");
    static_assert(NST * VM_PER_CHUNK < 64, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Byte offset of piece p (elements 8p..8p+7) of key `key` in a tile whose rows
// are R bytes: the piece-major layout of the file comment.
template <int R>
__device__ __forceinline__ int mf_tile_off(int key, int piece) {
    return (key >> 3) * (8 * R) + piece * 128 + (((key & 7) ^ ((piece & 1) << 2)) << 4);
}

// Byte offset of 16-byte piece p of row t (0..31) in an 8-bit tile of D-byte
// rows: row-major with the piece index XORed by f(t).  With a = bits 3-4 of
// t, e = bit 2 and c = bits 0-1, A = a ^ 2e, and f = A (D = 64), 2A + c/2
// (D = 128) or 4A + c (D = 256), the two fragment reads are free of bank
// conflicts: 16 lanes reading one 8-byte column of rows 8a' + 4e' + c' (S^T
// K rows, e' fixed) or of the 8 rows 8a' .. 8a'+7 (V^T transpose reads) all
// land on distinct 8-byte words of a 256-byte bank line.
template <int D>
__device__ __forceinline__ int kv8_f(int t) {
    const int A = (((t >> 3) ^ (((t >> 2) & 1) << 1)) & 3);
    if constexpr (D == 64) return A;
    else if constexpr (D == 128) return (A << 1) | ((t & 3) >> 1);
    else return (A << 2) | (t & 3);
}
template <int D>
__device__ __forceinline__ int kv8_off(int t, int p) {
    return t * D + ((p ^ kv8_f<D>(t)) << 4);
}

// Wait until this wave's DMA for the chunk `ahead` chunks before the newest
// one has landed in LDS (vmcnt counts instructions and completes in order).
template <int VM, int MAXA>
__device__ __forceinline__ void mf_wait_ahead(int ahead) {
    if constexpr (MAXA > 0) {
        if (ahead >= MAXA) {
            wait_vmcnt<MAXA * VM>();
            return;
        }
        mf_wait_ahead<VM, MAXA - 1>(ahead);
    } else {
        wait_vmcnt<0>();
    }
}

// A chunk's MFMA fragments: K rows (A operand of S^T) and V^T (A operand of O^T).
template <class C>
struct Frags {
    bf16x8_t k[C::KS];
    s16x4_t v[C::DB];
};

template <class C>
__device__ __forceinline__ void mf_read(const char *ka, const char *va, Frags<C> &f) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) f.k[ks] = *reinterpret_cast<const bf16x8_t *>(ka + ks * 512);
#pragma unroll
    for (int b = 0; b < C::DB; ++b) f.v[b] = lds_read_tr16(va + b * 256);
}

// One chunk: S^T, online softmax, O^T.  MASKED is the chunk holding the end of
// the key range: keys past tok_end get score -inf and their V entries
// (possibly NaN page tails) are replaced by zeros.
template <class C, bool MASKED>
__device__ __forceinline__ void mf_chunk(Frags<C> &f, const bf16x8_t (&qb)[C::KS], int key0,
                                         int tok_end, float scale_log2, float &m, float &mtrue,
                                         float &l, f32x4_t (&o)[C::DB]) {
    // ---- S^T: 16 keys x 16 heads, two independent accumulation chains ----
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ks += 2) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k[ks], qb[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k[ks + 1], qb[ks + 1], s1, 0, 0, 0);
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = (s0[i] + s1[i]) * scale_log2;
        if (MASKED && key0 + i >= tok_end) x[i] = NEG_INF;
    }
    const float cm = rows_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    mtrue = fmaxf(mtrue, cm);
    if constexpr (!MASKED) {
        // every score is finite: rescale (uniformly) only when some head's
        // chunk max passed its reference by more than the threshold
        const bool up = cm > m + MF_RESCALE_THRESHOLD;
        if (__builtin_amdgcn_ballot_w64(up)) {
            const float mn = up ? cm : m;
            const float alpha = exp2_diff(m, mn);  // m = -inf before the first key
            m = mn;
            l *= alpha;
#pragma unroll
            for (int b = 0; b < C::DB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[b][i] *= alpha;
        }
    } else {
        const float mn = fmaxf(m, cm);
        const float alpha = exp2_diff(m, mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[b][i] *= alpha;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pr[i] = MASKED ? exp2_diff(x[i], m) : __builtin_amdgcn_exp2f(x[i] - m);
        l += pr[i];
    }
    const uint2 pw = make_uint2(pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]));
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, pw);

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int b = 0; b < C::DB; ++b) {
        s16x4_t a = f.v[b];
        if constexpr (MASKED) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (key0 + i >= tok_end) a[i] = 0;
        }
        o[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[b], 0, 0, 0);
    }
}

// An 8-bit chunk's fragments, raw codes: K rows of both S^T blocks (8 dims
// of one key each) and V^T (8 keys of one column each).
template <class C>
struct Frags8 {
    uint2 k[2][C::KS];
    uint2 v[C::DB];
};

// Fragment reads of an 8-bit stage.  S^T block b2 row r holds key
// 8 (r / 4) + r % 4 + 4 b2, so the lane of column c and group g ends up with
// the scores of keys 8 g .. 8 g + 7.  The V^T transpose read: lane j of group g
// passes row 8 g + j / 2, bytes 16 b + 8 (j % 2) .. +7, and receives column
// 16 b + j of rows 8 g .. 8 g + 7.
template <class C, int D>
__device__ __forceinline__ void mf_read8(const char *st, int col, int grp, Frags8<C> &f) {
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
        const int t = 8 * (col >> 2) + (col & 3) + 4 * b2;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            f.k[b2][ks] = *reinterpret_cast<const uint2 *>(st + kv8_off<D>(t, 2 * ks + (grp >> 1)) +
                                                           8 * (grp & 1));
    }
    const int tv = 8 * grp + (col >> 1);
#pragma unroll
    for (int b = 0; b < C::DB; ++b) {
        typedef __attribute__((ext_vector_type(2))) int i32x2_t;
        const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t *)(st + C::TILE + kv8_off<D>(tv, b) +
                                                          8 * (col & 1)));
        f.v[b] = make_uint2((uint32_t)v[0], (uint32_t)v[1]);
    }
}

// One 32-key 8-bit chunk: S^T (two blocks), online softmax, O^T with K = 32.
template <class C, bool MASKED>
__device__ __forceinline__ void mf_chunk8(Frags8<C> &f, const bf16x8_t (&qb)[C::KS], int key0,
                                          int tok_end, float scale_log2, float &m, float &mtrue,
                                          float &l, f32x4_t (&o)[C::DB]) {
    f32x4_t s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
            s[b2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                e4m3x8_to_bf16(f.k[b2][ks].x, f.k[b2][ks].y), qb[ks], s[b2], 0, 0, 0);
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[j] = s[j >> 2][j & 3] * scale_log2;  // key key0 + j
        if (MASKED && key0 + j >= tok_end) x[j] = NEG_INF;
    }
    float cmax = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) cmax = fmaxf(cmax, x[j]);
    const float cm = rows_max(cmax);
    mtrue = fmaxf(mtrue, cm);
    if constexpr (!MASKED) {
        const bool up = cm > m + MF_RESCALE_THRESHOLD;
        if (__builtin_amdgcn_ballot_w64(up)) {
            const float mn = up ? cm : m;
            const float alpha = exp2_diff(m, mn);
            m = mn;
            l *= alpha;
#pragma unroll
            for (int b = 0; b < C::DB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[b][i] *= alpha;
        }
    } else {
        const float mn = fmaxf(m, cm);
        const float alpha = exp2_diff(m, mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[b][i] *= alpha;
    }
    float pr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        pr[j] = MASKED ? exp2_diff(x[j], m) : __builtin_amdgcn_exp2f(x[j] - m);
        l += pr[j];
    }
    const uint4 pw = make_uint4(pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]),
                                pack_bf16(pr[4], pr[5]), pack_bf16(pr[6], pr[7]));
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
    for (int b = 0; b < C::DB; ++b) {
        bf16x8_t a = e4m3x8_to_bf16(f.v[b].x, f.v[b].y);
        if constexpr (MASKED) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (key0 + j >= tok_end) a[j] = (__bf16)0.f;
        }
        o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[b], 0, 0, 0);
    }
}

template <int D, bool KV8, int NW, int NST>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(const AttnParams p) {
    using C = MfCfg<D, KV8, NW, NST>;
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];

    const int kvh = blockIdx.x;
    const int part = gridDim.z - 1 - blockIdx.z;
    const int r = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;  // MFMA column: head `col` of the group
    const int grp = lane >> 4;  // lane group: keys 4 grp .. 4 grp + 3 of a 16-key block
    constexpr int CT = C::CT;
    const int tok_begin = p.partition ? part * p.partition : 0;
    const int bs = p.block_size;
    const int lbs = p.log2_bs;
    const int c_begin = tok_begin / CT;
    const int ppc = bs < CT ? CT / bs : 1;  // pages per chunk: 1, 2 or 4
    const int cpw = 64 / ppc;               // chunks covered by one block-table window

    // Block-table window: lane i holds page (i / cpw) of the wave's chunk
    // kw0 + i % cpw; issued before the request's lengths arrive.
    const int32_t *bt_row = p.bt + (size_t)r * p.bt_stride;
    auto load_window = [&](int kw0) -> int {
        const int k = kw0 + lane % cpw;
        const int ch = c_begin + wave + k * NW;
        const int lp = ((ch * CT) >> lbs) + lane / cpw;
        const int v = lp < p.bt_stride ? bt_row[lp] : 0;
        return v < 0 ? 0 : (v >= p.num_blocks ? p.num_blocks - 1 : v);
    };
    int win_base = 0;
    int btv = load_window(0);

    // the request's window and length, loaded together
    const int q0 = p.cu_q[r];
    const int q1 = p.cu_q[r + 1];
    const int seq_len = p.seq_lens[r];
    if (q1 - q0 <= 0) return;
    if (tok_begin >= seq_len || seq_len <= 0) return;
    const int tok_end = p.partition ? min(seq_len, tok_begin + p.partition) : seq_len;
    const int nparts = p.partition ? (seq_len + p.partition - 1) / p.partition : 1;
    const int G = p.group;
    const int c_end = (tok_end + CT - 1) / CT;
    const int nchunks = c_end - c_begin;
    const int nmy = nchunks > wave ? (nchunks - wave + NW - 1) / NW : 0;

    const uint32_t row_stride = (uint32_t)p.hkv * C::R;  // bytes between tokens of a page
    const char *kc = reinterpret_cast<const char *>(p.kc);
    const int64_t v_minus_k = reinterpret_cast<const char *>(p.vc) - kc;
    const uint64_t page_bytes = (uint64_t)bs * row_stride;
    const uint64_t head_off = (uint64_t)kvh * C::R;

    // DMA lane offsets.  bf16: lane i of an instruction fills tile slot i of
    // a 1 KB block (8 pieces of one 8-key group), i.e. key (i % 8) ^ 4 ((i / 8) & 1)
    // of the group and piece 8 q + i / 8.  8-bit: instruction n fills rows
    // n RPI .. (n + 1) RPI - 1 of the tile, lane i the DW bytes at tile offset
    // n 64 DW + i DW, which hold piece s ^ f(row) of its row (s = the slot).
    const int dkey = (lane & 7) ^ (((lane >> 3) & 1) << 2);
    const uint32_t voff0 = (uint32_t)dkey * row_stride + (uint32_t)(lane >> 3) * 16;
    uint32_t voff8[KV8 ? C::NI : 1];
    if constexpr (KV8) {
        constexpr int LPR = C::R / C::DW;  // lanes per row
#pragma unroll
        for (int n = 0; n < C::NI; ++n) {
            const int ri = lane / LPR;     // row within the instruction
            const int w = lane % LPR;      // DW-byte word within the row
            const int t = n * C::RPI + ri;
            const int slot = w * C::DW / 16;
            const int piece = slot ^ kv8_f<D>(t);
            voff8[n] = (uint32_t)ri * row_stride + (uint32_t)(piece * 16 + (w * C::DW) % 16);
        }
    }
    const uint32_t lds_wave = lds_addr(lds) + (uint32_t)(wave * NST * C::SLOT);

    auto issue = [&](int k, int s) {
        if (k - win_base >= cpw) {  // slide the window (long unsplit ranges only)
            win_base = k;
            btv = load_window(k);
        }
        const int tok0 = (c_begin + wave + k * NW) * CT;
        const int idx = k - win_base;
        const int phys0 = __builtin_amdgcn_readlane(btv, idx);
        if constexpr (KV8) {
            // rows n RPI.. of the chunk are in page (n RPI) / bs of the chunk;
            // pages past the sequence hold only masked keys: page 0 is re-read
            const uint32_t ldsk = lds_wave + (uint32_t)(s * C::SLOT);
#pragma unroll
            for (int n = 0; n < C::NI; ++n) {
                const int t0 = n * C::RPI;
                const int j = bs < CT ? (t0 >> lbs) : 0;
                const int phys = (j == 0 || tok0 + j * bs >= seq_len)
                                     ? phys0
                                     : __builtin_amdgcn_readlane(btv, idx + j * cpw);
                const uint64_t off = (uint64_t)phys * page_bytes +
                                     (uint64_t)((tok0 + t0) & (bs - 1)) * row_stride + head_off;
                dma_lds<C::DW>(kc + off, voff8[n], ldsk + n * 64 * C::DW);
                dma_lds<C::DW>(kc + off + v_minus_k, voff8[n], ldsk + C::TILE + n * 64 * C::DW);
            }
        } else {
            const uint64_t off0 = (uint64_t)phys0 * page_bytes +
                                  (uint64_t)(tok0 & (bs - 1)) * row_stride + head_off;
            uint64_t off1 = off0 + 8ull * row_stride;
            if (ppc == 2) {
                // keys 8..15 live in the next page; past the sequence those keys
                // are masked, so page 0 is re-read instead.
                const int phys1 =
                    tok0 + 8 < seq_len ? __builtin_amdgcn_readlane(btv, idx + cpw) : phys0;
                off1 = (uint64_t)phys1 * page_bytes + head_off;
            }
            const char *kb[2] = {kc + off0, kc + off1};
            const uint32_t ldsk = lds_wave + (uint32_t)(s * C::SLOT);
            const uint32_t ldsv = ldsk + C::TILE;
#pragma unroll
            for (int gk = 0; gk < 2; ++gk)
#pragma unroll
                for (int q = 0; q < C::IPG; ++q)
                    dma_lds<16>(kb[gk], voff0 + q * 128, ldsk + gk * C::GROUP_BYTES + q * 1024);
#pragma unroll
            for (int gk = 0; gk < 2; ++gk)
#pragma unroll
                for (int q = 0; q < C::IPG; ++q)
                    dma_lds<16>(kb[gk] + v_minus_k, voff0 + q * 128,
                                ldsv + gk * C::GROUP_BYTES + q * 1024);
        }
    };

    // Chunk 0 first (its issue waits for the block-table window), then the
    // group's query rows (G R contiguous bytes) by DMA into this wave's query
    // area, then the other chunks ahead of the loop: the queries land with
    // chunk 0 and no compiler-counted load is outstanding once the chunk waits
    // start.
    constexpr int PRE = NST;  // chunks issued ahead of the loop
    bf16x8_t qb[C::KS];
    if (nmy > 0) {
        issue(0, 0);
        const uint32_t lds_q = lds_addr(lds) + (uint32_t)(C::STAGE_BYTES + wave * C::QBYTES);
        const char *qg = reinterpret_cast<const char *>(p.q) +
                         ((size_t)q0 * p.hq + (size_t)kvh * G) * C::QR;
        const int qbytes = G * C::QR;
#pragma unroll
        for (int j = 0; j < C::QI; ++j) {
            if (j * 1024 < qbytes) {
                const uint32_t off = (uint32_t)(j * 1024 + lane * 16);
                dma_lds<16>(qg, off < (uint32_t)qbytes ? off : 0u, lds_q + j * 1024);
            }
        }
#pragma unroll
        for (int s = 1; s < PRE; ++s)
            if (s < nmy) issue(s, s);
        // Q^T, the B operand of S^T: head `col` (zero past the group), dims
        // 32 ks + 8 grp .. +7 of k-step ks
        mf_wait_ahead<C::VM_PER_CHUNK, PRE - 1>(min(PRE, nmy) - 1);
        const char *qrow = lds + C::STAGE_BYTES + wave * C::QBYTES + col * C::QR + 16 * grp;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            if (col < G) {
                qb[ks] = *reinterpret_cast<const bf16x8_t *>(qrow + 64 * ks);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) qb[ks][e] = (__bf16)0.f;
            }
        }
    }

    // per lane: head `col`; reference max, true max, partial exp-sum of the
    // lane's keys, O^T rows 16 b + 4 grp + i of the head
    float m = NEG_INF, mtrue = NEG_INF, l = 0.f;
    f32x4_t o[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) o[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // 8-bit caches: the head's K scale joins the softmax scale
    const float scale_log2 = KV8 ? p.scale_log2 * p.k_scale[kvh] : p.scale_log2;
    // bf16 fragment addresses inside a stage: K rows `col`, pieces 4 ks + grp;
    // V^T transpose reads of key 4 grp + col / 4, elements 16 b + 4 (col % 4)
    const int ka_off = KV8 ? 0 : mf_tile_off<C::R>(col, grp);
    const int va_off =
        KV8 ? 0 : C::TILE + mf_tile_off<C::R>(4 * grp + (col >> 2), (col >> 1) & 1) + (col & 1) * 8;
    using F = typename std::conditional<KV8, Frags8<C>, Frags<C>>::type;
    auto read = [&](const char *st, F &f) {
        if constexpr (KV8)
            mf_read8<C, D>(st, col, grp, f);
        else
            mf_read<C>(st + ka_off, st + va_off, f);
    };

    // Land chunk k and read its fragments into registers (register staging):
    // its LDS stage is refilled right after the reads, so NST + 1 chunks are
    // in flight while the wave computes instead of NST - 1.
    auto stage = [&](int k, F &f) {
        mf_wait_ahead<C::VM_PER_CHUNK, NST - 1>(min(NST - 1, nmy - 1 - k));
        read(lds + (wave * NST + k % NST) * C::SLOT, f);
        if (k + NST < nmy) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage k is read
            issue(k + NST, k % NST);
        }
    };
    auto step = [&](F &f, auto masked, int key0) {
        if constexpr (KV8)
            mf_chunk8<C, decltype(masked)::value>(f, qb, key0, tok_end, scale_log2, m, mtrue, l, o);
        else
            mf_chunk<C, decltype(masked)::value>(f, qb, key0, tok_end, scale_log2, m, mtrue, l, o);
    };
    for (int k = 0; k < nmy - 1; ++k) {
        F f;
        stage(k, f);
        step(f, std::false_type{}, 0);
    }
    if (nmy > 0) {
        F f;
        stage(nmy - 1, f);
        // key of the lane's first score: 4 grp (bf16 block) or 8 grp (8-bit pair of blocks)
        const int key0 = (c_begin + wave + (nmy - 1) * NW) * CT + (KV8 ? 8 : 4) * grp;
        step(f, std::true_type{}, key0);
    }

    // ---- the wave's state: exp-sum over its 4 lane groups, everything
    // rescaled to the true max ----
    l = rows_sum(l);
    {
        const float f = exp2_diff(m, mtrue);
        l *= f;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[b][i] *= f;
    }

    // ---- one state per wave to LDS, then all threads merge the waves ----
    __syncthreads();  // every wave is done with its stages
    float *mrg = reinterpret_cast<float *>(lds);
    if (col < G) {
        float *st = mrg + wave * C::STATE_FLOATS;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
            *reinterpret_cast<f32x4_t *>(st + col * D + 16 * b + 4 * grp) = o[b];
        if (grp == 0) {
            st[C::GMAX * D + col] = mtrue;
            st[C::GMAX * D + C::GMAX + col] = l;
        }
    }
    __syncthreads();

    const bool direct = nparts <= 1;
    const float vscale = KV8 ? p.v_scale[kvh] : 1.0f;  // 8-bit caches: the head's V scale
    for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
        const int g = idx / D;
        const int d = idx - g * D;
        float M = NEG_INF;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, mrg[w * C::STATE_FLOATS + C::GMAX * D + g]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float *st = mrg + w * C::STATE_FLOATS;
            const float f = exp2_diff(st[C::GMAX * D + g], M);
            num += st[g * D + d] * f;
            den += st[C::GMAX * D + C::GMAX + g] * f;
        }
        const int h = kvh * G + g;
        float o_ = num / den;
        if (direct && p.sinks) {
            // the head's sink: one more denominator term, no value (log2 units)
            const float s2 = p.sinks[h] * LOG2E_F;
            const float Mx = fmaxf(M, s2);
            const float a = exp2_diff(M, Mx);
            o_ = num * a / (den * a + exp2_diff(s2, Mx));
        }
        if constexpr (KV8) o_ *= vscale;
        if (direct) {
            reinterpret_cast<uint16_t *>(p.out)[((size_t)q0 * p.hq + h) * D + d] = to_bf16(o_);
        } else {
            const size_t si = ((size_t)q0 * p.hq + h) * p.max_parts + part;
            p.tmp_out[si * D + d] = o_;
            if (d == 0) {
                p.max_logits[si] = M;
                p.exp_sums[si] = den;
            }
        }
    }
}

// Waves per workgroup and LDS stages per wave: 2 waves at D = 256 keep two
// workgroups on a CU (4 waves would need 144 KB of LDS).
constexpr int mf_nw(int D) { return D == 256 ? 2 : 4; }
constexpr int MF_NST = 2;

template <int D, bool KV8>
hipError_t launch_mf(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    constexpr int NW = mf_nw(D);
    constexpr int NST = MF_NST;
    const int parts = p.partition ? (p.max_seq_len + p.partition - 1) / p.partition : 1;
    const dim3 grid(p.hkv, p.num_seqs, parts);
    const dim3 block(NW * 64);
    if (li)
        *li = LaunchInfo{{(int)grid.x, (int)grid.y, (int)grid.z}, (int)block.x,
                         {MfCfg<D, KV8, NW, NST>::CT, NW, NST}, 0};
    hipLaunchKernelGGL((decode_mfma_kernel<D, KV8, NW, NST>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <bool KV8>
hipError_t launch_mf_d(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    switch (p.head_dim) {
        case 64: return launch_mf<64, KV8>(p, stream, li);
        case 128: return launch_mf<128, KV8>(p, stream, li);
        case 256: return launch_mf<256, KV8>(p, stream, li);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_mfma_supported(const AttnParams &p) {
    return !p.per_token && p.dtype == 1 && p.group >= 1 &&
           p.group <= 8 && (p.head_dim == 64 || p.head_dim == 128 || p.head_dim == 256);
}

hipError_t launch_decode_mfma(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    return p.kv8 ? launch_mf_d<true>(p, stream, li) : launch_mf_d<false>(p, stream, li);
}

}  // namespace pa
