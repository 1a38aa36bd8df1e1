// decode.hip -- paged GQA decode attention for gfx950 on the vector ALUs, for
// float32 batches: one workgroup per request (decode batches) or per query
// token (longer windows: every token's key range ends at its own causal
// position).  bf16 queries take the MFMA kernels (decode_rows.hip,
// decode_mfma.hip for decode batches, prefill.hip for longer windows).
//
// What it computes follows the vllm-metal kernel walkthrough ("What is Paged
// Attention"; GQA decode tips 1-4): softmax(q.k * scale) v over the keys of one
// request, read page by page through its block table, with all query heads of
// one GQA group served by the same workgroup so each K/V page is read from HBM
// once, the softmax kept online in registers in log2 space (exp2 only), and the
// key range optionally cut into 256/512-token partitions whose (max, exp-sum)
// statistics and normalised partial outputs are merged by the reduce kernel.
//
// The design is our own for CDNA4:
//  * grid = (partitions, kv_heads, requests); NW waves per workgroup take the
//    CT-token chunks of the partition round-robin, each wave with a private ring
//    of NST LDS stages, so no workgroup barrier is needed until the final merge;
//  * K/V rows move HBM -> LDS with gfx950's 16-byte global_load_lds_dwordx4,
//    fully coalesced (one wave instruction moves 1 KB), while the previous stage
//    is being consumed; vmcnt waits are explicit;
//  * the page-table walk is one wave-wide load of up to 64 entries per window,
//    then v_readlane per chunk (a scalar broadcast, no shuffles), and the DMA
//    base addresses are pure scalar arithmetic;
//  * a token's row is split over L lanes (32 bytes each: two 16-byte pieces);
//    QK^T is an fp32 FMA chain plus a DPP all-reduce over the L lanes;
//  * every lane keeps its own online-softmax state for its token subset; the
//    loop over a wave's full chunks has no data-dependent branch (only its
//    last chunk can hold the end of the range and is peeled off), so the
//    accumulators stay in their registers;
//  * at the end, every lane is rescaled to the wave-wide max and the lane
//    groups of the wave are summed in registers (DPP rotations inside each
//    16-lane row, then v_permlane16/32_swap across rows only as far as the
//    LDS merge area requires); the row states go to LDS and all threads of
//    the workgroup merge them.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// A lane's reference max m is only raised when a chunk's max exceeds it by
// more than this (log2 units); weights then stay below 2^RESCALE_THRESHOLD.
constexpr float RESCALE_THRESHOLD = 8.0f;


template <int D, int GT, int CT_, int NW_, int NST_>
struct DecodeCfg {
    static constexpr int CT = CT_;               // tokens per chunk (LDS stage)
    static constexpr int R = D * 4;              // bytes per Q/K/V row of one head
    static constexpr int L = R / 32;             // lanes per token (8 elements each)
    static constexpr int TPP = 64 / L;           // tokens per pass of the wave
    static constexpr int NP = CT / TPP;          // passes per chunk
    static constexpr int NI = CT * R / 1024;     // DMA instructions per chunk per tensor
    static constexpr int RPI = 1024 / R;         // rows moved by one DMA instruction
    static constexpr int SLOT = 2 * CT * R;      // bytes of one LDS stage (K rows, then V rows)
    static constexpr int NW = NW_;
    static constexpr int NST = NST_;
    static constexpr int VM_PER_CHUNK = 2 * NI;
    static constexpr int NE = 8;                 // elements per lane per row
    static constexpr int STATE_FLOATS = GT * D + 2 * GT;  // acc, then m, then l
    static constexpr int STAGE_BYTES = NW * NST * SLOT;
    // Merge states per wave: as many row states as fit in the staging LDS
    // (4 rows, or 2 halves when a token spans 32 lanes), else fewer after
    // merging rows in registers.
    static constexpr int ROWS = L <= 16 ? 4 : 2;  // lane groups of a wave (16- or 32-lane rows)
    static constexpr bool fits(int spw) { return NW * spw * STATE_FLOATS * 4 <= STAGE_BYTES; }
    static constexpr int SPW = fits(ROWS) ? ROWS : (fits(ROWS / 2) ? ROWS / 2 : 1);
    static constexpr int NS = NW * SPW;          // merge states of the workgroup
    static constexpr int MERGE_BYTES = NS * STATE_FLOATS * 4;
    static constexpr int LDS_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
    static_assert(L >= 8 && L <= 32, "row split");
    static_assert(NP >= 1 && CT % TPP == 0, "chunk covers whole passes");
    static_assert(NI >= 1 && RPI >= 1 && RPI <= 8 && CT * R % 1024 == 0, "dma shape");
    static_assert((NST - 1) * VM_PER_CHUNK < 64, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Element index (within the head's D) of word w of lane column c.
template <class C>
__device__ __forceinline__ int word_elem(int c, int w) {
    // two pieces per lane: piece i holds elements (i*L + c)*4 onward
    return ((w / 4) * C::L + c) * 4 + (w % 4);
}

// Wait until this wave's DMA for the chunk `ahead` chunks before the newest
// one has landed in LDS (vmcnt counts instructions and completes in order).
template <int VM, int MAXA>
__device__ __forceinline__ void wait_chunks_ahead(int ahead) {
    if constexpr (MAXA > 0) {
        if (ahead >= MAXA) {
            wait_vmcnt<MAXA * VM>();
            return;
        }
        wait_chunks_ahead<VM, MAXA - 1>(ahead);
    } else {
        wait_vmcnt<0>();
    }
}

// The lane's 8 fp32 words of a row: its two 16-byte pieces.
template <class C>
__device__ __forceinline__ void read_row_words(const char *lds_row, int c, uint32_t (&w)[8]) {
    const uint4 a = *reinterpret_cast<const uint4 *>(lds_row + c * 16);
    const uint4 b = *reinterpret_cast<const uint4 *>(lds_row + (C::L + c) * 16);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// Max over all 64 lanes of the wave.
__device__ __forceinline__ float wave_max(float x) {
    x = group_max<16>(x);
    const RowPair a = row_pair16(x);
    x = fmaxf(a.a, a.b);
    const RowPair b = row_pair32(x);
    return fmaxf(b.a, b.b);
}

// Sum of this lane's values with those of the lane the DPP row rotation CTRL
// brings in (same column, another lane group of the row).
template <int CTRL, int GT, int NE>
__device__ __forceinline__ void sum_rot(float (&l)[GT], float (&acc)[GT][NE]) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        l[g] += dpp<CTRL>(l[g]);
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[g][e] += dpp<CTRL>(acc[g][e]);
    }
}

// The same across the rows of the wave (rows 2i+1 onto 2i, or i+2 onto i).
template <bool X32, int GT, int NE>
__device__ __forceinline__ void sum_pairs(float (&l)[GT], float (&acc)[GT][NE]) {
    auto pair = [](float x) { return X32 ? row_pair32(x) : row_pair16(x); };
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        const RowPair pl = pair(l[g]);
        l[g] = pl.a + pl.b;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const RowPair pa = pair(acc[g][e]);
            acc[g][e] = pa.a + pa.b;
        }
    }
}

// One chunk staged in LDS: scores, online-softmax update and PV for this
// lane's tokens (the whole chunk is one softmax step).  MASKED is the chunk
// that holds the end of the key range: its tokens past the end get score -inf
// and their V rows (possibly NaN page tails) are replaced by zeros.  Only a
// wave's last chunk can be masked, so the loop over the others has no
// data-dependent branch at all (branches around the accumulators make the
// register allocator copy them on every iteration).
// getk(j, w) / getv(j, w) deliver the lane's 8 words of its token in pass j.
template <class C, int GT, bool MASKED, class GetK, class GetV>
__device__ __forceinline__ void chunk_step(GetK getk, GetV getv, int tip, int tok0, int tok_end,
                                           float scale_log2, const uint32_t (&qw)[GT][8],
                                           float (&m)[GT], float (&mtrue)[GT], float (&l)[GT],
                                           float (&accv)[GT][C::NE]) {
    constexpr int NE = C::NE;
    constexpr int NP = C::NP;
    // ---- scores of every pass ----
    float sc[NP][GT];
    bool valid[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const int t = j * C::TPP + tip;
        valid[j] = !MASKED || tok0 + t < tok_end;
        uint32_t kw[8];
        getk(j, kw);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float a = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w)
                a = fmaf(__uint_as_float(qw[g][w]), __uint_as_float(kw[w]), a);
            sc[j][g] = a;
        }
    }
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const float a = group_sum<C::L>(sc[j][g]) * scale_log2;
            sc[j][g] = (!MASKED || valid[j]) ? a : NEG_INF;
        }
    // ---- online softmax: new running max, rescale of l and acc ----
    // In an unmasked chunk every score is finite, so the new max is finite and
    // exp2 needs no -inf guard; the masked chunk guards both.
    if constexpr (!MASKED) {
        // Lazy: rescale (all lanes, uniformly) only when some lane's max grew
        // past its reference by more than the threshold.
        float mx[GT];
        bool up = false;
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            mx[g] = sc[0][g];
#pragma unroll
            for (int j = 1; j < NP; ++j) mx[g] = fmaxf(mx[g], sc[j][g]);
            up = up || mx[g] > m[g] + RESCALE_THRESHOLD;
            mtrue[g] = fmaxf(mtrue[g], mx[g]);
        }
        if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                const float mn = mx[g] > m[g] + RESCALE_THRESHOLD ? mx[g] : m[g];
                const float alpha = exp2_diff(m[g], mn);  // m = -inf before the first key
                m[g] = mn;
                l[g] *= alpha;
#pragma unroll
                for (int e = 0; e < NE; ++e) accv[g][e] *= alpha;
            }
        }
    } else {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float mx = sc[0][g];
#pragma unroll
            for (int j = 1; j < NP; ++j) mx = fmaxf(mx, sc[j][g]);
            const float mn = fmaxf(m[g], mx);
            const float alpha = MASKED ? exp2_diff(m[g], mn) : __builtin_amdgcn_exp2f(m[g] - mn);
            m[g] = mn;
            mtrue[g] = fmaxf(mtrue[g], mx);
            l[g] *= alpha;
#pragma unroll
            for (int e = 0; e < NE; ++e) accv[g][e] *= alpha;
        }
    }
    float pr[NP][GT];
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int g = 0; g < GT; ++g)
            pr[j][g] = (MASKED && sc[j][g] == NEG_INF) ? 0.f
                                                       : __builtin_amdgcn_exp2f(sc[j][g] - m[g]);

    // ---- PV ----
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        uint32_t vw[8];
        getv(j, vw);
        if (MASKED && !valid[j]) {
#pragma unroll
            for (int w = 0; w < 8; ++w) vw[w] = 0u;
        }
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            l[g] += pr[j][g];
#pragma unroll
            for (int w = 0; w < 8; ++w)
                accv[g][w] = fmaf(pr[j][g], __uint_as_float(vw[w]), accv[g][w]);
        }
    }
}

template <int D, int GT, int CT, int NW, int NST>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const AttnParams p) {
    using C = DecodeCfg<D, GT, CT, NW, NST>;
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];

    // Grid (hkv, rows, parts).  The KV heads of one partition are adjacent,
    // so the workgroups that run together read the same pages (all heads'
    // rows of a page are contiguous) rather than 1/Hkv of many different
    // pages.  Partitions are slowest and taken last-first: the last, often
    // partial, partitions of every request are dispatched first and the full
    // first partitions last, which shortens the tail.
    const int kvh = blockIdx.x;
    const int part = gridDim.z - 1 - blockIdx.z;
    const int zrow = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane % C::L;    // column of the row this lane holds
    const int tip = lane / C::L;  // token slot within a pass
    const int tok_begin = p.partition ? part * p.partition : 0;
    const int bs = p.block_size;
    const int lbs = p.log2_bs;
    const int c_begin = tok_begin / CT;
    const int ppc = bs < CT ? CT / bs : 1;  // pages per chunk: 1, or 2 for 8-token pages
    const int cpw = 64 / ppc;               // chunks covered by one block-table window

    // A workgroup serves one query token: request r's only token, or (per-token
    // launches) packed token `zrow`, whose keys end at its own causal position
    // ctx + j.
    int r = zrow, q0 = zrow;
    if (p.per_token) {
        int lo = 0, hi = p.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.cu_q[mid] <= q0) lo = mid; else hi = mid - 1;
        }
        r = lo;
    }

    // ---- this wave's block-table window: lane i holds page (i / cpw) of the
    // wave's chunk kw0 + i % cpw.  The load needs the request but not its
    // length (it is bounded by the table row), so it is in flight while the
    // lengths arrive. ----
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

    int seq_len;
    if (p.per_token) {
        const int q_len = p.cu_q[r + 1] - p.cu_q[r];
        seq_len = p.seq_lens[r] - q_len + (q0 - p.cu_q[r]) + 1;
    } else {
        q0 = p.cu_q[r];
        if (p.cu_q[r + 1] - q0 <= 0) return;
        seq_len = p.seq_lens[r];
    }
    if (tok_begin >= seq_len || seq_len <= 0) return;
    const int tok_end = p.partition ? min(seq_len, tok_begin + p.partition) : seq_len;
    const int nparts = p.partition ? (seq_len + p.partition - 1) / p.partition : 1;
    const int G = p.group;

    // ---- this wave's chunks ----
    const int c_end = (tok_end + CT - 1) / CT;
    const int nchunks = c_end - c_begin;
    const int nmy = nchunks > wave ? (nchunks - wave + NW - 1) / NW : 0;

    // ---- query registers: the lane's 8 words of each head of the group ----
    uint32_t qw[GT][8];
    {
        const char *qbase = reinterpret_cast<const char *>(p.q) +
                            ((size_t)q0 * p.hq + (size_t)kvh * G) * C::R;
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            if (g < G) {
                const uint4 a = *reinterpret_cast<const uint4 *>(qbase + g * C::R + c * 16);
                const uint4 b =
                    *reinterpret_cast<const uint4 *>(qbase + g * C::R + (C::L + c) * 16);
                qw[g][0] = a.x; qw[g][1] = a.y; qw[g][2] = a.z; qw[g][3] = a.w;
                qw[g][4] = b.x; qw[g][5] = b.y; qw[g][6] = b.z; qw[g][7] = b.w;
            } else {
#pragma unroll
                for (int w = 0; w < 8; ++w) qw[g][w] = 0u;
            }
        }
    }

    const uint32_t row_stride = (uint32_t)p.hkv * C::R;  // bytes between tokens of a page
    const char *kc = reinterpret_cast<const char *>(p.kc);
    const int64_t v_minus_k = reinterpret_cast<const char *>(p.vc) - kc;
    const uint64_t page_bytes = (uint64_t)bs * row_stride;
    const uint64_t head_off = (uint64_t)kvh * C::R;

    // ---- online softmax state (per lane, for its token subset) ----
    constexpr int NE = C::NE;
    float m[GT], mtrue[GT], l[GT];  // reference max, true max, exp-sum
    float accv[GT][NE];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        m[g] = NEG_INF;
        mtrue[g] = NEG_INF;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) accv[g][e] = 0.f;
    }
    const float scale_log2 = p.scale_log2;

    // Per-lane byte offsets of the rows this lane moves, relative to the row of
    // the chunk's first token (one per DMA instruction).
    uint32_t voff[C::NI];
#pragma unroll
    for (int ii = 0; ii < C::NI; ++ii) {
        const int row = ii * C::RPI + lane / (C::R / 16);
        const int piece = lane % (C::R / 16);
        voff[ii] = (uint32_t)row * row_stride + (uint32_t)piece * 16;
    }
    const uint32_t lds_wave = lds_addr(lds) + (uint32_t)(wave * NST * C::SLOT);

    // Issue the DMA of this wave's k-th chunk into stage s.  All address
    // arithmetic is on wave-uniform values.
    auto issue = [&](int k, int s) {
        if (k - win_base >= cpw) {  // slide the window (long unsplit ranges only)
            win_base = k;
            btv = load_window(k);
        }
        const int tok0 = (c_begin + wave + k * NW) * CT;
        const int idx = k - win_base;
        const int phys0 = __builtin_amdgcn_readlane(btv, idx);
        const uint64_t off0 = (uint64_t)phys0 * page_bytes +
                              (uint64_t)(tok0 & (bs - 1)) * row_stride + head_off;
        uint64_t off1 = off0;
        if (ppc == 2) {
            // rows 8..15 of the chunk live in the next page; past the sequence
            // those rows are masked, so page 0 is re-read instead.
            const int phys1 =
                tok0 + 8 < seq_len ? __builtin_amdgcn_readlane(btv, idx + cpw) : phys0;
            off1 = (uint64_t)phys1 * page_bytes + head_off - 8ull * row_stride;
        }
        const char *kb0 = kc + off0;
        const char *kb1 = kc + off1;
        const uint32_t ldsk = lds_wave + (uint32_t)(s * C::SLOT);
        const uint32_t ldsv = ldsk + CT * C::R;
#pragma unroll
        for (int ii = 0; ii < C::NI; ++ii)
            dma16(ii * C::RPI >= 8 ? kb1 : kb0, voff[ii], ldsk + ii * 1024);
#pragma unroll
        for (int ii = 0; ii < C::NI; ++ii)
            dma16((ii * C::RPI >= 8 ? kb1 : kb0) + v_minus_k, voff[ii], ldsv + ii * 1024);
    };

#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nmy) issue(s, s);

    // Every chunk but the wave's last is full: a branch-free loop over them,
    // then the last one, the only one that can hold the end of the range.
    auto stage = [&](int k, const char *&kst, const char *&vst) {
        if (k + NST - 1 < nmy) issue(k + NST - 1, (k + NST - 1) % NST);
        wait_chunks_ahead<C::VM_PER_CHUNK, NST - 1>(min(NST - 1, nmy - 1 - k));
        kst = lds + (wave * NST + k % NST) * C::SLOT;
        vst = kst + CT * C::R;
    };
    auto lds_rows = [&](const char *st) {
        return [=](int j, uint32_t (&w)[8]) { read_row_words<C>(st + (j * C::TPP + tip) * C::R, c, w); };
    };
    for (int k = 0; k < nmy - 1; ++k) {
        const char *kst, *vst;
        stage(k, kst, vst);
        chunk_step<C, GT, false>(lds_rows(kst), lds_rows(vst), tip, 0, 0, scale_log2, qw, m,
                                 mtrue, l, accv);
    }
    if (nmy > 0) {
        const char *kst, *vst;
        stage(nmy - 1, kst, vst);
        const int tok0 = (c_begin + wave + (nmy - 1) * NW) * CT;
        chunk_step<C, GT, true>(lds_rows(kst), lds_rows(vst), tip, tok0, tok_end, scale_log2, qw,
                                m, mtrue, l, accv);
    }

    // ---- merge the wave's lane groups: rescale every lane to the wave-wide
    // true max, after which merging is a plain sum (DPP rotation inside each
    // 16-lane row, then v_permlane16/32_swap across rows) ----
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        const float M = wave_max(mtrue[g]);
        const float f = exp2_diff(m[g], M);
        m[g] = M;
        l[g] *= f;
#pragma unroll
        for (int e = 0; e < NE; ++e) accv[g][e] *= f;
    }
    if constexpr (C::L == 8) {
        sum_rot<0x128, GT, NE>(l, accv);  // row_ror:8
    } else if constexpr (C::L == 4) {
        sum_rot<0x128, GT, NE>(l, accv);  // row_ror:8
        sum_rot<0x124, GT, NE>(l, accv);  // row_ror:4
    }
    // rows i and i+2 onto one state, then rows 2i and 2i+1, as LDS requires
    if constexpr (C::SPW * 2 <= C::ROWS) sum_pairs<true, GT, NE>(l, accv);
    if constexpr (C::ROWS == 4 && C::SPW == 1) sum_pairs<false, GT, NE>(l, accv);

    // ---- one state per wave to LDS, then all threads merge the waves ----
    __syncthreads();  // every wave is done with its stages
    float *mrg = reinterpret_cast<float *>(lds);
    {
        // state of lane group `row`: 16-lane rows (32-lane halves when L = 32)
        const int row = C::L <= 16 ? lane / 16 : lane / 32;
        float *st = mrg + (wave * C::SPW + row) * C::STATE_FLOATS;
        const bool writer = row < C::SPW && (C::L <= 16 ? lane % 16 : lane % 32) < C::L;
        if (writer) {
#pragma unroll
            for (int g = 0; g < GT; ++g)
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    st[g * D + word_elem<C>(c, w)] = accv[g][w];
                }
        }
        if (writer && c == 0) {
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                st[GT * D + g] = m[g];
                st[GT * D + GT + g] = l[g];
            }
        }
    }
    __syncthreads();

    const bool direct = nparts <= 1;
    for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
        const int g = idx / D;
        const int d = idx - g * D;
        // m of each wave is the exact running max of its scores (log2 units)
        float M = NEG_INF;
#pragma unroll
        for (int s = 0; s < C::NS; ++s) M = fmaxf(M, mrg[s * C::STATE_FLOATS + GT * D + g]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
            const float *st = mrg + s * C::STATE_FLOATS;
            const float f = exp2_diff(st[GT * D + g], M);
            num += st[g * D + d] * f;
            den += st[GT * D + GT + g] * f;
        }
        const int h = kvh * G + g;
        float o = num / den;
        if (direct && p.sinks) {
            // the head's sink: one more denominator term, no value (log2 units)
            const float s2 = p.sinks[h] * LOG2E_F;
            const float Mx = fmaxf(M, s2);
            const float a = exp2_diff(M, Mx);
            o = num * a / (den * a + exp2_diff(s2, Mx));
        }
        if (direct) {
            const size_t oi = ((size_t)q0 * p.hq + h) * D + d;
            reinterpret_cast<float *>(p.out)[oi] = o;
        } else {
            const size_t si = ((size_t)q0 * p.hq + h) * p.max_parts + part;
            p.tmp_out[si * D + d] = o;
            if (d == 0) {
                p.max_logits[si] = M;
                p.exp_sums[si] = den;
            }
        }
    }
}

// Chunk tokens and waves per workgroup by K/V row bytes (D = 64 -> 256 B,
// 128 -> 512 B, 256 -> 1 KB), two LDS stages per wave.
constexpr int decode_ct(int R) { return R >= 512 ? 8 : 16; }
constexpr int decode_nw(int R) { return R >= 1024 ? 2 : 4; }
constexpr int DECODE_NST = 2;

template <int D, int GT>
hipError_t launch_t(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    constexpr int CT = decode_ct(4 * D), NW = decode_nw(4 * D);
    const int parts = p.partition ? (p.max_seq_len + p.partition - 1) / p.partition : 1;
    const int rows = p.per_token ? p.total_q : p.num_seqs;
    const dim3 grid(p.hkv, rows, parts);
    dim3 block(NW * 64);
    if (li) *li = LaunchInfo{{(int)grid.x, (int)grid.y, (int)grid.z}, (int)block.x,
                             {CT, NW, DECODE_NST}, 0};
    hipLaunchKernelGGL((decode_kernel<D, GT, CT, NW, DECODE_NST>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    switch (p.group) {
        case 1: return launch_t<D, 1>(p, stream, li);
        case 2: return launch_t<D, 2>(p, stream, li);
        case 3:
        case 4: return launch_t<D, 4>(p, stream, li);
        case 5:
        case 6: return launch_t<D, 6>(p, stream, li);
        case 7:
        case 8: return launch_t<D, 8>(p, stream, li);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_supported(int dtype, int head_dim, int group) {
    return (dtype == 0 || dtype == 1) && (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
           group >= 1 && group <= 8;
}

bool decode_kv8_supported(int head_dim, int group) { return decode_supported(1, head_dim, group); }

// Routing of the decode path: bf16 queries (bf16 or 8-bit caches) to the MFMA
// kernels, float32 batches to the vector-ALU kernel above.
hipError_t launch_decode(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    if (p.dtype == 1) {
        if (decode_rows_supported(p)) return launch_decode_rows(p, stream, li);
        if (decode_mfma_supported(p)) return launch_decode_mfma(p, stream, li);
        return hipErrorInvalidValue;
    }
    if (p.kv8) return hipErrorInvalidValue;
    switch (p.head_dim) {
        case 64: return launch_d<64>(p, stream, li);
        case 128: return launch_d<128>(p, stream, li);
        case 256: return launch_d<256>(p, stream, li);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
