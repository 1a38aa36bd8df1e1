// decode.hip -- paged GQA decode attention for gfx950 (one query token per request).
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
//    16-token chunks of the partition round-robin, each with a private ring of
//    NST LDS stages, so no workgroup barrier is needed until the final merge;
//  * K/V rows move HBM -> LDS with gfx950's 16-byte global_load_lds_dwordx4,
//    fully coalesced (one wave instruction moves 1 KB), while the previous stage
//    is being consumed; vmcnt waits are explicit;
//  * the page-table walk is one wave-wide load of up to 64 entries per window,
//    then v_readlane per chunk (a scalar broadcast, no shuffles);
//  * a token's row is split over L lanes (32 bytes each); QK^T uses
//    v_dot2c_f32_bf16 on bf16 pairs and a DPP all-reduce over the L lanes;
//  * every lane keeps its own online-softmax state for its token subset; the
//    running max is only moved when a score exceeds it by more than 2^8
//    (the result is exact whatever reference max is used, since the partial
//    sum and the accumulator share it);
//  * PV pairs two tokens per lane: p is packed to bf16 pairs and V is
//    interleaved with v_perm_b32 so one v_dot2c does two multiply-adds;
//  * lane groups and waves are merged once at the end (bpermute, then LDS).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units: p may reach 2^8 before rescaling

template <typename T, int D, int GT, int NW_, int NST_>
struct DecodeCfg {
    static constexpr bool BF16 = sizeof(T) == 2;
    static constexpr int ELT = sizeof(T);
    static constexpr int R = D * ELT;            // bytes per K/V row of one head
    static constexpr int L = R / 32;             // lanes per token (32 bytes each)
    static constexpr int TPP = 64 / L;           // tokens per pass of the wave
    static constexpr int NP = CHUNK / TPP;       // passes per 16-token chunk
    static constexpr int EPW = 4 / ELT;          // elements per 32-bit word
    static constexpr int NI = CHUNK * R / 1024;  // DMA instructions per chunk per tensor
    static constexpr int RPI = 1024 / R;         // rows moved by one DMA instruction
    static constexpr int SLOT = 2 * CHUNK * R;   // bytes of one LDS stage (K rows, then V rows)
    static constexpr int NW = NW_;
    static constexpr int NST = NST_;
    static constexpr int VM_PER_CHUNK = 2 * NI;
    // softmax unit: passes handled per online-softmax update
    static constexpr int SU = (BF16 && NP >= 2) ? 2 : 1;
    static constexpr int STAGE_BYTES = NW * NST * SLOT;
    static constexpr int MERGE_BYTES = NW * (GT * D + 3 * GT) * 4;
    static constexpr int LDS_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
    static_assert(L >= 4 && L <= 32, "row split");
    static_assert(NI >= 1 && RPI >= 1 && CHUNK * R % 1024 == 0, "dma shape");
    static_assert((NST - 1) * VM_PER_CHUNK < 64, "vmcnt range");
    static_assert(NP % SU == 0, "pass pairing");
};

// Element index (within the head's D) of word w of lane column c.
template <class C>
__device__ __forceinline__ int word_elem(int c, int w) {
    // two 16-byte pieces per lane: piece i at byte (i*L + c)*16 of the row
    return ((w / 4) * C::L + c) * (16 / C::ELT) + (w % 4) * C::EPW;
}

template <class C>
__device__ __forceinline__ void read_row_words(const char *lds_row, int c, uint32_t (&w)[8]) {
    const uint4 a = *reinterpret_cast<const uint4 *>(lds_row + c * 16);
    const uint4 b = *reinterpret_cast<const uint4 *>(lds_row + (C::L + c) * 16);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

template <typename T, int D, int GT, int NW, int NST>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const AttnParams p) {
    using C = DecodeCfg<T, D, GT, NW, NST>;
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];

    const int r = blockIdx.z;
    const int kvh = blockIdx.y;
    const int part = blockIdx.x;
    const int q0 = p.cu_q[r];
    if (p.cu_q[r + 1] - q0 <= 0) return;
    const int seq_len = p.seq_lens[r];
    const int tok_begin = p.partition ? part * p.partition : 0;
    if (tok_begin >= seq_len || seq_len <= 0) return;
    const int tok_end = p.partition ? min(seq_len, tok_begin + p.partition) : seq_len;
    const int nparts = p.partition ? (seq_len + p.partition - 1) / p.partition : 1;
    const int G = p.group;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane % C::L;    // column of the row this lane holds
    const int tip = lane / C::L;  // token slot within a pass

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

    // ---- this wave's chunks ----
    const int bs = p.block_size;
    const int lbs = p.log2_bs;
    const int c_begin = tok_begin / CHUNK;
    const int c_end = (tok_end + CHUNK - 1) / CHUNK;
    const int nchunks = c_end - c_begin;
    const int nmy = nchunks > wave ? (nchunks - wave + NW - 1) / NW : 0;
    const int seq_pages = (seq_len + bs - 1) >> lbs;
    const int ppc = bs < CHUNK ? 2 : 1;  // pages per chunk (block_size 8 -> 2)
    const int cpw = 64 / ppc;            // chunks covered by one block-table window
    const int32_t *bt_row = p.bt + (size_t)r * p.bt_stride;

    // Window of block-table entries: lane i holds the page of this wave's
    // chunk (kw0 + i % cpw), half i / cpw of it.
    auto load_window = [&](int kw0) -> int {
        const int k = kw0 + lane % cpw;
        const int ch = c_begin + wave + k * NW;
        const int lp = ((ch * CHUNK) >> lbs) + lane / cpw;
        int v = 0;
        if (k < nmy && lp < seq_pages) v = bt_row[lp];
        v = v < 0 ? 0 : (v >= p.num_blocks ? p.num_blocks - 1 : v);
        return v;
    };

    // Per-lane byte offsets of the rows this lane moves, relative to the row of
    // the chunk's first token (one per DMA instruction).
    const uint32_t row_stride = (uint32_t)p.hkv * C::R;  // bytes between tokens of a page
    uint32_t voff[C::NI];
#pragma unroll
    for (int ii = 0; ii < C::NI; ++ii) {
        const int row = ii * C::RPI + lane / (C::R / 16);
        const int piece = lane % (C::R / 16);
        voff[ii] = (uint32_t)row * row_stride + (uint32_t)piece * 16u;
    }

    const uint32_t lds_wave = lds_addr(lds) + (uint32_t)(wave * NST * C::SLOT);
    const char *kc = reinterpret_cast<const char *>(p.kc);
    const char *vc = reinterpret_cast<const char *>(p.vc);
    const size_t head_off = (size_t)kvh * C::R;

    int win_base = 0;
    int btv = load_window(0);

    // Issue the DMA of this wave's k-th chunk into stage s.
    auto issue = [&](int k, int s) {
        if (k - win_base >= cpw) {  // slide the window (only for long unsplit ranges)
            win_base = k;
            btv = load_window(k);
        }
        const int ch = c_begin + wave + k * NW;
        const int tok0 = ch * CHUNK;
        const int idx = k - win_base;
        const int phys0 = __builtin_amdgcn_readlane(btv, idx);
        const int off0 = tok0 & (bs - 1);
        const size_t row0 = ((size_t)phys0 * bs + off0) * p.hkv;
        const char *kb0 = kc + row0 * C::R + head_off;
        const char *vb0 = vc + row0 * C::R + head_off;
        const char *kb1 = kb0;
        const char *vb1 = vb0;
        if (ppc == 2) {
            // rows 8..15 of the chunk live in the next page; when that page is
            // past the sequence its rows are masked, so re-read page 0 instead.
            int phys1 = phys0;
            if (tok0 + 8 < seq_len) phys1 = __builtin_amdgcn_readlane(btv, idx + cpw);
            const size_t row1 = ((size_t)phys1 * bs) * p.hkv;
            kb1 = kc + row1 * C::R + head_off - (size_t)8 * row_stride;
            vb1 = vc + row1 * C::R + head_off - (size_t)8 * row_stride;
        }
        const uint32_t ldsk = lds_wave + (uint32_t)(s * C::SLOT);
        const uint32_t ldsv = ldsk + CHUNK * C::R;
#pragma unroll
        for (int ii = 0; ii < C::NI; ++ii) {
            const bool hi = ii * C::RPI >= 8;
            dma16(hi ? kb1 : kb0, voff[ii], ldsk + ii * 1024);
        }
#pragma unroll
        for (int ii = 0; ii < C::NI; ++ii) {
            const bool hi = ii * C::RPI >= 8;
            dma16(hi ? vb1 : vb0, voff[ii], ldsv + ii * 1024);
        }
    };

    // ---- online softmax state (per lane, for its token subset) ----
    float m[GT], mt[GT], l[GT];
    constexpr int NE = 32 / C::ELT;  // elements per lane per row
    float accv[GT][NE];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        m[g] = NEG_INF;
        mt[g] = NEG_INF;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) accv[g][e] = 0.f;
    }

    // prologue
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nmy) issue(s, s);

    for (int k = 0; k < nmy; ++k) {
        const int s = k % NST;
        if (k + NST - 1 < nmy) issue(k + NST - 1, (k + NST - 1) % NST);
        // chunks issued after k that may stay in flight
        const int ahead = min(NST - 1, nmy - 1 - k);
        if constexpr (NST >= 3) {
            if (ahead >= 2) wait_vmcnt<2 * C::VM_PER_CHUNK>();
            else if (ahead == 1) wait_vmcnt<C::VM_PER_CHUNK>();
            else wait_vmcnt<0>();
        } else {
            if (ahead >= 1) wait_vmcnt<C::VM_PER_CHUNK>();
            else wait_vmcnt<0>();
        }

        const int ch = c_begin + wave + k * NW;
        const int tok0 = ch * CHUNK;
        const bool partial = tok0 + CHUNK > tok_end;
        const char *kst = lds + (wave * NST + s) * C::SLOT;
        const char *vst = kst + CHUNK * C::R;

#pragma unroll
        for (int u = 0; u < C::NP; u += C::SU) {
            float sc[C::SU][GT];
            bool valid[C::SU];
            // ---- scores ----
#pragma unroll
            for (int j = 0; j < C::SU; ++j) {
                const int t = (u + j) * C::TPP + tip;
                valid[j] = tok0 + t < tok_end;
                uint32_t kw[8];
                read_row_words<C>(kst + t * C::R, c, kw);
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    float a = 0.f;
                    if constexpr (C::BF16) {
#pragma unroll
                        for (int w = 0; w < 8; ++w) a = dot2(qw[g][w], kw[w], a);
                    } else {
#pragma unroll
                        for (int w = 0; w < 8; ++w)
                            a = fmaf(__uint_as_float(qw[g][w]), __uint_as_float(kw[w]), a);
                    }
                    sc[j][g] = a;
                }
            }
#pragma unroll
            for (int j = 0; j < C::SU; ++j)
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    const float a = group_sum<C::L>(sc[j][g]) * p.scale_log2;
                    sc[j][g] = valid[j] ? a : NEG_INF;
                }
            // ---- online softmax with lazy rescale ----
            float mx[GT];
            bool need = false;
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                mx[g] = sc[0][g];
#pragma unroll
                for (int j = 1; j < C::SU; ++j) mx[g] = fmaxf(mx[g], sc[j][g]);
                mt[g] = fmaxf(mt[g], mx[g]);
                need |= mx[g] > m[g] + RESCALE_THRESHOLD;
            }
            if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    if (mx[g] > m[g] + RESCALE_THRESHOLD) {
                        const float alpha = exp2_diff(m[g], mx[g]);
                        m[g] = mx[g];
                        l[g] *= alpha;
#pragma unroll
                        for (int e = 0; e < NE; ++e) accv[g][e] *= alpha;
                    }
                }
            }
            float pr[C::SU][GT];
#pragma unroll
            for (int j = 0; j < C::SU; ++j)
#pragma unroll
                for (int g = 0; g < GT; ++g)
                    pr[j][g] = sc[j][g] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(sc[j][g] - m[g]);

            // ---- PV ----
            uint32_t vw[C::SU][8];
#pragma unroll
            for (int j = 0; j < C::SU; ++j) {
                const int t = (u + j) * C::TPP + tip;
                read_row_words<C>(vst + t * C::R, c, vw[j]);
                if (partial && !valid[j]) {
#pragma unroll
                    for (int w = 0; w < 8; ++w) vw[j][w] = 0u;  // page tail may hold NaN
                }
            }
            if constexpr (C::BF16 && C::SU == 2) {
                uint32_t pk[GT];
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    pk[g] = pack_bf16(pr[0][g], pr[1][g]);
                    l[g] += bf16lo(pk[g]) + bf16hi(pk[g]);  // the weights actually applied
                }
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    const uint32_t lo = perm(vw[1][w], vw[0][w], 0x05040100u);
                    const uint32_t hi = perm(vw[1][w], vw[0][w], 0x07060302u);
#pragma unroll
                    for (int g = 0; g < GT; ++g) {
                        accv[g][2 * w] = dot2(pk[g], lo, accv[g][2 * w]);
                        accv[g][2 * w + 1] = dot2(pk[g], hi, accv[g][2 * w + 1]);
                    }
                }
            } else if constexpr (C::BF16) {
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    const float pb = bf16hi(pack_bf16(0.f, pr[0][g]));
                    l[g] += pb;
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        accv[g][2 * w] = fmaf(pb, bf16lo(vw[0][w]), accv[g][2 * w]);
                        accv[g][2 * w + 1] = fmaf(pb, bf16hi(vw[0][w]), accv[g][2 * w + 1]);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < C::SU; ++j)
#pragma unroll
                    for (int g = 0; g < GT; ++g) {
                        l[g] += pr[j][g];
#pragma unroll
                        for (int w = 0; w < 8; ++w)
                            accv[g][w] = fmaf(pr[j][g], __uint_as_float(vw[j][w]), accv[g][w]);
                    }
            }
        }
    }

    // ---- merge the lane groups of this wave (lanes with the same column) ----
#pragma unroll
    for (int off = C::L; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const float mo = __shfl_xor(m[g], off);
            const float lo = __shfl_xor(l[g], off);
            mt[g] = fmaxf(mt[g], __shfl_xor(mt[g], off));
            const float M = fmaxf(m[g], mo);
            const float fa = exp2_diff(m[g], M);
            const float fb = exp2_diff(mo, M);
            l[g] = l[g] * fa + lo * fb;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const float ao = __shfl_xor(accv[g][e], off);
                accv[g][e] = accv[g][e] * fa + ao * fb;
            }
            m[g] = M;
        }
    }

    // ---- merge the waves through LDS ----
    __syncthreads();  // every wave is done with its stages
    float *mrg = reinterpret_cast<float *>(lds);
    float *macc = mrg + wave * (GT * D + 3 * GT);
    if (tip == 0) {
#pragma unroll
        for (int g = 0; g < GT; ++g)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int d = word_elem<C>(c, w);
                if constexpr (C::BF16) {
                    macc[g * D + d] = accv[g][2 * w];
                    macc[g * D + d + 1] = accv[g][2 * w + 1];
                } else {
                    macc[g * D + d] = accv[g][w];
                }
            }
        if (c == 0) {
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                macc[GT * D + g] = m[g];
                macc[GT * D + GT + g] = mt[g];
                macc[GT * D + 2 * GT + g] = l[g];
            }
        }
    }
    __syncthreads();

    const bool direct = nparts <= 1;
    for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
        const int g = idx / D;
        const int d = idx - g * D;
        float M = NEG_INF, Mt = NEG_INF;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float *ws = mrg + w * (GT * D + 3 * GT) + GT * D;
            M = fmaxf(M, ws[g]);
            Mt = fmaxf(Mt, ws[GT + g]);
        }
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float *wb = mrg + w * (GT * D + 3 * GT);
            const float f = exp2_diff(wb[GT * D + g], M);
            num += wb[g * D + d] * f;
            den += wb[GT * D + 2 * GT + g] * f;
        }
        const float o = num / den;
        const int h = kvh * G + g;
        if (direct) {
            const size_t oi = ((size_t)q0 * p.hq + h) * D + d;
            if constexpr (C::BF16)
                reinterpret_cast<uint16_t *>(p.out)[oi] = to_bf16(o);
            else
                reinterpret_cast<float *>(p.out)[oi] = o;
        } else {
            const size_t si = ((size_t)q0 * p.hq + h) * p.max_parts + part;
            p.tmp_out[si * D + d] = o;
            if (d == 0) {
                p.max_logits[si] = Mt;
                p.exp_sums[si] = den * exp2_diff(M, Mt);
            }
        }
    }
}

template <typename T, int D, int GT>
struct DecodeTuning {
    // stages and waves per workgroup by row size
    static constexpr int R = D * (int)sizeof(T);
    static constexpr int NW = R >= 1024 ? 2 : 4;
    static constexpr int NST = 2;
};

template <typename T, int D, int GT>
hipError_t launch_t(const AttnParams &p, hipStream_t stream) {
    using Tn = DecodeTuning<T, D, GT>;
    const int parts = p.partition ? (p.max_seq_len + p.partition - 1) / p.partition : 1;
    dim3 grid(parts, p.hkv, p.num_seqs);
    dim3 block(Tn::NW * 64);
    hipLaunchKernelGGL((decode_kernel<T, D, GT, Tn::NW, Tn::NST>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const AttnParams &p, hipStream_t stream) {
    switch (p.group) {
        case 1: return launch_t<T, D, 1>(p, stream);
        case 2: return launch_t<T, D, 2>(p, stream);
        case 3:
        case 4: return launch_t<T, D, 4>(p, stream);
        case 5:
        case 6: return launch_t<T, D, 6>(p, stream);
        case 7:
        case 8: return launch_t<T, D, 8>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_dt(const AttnParams &p, hipStream_t stream) {
    switch (p.head_dim) {
        case 64: return launch_d<T, 64>(p, stream);
        case 128: return launch_d<T, 128>(p, stream);
        case 256: return launch_d<T, 256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_supported(int dtype, int head_dim, int group) {
    return (dtype == 0 || dtype == 1) && (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
           group >= 1 && group <= 8;
}

hipError_t launch_decode(const AttnParams &p, hipStream_t stream) {
    if (p.dtype == 1) return launch_dt<bf16_t>(p, stream);
    return launch_dt<float>(p, stream);
}

}  // namespace pa
