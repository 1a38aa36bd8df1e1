// reduce.hip -- merge of split-KV partials (vllm-metal kernel walkthrough, GQA
// decode tip 4: per-partition log2-space (max, exp-sum) statistics plus the
// normalised partial output, merged by one shared reducer).
//
// With n partitions for the token's position p (n = ceil((p+1)/P)):
// M = max_k m_k, w_k = l_k 2^(m_k - M), out = sum_k w_k o_k / sum_k w_k.
// Rows with n == 1 were finalised by the attention kernel and are skipped.
// Two launch shapes, both summing in a fixed order (deterministic):
//  * up to 16 partitions (prefill and mixed batches, decode up to 16*P
//    keys): one wave per (token, head) row, four rows per workgroup;
//  * more partitions (long decode): one workgroup per (token, head, 64-wide
//    slice of D), partitions spread over 16 lane groups (float4 per lane along
//    D), so a few very long rows still spread over many workgroups.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int RT = 256;      // threads per workgroup
constexpr int WCAP = 2048;   // partition weights kept in LDS
constexpr int ROWS_MAX_PARTS = 16;  // partitions per row up to which the row form is used

// Elements of D per workgroup: whole rows up to 128, 64-wide slices beyond.
template <int D>
constexpr int slice_of() { return D <= 128 ? D : 64; }

// grid = (total_q, Hq, D / slice): one workgroup per (token, head, slice of D)
template <typename T, int D>
__global__ __launch_bounds__(RT) void reduce_kernel(const ReduceParams p) {
    constexpr int DS = slice_of<D>();
    constexpr int LPG = DS / 4;   // lanes per partition group (float4 each)
    constexpr int KG = RT / LPG;  // partition groups
    __shared__ float wsh[WCAP];
    __shared__ float red[RT / 64];
    __shared__ float4 part_acc[KG][LPG];

    const int t = blockIdx.x;
    const int h = blockIdx.y;
    const int d0 = blockIdx.z * DS;
    const int tid = threadIdx.x;

    // owner request of token t: the r with cu[r] <= t < cu[r+1]
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.cu_q[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int q_len = p.cu_q[r + 1] - p.cu_q[r];
    const int pos = p.seq_lens[r] - q_len + (t - p.cu_q[r]);
    const int n = pos / p.partition + 1;
    if (n <= 1 || n > p.max_parts || pos < 0) return;

    const size_t srow = ((size_t)t * p.hq + h) * p.max_parts;
    const float *ml = p.max_logits + srow;
    const float *es = p.exp_sums + srow;

    // M = max_k m_k
    float mx = NEG_INF;
    for (int k = tid; k < n; k += RT) mx = fmaxf(mx, ml[k]);
    mx = group_max<64>(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < RT / 64; ++w) M = fmaxf(M, red[w]);
    // the head's sink joins the max and, once, the denominator (log2 units)
    const float s2 = p.sinks ? p.sinks[h] * LOG2E_F : NEG_INF;
    M = fmaxf(M, s2);
    __syncthreads();

    // w_k and their sum
    float ws = 0.f;
    for (int k = tid; k < n; k += RT) {
        const float w = es[k] * exp2_diff(ml[k], M);
        if (k < WCAP) wsh[k] = w;
        ws += w;
    }
    ws = group_sum<64>(ws);
    if ((tid & 63) == 0) red[tid >> 6] = ws;
    __syncthreads();
    float W = exp2_diff(s2, M);
#pragma unroll
    for (int w = 0; w < RT / 64; ++w) W += red[w];

    // sum_k w_k o_k over this slice, partitions spread over the groups
    const int kg = tid / LPG;
    const int d4 = tid % LPG;
    const float4 *o = reinterpret_cast<const float4 *>(p.tmp_out + srow * D + d0) + d4;
    float4 a = {0.f, 0.f, 0.f, 0.f};
    for (int k = kg; k < n; k += KG) {
        const float w = k < WCAP ? wsh[k] : es[k] * exp2_diff(ml[k], M);
        const float4 v = o[(size_t)k * (D / 4)];
        a.x = fmaf(w, v.x, a.x);
        a.y = fmaf(w, v.y, a.y);
        a.z = fmaf(w, v.z, a.z);
        a.w = fmaf(w, v.w, a.w);
    }
    part_acc[kg][d4] = a;
    __syncthreads();
    if (tid < LPG) {
        float4 s = part_acc[0][tid];
#pragma unroll
        for (int g = 1; g < KG; ++g) {
            const float4 v = part_acc[g][tid];
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        const float inv = 1.f / W;
        const size_t oi = ((size_t)t * p.hq + h) * D + d0 + tid * 4;
        if constexpr (sizeof(T) == 2) {
            uint2 pk;
            pk.x = pack_bf16(s.x * inv, s.y * inv);
            pk.y = pack_bf16(s.z * inv, s.w * inv);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.out) + oi) = pk;
        } else {
            float4 v = {s.x * inv, s.y * inv, s.z * inv, s.w * inv};
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.out) + oi) = v;
        }
    }
}

// One wave per (token, head) row, four rows per workgroup: for batches with
// many rows and at most 16 partitions per row (prefill and mixed batches),
// where a workgroup per row would be mostly launch overhead.  Lane k holds
// partition k's statistics; the partials are then accumulated in partition
// order, each lane owning D/64 consecutive elements of the row.
template <typename T, int D>
__global__ __launch_bounds__(256) void reduce_rows_kernel(const ReduceParams p) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // t * Hq + h
    if (row >= p.total_q * p.hq) return;
    const int t = row / p.hq;
    // owner request of token t (the last r with cu[r] <= t) and its lengths:
    // up to 64 requests in one round of loads, one request per lane
    int q_len, pos;
    if (p.num_seqs <= 64) {
        const bool in = lane < p.num_seqs;
        const int c0 = in ? p.cu_q[lane] : 0;
        const int c1 = in ? p.cu_q[lane + 1] : 0;
        const int sl = in ? p.seq_lens[lane] : 0;
        const uint64_t le = __ballot(in && c0 <= t);
        const int r = le ? 63 - __builtin_clzll(le) : 0;
        const int cr = __builtin_amdgcn_readlane(c0, r);
        q_len = __builtin_amdgcn_readlane(c1, r) - cr;
        pos = __builtin_amdgcn_readlane(sl, r) - q_len + (t - cr);
    } else {
        int lo = 0, hi = p.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.cu_q[mid] <= t) lo = mid; else hi = mid - 1;
        }
        q_len = p.cu_q[lo + 1] - p.cu_q[lo];
        pos = p.seq_lens[lo] - q_len + (t - p.cu_q[lo]);
    }
    const int n = pos / p.partition + 1;
    if (n <= 1 || n > p.max_parts || pos < 0 || n > ROWS_MAX_PARTS) return;

    // statistics and every partial of the row requested together
    const size_t srow = (size_t)row * p.max_parts;
    const float m = lane < n ? p.max_logits[srow + lane] : NEG_INF;
    const float es = lane < n ? p.exp_sums[srow + lane] : 0.f;
    const float *o = p.tmp_out + srow * D + lane * E;
    float v[ROWS_MAX_PARTS][E];
#pragma unroll
    for (int k = 0; k < ROWS_MAX_PARTS; ++k) {
        if (k < n) {
            if constexpr (E == 4) {
                const float4 x = *reinterpret_cast<const float4 *>(o + (size_t)k * D);
                v[k][0] = x.x; v[k][1] = x.y; v[k][2] = x.z; v[k][3] = x.w;
            } else if constexpr (E == 2) {
                const float2 x = *reinterpret_cast<const float2 *>(o + (size_t)k * D);
                v[k][0] = x.x; v[k][1] = x.y;
            } else {
                v[k][0] = o[(size_t)k * D];
            }
        }
    }
    // the head's sink joins the max and, once, the denominator (log2 units)
    const float s2 = p.sinks ? p.sinks[row % p.hq] * LOG2E_F : NEG_INF;
    const float M = fmaxf(group_max<64>(m), s2);
    const float w = lane < n ? es * exp2_diff(m, M) : 0.f;
    const float W = group_sum<64>(w) + exp2_diff(s2, M);

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int k = 0; k < ROWS_MAX_PARTS; ++k) {
        if (k < n) {
            const float wk = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(wk, v[k][e], acc[e]);
        }
    }
    const float inv = 1.f / W;
    const size_t oi = (size_t)row * D + lane * E;
    if constexpr (sizeof(T) == 2) {
        uint16_t *out = reinterpret_cast<uint16_t *>(p.out) + oi;
        if constexpr (E == 4) {
            uint2 pk;
            pk.x = pack_bf16(acc[0] * inv, acc[1] * inv);
            pk.y = pack_bf16(acc[2] * inv, acc[3] * inv);
            *reinterpret_cast<uint2 *>(out) = pk;
        } else if constexpr (E == 2) {
            *reinterpret_cast<uint32_t *>(out) = pack_bf16(acc[0] * inv, acc[1] * inv);
        } else {
            *out = (uint16_t)(pack_bf16(acc[0] * inv, 0.f) & 0xFFFFu);
        }
    } else {
        float *out = reinterpret_cast<float *>(p.out) + oi;
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = acc[e] * inv;
    }
}

template <typename T, int D>
hipError_t launch_td(const ReduceParams &p, hipStream_t stream, LaunchInfo *li) {
    // The row form serialises a row's partitions in one wave: right for many
    // rows with few partitions; a few long rows keep the slice form.
    if (p.max_parts <= ROWS_MAX_PARTS) {
        const int blocks = (int)(((int64_t)p.total_q * p.hq + 3) / 4);
        if (li) *li = LaunchInfo{{blocks, 1, 1}, 256, {0, 0, 0}, 0};
        hipLaunchKernelGGL((reduce_rows_kernel<T, D>), dim3(blocks), dim3(256), 0, stream, p);
    } else {
        const dim3 grid(p.total_q, p.hq, D / slice_of<D>());
        if (li) *li = LaunchInfo{{(int)grid.x, (int)grid.y, (int)grid.z}, RT, {0, 0, 0}, 1};
        hipLaunchKernelGGL((reduce_kernel<T, D>), grid, dim3(RT), 0, stream, p);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const ReduceParams &p, hipStream_t stream, LaunchInfo *li) {
    switch (p.head_dim) {
        case 64: return launch_td<T, 64>(p, stream, li);
        case 128: return launch_td<T, 128>(p, stream, li);
        case 256: return launch_td<T, 256>(p, stream, li);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_reduce(const ReduceParams &p, hipStream_t stream, LaunchInfo *li) {
    if (p.total_q == 0) return hipSuccess;
    return p.dtype == 1 ? launch_t<bf16_t>(p, stream, li) : launch_t<float>(p, stream, li);
}

}  // namespace pa
