// cache_write.hip -- reshape_and_cache and the kernel-page view of block tables.
//
// reshape_and_cache (vllm-metal kernel walkthrough, "three Metal kernels")
// scatters each new token's K and V rows into its cache slot.  With the cache
// laid out [num_blocks, block_size, Hkv, D], slot s = block*block_size + offset
// starts at byte s * (Hkv*D*elt) in every page-size view, so the copy needs no
// division.  Each thread moves one 16-byte piece of K and the same piece of V;
// consecutive threads cover consecutive bytes of a row, so reads and writes are
// fully coalesced 128-bit accesses.  Slots outside the pool are ignored rather
// than written.
//
// The 8-bit form (the library's own E4M3 scheme; the pages name KV
// quantisation kernels without giving one) stores each element of KV head g
// as the E4M3 code of the correctly rounded float32 quotient x / scale[g]:
// nearest code, ties to an even mantissa, saturating at 448, NaN to 0x7F.
// Each thread turns EPT elements of one head into one EPT-byte store: 16 for
// large writes (16-byte loads and stores), 4 for smaller ones (decode and
// mixed batches), whose time is the latency of the correctly rounded
// divisions, which four times the threads then share.
//
// expand_block_tables (unified-memory article, section six) rewrites a table of
// large cache blocks into the equivalent table of kernel pages: block b of
// `ratio` pages becomes pages ratio*b .. ratio*b + ratio-1.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4 *__restrict__ key, const uint4 *__restrict__ value, uint4 *__restrict__ kc,
    uint4 *__restrict__ vc, const int64_t *__restrict__ slots, int32_t num_tokens,
    int32_t pieces_per_row, int64_t num_slots) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t t = i / pieces_per_row;
    const int32_t c = (int32_t)(i - t * pieces_per_row);
    if (t >= num_tokens) return;
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots) return;
    const uint4 k = key[t * pieces_per_row + c];
    const uint4 v = value[t * pieces_per_row + c];
    kc[s * pieces_per_row + c] = k;
    vc[s * pieces_per_row + c] = v;
}

// E4M3 code of y: round to nearest, ties to even; |y| >= 448 and infinities
// saturate to +-448 (0x7E); NaN gives 0x7F; the sign of zero is kept.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t b = __float_as_uint(y);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;
    if (a >= 0x43e00000u) return sign | 0x7eu;  // 448 = 1.75 * 2^8
    if (a < 0x3c800000u) {
        // below 2^-6: the codes are the multiples of 2^-9 (code 8 = 2^-6 is
        // the smallest normal), so scale and round to an integer, ties to even
        return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    // normal range: keep 3 of the 23 mantissa bits, rounding to nearest even
    // (a carry moves into the exponent), then rebias the exponent 127 -> 7
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));
}

// N consecutive elements (bf16 or float32) as floats.
template <bool F32, int N>
__device__ __forceinline__ void load_n(const void *src, float (&f)[N]) {
    if constexpr (F32) {
#pragma unroll
        for (int j = 0; j < N / 4; ++j) {
            const float4 v = reinterpret_cast<const float4 *>(src)[j];
            f[4 * j] = v.x; f[4 * j + 1] = v.y; f[4 * j + 2] = v.z; f[4 * j + 3] = v.w;
        }
    } else if constexpr (N == 4) {
        const uint2 v = *reinterpret_cast<const uint2 *>(src);
        f[0] = bf16lo(v.x); f[1] = bf16hi(v.x); f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
    } else {
#pragma unroll
        for (int j = 0; j < N / 8; ++j) {
            const uint4 v = reinterpret_cast<const uint4 *>(src)[j];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                f[8 * j + 2 * k] = bf16lo(w[k]);
                f[8 * j + 2 * k + 1] = bf16hi(w[k]);
            }
        }
    }
}

// EPT codes packed little-endian into EPT / 4 words.
template <bool F32, int EPT>
struct Codes {
    uint32_t w[EPT / 4];
};
template <bool F32, int EPT>
__device__ __forceinline__ Codes<F32, EPT> quantize_n(const void *src, float scale) {
    float f[EPT];
    load_n<F32, EPT>(src, f);
    Codes<F32, EPT> c;
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
        uint32_t x = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) x |= e4m3_code(f[4 * j + k] / scale) << (8 * k);
        c.w[j] = x;
    }
    return c;
}

template <bool F32, int EPT>
__device__ __forceinline__ void store_codes(char *dst, const Codes<F32, EPT> &c) {
    if constexpr (EPT == 4)
        *reinterpret_cast<uint32_t *>(dst) = c.w[0];
    else
        *reinterpret_cast<uint4 *>(dst) = make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
}

template <bool F32, int EPT>
__global__ __launch_bounds__(256) void quantize_cache_kernel(
    const char *__restrict__ key, const char *__restrict__ value, char *__restrict__ kc,
    char *__restrict__ vc, const int64_t *__restrict__ slots, const float *__restrict__ k_scale,
    const float *__restrict__ v_scale, int32_t num_tokens, int32_t pieces_per_row,
    int32_t head_dim, int64_t num_slots) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t t = i / pieces_per_row;
    const int32_t c = (int32_t)(i - t * pieces_per_row);
    if (t >= num_tokens) return;
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots) return;
    const int32_t h = (c * EPT) / head_dim;  // EPT elements never straddle two heads
    const size_t src = ((size_t)t * pieces_per_row + c) * EPT * (F32 ? 4 : 2);
    const size_t dst = ((size_t)s * pieces_per_row + c) * EPT;
    store_codes<F32, EPT>(kc + dst, quantize_n<F32, EPT>(key + src, k_scale[h]));
    store_codes<F32, EPT>(vc + dst, quantize_n<F32, EPT>(value + src, v_scale[h]));
}

__global__ __launch_bounds__(256) void expand_block_tables_kernel(
    int32_t *__restrict__ dst, const int32_t *__restrict__ src, int32_t num_seqs,
    int32_t src_stride, int32_t src_blocks, int32_t dst_stride, int32_t ratio) {
    const int32_t r = blockIdx.y;
    const int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= num_seqs || j >= src_blocks * ratio) return;
    const int32_t b = j / ratio;
    const int32_t v = src[(size_t)r * src_stride + b];
    dst[(size_t)r * dst_stride + j] = v < 0 ? -1 : v * ratio + (j - b * ratio);
}

}  // namespace

hipError_t launch_reshape_and_cache(const void *key, const void *value, void *kc, void *vc,
                                    const int64_t *slots, int32_t num_tokens, int32_t row_bytes,
                                    int64_t num_slots, hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int32_t ppr = row_bytes / 16;
    const int64_t total = (int64_t)num_tokens * ppr;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4 *>(key), reinterpret_cast<const uint4 *>(value),
                       reinterpret_cast<uint4 *>(kc), reinterpret_cast<uint4 *>(vc), slots,
                       num_tokens, ppr, num_slots);
    return hipGetLastError();
}

hipError_t launch_quantize_cache(const void *key, const void *value, void *kc, void *vc,
                                 const int64_t *slots, const float *k_scale,
                                 const float *v_scale, int32_t num_tokens, int32_t row_elems,
                                 int32_t head_dim, int64_t num_slots, bool in_f32,
                                 hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    // 16 elements a thread unless that leaves fewer than 256K threads (a
    // 6,000-token write of 512-element rows still gains from 4)
    const bool small = (int64_t)num_tokens * (row_elems / 16) < 262144;
    const int32_t ept = small ? 4 : 16;
    const int32_t ppr = row_elems / ept;
    const int64_t total = (int64_t)num_tokens * ppr;
    const int64_t blocks = (total + 255) / 256;
    auto kernel = small ? (in_f32 ? quantize_cache_kernel<true, 4> : quantize_cache_kernel<false, 4>)
                        : (in_f32 ? quantize_cache_kernel<true, 16> : quantize_cache_kernel<false, 16>);
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const char *>(key), static_cast<const char *>(value),
                       static_cast<char *>(kc), static_cast<char *>(vc), slots, k_scale, v_scale,
                       num_tokens, ppr, head_dim, num_slots);
    return hipGetLastError();
}

hipError_t launch_expand_block_tables(int32_t *dst, const int32_t *src, int32_t num_seqs,
                                      int32_t src_stride, int32_t src_blocks, int32_t dst_stride,
                                      int32_t ratio, hipStream_t stream) {
    if (num_seqs == 0 || src_blocks == 0) return hipSuccess;
    const int32_t n = src_blocks * ratio;
    hipLaunchKernelGGL(expand_block_tables_kernel, dim3((n + 255) / 256, num_seqs), dim3(256), 0,
                       stream, dst, src, num_seqs, src_stride, src_blocks, dst_stride, ratio);
    return hipGetLastError();
}

}  // namespace pa
