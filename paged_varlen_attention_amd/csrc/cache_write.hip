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
