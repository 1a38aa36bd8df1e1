// block_copy.hip -- whole cache blocks copied between two caches by id pairs:
// the data movement behind evicting KV blocks to a host tier and restoring
// them (KV-offloading article).  On MI355X host memory is not the GPU's own,
// so instead of moving only table entries the blocks are copied: either cache
// may be device memory or pinned host memory, which the kernel reads and
// writes through the GPU's mapping of it.
//
// Grid (pair, K/V): one workgroup per block of one tensor.  Each thread keeps
// four 16-byte loads in flight before storing them, so a block over the host
// link has enough requests outstanding; pairs naming a block outside either
// pool are skipped.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int BT = 256;     // threads per workgroup
constexpr int UNROLL = 4;   // 16-byte loads in flight per thread

__global__ __launch_bounds__(BT) void copy_blocks_kernel(
    uint4 *__restrict__ dst_k, uint4 *__restrict__ dst_v, const uint4 *__restrict__ src_k,
    const uint4 *__restrict__ src_v, const int64_t *__restrict__ pairs, int64_t pieces,
    int64_t num_src, int64_t num_dst) {
    const int64_t s = pairs[2 * (int64_t)blockIdx.x];
    const int64_t d = pairs[2 * (int64_t)blockIdx.x + 1];
    if (s < 0 || s >= num_src || d < 0 || d >= num_dst) return;
    const uint4 *src = (blockIdx.y ? src_v : src_k) + s * pieces;
    uint4 *dst = (blockIdx.y ? dst_v : dst_k) + d * pieces;
    int64_t i = threadIdx.x;
    for (; i + (UNROLL - 1) * BT < pieces; i += UNROLL * BT) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = src[i + u * BT];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) dst[i + u * BT] = v[u];
    }
    for (; i < pieces; i += BT) dst[i] = src[i];
}

}  // namespace

hipError_t launch_copy_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                              const int64_t *pairs, int32_t num_pairs, int64_t block_bytes,
                              int64_t num_src, int64_t num_dst, hipStream_t stream) {
    if (num_pairs == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(BT), 0, stream,
                       reinterpret_cast<uint4 *>(dst_k), reinterpret_cast<uint4 *>(dst_v),
                       reinterpret_cast<const uint4 *>(src_k), reinterpret_cast<const uint4 *>(src_v),
                       pairs, block_bytes / 16, num_src, num_dst);
    return hipGetLastError();
}

}  // namespace pa
