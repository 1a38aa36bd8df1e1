// pa_internal.h -- launch parameters and launcher entry points shared by the
// C-ABI layer (pa_api.cpp) and the HIP kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Kernel page geometry.  Decode stages K/V through LDS in chunks of CHUNK
// tokens whatever the cache page size is (8, 16 or 32 tokens).
constexpr int CHUNK = 16;

struct AttnParams {
    void *out;
    const void *q;
    const void *kc;
    const void *vc;
    const int32_t *cu_q;
    const int32_t *seq_lens;
    const int32_t *bt;
    float *tmp_out;
    float *max_logits;
    float *exp_sums;
    int32_t num_seqs;
    int32_t total_q;
    int32_t max_q_len;
    int32_t max_seq_len;
    int32_t bt_stride;
    int32_t hq;
    int32_t hkv;
    int32_t group;          // hq / hkv
    int32_t head_dim;
    int32_t num_blocks;
    int32_t block_size;
    int32_t log2_bs;
    int32_t partition;      // 0 = no split
    int32_t max_parts;
    float scale_log2;       // scale * log2(e)
    const float *sinks;     // NULL or [hq] sink logits (natural-log units)
    int32_t dtype;
    int32_t kv8;            // caches hold E4M3 codes (dtype is then bf16)
    const float *k_scale;   // kv8: [hkv] scale of K codes, else NULL
    const float *v_scale;   // kv8: [hkv] scale of V codes, else NULL
    int32_t per_token;      // decode kernel: grid z indexes query tokens, not requests
    int32_t grid_tiles;     // tiled kernel: virtual q-tiles (set by its launcher)
    int32_t grid_parts;     // tiled kernel: partitions in the grid (set by its launcher)
};

struct ReduceParams {
    void *out;
    const float *tmp_out;
    const float *max_logits;
    const float *exp_sums;
    const int32_t *cu_q;
    const int32_t *seq_lens;
    int32_t num_seqs;
    int32_t total_q;
    int32_t hq;
    int32_t head_dim;
    int32_t partition;
    int32_t max_parts;
    const float *sinks;     // NULL or [hq] sink logits (natural-log units)
    int32_t dtype;
};

// What a launcher enqueued (for the dispatch record): grid in workgroups,
// threads per workgroup, and the kernel's tile parameters.
struct LaunchInfo {
    int32_t grid[3];
    int32_t block;
    int32_t tile[3];
    int32_t form;  // reduce: 0 = one wave per row, 1 = one workgroup per row slice
};

// Each launcher returns hipSuccess or the error of the launch; it assumes the
// caller validated every host-visible argument.  `li` may be NULL.
hipError_t launch_reshape_and_cache(const void *key, const void *value, void *kc, void *vc,
                                    const int64_t *slots, int32_t num_tokens, int32_t row_bytes,
                                    int64_t num_slots, hipStream_t stream);
// 8-bit cache write: E4M3 codes of row / scale[head]; in_f32 selects float32
// rows (else bf16).  row_elems = num_kv_heads * head_dim, a multiple of 16.
hipError_t launch_quantize_cache(const void *key, const void *value, void *kc, void *vc,
                                 const int64_t *slots, const float *k_scale,
                                 const float *v_scale, int32_t num_tokens, int32_t row_elems,
                                 int32_t head_dim, int64_t num_slots, bool in_f32,
                                 hipStream_t stream);
hipError_t launch_expand_block_tables(int32_t *dst, const int32_t *src, int32_t num_seqs,
                                      int32_t src_stride, int32_t src_blocks, int32_t dst_stride,
                                      int32_t ratio, hipStream_t stream);
hipError_t launch_copy_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                              const int64_t *pairs, int32_t num_pairs, int64_t block_bytes,
                              int64_t num_src, int64_t num_dst, hipStream_t stream);
hipError_t launch_decode(const AttnParams &p, hipStream_t stream, LaunchInfo *li);
// bf16 decode batches (one token per request, bf16 caches, group <= 8) on MFMA.
bool decode_mfma_supported(const AttnParams &p);
// The whole-row decode kernels (bf16 or 8-bit caches): whether a launch
// takes one (shape and launch-size rule, PA_DECODE_ROWS) and its launcher.
bool decode_rows_supported(const AttnParams &p);
hipError_t launch_decode_rows(const AttnParams &p, hipStream_t stream, LaunchInfo *li);
// Shape rule and launcher of the 8-bit whole-row kernel.
bool decode_rows8_shape(const AttnParams &p);
hipError_t launch_decode_rows8(const AttnParams &p, hipStream_t stream, LaunchInfo *li);
hipError_t launch_decode_mfma(const AttnParams &p, hipStream_t stream, LaunchInfo *li);
hipError_t launch_prefill(const AttnParams &p, hipStream_t stream, LaunchInfo *li);
hipError_t launch_reduce(const ReduceParams &p, hipStream_t stream, LaunchInfo *li);

// Device address of the calling thread's current device's copy of the
// library's static scratch (PA_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned),
// looked up once per device.
hipError_t noalloc_scratch(void **ptr);

// Whether a decode instantiation exists for this geometry.
bool decode_supported(int dtype, int head_dim, int group);
bool decode_kv8_supported(int head_dim, int group);
bool prefill_supported(int dtype, int head_dim, int group);
bool prefill_kv8_supported(int head_dim, int group);

}  // namespace pa
