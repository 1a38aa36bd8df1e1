/*
 * pa.h -- C ABI of libpa: paged variable-length attention for AMD MI355X (gfx950).
 *
 * The operations are those of the vllm-metal pages:
 *   - reshape_and_cache: scatter projected K/V rows into a paged cache
 *     (kernel walkthrough, "three Metal kernels");
 *   - varlen attention: packed queries [total_q, Hq, D] with request
 *     boundaries in cu_seqlens_q (v0.28.0 release post, "Packed queries and
 *     paged KV"), keys/values gathered through per-request block tables
 *     (kernel walkthrough, "What is Paged Attention"), grouped-query heads
 *     (kernel walkthrough, GQA decode section), causal masking of each
 *     request's new tokens against its cached prefix;
 *   - split-KV: long key ranges cut into partitions (256 or 512 tokens in the
 *     pages, any multiple of 256 here) whose
 *     log2-space (max, exp-sum) statistics and normalised partial outputs are
 *     merged by a separate reduce (kernel walkthrough, GQA decode tip 4);
 *   - the block-size view: a large cache block seen as several kernel pages
 *     with no data moved (unified-memory article, section six).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless the parameter says "host".  The
 *    library never frees, keeps or allocates them; buffers must stay alive
 *    until the work queued on `stream` has finished.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    Every call only enqueues work on it and returns without synchronising.
 *  - Tensors are dense and row-major with the shapes given; no strides.
 *  - dtype: PA_F32 (IEEE float32) or PA_BF16 (bfloat16, the upper half of a
 *    float32), the type of Q, `out` and new K/V rows.  Partials are float32.
 *  - kv_dtype: the caches' element type, either equal to dtype or PA_FP8_E4M3:
 *    8-bit OCP E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa bits,
 *    subnormals, NaN = 0x7F/0xFF, no infinities, largest magnitude 448) with
 *    one float32 scale per KV head for K (k_scale) and one for V (v_scale): a
 *    stored code c of KV head g stands for value(c) * scale[g].  The pages
 *    name KV quantisation kernels (kernel walkthrough, kernel table) but give no
 *    scheme; this one is the library's own.  k_scale / v_scale are device
 *    float32 [num_kv_heads], finite and > 0, and must be NULL for caches of
 *    dtype.  8-bit caches are read with bf16 queries (dtype PA_BF16).
 *  - Layouts:
 *      q, out            [total_q, num_q_heads, head_dim]
 *      key/value rows    [num_tokens, num_kv_heads, head_dim]
 *      key/value caches  [num_blocks, block_size, num_kv_heads, head_dim]
 *      block_tables      int32 [num_seqs, max_blocks_per_seq]; entries past a
 *                        request's last page are never read (use -1)
 *      cu_seqlens_q      int32 [num_seqs + 1], cu[0] = 0, cu[num_seqs] = total_q,
 *                        non-decreasing
 *      seq_lens          int32 [num_seqs]; keys visible to request r AFTER this
 *                        step, its own new tokens included: seq_lens[r] >= q_len(r)
 *      partials          tmp_out float32 [total_q, num_q_heads, max_partitions, head_dim]
 *                        max_logits, exp_sums float32 [total_q, num_q_heads, max_partitions]
 *  - Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *  - Causal alignment is bottom-right: query j of request r is at absolute
 *    position p = seq_lens[r] - q_len(r) + j and sees keys 0..p.
 *  - Cache slots past seq_lens[r] (page tails, unused pages) are never read
 *    into a result, whatever they hold (NaN included).
 *
 * Errors: every check a host can make is made before anything is enqueued; a
 * failing call returns a nonzero status and has written nothing.  Device-side
 * contents (cu_seqlens monotone, seq_len >= q_len, block ids < num_blocks,
 * slots < num_blocks*block_size, unique slots) are caller contracts and are not
 * checked.  A HIP launch error returns PA_EHIP.  No C++ exception crosses this
 * ABI.  There are no fallback paths: an unsupported case returns an error.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 };

enum {
    PA_OK = 0,
    PA_EINVAL = 1,        /* null pointer, negative/zero size, inconsistent sizes */
    PA_EUNSUPPORTED = 2,  /* valid but not implemented: head_dim, block_size, dtype, group size */
    PA_EWORKSPACE = 3,    /* partials buffers missing or too small for the partition count */
    PA_EHIP = 4           /* the HIP runtime reported an error while enqueuing */
};

/* Limits of this build. */
#define PA_MAX_GROUP 8          /* num_q_heads / num_kv_heads */
#define PA_MAX_SEQS 65535       /* requests per call */
#define PA_MAX_PARTITION 8192  /* largest partition_size accepted */
#define PA_SPLIT_FILL_NUM 9     /* the partition policy aims for 9/16 of a workgroup per CU */
#define PA_SPLIT_FILL_DEN 16
#define PA_SPLIT_BALANCE_NUM 3  /* ... with no item longer than 3/2 of the mean */
#define PA_SPLIT_BALANCE_DEN 2

/*
 * pa_reshape_and_cache -- write new K/V rows into the paged cache
 * (kernel walkthrough, "three Metal kernels": reshape_and_cache).
 *
 * For every t in [0, num_tokens): s = slot_mapping[t]; if s < 0 the token is
 * skipped; otherwise key_cache[s / block_size][s % block_size][:][:] = key[t]
 * and likewise for value.  With kv_dtype == dtype this is a bit copy: bytes
 * land unchanged.  With kv_dtype == PA_FP8_E4M3 every element x of KV head g is
 * stored as the E4M3 code of the correctly rounded float32 quotient
 * x / scale[g]: the nearest code, ties to an even mantissa; magnitudes above
 * 448 (infinities included) store +-448, NaN stores 0x7F, the sign of zero is
 * kept.  Slots must be unique among the tokens of one call (else which row
 * wins is unspecified).
 *   key, value        [num_tokens, num_kv_heads, head_dim], dtype
 *   key/value_cache   [num_blocks, block_size, num_kv_heads, head_dim], kv_dtype
 *   slot_mapping      int64 [num_tokens]
 *   k_scale, v_scale  float32 [num_kv_heads] for PA_FP8_E4M3, else NULL
 * block_size may be any positive value here (e.g. 144): a slot is the same
 * memory position in every page-size view of the cache.
 * Errors: PA_EINVAL (null pointer with num_tokens > 0, sizes <= 0, scales given
 *         for a cache of dtype or missing for an 8-bit one),
 *         PA_EUNSUPPORTED (dtype or kv_dtype; a cache row of
 *         num_kv_heads*head_dim elements not a multiple of 16 bytes; an 8-bit
 *         cache with head_dim not a multiple of 16).
 */
int pa_reshape_and_cache(const void *key, const void *value, void *key_cache, void *value_cache,
                         const int64_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t dtype,
                         int32_t kv_dtype, const float *k_scale, const float *v_scale,
                         void *stream);

/*
 * pa_copy_blocks -- copy whole cache blocks from one cache to another by id
 * pairs: the data movement of evicting KV blocks to a host tier and restoring
 * them (KV-offloading article; on MI355X host memory is not the GPU's, so
 * blocks are copied rather than re-pointed).
 *   for each i: dst_key[pairs[i][1]] = src_key[pairs[i][0]], same for V,
 * whole blocks of block_bytes (= block_size * Hkv * D * elt for the caches of
 * this library).  Either cache, and `pairs` (int64 [num_pairs][2]), may be
 * device memory or PINNED host memory (allocated pinned, e.g. hipHostMalloc
 * or torch's pin_memory); pageable host memory is refused with PA_EINVAL.
 * Pairs naming a block outside [0, num_src_blocks) or [0, num_dst_blocks) are
 * skipped.  Destination ids must be distinct, and no block may be both read
 * and written by one call (pairs run in parallel).  block_bytes must be a
 * positive multiple of 16 and every pointer 16-byte aligned.
 * Errors: PA_EINVAL, PA_EHIP.
 */
int pa_copy_blocks(void *dst_key, void *dst_value, const void *src_key, const void *src_value,
                   const int64_t *pairs, int32_t num_pairs, int64_t block_bytes,
                   int64_t num_src_blocks, int64_t num_dst_blocks, void *stream);

/*
 * pa_expand_block_tables -- kernel-page view of a block table whose cache
 * blocks hold `ratio` kernel pages each (unified-memory article, section six:
 * one 144-token block = nine 16-token pages, the cache viewed as
 * [num_blocks * ratio, block_size / ratio, ...] with no byte moved).
 *   dst[r][ratio*b + j] = ratio * src[r][b] + j  for b < src_blocks, j < ratio;
 *   negative src entries map to -1.
 *   src int32 [num_seqs, src_stride] (first src_blocks columns used),
 *   dst int32 [num_seqs, dst_stride], dst_stride >= src_blocks * ratio.
 * Errors: PA_EINVAL.
 */
int pa_expand_block_tables(int32_t *dst, const int32_t *src, int32_t num_seqs, int32_t src_stride,
                           int32_t src_blocks, int32_t dst_stride, int32_t ratio, void *stream);

/*
 * pa_varlen_attention -- unified paged variable-length attention.
 *
 * out[t][h][:] = sum_i softmax_i(scale * q[t][h] . k_i) v_i over the keys
 * i = 0..p of t's request, read through block_tables (see the conventions
 * above).  One call serves decode tokens, verify windows and prefill chunks
 * of any mix of requests.
 *
 * partition_size = 0: no split; `out` receives every row.
 * partition_size = P, a multiple of 256 up to PA_MAX_PARTITION (the pages use
 *   256 and 512; larger ones bound the work of one workgroup on long prefill
 *   rows): the keys of a row at position p are cut
 *   into n = ceil((p + 1) / P) partitions [kP, min((k+1)P, p+1)).
 *   Rows with n == 1 are written straight to `out`.  For rows with n >= 2,
 *   partition k < n writes
 *     max_logits[t][h][k] = max_i s_i,  s_i = scale * log2(e) * q.k_i
 *     exp_sums[t][h][k]   = sum_i 2^(s_i - max_logits)
 *     tmp_out[t][h][k][:] = sum_i 2^(s_i - max_logits) v_i / exp_sums
 *   and pa_split_kv_reduce must then be called to produce those rows of `out`.
 *   Entries for k >= n are not written.
 *   max_partitions >= ceil(max_seq_len / P) is the capacity of the partials.
 *
 * sinks: NULL, or device float32 [num_q_heads]: one attention-sink logit per
 *   query head (kernel walkthrough, "three Metal kernels": the decode kernel's
 *   sink support), in the units of scale * q.k.  The sink is one more term of
 *   the softmax denominator and carries no value:
 *     out[t][h][:] = sum_i e^(x_i) v_i / (e^(sinks[h]) + sum_i e^(x_i)),
 *   x_i = scale * q.k_i.  Partials never include it (pass the same sinks to
 *   pa_split_kv_reduce, which adds it once).  Values must be finite or -inf
 *   (-inf is the same as no sink).
 *
 * kv_dtype, k_scale, v_scale: the caches' element type and, for PA_FP8_E4M3,
 *   the per-KV-head scales (see the conventions).  An 8-bit cache gives the
 *   result of the definition above over the keys value(code) * k_scale and
 *   values value(code) * v_scale.
 *
 * Host scalars: max_q_len = max over requests of q_len (>= 1 unless
 * total_q == 0), max_seq_len = max of seq_lens; both must be upper bounds.
 * Supported: dtype PA_F32 / PA_BF16 with kv_dtype == dtype, or dtype PA_BF16
 * with kv_dtype PA_FP8_E4M3; head_dim 64, 128, 256; block_size 8, 16,
 * 32; num_q_heads % num_kv_heads == 0 with group size <= PA_MAX_GROUP.
 * Errors: PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE (P > 0 and a partial
 * buffer is NULL or max_partitions too small), PA_EHIP.
 */
int pa_varlen_attention(void *out, const void *q, const void *key_cache, const void *value_cache,
                        const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                        const int32_t *block_tables, int32_t num_seqs, int32_t total_q,
                        int32_t max_q_len, int32_t max_seq_len, int32_t max_blocks_per_seq,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t num_blocks, int32_t block_size, float scale,
                        const float *sinks, int32_t dtype, int32_t kv_dtype,
                        const float *k_scale, const float *v_scale, int32_t partition_size,
                        float *tmp_out, float *max_logits, float *exp_sums,
                        int32_t max_partitions, void *stream);

/*
 * pa_varlen_attention_noalloc -- pa_varlen_attention and, for
 * partition_size > 0, pa_split_kv_reduce in one call, with the split-KV
 * partials held in the library's own static device scratch instead of caller
 * buffers.  For callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * call allocates nothing and calls no allocating routine; the caller passes
 * the inputs and `out` only, and `out` receives every row.
 *   Scratch: PA_NOALLOC_SCRATCH_BYTES of device memory per GPU, reserved
 *   when the library is loaded and held until the process ends.  A call with
 *   P = partition_size > 0 needs the partials of
 *   n = ceil(max_seq_len / P) partitions, total_q * num_q_heads * n * (D + 2)
 *   float32 values (each of the three arrays 256-byte aligned); a call that
 *   needs more returns PA_EWORKSPACE before anything is enqueued.
 *   Every call on one GPU shares that GPU's scratch, which keeps the last
 *   call's contents: calls that overlap on one GPU (other streams, other
 *   threads) race and must be serialised by the caller.  No part of the
 *   scratch needs to start at zero: every partial the reduce reads is written
 *   by the attention launch of the same call.
 * Other arguments, the result and the errors are those of
 * pa_varlen_attention.  The dispatch record is the attention launch's.
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)
int pa_varlen_attention_noalloc(void *out, const void *q, const void *key_cache,
                                const void *value_cache, const int32_t *cu_seqlens_q,
                                const int32_t *seq_lens, const int32_t *block_tables,
                                int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                int32_t max_seq_len, int32_t max_blocks_per_seq,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t num_blocks, int32_t block_size, float scale,
                                const float *sinks, int32_t dtype, int32_t kv_dtype,
                                const float *k_scale, const float *v_scale,
                                int32_t partition_size, void *stream);

/*
 * pa_split_kv_reduce -- merge split-KV partials (kernel walkthrough, GQA decode
 * tip 4: the shared reducer).  For every row (t, h) with n >= 2 partitions
 * (n as above): M = max_k max_logits[k], w_k = exp_sums[k] * 2^(max_logits[k] - M),
 * out[t][h][:] = sum_k w_k tmp_out[k][:] / sum_k w_k, cast to dtype with
 * round-to-nearest-even.  With sinks (NULL or float32 [num_q_heads], as in
 * pa_varlen_attention), sigma = sinks[h] * log2(e) joins the max M and
 * 2^(sigma - M) the denominator.  Rows with n == 1 are left untouched.
 * Arguments mean what they mean in pa_varlen_attention.
 * Errors: PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP.
 */
int pa_split_kv_reduce(void *out, const float *tmp_out, const float *max_logits,
                       const float *exp_sums, const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                       int32_t num_seqs, int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                       const float *sinks, int32_t partition_size, int32_t max_partitions,
                       int32_t dtype, void *stream);

/*
 * pa_pick_partition_size -- host-only partition policy for decode batches.
 * The pages' rule (kernel walkthrough, "dispatch layer") is a work budget
 * proportional to the number of GPU cores, larger partitions tried first
 * (512 before 256).  This rule keeps that shape for the decode kernels the
 * launch would route to (whole-row or per KV head, which depends on the head
 * shape, dtype and partition count) and was calibrated on MI355X over decode
 * batches of 1..256 requests, 1K..64K keys and three head shapes (attention +
 * reduce as HIP graphs over cold pools): every partition pays a start-up, a
 * merge and a reduce share, so the largest size that still fills the GPU with
 * evenly sized workgroups wins.  With
 *   budget = num_cus * PA_SPLIT_FILL_NUM / PA_SPLIT_FILL_DEN,
 *   items(P) = sum_r ceil(seq_lens[r] / P)  (P = 0: one per request),
 *   workgroups(P) = items(P) for the whole-row kernel, items(P) * num_kv_heads
 *                   for the per-head kernel,
 * a size qualifies when workgroups(P) >= budget and the longest item streams
 * at most PA_SPLIT_BALANCE_NUM / PA_SPLIT_BALANCE_DEN times the mean key
 * count of an item.  Sizes are tried in the order 0, 8192, 4096, ..., 512
 * (sizes of at least twice the longest sequence skipped), those that route to
 * the whole-row kernel first where the head shape allows it; the first that
 * qualifies is returned, else 256.  0 when no sequence is longer than 256.
 * host_seq_lens is a HOST array.  dtype / kv_dtype as in
 * pa_varlen_attention.  num_cus <= 0 asks the current device.  Returns -1 on
 * bad arguments.  Enqueues nothing.
 */
int32_t pa_pick_partition_size(const int32_t *host_seq_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t dtype, int32_t kv_dtype,
                               int32_t num_cus);

/*
 * Dispatch record: what the calling thread's last pa_varlen_attention or
 * pa_split_kv_reduce call decided (the kernel walkthrough's dispatch layer,
 * made inspectable).  Environment switches, read at every call:
 *   PA_NO_SPLIT=1  pa_varlen_attention ignores partition_size (every row is
 *                  finished in place, partial buffers untouched) and
 *                  pa_split_kv_reduce does nothing.
 *   PA_DECODE_ROWS=0|1|2  decode batches with bf16 queries: 0 keeps the
 *                  per-KV-head decode kernel (grid = KV heads x requests x
 *                  partitions); 2 takes a whole-row kernel (grid = requests
 *                  x partitions, every KV head per workgroup) whenever the
 *                  head shape allows it; 1 (default) takes it when the launch
 *                  has at least 128 (request, partition) items over bf16
 *                  caches, 256 over 8-bit caches.  Results agree within
 *                  rounding either way.
 */
enum {
    PA_PATH_NONE = 0,        /* rejected, or nothing to do (empty batch) */
    PA_PATH_DECODE = 1,      /* decode kernels, one workgroup per request (and KV head) */
    PA_PATH_DECODE_TOKEN = 2,/* VALU decode kernel, one workgroup per query token */
    PA_PATH_TILED = 3,       /* bf16 MFMA tile kernel */
    PA_PATH_REDUCE_ROWS = 4, /* split-KV reduce, one wave per row */
    PA_PATH_REDUCE_SLICES = 5,/* split-KV reduce, one workgroup per row slice */
    PA_PATH_REDUCE_SKIP = 6  /* reduce disabled by PA_NO_SPLIT */
};
typedef struct {
    int32_t path;            /* PA_PATH_* */
    int32_t status;          /* the call's return value */
    int32_t partition_size;  /* partition actually used (0 = none) */
    int32_t split_disabled;  /* 1 if PA_NO_SPLIT overrode the caller's partition */
    int32_t grid[3];         /* launch grid in workgroups (0 if nothing launched) */
    int32_t block;           /* threads per workgroup */
    int32_t tile[3];         /* decode: chunk tokens, waves, LDS stages; tiled: keys per
                                tile, LDS stages, q tokens per tile; reduce: 0 */
} pa_dispatch_info;

/* Copy the calling thread's last record into *info.  Returns PA_EINVAL if
 * info is NULL. */
int pa_last_dispatch(pa_dispatch_info *info);

/* Bytes needed for the partials of a split call (tmp_out; max_logits and
 * exp_sums each).  Returns PA_EINVAL on bad sizes. */
int pa_partials_bytes(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                      int32_t max_partitions, size_t *tmp_out_bytes, size_t *stats_bytes);

/* Static text for a status code. */
const char *pa_status_string(int status);

/* Version of this ABI (major * 100 + minor). */
int pa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
