/*
 * pa_oracle.h -- plain fp64 CPU oracle for paged variable-length attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this code; only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source with the HIP path.
 *
 * It computes, slowly and directly, what the pages define:
 *   - the cache write that scatters projected K/V rows into fixed-size pages
 *     (vllm-metal kernel walkthrough, "three Metal kernels": reshape_and_cache);
 *   - masked softmax(Q K^T * scale) V over keys gathered through per-request
 *     block tables (same page, "What is Paged Attention"), for queries packed
 *     as [total_q, Hq, D] with request boundaries in cu_seqlens
 *     (v0.28.0 release post, "Packed queries and paged KV");
 *   - the split-KV form: per partition, the log2-space (max, exp-sum)
 *     statistics and the normalised partial output, and their merge
 *     (kernel walkthrough, GQA decode tip 4 "Split-KV partitions").
 *
 * Readings where the pages are silent (all of them stated in the design notes):
 *   - seq_lens[r] counts every key request r sees, its own new tokens included;
 *   - causal alignment is bottom-right: query j of request r sits at absolute
 *     position ctx + j, ctx = seq_lens[r] - q_len[r], and sees keys 0..ctx+j;
 *   - query head h reads KV head h / (Hq / Hkv);
 *   - caches are [num_blocks, block_size, Hkv, D]; logical key i of request r
 *     lives in block block_tables[r][i / block_size], slot i % block_size;
 *   - slot_mapping < 0 means "skip this token";
 *   - an attention sink (the kernel walkthrough's decode kernel lists sink
 *     support; the pages give no formula) is a per-query-head logit in the
 *     same units as scale * q.k that joins the softmax denominator and
 *     carries no value: out = sum_i e^(s_i) v_i / (e^sink + sum_i e^(s_i)).
 *     Split partials leave it out; the merge adds it once.
 *
 * Element types: PA_REF_F32 = IEEE float32, PA_REF_BF16 = bfloat16 (the upper
 * 16 bits of a float32).  Every input value is widened exactly to double and
 * all arithmetic is double; results are returned unrounded in double.
 *
 * 8-bit KV cache (PA_REF_FP8_E4M3).  The pages list KV quantisation kernels
 * (the kernel walkthrough's kernel table) but give no scheme, so this one is
 * ours, stated here in full:
 *   - the element format is the OCP 8-bit float E4M3 ("e4m3fn"): sign bit,
 *     4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 *     subnormals m/8 * 2^-6; the pattern with all exponent and mantissa bits
 *     set is NaN; there are no infinities; the largest magnitude is 448;
 *   - each KV head g has one float32 scale for K (k_scale[g]) and one for V
 *     (v_scale[g]); a stored code c stands for value(c) * scale[g];
 *   - the cache write stores, for an input element x of head g,
 *       code = E(fl32(x / scale[g])),
 *     where fl32 is the correctly rounded float32 quotient and E picks the
 *     nearest E4M3 value (ties to the code with an even last mantissa bit),
 *     magnitudes above 448 (infinities included) giving +-448 and NaN giving
 *     the code 0x7F.  The sign of zero is kept.
 *
 * Return value of every function: 0 on success, -1 on an argument the oracle
 * cannot interpret (bad dtype, negative sizes, a key index outside the block
 * table or the pool, or ctx < 0).
 */
#ifndef PA_ORACLE_H
#define PA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { PA_REF_F32 = 0, PA_REF_BF16 = 1, PA_REF_FP8_E4M3 = 2 };

/* Value of one E4M3 code (NaN for 0x7F and 0xFF). */
double pa_ref_e4m3_value(uint8_t code);

/* E(y) as defined above, for y already rounded to float32 by the caller. */
uint8_t pa_ref_e4m3_encode(double y);

/* Array forms of the two functions above (for the pins). */
int pa_ref_e4m3_values(double *out, const uint8_t *codes, int64_t n);
int pa_ref_e4m3_encode_f32(uint8_t *out, const float *y, int64_t n);

/* Threads the OpenMP runtime will use for the row loops. */
int pa_ref_num_threads(void);
/* Set the thread count of the row loop (timing only; results do not depend on it). */
void pa_ref_set_num_threads(int n);

/* Cache write: for t in [0, T): s = slot_mapping[t]; s < 0 -> skip;
 * caches[s / bs][s % bs][:][:] = rows[t][:][:], for K and V.  A byte copy. */
int pa_ref_reshape_and_cache(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int64_t *slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                             int32_t block_size, int32_t dtype);

/* Quantising cache write into 8-bit caches: for t in [0, T) with slot
 * s = slot_mapping[t] >= 0, head g and element d,
 *   key_cache[s / bs][s % bs][g][d] = E(fl32(key[t][g][d] / k_scale[g])),
 * likewise value with v_scale.  Rows are PA_REF_F32 or PA_REF_BF16 (`dtype`);
 * scales are float32 [num_kv_heads], finite and > 0.  Slots must be distinct
 * (tokens are written in parallel). */
int pa_ref_reshape_and_cache_fp8(const void *key, const void *value, uint8_t *key_cache,
                                 uint8_t *value_cache, const int64_t *slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t num_blocks, int32_t block_size, int32_t dtype,
                                 const float *k_scale, const float *v_scale);

/* Block copy between two caches (the KV-offloading article: evicting blocks to
 * a host tier and restoring them, by block-id lists): for each pair i,
 * dst[pairs[2i+1]] = src[pairs[2i]] for K and V, whole blocks of block_bytes,
 * in pair order; pairs naming a block outside either pool are skipped.  A
 * byte copy. */
int pa_ref_copy_blocks(void *dst_key, void *dst_value, const void *src_key, const void *src_value,
                       const int64_t *pairs, int32_t num_pairs, int64_t block_bytes,
                       int64_t num_src_blocks, int64_t num_dst_blocks);

/* Kernel-page view of a block table whose blocks hold `ratio` kernel pages:
 * dst[r][ratio*b + j] = ratio * src[r][b] + j, and -1 stays -1. */
int pa_ref_expand_block_tables(int32_t *dst, const int32_t *src, int32_t num_seqs,
                               int32_t src_stride, int32_t src_blocks, int32_t dst_stride,
                               int32_t ratio);

/* Attention for selected (token, head) pairs: out[n][D] (double) for
 * n in [0, n_rows), row n = (tok[n], head[n]).  Pass tok = head = NULL to
 * compute every (t, h) in the natural order t*Hq + h (out = [total_q][Hq][D]).
 * sinks: NULL, or float32 [num_q_heads] sink logits (see above).
 * kv_dtype: the caches' element type, equal to dtype or PA_REF_FP8_E4M3; for
 * the latter k_scale and v_scale are float32 [num_kv_heads] (NULL otherwise)
 * and each cached element is read as value(code) * scale of its KV head. */
int pa_ref_attention(double *out, const int32_t *tok, const int32_t *head, int32_t n_rows,
                     const void *q, const void *key_cache, const void *value_cache,
                     const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                     const int32_t *block_tables, int32_t num_seqs, int32_t total_q,
                     int32_t max_blocks_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t num_blocks, int32_t block_size, double scale,
                     int32_t dtype, int32_t kv_dtype, const float *k_scale,
                     const float *v_scale, const float *sinks);

/* Split-KV partials for every (t, h): partition k of the query at absolute
 * position p covers keys [k*P, min((k+1)*P, p+1)), k < ceil((p+1)/P).
 *   m[t][h][k]    = max over the partition of s_i * log2(e),  s_i = scale * q.k_i
 *   l[t][h][k]    = sum 2^(s_i*log2(e) - m)
 *   o[t][h][k][:] = sum 2^(s_i*log2(e) - m) * v_i / l
 * Entries for k >= ceil((p+1)/P) are left untouched.  Arrays are dense with
 * max_parts partitions per (t, h).  kv_dtype, k_scale, v_scale: as above. */
int pa_ref_attention_partials(double *o, double *m, double *l, const void *q,
                              const void *key_cache, const void *value_cache,
                              const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                              const int32_t *block_tables, int32_t num_seqs, int32_t total_q,
                              int32_t max_blocks_per_seq, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                              int32_t block_size, double scale, int32_t dtype,
                              int32_t kv_dtype, const float *k_scale, const float *v_scale,
                              int32_t partition_size, int32_t max_parts);

/* Merge of the partials above: with n = ceil((p+1)/P), M = max_k m_k,
 * w_k = l_k * 2^(m_k - M):  out[t][h][:] = sum_k w_k o_k / sum_k w_k.
 * With sinks (float32 [num_q_heads], natural-log logits), sigma = sink * log2(e)
 * joins the max and adds 2^(sigma - M) to the denominator once. */
int pa_ref_split_reduce(double *out, const double *o, const double *m, const double *l,
                        const int32_t *cu_seqlens_q, const int32_t *seq_lens, int32_t num_seqs,
                        int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                        int32_t partition_size, int32_t max_parts, const float *sinks);

#ifdef __cplusplus
}
#endif
#endif
