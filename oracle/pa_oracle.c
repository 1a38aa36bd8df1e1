/*
 * pa_oracle.c -- plain fp64 CPU oracle for paged variable-length attention.
 *
 * TEST INFRASTRUCTURE ONLY (see pa_oracle.h).  Deliberately slow and direct:
 * one (token, head) row at a time, keys in logical order, no blocking, no
 * fusion, no online rescaling.  The only parallelism is an OpenMP loop over
 * independent output rows, which does not change any row's arithmetic.
 */
#include "pa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static const double LOG2E = 1.4426950408889634073599246810018921;

int pa_ref_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the row loop from now on (the CPU baseline times 1 and all). */
void pa_ref_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Exact widening of one stored element to double.  bfloat16 is the upper
 * half of an IEEE float32, so shifting it up 16 bits gives that float. */
static double load_elem(const void *base, size_t idx, int dtype) {
    if (dtype == PA_REF_F32) {
        return (double)((const float *)base)[idx];
    } else {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

static int elem_bytes(int dtype) {
    return dtype == PA_REF_F32 ? 4 : (dtype == PA_REF_BF16 ? 2 : 0);
}

/* ---- OCP E4M3, written from the format's definition ---- */

double pa_ref_e4m3_value(uint8_t code) {
    int negative = code >> 7;
    int e = (code >> 3) & 15; /* biased exponent */
    int m = code & 7;         /* mantissa */
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);        /* subnormal: 0.m * 2^(1 - 7) */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7); /* normal: 1.m * 2^(e - 7) */
    return negative ? -mag : mag;
}

/* Values of all 256 codes (pa_ref_e4m3_value of each), filled once by
 * e4m3_table_init() before any parallel region reads it.  The encoder
 * searches entries 0x00..0x7E, the non-negative finite codes. */
static double e4m3_table[256];
static int e4m3_table_ready = 0;

static void e4m3_table_init(void) {
    if (e4m3_table_ready) return;
    for (int c = 0; c < 256; ++c) e4m3_table[c] = pa_ref_e4m3_value((uint8_t)c);
    e4m3_table_ready = 1;
}

/* Nearest code by exhaustive search over the 127 non-negative finite codes
 * (the table must be initialised); of two equally near codes the one with an
 * even last mantissa bit wins. */
static uint8_t e4m3_encode_searched(double y) {
    if (isnan(y)) return 0x7F;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs(y);
    if (a > 448.0) a = 448.0; /* saturate (infinities too) */
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double err = fabs(e4m3_table[c] - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(sign | best);
}

uint8_t pa_ref_e4m3_encode(double y) {
    e4m3_table_init();
    return e4m3_encode_searched(y);
}

int pa_ref_e4m3_values(double *out, const uint8_t *codes, int64_t n) {
    if (n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = pa_ref_e4m3_value(codes[i]);
    return 0;
}

int pa_ref_e4m3_encode_f32(uint8_t *out, const float *y, int64_t n) {
    if (n < 0) return -1;
    e4m3_table_init();
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode_searched((double)y[i]);
    return 0;
}

int pa_ref_reshape_and_cache(const void *key, const void *value, void *key_cache,
                             void *value_cache, const int64_t *slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                             int32_t block_size, int32_t dtype) {
    int eb = elem_bytes(dtype);
    if (!eb || num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
        return -1;
    size_t row = (size_t)num_kv_heads * head_dim * eb; /* bytes of one token's K (or V) */
    int64_t num_slots = (int64_t)num_blocks * block_size;
    for (int32_t t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0) continue;
        if (s >= num_slots) return -1;
        int64_t blk = s / block_size, off = s % block_size;
        size_t dst = ((size_t)blk * block_size + (size_t)off) * row;
        memcpy((char *)key_cache + dst, (const char *)key + (size_t)t * row, row);
        memcpy((char *)value_cache + dst, (const char *)value + (size_t)t * row, row);
    }
    return 0;
}

/* fl32(x / s): the quotient of two values that are exact in float32, rounded
 * to float32.  Dividing in double and rounding the double quotient to float
 * gives the correctly rounded float32 quotient (double carries more than
 * 2*24 + 2 significant bits, so the second rounding cannot go wrong). */
static float quotient_f32(double x, double s) { return (float)(x / s); }

int pa_ref_reshape_and_cache_fp8(const void *key, const void *value, uint8_t *key_cache,
                                 uint8_t *value_cache, const int64_t *slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t num_blocks, int32_t block_size, int32_t dtype,
                                 const float *k_scale, const float *v_scale) {
    if (!elem_bytes(dtype) || num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || !k_scale || !v_scale)
        return -1;
    int64_t num_slots = (int64_t)num_blocks * block_size;
    size_t row = (size_t)num_kv_heads * head_dim; /* elements (= bytes in the cache) per token */
    for (int32_t t = 0; t < num_tokens; ++t)
        if (slot_mapping[t] >= num_slots) return -1;
    e4m3_table_init();
    /* tokens are independent (slots are distinct), so the loop over them is
     * split across threads; each element's arithmetic is unchanged */
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0) continue;
        for (int32_t g = 0; g < num_kv_heads; ++g)
            for (int32_t d = 0; d < head_dim; ++d) {
                size_t src = (size_t)t * row + (size_t)g * head_dim + d;
                size_t dst = (size_t)s * row + (size_t)g * head_dim + d;
                key_cache[dst] = e4m3_encode_searched(
                    quotient_f32(load_elem(key, src, dtype), (double)k_scale[g]));
                value_cache[dst] = e4m3_encode_searched(
                    quotient_f32(load_elem(value, src, dtype), (double)v_scale[g]));
            }
    }
    return 0;
}

int pa_ref_copy_blocks(void *dst_key, void *dst_value, const void *src_key, const void *src_value,
                       const int64_t *pairs, int32_t num_pairs, int64_t block_bytes,
                       int64_t num_src_blocks, int64_t num_dst_blocks) {
    if (num_pairs < 0 || block_bytes <= 0 || num_src_blocks < 0 || num_dst_blocks < 0) return -1;
    for (int32_t i = 0; i < num_pairs; ++i) {
        int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
        if (s < 0 || s >= num_src_blocks || d < 0 || d >= num_dst_blocks) continue;
        memcpy((char *)dst_key + d * block_bytes, (const char *)src_key + s * block_bytes,
               (size_t)block_bytes);
        memcpy((char *)dst_value + d * block_bytes, (const char *)src_value + s * block_bytes,
               (size_t)block_bytes);
    }
    return 0;
}

int pa_ref_expand_block_tables(int32_t *dst, const int32_t *src, int32_t num_seqs,
                               int32_t src_stride, int32_t src_blocks, int32_t dst_stride,
                               int32_t ratio) {
    if (ratio <= 0 || dst_stride < src_blocks * ratio) return -1;
    for (int32_t r = 0; r < num_seqs; ++r)
        for (int32_t b = 0; b < src_blocks; ++b) {
            int32_t v = src[(size_t)r * src_stride + b];
            for (int32_t j = 0; j < ratio; ++j)
                dst[(size_t)r * dst_stride + (size_t)b * ratio + j] = v < 0 ? -1 : v * ratio + j;
        }
    return 0;
}

/* The request that owns packed token t: the r with cu[r] <= t < cu[r+1]. */
static int32_t owner_of(int32_t t, const int32_t *cu, int32_t num_seqs) {
    for (int32_t r = 0; r < num_seqs; ++r)
        if (cu[r] <= t && t < cu[r + 1]) return r;
    return -1;
}

typedef struct {
    const void *q, *kc, *vc;
    const int32_t *cu, *seq_lens, *bt;
    int32_t num_seqs, total_q, max_blocks, hq, hkv, d, num_blocks, bs, dtype;
    double scale;
    const float *sinks; /* NULL, or one logit per query head */
    int32_t kv_dtype;   /* dtype, or PA_REF_FP8_E4M3 */
    const float *k_scale, *v_scale; /* 8-bit caches: one scale per KV head */
} args_t;

/* Cached element `idx` of KV head g as a double: exact widening, or for an
 * 8-bit cache the code's value times the head's scale. */
static double load_kv(const args_t *a, const void *cache, const float *scale, size_t idx,
                      int32_t g) {
    if (a->kv_dtype == PA_REF_FP8_E4M3) /* table initialised before the row loops */
        return e4m3_table[((const uint8_t *)cache)[idx]] * (double)scale[g];
    return load_elem(cache, idx, a->kv_dtype);
}

/* Where logical key i of request r lives: index of element 0 of that key's
 * row for KV head g, in elements.  -1 if the block table does not hold it. */
static int64_t key_row(const args_t *a, int32_t r, int32_t i, int32_t g) {
    int32_t lb = i / a->bs;
    if (lb >= a->max_blocks) return -1;
    int32_t blk = a->bt[(size_t)r * a->max_blocks + lb];
    if (blk < 0 || blk >= a->num_blocks) return -1;
    int32_t off = i % a->bs;
    return (((int64_t)blk * a->bs + off) * a->hkv + g) * a->d;
}

/* Score s_i = scale * sum_d q[t][h][d] * k_i[g][d] for the query (t, h)
 * against keys [k0, k1) of request r.  Writes scores[i - k0].  Returns -1 on
 * an unreachable key. */
static int scores_for(const args_t *a, int32_t r, int32_t t, int32_t h, int32_t k0, int32_t k1,
                      double *scores) {
    int32_t G = a->hq / a->hkv;
    int32_t g = h / G;
    size_t qbase = ((size_t)t * a->hq + h) * a->d;
    for (int32_t i = k0; i < k1; ++i) {
        int64_t kr = key_row(a, r, i, g);
        if (kr < 0) return -1;
        double dot = 0.0;
        for (int32_t d = 0; d < a->d; ++d)
            dot += load_elem(a->q, qbase + d, a->dtype) * load_kv(a, a->kc, a->k_scale, (size_t)kr + d, g);
        scores[i - k0] = a->scale * dot;
    }
    return 0;
}

/* Absolute position of packed query token t (request r): ctx + j. */
static int64_t query_pos(const args_t *a, int32_t r, int32_t t) {
    int32_t q_len = a->cu[r + 1] - a->cu[r];
    int32_t ctx = a->seq_lens[r] - q_len;
    if (ctx < 0) return -1;
    return (int64_t)ctx + (t - a->cu[r]);
}

/* One output row: softmax over keys 0..p (natural exponent), weighted sum of V.
 * With a sink logit for head h, the sink is one more term of the softmax
 * denominator that carries no value: out = sum_i e^(s_i) v_i / (e^sink + sum_i e^(s_i)). */
static int attention_row(const args_t *a, int32_t t, int32_t h, double *out_row, double *scores) {
    int32_t r = owner_of(t, a->cu, a->num_seqs);
    if (r < 0) return -1;
    int64_t p = query_pos(a, r, t);
    if (p < 0) return -1;
    int32_t nk = (int32_t)p + 1; /* keys 0..p are visible (bottom-right causal) */
    if (scores_for(a, r, t, h, 0, nk, scores)) return -1;
    double m = -INFINITY;
    for (int32_t i = 0; i < nk; ++i) m = scores[i] > m ? scores[i] : m;
    double sink = a->sinks ? (double)a->sinks[h] : -INFINITY;
    if (sink > m) m = sink;
    double z = a->sinks ? exp(sink - m) : 0.0;
    for (int32_t i = 0; i < nk; ++i) {
        scores[i] = exp(scores[i] - m);
        z += scores[i];
    }
    int32_t g = h / (a->hq / a->hkv);
    for (int32_t d = 0; d < a->d; ++d) out_row[d] = 0.0;
    for (int32_t i = 0; i < nk; ++i) {
        int64_t vr = key_row(a, r, i, g);
        for (int32_t d = 0; d < a->d; ++d)
            out_row[d] += scores[i] * load_kv(a, a->vc, a->v_scale, (size_t)vr + d, g);
    }
    for (int32_t d = 0; d < a->d; ++d) out_row[d] /= z;
    return 0;
}

static int check_args(const args_t *a) {
    if (!elem_bytes(a->dtype)) return -1;
    if (a->kv_dtype == PA_REF_FP8_E4M3) {
        if (!a->k_scale || !a->v_scale) return -1;
    } else if (a->kv_dtype != a->dtype) {
        return -1;
    }
    if (a->num_seqs < 0 || a->total_q < 0 || a->hq <= 0 || a->hkv <= 0 || a->d <= 0 || a->bs <= 0)
        return -1;
    if (a->hq % a->hkv) return -1;
    if (a->num_seqs > 0 && a->cu[a->num_seqs] != a->total_q) return -1;
    return 0;
}

static int32_t longest_seq(const args_t *a) {
    int32_t mx = 1;
    for (int32_t r = 0; r < a->num_seqs; ++r) mx = a->seq_lens[r] > mx ? a->seq_lens[r] : mx;
    return mx;
}

int pa_ref_attention(double *out, const int32_t *tok, const int32_t *head, int32_t n_rows,
                     const void *q, const void *key_cache, const void *value_cache,
                     const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                     const int32_t *block_tables, int32_t num_seqs, int32_t total_q,
                     int32_t max_blocks_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t num_blocks, int32_t block_size, double scale,
                     int32_t dtype, int32_t kv_dtype, const float *k_scale,
                     const float *v_scale, const float *sinks) {
    args_t a = {q, key_cache, value_cache, cu_seqlens_q, seq_lens, block_tables, num_seqs,
                total_q, max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, num_blocks,
                block_size, dtype, scale, sinks, kv_dtype, k_scale, v_scale};
    if (check_args(&a)) return -1;
    e4m3_table_init();
    int64_t rows = (tok == NULL) ? (int64_t)total_q * num_q_heads : n_rows;
    int32_t maxk = longest_seq(&a);
    int err = 0;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)maxk);
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < rows; ++n) {
            int32_t t = tok ? tok[n] : (int32_t)(n / num_q_heads);
            int32_t h = head ? head[n] : (int32_t)(n % num_q_heads);
            if (!scores || t < 0 || t >= total_q || h < 0 || h >= num_q_heads ||
                attention_row(&a, t, h, out + (size_t)n * head_dim, scores)) {
#pragma omp atomic write
                err = 1;
            }
        }
        free(scores);
    }
    return err ? -1 : 0;
}

int pa_ref_attention_partials(double *o, double *m, double *l, const void *q,
                              const void *key_cache, const void *value_cache,
                              const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                              const int32_t *block_tables, int32_t num_seqs, int32_t total_q,
                              int32_t max_blocks_per_seq, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                              int32_t block_size, double scale, int32_t dtype,
                              int32_t kv_dtype, const float *k_scale, const float *v_scale,
                              int32_t partition_size, int32_t max_parts) {
    args_t a = {q, key_cache, value_cache, cu_seqlens_q, seq_lens, block_tables, num_seqs,
                total_q, max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, num_blocks,
                block_size, dtype, scale, NULL, kv_dtype, k_scale, v_scale};
    if (check_args(&a) || partition_size <= 0 || max_parts <= 0) return -1;
    e4m3_table_init();
    int64_t rows = (int64_t)total_q * num_q_heads;
    int err = 0;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)partition_size);
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < rows; ++n) {
            int32_t t = (int32_t)(n / num_q_heads), h = (int32_t)(n % num_q_heads);
            int32_t r = owner_of(t, a.cu, a.num_seqs);
            int64_t p = r < 0 ? -1 : query_pos(&a, r, t);
            int32_t parts = p < 0 ? 0 : (int32_t)((p + partition_size) / partition_size);
            if (!scores || p < 0 || parts > max_parts) {
#pragma omp atomic write
                err = 1;
                continue;
            }
            int32_t g = h / (num_q_heads / num_kv_heads);
            for (int32_t k = 0; k < parts; ++k) {
                int32_t k0 = k * partition_size;
                int32_t k1 = (int32_t)((int64_t)(k + 1) * partition_size < p + 1
                                           ? (int64_t)(k + 1) * partition_size
                                           : p + 1);
                if (scores_for(&a, r, t, h, k0, k1, scores)) {
#pragma omp atomic write
                    err = 1;
                    break;
                }
                size_t sidx = (size_t)n * max_parts + k;
                double mk = -INFINITY;
                for (int32_t i = 0; i < k1 - k0; ++i) {
                    scores[i] *= LOG2E; /* log2-space score */
                    mk = scores[i] > mk ? scores[i] : mk;
                }
                double lk = 0.0;
                for (int32_t i = 0; i < k1 - k0; ++i) {
                    scores[i] = exp2(scores[i] - mk);
                    lk += scores[i];
                }
                double *orow = o + sidx * head_dim;
                for (int32_t d = 0; d < head_dim; ++d) orow[d] = 0.0;
                for (int32_t i = 0; i < k1 - k0; ++i) {
                    int64_t vr = key_row(&a, r, k0 + i, g);
                    for (int32_t d = 0; d < head_dim; ++d)
                        orow[d] += scores[i] * load_kv(&a, a.vc, a.v_scale, (size_t)vr + d, g);
                }
                for (int32_t d = 0; d < head_dim; ++d) orow[d] /= lk;
                m[sidx] = mk;
                l[sidx] = lk;
            }
        }
        free(scores);
    }
    return err ? -1 : 0;
}

int pa_ref_split_reduce(double *out, const double *o, const double *m, const double *l,
                        const int32_t *cu_seqlens_q, const int32_t *seq_lens, int32_t num_seqs,
                        int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                        int32_t partition_size, int32_t max_parts, const float *sinks) {
    if (partition_size <= 0 || max_parts <= 0 || num_q_heads <= 0 || head_dim <= 0) return -1;
    for (int32_t t = 0; t < total_q; ++t) {
        int32_t r = owner_of(t, cu_seqlens_q, num_seqs);
        if (r < 0) return -1;
        int32_t q_len = cu_seqlens_q[r + 1] - cu_seqlens_q[r];
        int64_t p = (int64_t)(seq_lens[r] - q_len) + (t - cu_seqlens_q[r]);
        if (p < 0) return -1;
        int32_t parts = (int32_t)((p + partition_size) / partition_size);
        if (parts > max_parts) return -1;
        for (int32_t h = 0; h < num_q_heads; ++h) {
            size_t n = (size_t)t * num_q_heads + h;
            double M = -INFINITY;
            for (int32_t k = 0; k < parts; ++k) M = m[n * max_parts + k] > M ? m[n * max_parts + k] : M;
            /* the sink (natural-log logit) joins once, in log2 units like the statistics */
            double sink2 = sinks ? (double)sinks[h] * LOG2E : -INFINITY;
            if (sink2 > M) M = sink2;
            double wsum = sinks ? exp2(sink2 - M) : 0.0;
            double *orow = out + n * head_dim;
            for (int32_t d = 0; d < head_dim; ++d) orow[d] = 0.0;
            for (int32_t k = 0; k < parts; ++k) {
                double w = l[n * max_parts + k] * exp2(m[n * max_parts + k] - M);
                wsum += w;
                for (int32_t d = 0; d < head_dim; ++d)
                    orow[d] += w * o[(n * max_parts + k) * head_dim + d];
            }
            for (int32_t d = 0; d < head_dim; ++d) orow[d] /= wsum;
        }
    }
    return 0;
}
