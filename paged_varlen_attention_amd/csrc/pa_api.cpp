// pa_api.cpp -- the extern "C" entry points of libpa: argument validation,
// routing and launch.  Every check that the host can make happens here, before
// anything is enqueued, so a failing call has no side effects.  No exception
// crosses the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elt_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_BF16 ? 2 : 0); }

int log2_exact(int32_t v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return (1 << l) == v ? l : -1;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_EHIP; }

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Cache element type against the row dtype: PA_OK, or the status to return.
// Scales go with 8-bit caches only.
int check_kv(int32_t dtype, int32_t kv_dtype, const float *k_scale, const float *v_scale) {
    if (kv_dtype == PA_FP8_E4M3) {
        if (!k_scale || !v_scale || !aligned4(k_scale) || !aligned4(v_scale)) return PA_EINVAL;
        return PA_OK;
    }
    if (kv_dtype != dtype) return PA_EUNSUPPORTED;
    return (k_scale || v_scale) ? PA_EINVAL : PA_OK;
}

// Grid dimensions y and z are limited to 65535 workgroups.
constexpr int32_t GRID_YZ_MAX = 65535;

// The calling thread's last dispatch decision (pa_last_dispatch).
thread_local pa_dispatch_info g_last{};

void record_launch(pa_dispatch_info &rec, int32_t path, const pa::LaunchInfo &li) {
    rec.path = path;
    for (int i = 0; i < 3; ++i) {
        rec.grid[i] = li.grid[i];
        rec.tile[i] = li.tile[i];
    }
    rec.block = li.block;
}

// PA_NO_SPLIT=1 (read at every call) disables split-KV: attention finishes
// every row in place and the reduce does nothing.
bool split_disabled_by_env() {
    const char *v = std::getenv("PA_NO_SPLIT");
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

// Partition sizes: multiples of 256 keys up to PA_MAX_PARTITION.
bool partition_ok(int32_t P) { return P > 0 && P % 256 == 0 && P <= PA_MAX_PARTITION; }

int check_partitions(int32_t partition_size, int32_t max_seq_len, const float *tmp_out,
                     const float *max_logits, const float *exp_sums, int32_t max_partitions) {
    if (partition_size == 0) return PA_OK;
    if (!partition_ok(partition_size)) return PA_EUNSUPPORTED;
    if (!tmp_out || !max_logits || !exp_sums) return PA_EWORKSPACE;
    if (!aligned16(tmp_out)) return PA_EINVAL;
    const int64_t need = ((int64_t)max_seq_len + partition_size - 1) / partition_size;
    if (max_partitions < need || max_partitions <= 0) return PA_EWORKSPACE;
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return 300; }

const char *pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_EINVAL: return "invalid argument";
        case PA_EUNSUPPORTED: return "unsupported configuration";
        case PA_EWORKSPACE: return "split-KV partial buffers missing or too small";
        case PA_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int pa_partials_bytes(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                      int32_t max_partitions, size_t *tmp_out_bytes, size_t *stats_bytes) {
    if (total_q < 0 || num_q_heads <= 0 || head_dim <= 0 || max_partitions <= 0 ||
        !tmp_out_bytes || !stats_bytes)
        return PA_EINVAL;
    const size_t rows = (size_t)total_q * num_q_heads * max_partitions;
    *tmp_out_bytes = rows * head_dim * sizeof(float);
    *stats_bytes = rows * sizeof(float);
    return PA_OK;
}

int pa_reshape_and_cache(const void *key, const void *value, void *key_cache, void *value_cache,
                         const int64_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t dtype,
                         int32_t kv_dtype, const float *k_scale, const float *v_scale,
                         void *stream) {
    try {
        const int eb = elt_bytes(dtype);
        if (!eb) return PA_EUNSUPPORTED;
        const int kst = check_kv(dtype, kv_dtype, k_scale, v_scale);
        if (kst != PA_OK) return kst;
        if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 ||
            block_size <= 0)
            return PA_EINVAL;
        if (num_tokens == 0) return PA_OK;
        if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_EINVAL;
        const bool kv8 = kv_dtype == PA_FP8_E4M3;
        const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * (kv8 ? 1 : eb);
        if (row_bytes % 16 != 0 || row_bytes > (1 << 30)) return PA_EUNSUPPORTED;
        if (kv8 && head_dim % 16 != 0) return PA_EUNSUPPORTED;
        if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) ||
            !aligned16(value_cache))
            return PA_EINVAL;
        if (kv8)
            return hip_status(pa::launch_quantize_cache(
                key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale, num_tokens,
                (int32_t)row_bytes, head_dim, (int64_t)num_blocks * block_size, dtype == PA_F32,
                (hipStream_t)stream));
        return hip_status(pa::launch_reshape_and_cache(
            key, value, key_cache, value_cache, slot_mapping, num_tokens, (int32_t)row_bytes,
            (int64_t)num_blocks * block_size, (hipStream_t)stream));
    } catch (...) {
        return PA_EHIP;
    }
}

int pa_expand_block_tables(int32_t *dst, const int32_t *src, int32_t num_seqs, int32_t src_stride,
                           int32_t src_blocks, int32_t dst_stride, int32_t ratio, void *stream) {
    try {
        if (num_seqs < 0 || src_blocks < 0 || ratio <= 0 || src_stride < src_blocks ||
            (int64_t)dst_stride < (int64_t)src_blocks * ratio || num_seqs > GRID_YZ_MAX)
            return PA_EINVAL;
        if (num_seqs == 0 || src_blocks == 0) return PA_OK;
        if (!dst || !src) return PA_EINVAL;
        return hip_status(pa::launch_expand_block_tables(dst, src, num_seqs, src_stride,
                                                         src_blocks, dst_stride, ratio,
                                                         (hipStream_t)stream));
    } catch (...) {
        return PA_EHIP;
    }
}

}  // extern "C"

namespace {

int varlen_attention_impl(pa_dispatch_info &rec, void *out, const void *q, const void *key_cache,
                          const void *value_cache, const int32_t *cu_seqlens_q,
                          const int32_t *seq_lens, const int32_t *block_tables, int32_t num_seqs,
                          int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                          int32_t max_blocks_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t num_blocks, int32_t block_size, float scale,
                          const float *sinks, int32_t dtype, int32_t kv_dtype,
                          const float *k_scale, const float *v_scale, int32_t partition_size,
                          float *tmp_out, float *max_logits, float *exp_sums,
                          int32_t max_partitions, void *stream) {
    try {
        if (!elt_bytes(dtype)) return PA_EUNSUPPORTED;
        const int kst = check_kv(dtype, kv_dtype, k_scale, v_scale);
        if (kst != PA_OK) return kst;
        const bool kv8 = kv_dtype == PA_FP8_E4M3;
        if (kv8 && dtype != PA_BF16) return PA_EUNSUPPORTED;
        if (num_seqs < 0 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
            num_blocks <= 0 || block_size <= 0 || head_dim <= 0 || max_blocks_per_seq < 0)
            return PA_EINVAL;
        if (num_q_heads % num_kv_heads != 0) return PA_EINVAL;
        if (!std::isfinite(scale)) return PA_EINVAL;
        const int32_t group = num_q_heads / num_kv_heads;
        if (group > PA_MAX_GROUP) return PA_EUNSUPPORTED;
        if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_EUNSUPPORTED;
        const int lbs = log2_exact(block_size);
        if (block_size < 8 || block_size > 32 || lbs < 0) return PA_EUNSUPPORTED;
        if (partition_size != 0 && !partition_ok(partition_size)) return PA_EUNSUPPORTED;
        if (partition_size != 0 && split_disabled_by_env()) {
            partition_size = 0;
            rec.split_disabled = 1;
        }
        rec.partition_size = partition_size;
        if (total_q == 0 || num_seqs == 0) return PA_OK;
        if (num_seqs > GRID_YZ_MAX || num_kv_heads > GRID_YZ_MAX) return PA_EUNSUPPORTED;
        if (max_q_len < 1 || max_seq_len < max_q_len) return PA_EINVAL;
        if ((int64_t)max_blocks_per_seq * block_size < max_seq_len) return PA_EINVAL;
        if (!out || !q || !key_cache || !value_cache || !cu_seqlens_q || !seq_lens ||
            !block_tables)
            return PA_EINVAL;
        if (!aligned16(out) || !aligned16(q) || !aligned16(key_cache) || !aligned16(value_cache))
            return PA_EINVAL;
        if (reinterpret_cast<uintptr_t>(sinks) % alignof(float) != 0) return PA_EINVAL;
        const int st = check_partitions(partition_size, max_seq_len, tmp_out, max_logits,
                                        exp_sums, max_partitions);
        if (st != PA_OK) return st;

        pa::AttnParams p{};
        p.out = out;
        p.q = q;
        p.kc = key_cache;
        p.vc = value_cache;
        p.cu_q = cu_seqlens_q;
        p.seq_lens = seq_lens;
        p.bt = block_tables;
        p.tmp_out = tmp_out;
        p.max_logits = max_logits;
        p.exp_sums = exp_sums;
        p.num_seqs = num_seqs;
        p.total_q = total_q;
        p.max_q_len = max_q_len;
        p.max_seq_len = max_seq_len;
        p.bt_stride = max_blocks_per_seq;
        p.hq = num_q_heads;
        p.hkv = num_kv_heads;
        p.group = group;
        p.head_dim = head_dim;
        p.num_blocks = num_blocks;
        p.block_size = block_size;
        p.log2_bs = lbs;
        p.partition = partition_size;
        p.max_parts = partition_size ? max_partitions : 1;
        p.scale_log2 = scale * 1.44269504088896340736f;
        p.sinks = sinks;
        p.dtype = dtype;
        p.kv8 = kv8;
        p.k_scale = kv8 ? k_scale : nullptr;
        p.v_scale = kv8 ? v_scale : nullptr;

        // One query token per request -> the decode kernels (bf16 MFMA for bf16
        // caches, vector ALUs for 8-bit caches and fp32).  fp32 batches with
        // longer windows also use the latter, one workgroup per query token;
        // bf16 prefill and mixed batches (bf16 or 8-bit caches) go to the MFMA
        // tiles.
        if (max_q_len == 1 || dtype == PA_F32) {
            if (kv8 ? !pa::decode_kv8_supported(head_dim, group)
                    : !pa::decode_supported(dtype, head_dim, group))
                return PA_EUNSUPPORTED;
            p.per_token = max_q_len > 1;
            if (p.per_token && total_q > GRID_YZ_MAX) return PA_EUNSUPPORTED;
            const int64_t parts =
                partition_size ? ((int64_t)max_seq_len + partition_size - 1) / partition_size : 1;
            if (parts > GRID_YZ_MAX) return PA_EUNSUPPORTED;
            pa::LaunchInfo li{};
            const int lst = hip_status(pa::launch_decode(p, (hipStream_t)stream, &li));
            record_launch(rec, p.per_token ? PA_PATH_DECODE_TOKEN : PA_PATH_DECODE, li);
            return lst;
        }
        if (!(kv8 ? pa::prefill_kv8_supported(head_dim, group)
                  : pa::prefill_supported(dtype, head_dim, group)))
            return PA_EUNSUPPORTED;
        pa::LaunchInfo li{};
        const int lst = hip_status(pa::launch_prefill(p, (hipStream_t)stream, &li));
        record_launch(rec, PA_PATH_TILED, li);
        return lst;
    } catch (...) {
        return PA_EHIP;
    }
}

int split_kv_reduce_impl(pa_dispatch_info &rec, void *out, const float *tmp_out,
                         const float *max_logits, const float *exp_sums,
                         const int32_t *cu_seqlens_q, const int32_t *seq_lens, int32_t num_seqs,
                         int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                         const float *sinks, int32_t partition_size, int32_t max_partitions,
                         int32_t dtype, void *stream) {
    try {
        if (!elt_bytes(dtype)) return PA_EUNSUPPORTED;
        if (num_seqs < 0 || total_q < 0 || num_q_heads <= 0 || head_dim <= 0) return PA_EINVAL;
        if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_EUNSUPPORTED;
        if (!partition_ok(partition_size)) return PA_EUNSUPPORTED;
        if (split_disabled_by_env()) {  // attention finished every row in place
            rec.path = PA_PATH_REDUCE_SKIP;
            rec.split_disabled = 1;
            return PA_OK;
        }
        rec.partition_size = partition_size;
        if (total_q == 0 || num_seqs == 0) return PA_OK;
        if (num_q_heads > GRID_YZ_MAX) return PA_EUNSUPPORTED;
        if (!out || !cu_seqlens_q || !seq_lens) return PA_EINVAL;
        if (!tmp_out || !max_logits || !exp_sums || max_partitions <= 0) return PA_EWORKSPACE;
        if (!aligned16(out) || !aligned16(tmp_out)) return PA_EINVAL;
        if (reinterpret_cast<uintptr_t>(sinks) % alignof(float) != 0) return PA_EINVAL;
        pa::ReduceParams p{};
        p.out = out;
        p.tmp_out = tmp_out;
        p.max_logits = max_logits;
        p.exp_sums = exp_sums;
        p.cu_q = cu_seqlens_q;
        p.seq_lens = seq_lens;
        p.num_seqs = num_seqs;
        p.total_q = total_q;
        p.hq = num_q_heads;
        p.head_dim = head_dim;
        p.partition = partition_size;
        p.max_parts = max_partitions;
        p.sinks = sinks;
        p.dtype = dtype;
        pa::LaunchInfo li{};
        const int st = hip_status(pa::launch_reduce(p, (hipStream_t)stream, &li));
        record_launch(rec, li.form ? PA_PATH_REDUCE_SLICES : PA_PATH_REDUCE_ROWS, li);
        return st;
    } catch (...) {
        return PA_EHIP;
    }
}

}  // namespace

extern "C" {

int pa_varlen_attention(void *out, const void *q, const void *key_cache, const void *value_cache,
                        const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                        const int32_t *block_tables, int32_t num_seqs, int32_t total_q,
                        int32_t max_q_len, int32_t max_seq_len, int32_t max_blocks_per_seq,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t num_blocks, int32_t block_size, float scale,
                        const float *sinks, int32_t dtype, int32_t kv_dtype,
                        const float *k_scale, const float *v_scale, int32_t partition_size,
                        float *tmp_out, float *max_logits, float *exp_sums,
                        int32_t max_partitions, void *stream) {
    pa_dispatch_info rec{};
    rec.status = varlen_attention_impl(
        rec, out, q, key_cache, value_cache, cu_seqlens_q, seq_lens, block_tables, num_seqs,
        total_q, max_q_len, max_seq_len, max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim,
        num_blocks, block_size, scale, sinks, dtype, kv_dtype, k_scale, v_scale, partition_size,
        tmp_out, max_logits, exp_sums, max_partitions, stream);
    g_last = rec;
    return rec.status;
}

int pa_split_kv_reduce(void *out, const float *tmp_out, const float *max_logits,
                       const float *exp_sums, const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                       int32_t num_seqs, int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                       const float *sinks, int32_t partition_size, int32_t max_partitions,
                       int32_t dtype, void *stream) {
    pa_dispatch_info rec{};
    rec.status = split_kv_reduce_impl(rec, out, tmp_out, max_logits, exp_sums, cu_seqlens_q,
                                      seq_lens, num_seqs, total_q, num_q_heads, head_dim, sinks,
                                      partition_size, max_partitions, dtype, stream);
    g_last = rec;
    return rec.status;
}

int pa_varlen_attention_noalloc(void *out, const void *q, const void *key_cache,
                                const void *value_cache, const int32_t *cu_seqlens_q,
                                const int32_t *seq_lens, const int32_t *block_tables,
                                int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                int32_t max_seq_len, int32_t max_blocks_per_seq,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t num_blocks, int32_t block_size, float scale,
                                const float *sinks, int32_t dtype, int32_t kv_dtype,
                                const float *k_scale, const float *v_scale,
                                int32_t partition_size, void *stream) {
    pa_dispatch_info rec{};
    rec.status = [&]() -> int {
        try {
            float *tmp = nullptr, *ml = nullptr, *es = nullptr;
            int32_t parts = 0;
            if (partition_size != 0 && !split_disabled_by_env()) {
                // Size the partials before anything is enqueued; the checks
                // pa_varlen_attention makes itself come first.
                if (!partition_ok(partition_size)) return PA_EUNSUPPORTED;
                if (total_q < 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len < 0)
                    return PA_EINVAL;
                if (num_q_heads > GRID_YZ_MAX) return PA_EUNSUPPORTED;
                parts = (int32_t)(((int64_t)max_seq_len + partition_size - 1) / partition_size);
                if (parts < 1) parts = 1;
                const uint64_t rows = (uint64_t)total_q * num_q_heads * parts;
                auto up = [](uint64_t b) { return (b + 255) & ~(uint64_t)255; };
                const uint64_t tmp_b = up(rows * head_dim * 4), st_b = up(rows * 4);
                if (tmp_b + 2 * st_b > PA_NOALLOC_SCRATCH_BYTES) return PA_EWORKSPACE;
                void *base = nullptr;
                if (pa::noalloc_scratch(&base) != hipSuccess || !base) return PA_EHIP;
                tmp = static_cast<float *>(base);
                ml = reinterpret_cast<float *>(static_cast<char *>(base) + tmp_b);
                es = reinterpret_cast<float *>(static_cast<char *>(base) + tmp_b + st_b);
            }
            const int st = varlen_attention_impl(
                rec, out, q, key_cache, value_cache, cu_seqlens_q, seq_lens, block_tables,
                num_seqs, total_q, max_q_len, max_seq_len, max_blocks_per_seq, num_q_heads,
                num_kv_heads, head_dim, num_blocks, block_size, scale, sinks, dtype, kv_dtype,
                k_scale, v_scale, parts ? partition_size : 0, tmp, ml, es, parts, stream);
            if (st != PA_OK || !parts || total_q == 0 || num_seqs == 0) return st;
            pa_dispatch_info rrec{};
            return split_kv_reduce_impl(rrec, out, tmp, ml, es, cu_seqlens_q, seq_lens, num_seqs,
                                        total_q, num_q_heads, head_dim, sinks, partition_size,
                                        parts, dtype, stream);
        } catch (...) {
            return PA_EHIP;
        }
    }();
    g_last = rec;
    return rec.status;
}

int pa_last_dispatch(pa_dispatch_info *info) {
    if (!info) return PA_EINVAL;
    *info = g_last;
    return PA_OK;
}

// Device address of memory the GPU may touch: device memory as is, pinned
// host memory through its mapping; nullptr for pageable host memory.
static void *device_address(const void *ptr) {
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, ptr) != hipSuccess) {
        (void)hipGetLastError();  // clear the query's error
        return nullptr;
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) return const_cast<void *>(ptr);
    if (a.type == hipMemoryTypeHost && a.devicePointer && a.hostPointer)
        return static_cast<char *>(a.devicePointer) +
               (static_cast<const char *>(ptr) - static_cast<const char *>(a.hostPointer));
    return nullptr;
}

int pa_copy_blocks(void *dst_key, void *dst_value, const void *src_key, const void *src_value,
                   const int64_t *pairs, int32_t num_pairs, int64_t block_bytes,
                   int64_t num_src_blocks, int64_t num_dst_blocks, void *stream) {
    try {
        if (num_pairs < 0 || block_bytes <= 0 || block_bytes % 16 != 0 || num_src_blocks < 0 ||
            num_dst_blocks < 0)
            return PA_EINVAL;
        if (num_pairs == 0) return PA_OK;
        if (num_pairs > 65535 * 256 || num_src_blocks > INT64_MAX / block_bytes ||
            num_dst_blocks > INT64_MAX / block_bytes)
            return PA_EINVAL;
        if (!dst_key || !dst_value || !src_key || !src_value || !pairs) return PA_EINVAL;
        if (!aligned16(dst_key) || !aligned16(dst_value) || !aligned16(src_key) ||
            !aligned16(src_value) || reinterpret_cast<uintptr_t>(pairs) % 8 != 0)
            return PA_EINVAL;
        void *dk = device_address(dst_key), *dv = device_address(dst_value);
        void *sk = device_address(src_key), *sv = device_address(src_value);
        void *pr = device_address(pairs);
        if (!dk || !dv || !sk || !sv || !pr) return PA_EINVAL;
        return hip_status(pa::launch_copy_blocks(dk, dv, sk, sv, static_cast<const int64_t *>(pr),
                                                 num_pairs, block_bytes, num_src_blocks,
                                                 num_dst_blocks, (hipStream_t)stream));
    } catch (...) {
        return PA_EHIP;
    }
}

int32_t pa_pick_partition_size(const int32_t *host_seq_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t dtype, int32_t kv_dtype,
                               int32_t num_cus) {
    try {
        if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
            num_q_heads % num_kv_heads != 0 || block_size <= 0 || !elt_bytes(dtype) ||
            (kv_dtype != dtype && kv_dtype != PA_FP8_E4M3) || (num_seqs > 0 && !host_seq_lens))
            return -1;
        if (num_cus <= 0) {
            int dev = 0;
            if (hipGetDevice(&dev) != hipSuccess) return -1;
            if (hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess)
                return -1;
        }
        int32_t max_len = 0;
        for (int32_t r = 0; r < num_seqs; ++r) {
            if (host_seq_lens[r] < 0) return -1;
            max_len = host_seq_lens[r] > max_len ? host_seq_lens[r] : max_len;
        }
        if (max_len <= 256) return 0;
        // The decode kernel each partition size routes to (the same rule the
        // launch applies): whole-row (one workgroup per request and
        // partition) or per KV head (one per KV head, request and partition).
        pa::AttnParams p{};
        p.num_seqs = num_seqs;
        p.max_seq_len = max_len;
        p.hq = num_q_heads;
        p.hkv = num_kv_heads;
        p.group = num_q_heads / num_kv_heads;
        p.head_dim = head_dim;
        p.block_size = block_size;
        p.dtype = dtype;
        p.kv8 = kv_dtype == PA_FP8_E4M3;
        auto rows_kernel = [&](int32_t P) {
            p.partition = P;
            return pa::decode_rows_supported(p);
        };
        const int64_t budget = (int64_t)num_cus * PA_SPLIT_FILL_NUM / PA_SPLIT_FILL_DEN;
        // A partition size qualifies when its launch has at least `budget`
        // workgroups and no workgroup streams more than 3/2 of the mean key
        // count (unequal items leave CUs idle while the longest finishes).
        auto qualifies = [&](int32_t P) {
            int64_t items = 0, keys = 0;
            int32_t longest = 0;
            for (int32_t r = 0; r < num_seqs; ++r) {
                const int32_t L = host_seq_lens[r];
                if (L <= 0) continue;
                items += P ? (L + P - 1) / P : 1;
                keys += L;
                const int32_t lk = P && L > P ? P : L;
                longest = lk > longest ? lk : longest;
            }
            if (!items) return false;
            const int64_t wgs = rows_kernel(P) ? items : items * num_kv_heads;
            return wgs >= budget && (int64_t)longest * items * PA_SPLIT_BALANCE_DEN <=
                                        keys * PA_SPLIT_BALANCE_NUM;
        };
        static const int32_t order[] = {0, 8192, 4096, 2048, 1024, 512};
        // Whole-row launches stream whole cache rows, faster per byte than
        // per-head slices: where the head shape allows them, the sizes that
        // route there are tried first.
        bool any_rows = false;
        for (int32_t P : order) any_rows = any_rows || ((P == 0 || P < 2 * max_len) && rows_kernel(P));
        for (int pass = any_rows ? 0 : 1; pass < 2; ++pass)
            for (int32_t P : order) {
                if (P && P >= 2 * max_len) continue;  // one partition per request: as P = 0
                if (pass == 0 && !rows_kernel(P)) continue;
                if (qualifies(P)) return P;
            }
        return 256;
    } catch (...) {
        return -1;
    }
}

}  // extern "C"
