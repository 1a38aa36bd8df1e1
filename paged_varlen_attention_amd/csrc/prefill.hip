// prefill.hip -- tiled bf16-MFMA paged attention for prefill and mixed batches.
//
// What it computes follows the pages: packed varlen queries [total_q, Hq, D]
// with request boundaries in cu_seqlens (v0.28.0 release post, "Packed queries
// and paged KV"), keys and values read through each request's block table
// (kernel walkthrough, "What is Paged Attention"), query heads of one GQA group
// sharing a KV head, each request's new tokens causally masked against its
// cached prefix (bottom-right: query j at position ctx + j sees keys 0..ctx+j),
// and a FlashAttention-2 style tiled online softmax (kernel walkthrough, "three
// Metal kernels": the tiled prefill kernel) in log2 space.
//
// The design is our own for CDNA4 (gfx950):
//  * one workgroup = one q-tile of one request x one KV head (x one split-KV
//    partition); 4 waves (8 at D = 256 on large batches) x 32 rows, the rows
//    being (token, head-of-group) pairs, so every K/V tile loaded serves the
//    whole GQA group;
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: Q^T stays in registers as the
//    B operand for the whole key loop, K tiles are the A operand read from LDS;
//    a lane's accumulator column is one query row, so the softmax statistics
//    are per lane plus one v_permlane32_swap;
//  * O^T += V^T P^T: P^T comes straight from the S^T accumulator registers and
//    the V^T A-operand fragments come from the row-major V tile through
//    ds_read_b64_tr_b16 (gfx950's LDS transpose read), so V needs no transpose
//    pass;
//  * K and V tiles move HBM -> LDS by global_load_lds_dwordx4 into a
//    swizzled piece-major layout (bank-conflict-free fragment reads);
//    NST stages, one barrier per N-key tile;
//  * requests are mapped to workgroups without a host pass: virtual tile x
//    belongs to the last request r with cu[r]/BQ + r <= x (surplus tiles exit);
//  * 8-bit E4M3 caches (the library's own KV quantisation): tiles arrive by
//    DMA as raw codes (key rows in key order, 16-byte pieces swizzled by key;
//    one instruction = whole rows of one page), and the fragment reads take
//    them directly -- K by ds_read_b64, V^T by ds_read_b64_tr_b8 (8 keys x 1
//    dim per lane, the same k-slots as the bf16 path) -- widened in registers
//    by v_cvt_scalef32_pk_bf16_fp8 (exact) right before their MFMA; V codes
//    of keys past the sequence are zeroed in registers.  Half the LDS bytes
//    and no conversion pass: the same one barrier per tile as bf16 caches.
//    The head's K scale joins the softmax scale and its V scale the final
//    normaliser.
#include "prefill_tile.h"

namespace pa {
namespace {

// Keys per tile and LDS stages by head size.  Waves per workgroup: 4, or at
// D >= 128 on large batches over bf16 caches 8 (one workgroup per CU, each
// K/V tile in LDS serving 256 rows): 5% faster on long uniform prompts at
// D = 256 and 6% at D = 128 (8 x 4,096 new tokens over 4,096 cached: 1.55
// against 1.65 ms), but 3-4% slower on ragged batches of a few hundred
// workgroups, whose critical path the larger q-tiles lengthen.  The switch is at PREFILL_WIDE_ITEMS work
// items of 8-wave size (4 per CU on 256 CUs).  The 8-wave form (one
// workgroup per CU) has the LDS for a third stage.  Over 8-bit caches the
// 8-wave form runs short of registers (3 stages: spills inside the key loop,
// 4,057 against 2,984 us on the uniform prefill; 2 stages: 3,135-3,146
// against 3,083-3,106 us for 4 waves), so 8-bit caches keep 4 waves.
constexpr int PREFILL_WIDE_ITEMS = 1024;
constexpr int prefill_n(int D) { return D >= 256 ? 32 : 64; }

template <int D, bool KV8, int NWV>
hipError_t launch_dw(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    return launch_tiles<D, prefill_n(D), NWV == 8 ? 3 : 2, KV8, NWV, 1>(p, stream, li);
}

template <int D, bool KV8>
hipError_t launch_d(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    if constexpr (D >= 128 && !KV8) {
        const int64_t bq8 = 8 * (32 / p.group);
        const int64_t parts = p.partition ? (p.max_seq_len + p.partition - 1) / p.partition : 1;
        const int64_t items8 = (p.total_q / bq8 + p.num_seqs) * p.hkv * parts;
        if (items8 >= PREFILL_WIDE_ITEMS) return launch_dw<D, KV8, 8>(p, stream, li);
    }
    return launch_dw<D, KV8, 4>(p, stream, li);
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int group) {
    return dtype == 1 && (head_dim == 64 || head_dim == 128 || head_dim == 256) && group >= 1 &&
           group <= 8;
}

bool prefill_kv8_supported(int head_dim, int group) {
    return (head_dim == 64 || head_dim == 128 || head_dim == 256) && group >= 1 && group <= 8;
}

hipError_t launch_prefill(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    if (p.kv8) {
        switch (p.head_dim) {
            case 64: return launch_d<64, true>(p, stream, li);
            case 128: return launch_d<128, true>(p, stream, li);
            case 256: return launch_d<256, true>(p, stream, li);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.head_dim) {
        case 64: return launch_d<64, false>(p, stream, li);
        case 128: return launch_d<128, false>(p, stream, li);
        case 256: return launch_d<256, false>(p, stream, li);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
