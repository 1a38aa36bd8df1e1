// prefill_tile.h -- the tiled bf16-MFMA attention kernel template and its
// launcher (instantiated in prefill.hip; what it computes and how is
// described there).  RB is the number of 32-row column blocks a wave holds;
// every K and V^T fragment read from LDS feeds RB MFMAs.  The library builds
// RB = 1: two blocks per wave (64 query rows, one wave per SIMD, accumulators
// in AGPRs) were parity-green but 19% slower on uniform D = 128 prefill and
// spilled at D = 256, since one wave per SIMD leaves the LDS and MFMA
// latencies exposed.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units

template <int D, int N_, int NST_, bool KV8_ = false, int NWV_ = 4, int RB_ = 1>
struct PrefillCfg {
    static constexpr bool KV8 = KV8_;             // caches hold E4M3 codes
    static constexpr int NWV = NWV_;              // waves per workgroup (4 or 8)
    static constexpr int RB = RB_;                // 32-row column blocks per wave (1 or 2)
    static constexpr int NTH = NWV * 64;          // threads per workgroup
    static constexpr int N = N_;                  // keys per tile
    static constexpr int NST = NST_;              // LDS stages
    static constexpr int NB = N / 32;             // 32-key blocks of S^T per tile
    static constexpr int R = D * 2;               // bytes of a K/V row of one head
    static constexpr int KS = D / 16;             // MFMA k-steps of QK^T
    static constexpr int DB = D / 32;             // 32-row blocks of O^T
    static constexpr int T_BYTES = N * R;         // one K (or V) tile
    static constexpr int STAGE = 2 * T_BYTES;     // K tile, then V tile
    static constexpr int PPR = R / 16;            // 16-byte pieces per row
    static constexpr int KG = 8;                  // keys per group in the tile layout
    static constexpr int GROUP_BYTES = KG * R;    // one key group: PPR pieces x KG keys
    static constexpr int IPG = GROUP_BYTES / 1024;  // DMA instructions per key group
    static constexpr int NI = T_BYTES / 1024;     // DMA instructions per tile
    static constexpr int NI_W = NI / NWV;         // per wave, per tensor
    // 8-bit caches: NST stages of raw tiles (K tile, then V tile, N*D bytes
    // each, row-major by key with swizzled 16-byte pieces) that the MFMA
    // fragment reads take directly
    static constexpr int RG = KV8 ? D : R;        // bytes of a cached K/V row of one head
    static constexpr int RAW_T = N * D;           // one 8-bit tile
    static constexpr int RAW_STAGE = 2 * RAW_T;
    // 8-bit DMA: D >= 128 moves 1024 / D whole rows per instruction (16 bytes
    // a lane); 64-byte rows (D = 64) move 4 rows per instruction (4 bytes a
    // lane).  Either way an instruction never spans two pages.
    static constexpr bool ROWS8 = D < 128;
    static constexpr int DW8 = ROWS8 ? 4 : 16;
    static constexpr int RPI8 = 64 * DW8 / D;     // rows per 8-bit DMA instruction
    static constexpr int PPR8 = D / 16;           // 16-byte pieces per 8-bit row
    static constexpr int NI8_W = RAW_T / (64 * DW8) / NWV;  // per wave, per tensor, 8-bit
    static constexpr int LDS_BYTES = KV8 ? NST * RAW_STAGE : NST * STAGE;
    static_assert(!KV8 || ((D == 64 || D >= 128) && RAW_T % (64 * DW8 * NWV) == 0),
                  "8-bit tile shape");
    static_assert(NI % NWV == 0, "tile split over the waves");
    static_assert(RB == 1 || (RB == 2 && !KV8 && NWV == 4), "two row blocks: bf16 caches, 4 waves");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(2 * NI_W * (NST - 1) < 64, "vmcnt range");
    static_assert(2 * NI8_W * (NST - 1) < 64, "vmcnt range");
};

// Tile layout in LDS (K and V alike).  Keys come in groups of KG = 8; a
// group stores piece-major: piece p (16 bytes: elements 8p..8p+7) of its 8
// keys is one 128-byte line.  Odd key groups store the two lines of each
// piece pair swapped (stored piece s = p ^ (group & 1)), and the key slot is
// XORed with 4 when bits 0 and 1 of s differ:
//   off(key, p) = (key / 8) * 8R + s * 128 + ((key % 8) ^ 4 ((s ^ s / 2) & 1)) * 16.
// The LDS serves 256 bytes (64 banks) a cycle, so every 16 lanes of a
// ds_read_b128 and every 32 lanes of a ds_read_b64_tr_b16 must cover all
// banks (the counters showed half of the LDS cycles lost to conflicts with
// the plain piece-major layout; with this one there are none):
// * S^T A operand (ds_read_b128): 8 consecutive lanes read 8 keys of one
//   piece -- one line -- and the next 8 lanes the same piece of the next key
//   group, which the swap puts on the other half of the banks; the address
//   changes with the k-step by an immediate (two bases, by k-step parity).
// * V^T A operand (ds_read_b64_tr_b16): 32 lanes read 4 keys x 4 adjacent
//   pieces; the slot XOR puts the four 64-byte runs on four bank quarters.
// * DMA: one global_load_lds_dwordx4 fills 1 KB = 8 pieces of one key group
//   with 128 contiguous bytes of each key row (one 8-key group never spans
//   two pages since pages hold a multiple of 8 keys); a lane's source offset
//   inside the page is one of two values (even or odd key group).
template <class C>
__device__ __forceinline__ int tile_off(int key, int piece) {
    const int sp = piece ^ ((key >> 3) & 1);  // odd key groups swap the lines of a piece pair
    return (key >> 3) * C::GROUP_BYTES + sp * 128 + (((key & 7) ^ (((sp ^ (sp >> 1)) & 1) << 2)) << 4);
}

// 8-bit tile layout in LDS (K and V alike): key rows of D bytes in key order;
// the 16-byte piece p of key k's row is stored at piece slot p ^ kv8_swz(k)
// (kv8_swz < D / 16 depends on bits 0-3 of the key only).  The LDS serves 256
// bytes a cycle; per 32 lanes:
// * K (S^T A operand, ds_read_b64): the 32 keys of a block, one 8-byte half
//   of one piece each.  Every 16-byte slot of the 256-byte bank window is hit
//   by exactly 2 keys -- the least possible, since a piece's other half is
//   not read -- so a read takes 4 cycles for 512 bytes, as the bf16 b128
//   reads take for 1 KB.
// * V^T (O^T A operand, ds_read_b64_tr_b8): in each 16 lanes, lanes 2m and
//   2m+1 point at the two halves of one piece of key row m, the 8 rows being
//   keys 4h .. 4h+3 and 8+4h .. 11+4h (the k-slot order of the bf16 path),
//   and the two 16-lane groups of a half wave read pieces 2db and 2db+1: the
//   swizzle gives the 16 (row, piece) pairs 16 distinct slots.
template <int D>
__device__ __forceinline__ int kv8_swz(int k) {
    if constexpr (D == 256) return ((k & 3) << 1) | (((k >> 3) & 1) << 3) | ((k >> 2) & 1);
    else if constexpr (D == 128) return (((k >> 1) & 1) << 1) | (((k >> 3) & 1) << 2) | ((k >> 2) & 1);
    else return (((k >> 3) & 1) << 1) | ((k >> 2) & 1);
}

// Wait until the DMA of the tile `ahead` tiles before the newest one landed.
template <int VM, int MAXA>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
    if constexpr (MAXA > 0) {
        if (ahead >= MAXA) {
            wait_vmcnt<MAXA * VM>();
            return;
        }
        wait_tiles_ahead<VM, MAXA - 1>(ahead);
    } else {
        wait_vmcnt<0>();
    }
}

// Waves per SIMD the register budget is sized for: 2 (at most 256 registers
// a lane; D = 256 keeps 192 of them for O^T and Q^T).
constexpr int PREFILL_WAVES_PER_SIMD = 2;

// LDS fragment reads in flight ahead of their MFMA (K for S^T, V^T for O^T).
constexpr int prefill_pf(int D) { return D >= 256 ? 2 : 4; }
// Consecutive work items kept on one XCD (its L2 serves their shared keys).
constexpr int XCD_CHUNK = 8;

template <int D, int N, int NST, bool KV8, int NWV, int RB>
__global__ __launch_bounds__(NWV * 64, RB == 1 ? PREFILL_WAVES_PER_SIMD * 4 / NWV : 1) void prefill_kernel(
    const AttnParams p) {
    using C = PrefillCfg<D, N, NST, KV8, NWV, RB>;
    constexpr int PF_K = prefill_pf(D), PF_V = prefill_pf(D);
    __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = p.group;
    const int TPW = 32 * RB / G;  // tokens per wave
    const int BQ = C::NWV * TPW;  // tokens per workgroup

    // ---- which request, q-tile, KV head and partition (XCD-aware order) ----
    // Workgroups go to the 8 XCDs round-robin by launch index L.  Work items
    // come in chunks of XCD_CHUNK consecutive virtual q-tiles of one (KV head,
    // partition) -- q-tiles of one request that read the same keys -- and each
    // chunk is kept on one XCD so its L2 serves the repeats; round k of the
    // launch hands chunks 8k..8k+7 to the 8 XCDs.  Chunks are taken last-first
    // (later q-tiles see more keys).
    // Unsplit launches interleave the KV heads chunk by chunk, so the longest
    // q-tiles of every head start first, and deal the rounds serpentine (XCD x
    // takes the x-th chunk of even rounds and the (7-x)-th of odd ones): costs
    // fall steadily along that order, and the two directions even them out
    // over the XCDs.  The deal starts at the last real q-tile, surplus virtual
    // tiles come last, so the pairing keeps its phase.
    // Against plain rounds with the surplus first, this deal measured 4-5%
    // faster on the uniform 8 x 4,096-token prefill and the mixed batch of
    // eight ~750-token prompts.  Split launches take the partitions slowest,
    // in plain rounds, which measured faster for them (the verify batch at
    // 1,024-key partitions: 99 against 115 us head-interleaved, 101 against
    // 106 serpentine).
    // (grid_tiles is a multiple of XCD_CHUNK.)
    const int n_items = p.grid_tiles * p.hkv * p.grid_parts;
    int lam;
    {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, round = slot / XCD_CHUNK;
        const int cx = (p.grid_parts == 1 && (round & 1)) ? 7 - xcd : xcd;
        lam = (round * 8 + cx) * XCD_CHUNK + slot % XCD_CHUNK;
    }
    if (lam >= n_items) return;
    // Up to 64 requests, the virtual tiles list the requests by key count,
    // fewest first, each with exactly its own q-tiles, so that the last-first
    // dispatch starts the requests with the most keys (and their longest
    // q-tiles) first -- a decode row over a long context costs as much as a
    // prompt's last q-tile and must not come last.  Every wave computes the
    // same table, one request per lane.  Beyond 64 requests request r owns
    // virtual tiles from cu_q[r] / BQ + r on (one more than it can fill).
    const bool listed = p.num_seqs <= 64;
    int start = 0, nt = 0, real_tiles = p.grid_tiles;
    int c0 = 0, ql = 0, sl = 0;  // listed: request `lane`'s first token, token and key counts
    if (listed) {
        const int i = lane;
        if (i < p.num_seqs) {
            c0 = p.cu_q[i];
            ql = p.cu_q[i + 1] - c0;
            sl = p.seq_lens[i];
        }
        nt = ql > 0 ? (ql + BQ - 1) / BQ : 0;
        real_tiles = 0;
        for (int j = 0; j < p.num_seqs; ++j) {
            const int slj = __builtin_amdgcn_readlane(sl, j);
            const int ntj = __builtin_amdgcn_readlane(nt, j);
            start += (slj < sl || (slj == sl && j < i)) ? ntj : 0;
            real_tiles += ntj;
        }
    }
    int part, kvh, x;
    if (p.grid_parts == 1) {
        const int chunk = lam / XCD_CHUNK;
        part = 0;
        kvh = chunk % p.hkv;
        const int xc = (real_tiles + XCD_CHUNK - 1) / XCD_CHUNK - 1 - chunk / p.hkv;
        if (xc < 0) return;  // surplus chunk
        x = xc * XCD_CHUNK + XCD_CHUNK - 1 - lam % XCD_CHUNK;
    } else {
        lam = n_items - 1 - lam;
        x = lam % p.grid_tiles;
        kvh = (lam / p.grid_tiles) % p.hkv;
        part = lam / (p.grid_tiles * p.hkv);
    }
    // (listed: the request's bounds come from the lane that loaded them, so
    // no second round of loads stands between the mapping and the first DMA)
    int r, tile, q_begin, q_len, seq_len;
    if (listed) {
        const uint64_t mine = __ballot(lane < p.num_seqs && x >= start && x < start + nt);
        if (!mine) return;  // surplus virtual tile
        r = (int)__builtin_ctzll(mine);
        tile = x - __builtin_amdgcn_readlane(start, r);
        q_begin = __builtin_amdgcn_readlane(c0, r);
        q_len = __builtin_amdgcn_readlane(ql, r);
        seq_len = __builtin_amdgcn_readlane(sl, r);
    } else {
        int lo = 0, hi = p.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.cu_q[mid] / BQ + mid <= x) lo = mid; else hi = mid - 1;
        }
        r = lo;
        tile = x - (p.cu_q[r] / BQ + r);
        q_begin = p.cu_q[r];
        q_len = p.cu_q[r + 1] - q_begin;
        seq_len = p.seq_lens[r];
    }
    const int j0 = tile * BQ;  // first token of the tile within the request
    if (tile < 0 || j0 >= q_len) return;
    const int ctx = seq_len - q_len;
    const int j_last = min(q_len, j0 + BQ) - 1;
    // keys of this workgroup: the partition, cut at the last token's position
    const int k_lo = p.partition ? part * p.partition : 0;
    const int k_part_end = p.partition ? k_lo + p.partition : seq_len;
    const int k_hi = min(k_part_end, ctx + j_last + 1);
    if (k_lo >= k_hi) return;

    // ---- this lane's query rows (column q of each of the RB S^T blocks):
    // row i = 32 blk + q of the wave is token i / G, head i % G ----
    const int q = lane & 31;
    const int h = lane >> 5;
    bool row_valid[RB];
    int pos[RB], t_glob[RB], head[RB];
#pragma unroll
    for (int blk = 0; blk < RB; ++blk) {
        const int ri = 32 * blk + q;
        const int tl = min(wave * TPW + ri / G, j_last - j0);  // padding rows repeat the last token
        row_valid[blk] = ri < TPW * G && j0 + wave * TPW + ri / G <= j_last;
        const int jq = j0 + tl;       // token index within the request
        pos[blk] = ctx + jq;          // absolute position: sees keys 0..pos
        t_glob[blk] = q_begin + jq;
        head[blk] = kvh * G + ri % G;
    }

    // Q^T B operand: 8 bf16 of d = 16*ks + 8*h .. +8 of this row, per k-step
    // A negative scale is folded into Q (flipping bf16 sign bits is exact), so
    // the running max can be taken on the raw scores and the scale applied
    // inside the exponent; a zero scale becomes the smallest normal float,
    // which leaves every visible weight exactly 1 and masked ones 0.
    // (8-bit caches: S holds code units of K, so the head's K scale joins it)
    const float sl2 =
        fmaxf(fabsf(p.scale_log2) * (KV8 ? p.k_scale[kvh] : 1.f),
              1.17549435e-38f);
    bf16x8_t qb[RB][C::KS];
    {
        const uint32_t flip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
        for (int blk = 0; blk < RB; ++blk) {
            const uint4 *qrow = reinterpret_cast<const uint4 *>(
                reinterpret_cast<const uint16_t *>(p.q) + ((size_t)t_glob[blk] * p.hq + head[blk]) * D);
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                uint4 v = qrow[2 * ks + h];
                v.x ^= flip; v.y ^= flip; v.z ^= flip; v.w ^= flip;
                qb[blk][ks] = __builtin_bit_cast(bf16x8_t, v);
            }
        }
    }

    // ---- block-table window: lane i holds page (win_page + i) of the request ----
    const int bs = p.block_size, lbs = p.log2_bs;
    const int seq_pages = (seq_len + bs - 1) >> lbs;
    const int32_t *bt_row = p.bt + (size_t)r * p.bt_stride;
    auto load_window = [&](int page0) {
        const int lp = page0 + lane;
        int v = lp < seq_pages && lp < p.bt_stride ? bt_row[lp] : 0;
        return v < 0 ? 0 : (v >= p.num_blocks ? p.num_blocks - 1 : v);
    };
    int win_page = k_lo >> lbs;
    int btv = load_window(win_page);

    const uint32_t row_stride = (uint32_t)p.hkv * C::RG;
    const uint64_t page_bytes = (uint64_t)bs * row_stride;
    const uint64_t head_off = (uint64_t)kvh * C::RG;
    const char *kc = reinterpret_cast<const char *>(p.kc);
    const int64_t v_minus_k = reinterpret_cast<const char *>(p.vc) - kc;

    // DMA: this wave moves instructions c = wave*NI_W + i of each tile.
    // Instruction c covers key group c / IPG, pieces 8*(c % IPG) .. +7; lane l
    // brings piece 8*(c % IPG) + l/8 of key slot l%8 (its key is the slot
    // XORed back, which is the same involution).
    const uint32_t dma_voff =
        (uint32_t)((lane & 7) ^ ((((lane >> 3) ^ (lane >> 4)) & 1) << 2)) * row_stride +
        (uint32_t)(lane >> 3) * 16u;
    // odd key groups: the line of stored piece 8q + l/8 holds piece 8q + (l/8 ^ 1)
    const uint32_t dma_voff_odd = dma_voff + (uint32_t)((((lane >> 3) ^ 1) - (lane >> 3)) * 16);
    const uint32_t lds0 = lds_addr(lds);

    auto issue = [&](int kt, int stage) {
        const int lp0 = kt >> lbs;
        if (lp0 + ((C::N - 1) >> lbs) - win_page >= 64) {  // long ranges: slide the window
            win_page = lp0;
            btv = load_window(win_page);
        }
#pragma unroll
        for (int i = 0; i < C::NI_W; ++i) {
            const int c = wave * C::NI_W + i;
            const int k8 = kt + C::KG * (c / C::IPG);  // first key of the group
            const int lp = min(k8 >> lbs, seq_pages - 1);
            const int phys = __builtin_amdgcn_readlane(btv, lp - win_page);
            const char *base = kc + (uint64_t)phys * page_bytes + head_off +
                               (uint32_t)(k8 & (bs - 1)) * row_stride + 128 * (c % C::IPG);
            const uint32_t l = lds0 + stage * C::STAGE + c * 1024;
            const uint32_t vo = ((c / C::IPG) & 1) ? dma_voff_odd : dma_voff;
            dma16(base, vo, l);
            dma16(base + v_minus_k, vo, l + C::T_BYTES);
        }
    };

    // 8-bit caches: instruction c of a raw tile covers key rows c RPI8 ..
    // c RPI8 + RPI8 - 1 and lands at c * 64 DW8 of the tile; lane l writes
    // slot l % PPR8 (16 bytes; D = 64: dword l % 4 of slot (l % 16) / 4) of
    // row l / (PPR8 or 16), fetching that row's piece slot ^ kv8_swz(row).
    uint32_t voff8[C::NI8_W];
#pragma unroll
    for (int i = 0; i < C::NI8_W; ++i) {
        const int c = wave * C::NI8_W + i;
        if constexpr (C::ROWS8) {
            const int row = 4 * c + (lane >> 4);
            voff8[i] = (uint32_t)(lane >> 4) * row_stride +
                       (uint32_t)((((lane & 15) >> 2) ^ kv8_swz<D>(row)) << 4) + (uint32_t)(lane & 3) * 4u;
        } else {
            const int row = C::RPI8 * c + lane / C::PPR8;
            voff8[i] = (uint32_t)(lane / C::PPR8) * row_stride +
                       (uint32_t)(((lane % C::PPR8) ^ kv8_swz<D>(row)) << 4);
        }
    }
    auto issue8 = [&](int kt, int stage) {
        const int lp0 = kt >> lbs;
        if (lp0 + ((C::N - 1) >> lbs) - win_page >= 64) {  // long ranges: slide the window
            win_page = lp0;
            btv = load_window(win_page);
        }
#pragma unroll
        for (int i = 0; i < C::NI8_W; ++i) {
            const int c = wave * C::NI8_W + i;
            const int k8 = kt + C::RPI8 * c;  // first key of the instruction
            const int lp = min(k8 >> lbs, seq_pages - 1);
            const int phys = __builtin_amdgcn_readlane(btv, lp - win_page);
            const char *base = kc + (uint64_t)phys * page_bytes + head_off +
                               (uint32_t)(k8 & (bs - 1)) * row_stride;
            const uint32_t l = lds0 + stage * C::RAW_STAGE + c * 64 * C::DW8;
            dma_lds<C::DW8>(base, voff8[i], l);
            dma_lds<C::DW8>(base + v_minus_k, voff8[i], l + C::RAW_T);
        }
    };

    // ---- online softmax state (column q) ----
    f32x16_t o[RB][C::DB];
#pragma unroll
    for (int blk = 0; blk < RB; ++blk)
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[blk][db][j] = 0.f;
    // m: reference max of the row's scaled scores (log2 units), shared by the
    // lane pair; it is only raised when a tile's max exceeds it by more than
    // RESCALE_THRESHOLD, so weights stay below 2^RESCALE_THRESHOLD.
    float m[RB], mtrue[RB], l[RB];  // reference max, true running max, this lane's half of the exp-sum
    int lim0[RB];
    const int k_vis_end = min(k_hi, seq_len);  // keys past this are never visible
#pragma unroll
    for (int blk = 0; blk < RB; ++blk) {
        m[blk] = NEG_INF;
        mtrue[blk] = NEG_INF;
        l[blk] = 0.f;
        // register j of key block b holds key kt + 32*b + 8*(j/4) + 4*h + (j%4);
        // it is visible when that offset from kt + 4*h is <= lim0 - kt
        lim0[blk] = min(pos[blk], k_vis_end - 1) - 4 * h;
    }

    // Per-lane LDS bases; everything else in a fragment address is an
    // immediate.  K: lane reads key 32b + (lane&31), piece 2ks + h.  V^T: in
    // each 16-lane group, lane s points at key 4h + s/4 (+ 8 for the second
    // read, + 16 per k-step, + 32 per block) and at d = 32db + 16*(group&1)
    // + 4*(s%4), i.e. piece 4db + 2*(group&1) + (s/2)%2, byte 8*(s%2).
    const int tg = lane >> 4;
    const int ts = lane & 15;
    const int kg = (lane & 31) >> 3;  // key group of the lane's key; odd ones swap line pairs
    const int kp = h ^ (kg & 1);
    // the key slot's XOR follows the parity of the stored piece's two low
    // bits, which alternates with the k-step
    const int k_base = kg * C::GROUP_BYTES + kp * 128 + (((lane & 7) ^ (kp << 2)) << 4);
    const int k_base_odd = kg * C::GROUP_BYTES + kp * 128 + (((lane & 7) ^ ((kp ^ 1) << 2)) << 4);
    const int v_pb = (ts >> 1) & 1;
    const int v_base = (2 * (tg & 1) + v_pb) * 128 +
                       (((4 * h + (ts >> 2)) ^ ((v_pb ^ (tg & 1)) << 2)) << 4) + 8 * (ts & 1);
    // the same key slot in the odd key group (key + 8): its piece pair swapped
    const int v_base_odd = C::GROUP_BYTES + (2 * (tg & 1) + (v_pb ^ 1)) * 128 +
                           (((4 * h + (ts >> 2)) ^ ((v_pb ^ 1 ^ (tg & 1)) << 2)) << 4) + 8 * (ts & 1);

    // 8-bit fragment bases (the k-step or dim block enters by an XOR of bits
    // 4..7, the key block and k-step pair by an immediate): K key lane & 31,
    // half h; V^T key row k0 of the lane's 16-lane group (the bf16 path's
    // k-slot order), piece 2db + (group & 1), half ts & 1.
    const int k8_base = (((lane & 31) * D + 8 * h) | (kv8_swz<D>(lane & 31) << 4));
    const int v8_k0 = (ts >> 1) < 4 ? 4 * h + (ts >> 1) : 8 + 4 * h + (ts >> 1) - 4;
    const int v8_base = ((v8_k0 * D + 8 * (ts & 1)) | (((tg & 1) ^ kv8_swz<D>(v8_k0)) << 4));

    const int ntiles = (k_hi - k_lo + C::N - 1) / C::N;
    constexpr int VM = 2 * C::NI_W;
    constexpr int VM8 = 2 * C::NI8_W;
    if constexpr (KV8) {
#pragma unroll
        for (int s = 0; s < NST - 1; ++s)
            if (s < ntiles) issue8(k_lo + s * C::N, s);
    } else {
#pragma unroll
        for (int s = 0; s < NST - 1; ++s)
            if (s < ntiles) issue(k_lo + s * C::N, s);
    }

    for (int it = 0; it < ntiles; ++it) {
        const int kt = k_lo + it * C::N;
        const int stage = it % NST;
        const char *kst;
        char *vst;
        if constexpr (KV8) {
            if (it + NST - 1 < ntiles) issue8(kt + (NST - 1) * C::N, (it + NST - 1) % NST);
            wait_tiles_ahead<VM8, NST - 1>(min(NST - 1, ntiles - 1 - it));
            kst = lds + stage * C::RAW_STAGE;
            vst = const_cast<char *>(kst) + C::RAW_T;
            __syncthreads();  // every wave's DMA share of this tile is in
        } else {
            if (it + NST - 1 < ntiles) issue(kt + (NST - 1) * C::N, (it + NST - 1) % NST);
            wait_tiles_ahead<VM, NST - 1>(min(NST - 1, ntiles - 1 - it));
            kst = lds + stage * C::STAGE;
            vst = const_cast<char *>(kst) + C::T_BYTES;
            if (kt + C::N > seq_len) {
                // V rows past the sequence may hold anything (NaN): zero them, since
                // p = 0 does not cancel a NaN inside the MFMA
                __syncthreads();
                for (int i = threadIdx.x; i < C::N * C::PPR; i += C::NTH) {
                    const int row = i / C::PPR;
                    if (kt + row >= seq_len)
                        *reinterpret_cast<uint4 *>(vst + tile_off<C>(row, i % C::PPR)) =
                            make_uint4(0, 0, 0, 0);
                }
            }
            __syncthreads();  // every wave's DMA share of this tile is in
        }

        // ---- S^T = K Q^T, 32-key blocks ----
        // K fragments are streamed PF_K reads ahead of their MFMA (the
        // scheduling barriers keep the compiler from hoisting all of them,
        // which would cost registers the occupancy target does not have)
        f32x16_t s[RB][C::NB];
#pragma unroll
        for (int b = 0; b < C::NB; ++b) {
#pragma unroll
            for (int blk = 0; blk < RB; ++blk) s[blk][b] = f32x16_t{};
            // (8-bit caches: the raw 8 codes are in flight, widened at use)
            using KFrag = std::conditional_t<KV8, uint2, uint4>;
            auto kread = [&](int ks) -> KFrag {
                if constexpr (KV8)
                    return *reinterpret_cast<const uint2 *>(kst + (k8_base ^ (ks << 4)) + b * 32 * D);
                else
                    return *reinterpret_cast<const uint4 *>(kst + ((ks & 1) ? k_base_odd : k_base) +
                                                            b * 4 * C::GROUP_BYTES + ks * 256);
            };
            KFrag ka[PF_K];
#pragma unroll
            for (int ks = 0; ks < PF_K; ++ks) ka[ks] = kread(ks);
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                uint4 a;
                if constexpr (KV8)
                    a = __builtin_bit_cast(uint4, e4m3x8_to_bf16(ka[ks % PF_K].x, ka[ks % PF_K].y));
                else
                    a = ka[ks % PF_K];
                if (ks + PF_K < C::KS) ka[ks % PF_K] = kread(ks + PF_K);
                // one K fragment serves every row block of the wave
#pragma unroll
                for (int blk = 0; blk < RB; ++blk)
                    s[blk][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, a), qb[blk][ks], s[blk][b], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // ---- mask (boundary tiles only), online softmax on raw scores ----
        if (kt + C::N - 1 > ctx + j0 || kt + C::N > k_vis_end) {
#pragma unroll
            for (int blk = 0; blk < RB; ++blk) {
                const int lim = lim0[blk] - kt;
#pragma unroll
                for (int b = 0; b < C::NB; ++b)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        if (32 * b + 8 * (j >> 2) + (j & 3) > lim) s[blk][b][j] = NEG_INF;
            }
        }
        float mx[RB];
        bool up_any = false;
#pragma unroll
        for (int blk = 0; blk < RB; ++blk) {
            mx[blk] = NEG_INF;
#pragma unroll
            for (int b = 0; b < C::NB; ++b)
#pragma unroll
                for (int j = 0; j < 16; ++j) mx[blk] = fmaxf(mx[blk], s[blk][b][j]);
            const RowPair pm = row_pair32(mx[blk]);
            mx[blk] = fmaxf(pm.a, pm.b) * sl2;
            mtrue[blk] = fmaxf(mtrue[blk], mx[blk]);
            up_any = up_any || mx[blk] > m[blk] + RESCALE_THRESHOLD;
        }
        if (__builtin_amdgcn_ballot_w64(up_any)) {
#pragma unroll
            for (int blk = 0; blk < RB; ++blk) {
                const bool up = mx[blk] > m[blk] + RESCALE_THRESHOLD;
                const float alpha = up ? __builtin_amdgcn_exp2f(m[blk] - mx[blk]) : 1.f;
                m[blk] = up ? mx[blk] : m[blk];
                l[blk] *= alpha;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int j = 0; j < 16; ++j) o[blk][db][j] *= alpha;
            }
        }
        float msub[RB];
#pragma unroll
        for (int blk = 0; blk < RB; ++blk)
            msub[blk] = m[blk] == NEG_INF ? 0.f : m[blk];  // rows with no visible key yet
        // ---- per 32-key block: P (bf16), then O^T += V^T P^T over its two k-steps ----
#pragma unroll
        for (int b = 0; b < C::NB; ++b) {
            uint32_t pk[RB][8];
#pragma unroll
            for (int blk = 0; blk < RB; ++blk)
#pragma unroll
                for (int j = 0; j < 16; j += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[blk][b][j], sl2, -msub[blk]));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[blk][b][j + 1], sl2, -msub[blk]));
                    pk[blk][j / 2] = pack_bf16(p0, p1);
                    // sums the bf16 weights actually applied
                    l[blk] = dot2(pk[blk][j / 2], 0x3F803F80u, l[blk]);
                }
            // V^T fragments, streamed PF_V MFMAs ahead; MFMA i = (ks2, db)
            // 8-bit caches: V codes of keys past the sequence may be anything
            // (NaN codes), and p = 0 does not cancel a NaN inside the MFMA, so
            // their bytes are zeroed in registers: byte m of a V^T fragment is
            // key 32b + 16 ks2 + 4h + m (m < 4) or + 8 + 4h + m - 4.
            uint2 vmask[2] = {make_uint2(~0u, ~0u), make_uint2(~0u, ~0u)};
            if constexpr (KV8) {
                if (kt + 32 * (b + 1) > seq_len) {
                    auto bytes_below = [](int n) -> uint32_t {  // bytes 0 .. n-1 kept
                        return n >= 4 ? ~0u : (n <= 0 ? 0u : (1u << (8 * n)) - 1u);
                    };
#pragma unroll
                    for (int ks2 = 0; ks2 < 2; ++ks2) {
                        const int lim = seq_len - kt - 32 * b - 16 * ks2 - 4 * h;
                        vmask[ks2] = make_uint2(bytes_below(lim), bytes_below(lim - 8));
                    }
                }
            }
            using VFrag = std::conditional_t<KV8, uint2, bf16x8_t>;
            auto vread = [&](int i) -> VFrag {
                if constexpr (KV8) {
                    return lds_read_tr8(vst + (v8_base ^ ((2 * (i % C::DB)) << 4)) +
                                        (16 * (i / C::DB) + 32 * b) * D);
                } else {
                    const char *a = vst + v_base + (4 * b + 2 * (i / C::DB)) * C::GROUP_BYTES +
                                    (i % C::DB) * 512;
                    const s16x4_t lo = lds_read_tr16(a);
                    const s16x4_t hi = lds_read_tr16(a - v_base + v_base_odd);
                    const s16x4_t av[2] = {lo, hi};
                    return __builtin_bit_cast(bf16x8_t, av);
                }
            };
            VFrag va[PF_V];
#pragma unroll
            for (int i = 0; i < PF_V; ++i) va[i] = vread(i);
#pragma unroll
            for (int i = 0; i < 2 * C::DB; ++i) {
                const int ks2 = i / C::DB, db = i % C::DB;
                bf16x8_t a;
                if constexpr (KV8)
                    a = e4m3x8_to_bf16(va[i % PF_V].x & vmask[ks2].x, va[i % PF_V].y & vmask[ks2].y);
                else
                    a = va[i % PF_V];
                if (i + PF_V < 2 * C::DB) va[i % PF_V] = vread(i + PF_V);
                // one V^T fragment serves every row block of the wave
#pragma unroll
                for (int blk = 0; blk < RB; ++blk) {
                    const u32x4_t pb = {pk[blk][4 * ks2], pk[blk][4 * ks2 + 1], pk[blk][4 * ks2 + 2],
                                        pk[blk][4 * ks2 + 3]};
                    o[blk][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        a, __builtin_bit_cast(bf16x8_t, pb), o[blk][db], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // everyone is done with this stage before it is refilled
        __syncthreads();
    }

    // ---- finish: full exp-sum of each row, normalise, store ----
#pragma unroll
    for (int blk = 0; blk < RB; ++blk) {
        const RowPair pl = row_pair32(l[blk]);
        const float lb = pl.a + pl.b;
        if (!row_valid[blk]) continue;
        const int n_parts = p.partition ? pos[blk] / p.partition + 1 : 1;
        if (p.partition && part >= n_parts) continue;  // no keys of this row here
        // 8-bit caches: O holds code units of V, so the head's V scale joins 1/l
        float inv = (KV8 ? p.v_scale[kvh] : 1.f) / lb;
        if (n_parts == 1 && p.sinks) {
            // the head's sink: one more denominator term, no value (log2 units)
            const float s2 = p.sinks[head[blk]] * LOG2E_F;
            const float Mx = fmaxf(m[blk], s2);
            const float a = exp2_diff(m[blk], Mx);
            inv = (KV8 ? p.v_scale[kvh] : 1.f) * a / (lb * a + exp2_diff(s2, Mx));
        }
        if (n_parts == 1) {
            uint16_t *orow =
                reinterpret_cast<uint16_t *>(p.out) + ((size_t)t_glob[blk] * p.hq + head[blk]) * D;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int d = db * 32 + 8 * a + 4 * h;
                    uint2 w;
                    w.x = pack_bf16(o[blk][db][4 * a] * inv, o[blk][db][4 * a + 1] * inv);
                    w.y = pack_bf16(o[blk][db][4 * a + 2] * inv, o[blk][db][4 * a + 3] * inv);
                    *reinterpret_cast<uint2 *>(orow + d) = w;
                }
        } else {
            const size_t si = ((size_t)t_glob[blk] * p.hq + head[blk]) * p.max_parts + part;
            float *orow = p.tmp_out + si * D;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int d = db * 32 + 8 * a + 4 * h;
                    float4 w = {o[blk][db][4 * a] * inv, o[blk][db][4 * a + 1] * inv,
                                o[blk][db][4 * a + 2] * inv, o[blk][db][4 * a + 3] * inv};
                    *reinterpret_cast<float4 *>(orow + d) = w;
                }
            if (h == 0) {
                p.max_logits[si] = mtrue[blk];
                p.exp_sums[si] = lb * __builtin_amdgcn_exp2f(m[blk] - mtrue[blk]);
            }
        }
    }
}

// Launch of the tile kernel over the whole batch: a 1-D grid of virtual work
// items (q-tile, KV head, partition), padded to whole XCD chunks; surplus
// workgroups exit at once.
template <int D, int N, int NST, bool KV8, int NWV, int RB>
hipError_t launch_tiles(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    const int TPW = 32 * RB / p.group;
    const int BQ = NWV * TPW;
    AttnParams q = p;
    q.grid_tiles = (p.total_q / BQ + p.num_seqs + XCD_CHUNK - 1) / XCD_CHUNK * XCD_CHUNK;
    q.grid_parts = p.partition ? (p.max_seq_len + p.partition - 1) / p.partition : 1;
    const int64_t items = (int64_t)q.grid_tiles * p.hkv * q.grid_parts;
    if (items > INT32_MAX - 4096) return hipErrorInvalidConfiguration;
    const int64_t unit = 8 * XCD_CHUNK;
    const int blocks = (int)((items + unit - 1) / unit * unit);
    if (li) *li = LaunchInfo{{blocks, 1, 1}, NWV * 64, {N, NST, BQ}, 0};
    hipLaunchKernelGGL((prefill_kernel<D, N, NST, KV8, NWV, RB>), dim3(blocks), dim3(NWV * 64), 0,
                       stream, q);
    return hipGetLastError();
}

}  // namespace
}  // namespace pa
