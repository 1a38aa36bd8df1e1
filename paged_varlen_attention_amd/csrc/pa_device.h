// pa_device.h -- small gfx950 device helpers shared by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float LOG2E = 1.44269504088896340736f;

// Storage type of a bf16 element: its 16 raw bits.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float x) {
    __bf16 v = (__bf16)x;
    return __builtin_bit_cast(uint16_t, v);
}

// c + a.lo*b.lo + a.hi*b.hi with bf16 pairs, fp32 accumulate (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// The same with the three-operand encoding (v_dot2_f32_bf16): the result
// register is not tied to the accumulator, which keeps the register allocator
// from copying loop-carried accumulators around branches.
__device__ __forceinline__ float dot2_untied(uint32_t a, uint32_t b, float c) {
    float d;
    asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// v_perm_b32 byte select; s0 supplies bytes 4..7, s1 bytes 0..3.
__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
    return __builtin_amdgcn_perm(s0, s1, sel);
}

// exp2 of (a - m) that is 0 when a is -inf (also when m is -inf).
constexpr float LOG2E_F = 1.44269504088896341f;

__device__ __forceinline__ float exp2_diff(float a, float m) {
    return a == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(a - m);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum / max over aligned groups of N consecutive lanes (N = 1..64); every lane
// of a group receives the group's result.  DPP inside a 16-lane row, then
// bpermute for the cross-row steps.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    if constexpr (N >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror
    if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}
template <int N>
__device__ __forceinline__ float group_max(float x) {
    if constexpr (N >= 2) x = fmaxf(x, dpp<0xB1>(x));
    if constexpr (N >= 4) x = fmaxf(x, dpp<0x4E>(x));
    if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
    if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
    if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
    if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

// Cross-row exchange (gfx950 v_permlane16_swap / v_permlane32_swap) of a value
// with itself: returns the two values of the row pair this lane belongs to,
// {row 2i, row 2i+1} for the 16-lane form and {row i, row i+2} for the 32-lane
// form, in the same order in every lane of the pair.
struct RowPair {
    float a, b;
};
__device__ __forceinline__ RowPair row_pair16(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ RowPair row_pair32(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Max and sum over the 4 lane groups (16-lane rows) of the wave: lanes c,
// c+16, c+32 and c+48 (one column of a 16x16 MFMA accumulator) get the same
// result.
__device__ __forceinline__ float rows_max(float x) {
    const RowPair a = row_pair16(x);
    x = fmaxf(a.a, a.b);
    const RowPair b = row_pair32(x);
    return fmaxf(b.a, b.b);
}
__device__ __forceinline__ float rows_sum(float x) {
    const RowPair a = row_pair16(x);
    x = a.a + a.b;
    const RowPair b = row_pair32(x);
    return b.a + b.b;
}

// ---- direct global -> LDS loads (gfx950 global_load_lds_dwordx4) ---------
//
// Each active lane copies 16 bytes from (sbase + voff) to LDS address
// lds + 16*lane.  Issued through inline asm so that the order of issue and the
// vmcnt waits are ours: the compiler neither reorders these against each
// other (volatile + memory clobber) nor inserts conservative vmcnt(0) waits in
// front of the LDS reads that consume them.  M0 carries the LDS base and is
// set in the same statement.
// A pointer the caller knows to be the same in every lane, moved to SGPRs.
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    sbase = uniform_ptr(sbase);
    lds = __builtin_amdgcn_readfirstlane(lds);
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"  // an LDS DMA reading M0 right after an SALU write needs a wait state
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory", "m0");
}

// The same with 4 bytes per lane (global_load_lds_dword): lane i's dword lands
// at lds + 4*i.
__device__ __forceinline__ void dma4(const void *sbase, uint32_t voff, uint32_t lds) {
    sbase = uniform_ptr(sbase);
    lds = __builtin_amdgcn_readfirstlane(lds);
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, %1"
        :
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// Direct global -> LDS load of BYTES (16 or 4) per lane.
template <int BYTES>
__device__ __forceinline__ void dma_lds(const void *sbase, uint32_t voff, uint32_t lds) {
    static_assert(BYTES == 16 || BYTES == 4, "LDS DMA width");
    if constexpr (BYTES == 16)
        dma16(sbase, voff, lds);
    else
        dma4(sbase, voff, lds);
}

// Wait until at most N vector-memory instructions of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Every lane passes the
// address of 4 consecutive 16-bit elements; within each group of 16 lanes,
// lane i receives element i%4 of the chunks of lanes i/4, i/4+4, i/4+8 and
// i/4+12, in that order.  `p` must point into LDS.
__device__ __forceinline__ s16x4_t lds_read_tr16(const void *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)(p));
}

// Eight E4M3 codes (two words, byte 0 first) -> eight bf16, exactly
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1).
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    const uint4 v = make_uint4(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true)));
    return __builtin_bit_cast(bf16x8_t, v);
}

// gfx950 LDS transpose read of bytes (ds_read_b64_tr_b8).  Every lane passes
// the address of 8 consecutive bytes; within each group of 16 lanes, lane i
// receives byte i%8 of the chunks of lanes i/8, i/8+2, .., i/8+14, in that
// order (lanes 2m and 2m+1 together hold row m of an 8 x 16 byte block, and
// lane i gets its column i).  `p` must point into LDS.
__device__ __forceinline__ uint2 lds_read_tr8(const void *p) {
    typedef __attribute__((ext_vector_type(2))) int i32x2_t;
    const i32x2_t w =
        __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t *)(p));
    return make_uint2((uint32_t)w[0], (uint32_t)w[1]);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)p;
}

}  // namespace pa
