// q8_device.hpp -- device-side building blocks shared by the q8stream kernels.
//
// Everything here is gfx950 (CDNA4) code: wave64, DPP row operations, the
// packed bf16 dot (v_dot2_f32_bf16), the signed int8 dot (v_dot4_i32_i8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Q8_0 block scale from the block's largest magnitude: the fp32 quotient
// amax / 127 (IEEE division, correctly rounded) rounded to binary16 with the
// hardware's round-to-nearest-even conversion
// [fak MODEL-BASELINE-RESULTS, ACT 3, "How it was closed", item 1: d = maxabs/127].
__device__ __forceinline__ uint16_t block_scale_bits(float amax) {
    const float d = amax / 127.0f;
    return __builtin_bit_cast(uint16_t, (_Float16)d);
}

// One code: round half away from zero of the correctly rounded fp32 quotient
// v / s by the stored scale, clamped to [-127, 127]; zero scale gives zero
// [fak MODEL-BASELINE-RESULTS, ACT 4, "Correctness": math.Round semantics,
// never add-0.5-and-truncate].  roundf() is half-away-from-zero.
__device__ __forceinline__ int block_code(float v, float s) {
    // branch-free: a zero scale's quotient (inf / NaN) is discarded by the select
    const float r = fminf(fmaxf(roundf(v / s), -127.0f), 127.0f);
    return s == 0.0f ? 0 : (int)r;
}

// ---------------------------------------------------------------- conversions

// Four int8 codes (one dword) -> two dwords of packed bf16 pairs.  Codes are
// small integers, exact in fp32 and in bf16, so taking the upper half of the
// fp32 pattern is an exact conversion.
__device__ __forceinline__ void i8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    const float f0 = (float)(int)(int8_t)(w);
    const float f1 = (float)(int)(int8_t)(w >> 8);
    const float f2 = (float)(int)(int8_t)(w >> 16);
    const float f3 = (float)((int)w >> 24);
    lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                          __builtin_bit_cast(bf16x2, b), c, false);
}

// Exact int32 dot of one 32-element Q8 block split over a lane pair (lanes 2i
// and 2i + 1): each lane holds one 16-byte half of the weight and activation
// codes and takes its four signed v_dot4_i32_i8 (half_dot), and one DPP step
// adds the partner's half [fak MODEL-BASELINE-RESULTS, ACT 3 item 3: signed x
// signed int8 block dot].  |sum| <= 32 * 127 * 127 = 516,128, far inside
// int32.  Every lane of the wave must execute these (the DPP step reads the
// partner's register).
__device__ __forceinline__ int half_dot(const u32x4& w, const u32x4& x) {
    int s = 0;
    s = __builtin_amdgcn_sdot4((int)w.x, (int)x.x, s, false);
    s = __builtin_amdgcn_sdot4((int)w.y, (int)x.y, s, false);
    s = __builtin_amdgcn_sdot4((int)w.z, (int)x.z, s, false);
    s = __builtin_amdgcn_sdot4((int)w.w, (int)x.w, s, false);
    return s;
}
__device__ __forceinline__ int pair_swap(int v) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);        // quad_perm [1,0,3,2]
}
// One block sum, on both lanes of the pair.
__device__ __forceinline__ int block_dot_halves(const u32x4& w, const u32x4& x) {
    const int s = half_dot(w, x);
    return s + pair_swap(s);
}
// Two block sums at once, one per lane: the even lane ends with block sum A
// (wa . xa), the odd lane with block sum B (wb . xb).  Each lane sends its
// partner its half of the product it does not keep, so one DPP add finishes
// both and neither lane converts or folds a sum twice.
__device__ __forceinline__ int block_dot_pair(const u32x4& wa, const u32x4& xa, const u32x4& wb,
                                              const u32x4& xb, bool even) {
    const int ha = half_dot(wa, xa), hb = half_dot(wb, xb);
    return (even ? ha : hb) + pair_swap(even ? hb : ha);
}

// ---------------------------------------------------------------- buffer loads

// raw buffer descriptor word 3 for gfx9-family targets: untyped 32-bit data
constexpr int kRsrcWord3 = 0x00020000;
// cache-policy bit of a buffer load: non-temporal (streamed once)
constexpr int kLoadNT = 2;

// Buffer descriptor over [base, base + bytes); offsets at or past `bytes` read
// as zero without touching memory.  `bytes` must be below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             bytes > 0 ? (int)bytes : 0, kRsrcWord3);
}

// The same with a 32-bit range (no 64-bit compare in the address arithmetic).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc32(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes > 0 ? bytes : 0,
                                             kRsrcWord3);
}

// Ties a value to this point of the program: nothing computed from it is moved
// above, so a value fetched early stays in flight until here (work on it would
// otherwise be hoisted next to its load, which then waits at once).
template <typename T>
__device__ __forceinline__ void pin(T& v) { asm volatile("" : "+v"(v)); }

// ---------------------------------------------------------------- reductions

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over each row of 16 lanes with a fixed DPP tree (xor 1, xor 2, half-row
// mirror, row mirror).  Every lane of the row ends with the same bits: each step
// adds a pair of values in both orders, and fp32 addition is commutative.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);   // row_half_mirror
    v += dpp_f<0x140>(v);   // row_mirror
    return v;
}

// Lane l and its partner l ^ 16 (l ^ 32) through the gfx950 permlane swaps,
// which exchange the halves of every 32-lane (64-lane) group in the vector
// ALU instead of through LDS: with both operands v, the two results hold the
// lower and the upper partner's value on every lane, so a sum adds the same
// two values in the same order on both partners (identical bits, and the same
// as v + shfl_xor(v, 16 or 32), fp32 addition being commutative).
__device__ __forceinline__ float xor16_sum(float v) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
// The value of lane l ^ 32.
__device__ __forceinline__ float xor32_value(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((threadIdx.x & 32) ? s[0] : s[1]);
}

// Sum over groups of G lanes (G = 16, 32 or 64), same fixed order everywhere.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    v = row16_sum(v);
    if (G >= 32) v = xor16_sum(v);
    if (G >= 64) v = xor32_sum(v);
    return v;
}

// Sum over the lanes of one parity in each group of G lanes (G = 16, 32 or
// 64): a butterfly over lane ^ 2, lane ^ 4, lane ^ 8 (then the permlane
// swaps), each step adding the same two values in both orders, so every lane
// of a parity class ends with the same bits and equal inputs give equal sums
// wherever they sit.  Lane ^ 4 is the half-row mirror (lane -> 7 - lane in
// each 8) read back through a reversal of each quad.
template <int G>
__device__ __forceinline__ float group_sum_parity(float v) {
    v += dpp_f<0x4E>(v);                   // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp_f<0x1B>(dpp_f<0x141>(v));     // quad_perm [3,2,1,0] of the half-row mirror: lane ^ 4
    v += dpp_f<0x128>(v);                  // row_ror:8: lane ^ 8
    if (G >= 32) v = xor16_sum(v);
    if (G >= 64) v = xor32_sum(v);
    return v;
}

}  // namespace q8
