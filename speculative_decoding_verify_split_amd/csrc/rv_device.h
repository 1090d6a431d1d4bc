// Device-side helpers shared by the rapid_verify kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hardware base-2 exponential / logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ i32x4 buffer_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
}

// Same, with the non-temporal cache policy (the `nt` bit of the buffer
// instruction's cache-policy field): for data read exactly once, such as
// the KV stream.  Measured on MI355X with the history pass's tile pattern:
// ~7.0 TB/s of streaming reads versus ~6.0 TB/s with the default policy.
__device__ __forceinline__ i32x4 buffer_load16_stream(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 2);
}

// Lane permutations used by the all-reductions below.  Every step pairs
// lanes symmetrically (an involution), so both lanes of a pair compute
// op(a, b) and op(b, a): max and + are commutative, hence every lane ends
// with the bit-identical result, and the order of combination is fixed.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i inside each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i inside each 16

// Partner across 16-lane rows (i <-> i ^ 16) or wave halves (i <-> i ^ 32),
// with the gfx950 row-swap permutes: swapping a value with a copy of itself
// leaves {own, partner} in the two results.
__device__ __forceinline__ float2 swap16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 swap32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_f<kDppXor1>(v);
  v = v + dpp_f<kDppXor2>(v);
  v = v + dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  float2 a = swap16(v);
  v = fmaxf(a.x, a.y);
  a = swap32(v);
  return fmaxf(a.x, a.y);
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  float2 a = swap16(v);
  v = a.x + a.y;
  a = swap32(v);
  return a.x + a.y;
}

// Round-to-nearest-even fp32 -> bf16 bit pattern.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

}  // namespace rv
