// Device helpers shared by the paged-attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <tuple>
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

// Launch `kernel` on `stream` and return this launch's own status (hipLaunchKernel's),
// so that an error left pending by the caller's earlier HIP calls is neither reported
// for this launch nor cleared. The arguments are converted to the kernel's parameter
// types first.
template <typename... P, typename... A>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                                A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
  std::tuple<std::decay_t<P>...> vals(std::forward<A>(args)...);
  void* argv[sizeof...(P) > 0 ? sizeof...(P) : 1] = {};
  std::apply(
      [&argv](auto&... v) {
        int i = 0;
        ((argv[i++] = static_cast<void*>(&v)), ...);
      },
      vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
}


// ------------------------------------------------------------------ element traits
// KV element kinds (same numbering as the PA_* dtype enum).
constexpr int kF32 = PA_F32;
constexpr int kBF16 = PA_BF16;
constexpr int kFP8 = PA_FP8_E4M3;
constexpr int kINT8 = PA_INT8;

// Pools of one-byte codes with per-token-per-head fp32 scales.
template <int T>
constexpr bool kQuant = T == kFP8 || T == kINT8;
// Largest code magnitude: the absmax of a row maps to it.
template <int T>
constexpr float kQMax = T == kFP8 ? 448.0f : 127.0f;

template <int T>
struct ElemBytes;
template <>
struct ElemBytes<kF32> { static constexpr int value = 4; };
template <>
struct ElemBytes<kBF16> { static constexpr int value = 2; };
template <>
struct ElemBytes<kFP8> { static constexpr int value = 1; };
template <>
struct ElemBytes<kINT8> { static constexpr int value = 1; };

// ------------------------------------------------------------------ bf16 <-> f32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------------ OCP e4m3fn
// Encode a finite fp32 value to e4m3fn: round to nearest even, saturate to +-448
// (code 0x7E), keep the sign (so -0 and negative underflow give 0x80).
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7fffffffu);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    // subnormal range: value = m * 2^-9, m = round-half-even(a * 512) in [0, 8]
    // (m == 8 is the smallest normal, whose code is also 8)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // normal range: drop 20 mantissa bits with round-half-even, then rebias the
    // exponent from 127 to 7 (3 mantissa bits sit right below the exponent)
    uint32_t ua = u & 0x7fffffffu;
    ua += 0x7ffffu + ((ua >> 20) & 1u);
    code = (ua >> 20) - (120u << 3);
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return sign | code;
}

// Two e4m3fn codes (bytes 0,1 or 2,3 of w) -> two fp32 values (exact).
__device__ __forceinline__ void e4m3x2_to_f32(uint32_t w, bool high, float& a, float& b) {
  typedef float float2_t __attribute__((ext_vector_type(2)));
  float2_t r = high ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  a = r[0];
  b = r[1];
}

// Two e4m3fn codes (bytes 0,1 or 2,3 of w) -> their bf16 pair (exact: every e4m3fn
// value, subnormals included, is a bf16 value; the unit scale leaves them unchanged).
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool high) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  const bf2_t r = high ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// Two fp32 values rounded to nearest even into a bf16 pair (lo, hi).
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf2 bf16x2_rne(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  const f2_t x = {lo, hi};
  return __builtin_convertvector(x, bf2);
}

// ------------------------------------------------------------------ symmetric int8
// Round to nearest even and clamp to [-127, 127]; the code as its two's complement byte.
__device__ __forceinline__ uint32_t f32_to_i8sym(float y) {
  const float r = fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f);
  return (uint32_t)(int32_t)r & 0xffu;
}

// Bytes 0,1 (or 2,3) of w as signed codes -> two fp32 values (exact).
__device__ __forceinline__ void i8x2_to_f32(uint32_t w, bool high, float& a, float& b) {
  const int32_t x = (int32_t)(high ? w : w << 16);
  a = (float)((x << 8) >> 24);
  b = (float)(x >> 24);
}

// Pack the bf16 images of two fp32 values that are exactly representable in bf16
// (low half = lo, high half = hi).
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Two one-byte codes of a quantised pool -> fp32 values / their bf16 pair (exact:
// every e4m3fn value and every integer in [-127, 127] is a bf16 value).
template <int KVT>
__device__ __forceinline__ void q8x2_to_f32(uint32_t w, bool high, float& a, float& b) {
  if constexpr (KVT == kFP8) e4m3x2_to_f32(w, high, a, b);
  else i8x2_to_f32(w, high, a, b);
}
template <int KVT>
__device__ __forceinline__ uint32_t q8x2_to_bf16x2(uint32_t w, bool high) {
  if constexpr (KVT == kFP8) {
    return e4m3x2_to_bf16x2(w, high);
  } else {
    float a, b;
    i8x2_to_f32(w, high, a, b);
    return pack_bf16_exact(a, b);
  }
}

// ------------------------------------------------------------------ streaming loads
// KV rows are read once per call: non-temporal loads keep them from displacing
// reusable lines and measurably raise achieved read bandwidth on gfx950.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ uint2 ld_stream8(const void* p) {
  const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(t[0], t[1]);
}
__device__ __forceinline__ uint32_t ld_stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const unsigned int*>(p));
}

// ------------------------------------------------------------------ cross-lane
// DPP controls (within 4-lane quads / 16-lane rows of a wave64).
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kRowRor12 = 0x12C;

// All rows and banks enabled and bound_ctrl set: every control used here (quad perms,
// row mirrors, row rotates) reads an in-range lane, so no lane keeps an "old" value and
// the destination needs no initialising move.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}

// Exchange with lane ^ 32 / lane ^ 16 through gfx950's lane-swap instructions (VALU, no
// LDS round trip). With x as both operands, v_permlane32_swap returns (x[l mod 32] in
// the low half of the first result mirrored up, x of the upper half in the second), so
// the two results of every lane are {x[l], x[l ^ 32]} in some order; likewise for
// v_permlane16_swap and rows of 16 lanes. Sums and maxima of the pair are therefore
// the same on both lanes of a pair (IEEE add and max are commutative).
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace pa
