// Device-side helpers of libpagedkv: element types, conversions, the E4M3 encoder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// Storage tags of the pools (template parameters).
enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// OCP FP8 E4M3FN code -> float, from the format definition (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xfu;
  const uint32_t m = c & 7u;
  float mag;
  if (e == 0xfu && m == 7u) {
    mag = __uint_as_float(0x7fc00000u);
  } else if (e == 0) {
    mag = float(m) * 0.001953125f;                       // m * 2^-9
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return __uint_as_float(__float_as_uint(mag) | sign);
}

// float -> OCP FP8 E4M3FN code: round to nearest, ties to even, saturate at +-448,
// NaN -> 0x7F, sign kept (negative values that round to zero give 0x80).  Both
// rounding paths are computed and the result selected, without branches: a cache
// write encodes every element, and per-element branches cost more than the paths.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  const float af = __uint_as_float(a);
  // below 2^-6: steps of 2^-9; af * 512 is exact, rint rounds half to even, and 8
  // gives code 0x08 = 2^-6
  const uint32_t sub = uint32_t(__builtin_rintf(fminf(af, 0.015625f) * 512.0f));
  // normal: keep 3 of 23 mantissa bits, rounding at bit 20 to nearest even (a carry
  // into the exponent is the correct next binade), exponent bias 127 -> 7
  const uint32_t nrm = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  uint32_t r = af < 0.015625f ? sub : nrm;
  r = af > 448.0f ? 0x7eu : r;                           // saturate (incl. inf)
  return a > 0x7f800000u ? 0x7fu : (sign | r);           // NaN
}

template <int KV>
struct KvTraits;
template <>
struct KvTraits<KV_F32> { typedef float T; static constexpr int bytes = 4; };
template <>
struct KvTraits<KV_BF16> { typedef uint16_t T; static constexpr int bytes = 2; };
template <>
struct KvTraits<KV_FP8> { typedef uint8_t T; static constexpr int bytes = 1; };

// Pool element -> float (fp8 without its scale).
template <int KV>
__device__ __forceinline__ float kv_to_f32(typename KvTraits<KV>::T x);
template <>
__device__ __forceinline__ float kv_to_f32<KV_F32>(float x) { return x; }
template <>
__device__ __forceinline__ float kv_to_f32<KV_BF16>(uint16_t x) { return bf16_to_f32(x); }
template <>
__device__ __forceinline__ float kv_to_f32<KV_FP8>(uint8_t x) { return e4m3_to_f32(x); }

}  // namespace pkv
