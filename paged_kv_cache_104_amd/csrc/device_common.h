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

// float -> OCP FP8 E4M3FN code: round to nearest, ties to even (subnormals in steps of
// 2^-9), saturate at +-448, NaN -> 0x7F, sign kept (negative values that round to zero
// give 0x80).  The conversion instruction rounds the same way but codes magnitudes past
// 448 (infinities too) as NaN and every NaN as 0xFF, so its input is first clamped to
// +-448, and a NaN enters as +inf, which it codes 0x7F.  A cache write encodes every
// element; three instructions per element (and one per pair for the conversion) keep
// that write bound by memory rather than by the encode.
__device__ __forceinline__ float e4m3_saturate(float y) {
  return y != y ? __builtin_inff() : __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f);
}

__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const float c = e4m3_saturate(y);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false)) & 0xffu;
}

// The codes of a, b, c, d in bytes 0, 1, 2, 3 of one word.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_saturate(a), e4m3_saturate(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_saturate(c), e4m3_saturate(d), w, true);
  return uint32_t(w);
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
