// Device-side helpers shared by the libmla kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef short v2i16_t __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))
#define MLA_CONST __attribute__((address_space(4)))

namespace mla {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bfloat16 (hardware conversion on gfx950).
__device__ __forceinline__ __bf16 f32_to_bf16(float f) { return static_cast<__bf16>(f); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// OCP E4M3 (e4m3fn) encoder: 4 exponent bits (bias 7), 3 mantissa bits, no
// infinities, NaN = S.1111.111.  Rounds to nearest, ties to even, and
// saturates finite magnitudes to 448 (code 0x7E).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t bits = __float_as_uint(x);
  uint32_t sign = (bits >> 24) & 0x80u;
  uint32_t abits = bits & 0x7FFFFFFFu;
  if (abits > 0x7F800000u) return 0x7Fu | sign;           // NaN
  float a = __uint_as_float(abits);
  if (a >= 448.0f) return 0x7Eu | sign;                    // saturate (incl. inf)
  if (abits < 0x3C800000u) {                               // a < 2^-6: subnormal grid 2^-9
    uint32_t m = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));  // exact scaling, RNE
    return m | sign;                                       // m == 8 is the smallest normal
  }
  // normal: keep 3 mantissa bits, round to nearest even on the dropped 20 bits
  uint32_t r = abits + 0x7FFFFu + ((abits >> 20) & 1u);
  int e = static_cast<int>(r >> 23) - 127;
  uint32_t m = (r >> 20) & 7u;
  if (e > 8 || (e == 8 && m == 7u)) return 0x7Eu | sign;   // rounded past 448
  return (static_cast<uint32_t>(e + 7) << 3) | m | sign;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  uint32_t s = code & 0x80u, e = (code >> 3) & 0xFu, m = code & 7u;
  float v = (e == 0) ? static_cast<float>(m) * 0.001953125f            // m * 2^-9
                     : __uint_as_float(((e + 120u) << 23) | (m << 20)); // (1+m/8) 2^(e-7)
  return s ? -v : v;
}

// Rotary embedding: pair k of a d_r-wide vector at `pos` turns by
// pos / theta^(2k/d_r).  The angle and its reduction to [-pi, pi] are done in
// double (at the 131072-token positions a float angle would be off by ~1e-2
// rad); the reduced angle then goes through float sin/cos.
__device__ __forceinline__ void rope_cos_sin_inv(int pos, double inv_freq, float* c, float* s) {
  const double ang = static_cast<double>(pos) * inv_freq;
  const double red = ang - 6.283185307179586477 * rint(ang * 0.15915494309189533577);
  sincosf(static_cast<float>(red), s, c);
}

__device__ __forceinline__ void rope_cos_sin(int pos, int k, int d_r, float theta, float* c,
                                             float* s) {
  rope_cos_sin_inv(pos, exp2(-(2.0 * k / d_r) * log2(static_cast<double>(theta))), c, s);
}

// Inverse frequencies theta^(-2k/64) of a 64-wide rotary part, computed on
// the host in double and passed by value to the kernels that need them.
struct RopeTable64 {
  double inv[32];
};

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace mla
