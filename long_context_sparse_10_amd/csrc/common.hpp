// Device helpers shared by the gfx950 kernels of libcsa: number formats,
// wave reductions, RoPE angles and row encoders.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// round-to-nearest-even fp32 -> bf16 bits (finite inputs; overflow gives inf)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ------------------------------------------------------------------ OCP e4m3 (FN)
// encode with round-to-nearest-even, saturating at +-448 (no inf / NaN produced)
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
  const float a = fabsf(f);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a >= 0.015625f) {                       // normal: 2^-6 <= a < 448
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);         // RNE to 3 mantissa bits
    const uint32_t e = (u >> 23) - 120u;      // biased e4m3 exponent (1..15)
    const uint32_t mant = (u >> 20) & 7u;
    if (e > 15u || (e == 15u && mant == 7u)) return sign | 0x7Eu;
    return sign | (e << 3) | mant;
  }
  // subnormal: multiples of 2^-9; a * 512 is exact, rintf is RNE
  return sign | (uint32_t)rintf(a * 512.0f);  // 8 -> 0x08 = 2^-6, still correct
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t em = code & 0x7Fu;
  float v = em >= 8u ? __uint_as_float((em << 20) + (120u << 23)) : (float)em * 0.001953125f;
  return __uint_as_float(__float_as_uint(v) | ((code & 0x80u) << 24));
}

// ------------------------------------------------------------------ E2M1 / MXFP4
// E2M1 code of a value already divided by its block scale (RNE, saturating at 6)
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
  const float a = fabsf(v);
  uint32_t code;
  if (a <= 0.25f) code = 0;
  else if (a < 0.75f) code = 1;
  else if (a <= 1.25f) code = 2;
  else if (a < 1.75f) code = 3;
  else if (a <= 2.5f) code = 4;
  else if (a < 3.5f) code = 5;
  else if (a <= 5.0f) code = 6;
  else code = 7;
  return sign | code;
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t code) {
  // magnitudes of codes 0..7 = {0, .5, 1, 1.5, 2, 3, 4, 6}
  const uint32_t c = code & 7u;
  float v;
  if (c < 2u) v = 0.5f * (float)c;
  else v = __uint_as_float(((c >> 1) + 126u) << 23) * (1.0f + 0.5f * (float)(c & 1u));
  return (code & 8u) ? -v : v;
}

// e8m0 scale exponent (unbiased) of a block whose largest magnitude is amax:
// floor(log2 amax) - 2, clamped to [-127, 127]; zero / subnormal blocks get -127
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  if (ef == 0) return -127;
  const int e = ef - 127 - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ __forceinline__ float exp2i(int e) {  // 2^e for -149 <= e <= 127, exact
  if (e >= -126) return __uint_as_float((uint32_t)(e + 127) << 23);
  return __uint_as_float(1u << (e + 149));
}

// ------------------------------------------------------------------ reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// ------------------------------------------------------------------ RoPE
// Pair u of d_r RoPE channels turns by pos * f_u, f_u = theta^(-2u/d_r).  The
// host passes base = theta^(-2/d_r) in fp64; a kernel forms f_u = base^u by
// binary powering (relative error < 2e-15), the angle pos * f_u in fp64 and
// reduces it to a quarter turn in fp64, so positions up to 2^31 keep full fp32
// accuracy.  sin / cos of the remainder |t| <= pi/4 come from their Taylor
// series (truncation below 3e-9), evaluated in fp32 without branches.
struct Rope {
  double base;  // theta^(-2/d_r)
  int d_r;
};

inline Rope make_rope(int d_r, float theta) {
  Rope r;
  r.d_r = d_r;
  r.base = d_r > 0 ? pow((double)theta, -2.0 / (double)d_r) : 1.0;
  return r;
}

__device__ __forceinline__ double rope_freq(double base, int u) {
  double f = 1.0, p = base;
  for (int e = u; e > 0; e >>= 1) {
    if (e & 1) f *= p;
    p *= p;
  }
  return f;
}

// sin and cos of an angle given in fp64 radians
__device__ __forceinline__ void sincos_fp64_angle(double ang, float* s, float* c) {
  const double q = rint(ang * 0.6366197723675814);        // quarter turns
  const float t = (float)fma(-q, 1.5707963267948966, ang);  // |t| <= pi/4
  const float t2 = t * t;
  const float sp = t * (1.0f + t2 * (-1.0f / 6 + t2 * (1.0f / 120 + t2 * (-1.0f / 5040 + t2 * (1.0f / 362880)))));
  const float cp = 1.0f + t2 * (-0.5f + t2 * (1.0f / 24 + t2 * (-1.0f / 720 + t2 * (1.0f / 40320 + t2 * (-1.0f / 3628800)))));
  const int n = (int)((long long)q & 3);
  const float ss = (n & 1) ? cp : sp;
  const float cc = (n & 1) ? sp : cp;
  *s = (n & 2) ? -ss : ss;
  *c = ((n + 1) & 2) ? -cc : cc;
}

__device__ __forceinline__ void rope_cs(const Rope& r, double pos, int u, float* c, float* s) {
  sincos_fp64_angle(pos * rope_freq(r.base, u), s, c);
}

// ------------------------------------------------------------------ row formats
__host__ __device__ inline int64_t row_bytes(csa_dtype t, int c, int rope_dims) {
  switch (t) {
    case CSA_F32: return 4ll * c;
    case CSA_BF16: return 2ll * c;
    case CSA_FP8MIX: return (int64_t)(c - rope_dims) + 2ll * rope_dims;
    case CSA_MXFP4: return c / 2;
    default: break;
  }
  return 0;
}

// read element j of a row stored as f32 / bf16
__device__ __forceinline__ float load_elem(const void* row, csa_dtype t, int j) {
  if (t == CSA_F32) return reinterpret_cast<const float*>(row)[j];
  return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[j]);
}

// read element j of a KV row in f32 / bf16 / fp8mix
__device__ __forceinline__ float load_kv_elem(const uint8_t* row, csa_dtype t, int c, int d_r,
                                              int j) {
  if (t == CSA_F32) return reinterpret_cast<const float*>(row)[j];
  if (t == CSA_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[j]);
  const int body = c - d_r;
  if (j < body) return e4m3_to_f32(row[j]);
  return bf16_to_f32(reinterpret_cast<const uint16_t*>(row + body)[j - body]);
}

}  // namespace csa
