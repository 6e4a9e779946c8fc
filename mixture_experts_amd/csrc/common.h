// Internal helpers shared by the gfx950 kernels of the MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

// 1: the GEMM kernels copy activations and weights into LDS with 64-bit (FLAT)
// addresses even where 32-bit buffer offsets would do.  The production library is
// built with 0; a second build with 1 lets the tests exercise the 64-bit form.
#ifndef MOE_FORCE_FLAT_COPIES
#define MOE_FORCE_FLAT_COPIES 0
#endif

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) double f64x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16 / fp32 bits
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ------------------------------------------------------------------ e4m3fn encoding
// OCP FP8 E4M3 ("fn": no infinity; S.1111.111 is NaN; max finite 448).
// Round to nearest, ties to the even code, saturate at 448, keep the sign bit.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(v);
  if (a != a) return 0x7fu;
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7eu;
  } else if (a < 0.015625f) {                       // below 2^-6: e4m3 subnormal step 2^-9
    code = uint32_t(rintf(a * 512.0f));               // exact product; rintf is nearest-even
  } else {
    uint32_t ua = __float_as_uint(a);
    int e = int(ua >> 23) - 127;                      // -6 .. 8
    uint32_t mant = ua & 0x7fffffu;
    uint32_t r = mant >> 20, rem = mant & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    if (r == 8u) { r = 0u; ++e; }
    code = uint32_t((e + 7) << 3) | r;
    if (code > 0x7eu) code = 0x7eu;
  }
  return sign | code;
}

__device__ __forceinline__ float exp2i(int e) {      // 2^e for e in [-149, 127], exact
  if (e >= -126) return __uint_as_float(uint32_t(e + 127) << 23);
  return __uint_as_float(1u << (e + 149));
}

// ------------------------------------------------------------------ NVFP4 (e2m1 + e4m3 per 16)
// e4m3fn code -> value (finite codes; exact in fp32).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;   // m * 2^-9
  return (c & 0x80u) ? -mag : mag;
}

// e2m1 code of v: nearest grid value (0, 0.5, 1, 1.5, 2, 3, 4, 6), ties to the even
// code, saturating at 6; the sign bit is kept.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  const float a = fabsf(v);
  const uint32_t c = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                     uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t m = c & 7u;
  const float mag = m < 2u ? 0.5f * float(m) : __uint_as_float(((m >> 1) + 126u) << 23) * ((m & 1u) ? 1.5f : 1.0f);
  return (c & 8u) ? -mag : mag;
}

// Scale of an NVFP4 group from its amax: e4m3(amax / 6), or 1 when that rounds to 0.
__device__ __forceinline__ float nvfp4_scale(float amax) {
  const float s = e4m3_to_f32(f32_to_e4m3(amax / 6.0f));
  return s > 0.0f ? s : 1.0f;
}

// NVFP4 value of v in a group of scale s: e2m1(v / s) * s, exact in fp32 and fp16.
__device__ __forceinline__ float nvfp4_value(float v, float s) { return e2m1_to_f32(f32_to_e2m1(v / s)) * s; }

// Least integer e with amax <= 448 * 2^e (amax >= 0 finite); 0 for amax == 0; clamped to [-127, 127].
__device__ __forceinline__ int mx_exponent_e4m3(float amax) {
  if (!(amax > 0.0f)) return 0;
  uint32_t u = __float_as_uint(amax);
  int ebits = int(u >> 23);
  int ea;
  float m;
  if (ebits == 0) {                                   // fp32 subnormal: amax = mant * 2^-149
    uint32_t mant = u & 0x7fffffu;
    int p = 31 - __clz(int(mant));                    // position of the leading one
    ea = p - 149;
    m = float(mant) * exp2i(-p);                      // exact: in [1, 2)
  } else {
    ea = ebits - 127;
    m = __uint_as_float((u & 0x7fffffu) | 0x3f800000u); // mantissa in [1, 2)
  }
  int e = (m <= 1.75f) ? ea - 8 : ea - 7;           // 448 = 1.75 * 2^8
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ------------------------------------------------------------------ wave helpers
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor(uint32_t(v), off, 64);
    uint32_t hi = __shfl_xor(uint32_t(v >> 32), off, 64);
    uint64_t o = (uint64_t(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float max_over_lanes32(float v) {   // within each 32-lane half
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Order-preserving map of an fp32 to uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t orderable_f32(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// SwiGLU of one (gate, up) pair.  limit > 0 (swiglu_limit, DeepSeek-V4-Pro
// overview, FFN entry) first clamps the gate to at most the limit and the up
// projection to [-limit, limit].
__device__ __forceinline__ float swiglu_f32(float g, float u, float limit) {
  if (limit > 0.0f) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  return silu_f32(g) * u;
}

}  // namespace moe
