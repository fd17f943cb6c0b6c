// Device-side types and helpers shared by the gfx950 kernels of the MLA chunk step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_types.h"

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

namespace mla {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// 32x32x16 bf16 MFMA, D = A(32x16) * B(16x32) + C.  Lane l supplies A row l%32 and
// B column l%32, eight consecutive k of the 16 (group l/32).  Lane l receives
// column l%32 of D, rows 8*i + 4*(l/32) + j in acc[4*i + j].
__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA.  Lane l supplies A row l%16 / B column l%16 with eight
// consecutive k (group l/16).  Lane l receives column l%16, rows 4*(l/16)+j in acc[j].
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// sin and cos of the angle pos * omega.  The product is formed and reduced to
// [-pi, pi] in fp64 (a frame index of a long rollout times a frequency near 1 is far
// beyond what an fp32 product or argument resolves), and only the reduced angle goes
// through the fp32 sincos.
__device__ __forceinline__ void rope_sincos(double pos, double omega, float &s, float &c) {
  const double two_pi = 6.283185307179586;
  const double a = pos * omega;
  const double r = fma(-two_pi, rint(a * (1.0 / two_pi)), a);
  sincosf((float)r, &s, &c);
}

// (re, im) turned by the angle whose sine and cosine are s and c, with the fused
// multiply-adds spelled out, so that every kernel that rotates (whatever code the
// compiler inlines this into) gives the same bits.
__device__ __forceinline__ void rotate_by(float &re, float &im, float s, float c) {
  const float r = fmaf(re, c, -(im * s));
  const float i = fmaf(re, s, im * c);
  re = r;
  im = i;
}

// Rotate pair (re, im) by angle pos * omega (counter-clockwise).
__device__ __forceinline__ void rope_rotate(float &re, float &im, double pos, double omega) {
  float s, c;
  rope_sincos(pos, omega, s, c);
  rotate_by(re, im, s, c);
}

}  // namespace mla
