// Measurement probe, not part of the MLA path: a loop of independent bf16 MFMAs
// (v_mfma_f32_32x32x16_bf16) that measures the matrix-core rate this device
// sustains, as a companion to the rated peak in roofline figures.  Two waves per
// SIMD, four independent accumulation chains per wave.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_probe.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__global__ __launch_bounds__(512) void k_mfma_loop(float *out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)(threadIdx.x + e));
    b[e] = (__bf16)(1e-3f * (float)(e + 1));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int mla_probe_mfma_bf16(int blocks, int iters, float *out, void *stream) {
  if (blocks <= 0 || iters <= 0 || !out) return -1;
  hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(512), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

double mla_probe_mfma_bf16_flop(int blocks, int iters) {
  return (double)blocks * 8 /* waves */ * iters * 4 /* chains */ * (2.0 * 32 * 32 * 16);
}

}  // extern "C"
