// Value absorption into the output projection (VideoMLA App. E Eq. 10-11):
// B_h = W_O[:, h d_h : (h+1) d_h] W^V_up,h, so a step can map the latent attention
// output straight to the model width, y = sum_h B_h O_lat,h, with no per-head
// value up-projection.  B is stored [d][n_h d_c] (row n, column h d_c + c), the
// [out][in] layout of W_O, so y = O_lat B^T is one GEMM over K = n_h d_c.
// This is a weight preparation done once per weight set (2 d n_h d_h d_c FLOP,
// 0.9 GFLOP at the Wan-1.3B shape): one thread per element of B, the d_h products
// summed in fp32 and rounded once to the storage type.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void k_absorb_value(const T *__restrict__ w_o,
                                                      const T *__restrict__ w_v,
                                                      T *__restrict__ w_b, int d, int n_h,
                                                      int d_h, int d_c) {
  const int64_t cols = (int64_t)n_h * d_c;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)d * cols) return;
  const int64_t n = idx / cols;
  const int hc = (int)(idx - n * cols), h = hc / d_c, c = hc - h * d_c;
  const T *o = w_o + n * n_h * d_h + (int64_t)h * d_h;         // row n of W_O, head h
  const T *v = w_v + (int64_t)h * d_h * d_c + c;               // column c of W^V_up,h
  float acc = 0.f;
  for (int k = 0; k < d_h; ++k) acc += to_f32(o[k]) * to_f32(v[(int64_t)k * d_c]);
  w_b[idx] = from_f32<T>(acc);
}

}  // namespace

hipError_t absorb_value(const void *w_o, const void *w_v, void *w_b, int d, int n_h, int d_h,
                        int d_c, bool bf16_io, hipStream_t st) {
  const int64_t total = (int64_t)d * n_h * d_c;
  if (total <= 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (bf16_io)
    hipLaunchKernelGGL(k_absorb_value<bf16>, grid, dim3(256), 0, st, (const bf16 *)w_o,
                       (const bf16 *)w_v, (bf16 *)w_b, d, n_h, d_h, d_c);
  else
    hipLaunchKernelGGL(k_absorb_value<float>, grid, dim3(256), 0, st, (const float *)w_o,
                       (const float *)w_v, (float *)w_b, d, n_h, d_h, d_c);
  return hipGetLastError();
}

}  // namespace mla
