// Weight preparation for the absorbed forms of VideoMLA App. E.
//
// Value absorption into the output projection (Eq. 10-11):
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

// The latent query projection: for head h, rows h DK + c (c < d_c) hold
// W_qk,h = (W^K_up,h)^T W^Q_up,h (the transpose of App. E's A_h, Eq. 8-9), rows
// h DK + d_c + r copy W^Q_R,h, DK = d_c + d_rope, so c^Q maps to a whole absorbed
// query row [q~_h | q^R_h] in one GEMM.  One thread per element; the d_nope
// products summed in fp32.
template <typename T>
__global__ __launch_bounds__(256) void k_absorb_query(const T *__restrict__ w_k,
                                                      const T *__restrict__ w_q,
                                                      const T *__restrict__ w_r,
                                                      T *__restrict__ w_out, int n_h, int d_nope,
                                                      int d_c, int d_rope, int d_q) {
  const int DK = d_c + d_rope;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n_h * DK * d_q) return;
  const int64_t hj = idx / d_q;
  const int k = (int)(idx - hj * d_q), h = (int)(hj / DK), j = (int)(hj - (int64_t)h * DK);
  if (j >= d_c) {
    w_out[idx] = w_r[((int64_t)h * d_rope + (j - d_c)) * d_q + k];
    return;
  }
  const T *kk = w_k + (int64_t)h * d_nope * d_c + j;  // column j of W^K_up,h
  const T *qq = w_q + (int64_t)h * d_nope * d_q + k;  // column k of W^Q_up,h
  float acc = 0.f;
  for (int n = 0; n < d_nope; ++n) acc += to_f32(kk[(int64_t)n * d_c]) * to_f32(qq[(int64_t)n * d_q]);
  w_out[idx] = from_f32<T>(acc);
}

}  // namespace

hipError_t absorb_query(const void *w_k, const void *w_q, const void *w_r, void *w_out, int n_h,
                        int d_nope, int d_c, int d_rope, int d_q, bool bf16_io, hipStream_t st) {
  const int64_t total = (int64_t)n_h * (d_c + d_rope) * d_q;
  if (total <= 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (bf16_io)
    hipLaunchKernelGGL(k_absorb_query<bf16>, grid, dim3(256), 0, st, (const bf16 *)w_k,
                       (const bf16 *)w_q, (const bf16 *)w_r, (bf16 *)w_out, n_h, d_nope, d_c,
                       d_rope, d_q);
  else
    hipLaunchKernelGGL(k_absorb_query<float>, grid, dim3(256), 0, st, (const float *)w_k,
                       (const float *)w_q, (const float *)w_r, (float *)w_out, n_h, d_nope, d_c,
                       d_rope, d_q);
  return hipGetLastError();
}

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
