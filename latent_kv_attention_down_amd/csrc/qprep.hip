// Query-side elementwise kernels of the MLA chunk step (paper §3.1 Eq. 3-4,
// §3.2 Eq. 6, App. D.2, App. E Eq. 8-9):
//  * RMSNorm of the query latent c^Q (one wave per row);
//  * rotation of the per-head positional query and its store, pre-scaled, into the
//    rope columns of the absorbed query rows (the same launch clears the attention's
//    overflow flags, saving a launch of its own);
//  * the per-head transpose of W^K_up used by the absorption GEMM
//    q~_h = (W^K_up,h)^T q^nope_h.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {
namespace {

template <typename OutT, typename GT>
__global__ __launch_bounds__(256) void k_rmsnorm_rows(const float *in, const GT *g, OutT *out,
                                                      int rows, int cols, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float *r = in + (int64_t)row * cols;
  float ss = 0.f;
  for (int c = lane; c < cols; c += 64) ss += r[c] * r[c];
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)cols + eps);
  for (int c = lane; c < cols; c += 64) {
    float gain = g ? to_f32(g[c]) : 1.0f;
    out[(int64_t)row * cols + c] = from_f32<OutT>(r[c] * inv * gain);
  }
}

template <typename OutT>
__global__ __launch_bounds__(256) void k_rope_q(RopeQArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one pair per thread
  if (idx < a.n_zero) a.zero[idx] = 0;
  const int P = a.d_rope / 2;
  const int64_t total = (int64_t)a.M * a.n_h * P;
  if (idx >= total) return;
  const int p = idx % P;
  const int64_t mh = idx / P;
  const int h = mh % a.n_h;
  const int m = mh / a.n_h;
  const int i = m % a.T_q, n = i % a.tpf;
  const float pos[3] = {(float)(a.t0 + i / a.tpf), (float)(n / a.grid_w), (float)(n % a.grid_w)};
  const float *src = a.q_r + (int64_t)m * a.n_h * a.d_rope + h * a.d_rope + 2 * p;
  float re = src[0], im = src[1];
  rope_rotate(re, im, pos[a.rope.axis[p]], a.rope.omega[p]);
  OutT *dst = (OutT *)a.q_lat + mh * (a.d_c + a.d_rope) + a.d_c + 2 * p;
  dst[0] = from_f32<OutT>(re * a.scale);
  dst[1] = from_f32<OutT>(im * a.scale);
}

template <typename T>
__global__ __launch_bounds__(256) void k_transpose_heads(const T *w, T *wt, int n_h, int d_nope,
                                                         int d_c) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)n_h * d_nope * d_c;
  if (idx >= total) return;
  const int n = idx % d_nope;
  const int64_t hc = idx / d_nope;
  const int c = hc % d_c, h = hc / d_c;
  wt[idx] = w[((int64_t)h * d_nope + n) * d_c + c];  // wt[h][c][n]
}

}  // namespace

hipError_t rmsnorm_rows(const float *in, const void *g, void *out, int rows, int cols, float eps,
                        bool out_bf16, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  dim3 grid((rows + 3) / 4);
  if (out_bf16)
    hipLaunchKernelGGL((k_rmsnorm_rows<bf16, bf16>), grid, dim3(256), 0, st, in, (const bf16 *)g,
                       (bf16 *)out, rows, cols, eps);
  else
    hipLaunchKernelGGL((k_rmsnorm_rows<float, float>), grid, dim3(256), 0, st, in,
                       (const float *)g, (float *)out, rows, cols, eps);
  return hipGetLastError();
}

hipError_t rope_q(const RopeQArgs &a, bool bf16_out, hipStream_t st) {
  int64_t total = (int64_t)a.M * a.n_h * (a.d_rope / 2);
  if (a.n_zero > total) total = a.n_zero;
  if (total <= 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256));
  if (bf16_out)
    hipLaunchKernelGGL(k_rope_q<bf16>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_rope_q<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t transpose_heads(const void *w, void *w_t, int n_h, int d_nope, int d_c, int esz,
                           hipStream_t st) {
  const int64_t total = (int64_t)n_h * d_nope * d_c;
  if (total <= 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256));
  if (esz == 2)
    hipLaunchKernelGGL(k_transpose_heads<bf16>, grid, dim3(256), 0, st, (const bf16 *)w,
                       (bf16 *)w_t, n_h, d_nope, d_c);
  else
    hipLaunchKernelGGL(k_transpose_heads<float>, grid, dim3(256), 0, st, (const float *)w,
                       (float *)w_t, n_h, d_nope, d_c);
  return hipGetLastError();
}

}  // namespace mla
