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
#include "rope_q_item.h"

namespace mla {
namespace {

// One wave per row; four columns per lane and step when cols % 4 == 0 (16-byte
// loads, the gains read the same way), one otherwise.
template <typename OutT, typename GT>
__global__ __launch_bounds__(256) void k_rmsnorm_rows(const float *in, const GT *g, OutT *out,
                                                      int rows, int cols, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float *r = in + (int64_t)row * cols;
  OutT *o = out + (int64_t)row * cols;
  float ss = 0.f;
  if (cols % 4 == 0) {
    const float4 *r4 = (const float4 *)r;
    for (int c = lane; c < cols / 4; c += 64) {
      const float4 v = r4[c];
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)cols + eps);
    for (int c = lane; c < cols / 4; c += 64) {
      const float4 v = r4[c];
      float gn[4] = {1.f, 1.f, 1.f, 1.f};
      if (g)
#pragma unroll
        for (int e = 0; e < 4; ++e) gn[e] = to_f32(g[4 * c + e]);
      o[4 * c + 0] = from_f32<OutT>(v.x * inv * gn[0]);
      o[4 * c + 1] = from_f32<OutT>(v.y * inv * gn[1]);
      o[4 * c + 2] = from_f32<OutT>(v.z * inv * gn[2]);
      o[4 * c + 3] = from_f32<OutT>(v.w * inv * gn[3]);
    }
    return;
  }
  for (int c = lane; c < cols; c += 64) ss += r[c] * r[c];
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)cols + eps);
  for (int c = lane; c < cols; c += 64) {
    float gain = g ? to_f32(g[c]) : 1.0f;
    o[c] = from_f32<OutT>(r[c] * inv * gain);
  }
}

// PG pairs per thread (4 when the pair count allows: 32-byte reads of q^R).
template <typename OutT, int PG>
__global__ __launch_bounds__(256) void k_rope_q(RopeQArgs a) {
  rope_q_item<OutT, PG>(a, (int64_t)blockIdx.x * 256 + threadIdx.x);
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
  const int P = a.d_rope / 2;
  const bool by4 = P % 4 == 0;  // q^R rows are 16-byte aligned when d_rope % 8 == 0
  const int64_t total = rope_q_items(a, by4 ? 4 : 1);
  if (total <= 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256));
  if (bf16_out && by4)
    hipLaunchKernelGGL((k_rope_q<bf16, 4>), grid, dim3(256), 0, st, a);
  else if (bf16_out)
    hipLaunchKernelGGL((k_rope_q<bf16, 1>), grid, dim3(256), 0, st, a);
  else if (by4)
    hipLaunchKernelGGL((k_rope_q<float, 4>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_rope_q<float, 1>), grid, dim3(256), 0, st, a);
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
