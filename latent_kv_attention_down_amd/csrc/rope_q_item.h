// The query RoPE of the MLA chunk step (§3.2 Eq. 6 on the per-head positional
// query, App. E Eq. 12 for its place in the absorbed query row), one work item
// at a time, so that the same code serves the query kernel of its own and the
// workgroups it rides along with in the cache write's launch.  Item idx rotates PG
// pairs of one (token, head) row and stores them, pre-scaled, into the rope
// columns of q_lat; items below n_zero also clear one int of the attention's
// overflow flags.
#pragma once
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

template <typename OutT, int PG>
__device__ __forceinline__ void rope_q_item(const RopeQArgs &a, int64_t idx) {
  if (idx < a.n_zero) a.zero[idx] = 0;
  const int P = a.d_rope / 2, NG = P / PG;
  const int64_t total = (int64_t)a.M * a.n_h * NG;
  if (idx >= total) return;
  const int p0 = (int)(idx % NG) * PG;
  const int64_t mh = idx / NG;
  const int h = mh % a.n_h;
  const int m = mh / a.n_h;
  const int i = m % a.T_q, n = i % a.tpf;
  const double pos[3] = {(double)(a.t0 + i / a.tpf), (double)(n / a.grid_w), (double)(n % a.grid_w)};
  OutT *dst = (OutT *)a.q_lat + mh * (a.d_c + a.d_rope) + a.d_c + 2 * p0;
  float v[2 * PG];
  float scale = a.scale;
  if (a.in_place) {  // the GEMM already wrote scale * q^R here
#pragma unroll
    for (int e = 0; e < 2 * PG; ++e) v[e] = to_f32(dst[e]);
    scale = 1.f;
  } else if (PG == 4) {
    const float *src = a.q_r + (int64_t)m * a.n_h * a.d_rope + h * a.d_rope + 2 * p0;
    const float4 lo = *(const float4 *)src, hi = *(const float4 *)(src + 4);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  } else {
    const float *src = a.q_r + (int64_t)m * a.n_h * a.d_rope + h * a.d_rope + 2 * p0;
#pragma unroll
    for (int e = 0; e < 2 * PG; ++e) v[e] = src[e];
  }
#pragma unroll
  for (int q = 0; q < PG; ++q) {
    rope_rotate(v[2 * q], v[2 * q + 1], pos[a.rope.axis[p0 + q]], a.rope.omega[p0 + q]);
    dst[2 * q] = from_f32<OutT>(v[2 * q] * scale);
    dst[2 * q + 1] = from_f32<OutT>(v[2 * q + 1] * scale);
  }
}

// Work items of one query RoPE pass (PG = 4 when the pair count allows).
__host__ __device__ inline int64_t rope_q_items(const RopeQArgs &a, int pg) {
  const int64_t t = (int64_t)a.M * a.n_h * (a.d_rope / 2 / pg);
  return t > a.n_zero ? t : a.n_zero;
}

}  // namespace mla
