// Window assembly (VideoMLA §3.2 Eq. 5: the cache keeps k^R unrotated; App.
// D.4-D.5: the attended context is the sink frame(s) plus the most recent local
// frames, re-indexed to local temporal coordinates).  Context frame i -- sink
// frames first, then the local frames in time order -- is copied from its ring
// slot into rows i*tpf .. of a contiguous window in the interleaved row layout
// [c^KV | k].  Under read-time rotation its d_rope positional columns are rotated
// by 3D-RoPE at (i, y, x); a ring kept in another layout (the two tensors of
// App. D.4 with their own strides) is gathered the same way without rotation.
// The latent columns are copied unchanged.  The attention kernels then read the
// window as one contiguous range.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {
namespace {

// Ring row (within its request) that holds row j of the context.
__device__ __forceinline__ int64_t source_row(const AssembleArgs &a, int64_t j) {
  const int64_t i = j / a.tpf, n = j % a.tpf;
  const int64_t f = i < a.n_sink ? i : a.first_local + (i - a.n_sink);
  const int64_t slot = f < a.S ? f : a.S + (f - a.S) % a.W;
  return slot * a.tpf + n;
}

// Column c (of d_c + d_rope) of ring row `row` of request b.
template <typename T>
__device__ __forceinline__ const T *ring_src(const AssembleArgs &a, int b, int64_t row, int c) {
  return c < a.d_c ? (const T *)a.ring.c_kv + b * a.ring.c_batch + row * a.ring.c_row + c
                   : (const T *)a.ring.k_r + b * a.ring.r_batch + row * a.ring.r_row + (c - a.d_c);
}

// bf16: one thread per 16 bytes (8 columns) of a window row.  d_c is a multiple
// of 8, so a piece is either latent (copied) or four RoPE pairs (rotated).
__global__ __launch_bounds__(256) void k_assemble_bf16(AssembleArgs a) {
  const int DK = a.d_c + a.d_rope, CPR = DK / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.nk * CPR;
  if (idx >= total) return;
  const int ch = (int)(idx % CPR);
  const int64_t bj = idx / CPR;
  const int b = (int)(bj / a.nk);
  const int64_t j = bj % a.nk;
  const bf16x8 v = *(const bf16x8 *)ring_src<bf16>(a, b, source_row(a, j), ch * 8);
  bf16x8 out = v;
  if (a.rotate && ch * 8 >= a.d_c) {
    const int64_t i = j / a.tpf, n = j % a.tpf;
    const double pos[3] = {(double)i, (double)(n / a.grid_w), (double)(n % a.grid_w)};
    const int p0 = (ch * 8 - a.d_c) / 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float re = (float)v[2 * q], im = (float)v[2 * q + 1];
      rope_rotate(re, im, pos[a.rope.axis[p0 + q]], a.rope.omega[p0 + q]);
      out[2 * q] = (bf16)re;
      out[2 * q + 1] = (bf16)im;
    }
  }
  *(bf16x8 *)((bf16 *)a.win + ((int64_t)b * a.nk + j) * DK + ch * 8) = out;
}

// fp32: one thread per element.
__global__ __launch_bounds__(256) void k_assemble_f32(AssembleArgs a) {
  const int DK = a.d_c + a.d_rope;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.nk * DK;
  if (idx >= total) return;
  const int c = (int)(idx % DK);
  const int64_t bj = idx / DK;
  const int b = (int)(bj / a.nk);
  const int64_t j = bj % a.nk;
  const int64_t row = source_row(a, j);
  float v = *ring_src<float>(a, b, row, c);
  if (a.rotate && c >= a.d_c) {
    const int p = (c - a.d_c) / 2, e = (c - a.d_c) % 2;
    const int64_t i = j / a.tpf, n = j % a.tpf;
    const double pos[3] = {(double)i, (double)(n / a.grid_w), (double)(n % a.grid_w)};
    float re = *ring_src<float>(a, b, row, a.d_c + 2 * p);
    float im = *ring_src<float>(a, b, row, a.d_c + 2 * p + 1);
    rope_rotate(re, im, pos[a.rope.axis[p]], a.rope.omega[p]);
    v = e == 0 ? re : im;
  }
  ((float *)a.win)[((int64_t)b * a.nk + j) * DK + c] = v;
}

}  // namespace

hipError_t assemble_window(const AssembleArgs &a, bool bf16_io, hipStream_t st) {
  const int DK = a.d_c + a.d_rope;
  const int64_t total = (int64_t)a.B * a.nk * (bf16_io ? DK / 8 : DK);
  if (total <= 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (bf16_io)
    hipLaunchKernelGGL(k_assemble_bf16, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_assemble_f32, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
