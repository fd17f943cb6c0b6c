// Cache write of the VideoMLA chunk step (paper §3.1 Eq. 1, App. D.2, §3.2 Eq. 5,
// App. D.4): one fused kernel computes [W^KV_down; W^K_R] x for a block of tokens,
// RMS-normalises the d_c latent columns (times the gain), rotates the d_rope
// positional columns by 3D-RoPE at the token's absolute (t, y, x), rounds to the
// cache type and stores the row into ring slot (frame mod W).
//  * bf16: 32 tokens per workgroup and the full N = d_c + d_rope columns, one
//    wave per 32 columns with 16x16x32 MFMA tiles; the fp32 results are reread
//    from LDS for the row-wise norm and rotation and stored as 16-byte chunks.
//  * fp32: one token per workgroup, SIMT dot products.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {
namespace {

constexpr int kBM = 32;   // tokens per workgroup (bf16 path)

// Row-wise finish on an fp32 tile in LDS: tile[r * ld + c] holds the projections
// of token m0 + r.  8 threads per row.  Results are written back into the tile.
template <typename T>
__device__ void finish_rows(float *tile, int ld, int rows, int m0, const CacheWriteArgs &a) {
  const int N = a.d_c + a.d_rope;
  const int t = threadIdx.x, r = t >> 3, sub = t & 7;
  const bool active = r < rows && (m0 + r) < a.M;
  float ss = 0.f;
  if (active)
    for (int c = sub; c < a.d_c; c += 8) {
      float v = tile[r * ld + c];
      ss += v * v;
    }
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  ss += __shfl_xor(ss, 4, 64);
  if (!active) return;
  const float inv = 1.0f / sqrtf(ss / (float)a.d_c + a.eps);
  const T *g = (const T *)a.g_kv;
  for (int c = sub; c < a.d_c; c += 8) {
    float gain = g ? to_f32(g[c]) : 1.0f;
    tile[r * ld + c] = tile[r * ld + c] * inv * gain;
  }
  const int m = m0 + r, i = m % a.T_q, n = i % a.tpf;
  const float pos[3] = {(float)(a.t0 + i / a.tpf), (float)(n / a.grid_w), (float)(n % a.grid_w)};
  for (int p = sub; p < a.rope.n_pairs; p += 8) {
    float re = tile[r * ld + a.d_c + 2 * p], im = tile[r * ld + a.d_c + 2 * p + 1];
    rope_rotate(re, im, pos[a.rope.axis[p]], a.rope.omega[p]);
    tile[r * ld + a.d_c + 2 * p] = re;
    tile[r * ld + a.d_c + 2 * p + 1] = im;
  }
  (void)N;
}

__device__ __forceinline__ int64_t ring_row(const CacheWriteArgs &a, int m) {
  const int b = m / a.T_q, i = m % a.T_q;
  const int64_t f = a.t0 + i / a.tpf;
  return (int64_t)b * a.cache_batch_rows + (f % a.W) * a.tpf + (i % a.tpf);
}

// bf16: the 32-token x tile stays in LDS for the whole reduction; wave w owns
// output columns [32w, 32w+32) and streams those weight rows from global memory
// straight into 16x16x32 MFMA B operands (lane: column l%16, 8 consecutive k),
// PREF k-steps ahead, so the per-CU weight stream is not serialised behind one
// load round trip per k-step.
template <int N>
__global__ __launch_bounds__(64 * (N / 32)) void k_cache_write_bf16(CacheWriteArgs a) {
  constexpr int NWAVE = N / 32;
  constexpr int NT = 64 * NWAVE;
  constexpr int PREF = 8;  // k-steps of 32 in flight per lane
  constexpr int LDO = N + 4;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int LDX = a.d + 8;
  bf16 *sX = (bf16 *)smem;
  float *tile = (float *)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kg = (lane >> 4) * 8;
  const int m0 = blockIdx.x * kBM;
  const bf16 *X = (const bf16 *)a.x;

  // x tile -> LDS (rows past the end are zero), XB loads in flight per thread
  constexpr int XB = 16;
  const int cpr = a.d / 8, nchunk = kBM * cpr;
  for (int c0 = 0; c0 < nchunk; c0 += XB * NT) {
    uint4 v[XB];
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int c = c0 + i * NT + tid, r = c / cpr, gm = m0 + r;
      v[i] = (c < nchunk && gm < a.M) ? *(const uint4 *)(X + (int64_t)gm * a.d + (c % cpr) * 8)
                                      : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int c = c0 + i * NT + tid;
      if (c < nchunk) *(uint4 *)(sX + (c / cpr) * LDX + (c % cpr) * 8) = v[i];
    }
  }

  // this lane's two weight rows (columns n of the two 16-wide output tiles)
  const bf16 *wrow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = wave * 32 + j * 16 + l16;
    wrow[j] = (n < a.d_c ? (const bf16 *)a.w_kv + (int64_t)n * a.d
                         : (const bf16 *)a.w_kr + (int64_t)(n - a.d_c) * a.d) + kg;
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  auto step = [&](int k, const bf16x8 (&b)[2]) {
    const bf16x8 a0 = *(const bf16x8 *)(sX + l16 * LDX + k + kg);
    const bf16x8 a1 = *(const bf16x8 *)(sX + (16 + l16) * LDX + k + kg);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[0][j] = mfma16(a0, b[j], acc[0][j]);
      acc[1][j] = mfma16(a1, b[j], acc[1][j]);
    }
  };
  const int nsteps = a.d / 32, nfull = nsteps / PREF;
  bf16x8 cur[PREF][2], nxt[PREF][2];
  if (nfull > 0) {
#pragma unroll
    for (int s = 0; s < PREF; ++s)
#pragma unroll
      for (int j = 0; j < 2; ++j) cur[s][j] = *(const bf16x8 *)(wrow[j] + s * 32);
  }
  for (int c = 0; c < nfull; ++c) {
    const int kbase = c * PREF * 32;
    if (c + 1 < nfull) {
#pragma unroll
      for (int s = 0; s < PREF; ++s)
#pragma unroll
        for (int j = 0; j < 2; ++j) nxt[s][j] = *(const bf16x8 *)(wrow[j] + kbase + (PREF + s) * 32);
    }
#pragma unroll
    for (int s = 0; s < PREF; ++s) step(kbase + s * 32, cur[s]);
#pragma unroll
    for (int s = 0; s < PREF; ++s)
#pragma unroll
      for (int j = 0; j < 2; ++j) cur[s][j] = nxt[s][j];
  }
  for (int st = nfull * PREF; st < nsteps; ++st) {  // remaining k-steps, one at a time
    bf16x8 b[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8 *)(wrow[j] + st * 32);
    step(st * 32, b);
  }
  __syncthreads();
  // accumulators -> fp32 tile: lane holds column l16, rows 4*(lane/16)+r of each 16x16 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        tile[(i * 16 + (lane >> 4) * 4 + r) * LDO + wave * 32 + j * 16 + l16] = acc[i][j][r];
  __syncthreads();
  finish_rows<bf16>(tile, LDO, kBM, m0, a);
  __syncthreads();
  // 16-byte stores of the finished rows into the ring
  bf16 *cache = (bf16 *)a.cache;
  for (int id = tid; id < kBM * (N / 8); id += NT) {
    const int r = id / (N / 8), c8 = (id % (N / 8)) * 8, m = m0 + r;
    if (m >= a.M) continue;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)tile[r * LDO + c8 + e];
    *(bf16x8 *)(cache + ring_row(a, m) * N + c8) = v;
  }
}

template <int N>
hipError_t launch_bf16(const CacheWriteArgs &a, hipStream_t st) {
  const size_t lds_x = (size_t)kBM * (a.d + 8) * 2, lds_t = (size_t)kBM * (N + 4) * 4;
  const size_t lds = lds_x > lds_t ? lds_x : lds_t;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void *)k_cache_write_bf16<N>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_cache_write_bf16<N>, dim3((a.M + kBM - 1) / kBM), dim3(64 * (N / 32)), lds,
                     st, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_cache_write_f32(CacheWriteArgs a) {
  extern __shared__ float dyn[];
  const int N = a.d_c + a.d_rope;
  float *xs = dyn;          // d
  float *tile = dyn + a.d;  // N (+ pad)
  const int m = blockIdx.x, tid = threadIdx.x;
  const float *X = (const float *)a.x + (int64_t)m * a.d;
  for (int k = tid; k < a.d; k += 256) xs[k] = X[k];
  __syncthreads();
  for (int j = tid; j < N; j += 256) {
    const float *wr = j < a.d_c ? (const float *)a.w_kv + (int64_t)j * a.d
                                : (const float *)a.w_kr + (int64_t)(j - a.d_c) * a.d;
    float s = 0.f;
    for (int k = 0; k < a.d; ++k) s += wr[k] * xs[k];
    tile[j] = s;
  }
  __syncthreads();
  finish_rows<float>(tile, N, 1, m, a);
  __syncthreads();
  float *cache = (float *)a.cache;
  const int64_t row = ring_row(a, m);
  for (int j = tid; j < N; j += 256) cache[row * N + j] = tile[j];
}

}  // namespace

hipError_t cache_write_bf16(const CacheWriteArgs &a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  switch (a.d_c + a.d_rope) {
    case 160: return launch_bf16<160>(a, st);
    case 224: return launch_bf16<224>(a, st);
    case 256: return launch_bf16<256>(a, st);
    case 288: return launch_bf16<288>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t cache_write_f32(const CacheWriteArgs &a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  size_t lds = (size_t)(a.d + a.d_c + a.d_rope) * sizeof(float);
  hipLaunchKernelGGL(k_cache_write_f32, dim3(a.M), dim3(256), lds, st, a);
  return hipGetLastError();
}

}  // namespace mla
