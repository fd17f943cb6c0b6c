// Cache write of the VideoMLA chunk step (paper §3.1 Eq. 1, App. D.2, §3.2 Eq. 5,
// App. D.4): one fused kernel computes [W^KV_down; W^K_R] x for a block of tokens,
// RMS-normalises the d_c latent columns (times the gain), rotates the d_rope
// positional columns by 3D-RoPE at the token's absolute (t, y, x), rounds to the
// cache type and stores the row into ring slot (frame mod W).
//  * bf16: 32 tokens per workgroup, the full N = d_c + d_rope columns, 16x16x32
//    MFMA tiles spread over 4 waves, K tiles of 32 through LDS; the fp32 results
//    are then reread from LDS for the row-wise norm and rotation and stored as
//    16-byte chunks.
//  * fp32: one token per workgroup, SIMT dot products.
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {
namespace {

constexpr int kBM = 32;   // tokens per workgroup (bf16 path)
constexpr int kBK = 32;
constexpr int kLds = kBK + 8;

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

template <int N>
__global__ __launch_bounds__(256) void k_cache_write_bf16(CacheWriteArgs a) {
  constexpr int TILES = (kBM / 16) * (N / 16);
  static_assert(TILES % 4 == 0, "tiles must split evenly over 4 waves");
  constexpr int TPW = TILES / 4;
  constexpr int LDO = N + 4;  // fp32 epilogue tile stride
  constexpr int STAGE = (kBM + N) * kLds * 2;
  constexpr int EPI = kBM * LDO * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGE > EPI ? STAGE : EPI];
  bf16 *sX = (bf16 *)smem;
  bf16 *sW = sX + kBM * kLds;
  float *tile = (float *)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * kBM;
  const bf16 *X = (const bf16 *)a.x;
  const bf16 *Wkv = (const bf16 *)a.w_kv, *Wkr = (const bf16 *)a.w_kr;

  constexpr int W_CH = (N * 4 + 255) / 256;
  uint4 rx, rw[W_CH];
  auto load = [&](int k0) {
    if (tid < kBM * 4) {
      int r = tid >> 2, kc = (tid & 3) * 8, gm = m0 + r;
      rx = gm < a.M ? *(const uint4 *)(X + (int64_t)gm * a.d + k0 + kc) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < W_CH; ++c) {
      int id = tid + c * 256;
      if (id < N * 4) {
        int r = id >> 2, kc = (id & 3) * 8;
        const bf16 *src = r < a.d_c ? Wkv + (int64_t)r * a.d : Wkr + (int64_t)(r - a.d_c) * a.d;
        rw[c] = *(const uint4 *)(src + k0 + kc);
      }
    }
  };
  auto store = [&]() {
    if (tid < kBM * 4) *(uint4 *)(sX + (tid >> 2) * kLds + (tid & 3) * 8) = rx;
#pragma unroll
    for (int c = 0; c < W_CH; ++c) {
      int id = tid + c * 256;
      if (id < N * 4) *(uint4 *)(sW + (id >> 2) * kLds + (id & 3) * 8) = rw[c];
    }
  };

  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int l16 = lane & 15, kg = (lane >> 4) * 8;
  const int nk = a.d / kBK;
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store();
    __syncthreads();
    if (kt + 1 < nk) load((kt + 1) * kBK);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int tile_id = wave + 4 * t, tr = tile_id % (kBM / 16), tc = tile_id / (kBM / 16);
      bf16x8 av = *(const bf16x8 *)(sX + (tr * 16 + l16) * kLds + kg);
      bf16x8 bv = *(const bf16x8 *)(sW + (tc * 16 + l16) * kLds + kg);
      acc[t] = mfma16(av, bv, acc[t]);
    }
  }
  __syncthreads();
  // spill the accumulators to the fp32 tile: lane holds column l16, rows 4*(lane/16)+j
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile_id = wave + 4 * t, tr = tile_id % (kBM / 16), tc = tile_id / (kBM / 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) tile[(tr * 16 + (lane >> 4) * 4 + j) * LDO + tc * 16 + l16] = acc[t][j];
  }
  __syncthreads();
  finish_rows<bf16>(tile, LDO, kBM, m0, a);
  __syncthreads();
  // 16-byte stores of the finished rows into the ring
  bf16 *cache = (bf16 *)a.cache;
  for (int id = tid; id < kBM * (N / 8); id += 256) {
    const int r = id / (N / 8), c8 = (id % (N / 8)) * 8, m = m0 + r;
    if (m >= a.M) continue;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)tile[r * LDO + c8 + e];
    *(bf16x8 *)(cache + ring_row(a, m) * N + c8) = v;
  }
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
  dim3 grid((a.M + kBM - 1) / kBM);
  switch (a.d_c + a.d_rope) {
    case 160: hipLaunchKernelGGL(k_cache_write_bf16<160>, grid, dim3(256), 0, st, a); break;
    case 224: hipLaunchKernelGGL(k_cache_write_bf16<224>, grid, dim3(256), 0, st, a); break;
    case 256: hipLaunchKernelGGL(k_cache_write_bf16<256>, grid, dim3(256), 0, st, a); break;
    case 288: hipLaunchKernelGGL(k_cache_write_bf16<288>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t cache_write_f32(const CacheWriteArgs &a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  size_t lds = (size_t)(a.d + a.d_c + a.d_rope) * sizeof(float);
  hipLaunchKernelGGL(k_cache_write_f32, dim3(a.M), dim3(256), lds, st, a);
  return hipGetLastError();
}

}  // namespace mla
