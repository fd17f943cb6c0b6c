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
#include "rope_q_item.h"
#include "gemm_tile.h"

namespace mla {
namespace {

constexpr int kBM = 32;   // tokens per workgroup (bf16 path)

// Cross-lane steps inside a 16-lane row with DPP (no LDS round trip): the partner
// of lane l^1, and the sum over the row (quad swaps, then half-row and row mirrors,
// which pair up every 4- and 8-lane group with its complement).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor1(float v) { return dpp_mov<0xB1>(v); }  // quad_perm [1,0,3,2]
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}

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
  if (!a.rotate) return;
  const int m = m0 + r, i = m % a.T_q, n = i % a.tpf;
  const double pos[3] = {(double)(a.t0 + i / a.tpf), (double)(n / a.grid_w), (double)(n % a.grid_w)};
  for (int p = sub; p < a.rope.n_pairs; p += 8) {
    float re = tile[r * ld + a.d_c + 2 * p], im = tile[r * ld + a.d_c + 2 * p + 1];
    rope_rotate(re, im, pos[a.rope.axis[p]], a.rope.omega[p]);
    tile[r * ld + a.d_c + 2 * p] = re;
    tile[r * ld + a.d_c + 2 * p + 1] = im;
  }
  (void)N;
}

// Address of column c (of the d_c + d_rope) of the ring row that chunk token m
// goes to: request m / T_q, slot of its frame, token within the frame.  A
// 16-byte piece of 8 columns never straddles the two parts (d_c % 8 == 0 on the
// bf16 path).
template <typename T>
__device__ __forceinline__ T *ring_elem(const CacheWriteArgs &a, int m, int c) {
  const int b = m / a.T_q, i = m % a.T_q;
  const int64_t f = a.t0 + i / a.tpf;
  const int64_t slot = f < a.S ? f : a.S + (f - a.S) % a.W;
  const int64_t row = slot * a.tpf + (i % a.tpf);
  return c < a.d_c ? (T *)a.ring.c_kv + b * a.ring.c_batch + row * a.ring.c_row + c
                   : (T *)a.ring.k_r + b * a.ring.r_batch + row * a.ring.r_row + (c - a.d_c);
}

// bf16: the 32-token x tile stays in LDS for the whole reduction; wave w owns
// output columns [32w, 32w+32) and streams those weight rows from global memory
// straight into 16x16x32 MFMA B operands through a ring of PREF k-steps per lane
// (each slot is refilled right after its MFMAs, so PREF steps stay in flight).
// The first weight loads are issued before the x tile's, so the L2-resident
// weights arrive while x comes from HBM.  The finish works on the accumulators:
// per-token sums of squares are reduced across the 16 lanes of a column tile and
// across waves through LDS, the RoPE pair partner is the neighbouring lane, and
// the bf16 rows go through a small LDS tile for 16-byte ring stores.
template <int N>
__global__ __launch_bounds__(64 * (N / 32)) void k_cache_write_bf16(CacheWriteArgs a) {
  constexpr int NWAVE = N / 32;
  constexpr int NT = 64 * NWAVE;
  // k-steps of 32 in flight per lane; nine waves (N = 288) leave fewer registers
  constexpr int PREF = N <= 256 ? 12 : 6;
  constexpr int LDT = N + 8; // row stride (elements) of the bf16 output tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int LDX = a.d + 8;
  bf16 *sX = (bf16 *)smem;
  bf16 *tileo = (bf16 *)smem;                            // after the reduction
  float *ssum = (float *)(smem + kBM * LDT * 2);         // [NWAVE][kBM]
  float *sinv = ssum + NWAVE * kBM;                      // [kBM]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, kg = (lane >> 4) * 8;
  const int m0 = blockIdx.x * kBM;
  const int nsteps = a.d / 32;
  const bf16 *X = (const bf16 *)a.x;

  // this lane's two weight rows (columns n of the two 16-wide output tiles)
  const bf16 *wrow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = wave * 32 + j * 16 + l16;
    wrow[j] = (n < a.d_c ? (const bf16 *)a.w_kv + (int64_t)n * a.d
                         : (const bf16 *)a.w_kr + (int64_t)(n - a.d_c) * a.d) + kg;
  }
  // Every workgroup needs all of W.  Workgroups start the k loop at different
  // k-steps (step st reads k-block (st + rot) mod nsteps), so at any moment they
  // request different weight lines and the reads spread over all L2 channels
  // instead of queueing on the few that hold one k-block.
  const int rot = (int)((blockIdx.x * 7u) % (unsigned)nsteps);
  auto kblk = [&](int st) { return st + rot < nsteps ? st + rot : st + rot - nsteps; };
  bf16x8 ring[PREF][2];
#pragma unroll
  for (int s = 0; s < PREF; ++s)
    if (s < nsteps)
#pragma unroll
      for (int j = 0; j < 2; ++j) ring[s][j] = *(const bf16x8 *)(wrow[j] + kblk(s) * 32);

  // x tile -> LDS (rows past the end are zero), XB loads in flight per thread
  constexpr int XB = N <= 256 ? 16 : 8;
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
  __syncthreads();

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // x fragments of step st (tokens l16 and 16 + l16), read one step ahead
  auto xfr = [&](int st, int h) {
    return *(const bf16x8 *)(sX + (h * 16 + l16) * LDX + kblk(st) * 32 + kg);
  };
  auto mma = [&](const bf16x8 (&xa)[2], const bf16x8 (&w)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[0][j] = mfma16(xa[0], w[j], acc[0][j]);
      acc[1][j] = mfma16(xa[1], w[j], acc[1][j]);
    }
  };
  // Whole chunks of PREF steps run without branches: every step refills its ring
  // slot (past the end with a clamped, unused k-block), so the number of loads in
  // flight is the same on every path and each wait is for exactly the slot's load.
  const int nfull = nsteps / PREF;
  bf16x8 xa[2][2];
  xa[0][0] = xfr(0, 0);
  xa[0][1] = xfr(0, 1);
  for (int c = 0; c < nfull * PREF; c += PREF) {
#pragma unroll
    for (int s = 0; s < PREF; ++s) {
      const int st = c + s, nx = min(st + 1, nsteps - 1);
      xa[(s + 1) & 1][0] = xfr(nx, 0);
      xa[(s + 1) & 1][1] = xfr(nx, 1);
      mma(xa[s & 1], ring[s]);
      const int kr = kblk(min(st + PREF, nsteps - 1)) * 32;
#pragma unroll
      for (int j = 0; j < 2; ++j) ring[s][j] = *(const bf16x8 *)(wrow[j] + kr);
    }
  }
  // remaining steps (nsteps not a multiple of PREF): their weights are in the ring
#pragma unroll
  for (int s = 0; s < PREF; ++s) {
    const int st = nfull * PREF + s;
    if (st < nsteps) {
      const bf16x8 xt[2] = {xfr(st, 0), xfr(st, 1)};
      mma(xt, ring[s]);
    }
  }

  // Lane holds column l16 of each 16x16 tile, tokens 16i + 4(lane/16) + r.
  const bool latent = wave * 32 < a.d_c;  // d_c is a multiple of 32: whole waves
  __syncthreads();                         // x tile no longer read
  if (latent) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float q = row16_sum(acc[i][0][r] * acc[i][0][r] + acc[i][1][r] * acc[i][1][r]);
        if (l16 == 0) ssum[wave * kBM + i * 16 + (lane >> 4) * 4 + r] = q;
      }
  }
  __syncthreads();
  if (tid < kBM) {
    float q = 0.f;
    for (int w = 0; w < a.d_c / 32; ++w) q += ssum[w * kBM + tid];
    sinv[tid] = 1.0f / sqrtf(q / (float)a.d_c + a.eps);
  }
  __syncthreads();

  if (latent) {
    const bf16 *gk = (const bf16 *)a.g_kv;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = wave * 32 + j * 16 + l16;
      const float gain = gk ? to_f32(gk[col]) : 1.0f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = i * 16 + (lane >> 4) * 4 + r;
          tileo[t * LDT + col] = (bf16)(acc[i][j][r] * sinv[t] * gain);
        }
    }
  } else {
    // RoPE columns: pair p = (col - d_c)/2 holds (re, im) in lanes l16 even / odd.
    // The wave's pairs are p0 + (0..15); each lane picks its two (axis, omega)
    // with wave-uniform table reads.
    const int p0 = (wave * 32 - a.d_c) / 2;
    int ax[2] = {0, 0};
    double om[2] = {0.0, 0.0};
    for (int q = 0; q < 16; ++q) {
      const int pq = p0 + q;
      const int axq = a.rope.axis[pq];
      const double omq = a.rope.omega[pq];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (j * 8 + (l16 >> 1) == q) {
          ax[j] = axq;
          om[j] = omq;
        }
    }
    const bool even = (l16 & 1) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = i * 16 + (lane >> 4) * 4 + r, m = m0 + t, ti = m % a.T_q, n = ti % a.tpf;
        const double pos[3] = {(double)(a.t0 + ti / a.tpf), (double)(n / a.grid_w), (double)(n % a.grid_w)};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float v = acc[i][j][r], other = dpp_xor1(v);
          float re = even ? v : other, im = even ? other : v;
          if (a.rotate) rope_rotate(re, im, pos[ax[j]], om[j]);
          tileo[t * LDT + wave * 32 + j * 16 + l16] = (bf16)(even ? re : im);
        }
      }
  }
  __syncthreads();
  // 16-byte stores of the finished rows into the ring
  for (int id = tid; id < kBM * (N / 8); id += NT) {
    const int r = id / (N / 8), c8 = (id % (N / 8)) * 8, m = m0 + r;
    if (m < a.M) *(bf16x8 *)ring_elem<bf16>(a, m, c8) = *(const bf16x8 *)(tileo + r * LDT + c8);
  }
}

// bf16 with direct global->LDS loads (d a multiple of 64).  Per 64-wide k chunk a
// stage holds the 32 x rows and all N weight rows (128 bytes each), filled by
// global_load_lds_dwordx4: wave w brings its own 32 weight rows, waves 0-3 the x
// rows.  NS stages are in flight.  16-byte chunk c of stage row r sits at chunk
// c ^ ((r >> 1) & 7), which keeps the 16-row fragment reads free of bank
// conflicts; the swizzle is applied on the global side of each load.  The RoPE
// cos/sin of the workgroup's (token, pair)s are computed by all threads while the
// first stages are in flight.  The finish is that of k_cache_write_bf16.
template <int N, int BM = kBM>
struct CwDma {
  static constexpr int NWAVE = N / 32, NT = 64 * NWAVE;
  static constexpr int KC = 64;                         // k per stage
  static constexpr int XB = BM * KC * 2;                // x bytes per stage
  static constexpr int WB = N * KC * 2;                 // weight bytes per stage
  static constexpr int SB = XB + WB;
  static constexpr int MAX_PAIRS = 32;
  static constexpr int RTAB = BM * MAX_PAIRS * 8;       // (cos, sin) of the tile's pairs
  static constexpr int NS_MAX = N <= 256 ? 4 : 3;
  static constexpr int NS = SB * NS_MAX + RTAB <= 163840 ? NS_MAX
                          : SB * (NS_MAX - 1) + RTAB <= 163840 ? NS_MAX - 1 : 2;  // stages
  static constexpr size_t LDS = (size_t)SB * NS + RTAB;
  static constexpr int RT = BM / 16;                    // 16-row MFMA tiles
  static constexpr int XR = BM / 8;                     // x load instructions per stage
  static constexpr int XW = XR <= NWAVE ? XR : (XR % NWAVE == 0 ? NWAVE : XR / 2);  // loading waves
  static constexpr int XQ = XR / XW;                    // ... and instructions each
  static_assert(BM % 16 == 0 && XW * XQ == XR && XW <= NWAVE, "x rows split evenly over waves");
  static_assert(LDS <= 163840, "LDS");
  static_assert(NWAVE >= 4, "at least four waves");
};

__device__ __forceinline__ int cw_swz(int row) { return (row >> 1) & 7; }

// wait until this wave's loads of the stages after the current one are all that
// is outstanding (LPS loads per stage)
template <int LPS>
__device__ __forceinline__ void wait_stage(int after) {
  if (after >= 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPS) : "memory");
  else if (after == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// One workgroup's tile: BM tokens, all N columns (32 by default; taller tiles let
// fewer workgroups cover the chunk, for a launch beside other work).
template <int N, int BM = kBM>
__device__ __forceinline__ void cache_write_dma_block(const CacheWriteArgs &a, int block) {
  using C = CwDma<N, BM>;
  constexpr int NT = C::NT, KC = C::KC, NS = C::NS, NWAVE = C::NWAVE, RT = C::RT, XQ = C::XQ;
  constexpr int LDT = N + 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  typedef __attribute__((address_space(3))) void lds_void;
  float2 *rtab = (float2 *)(smem + (size_t)C::SB * NS);  // [BM][n_pairs]: (cos, sin)
  bf16 *tileo = (bf16 *)smem;                             // after the k loop
  float *ssum = (float *)(smem + BM * LDT * 2);           // [NWAVE][BM]
  float *sinv = ssum + NWAVE * BM;                        // [BM]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, kg = lane >> 4;
  const int m0 = block * BM;
  const int nk = a.d / KC;
  const int np = a.d_rope / 2;

  // sources of this lane's loads: load i of wave w fills stage rows 8i + lane/8 of
  // the wave's weight rows (and, for waves below XW, x rows 8(w XQ + q) + lane/8),
  // slot lane%8
  const int slot = lane & 7, rsub = lane >> 3;
  const bf16 *wsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * i + rsub, n = wave * 32 + row;
    const bf16 *base = n < a.d_c ? (const bf16 *)a.w_kv + (int64_t)n * a.d
                                 : (const bf16 *)a.w_kr + (int64_t)(n - a.d_c) * a.d;
    wsrc[i] = base + (slot ^ cw_swz(row)) * 8;
  }
  const bool xload = wave < C::XW;
  const bf16 *xsrc[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int row = 8 * (wave * XQ + q) + rsub, gm = min(m0 + row, a.M - 1);  // past M: any valid row
    xsrc[q] = (const bf16 *)a.x + (int64_t)gm * a.d + (slot ^ cw_swz(row)) * 8;
  }
  auto issue = [&](int kc) {
    unsigned char *st = smem + (size_t)(kc % NS) * C::SB;
    const int k0 = kc * KC;
    if (xload)
#pragma unroll
      for (int q = 0; q < XQ; ++q)
        __builtin_amdgcn_global_load_lds((const void *)(xsrc[q] + k0),
                                         (lds_void *)(st + (wave * XQ + q) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds((const void *)(wsrc[i] + k0),
                                       (lds_void *)(st + C::XB + wave * 4096 + i * 1024), 16, 0, 0);
  };
#pragma unroll
  for (int kc = 0; kc < NS - 1; ++kc)
    if (kc < nk) issue(kc);

  // RoPE table of this workgroup's tokens (keys kept unrotated need none)
  for (int e = tid; a.rotate && e < BM * np; e += NT) {
    const int t = e / np, p = e % np, m = m0 + t, ti = m % a.T_q, n = ti % a.tpf;
    const int ax = a.rope.axis[p];
    const double om = a.rope.omega[p];
    const double pos = ax == 0 ? (double)(a.t0 + ti / a.tpf) : (ax == 1 ? (double)(n / a.grid_w) : (double)(n % a.grid_w));
    float sn, cs;
    rope_sincos(pos, om, sn, cs);
    rtab[e] = make_float2(cs, sn);
  }

  f32x4 acc[RT][2];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < nk; ++kc) {
    const int after = min(NS - 2, nk - 1 - kc);
    if (xload)
      wait_stage<4 + XQ>(after);
    else
      wait_stage<4>(after);
    // A bare barrier: __syncthreads() would also wait for the later stages' loads,
    // which are meant to stay in flight.  Before it this wave's reads of the stage
    // refilled next (read in the previous chunk) are complete; the clobbers keep the
    // compiler from moving LDS accesses across it.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kc + NS - 1 < nk) issue(kc + NS - 1);
    const unsigned char *st = smem + (size_t)(kc % NS) * C::SB;
    const unsigned char *sw = st + C::XB + wave * 4096;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 wb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 16 * h + l16, ch = (4 * s + kg) ^ cw_swz(row);
        wb[h] = *(const bf16x8 *)(sw + row * 128 + ch * 16);
      }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int row = 16 * i + l16, ch = (4 * s + kg) ^ cw_swz(row);
        const bf16x8 xa = *(const bf16x8 *)(st + row * 128 + ch * 16);
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16(xa, wb[j], acc[i][j]);
      }
    }
  }

  // Lane holds column l16 of each 16x16 tile, tokens 16i + 4(lane/16) + r.
  const bool latent = wave * 32 < a.d_c;
  __syncthreads();  // stages no longer read
  if (latent) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float q = row16_sum(acc[i][0][r] * acc[i][0][r] + acc[i][1][r] * acc[i][1][r]);
        if (l16 == 0) ssum[wave * BM + i * 16 + (lane >> 4) * 4 + r] = q;
      }
  }
  __syncthreads();
  if (tid < BM) {
    float q = 0.f;
    for (int w = 0; w < a.d_c / 32; ++w) q += ssum[w * BM + tid];
    sinv[tid] = 1.0f / sqrtf(q / (float)a.d_c + a.eps);
  }
  __syncthreads();
  if (latent) {
    const bf16 *gk = (const bf16 *)a.g_kv;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = wave * 32 + j * 16 + l16;
      const float gain = gk ? to_f32(gk[col]) : 1.0f;
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = i * 16 + (lane >> 4) * 4 + r;
          tileo[t * LDT + col] = (bf16)(acc[i][j][r] * sinv[t] * gain);
        }
    }
  } else {
    // RoPE columns: pair p = (col - d_c)/2 holds (re, im) in lanes l16 even / odd
    const bool even = (l16 & 1) == 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = wave * 32 + j * 16 + l16, p = (col - a.d_c) >> 1;
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = i * 16 + (lane >> 4) * 4 + r;
          const float v = acc[i][j][r], other = dpp_xor1(v);
          float re = even ? v : other, im = even ? other : v;
          const float2 cs = a.rotate ? rtab[t * np + p] : make_float2(1.f, 0.f);
          rotate_by(re, im, cs.y, cs.x);
          tileo[t * LDT + col] = (bf16)(even ? re : im);
        }
    }
  }
  __syncthreads();
  for (int id = tid; id < BM * (N / 8); id += NT) {
    const int r = id / (N / 8), c8 = (id % (N / 8)) * 8, m = m0 + r;
    if (m < a.M) *(bf16x8 *)ring_elem<bf16>(a, m, c8) = *(const bf16x8 *)(tileo + r * LDT + c8);
  }
}

template <int N>
__global__ __launch_bounds__(64 * (N / 32)) void k_cache_write_dma(CacheWriteArgs a) {
  cache_write_dma_block<N>(a, blockIdx.x);
}

// The same write with the chunk step's query RoPE riding along: the first cw_blocks
// workgroups write the cache, the rest (on the CUs those leave idle: 147 of 256 at
// the Wan-1.3B chunk) rotate the rope columns of the absorbed query rows in place and
// clear the attention's overflow flags, work items strided over them.  The two jobs
// share no data; one launch replaces two.
template <int N>
__global__ __launch_bounds__(64 * (N / 32)) void k_cache_write_dma_rope(CacheWriteArgs a, RopeQArgs r,
                                                                        int cw_blocks) {
  if ((int)blockIdx.x < cw_blocks) {
    cache_write_dma_block<N>(a, blockIdx.x);
    return;
  }
  const int64_t items = rope_q_items(r, 4);
  const int64_t stride = (int64_t)(gridDim.x - cw_blocks) * blockDim.x;
  for (int64_t idx = (int64_t)(blockIdx.x - cw_blocks) * blockDim.x + threadIdx.x; idx < items;
       idx += stride)
    rope_q_item<bf16, 4>(r, idx);
}

template <int N>
hipError_t launch_dma_rope(const CacheWriteArgs &a, const RopeQArgs &r, int rope_blocks,
                           hipStream_t st) {
  using C = CwDma<N>;
  hipError_t e = hipFuncSetAttribute((const void *)k_cache_write_dma_rope<N>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  if (e != hipSuccess) return e;
  const int cw = (a.M + kBM - 1) / kBM;
  hipLaunchKernelGGL(k_cache_write_dma_rope<N>, dim3(cw + rope_blocks), dim3(C::NT), C::LDS, st, a,
                     r, cw);
  return hipGetLastError();
}

// The step's absorbed query GEMM (256x256 tiles whose rows are scaled by their RMS)
// with the cache write of the same step in one launch: the GEMM's 209 tiles leave 47
// of 256 CUs idle for its ~32 us, and the write, in tiles of kBMQ tokens (42 at the
// Wan-1.3B chunk, each ~1 MB of weights and x), fits beside it.  Workgroups below
// g_tiles run GEMM tiles with the numbering of the GEMM's own launch (so the same
// XCD-aware tile order); the rest write the cache with the first N/32 of their waves
// (the others end at once; barriers wait only for waves still running).  The jobs
// share no data.
constexpr int kBMQ = 112;
using QueryTile = GemmDma<256, 256, 128, 64, 64, 2, false, EP_ROW_RMS>;

template <int N>
__global__ __launch_bounds__(QueryTile::NT) __attribute__((amdgpu_waves_per_eu(2, 8)))
void k_query_gemm_cache_write(GemmArgs g, int g_nbx, int g_tiles, CacheWriteArgs a, RopeQArgs r) {
  if ((int)blockIdx.x < g_tiles) {
    // the query rows come out rotated (the step's RoPE pass, done in the tile)
    gemm_dma_tile<256, 256, 128, 64, 64, 2, false, EP_ROW_RMS, true>(g, blockIdx.x, g_nbx, g_tiles, 0,
                                                                     &r);
    return;
  }
  if ((int)blockIdx.x == g_tiles)  // the attention's overflow flags, cleared on the way
    for (int i = threadIdx.x; i < r.n_zero; i += blockDim.x) r.zero[i] = 0;
  if ((int)threadIdx.x >= CwDma<N, kBMQ>::NT) return;
  cache_write_dma_block<N, kBMQ>(a, blockIdx.x - g_tiles);
}

template <int N>
hipError_t launch_dma(const CacheWriteArgs &a, hipStream_t st) {
  using C = CwDma<N>;
  hipError_t e = hipFuncSetAttribute((const void *)k_cache_write_dma<N>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_cache_write_dma<N>, dim3((a.M + kBM - 1) / kBM), dim3(C::NT), C::LDS, st, a);
  return hipGetLastError();
}

template <int N>
hipError_t launch_bf16(const CacheWriteArgs &a, hipStream_t st) {
  const size_t lds_x = (size_t)kBM * (a.d + 8) * 2;
  const size_t lds_t = (size_t)kBM * (N + 8) * 2 + (size_t)(N / 32 + 1) * kBM * 4;
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
  for (int j = tid; j < N; j += 256) *ring_elem<float>(a, m, j) = tile[j];
}

}  // namespace

hipError_t cache_write_bf16(const CacheWriteArgs &a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (a.d % CwDma<224>::KC == 0 && a.d_rope / 2 <= CwDma<224>::MAX_PAIRS) {
    switch (a.d_c + a.d_rope) {
      case 160: return launch_dma<160>(a, st);
      case 224: return launch_dma<224>(a, st);
      case 256: return launch_dma<256>(a, st);
      case 288: return launch_dma<288>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.d_c + a.d_rope) {
    case 160: return launch_bf16<160>(a, st);
    case 224: return launch_bf16<224>(a, st);
    case 256: return launch_bf16<256>(a, st);
    case 288: return launch_bf16<288>(a, st);
    default: return hipErrorInvalidValue;
  }
}

int query_gemm_cache_write_blocks(const GemmArgs &g, const CacheWriteArgs &a) {
  if (a.M <= 0 || a.d_c + a.d_rope != 224 || a.d % CwDma<224>::KC != 0 ||
      a.d_rope / 2 > CwDma<224>::MAX_PAIRS)
    return 0;
  if (g.batch != 1 || !g.ssq_in || g.ssq_out || g.N < 512 || g.K % 64 != 0) return 0;
  const int tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256);
  if (tiles < 200) return 0;  // the GEMM would not take 256x256 tiles
  return tiles + (a.M + kBMQ - 1) / kBMQ;
}

hipError_t query_gemm_cache_write(const GemmArgs &g, const CacheWriteArgs &a, const RopeQArgs &r,
                                  hipStream_t st) {
  const int total = query_gemm_cache_write_blocks(g, a);
  if (total <= 0 || !r.in_place || r.d_c % 8 || (r.d_c + r.d_rope) % 8 || r.d_c + r.d_rope < 64 ||
      (int64_t)r.n_h * (r.d_c + r.d_rope) != g.N || r.M != g.M)
    return hipErrorInvalidValue;
  const int nbx = (g.N + 255) / 256, tiles = nbx * ((g.M + 255) / 256);
  // the GEMM tile with its rotation table, or the write's tile
  constexpr size_t lds_g = QueryTile::LDS + RopeLds<256>::BYTES;
  static_assert(lds_g <= 163840, "LDS");
  const size_t lds = lds_g > CwDma<224, kBMQ>::LDS ? lds_g : CwDma<224, kBMQ>::LDS;
  hipError_t e = hipFuncSetAttribute((const void *)k_query_gemm_cache_write<224>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_query_gemm_cache_write<224>, dim3(total), dim3(QueryTile::NT), lds, st, g, nbx,
                     tiles, a, r);
  return hipGetLastError();
}

bool cache_write_takes_rope(const CacheWriteArgs &a, const RopeQArgs &r) {
  const int n = a.d_c + a.d_rope;
  return a.M > 0 && a.d % CwDma<224>::KC == 0 && a.d_rope / 2 <= CwDma<224>::MAX_PAIRS &&
         (n == 160 || n == 224 || n == 256 || n == 288) && r.in_place && (r.d_rope / 2) % 4 == 0;
}

hipError_t cache_write_bf16_rope(const CacheWriteArgs &a, const RopeQArgs &r, int rope_blocks,
                                 hipStream_t st) {
  if (!cache_write_takes_rope(a, r) || rope_blocks < 1) return hipErrorInvalidValue;
  switch (a.d_c + a.d_rope) {
    case 160: return launch_dma_rope<160>(a, r, rope_blocks, st);
    case 224: return launch_dma_rope<224>(a, r, rope_blocks, st);
    case 256: return launch_dma_rope<256>(a, r, rope_blocks, st);
    case 288: return launch_dma_rope<288>(a, r, rope_blocks, st);
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
