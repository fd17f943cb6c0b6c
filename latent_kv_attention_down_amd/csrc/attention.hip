// Latent chunk attention of the VideoMLA step (paper §3.3 Eq. 7 in the absorbed
// form of App. E, Eq. 8, 12 and 16).
//
// Rows are (token, head) pairs of absorbed queries q_lat = [q~_h | q^rope_h] of
// width DK = d_c + d_rope, pre-scaled by log2(e)/sqrt(d_h); keys are the ring rows
// K_j = [c_j | k^rope_j] shared by every head.  For each row the kernel takes
// s_j = q_lat . K_j over the valid window, a base-2 softmax in fp32, and
// O = sum_j a_j c_j over the d_c latent columns (V is the first d_c columns of K).
//
// gfx950 mapping (bf16):
//  * a workgroup is 4 waves; each wave owns QT tiles of 32 query rows and keeps
//    their q_lat in registers as MFMA B operands for the whole window;
//  * key tiles of 64 ring rows are staged once per workgroup in LDS twice: key-
//    major (A operand of S^T = K Q^T, contraction over features) and, for the d_c
//    latent columns, feature-major (A operand of O^T = V^T P^T, contraction over
//    keys).  The transposed copy is written from the registers that carry the
//    global loads, so HBM/L2 is read once per tile;
//  * S^T comes out of v_mfma_f32_32x32x16_bf16 with one query per lane column, so
//    the row max needs one cross-lane step (lane l and l^32) and the bf16
//    probabilities feed the next MFMA as its B operand without a shuffle;
//  * fast path: each row's softmax reference is the max of the first key tile the
//    workgroup sees for it and is never moved, so O is never rescaled inside the
//    loop (a rescale would drag the AGPR-resident accumulators through VGPRs).
//    Any row whose later scores exceed the reference by more than 64 (base 2) has
//    its row tile flagged, and the safe kernel (reference raised lazily, O
//    rescaled) recomputes exactly those row tiles.  Below that bound every weight
//    is at most 2^64, far inside fp32 and bf16 range;
//  * the fast grid is persistent: workgroup g takes the flat range
//    [gT/G, (g+1)T/G) of T = (row tiles) x (key tiles) tile steps, so every CU gets
//    the same work.  A row tile finished by one workgroup is written directly; one
//    split across workgroups leaves normalised bf16 partials plus (m, l) per row,
//    merged by k_attn_merge in a fixed order (deterministic, no atomics).
#include "mla_device.h"
#include "mla_launch.h"

namespace mla {
namespace {

constexpr int BN = kAttnKeyTile;      // keys per tile
constexpr float kFastHeadroom = 64.f;  // log2 units above the fixed reference
constexpr float kSafeThreshold = 8.f;  // lazy rescale threshold of the safe kernel
constexpr int kSafeQT = 1;

struct Sched {
  int B, R, RTb, RT;
  int nk, KT;
  int start0, len0;
  int64_t cache_rows;
  int64_t T;
  int G;
};

__host__ __device__ __forceinline__ int wg_of(const Sched &s, int64_t flat) {
  return (int)(((flat + 1) * s.G - 1) / s.T);
}

template <int DC, int DR, int QT>
struct Cfg {
  static constexpr int DK = DC + DR;
  static constexpr int KB = DK / 16;
  static constexpr int FT = DC / 32;
  static constexpr int RW = 4 * QT * 32;
  static constexpr int KS = DK + 8;
  static constexpr int VS = BN + 8;
  static constexpr int LAT_PER_T = (BN / 2) * (DC / 8) / 256;
  static constexpr int ROPE_CH = BN * (DR / 8);
  static constexpr int ROPE_PER_T = (ROPE_CH + 255) / 256;
  static constexpr size_t LDS = (size_t)(BN * KS + DC * VS) * 2;
  static constexpr size_t REC = (size_t)RW * DC * 2 + (size_t)RW * 8;
  static_assert((BN / 2) * (DC / 8) % 256 == 0, "latent cells must split evenly");
  static_assert(DK % 16 == 0 && DC % 32 == 0, "bad widths");
};

// One workgroup's view of the ring: global -> registers -> LDS (key-major K and
// feature-major V^T), and the two MFMA contractions of a key tile.
template <int DC, int DR, int QT>
struct Tile {
  using C = Cfg<DC, DR, QT>;
  static constexpr int DK = C::DK, KB = C::KB, FT = C::FT, KS = C::KS, VS = C::VS;
  bf16 *Ks, *Vt;
  const bf16 *cb;  // this request's ring
  int nk, start0, len0;
  uint4 lat0[C::LAT_PER_T], lat1[C::LAT_PER_T], rop[C::ROPE_PER_T];

  __device__ __forceinline__ int64_t key_row(int kk) const {
    return kk < len0 ? (int64_t)(start0 + kk) : (int64_t)(kk - len0);
  }

  __device__ __forceinline__ void load(int kt, int tid) {
#pragma unroll
    for (int c = 0; c < C::LAT_PER_T; ++c) {
      const int cell = tid + 256 * c, p = cell / (DC / 8), ch = cell % (DC / 8);
      const int kk = kt * BN + 2 * p;
      lat0[c] = kk < nk ? *(const uint4 *)(cb + key_row(kk) * DK + ch * 8) : make_uint4(0, 0, 0, 0);
      lat1[c] = kk + 1 < nk ? *(const uint4 *)(cb + key_row(kk + 1) * DK + ch * 8)
                            : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < C::ROPE_PER_T; ++c) {
      const int id = tid + 256 * c;
      if (id < C::ROPE_CH) {
        const int key = id / (DR / 8), ch = id % (DR / 8), kk = kt * BN + key;
        rop[c] = kk < nk ? *(const uint4 *)(cb + key_row(kk) * DK + DC + ch * 8)
                         : make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void store(int tid) {
#pragma unroll
    for (int c = 0; c < C::LAT_PER_T; ++c) {
      const int cell = tid + 256 * c, p = cell / (DC / 8), ch = cell % (DC / 8);
      *(uint4 *)(Ks + (2 * p) * KS + ch * 8) = lat0[c];
      *(uint4 *)(Ks + (2 * p + 1) * KS + ch * 8) = lat1[c];
      const uint32_t *a0 = (const uint32_t *)&lat0[c], *a1 = (const uint32_t *)&lat1[c];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = (a0[d] & 0xffffu) | (a1[d] << 16);
        const uint32_t hi = (a0[d] >> 16) | (a1[d] & 0xffff0000u);
        *(uint32_t *)(Vt + (ch * 8 + 2 * d) * VS + 2 * p) = lo;
        *(uint32_t *)(Vt + (ch * 8 + 2 * d + 1) * VS + 2 * p) = hi;
      }
    }
#pragma unroll
    for (int c = 0; c < C::ROPE_PER_T; ++c) {
      const int id = tid + 256 * c;
      if (id < C::ROPE_CH) {
        const int key = id / (DR / 8), ch = id % (DR / 8);
        *(uint4 *)(Ks + key * KS + DC + ch * 8) = rop[c];
      }
    }
  }

  // S^T (keys x queries) for the 64 keys of tile kt; masked keys get -inf.
  __device__ __forceinline__ void scores(f32x16 (&S)[2][QT], const bf16x8 (&Qr)[QT][KB], int kt,
                                         int l32, int g) const {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[t][qt][r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 a = *(const bf16x8 *)(Ks + (t * 32 + l32) * KS + kb * 16 + g * 8);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) S[t][qt] = mfma32(a, Qr[qt][kb], S[t][qt]);
      }
    }
    if ((kt + 1) * BN > nk) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * BN + t * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          if (key >= nk)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) S[t][qt][r] = -INFINITY;
        }
    }
  }

  // O^T (features x queries) += V^T P^T over the tile's four 16-key blocks.
  __device__ __forceinline__ void values(f32x16 (&O)[FT][QT], const bf16x8 (&P)[BN / 16][QT],
                                         int l32, int g) const {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
        const bf16 *vr = Vt + (ft * 32 + l32) * VS + kb * 16 + g * 4;
        const uint2 lo = *(const uint2 *)vr, hi = *(const uint2 *)(vr + 8);
        uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8 a = *(const bf16x8 *)&u;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) O[ft][qt] = mfma32(a, P[kb][qt], O[ft][qt]);
      }
    }
  }
};

// Probabilities of one query tile as bf16 B operands: slot e of block 2t+h holds
// key t*32 + 16h + 4g + e, slot 4+e key t*32 + 16h + 8 + 4g + e (the MFMA output
// rows of S^T), matching the V^T fragments read in Tile::values.
template <int QT>
__device__ __forceinline__ float exp_and_pack(f32x16 (&S)[2][QT], bf16x8 (&P)[BN / 16][QT], int qt,
                                              float m) {
  float ls = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(S[t][qt][r] - m);
      S[t][qt][r] = p;
      ls += p;
    }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[e] = (bf16)S[t][qt][(2 * h) * 4 + e];
        pv[4 + e] = (bf16)S[t][qt][(2 * h + 1) * 4 + e];
      }
      P[2 * t + h][qt] = pv;
    }
  return ls;
}

template <int QT>
__device__ __forceinline__ float tile_max(const f32x16 (&S)[2][QT], int qt) {
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[t][qt][r]);
  return fmaxf(mx, __shfl_xor(mx, 32, 64));
}

template <int DK, int QT, int KB>
__device__ __forceinline__ void load_queries(bf16x8 (&Qr)[QT][KB], const bf16 *q, const Sched &s,
                                             int b, int row_base, int l32, int g) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = row_base + qt * 32 + l32;
    const bf16 *qr = q + ((int64_t)b * s.R + row) * DK + g * 8;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (row < s.R) {
        Qr[qt][kb] = *(const bf16x8 *)(qr + kb * 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) Qr[qt][kb][e] = (bf16)0.f;
      }
    }
  }
}

// Normalise and store 32 rows x DC: lane holds row l32, features ft*32 + 8i + 4g + j.
template <int FT, int QT>
__device__ __forceinline__ void store_rows(bf16 *dst, int64_t ld, const f32x16 (&O)[FT][QT], int qt,
                                           float inv, int g) {
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16 v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] = (bf16)(O[ft][qt][4 * i + j] * inv);
      *(uint2 *)(dst + ft * 32 + i * 8 + g * 4) = *(const uint2 *)v4;
    }
  (void)ld;
}

template <int DC, int DR, int QT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_latent_attn(const bf16 *__restrict__ q, const bf16 *__restrict__ cache,
                   bf16 *__restrict__ o, unsigned char *__restrict__ part, int *__restrict__ flags,
                   Sched s) {
  using C = Cfg<DC, DR, QT>;
  constexpr int KB = C::KB, FT = C::FT, RW = C::RW;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  Tile<DC, DR, QT> tl;
  tl.Ks = (bf16 *)lds;
  tl.Vt = tl.Ks + BN * C::KS;
  tl.nk = s.nk;
  tl.start0 = s.start0;
  tl.len0 = s.len0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int wg = blockIdx.x;
  const int64_t begin = (int64_t)wg * s.T / s.G, end = (int64_t)(wg + 1) * s.T / s.G;

  bf16x8 Qr[QT][KB];
  f32x16 O[FT][QT];
  bf16x8 P[BN / 16][QT];
  float m[QT], l[QT];

  int64_t flat = begin;
  while (flat < end) {
    const int rt = (int)(flat / s.KT);
    const int kt0 = (int)(flat - (int64_t)rt * s.KT);
    const int kt1 = (int)min((int64_t)s.KT, end - (int64_t)rt * s.KT);
    const int b = rt / s.RTb;
    const int row0 = (rt % s.RTb) * RW;
    tl.cb = cache + (int64_t)b * s.cache_rows * C::DK;

    load_queries<C::DK, QT, KB>(Qr, q, s, b, row0 + wave * QT * 32, l32, g);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      l[qt] = 0.f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[ft][qt][r] = 0.f;
    }
    bool over = false;

    tl.load(kt0, tid);
    for (int kt = kt0; kt < kt1; ++kt) {
      __syncthreads();
      tl.store(tid);
      __syncthreads();
      if (kt + 1 < kt1) tl.load(kt + 1, tid);

      f32x16 S[2][QT];
      tl.scores(S, Qr, kt, l32, g);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mx = tile_max<QT>(S, qt);
        if (kt == kt0) m[qt] = mx;  // fixed reference for this piece
        over |= mx > m[qt] + kFastHeadroom;
        l[qt] += exp_and_pack<QT>(S, P, qt, m[qt]);
      }
      tl.values(O, P, l32, g);
    }

    if (over) flags[rt] = 1;
    const bool whole = (kt0 == 0 && kt1 == s.KT);
    unsigned char *rec = part + (size_t)(wg + rt) * C::REC;
    float *rec_m = (float *)(rec + (size_t)RW * DC * 2);
    float *rec_l = rec_m + RW;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float lt = l[qt] + __shfl_xor(l[qt], 32, 64);
      const int lrow = wave * QT * 32 + qt * 32 + l32;
      const int row = row0 + lrow;
      if (row < s.R) {
        bf16 *dst = whole ? o + ((int64_t)b * s.R + row) * DC : (bf16 *)rec + (int64_t)lrow * DC;
        store_rows<FT, QT>(dst, DC, O, qt, 1.0f / lt, g);
        if (!whole && g == 0) {
          rec_m[lrow] = m[qt];
          rec_l[lrow] = lt;
        }
      }
    }
    flat = (int64_t)rt * s.KT + kt1;
  }
}

// Merge the pieces of every row tile that more than one workgroup worked on.
template <int DC, int DR, int QT>
__global__ __launch_bounds__(256) void k_attn_merge(bf16 *__restrict__ o,
                                                    const unsigned char *__restrict__ part, Sched s) {
  using C = Cfg<DC, DR, QT>;
  constexpr int RW = C::RW;
  constexpr int PER = (DC + 63) / 64;
  const int rt = blockIdx.x;
  const int g0 = wg_of(s, (int64_t)rt * s.KT), g1 = wg_of(s, (int64_t)rt * s.KT + s.KT - 1);
  if (g0 == g1) return;
  const int b = rt / s.RTb, row0 = (rt % s.RTb) * RW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int lrow = wave; lrow < RW; lrow += 4) {
    const int row = row0 + lrow;
    if (row >= s.R) break;
    float mmax = -INFINITY;
    for (int gg = g0; gg <= g1; ++gg) {
      const float *rm = (const float *)(part + (size_t)(gg + rt) * C::REC + (size_t)RW * DC * 2);
      mmax = fmaxf(mmax, rm[lrow]);
    }
    float wsum = 0.f;
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    for (int gg = g0; gg <= g1; ++gg) {
      const unsigned char *rec = part + (size_t)(gg + rt) * C::REC;
      const float *rm = (const float *)(rec + (size_t)RW * DC * 2);
      const float w = rm[RW + lrow] * fast_exp2(rm[lrow] - mmax);
      wsum += w;
      const bf16 *ro = (const bf16 *)rec + (int64_t)lrow * DC;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int f = lane + 64 * i;
        if (f < DC) acc[i] += w * (float)ro[f];
      }
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int f = lane + 64 * i;
      if (f < DC) o[((int64_t)b * s.R + row) * DC + f] = (bf16)(acc[i] * inv);
    }
  }
}

// Safe recomputation of the row tiles the fast kernel flagged: the whole window per
// workgroup, reference max raised lazily (by more than kSafeThreshold) with O
// rescaled, result written directly.  Workgroups of unflagged tiles exit at once.
template <int DC, int DR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_latent_attn_safe(const bf16 *__restrict__ q, const bf16 *__restrict__ cache,
                        bf16 *__restrict__ o, const int *__restrict__ flags, Sched s,
                        int fast_rw) {
  constexpr int QT = kSafeQT;
  using C = Cfg<DC, DR, QT>;
  constexpr int KB = C::KB, FT = C::FT, RW = C::RW;
  const int RTb = (s.R + RW - 1) / RW;
  const int b = blockIdx.x / RTb, row0 = (blockIdx.x % RTb) * RW;
  if (!flags[b * s.RTb + row0 / fast_rw]) return;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  Tile<DC, DR, QT> tl;
  tl.Ks = (bf16 *)lds;
  tl.Vt = tl.Ks + BN * C::KS;
  tl.nk = s.nk;
  tl.start0 = s.start0;
  tl.len0 = s.len0;
  tl.cb = cache + (int64_t)b * s.cache_rows * C::DK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  bf16x8 Qr[QT][KB];
  f32x16 O[FT][QT];
  bf16x8 P[BN / 16][QT];
  float m[QT], l[QT];
  load_queries<C::DK, QT, KB>(Qr, q, s, b, row0 + wave * QT * 32, l32, g);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -1e30f;
    l[qt] = 0.f;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[ft][qt][r] = 0.f;
  }
  tl.load(0, tid);
  for (int kt = 0; kt < s.KT; ++kt) {
    __syncthreads();
    tl.store(tid);
    __syncthreads();
    if (kt + 1 < s.KT) tl.load(kt + 1, tid);
    f32x16 S[2][QT];
    tl.scores(S, Qr, kt, l32, g);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mx = tile_max<QT>(S, qt);
      if (__any(mx > m[qt] + kSafeThreshold)) {
        const float mn = fmaxf(m[qt], mx);
        const float al = fast_exp2(m[qt] - mn);
        m[qt] = mn;
        l[qt] *= al;
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
#pragma unroll
          for (int r = 0; r < 16; ++r) O[ft][qt][r] *= al;
      }
      l[qt] += exp_and_pack<QT>(S, P, qt, m[qt]);
    }
    tl.values(O, P, l32, g);
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = l[qt] + __shfl_xor(l[qt], 32, 64);
    const int row = row0 + wave * QT * 32 + qt * 32 + l32;
    if (row < s.R) store_rows<FT, QT>(o + ((int64_t)b * s.R + row) * DC, DC, O, qt, 1.0f / lt, g);
  }
}

__global__ void k_fill_i32(int *p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Generic fp32 path: one wave per query row, keys one at a time.
__global__ __launch_bounds__(256) void k_latent_attn_f32(const float *__restrict__ q,
                                                         const float *__restrict__ cache,
                                                         float *__restrict__ o, Sched s, int DC,
                                                         int DR) {
  constexpr int MAXF = 8;  // features per lane: DC, DK <= 512
  const int DK = DC + DR;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)s.B * s.R) return;
  const int b = (int)(row / s.R);
  float qv[MAXF], acc[MAXF];
#pragma unroll
  for (int i = 0; i < MAXF; ++i) {
    const int f = lane + 64 * i;
    qv[i] = f < DK ? q[row * DK + f] : 0.f;
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float *cb = cache + (int64_t)b * s.cache_rows * DK;
  for (int kk = 0; kk < s.nk; ++kk) {
    const int64_t kr = kk < s.len0 ? (int64_t)(s.start0 + kk) : (int64_t)(kk - s.len0);
    const float *k = cb + kr * DK;
    float sp = 0.f;
#pragma unroll
    for (int i = 0; i < MAXF; ++i) {
      const int f = lane + 64 * i;
      if (f < DK) sp += qv[i] * k[f];
    }
    const float sc = wave_sum(sp);
    const float mn = fmaxf(m, sc);
    const float al = exp2f(m - mn), p = exp2f(sc - mn);
    l = l * al + p;
#pragma unroll
    for (int i = 0; i < MAXF; ++i) {
      const int f = lane + 64 * i;
      acc[i] = acc[i] * al + (f < DC ? p * k[f] : 0.f);
    }
    m = mn;
  }
#pragma unroll
  for (int i = 0; i < MAXF; ++i) {
    const int f = lane + 64 * i;
    if (f < DC) o[row * DC + f] = acc[i] / l;
  }
}

Sched make_sched(const AttnArgs &a, int rows_per_wg) {
  Sched s;
  s.B = a.B;
  s.R = a.R;
  s.RTb = (a.R + rows_per_wg - 1) / rows_per_wg;
  s.RT = s.B * s.RTb;
  s.nk = a.nk;
  s.KT = (a.nk + BN - 1) / BN;
  s.start0 = a.start0;
  s.len0 = a.len0;
  s.cache_rows = a.cache_rows;
  s.T = (int64_t)s.RT * s.KT;
  s.G = (int)((int64_t)a.grid < s.T ? (int64_t)a.grid : s.T);
  return s;
}

template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <int DC, int DR, int QT>
hipError_t launch(const AttnArgs &a, hipEvent_t ev0, hipEvent_t ev1, hipStream_t st) {
  using C = Cfg<DC, DR, QT>;
  using CS = Cfg<DC, DR, kSafeQT>;
  Sched s = make_sched(a, C::RW);
  if (s.T <= 0) return hipSuccess;
  hipError_t e = allow_lds(k_latent_attn<DC, DR, QT>, C::LDS);
  if (e == hipSuccess) e = allow_lds(k_latent_attn_safe<DC, DR>, CS::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_fill_i32, dim3((s.RT + 255) / 256), dim3(256), 0, st, a.flags, s.RT, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_latent_attn<DC, DR, QT>), dim3(s.G), dim3(256), C::LDS, st,
                     (const bf16 *)a.q, (const bf16 *)a.cache, (bf16 *)a.o,
                     (unsigned char *)a.part, a.flags, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_attn_merge<DC, DR, QT>), dim3(s.RT), dim3(256), 0, st, (bf16 *)a.o,
                     (const unsigned char *)a.part, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int safe_tiles = s.B * ((s.R + CS::RW - 1) / CS::RW);
  hipLaunchKernelGGL((k_latent_attn_safe<DC, DR>), dim3(safe_tiles), dim3(256), CS::LDS, st,
                     (const bf16 *)a.q, (const bf16 *)a.cache, (bf16 *)a.o,
                     (const int *)a.flags, s, C::RW);
  return hipGetLastError();
}

}  // namespace

bool latent_attention_bf16_supported(int dc, int dr) {
  return (dc == 192 && dr == 32) || (dc == 128 && dr == 32) || (dc == 256 && dr == 32) ||
         (dc == 192 && dr == 64);
}

int latent_attention_rows_per_wg(int dc, int dr) {
  (void)dr;
  return dc >= 256 ? Cfg<256, 32, 1>::RW : Cfg<192, 32, 2>::RW;
}

size_t latent_attention_record_bytes(int dc, int dr) {
  const size_t rw = (size_t)latent_attention_rows_per_wg(dc, dr);
  return rw * dc * 2 + rw * 8;
}

hipError_t latent_attention_bf16(const AttnArgs &a, hipEvent_t ev0, hipEvent_t ev1,
                                 hipStream_t st) {
  if (a.DC == 192 && a.DR == 32) return launch<192, 32, 2>(a, ev0, ev1, st);
  if (a.DC == 128 && a.DR == 32) return launch<128, 32, 2>(a, ev0, ev1, st);
  if (a.DC == 256 && a.DR == 32) return launch<256, 32, 1>(a, ev0, ev1, st);
  if (a.DC == 192 && a.DR == 64) return launch<192, 64, 2>(a, ev0, ev1, st);
  return hipErrorInvalidValue;
}

hipError_t latent_attention_f32(const AttnArgs &a, hipEvent_t ev0, hipEvent_t ev1,
                                hipStream_t st) {
  if (a.DC + a.DR > 512 || a.DC > 512) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)a.B * a.R;
  if (rows <= 0 || a.nk <= 0) return hipSuccess;
  Sched s = make_sched(a, 1);
  hipError_t e;
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_latent_attn_f32, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                     (const float *)a.q, (const float *)a.cache, (float *)a.o, s, a.DC, a.DR);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace mla
