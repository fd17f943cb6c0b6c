// The direct-load GEMM tile of the chunk step's projections (the configuration,
// chunk swizzle and one workgroup's output tile), in a header so that a launch can
// run these tiles beside other work (the cache write rides beside the query GEMM).
// The design is described at the top of gemm.hip.
#pragma once
#include <type_traits>

#include "mla_device.h"
#include "mla_launch.h"

namespace mla {

// Epilogue modes of k_gemm_dma (GemmArgs): plain, producer of row sums of squares
// with a column scale, consumer scaling rows by them.
enum { EP_PLAIN = 0, EP_SSQ_OUT = 1, EP_ROW_RMS = 2 };

template <int BM, int BN, int WTM, int WTN, int KC, int NS, bool OUT_F32, int EP = EP_PLAIN>
struct GemmDma {
  static constexpr int NW = (BM / WTM) * (BN / WTN), NT = NW * 64;
  static constexpr int ROWB = KC * 2;                  // bytes per stage row
  static constexpr int RPL = 1024 / ROWB;              // rows per 1 KB load
  static constexpr int A_LOADS = BM / RPL, B_LOADS = BN / RPL;
  static constexpr int LPW = (A_LOADS + B_LOADS) / NW;  // loads per wave per stage
  static constexpr int SB = (BM + BN) * ROWB;          // stage bytes
  // the epilogue reuses the stages as a BM x (BN + one 16-byte piece) output tile,
  // fp32 when the producer epilogue sums squares; past both, the producer keeps the
  // tile's BN column scales and the consumer its BM row scales for the whole kernel
  static constexpr int OUT_B = (OUT_F32 || EP == EP_SSQ_OUT) ? 4 : 2;
  static constexpr size_t EPI = (size_t)BM * (BN + 16 / OUT_B) * OUT_B;
  static constexpr size_t XOFF = (size_t)SB * NS > EPI ? (size_t)SB * NS : EPI;
  static constexpr size_t LDS =
      XOFF + (EP == EP_SSQ_OUT ? (size_t)BN * 4 : EP == EP_ROW_RMS ? (size_t)BM * 4 : 0);
  static_assert(!(OUT_F32 && EP != EP_PLAIN), "row-sum epilogues write bf16");
  static_assert(LDS <= 163840, "LDS");
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(LPW * NW == A_LOADS + B_LOADS, "loads do not split over the waves");
  static_assert(NS >= 2 && NS <= 4, "stage count");
};

template <int KC>
__device__ __forceinline__ int gswz(int row) { return (row >> 1) & (KC / 8 - 1); }

// LDS a rotating tile keeps past its own: the cos and sin of every rope pair at each
// position its axis takes in the chunk (frame within the chunk, row and column of the
// token grid; pair p's run starts at entry p * S, S the longest of the three spans),
// the axis of each pair, and each tile row's three axis positions.  A tile whose
// pairs would need more entries rotates without it.
template <int BM>
struct RopeLds {
  static constexpr int ENTRIES = 2048, MAX_PAIRS = 64;
  static constexpr size_t AX = (size_t)ENTRIES * 8, ROWS = AX + MAX_PAIRS * 4;
  static constexpr size_t BYTES = (ROWS + (size_t)BM * 3 * 4 + 15) / 16 * 16;
};

// Fills the table at `base` for the tile rows m0 .. m0 + BM - 1 (rows past M take
// row M - 1's positions) and returns S, or 0 (nothing written) when it does not fit.
// Each entry is what rope_sincos gives for that pair and position, as in the separate
// RoPE pass.  A wave takes whole pairs, so that a pair's axis and frequency are
// wave-uniform scalar reads of the kernel arguments.
template <int BM, int NT>
__device__ __forceinline__ int rope_lds_build(const RopeQArgs &r, unsigned char *base, int m0,
                                              int M) {
  using T = RopeLds<BM>;
  const int np = r.d_rope / 2;
  const int n_t = (r.T_q + r.tpf - 1) / r.tpf, n_y = (r.tpf + r.grid_w - 1) / r.grid_w,
            n_x = r.grid_w;
  const int S = max(n_t, max(n_y, n_x));
  if (np > T::MAX_PAIRS || np * S > T::ENTRIES) return 0;
  float2 *ct = (float2 *)base;
  int *ax = (int *)(base + T::AX), *rp = (int *)(base + T::ROWS);
  const int tid = threadIdx.x, lane = tid & 63;
  for (int p = __builtin_amdgcn_readfirstlane(tid >> 6); p < np; p += NT / 64) {
    const int a = r.rope.axis[p], n = a == 0 ? n_t : a == 1 ? n_y : n_x;
    const double om = r.rope.omega[p];
    for (int idx = lane; idx < n; idx += 64) {
      const double pos = a == 0 ? (double)(r.t0 + idx) : (double)idx;
      float s, c;
      rope_sincos(pos, om, s, c);
      ct[p * S + idx] = make_float2(c, s);
    }
    if (lane == 0) ax[p] = a;
  }
  for (int rr = tid; rr < BM; rr += NT) {
    const int m = min(m0 + rr, M - 1), i = m % r.T_q, nn = i % r.tpf;
    rp[3 * rr] = i / r.tpf;
    rp[3 * rr + 1] = nn / r.grid_w;
    rp[3 * rr + 2] = nn % r.grid_w;
  }
  return S;
}

// One output tile; lin is the workgroup's linear index among the total tiles of the
// launch (nbx tiles across N), b its batch.  With ROPE (the absorbed query GEMM, bf16
// output), the tile's columns that are a head's rope columns of q_lat (column n is
// column n mod (d_c + d_rope) of head n / (d_c + d_rope)) are rotated by 3D-RoPE at
// their row's token position while the tile sits in LDS, exactly as the separate
// RoPE pass would rotate them in q_lat (rope_q_item), before the tile is stored.
template <int BM, int BN, int WTM, int WTN, int KC, int NS, bool OUT_F32, int EP, bool ROPE = false>
__device__ __forceinline__ void gemm_dma_tile(const GemmArgs &g, int lin, int nbx, int total, int b,
                                              const RopeQArgs *rq = nullptr) {
  using D = GemmDma<BM, BN, WTM, WTN, KC, NS, OUT_F32, EP>;
  constexpr int TM = D::TM, TN = D::TN, LPW = D::LPW, RPL = D::RPL, CPR = KC / 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  typedef __attribute__((address_space(3))) void lds_void;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (BN / WTN), wn = wave % (BN / WTN);
  // Workgroups go to the 8 XCDs round-robin by linear id.  Tiles are renumbered
  // so that each XCD gets a contiguous run of the row-major tile order: the column
  // tiles that share an A row block then run on one XCD and reuse its L2.
  int m_t, n_t;
  {
    const int xcd = lin % 8, slot = lin / 8, q = total / 8, rem = total % 8;
    const int t = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + slot;
    m_t = t / nbx;
    n_t = t % nbx;
  }
  const int m0 = m_t * BM, n0 = n_t * BN;
  const bf16 *A = (const bf16 *)g.A + b * g.sA;
  const bf16 *B = (const bf16 *)g.B + b * g.sB;

  // this lane's source rows: load L = wave*LPW + i covers stage rows L*RPL.. of A
  // (then of B), lane -> row lane / CPR, 16-byte slot lane % CPR
  const bf16 *src[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int L = wave * LPW + i;
    const bool isA = L < D::A_LOADS;
    const int row = (isA ? L : L - D::A_LOADS) * RPL + lane / CPR;   // row within the tile
    const int ch = (lane % CPR) ^ gswz<KC>(row);
    if (isA)
      src[i] = A + (int64_t)min(m0 + row, g.M - 1) * g.lda + ch * 8;
    else
      src[i] = B + (int64_t)min(n0 + row, g.N - 1) * g.ldb + ch * 8;
  }
  auto issue = [&](int kc) {
    unsigned char *st = smem + (size_t)(kc % NS) * D::SB;
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      __builtin_amdgcn_global_load_lds((const void *)(src[i] + kc * KC),
                                       (lds_void *)(st + (wave * LPW + i) * 1024), 16, 0, 0);
  };
  const int nk = g.K / KC;
#pragma unroll
  for (int kc = 0; kc < NS - 1; ++kc)
    if (kc < nk) issue(kc);
  // Epilogue operands, fetched while the first stages are in flight (their wait
  // coincides with that of stage 0, which the loop needs anyway) and kept in LDS past
  // the stages: the tile's column scales (producer), or 1 / RMS of each of its rows
  // from the producer's pieces, summed in a fixed order (consumer).
  float *xs = (float *)(smem + D::XOFF);
  if (EP == EP_SSQ_OUT)
    for (int c = tid; c < BN; c += D::NT)
      xs[c] = (g.col_scale && n0 + c < g.N) ? to_f32(((const bf16 *)g.col_scale)[n0 + c]) : 1.0f;
  if (EP == EP_ROW_RMS)
    for (int r = tid; r < BM; r += D::NT) {
      const int64_t row = min(m0 + r, g.M - 1);
      float ss = 0.f;
#pragma unroll 4
      for (int p = 0; p < g.ssq_parts; ++p) ss += g.ssq_in[(int64_t)p * g.M + row];
      xs[r] = 1.0f / sqrtf(ss * g.ssq_scale + g.ssq_eps);
    }
  // A rotating tile's cos and sin table, built in the same shadow (LDS past D::LDS).
  int tab = 0;
  if constexpr (ROPE) tab = rope_lds_build<BM, D::NT>(*rq, smem + D::LDS, m0, g.M);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int l32 = lane & 31, g8 = lane >> 5;
  constexpr int KS = KC / 16;  // k-steps per chunk
  // wait until stage kc has landed (every later stage may still be in flight),
  // then make it visible to the workgroup.  This wave's own LDS reads are drained
  // first: after the barrier another wave may refill the stage they read.
  auto arrive = [&](int kc) {
    const int after = min(NS - 2, nk - 1 - kc);
    if (after >= 2)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * LPW) : "memory");
    else if (after == 1)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(LPW) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    // a bare barrier: __syncthreads would also wait for the later stages' loads
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  constexpr int NB = KS >= 3 ? KS : 2;  // fragment buffers
  bf16x8 af[NB][TM], bfr[NB][TN];
  auto frags = [&](int kc, int s, int p) {
    const unsigned char *sa = smem + (size_t)(kc % NS) * D::SB;
    const unsigned char *sb = sa + BM * D::ROWB;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * WTM + i * 32 + l32;
      af[p][i] = *(const bf16x8 *)(sa + row * D::ROWB + ((2 * s + g8) ^ gswz<KC>(row)) * 16);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wn * WTN + j * 32 + l32;
      bfr[p][j] = *(const bf16x8 *)(sb + row * D::ROWB + ((2 * s + g8) ^ gswz<KC>(row)) * 16);
    }
  };
  arrive(0);
  if (NS - 1 < nk) issue(NS - 1);
  if constexpr (KS >= 3) {
    // Fragments two k-steps ahead (buffer s for k-step s), each read slotted between
    // two MFMAs of the step.  Two steps before a chunk ends the next stage is awaited:
    // by then every wave holds the current stage's last fragments (or has them in
    // flight, drained by the wait), so the stage can be refilled.  The last chunk is
    // peeled so that no branch splits the steps.
    auto step = [&](int s) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[s][i], bfr[s][j], acc[i][j]);
#pragma unroll
      for (int q = 0; q < TM * TN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (q < TM + TN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };
    frags(0, 0, 0);
    frags(0, 1, 1);
    for (int kc = 0; kc + 1 < nk; ++kc) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 2 < KS) {
          frags(kc, s + 2, s + 2);
        } else {
          if (s + 2 == KS) {
            arrive(kc + 1);
            if (kc + NS < nk) issue(kc + NS);
          }
          frags(kc + 1, s + 2 - KS, s + 2 - KS);
        }
        step(s);
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 2 < KS) frags(nk - 1, s + 2, s + 2);
      step(s);
    }
  } else {
    frags(0, 0, 0);
    for (int kc = 0; kc < nk; ++kc) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int p = (kc * KS + s) & 1;
        if (s + 1 < KS) {
          frags(kc, s + 1, p ^ 1);
        } else if (kc + 1 < nk) {
          arrive(kc + 1);
          if (kc + NS < nk) issue(kc + NS);
          frags(kc + 1, 0, p ^ 1);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[p][i], bfr[p][j], acc[i][j]);
      }
    }
  }

  // Results through LDS for 16-byte stores.  acc[i][j][4q + r] is row
  // 8q + 4*(lane/32) + r, column l32 of the 32x32 tile.
  typedef typename std::conditional<OUT_F32, float, bf16>::type OutT;
  typedef typename std::conditional<OUT_F32 || EP == EP_SSQ_OUT, float, bf16>::type TileT;
  constexpr int VEC = 16 / sizeof(TileT), LDC = BN + VEC;  // padded row of the tile
  TileT *tile = (TileT *)smem;
  __syncthreads();  // stages no longer read
  const float *rs = xs;  // row scales (consumer), written before the k loop
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    // the lane's 16 rows of this 32-row tile come in four runs of four consecutive
    // rows: their scales are four 16-byte reads
    f32x4 rsv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      rsv[q] = EP == EP_ROW_RMS ? *(const f32x4 *)(rs + wm * WTM + i * 32 + q * 8 + g8 * 4)
                                : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * WTM + i * 32 + (r >> 2) * 8 + g8 * 4 + (r & 3);
        float v = acc[i][j][r] * g.alpha;
        if (EP == EP_ROW_RMS) v *= rsv[r >> 2][r & 3];
        tile[row * LDC + wn * WTN + j * 32 + l32] = (TileT)v;
      }
  }
  __syncthreads();
  if constexpr (ROPE) {
    static_assert(!OUT_F32 && EP != EP_SSQ_OUT, "the rotation works on a bf16 tile");
    // The tile's rope columns: runs of 8-column chunks, one per head whose rope
    // columns meet the tile (at most BN / dk + 2 of them; the launcher keeps dk >= 64).
    constexpr int MAXRUN = BN / 64 + 2;
    const int dk = rq->d_c + rq->d_rope, n_end = min(n0 + BN, g.N);
    int run_a[MAXRUN], run_n[MAXRUN], nc = 0;
#pragma unroll
    for (int s = 0; s < MAXRUN; ++s) {
      const int h = n0 / dk + s - 1;
      const int a = max(h * dk + rq->d_c, n0), e = min(h * dk + dk, n_end);
      run_a[s] = (a - n0) / 8;
      run_n[s] = h >= 0 && e > a ? (e - a) / 8 : 0;
      nc += run_n[s];
    }
    for (int id = tid; id < BM * nc; id += D::NT) {
      const int r = id / nc, m = m0 + r;
      int k = id - r * nc, c8 = -1;
#pragma unroll
      for (int s = 0; s < MAXRUN; ++s) {
        if (c8 < 0 && k < run_n[s]) c8 = (run_a[s] + k) * 8;
        else if (c8 < 0) k -= run_n[s];
      }
      if (m >= g.M) continue;
      const int p0 = ((n0 + c8) % dk - rq->d_c) / 2;  // four pairs from here
      bf16x8 *t = (bf16x8 *)((bf16 *)tile + r * LDC + c8);
      bf16x8 v = *t;
      if (tab) {
        using T = RopeLds<BM>;
        const float2 *ct = (const float2 *)(smem + D::LDS);
        const int *ax = (const int *)(smem + D::LDS + T::AX);
        const int *rp = (const int *)(smem + D::LDS + T::ROWS) + 3 * r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float re = to_f32(v[2 * q]), im = to_f32(v[2 * q + 1]);
          const float2 cs = ct[(p0 + q) * tab + rp[ax[p0 + q]]];
          rotate_by(re, im, cs.y, cs.x);
          v[2 * q] = (bf16)re;
          v[2 * q + 1] = (bf16)im;
        }
      } else {
        const int i = m % rq->T_q, nn = i % rq->tpf;
        const double pos[3] = {(double)(rq->t0 + i / rq->tpf), (double)(nn / rq->grid_w),
                               (double)(nn % rq->grid_w)};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float re = to_f32(v[2 * q]), im = to_f32(v[2 * q + 1]);
          rope_rotate(re, im, pos[rq->rope.axis[p0 + q]], rq->rope.omega[p0 + q]);
          v[2 * q] = (bf16)re;
          v[2 * q + 1] = (bf16)im;
        }
      }
      *t = v;
    }
    __syncthreads();
  }
  OutT *C = (OutT *)g.C + b * g.sC;
  if (EP == EP_SSQ_OUT) {
    // sums of squares of each row over 64-column pieces, one thread per (row, piece),
    // in a fixed order (the starting column rotates with the row to spread the banks)
    for (int id = tid; id < BM * (BN / 64); id += D::NT) {
      const int r = id % BM, col0 = (id / BM) * 64;
      if (m0 + r < g.M && n0 + col0 < g.N) {
        // 16 independent 16-byte reads, summed as a fixed tree; columns past N hold
        // the results of a clamped row of B and are left out
        float part[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const f32x4 v = *(const f32x4 *)(tile + r * LDC + col0 + 4 * q);
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) t += (n0 + col0 + 4 * q + e < g.N) ? v[e] * v[e] : 0.f;
          part[q] = t;
        }
#pragma unroll
        for (int w = 8; w > 0; w >>= 1)
#pragma unroll
          for (int q = 0; q < w; ++q) part[q] += part[q + w];
        g.ssq_out[(int64_t)((n0 + col0) / 64) * g.M + m0 + r] = part[0];
      }
    }
    // bf16 output, each column scaled
    for (int id = tid; id < BM * (BN / 8); id += D::NT) {
      const int r = id / (BN / 8), c = (id % (BN / 8)) * 8;
      if (m0 + r < g.M && n0 + c < g.N) {
        const f32x4 a = *(const f32x4 *)(tile + r * LDC + c), b4 = *(const f32x4 *)(tile + r * LDC + c + 4);
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = (bf16)(a[e] * xs[c + e]);
          o[4 + e] = (bf16)(b4[e] * xs[c + 4 + e]);
        }
        *(bf16x8 *)((bf16 *)C + (int64_t)(m0 + r) * g.ldc + n0 + c) = o;
      }
    }
    return;
  }
  for (int id = tid; id < BM * (BN / VEC); id += D::NT) {
    const int r = id / (BN / VEC), c = (id % (BN / VEC)) * VEC;
    if (m0 + r < g.M && n0 + c < g.N)
      *(uint4 *)(C + (int64_t)(m0 + r) * g.ldc + n0 + c) = *(const uint4 *)(tile + r * LDC + c);
  }
}

}  // namespace mla
