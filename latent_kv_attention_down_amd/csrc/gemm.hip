// Projection GEMMs of the MLA chunk step: C = alpha * A * B^T with both operands
// K-contiguous (x W^T for row-major [out][in] weights).
//  * bf16, direct loads (K a multiple of 32, 16-byte aligned rows): BM x BN tiles,
//    waves of WTM x WTN built from 32x32x16 MFMAs (256x256 tiles of 128x64 waves for
//    large problems, 256x128 / 128x128 / 128x64 tiles of 64x64 or 64x32 waves else).  KC-wide k chunks of A and B go
//    through an NS-stage LDS ring filled by global_load_lds_dwordx4 (vector loads
//    into registers top out near 34 GB/s per CU, the direct path near 64-70 GB/s
//    per CU for L2-resident operands with the whole chip busy).  Optionally the
//    epilogue also produces per-row sums of squares of the result and scales its
//    columns (the RMSNorm of c^Q taken apart), or scales rows by the RMS those sums
//    give (see GemmArgs).  16-byte chunk c of stage row r sits at chunk
//    c ^ ((r >> 1) & (KC/8 - 1)), applied on the global side of each load, so the
//    32-row fragment reads are free of bank conflicts.  Rows past M or N read a
//    clamped valid row; their results are not stored.
//  * bf16, register-staged: 2x2 waves, each a (BM/2)x(BN/2) block of MFMA tiles,
//    two padded LDS stages (the fallback for other shapes).
//  * fp32: plain 16x16 SIMT tiles (the small fp32 path).
#include <type_traits>

#include "mla_device.h"
#include "mla_launch.h"

namespace mla {
namespace {

template <int BM, int BN, int BK, bool OUT_F32>
__global__ __launch_bounds__(256) void k_gemm_bf16_nt(GemmArgs g) {
  constexpr int TM = BM / 64, TN = BN / 64;  // 32x32 tiles per wave
  constexpr int LS = BK + 8;                 // LDS row stride (pads rows by 16 B)
  constexpr int CPR = BK / 8;                // 16-byte chunks per tile row
  constexpr int A_CH = BM * CPR / 256;       // chunks per thread
  constexpr int B_CH = BN * CPR / 256;
  constexpr int STAGE = (BM + BN) * LS;
  static_assert(A_CH * 256 == BM * CPR && B_CH * 256 == BN * CPR, "tile/threads mismatch");
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN, b = blockIdx.z;
  const bf16 *A = (const bf16 *)g.A + b * g.sA;
  const bf16 *B = (const bf16 *)g.B + b * g.sB;

  uint4 ra[A_CH], rb[B_CH];
  auto load = [&](int k0) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int id = tid + c * 256, r = id / CPR, kc = (id % CPR) * 8, gm = m0 + r;
      ra[c] = gm < g.M ? *(const uint4 *)(A + (int64_t)gm * g.lda + k0 + kc) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < B_CH; ++c) {
      const int id = tid + c * 256, r = id / CPR, kc = (id % CPR) * 8, gn = n0 + r;
      rb[c] = gn < g.N ? *(const uint4 *)(B + (int64_t)gn * g.ldb + k0 + kc) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int st) {
    bf16 *sA = smem + st * STAGE, *sB = sA + BM * LS;
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int id = tid + c * 256;
      *(uint4 *)(sA + (id / CPR) * LS + (id % CPR) * 8) = ra[c];
    }
#pragma unroll
    for (int c = 0; c < B_CH; ++c) {
      const int id = tid + c * 256;
      *(uint4 *)(sB + (id / CPR) * LS + (id % CPR) * 8) = rb[c];
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int l32 = lane & 31, kg = (lane >> 5) * 8;
  const int nk = g.K / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK);
    const bf16 *sA = smem + st * STAGE, *sB = sA + BM * LS;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const bf16x8 *)(sA + (wm * (BM / 2) + i * 32 + l32) * LS + ks + kg);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *(const bf16x8 *)(sB + (wn * (BN / 2) + j * 32 + l32) * LS + ks + kg);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) store(st ^ 1);
    __syncthreads();
  }

  // lane holds column l32 of each 32x32 tile, rows 8*(r/4) + 4*(lane/32) + r%4
  const int g4 = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * (BN / 2) + j * 32 + l32;
      if (col >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * (BM / 2) + i * 32 + (r >> 2) * 8 + g4 + (r & 3);
        if (row >= g.M) continue;
        const float v = acc[i][j][r] * g.alpha;
        if (OUT_F32)
          ((float *)g.C)[b * g.sC + (int64_t)row * g.ldc + col] = v;
        else
          ((bf16 *)g.C)[b * g.sC + (int64_t)row * g.ldc + col] = (bf16)v;
      }
    }
}

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

template <int BM, int BN, int WTM, int WTN, int KC, int NS, bool OUT_F32, int EP>
__global__ __launch_bounds__((BM / WTM) * (BN / WTN) * 64)
__attribute__((amdgpu_waves_per_eu(WTM * WTN >= 128 * 64 ? 2 : 4, 8)))
void k_gemm_dma(GemmArgs g) {
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
    const int nbx = gridDim.x, total = nbx * gridDim.y, lin = blockIdx.y * nbx + blockIdx.x;
    const int xcd = lin % 8, slot = lin / 8, q = total / 8, rem = total % 8;
    const int t = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + slot;
    m_t = t / nbx;
    n_t = t % nbx;
  }
  const int m0 = m_t * BM, n0 = n_t * BN, b = blockIdx.z;
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
    __syncthreads();
  };
  bf16x8 af[2][TM], bfr[2][TN];
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
  // Fragments run one k-step ahead.  At a chunk's last k-step the next stage is
  // awaited first: once every wave has passed that barrier it has read all of the
  // current stage into registers, so the stage can be refilled (chunk kc + NS).
  arrive(0);
  if (NS - 1 < nk) issue(NS - 1);
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

template <int BM, int BN, int WTM, int WTN, int KC, int NS, bool OUT_F32, int EP = EP_PLAIN>
hipError_t launch_dma(const GemmArgs &g, hipStream_t st) {
  using D = GemmDma<BM, BN, WTM, WTN, KC, NS, OUT_F32, EP>;
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, g.batch);
  const auto kern = k_gemm_dma<BM, BN, WTM, WTN, KC, NS, OUT_F32, EP>;
  if (D::LDS > 65536) {
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)D::LDS);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, dim3(D::NT), D::LDS, st, g);
  return hipGetLastError();
}

template <int BM, int BN, int WTM, int WTN, int KC, int NS>
hipError_t launch_dma(const GemmArgs &g, bool out_f32, hipStream_t st) {
  if (g.ssq_out) return launch_dma<BM, BN, WTM, WTN, KC, NS, false, EP_SSQ_OUT>(g, st);
  if (g.ssq_in) return launch_dma<BM, BN, WTM, WTN, KC, NS, false, EP_ROW_RMS>(g, st);
  return out_f32 ? launch_dma<BM, BN, WTM, WTN, KC, NS, true>(g, st)
                 : launch_dma<BM, BN, WTM, WTN, KC, NS, false>(g, st);
}

template <int KC>
hipError_t gemm_dma(const GemmArgs &g, bool out_f32, hipStream_t st) {
  const int64_t mt128 = (g.M + 127) / 128;
  // 256x256 tiles of eight 128x64 waves, two per SIMD, read 0.75 KB of LDS per MFMA
  // instead of 1 KB and fetch 128 FLOP per byte instead of 85; bf16 output only (an
  // fp32 output tile of that size does not fit the LDS).  Two 64-wide k stages
  // measured faster than four 32-wide ones.  Taken when there are enough of them to
  // cover most of the 256 CUs: the 21-frame clip and batched requests, and at the
  // 3-frame chunk the 2688-wide query GEMM (209 tiles in one round, against 399 of
  // 256x128 in two); the chunk's output projection (114 tiles) stays at 256x128.
  const int64_t tiles256 = ((g.M + 255) / 256) * ((g.N + 255) / 256) * g.batch;
  if (!out_f32 && !g.ssq_out && g.N >= 512 && tiles256 >= 200) {
    if (g.ssq_in) return launch_dma<256, 256, 128, 64, 64, 2, false, EP_ROW_RMS>(g, st);
    return launch_dma<256, 256, 128, 64, 64, 2, false>(g, st);
  }
  if (g.N >= 1024) return launch_dma<256, 128, 64, 64, KC, 3>(g, out_f32, st);
  // 128x128 tiles with two 64-wide stages (64 KB of LDS, 68 KB with an fp32 output
  // tile) leave room for a second workgroup on the CU: the per-head W^V_up GEMM
  // (K = 192, three k chunks, 444 tiles) then runs in one round, 9.4 us against
  // 13.4 us with four stages, and W^Q_down is no slower (20.8 against 21.6 us).
  if (g.N % 128 == 0 && mt128 * (g.N / 128) * g.batch >= 200)
    return launch_dma<128, 128, 64, 64, KC, KC == 64 ? 2 : 4>(g, out_f32, st);
  return launch_dma<128, 64, 64, 32, KC, 4>(g, out_f32, st);
}

__global__ __launch_bounds__(256) void k_gemm_f32_nt(GemmArgs g) {
  __shared__ float sA[16][17], sB[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row = blockIdx.y * 16 + ty, col = blockIdx.x * 16 + tx, b = blockIdx.z;
  const float *A = (const float *)g.A + b * g.sA;
  const float *B = (const float *)g.B + b * g.sB;
  float acc = 0.f;
  for (int k0 = 0; k0 < g.K; k0 += 16) {
    int ar = blockIdx.y * 16 + ty, br = blockIdx.x * 16 + ty;
    sA[ty][tx] = (ar < g.M && k0 + tx < g.K) ? A[(int64_t)ar * g.lda + k0 + tx] : 0.f;
    sB[ty][tx] = (br < g.N && k0 + tx < g.K) ? B[(int64_t)br * g.ldb + k0 + tx] : 0.f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) acc += sA[ty][k] * sB[tx][k];
    __syncthreads();
  }
  if (row < g.M && col < g.N) ((float *)g.C)[b * g.sC + (int64_t)row * g.ldc + col] = acc * g.alpha;
}

template <int BM, int BN, int BK>
hipError_t launch_bf16(const GemmArgs &g, bool out_f32, hipStream_t st) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, g.batch);
  if (out_f32)
    hipLaunchKernelGGL((k_gemm_bf16_nt<BM, BN, BK, true>), grid, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((k_gemm_bf16_nt<BM, BN, BK, false>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_bf16_nt(const GemmArgs &g, bool out_f32, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  const bool extra = g.ssq_out || g.ssq_in || g.col_scale;
  if (extra && (out_f32 || g.batch != 1 || (g.ssq_out && g.ssq_in))) return hipErrorInvalidValue;
  // direct loads need 16-byte aligned rows; the 16-byte tile stores need the same
  // of C and whole 16-byte pieces of every row (N a multiple of 8 bf16 / 4 fp32)
  const int vec = out_f32 ? 4 : 8;
  const bool aligned = ((uintptr_t)g.A % 16 == 0) && ((uintptr_t)g.B % 16 == 0) &&
                       ((uintptr_t)g.C % 16 == 0) && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
                       g.sA % 8 == 0 && g.sB % 8 == 0 && g.ldc % vec == 0 && g.sC % vec == 0 &&
                       g.N % vec == 0;
  if (aligned && g.K > 0 && g.K % 64 == 0) return gemm_dma<64>(g, out_f32, st);
  if (aligned && g.K > 0 && g.K % 32 == 0) return gemm_dma<32>(g, out_f32, st);
  if (extra) return hipErrorInvalidValue;  // the epilogue work needs the direct-load path
  // 128x128 tiles when N fills them and there are enough tiles for the chip
  // (two workgroups fit per CU); otherwise 64x64.
  const int64_t tiles128 = (int64_t)((g.M + 127) / 128) * ((g.N + 127) / 128) * g.batch;
  const bool big = (g.N % 128 == 0) && tiles128 >= 200;
  if (g.K % 64 == 0)
    return big ? launch_bf16<128, 128, 64>(g, out_f32, st) : launch_bf16<64, 64, 64>(g, out_f32, st);
  return big ? launch_bf16<128, 128, 32>(g, out_f32, st) : launch_bf16<64, 64, 32>(g, out_f32, st);
}

hipError_t gemm_f32_nt(const GemmArgs &g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  dim3 grid((g.N + 15) / 16, (g.M + 15) / 16, g.batch);
  hipLaunchKernelGGL(k_gemm_f32_nt, grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace mla
