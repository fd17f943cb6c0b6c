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
#include "gemm_tile.h"

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

template <int BM, int BN, int WTM, int WTN, int KC, int NS, bool OUT_F32, int EP>
// Up to 256 registers per wave: the fragments of four k-steps are in flight at once.
__global__ __launch_bounds__((BM / WTM) * (BN / WTN) * 64)
__attribute__((amdgpu_waves_per_eu(2, 8)))
void k_gemm_dma(GemmArgs g) {
  gemm_dma_tile<BM, BN, WTM, WTN, KC, NS, OUT_F32, EP>(g, blockIdx.y * gridDim.x + blockIdx.x,
                                                       gridDim.x, gridDim.x * gridDim.y, blockIdx.z);
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
  // 13.4 us with four stages.  Where the tiles fit on the CUs in one round anyway
  // (W^Q_down of the 3-frame chunk: 222 tiles) a third stage keeps two in flight and
  // eight 64x32 waves replace four 64x64 ones: 17.6 against 21.0 us.
  const int64_t t128 = mt128 * (g.N / 128) * g.batch;
  if (g.N % 128 == 0 && t128 >= 200) {
    if (KC == 64 && t128 <= 256) return launch_dma<128, 128, 64, 32, KC, 3>(g, out_f32, st);
    return launch_dma<128, 128, 64, 64, KC, KC == 64 ? 2 : 4>(g, out_f32, st);
  }
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

// The absorbed query GEMM alone (256x256 tiles, rows scaled by their RMS) with the
// query's RoPE columns rotated in its tiles, exactly as the separate RoPE pass rotates
// them; the first tile also clears the attention's overflow flags, the other duty of
// that pass.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 8)))
void k_query_gemm_rope(GemmArgs g, RopeQArgs r) {
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  if (lin == 0)
    for (int i = threadIdx.x; i < r.n_zero; i += blockDim.x) r.zero[i] = 0;
  gemm_dma_tile<256, 256, 128, 64, 64, 2, false, EP_ROW_RMS, true>(g, lin, gridDim.x,
                                                                   gridDim.x * gridDim.y, 0, &r);
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

bool query_gemm_rope_applies(const GemmArgs &g, const RopeQArgs &r) {
  const int64_t tiles = (int64_t)((g.M + 255) / 256) * ((g.N + 255) / 256);
  const int dk = r.d_c + r.d_rope;
  return g.batch == 1 && g.ssq_in && !g.ssq_out && g.N >= 512 && g.K > 0 && g.K % 64 == 0 &&
         tiles >= 200 && r.in_place && r.d_c % 8 == 0 && dk % 8 == 0 && dk >= 64 &&
         (int64_t)r.n_h * dk == g.N && r.M == g.M && (uintptr_t)g.A % 16 == 0 &&
         (uintptr_t)g.B % 16 == 0 && (uintptr_t)g.C % 16 == 0 && g.lda % 8 == 0 &&
         g.ldb % 8 == 0 && g.ldc % 8 == 0;
}

hipError_t query_gemm_rope(const GemmArgs &g, const RopeQArgs &r, hipStream_t st) {
  if (!query_gemm_rope_applies(g, r)) return hipErrorInvalidValue;
  using D = GemmDma<256, 256, 128, 64, 64, 2, false, EP_ROW_RMS>;
  constexpr size_t lds = D::LDS + RopeLds<256>::BYTES;  // the tile, then its rotation table
  static_assert(lds <= 163840, "LDS");
  hipError_t e = hipFuncSetAttribute((const void *)k_query_gemm_rope,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_query_gemm_rope, dim3((g.N + 255) / 256, (g.M + 255) / 256), dim3(D::NT),
                     lds, st, g, r);
  return hipGetLastError();
}

}  // namespace mla
