// Internal host-side launchers of the gfx950 kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_types.h"

namespace mla {

// C[b] = alpha * A[b] (M x K, row stride lda) * B[b]^T (B is N x K, row stride ldb);
// batch b offsets each operand by its batch stride (elements).
struct GemmArgs {
  const void *A;
  int64_t lda, sA;
  const void *B;
  int64_t ldb, sB;
  void *C;
  int64_t ldc, sC;
  int M, N, K, batch;
  float alpha;
  // Optional epilogue work (bf16 output, direct-load path, batch 1; null / 0 = none):
  //  producer: ssq_out[(n / 64) * M + m] = sum over the 64-column piece of
  //    (alpha * acc)^2, and the stored value is alpha * acc * col_scale[n] (bf16
  //    vector, or ones when col_scale is null);
  //  consumer: row m is multiplied by 1 / sqrt(ssq_scale * sum_{p < ssq_parts}
  //    ssq_in[p * M + m] + ssq_eps) before rounding.
  const void *col_scale = nullptr;
  float *ssq_out = nullptr;
  const float *ssq_in = nullptr;
  int ssq_parts = 0;
  float ssq_scale = 0.f, ssq_eps = 0.f;
};
hipError_t gemm_bf16_nt(const GemmArgs &g, bool out_f32, hipStream_t st);
hipError_t gemm_f32_nt(const GemmArgs &g, hipStream_t st);

// The ring of one layer in two parts: element i of row r of request b is at
// c_kv + b * c_batch + r * c_row + i (i < d_c) and k_r + b * r_batch + r * r_row + i
// (i < d_rope), in elements.  The interleaved layout has k_r = c_kv + d_c and both
// row strides d_c + d_rope.
struct RingParts {
  void *c_kv, *k_r;
  int64_t c_row, r_row, c_batch, r_batch;
};

// Fused cache write: [W_kv_down; W_kr] x -> RMSNorm(latent) * g, RoPE(k^R) -> ring rows.
struct CacheWriteArgs {
  const void *x, *w_kv, *w_kr, *g_kv;
  RingParts ring;
  int M;          // B * tokens in the chunk
  int T_q;        // tokens in the chunk per request
  int d, d_c, d_rope, tpf, grid_w, W;
  int S;                     // sink frames: frame f < S in slot f, else S + (f - S) mod W
  int rotate;                // 1: rotate k^R at the absolute position; 0: store it as is
  int64_t t0;
  float eps;
  RopeTable rope;
};
hipError_t cache_write_bf16(const CacheWriteArgs &a, hipStream_t st);
hipError_t cache_write_f32(const CacheWriteArgs &a, hipStream_t st);

// out[r] = in[r] / sqrt(mean(in[r]^2) + eps) * g  (in fp32, out bf16 or fp32).
hipError_t rmsnorm_rows(const float *in, const void *g, void *out, int rows, int cols, float eps,
                        bool out_bf16, hipStream_t st);

// q_lat[(m*n_h + h), d_c + i] = scale * RoPE(q_r[m, h*d_rope + i]) at token m's position.
struct RopeQArgs {
  const float *q_r;
  void *q_lat;
  int M, T_q, n_h, d_rope, d_c, tpf, grid_w;
  int64_t t0;
  float scale;
  RopeTable rope;
  int *zero;   // n_zero ints set to 0 on the way (the attention's overflow flags), or null
  int n_zero;
  bool in_place;  // q_r is null: rotate the (already scaled) RoPE columns of q_lat in place
};
hipError_t rope_q(const RopeQArgs &a, bool bf16_out, hipStream_t st);
// The bf16 cache write with the in-place query RoPE of the same step in one launch:
// rope_blocks workgroups beside the cache write's own (bf16, in-place, pair count a
// multiple of 4, a shape the direct-load cache write covers: cache_write_takes_rope).
bool cache_write_takes_rope(const CacheWriteArgs &a, const RopeQArgs &r);
hipError_t cache_write_bf16_rope(const CacheWriteArgs &a, const RopeQArgs &r, int rope_blocks,
                                 hipStream_t st);
// The absorbed query GEMM g (bf16, rows scaled by ssq_in, 256x256 tiles) with the
// in-place query RoPE r done in its tiles, and the bf16 cache write a, in one launch
// (r's flags are cleared on the way).  query_gemm_cache_write_blocks: the launch's
// workgroups, or 0 where the pair does not apply (then run them apart).
int query_gemm_cache_write_blocks(const GemmArgs &g, const CacheWriteArgs &a);
hipError_t query_gemm_cache_write(const GemmArgs &g, const CacheWriteArgs &a, const RopeQArgs &r,
                                  hipStream_t st);
// The same absorbed query GEMM alone, with the in-place query RoPE r done in its tiles
// and r's flags cleared, in one launch; query_gemm_rope_applies: where it can run.
bool query_gemm_rope_applies(const GemmArgs &g, const RopeQArgs &r);
hipError_t query_gemm_rope(const GemmArgs &g, const RopeQArgs &r, hipStream_t st);

// Window assembly: context frame i (the n_sink sink frames, then frames
// first_local, first_local+1, ...) is copied from its ring slot to rows i*tpf .. of
// `win` in the interleaved layout; with `rotate` the d_rope positional columns are
// rotated at (i, y, x) on the way (read-time rotation), else copied as stored.
struct AssembleArgs {
  RingParts ring;     // read only
  void *win;          // (B, nk, d_c + d_rope)
  int B, tpf, grid_w, d_c, d_rope;
  int64_t nk;
  int S, W, n_sink;
  int64_t first_local;
  int rotate;
  RopeTable rope;
};
hipError_t assemble_window(const AssembleArgs &a, bool bf16, hipStream_t st);

// w_t[h][c][n] = w_k_up[h*d_nope + n][c]  (per-head transpose, element size esz).
hipError_t transpose_heads(const void *w, void *w_t, int n_h, int d_nope, int d_c, int esz,
                           hipStream_t st);

// Latent query projection [n_h*(d_c+d_rope)][d_q]: per head W_qk,h = (W^K_up,h)^T
// W^Q_up,h, then the head's W^Q_R rows.
hipError_t absorb_query(const void *w_k, const void *w_q, const void *w_r, void *w_out, int n_h,
                        int d_nope, int d_c, int d_rope, int d_q, bool bf16_io, hipStream_t st);

// B = [B_1 .. B_nh], B_h = W_O[:, h*d_h:(h+1)*d_h] W^V_up,h, stored [d][n_h*d_c].
hipError_t absorb_value(const void *w_o, const void *w_v, void *w_b, int d, int n_h, int d_h,
                        int d_c, bool bf16_io, hipStream_t st);

// Latent attention over the ring window.
struct AttnArgs {
  const void *q;       // (B, R, DK)
  const void *cache;   // (B, cache_rows, DK)
  void *o;             // (B, R, DC)
  void *part;          // split records (bf16 path)
  int *flags;          // one int per fast row tile (bf16 path)
  int B, R, DC, DR;
  int64_t cache_rows;  // rows per request in the ring
  int nk;              // valid keys
  int start0, len0;    // first contiguous row range of the window; the rest starts at row 0
  int grid;            // persistent workgroups
  bool flags_zeroed;   // flags already cleared by an earlier kernel on the stream
  // Chunk-causal blocks: the R rows are nblk blocks of blk_rows rows; block k
  // attends the first min(nk0 + (k + 1) * blk_keys, nk) keys.  No mask: nblk = 1,
  // blk_rows = R, blk_keys = nk, nk0 = 0.
  int nblk, blk_rows, blk_keys, nk0;
  // Row sums (weights relative to the first key tile's max) above this make the
  // kernel recompute that piece exactly: 2^64 (overflow guard), or lower to force it.
  float sum_limit;
  // Score MFMAs in the compiler's own form instead of the inline-asm one (a check:
  // both give the same bits).
  bool builtin_scores;
  // Optional (bf16 path): the per-head value up-projection out_heads[m][h*d_head + n]
  // = sum_c W^V_up[h*d_head + n][c] O_lat[m*n_h + h][c] for the M = B*T_q tokens,
  // with the rows of split row tiles combined from their records while they are
  // loaded, instead of a merge pass into o.  Rows of split row tiles are then not
  // written to o.  out_heads null: the merge pass, o complete.
  const void *w_v_up = nullptr;
  void *out_heads = nullptr;
  int n_h = 0, d_head = 0, T_q = 0;
};
// Row tiles (with causal blocks, a block's last tile may be partial) and
// (row tile, key tile) steps of the bf16 kernel for these arguments.
struct AttnCounts {
  int64_t row_tiles;
  int64_t steps;
};
AttnCounts latent_attention_counts(const AttnArgs &a);
hipError_t latent_attention_bf16(const AttnArgs &a, hipEvent_t ev0, hipEvent_t ev1,
                                 hipStream_t st);
hipError_t latent_attention_f32(const AttnArgs &a, hipEvent_t ev0, hipEvent_t ev1,
                                hipStream_t st);
bool latent_attention_bf16_supported(int dc, int dr);
constexpr int kAttnKeyTile = 64;  // keys per tile of the bf16 kernel
// Launch geometry of the bf16 kernel for (d_c, d_rope): query rows per workgroup,
// workgroups resident per CU, and bytes of one split record (rows x d_c bf16 plus
// m and l in fp32 per row).
struct AttnLayout {
  int rows_per_wg;
  int wgs_per_cu;
  size_t record_bytes;
};
AttnLayout latent_attention_layout(int dc, int dr);

}  // namespace mla
