/*
 * mla.h -- C ABI of the MI355X (gfx950) VideoMLA latent-KV chunk step.
 *
 * The operation is the per-layer attention of the VideoMLA paper ("VideoMLA:
 * Low-Rank Latent KV Cache for Minute-Scale Autoregressive Video Diffusion"):
 *   - each new token x writes a content latent c^KV = RMSNorm(W^KV_down x)
 *     (§3.1 Eq. 1, App. D.2) and a head-shared positional key
 *     k^R = W^K_R x rotated by 3D-RoPE (§3.2 Eq. 5) into a ring-buffer cache
 *     of whole latent frames with FIFO eviction (App. D.4);
 *   - the query chunk attends over the valid window with per-head scores
 *     q^nope.k^nope + q^rope.k^rope scaled by 1/sqrt(d_nope + d_rope)
 *     (§3.3 Eq. 7), evaluated in the absorbed latent form of App. E
 *     (Eq. 8-9 and 12), softmax over the window, value sum accumulated in
 *     latent space and up-projected per head through W^V_up (Eq. 2);
 *   - heads are mixed by W_O (§3.3), or, with the value up-projection absorbed,
 *     by B_h = W_O,h W^V_up,h applied to the latent output (App. E Eq. 10-11);
 *   - a chunk may also be a whole clip attended with chunk-causal blocks, the
 *     training-time forward (§3.3 with the block masks of App. D.4).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA storage).
 *     The caller owns all memory; the library allocates nothing and keeps no
 *     state between calls except the thread-local error string and timing
 *     hook below.
 *   - Element type of x, weights, gains, cache, out_heads and y is cfg->dtype:
 *     MLA_BF16 (bfloat16 storage, fp32 accumulation) or MLA_F32.
 *   - Matrices are row-major [out][in] (y = W x is y_i = sum_k W[i][k] x_k).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  Arguments are validated on the host first: an invalid argument
 *     returns a negative status before anything is launched.  A failed launch
 *     returns MLA_ERR_HIP and mla_last_error() gives the HIP message.  Device
 *     faults surface at the caller's next synchronisation.  No C++ exception
 *     crosses this boundary.
 *   - Two calls that write the same cache, or share a workspace, must not run
 *     concurrently.
 *   - Safe-path hook: the bf16 attention kernel recomputes a row tile on its
 *     slower, rescaling path when its row sums, taken against the first key tile's
 *     maximum, exceed 2^64 (scores more than 64 above it, base 2).  With the
 *     environment variable MLA_ATTN_OVERFLOW_LIMIT=v (a number > 0, below 2^64)
 *     the bound is v instead, so that path can be exercised on ordinary data;
 *     results are exact either way.
 *   - Score-MFMA check: the bf16 attention kernel issues its score MFMAs as
 *     inline assembly, spacing their consumers by hand.  With the environment
 *     variable MLA_ATTN_SCORE_MFMA=builtin it runs the same kernel with the
 *     compiler's own MFMA form instead; the results are the same bits, which is
 *     what the hook is for (it is slower).
 *   - Failure injection: with the environment variable MLA_FAULT_INJECT=launch,
 *     every entry point that would launch a kernel returns MLA_ERR_HIP after
 *     its argument checks and before anything reaches the HIP runtime, with
 *     mla_last_error() naming the injection, so a caller's handling of launch
 *     failures can be exercised without a GPU.  Unset (the default), it has no
 *     effect.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* a null pointer, a bad dimension or window      */
  MLA_ERR_UNSUPPORTED = -2, /* valid, but not built for this shape and dtype  */
  MLA_ERR_ALIGNMENT = -3,   /* a pointer is not 16-byte aligned               */
  MLA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required     */
  MLA_ERR_HIP = -5          /* the HIP runtime refused a launch               */
} mla_status;

typedef enum { MLA_BF16 = 0, MLA_F32 = 1 } mla_dtype;

/* Where the shared positional key k^R is rotated (§3.2 Eq. 5, App. D.5).
 *   MLA_ROPE_AT_WRITE: rotated at the token's absolute position when it is written.
 *   MLA_ROPE_AT_READ:  stored unrotated; when a chunk attends, the window is
 *     assembled with window-local temporal coordinates (frame i of the attended
 *     context -- sink frames first, then the local frames in time order -- takes
 *     t = i) and the chunk's queries are rotated in the same frame of reference.
 *     Needed for a sink frame (the long-rollout cache of App. D.4).              */
typedef enum { MLA_ROPE_AT_WRITE = 0, MLA_ROPE_AT_READ = 1 } mla_rope_mode;

/* Layer shape, token grid and ring geometry (VideoMLA Table 4, App. D.1-D.3). */
typedef struct {
  int32_t d_model;       /* d: model width (1536)                                  */
  int32_t n_heads;       /* n_h (12)                                               */
  int32_t d_head;        /* d_h = d_nope + d_rope (128); value width per head      */
  int32_t d_nope;        /* NoPE query/key width per head (96)                     */
  int32_t d_rope;        /* RoPE width, shared key and per-head query (32), even   */
  int32_t d_c;           /* KV latent width (192)                                  */
  int32_t d_q;           /* query latent width (768)                               */
  int32_t rope_pairs[3]; /* complex pairs on the t, y, x axes; sum = d_rope / 2    */
  float rope_theta;      /* frequency base; pair k of axis a turns by              */
                         /* theta^(-2k/D_a) per position, D_y = D_x = 2*(d_head/6),*/
                         /* D_t = d_head - 2*D_y (highest bands first, §3.2)       */
  float rope_freq[64];   /* explicit radians per position of pair p (the t pairs,  */
                         /* then y, then x; entries past d_rope/2 ignored), each   */
                         /* finite.  All d_rope/2 entries zero: the table is       */
                         /* derived from rope_theta as above.                      */
  int32_t grid_h;        /* latent tokens per frame = grid_h * grid_w (30 x 52)    */
  int32_t grid_w;
  int32_t window_frames; /* W: local ring capacity in latent frames (21, or 6)     */
  int32_t dtype;         /* mla_dtype                                              */
  float rms_eps;         /* RMSNorm epsilon (1e-6)                                 */
  int32_t rope_mode;     /* mla_rope_mode                                          */
  int32_t sink_frames;   /* S: leading frames kept for good (0, or 1 in App. D.4); */
                         /* S > 0 needs MLA_ROPE_AT_READ                           */
} mla_config;

/* Weights, element type cfg->dtype, row-major [out][in] (App. D.2 shapes).      */
typedef struct {
  const void *w_kv_down; /* W^KV_down  d_c x d              (Eq. 1)                */
  const void *w_kr;      /* W^K_R      d_rope x d           (Eq. 5)                */
  const void *g_kv;      /* RMSNorm gain of c^KV, d_c; NULL = ones                 */
  const void *w_q_down;  /* W^Q_down   d_q x d              (Eq. 3)                */
  const void *g_q;       /* RMSNorm gain of c^Q, d_q; NULL = ones                  */
  const void *w_q_up;    /* W^Q_up     (n_h*d_nope) x d_q, head h = rows h*d_nope..*/
  const void *w_qr;      /* W^Q_R      (n_h*d_rope) x d_q   (Eq. 6)                */
  const void *w_k_up;    /* W^K_up     (n_h*d_nope) x d_c   (Eq. 2)                */
  const void *w_v_up;    /* W^V_up     (n_h*d_head) x d_c   (Eq. 2)                */
  const void *w_o;       /* W_O        d x (n_h*d_head)                            */
  const void *w_b;       /* optional: B = [B_1 .. B_nh], d x (n_h*d_c), B_h =       */
                         /* W_O[:, h*d_h:(h+1)*d_h] W^V_up,h (App. E Eq. 10-11),    */
                         /* as written by mla_value_absorbed_weights.  When set,    */
                         /* mla_step computes y = sum_h B_h O_lat,h in one GEMM     */
                         /* and needs neither w_v_up nor w_o; NULL: W^V_up then W_O */
  const void *w_qlat;    /* optional: the latent query projection, (n_h*(d_c +     */
                         /* d_rope)) x d_q: rows h*(d_c+d_rope) .. +d_c-1 hold     */
                         /* W_qk,h = (W^K_up,h)^T W^Q_up,h (App. E Eq. 8-9), the  */
                         /* next d_rope rows W^Q_R,h, as written by                */
                         /* mla_query_absorbed_weights.  When set, every absorbed  */
                         /* query row comes from c^Q in one GEMM, its RoPE part     */
                         /* rotated in place (then w_q_up, w_k_up and w_qr are not */
                         /* needed); NULL: W^Q_up, (W^K_up,h)^T and W^Q_R apart     */
} mla_weights;

/*
 * Where one layer's ring cache lives (App. D.4 keeps the inference cache as the
 * two tensors c^KV, B x T_cache x d_c, and k^R, B x T_cache x d_rope).  Element
 * i of ring row r of request b is at
 *     c_kv + b * c_kv_batch_stride + r * c_kv_row_stride + i   (i < d_c)
 *     k_r  + b * k_r_batch_stride  + r * k_r_row_stride  + i   (i < d_rope)
 * in units of the element type cfg->dtype.  Rules (INVALID_ARG or ALIGNMENT
 * otherwise): both pointers non-NULL and 16-byte aligned, distinct; row strides
 * at least the part's width; row and batch strides multiples of 16 bytes; with
 * batch > 1 a batch stride of at least (S + W) * tpf rows.  The two parts and the
 * requests must not overlap.
 * The interleaved layout -- one buffer of mla_cache_bytes(), row = [c^KV | k] of
 * d_c + d_rope elements, k_r = c_kv + d_c, both row strides d_c + d_rope, both
 * batch strides (S + W) * tpf * (d_c + d_rope), as mla_cache_interleaved() fills
 * it -- is read in place by the attention kernels.  Any other layout is accepted
 * by every entry point: its attended rows are first gathered into the workspace
 * in that layout, which costs one extra read and write of the attended window.
 */
typedef struct {
  void *c_kv;
  void *k_r;
  int64_t c_kv_row_stride;
  int64_t k_r_row_stride;
  int64_t c_kv_batch_stride;
  int64_t k_r_batch_stride;
} mla_cache;

/* The chunk being generated and the window it sees.                             */
typedef struct {
  int32_t batch;          /* B >= 1 independent requests (separate caches)        */
  int32_t chunk_frames;   /* C: latent frames in the query chunk (3)              */
  int64_t t0;             /* absolute index of the chunk's first latent frame,    */
                          /* >= 0 and as large as a rollout gets: rotation angles */
                          /* are formed and reduced mod 2 pi in fp64 from the     */
                          /* exact index                                           */
  int32_t n_valid_frames; /* local frames attended after the chunk is written:    */
                          /* frames t0+C-n_valid .. t0+C-1, none of them a sink   */
                          /* frame, n_valid <= W and covering every chunk frame   */
                          /* >= S.  The sink frames written so far (f < S) are    */
                          /* attended as well.                                    */
  int32_t causal_frames;  /* 0: every chunk token attends the whole window (the   */
                          /* inference step).  k > 0, dividing chunk_frames: the  */
                          /* chunk-causal forward of training (§3.3 with the      */
                          /* block masks of App. D.4): chunk frames form blocks   */
                          /* of k, and a token of block j attends the context     */
                          /* before the chunk plus blocks 0..j only.  Used by     */
                          /* chunk_attention, step and latent_attention; the      */
                          /* cache write ignores it.                              */
} mla_chunk;

/*
 * Ring contents (every entry point that takes `cache`): S + W latent-frame slots
 * per request, (S + W) * grid_h * grid_w rows.  Frame f < S occupies slot f for
 * good; frame f >= S occupies slot S + (f - S) mod W (FIFO over the local slots).
 * Token n of the frame (row-major over the grid) is row slot * grid_h * grid_w +
 * n, holding c^KV (d_c) and k (d_rope) with k = RoPE3D(k^R) at the token's
 * absolute position (t, y, x) = (f, n / grid_w, n % grid_w) under
 * MLA_ROPE_AT_WRITE, or the unrotated k^R under MLA_ROPE_AT_READ.  Only the
 * d_c + d_rope scalars per token are stored (App. E, Eq. 13).
 */

/* Host-only checks of cfg and chunk (no HIP call).  MLA_OK, INVALID_ARG or
 * UNSUPPORTED.  UNSUPPORTED: the bf16 path needs d_model, d_q, d_c, d_nope and
 * n_heads*d_head divisible by 32, d_rope divisible by 16 and (d_c, d_rope) one
 * of (128,32), (192,32), (256,32), (192,64); the fp32 path has no such limits. */
int mla_validate(const mla_config *cfg, const mla_chunk *chunk);

/* Bytes of device workspace mla_chunk_attention / mla_step need for this
 * problem; 0 if cfg/chunk are invalid.  Host-only. */
size_t mla_workspace_bytes(const mla_config *cfg, const mla_chunk *chunk);

/* Bytes of the ring cache for `batch` requests: batch * (S + W) *
 * tokens_per_frame * (d_c + d_rope) * element size.  0 if cfg is invalid.
 * Host-only. */
size_t mla_cache_bytes(const mla_config *cfg, int32_t batch);

/* Fill *cache with the interleaved layout over `base`, a buffer of
 * mla_cache_bytes(cfg, batch) bytes (see mla_cache).  MLA_OK, or INVALID_ARG /
 * ALIGNMENT for an invalid cfg, a NULL or misaligned base, or batch < 1.
 * Host-only; writes nothing but *cache. */
int mla_cache_interleaved(const mla_config *cfg, int32_t batch, void *base, mla_cache *cache);

/*
 * Cache write (§3.1 Eq. 1, App. D.2 RMSNorm, §3.2 Eq. 5, App. D.4 FIFO).
 *   x     (B, C * grid_h * grid_w, d) tokens of frames t0 .. t0+C-1, in order.
 *   cache ring described above (any layout mla_cache allows); the rows of the
 *         slots of frames t0 .. t0+C-1 are overwritten, evicting the frames that
 *         held them; nothing else is touched.  Only batch, chunk_frames and t0 of
 *         `chunk` are used; the chunk's frames >= S must fit the W local slots.
 * One fused kernel: [W^KV_down; W^K_R] x, RMSNorm of the latent, rotation of
 * k^R (MLA_ROPE_AT_WRITE only), rounding to cfg->dtype and the ring store.
 */
int mla_cache_write(const mla_config *cfg, const mla_weights *w, const mla_chunk *chunk,
                    const void *x, const mla_cache *cache, void *stream);

/*
 * Chunk attention (§3.3 Eq. 7 in the absorbed form of App. E Eq. 8-12).
 *   x         (B, C * tpf, d) the chunk's tokens (queries); frames t0 ..
 *   cache     ring holding the n_valid_frames window, the chunk's own frames
 *             included (write them first with mla_cache_write); read only.
 *   out_heads (B, C * tpf, n_h * d_head): head outputs o_h = W^V_up,h sum_j a_j c_j,
 *             concatenated over heads (before W_O).
 *   workspace device scratch of at least mla_workspace_bytes(cfg, chunk).
 * Every query attends to every valid cached token (no mask inside the window),
 * unless chunk->causal_frames cuts the chunk into causal blocks (see mla_chunk).
 * Under MLA_ROPE_AT_READ, or with a cache that is not in the interleaved layout,
 * the attended frames are first gathered into the workspace in context order
 * (under MLA_ROPE_AT_READ with k^R rotated at window-local positions).
 */
int mla_chunk_attention(const mla_config *cfg, const mla_weights *w, const mla_chunk *chunk,
                        const void *x, const mla_cache *cache, void *out_heads,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * One layer's chunk step: the work of mla_cache_write, then mla_chunk_attention,
 * then the output projection y = W_O out_heads (§3.3).  Parts that do not depend on
 * each other may run in another order or share a launch (with the absorbed bf16
 * query, the query GEMMs run first and the cache write shares a launch with the
 * query GEMM or with the query's RoPE pass); the cache write always precedes the
 * attention.  With w->w_b set, the value
 * up-projection and W_O are replaced by y = sum_h B_h O_lat,h (App. E Eq. 10-11),
 * one GEMM over the n_h * d_c latent outputs; the result is the same up to
 * rounding.
 *   y  (B, C * tpf, d).
 */
int mla_step(const mla_config *cfg, const mla_weights *w, const mla_chunk *chunk,
             const void *x, const mla_cache *cache, void *y, void *workspace, size_t ws_bytes,
             void *stream);

/*
 * mla_step without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It computes exactly what mla_step computes (the same kernels, bit for
 * bit), using a scratch array of MLA_STATIC_SCRATCH_BYTES that the library keeps in
 * the memory of every GPU it runs on until the process ends; it allocates nothing.
 * A problem whose mla_workspace_bytes() exceeds that size is refused with
 * MLA_ERR_WORKSPACE before anything is launched (one Wan-1.3B request at the
 * 21- or 42-frame window fits).  Every call on one GPU uses that GPU's array, which
 * keeps the last call's contents (the step clears what it needs cleared itself):
 * calls that overlap on one GPU -- two streams, two threads -- race on it and must
 * be serialised by the caller.  Other arguments and errors as mla_step.
 */
#define MLA_STATIC_SCRATCH_BYTES ((size_t)256 << 20)
int mla_step_static(const mla_config *cfg, const mla_weights *w, const mla_chunk *chunk,
                    const void *x, const mla_cache *cache, void *y, void *stream);

/*
 * Value absorption into the output projection (App. E Eq. 10-11), a weight
 * preparation done once per weight set:
 *   w_b (d, n_h * d_c) cfg->dtype, written: column h*d_c + c of row n is
 *       sum_k W_O[n][h*d_head + k] * W^V_up[h*d_head + k][c], summed in fp32
 *       and rounded once.  16-byte aligned, caller-owned.
 * Needs w->w_v_up and w->w_o.  Asynchronous on `stream`; INVALID_ARG or
 * ALIGNMENT before any launch, MLA_ERR_HIP if the launch fails.
 */
int mla_value_absorbed_weights(const mla_config *cfg, const mla_weights *w, void *w_b,
                               void *stream);

/*
 * Query-side absorption (App. E Eq. 8-9), a weight preparation done once per
 * weight set:
 *   w_qlat ((n_h * (d_c + d_rope)), d_q) cfg->dtype, written: for head h, row
 *        h*(d_c+d_rope) + c (c < d_c) column k is sum_n W^K_up[h*d_nope + n][c] *
 *        W^Q_up[h*d_nope + n][k], summed in fp32 and rounded once; rows
 *        h*(d_c+d_rope) + d_c + r copy W^Q_R[h*d_rope + r].  16-byte aligned,
 *        caller-owned.
 * Needs w->w_k_up, w->w_q_up and w->w_qr.  Asynchronous on `stream`; INVALID_ARG or
 * ALIGNMENT before any launch, MLA_ERR_HIP if the launch fails.
 */
int mla_query_absorbed_weights(const mla_config *cfg, const mla_weights *w, void *w_qlat,
                               void *stream);

/*
 * The latent attention loop on its own (App. E Eq. 8, 12 and 16): the inner call
 * of mla_chunk_attention, exposed so it can be timed and checked in isolation.
 *   q_lat  (B, C*tpf*n_h, d_c + d_rope) cfg->dtype; row (token*n_h + h) holds
 *          [ (W^K_up,h)^T q^nope_h | RoPE3D(q^R_h) ] multiplied by
 *          log2(e) / sqrt(d_nope + d_rope).
 *   cache  the ring, as above (read only).
 *   o_lat  (B, C*tpf*n_h, d_c) cfg->dtype: sum_j a_j c_j with a the softmax over
 *          the window of the scores q_lat . [c_j | k_rope_j] (base-2 logits).
 *   workspace  at least mla_workspace_bytes(cfg, chunk) bytes.
 * Needs MLA_ROPE_AT_WRITE and S = 0 (MLA_ERR_UNSUPPORTED otherwise): the cache is
 * attended as stored.
 */
int mla_latent_attention(const mla_config *cfg, const mla_chunk *chunk, const void *q_lat,
                         const mla_cache *cache, void *o_lat, void *workspace, size_t ws_bytes,
                         void *stream);

/* Measurement hook: when both are non-NULL, later calls on this thread record
 * the hipEvent_t `ev_start` just before and `ev_stop` just after the launch of
 * the latent-attention kernel (not its split merge), on the call's stream.
 * Pass NULLs to clear. */
void mla_set_timing_events(void *ev_start, void *ev_stop);

/* Number of workgroups the latent-attention kernel launches for this problem
 * (one persistent workgroup per compute unit, capped by the work); host-only
 * apart from one device-attribute query. */
int mla_attention_grid(const mla_config *cfg, const mla_chunk *chunk);

/* Where the bf16 attention leaves its overflow flags in the workspace: *offset
 * (bytes from the workspace start) and *count int32 flags, one per row tile of
 * the fast kernel.  After a call, a nonzero flag means that some of that row
 * tile's scores rose more than 64 (base 2) above the maximum of the first key
 * tile a workgroup saw for it, so the attention kernel recomputed that
 * workgroup's part of the row tile against the exact maximum (exact either way).  Host-only; MLA_OK, or INVALID_ARG for
 * an invalid cfg/chunk or NULL outputs; *count = 0 on the fp32 path. */
int mla_overflow_flags(const mla_config *cfg, const mla_chunk *chunk, size_t *offset,
                       int64_t *count);

const char *mla_status_string(int status);
/* Thread-local text of the last failure on this thread ("" if none). */
const char *mla_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H */
