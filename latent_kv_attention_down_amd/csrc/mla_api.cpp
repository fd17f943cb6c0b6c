// Host side of the C ABI declared in include/mla.h: argument validation, ring and
// window index arithmetic, workspace carving and the launch sequence of the MLA
// chunk step on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "mla.h"
#include "mla_launch.h"

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

constexpr int kMaxAttnGrid = 512;  // persistent attention workgroups, upper bound
constexpr size_t kAlign = 256;
constexpr size_t kStaticScratchBytes = MLA_STATIC_SCRATCH_BYTES;  // mla_step_static

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int fail(int status, const std::string &msg) {
  g_last_error = msg;
  return status;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

#define MLA_TRY_LOCAL(expr)      \
  do {                           \
    int s_ = (expr);             \
    if (s_ != MLA_OK) return s_; \
  } while (0)

// Shapes derived from the config and chunk.
struct Dims {
  int64_t tpf;          // tokens per latent frame
  int64_t T_q;          // chunk tokens per request
  int64_t M;            // B * T_q
  int64_t R;            // rows per request = T_q * n_h
  int64_t DK;           // d_c + d_rope
  int64_t ring;         // (S + W) * tpf cache rows per request
  int64_t n_sink;       // sink frames attended (those written so far)
  int64_t first_local;  // first local frame attended
  int64_t nk;           // attended keys: (n_sink + n_valid) * tpf
  bool at_read;         // keys rotated on window assembly
  bool gathered;        // the window is gathered into the workspace (read-time
                        // rotation, or a ring not in the interleaved layout)
  int64_t start0;       // keys read in place: the window as (up to) two ring ranges,
  int64_t len0;         // [start0, start0 + len0) then [0, nk - len0)
  int64_t t0_q;         // temporal coordinate of the chunk's first frame for queries
  int64_t nblk;         // chunk-causal blocks (1: no mask)
  int64_t blk_rows;     // rows per block: causal_frames * tpf * n_h (R without a mask)
  int64_t blk_keys;     // keys each block adds: causal_frames * tpf (nk without a mask)
  int64_t nk0;          // keys before the chunk in context order (0 without a mask)
  size_t esz;
};

// in_place: the ring is in the interleaved layout, so the attention kernels can
// read it where it is (see mla_cache).
Dims dims(const mla_config &c, const mla_chunk &k, bool in_place = true) {
  Dims d;
  d.tpf = (int64_t)c.grid_h * c.grid_w;
  d.T_q = (int64_t)k.chunk_frames * d.tpf;
  d.M = (int64_t)k.batch * d.T_q;
  d.R = d.T_q * c.n_heads;
  d.DK = (int64_t)c.d_c + c.d_rope;
  const int64_t S = c.sink_frames;
  d.ring = (S + c.window_frames) * d.tpf;
  const int64_t last = k.t0 + k.chunk_frames - 1;
  d.n_sink = std::min<int64_t>(S, last + 1);
  d.first_local = last - k.n_valid_frames + 1;
  d.nk = (d.n_sink + k.n_valid_frames) * d.tpf;
  d.at_read = c.rope_mode == MLA_ROPE_AT_READ;
  d.gathered = d.at_read || !in_place;
  // queries: frame i of the read-time context has temporal coordinate i (the
  // chunk's frames are consecutive); otherwise the absolute frame index (S == 0)
  d.t0_q = !d.at_read ? k.t0 : (k.t0 < S ? k.t0 : d.n_sink + (k.t0 - d.first_local));
  if (d.gathered) {
    // the gathered window is one contiguous range in context order
    d.start0 = 0;
    d.len0 = d.nk;
  } else {  // S == 0
    const int64_t slot0 = d.first_local % c.window_frames;
    const int64_t run = std::min<int64_t>(k.n_valid_frames, c.window_frames - slot0);
    d.start0 = slot0 * d.tpf;
    d.len0 = run * d.tpf;
  }
  // the chunk's frames are the last C frames of the context (sinks included when
  // the chunk starts inside them)
  if (k.causal_frames > 0) {
    d.nblk = k.chunk_frames / k.causal_frames;
    d.blk_keys = (int64_t)k.causal_frames * d.tpf;
    d.blk_rows = d.blk_keys * c.n_heads;
    d.nk0 = d.nk - d.T_q;
  } else {
    d.nblk = 1;
    d.blk_rows = d.R;
    d.blk_keys = d.nk;
    d.nk0 = 0;
  }
  d.esz = c.dtype == MLA_BF16 ? 2 : 4;
  return d;
}

// An explicit frequency table is given when any of the d_rope / 2 entries is set.
bool explicit_freq(const mla_config &c) {
  for (int p = 0; p < c.d_rope / 2 && p < 64; ++p)
    if (c.rope_freq[p] != 0.f) return true;
  return false;
}

int validate_config(const mla_config *c) {
  if (!c) return fail(MLA_ERR_INVALID_ARG, "cfg is NULL");
  if (c->d_model <= 0 || c->n_heads <= 0 || c->d_head <= 0 || c->d_nope <= 0 || c->d_rope <= 0 ||
      c->d_c <= 0 || c->d_q <= 0)
    return fail(MLA_ERR_INVALID_ARG, "dimensions must be positive");
  if (c->d_nope + c->d_rope != c->d_head)
    return fail(MLA_ERR_INVALID_ARG, "d_nope + d_rope must equal d_head");
  if (c->d_rope % 2 != 0) return fail(MLA_ERR_INVALID_ARG, "d_rope must be even");
  if (c->d_rope / 2 > 64) return fail(MLA_ERR_INVALID_ARG, "at most 64 RoPE pairs");
  for (int a = 0; a < 3; ++a)
    if (c->rope_pairs[a] < 0) return fail(MLA_ERR_INVALID_ARG, "negative rope_pairs");
  if (c->rope_pairs[0] + c->rope_pairs[1] + c->rope_pairs[2] != c->d_rope / 2)
    return fail(MLA_ERR_INVALID_ARG, "rope_pairs must sum to d_rope / 2");
  for (int p = 0; p < c->d_rope / 2; ++p)
    if (!std::isfinite(c->rope_freq[p])) return fail(MLA_ERR_INVALID_ARG, "rope_freq must be finite");
  if (!explicit_freq(*c) && (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta)))
    return fail(MLA_ERR_INVALID_ARG, "rope_theta must be positive and finite");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps))
    return fail(MLA_ERR_INVALID_ARG, "rms_eps must be >= 0 and finite");
  if (c->grid_h <= 0 || c->grid_w <= 0) return fail(MLA_ERR_INVALID_ARG, "grid must be positive");
  if (c->window_frames <= 0) return fail(MLA_ERR_INVALID_ARG, "window_frames must be positive");
  if (c->dtype != MLA_BF16 && c->dtype != MLA_F32) return fail(MLA_ERR_INVALID_ARG, "unknown dtype");
  if (c->rope_mode != MLA_ROPE_AT_WRITE && c->rope_mode != MLA_ROPE_AT_READ)
    return fail(MLA_ERR_INVALID_ARG, "unknown rope_mode");
  if (c->sink_frames < 0) return fail(MLA_ERR_INVALID_ARG, "sink_frames must be >= 0");
  if (c->sink_frames > 0 && c->rope_mode != MLA_ROPE_AT_READ)
    return fail(MLA_ERR_INVALID_ARG, "sink frames need MLA_ROPE_AT_READ (window-local re-indexing)");
  const int64_t ring = ((int64_t)c->sink_frames + c->window_frames) * c->grid_h * c->grid_w;
  if (ring >= (int64_t)1 << 30) return fail(MLA_ERR_INVALID_ARG, "ring too large");
  if (c->dtype == MLA_BF16) {
    if (c->d_model % 32 || c->d_q % 32 || c->d_c % 32 || c->d_nope % 32 ||
        (c->n_heads * c->d_head) % 32 || c->d_rope % 16)
      return fail(MLA_ERR_UNSUPPORTED,
                  "bf16 path needs d_model, d_q, d_c, d_nope, n_heads*d_head % 32 == 0 and "
                  "d_rope % 16 == 0");
    // the attention kernel addresses one request's ring (or assembled window) with
    // 32-bit byte offsets
    if (ring * (c->d_c + c->d_rope) * 2 >= ((int64_t)1 << 31))
      return fail(MLA_ERR_UNSUPPORTED, "bf16 path needs a ring of under 2 GiB per request");
    if (!mla::latent_attention_bf16_supported(c->d_c, c->d_rope))
      return fail(MLA_ERR_UNSUPPORTED,
                  "bf16 path is built for (d_c, d_rope) in {(128,32), (192,32), (256,32), (192,64)}");
  } else {
    if (c->d_c + c->d_rope > 512) return fail(MLA_ERR_UNSUPPORTED, "fp32 path needs d_c + d_rope <= 512");
  }
  return MLA_OK;
}

// Chunk frames at or after the sink: they need local slots.
int64_t local_chunk_frames(const mla_config *c, const mla_chunk *k) {
  const int64_t end = k->t0 + k->chunk_frames;
  return std::max<int64_t>(0, end - std::max<int64_t>(k->t0, c->sink_frames));
}

// Checks every entry point needs: the chunk itself and its place in the ring.
int validate_chunk_write(const mla_config *c, const mla_chunk *k) {
  if (!k) return fail(MLA_ERR_INVALID_ARG, "chunk is NULL");
  if (k->batch <= 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1");
  if (k->chunk_frames <= 0) return fail(MLA_ERR_INVALID_ARG, "chunk_frames must be >= 1");
  if (k->t0 < 0) return fail(MLA_ERR_INVALID_ARG, "t0 must be >= 0");
  if (local_chunk_frames(c, k) > c->window_frames)
    return fail(MLA_ERR_INVALID_ARG, "chunk_frames must fit the window_frames local slots");
  if (k->causal_frames < 0 || (k->causal_frames > 0 && k->chunk_frames % k->causal_frames != 0))
    return fail(MLA_ERR_INVALID_ARG, "causal_frames must be 0 or divide chunk_frames");
  const int64_t rows = (int64_t)k->batch * k->chunk_frames * c->grid_h * c->grid_w * c->n_heads;
  if (rows >= (int64_t)1 << 30) return fail(MLA_ERR_INVALID_ARG, "chunk too large");
  return MLA_OK;
}

// Attention also needs the window: n_valid local frames ending at the chunk's
// last frame, covering every chunk frame that is not a sink, none of them a sink.
int validate_chunk(const mla_config *c, const mla_chunk *k) {
  MLA_TRY_LOCAL(validate_chunk_write(c, k));
  const int64_t need = local_chunk_frames(c, k);
  if (k->n_valid_frames < need || k->n_valid_frames > c->window_frames)
    return fail(MLA_ERR_INVALID_ARG,
                "need (chunk frames at or after the sink) <= n_valid_frames <= window_frames");
  if (k->n_valid_frames > 0 &&
      k->t0 + k->chunk_frames - k->n_valid_frames < (int64_t)c->sink_frames)
    return fail(MLA_ERR_INVALID_ARG, c->sink_frames ? "local window reaches into the sink frames"
                                                    : "window reaches before frame 0");
  return MLA_OK;
}

int validate(const mla_config *c, const mla_chunk *k) {
  int s = validate_config(c);
  if (s != MLA_OK) return s;
  return validate_chunk(c, k);
}

// write: the cache-write weights; attend: the query side and W^K_up; heads: the
// per-head outputs (W^V_up); project: y, either through w_b or through W^V_up
// and W_O.
int validate_weights(const mla_config &c, const mla_weights *w, bool write, bool attend,
                     bool heads, bool project) {
  if (!w) return fail(MLA_ERR_INVALID_ARG, "weights is NULL");
  if (write && (!w->w_kv_down || !w->w_kr)) return fail(MLA_ERR_INVALID_ARG, "w_kv_down/w_kr NULL");
  if (attend && (!w->w_q_down || (!w->w_qlat && (!w->w_q_up || !w->w_k_up || !w->w_qr))))
    return fail(MLA_ERR_INVALID_ARG, "need w_q_down, and w_qlat or all of w_q_up, w_k_up, w_qr");
  if (heads && !w->w_v_up) return fail(MLA_ERR_INVALID_ARG, "w_v_up is NULL");
  if (project && !w->w_b && (!w->w_v_up || !w->w_o))
    return fail(MLA_ERR_INVALID_ARG, "need w_b, or w_v_up and w_o");
  const void *ptrs[] = {w->w_kv_down, w->w_kr, w->w_q_down, w->w_q_up, w->w_qr,
                        w->w_k_up,    w->w_v_up, w->w_o,    w->w_b, w->w_qlat};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return fail(MLA_ERR_ALIGNMENT, "weights must be 16-byte aligned");
  (void)c;
  return MLA_OK;
}

// RoPE table: pair k of axis a turns by theta^(-2k / D_a) per unit position with
// D_y = D_x = 2 * floor(d_head / 6) and D_t = d_head - 2 * D_y; the pairs of each
// axis take its highest-frequency bands (k = 0, 1, ...).
// An explicit rope_freq table replaces the derived bands entry for entry.
mla::RopeTable rope_table(const mla_config &c) {
  mla::RopeTable t;
  std::memset(&t, 0, sizeof(t));
  const int d_sp = 2 * (c.d_head / 6);
  const int width[3] = {c.d_head - 2 * d_sp, d_sp, d_sp};
  const bool given = explicit_freq(c);
  int p = 0;
  for (int a = 0; a < 3; ++a)
    for (int k = 0; k < c.rope_pairs[a]; ++k, ++p) {
      t.axis[p] = a;
      t.omega[p] = given ? (double)c.rope_freq[p]
                         : std::pow((double)c.rope_theta, -2.0 * k / (double)width[a]);
    }
  t.n_pairs = p;
  return t;
}

// Compute units of the current device (capped), the persistent grid's unit.
int attn_grid_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  return cus < kMaxAttnGrid ? cus : kMaxAttnGrid;
}

// Attention geometry (no pointers): rows, keys, ring ranges and causal blocks.
mla::AttnArgs attn_shape(const mla_config &c, const mla_chunk &k, const Dims &d) {
  mla::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.B = k.batch;
  a.R = (int)d.R;
  a.DC = c.d_c;
  a.DR = c.d_rope;
  a.cache_rows = d.gathered ? d.nk : d.ring;
  a.nk = (int)d.nk;
  a.start0 = (int)d.start0;
  a.len0 = (int)d.len0;
  a.grid = 0;  // set at launch (a device query)
  a.nblk = (int)d.nblk;
  a.blk_rows = (int)d.blk_rows;
  a.blk_keys = (int)d.blk_keys;
  a.nk0 = (int)d.nk0;
  return a;
}

// Workspace carving (offsets in bytes, each 256-aligned).
struct Workspace {
  size_t u_q, c_q, q_nope, q_r, w_t, q_lat, o_lat, part, flags, out_heads, win, total;
  int64_t n_flags;  // overflow flags of the bf16 attention (one per row tile)
};

Workspace carve(const mla_config &c, const mla_chunk &k) {
  const Dims d = dims(c, k);
  Workspace w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  w.u_q = take((size_t)d.M * c.d_q * 4);
  w.c_q = take((size_t)d.M * c.d_q * d.esz);
  w.q_nope = take((size_t)d.M * c.n_heads * c.d_nope * d.esz);
  w.q_r = take((size_t)d.M * c.n_heads * c.d_rope * 4);
  w.w_t = take((size_t)c.n_heads * c.d_c * c.d_nope * d.esz);
  w.q_lat = take((size_t)k.batch * d.R * d.DK * d.esz);
  w.o_lat = take((size_t)k.batch * d.R * c.d_c * d.esz);
  size_t part = 0, flags = 0;
  w.n_flags = 0;
  if (c.dtype == MLA_BF16) {
    // split records are indexed (workgroup + row tile) < grid + row tiles
    const mla::AttnLayout al = mla::latent_attention_layout(c.d_c, c.d_rope);
    const int64_t rt = mla::latent_attention_counts(attn_shape(c, k, d)).row_tiles;
    part = (size_t)((int64_t)kMaxAttnGrid * al.wgs_per_cu + rt) * al.record_bytes;
    flags = (size_t)rt * sizeof(int);
    w.n_flags = rt;
  }
  w.part = take(part);
  w.flags = take(flags);
  w.out_heads = take((size_t)d.M * c.n_heads * c.d_head * d.esz);
  // the attended frames gathered in context order (read-time rotation, or a ring
  // that is not in the interleaved layout); the workspace size does not depend on
  // the ring's layout, so the room is always there
  w.win = take((size_t)k.batch * d.nk * d.DK * d.esz);
  w.total = off;
  return w;
}

int hip_fail(hipError_t e, const char *stage) {
  return fail(MLA_ERR_HIP, std::string(stage) + ": " + hipGetErrorString(e));
}

#define MLA_HIP(call, stage)                      \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hip_fail(e_, stage); \
  } while (0)

// The ring parts of a validated cache descriptor.
mla::RingParts ring_parts(const mla_cache &r) {
  mla::RingParts p;
  p.c_kv = r.c_kv;
  p.k_r = r.k_r;
  p.c_row = r.c_kv_row_stride;
  p.r_row = r.k_r_row_stride;
  p.c_batch = r.c_kv_batch_stride;
  p.r_batch = r.k_r_batch_stride;
  return p;
}

// Checks of a cache descriptor (the rules stated with mla_cache in mla.h).
int validate_cache(const mla_config &c, int32_t batch, const mla_cache *r) {
  if (!r) return fail(MLA_ERR_INVALID_ARG, "cache is NULL");
  if (!r->c_kv || !r->k_r) return fail(MLA_ERR_INVALID_ARG, "cache parts c_kv and k_r must be set");
  if (r->c_kv == r->k_r) return fail(MLA_ERR_INVALID_ARG, "cache parts c_kv and k_r coincide");
  if (!aligned16(r->c_kv) || !aligned16(r->k_r))
    return fail(MLA_ERR_ALIGNMENT, "cache parts must be 16-byte aligned");
  const int64_t esz = c.dtype == MLA_BF16 ? 2 : 4, per16 = 16 / esz;
  if (r->c_kv_row_stride < c.d_c || r->k_r_row_stride < c.d_rope)
    return fail(MLA_ERR_INVALID_ARG, "cache row strides must cover d_c and d_rope elements");
  if (r->c_kv_row_stride % per16 || r->k_r_row_stride % per16 || r->c_kv_batch_stride % per16 ||
      r->k_r_batch_stride % per16)
    return fail(MLA_ERR_ALIGNMENT, "cache strides must be multiples of 16 bytes");
  const int64_t rows = ((int64_t)c.sink_frames + c.window_frames) * c.grid_h * c.grid_w;
  if (batch > 1 && (r->c_kv_batch_stride < rows * r->c_kv_row_stride ||
                    r->k_r_batch_stride < rows * r->k_r_row_stride))
    return fail(MLA_ERR_INVALID_ARG, "cache batch strides must hold a whole ring per request");
  if (r->c_kv_batch_stride < 0 || r->k_r_batch_stride < 0)
    return fail(MLA_ERR_INVALID_ARG, "cache batch strides must be >= 0");
  return MLA_OK;
}

// The interleaved layout: rows of d_c + d_rope elements, k_r right after c_kv,
// requests one ring after another.  The attention kernels read it in place.
bool cache_in_place(const mla_config &c, int32_t batch, const mla_cache &r) {
  const int64_t dk = (int64_t)c.d_c + c.d_rope, esz = c.dtype == MLA_BF16 ? 2 : 4;
  const int64_t rows = ((int64_t)c.sink_frames + c.window_frames) * c.grid_h * c.grid_w;
  if ((const unsigned char *)r.k_r != (const unsigned char *)r.c_kv + c.d_c * esz) return false;
  if (r.c_kv_row_stride != dk || r.k_r_row_stride != dk) return false;
  if (batch > 1 && (r.c_kv_batch_stride != rows * dk || r.k_r_batch_stride != rows * dk)) return false;
  return true;
}

// MLA_ATTN_OVERFLOW_LIMIT=v (a number > 0): the fast attention kernel recomputes
// (and flags) the pieces whose row sums exceed v instead of 2^64, so its exact
// path can be exercised on ordinary data; unset or invalid: 2^64.
float overflow_limit() {
  const char *v = std::getenv("MLA_ATTN_OVERFLOW_LIMIT");
  if (!v || !*v) return 0.f;
  char *end = nullptr;
  const float f = std::strtof(v, &end);
  return (end && *end == 0 && f > 0.f && std::isfinite(f)) ? f : 0.f;
}

// MLA_ATTN_SCORE_MFMA=builtin: the fast attention kernel issues its score MFMAs in
// the compiler's form instead of inline asm (same results, bit for bit).
bool builtin_scores() {
  const char *v = std::getenv("MLA_ATTN_SCORE_MFMA");
  return v && std::strcmp(v, "builtin") == 0;
}

// MLA_FAULT_INJECT=launch: refuse every launch before it reaches the HIP runtime.
int launch_gate() {
  const char *v = std::getenv("MLA_FAULT_INJECT");
  if (v && std::strcmp(v, "launch") == 0)
    return fail(MLA_ERR_HIP, "MLA_FAULT_INJECT=launch: launch refused before reaching the HIP runtime");
  return MLA_OK;
}

mla::CacheWriteArgs cache_write_args(const mla_config &c, const mla_weights &w, const mla_chunk &k,
                                     const void *x, const mla_cache &cache) {
  const Dims d = dims(c, k);
  mla::CacheWriteArgs a;
  a.x = x;
  a.w_kv = w.w_kv_down;
  a.w_kr = w.w_kr;
  a.g_kv = w.g_kv;
  a.ring = ring_parts(cache);
  a.M = (int)d.M;
  a.T_q = (int)d.T_q;
  a.d = c.d_model;
  a.d_c = c.d_c;
  a.d_rope = c.d_rope;
  a.tpf = (int)d.tpf;
  a.grid_w = c.grid_w;
  a.W = c.window_frames;
  a.S = c.sink_frames;
  a.rotate = d.at_read ? 0 : 1;
  a.t0 = k.t0;
  a.eps = c.rms_eps;
  a.rope = rope_table(c);
  return a;
}

int run_cache_write(const mla_config &c, const mla_weights &w, const mla_chunk &k, const void *x,
                    const mla_cache &cache, hipStream_t st) {
  const mla::CacheWriteArgs a = cache_write_args(c, w, k, x, cache);
  if (c.dtype == MLA_BF16)
    MLA_HIP(mla::cache_write_bf16(a, st), "cache write");
  else
    MLA_HIP(mla::cache_write_f32(a, st), "cache write");
  return MLA_OK;
}

// The attended keys: the ring itself when it is in the interleaved layout and keys
// were rotated at write; otherwise the attended frames gathered in context order
// into the workspace (rotated at window-local positions under read-time rotation,
// §3.2 Eq. 5, App. D.4-D.5; copied as stored for another layout).
int attended_keys(const mla_config &c, const mla_chunk &k, const Dims &d, const mla_cache &cache,
                  unsigned char *ws, const void **keys, hipStream_t st) {
  if (!d.gathered) {
    *keys = cache.c_kv;
    return MLA_OK;
  }
  const Workspace L = carve(c, k);
  mla::AssembleArgs wa;
  wa.ring = ring_parts(cache);
  wa.win = ws + L.win;
  wa.B = k.batch;
  wa.tpf = (int)d.tpf;
  wa.grid_w = c.grid_w;
  wa.d_c = c.d_c;
  wa.d_rope = c.d_rope;
  wa.nk = d.nk;
  wa.S = c.sink_frames;
  wa.W = c.window_frames;
  wa.n_sink = (int)d.n_sink;
  wa.first_local = d.first_local;
  wa.rotate = d.at_read ? 1 : 0;
  wa.rope = rope_table(c);
  MLA_HIP(mla::assemble_window(wa, c.dtype == MLA_BF16, st), "window assembly");
  *keys = ws + L.win;
  return MLA_OK;
}

// Latent attention over `keys`: the ring itself, or the window gathered in context
// order in the workspace.
int run_latent_attention(const mla_config &c, const mla_chunk &k, const Dims &d, const void *q_lat,
                         const void *keys, void *o_lat, unsigned char *ws, bool flags_zeroed,
                         hipStream_t st, const void *w_v_up = nullptr, void *out_heads = nullptr) {
  const Workspace L = carve(c, k);
  mla::AttnArgs a = attn_shape(c, k, d);
  if (out_heads) {  // bf16: the value up-projection takes the place of the merge pass
    a.w_v_up = w_v_up;
    a.out_heads = out_heads;
    a.n_h = c.n_heads;
    a.d_head = c.d_head;
    a.T_q = (int)d.T_q;
  }
  a.q = q_lat;
  a.cache = keys;
  a.o = o_lat;
  a.part = ws + L.part;
  a.flags = (int *)(ws + L.flags);
  a.flags_zeroed = flags_zeroed;
  a.grid = attn_grid_cus();
  a.sum_limit = overflow_limit();
  a.builtin_scores = builtin_scores();
  if (c.dtype == MLA_BF16)
    MLA_HIP(mla::latent_attention_bf16(a, g_ev_start, g_ev_stop, st), "latent attention");
  else
    MLA_HIP(mla::latent_attention_f32(a, g_ev_start, g_ev_stop, st), "latent attention");
  return MLA_OK;
}

mla::GemmArgs gemm(const void *A, int64_t lda, int64_t sA, const void *B, int64_t ldb, int64_t sB,
                   void *C, int64_t ldc, int64_t sC, int64_t M, int N, int K, int batch, float alpha) {
  mla::GemmArgs g;
  g.A = A;
  g.lda = lda;
  g.sA = sA;
  g.B = B;
  g.ldb = ldb;
  g.sB = sB;
  g.C = C;
  g.ldc = ldc;
  g.sC = sC;
  g.M = (int)M;
  g.N = N;
  g.K = K;
  g.batch = batch;
  g.alpha = alpha;
  return g;
}

int run_gemm(const mla_config &c, const mla::GemmArgs &g, bool out_f32, hipStream_t st,
             const char *stage) {
  if (c.dtype == MLA_BF16)
    MLA_HIP(mla::gemm_bf16_nt(g, out_f32, st), stage);
  else
    MLA_HIP(mla::gemm_f32_nt(g, st), stage);
  return MLA_OK;
}

#define MLA_TRY(expr)           \
  do {                          \
    int s_ = (expr);            \
    if (s_ != MLA_OK) return s_; \
  } while (0)

// Query preparation (Eq. 3-4, 6; App. E Eq. 8-9): the absorbed query rows in the
// workspace.  Where the absorbed query GEMM takes 256x256 tiles it rotates the rope
// columns in its tiles and clears the attention's flags (*rotated then says so);
// otherwise the RoPE pass (its arguments in *rq_out) does that, launched here unless
// the caller takes it over (launch_rope false).  With `ride` (a cache write of the
// same step) the GEMM and that write share one launch where they fit (*wrote).
int prepare_queries(const mla_config &c, const mla_weights &w, const mla_chunk &k, const void *x,
                    unsigned char *ws, hipStream_t st, bool launch_rope, mla::RopeQArgs *rq_out,
                    const mla::CacheWriteArgs *ride = nullptr, bool *wrote = nullptr,
                    bool *rotated = nullptr) {
  bool rot = false;
  if (wrote) *wrote = false;
  const Dims d = dims(c, k);
  const Workspace L = carve(c, k);
  const bool bf = c.dtype == MLA_BF16;
  const int nh = c.n_heads;
  const float scale = (float)(1.4426950408889634 / std::sqrt((double)(c.d_nope + c.d_rope)));
  float *u_q = (float *)(ws + L.u_q);
  void *c_q = ws + L.c_q, *q_nope = ws + L.q_nope, *w_t = ws + L.w_t;
  float *q_r = (float *)(ws + L.q_r);
  unsigned char *q_lat = ws + L.q_lat;
  // RoPE3D(q^R_h) into the last d_rope columns, same scale (Eq. 6, 12)
  mla::RopeQArgs rq;
  rq.q_r = q_r;
  rq.q_lat = q_lat;
  rq.M = (int)d.M;
  rq.T_q = (int)d.T_q;
  rq.n_h = nh;
  rq.d_rope = c.d_rope;
  rq.d_c = c.d_c;
  rq.tpf = (int)d.tpf;
  rq.grid_w = c.grid_w;
  rq.t0 = d.t0_q;  // absolute, or the chunk's place in the re-indexed context (App. D.5)
  rq.scale = scale;
  rq.rope = rope_table(c);
  rq.zero = (int *)(ws + L.flags);  // the attention's overflow flags (bf16 path)
  rq.n_zero = (int)L.n_flags;
  rq.in_place = w.w_qlat != nullptr;
  if (rq.in_place) rq.q_r = nullptr;

  if (w.w_qlat && bf) {
    // c^Q = RMSNorm(W^Q_down x) * g_q (Eq. 3, App. D.2) taken apart over the two GEMMs:
    // the first stores u * g_q (u = W^Q_down x) with the sums of squares of u per row in
    // 64-column pieces; the second sums them and scales each row by 1 / RMS(u) on its
    // way out.  Every absorbed query row [q~_h | q^R_h] = W_qlat,h c^Q, scaled, comes out
    // of that one GEMM: W_qlat,h = [(W^K_up,h)^T W^Q_up,h ; W^Q_R,h] prepared once
    // (App. E Eq. 8-9).
    float *ssq = u_q;  // (d_q / 64 pieces) x M fp32
    mla::GemmArgs g1 = gemm(x, c.d_model, 0, w.w_q_down, c.d_model, 0, c_q, c.d_q, 0, d.M, c.d_q,
                            c.d_model, 1, 1.f);
    g1.col_scale = w.g_q;
    g1.ssq_out = ssq;
    MLA_TRY(run_gemm(c, g1, false, st, "query down-projection"));
    mla::GemmArgs g2 = gemm(c_q, c.d_q, 0, w.w_qlat, c.d_q, 0, q_lat, (int64_t)nh * d.DK, 0, d.M,
                            (int)(nh * d.DK), c.d_q, 1, scale);
    g2.ssq_in = ssq;
    g2.ssq_parts = (c.d_q + 63) / 64;
    g2.ssq_scale = 1.0f / (float)c.d_q;
    g2.ssq_eps = c.rms_eps;
    // The query's RoPE columns are rotated in the GEMM's tiles (and the attention's flags
    // cleared) where the GEMM takes 256x256 tiles; in mla_step the cache write shares
    // that launch where it fits beside it.
    const int both = ride ? mla::query_gemm_cache_write_blocks(g2, *ride) : 0;
    if (both > 0 && both <= attn_grid_cus()) {
      MLA_HIP(mla::query_gemm_cache_write(g2, *ride, rq, st),
              "absorbed query projection with query rope and cache write");
      if (wrote) *wrote = true;
      rot = true;
    } else if (mla::query_gemm_rope_applies(g2, rq)) {
      MLA_HIP(mla::query_gemm_rope(g2, rq, st), "absorbed query projection with query rope");
      rot = true;
    } else {
      MLA_TRY(run_gemm(c, g2, false, st, "absorbed query projection"));
    }
  } else {
    // c^Q = RMSNorm(W^Q_down x)  (Eq. 3, App. D.2)
    MLA_TRY(run_gemm(c, gemm(x, c.d_model, 0, w.w_q_down, c.d_model, 0, u_q, c.d_q, 0, d.M, c.d_q,
                             c.d_model, 1, 1.f),
                     true, st, "query down-projection"));
    MLA_HIP(mla::rmsnorm_rows(u_q, w.g_q, c_q, (int)d.M, c.d_q, c.rms_eps, bf, st), "query rmsnorm");
    if (w.w_qlat) {
      // every absorbed query row [q~_h | q^R_h] = W_qlat,h c^Q, scaled, in one GEMM:
      // W_qlat,h = [(W^K_up,h)^T W^Q_up,h ; W^Q_R,h] prepared once (App. E Eq. 8-9)
      MLA_TRY(run_gemm(c, gemm(c_q, c.d_q, 0, w.w_qlat, c.d_q, 0, q_lat, (int64_t)nh * d.DK, 0, d.M,
                               (int)(nh * d.DK), c.d_q, 1, scale),
                       false, st, "absorbed query projection"));
    } else {
      // q^R = W^Q_R c^Q (Eq. 6); q^nope = W^Q_up c^Q (Eq. 4), then q~_h =
      // (W^K_up,h)^T q^nope_h, scaled (App. E Eq. 8-9 applied to the query)
      MLA_TRY(run_gemm(c, gemm(c_q, c.d_q, 0, w.w_qr, c.d_q, 0, q_r, (int64_t)nh * c.d_rope, 0, d.M,
                               nh * c.d_rope, c.d_q, 1, 1.f),
                       true, st, "positional query projection"));
      MLA_TRY(run_gemm(c, gemm(c_q, c.d_q, 0, w.w_q_up, c.d_q, 0, q_nope, (int64_t)nh * c.d_nope, 0,
                               d.M, nh * c.d_nope, c.d_q, 1, 1.f),
                       false, st, "query up-projection"));
      MLA_HIP(mla::transpose_heads(w.w_k_up, w_t, nh, c.d_nope, c.d_c, (int)d.esz, st),
              "key up transpose");
      MLA_TRY(run_gemm(c, gemm(q_nope, (int64_t)nh * c.d_nope, c.d_nope, w_t, c.d_nope,
                               (int64_t)c.d_c * c.d_nope, q_lat, (int64_t)nh * d.DK, d.DK, d.M, c.d_c,
                               c.d_nope, nh, scale),
                       false, st, "key absorption"));
    }
  }
  if (rq_out) *rq_out = rq;
  if (rotated) *rotated = rot;
  if (launch_rope && !rot) MLA_HIP(mla::rope_q(rq, bf, st), "query rope");
  return MLA_OK;
}

// Latent attention over the window and, when out_heads is given, the per-head value
// up-projection, on queries prepared by prepare_queries.
int attend(const mla_config &c, const mla_weights &w, const mla_chunk &k, const mla_cache &cache,
           void *out_heads, unsigned char *ws, hipStream_t st) {
  const Dims d = dims(c, k, cache_in_place(c, k.batch, cache));
  const Workspace L = carve(c, k);
  const int nh = c.n_heads;
  unsigned char *q_lat = ws + L.q_lat, *o_lat = ws + L.o_lat;
  const void *keys = nullptr;
  MLA_TRY(attended_keys(c, k, d, cache, ws, &keys, st));
  // softmax over the window, latent value sum (Eq. 7 absorbed, Eq. 12, 16).  In bf16
  // the value up-projection (Eq. 2) combines the split row tiles as it loads them
  // where they are a large share (at most four row tiles per attention workgroup:
  // the single chunk, small batches); otherwise a merge pass completes O_lat first.
  if (out_heads && c.dtype == MLA_BF16 &&
      mla::latent_attention_counts(attn_shape(c, k, d)).row_tiles <= 4 * (int64_t)attn_grid_cus())
    return run_latent_attention(c, k, d, q_lat, keys, o_lat, ws, true, st, w.w_v_up, out_heads);
  MLA_TRY(run_latent_attention(c, k, d, q_lat, keys, o_lat, ws, true, st));
  if (!out_heads) return MLA_OK;  // O_lat stays in the workspace
  // o_h = W^V_up,h O_lat,h  (Eq. 2)
  MLA_TRY(run_gemm(c, gemm(o_lat, (int64_t)nh * c.d_c, c.d_c, w.w_v_up, c.d_c,
                           (int64_t)c.d_head * c.d_c, out_heads, (int64_t)nh * c.d_head, c.d_head,
                           d.M, c.d_head, c.d_c, nh, 1.f),
                   false, st, "value up-projection"));
  return MLA_OK;
}

// Query preparation, latent attention and, when out_heads is given, the per-head
// value up-projection.
int run_chunk_attention(const mla_config &c, const mla_weights &w, const mla_chunk &k,
                        const void *x, const mla_cache &cache, void *out_heads, unsigned char *ws,
                        hipStream_t st) {
  MLA_TRY(prepare_queries(c, w, k, x, ws, st, true, nullptr));
  return attend(c, w, k, cache, out_heads, ws, st);
}

int check_ws(const mla_config &c, const mla_chunk &k, void *ws, size_t ws_bytes) {
  const size_t need = carve(c, k).total;
  if (!ws || ws_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(MLA_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  return MLA_OK;
}

// Checks of mla_step's arguments other than the workspace.
int validate_step(const mla_config *cfg, const mla_weights *w, const mla_chunk *chunk,
                  const void *x, const mla_cache *cache, const void *y) {
  MLA_TRY(validate(cfg, chunk));
  MLA_TRY(validate_weights(*cfg, w, true, true, false, true));
  if (!x || !y) return fail(MLA_ERR_INVALID_ARG, "x or y is NULL");
  if (!aligned16(x) || !aligned16(y))
    return fail(MLA_ERR_ALIGNMENT, "x and y must be 16-byte aligned");
  MLA_TRY(validate_cache(*cfg, chunk->batch, cache));
  return MLA_OK;
}

// The chunk step on validated arguments: cache write, chunk attention, output
// projection (§3.3), in `ws` laid out by carve().  With the absorbed bf16 query the
// query GEMMs run first and the query's in-place RoPE pass (with the flag clearing)
// rides in the cache write's launch, on the CUs the write leaves idle; the write
// still precedes the attention, which reads the chunk's own frames.
int run_step(const mla_config &c, const mla_weights &w, const mla_chunk &k, const void *x,
             const mla_cache &cache, void *y, unsigned char *ws, hipStream_t st) {
  const Workspace L = carve(c, k);
  const Dims d = dims(c, k);
  const mla::CacheWriteArgs cw = cache_write_args(c, w, k, x, cache);
  // Where they fit, the cache write shares the absorbed query GEMM's launch (the GEMM
  // leaves 47 of 256 CUs idle at the Wan-1.3B chunk); otherwise the query's RoPE pass
  // shares the cache write's launch, fused only where the CUs the write leaves idle can
  // take the RoPE items at no more than 8 per thread (each item is a dependent
  // read-modify-write, so a thread's items run one after another): the single-request
  // chunk, not batches or clips.
  const int cw_blocks = (int)((d.M + 31) / 32), cus = attn_grid_cus();
  const int64_t rope_items = d.M * c.n_heads * (c.d_rope / 8);
  const int64_t wg_threads = 2 * (c.d_c + c.d_rope);  // the cache write's workgroup: 64 * N / 32
  const int64_t rope_needed = (rope_items + 8 * wg_threads - 1) / (8 * wg_threads);
  const bool absorbed_bf16 = c.dtype == MLA_BF16 && w.w_qlat;
  if (absorbed_bf16) {
    mla::RopeQArgs rq;
    bool wrote = false, rotated = false;
    MLA_TRY(prepare_queries(c, w, k, x, ws, st, false, &rq, &cw, &wrote, &rotated));
    if (wrote) {
      // the cache write, the query's RoPE and the flags are done
    } else if (rotated) {
      MLA_TRY(run_cache_write(c, w, k, x, cache, st));  // the RoPE and the flags are done
    } else if (mla::cache_write_takes_rope(cw, rq) && cw_blocks + rope_needed <= cus) {
      MLA_HIP(mla::cache_write_bf16_rope(cw, rq, cus - cw_blocks, st), "cache write with query rope");
    } else {
      MLA_TRY(run_cache_write(c, w, k, x, cache, st));
      MLA_HIP(mla::rope_q(rq, true, st), "query rope");
    }
  } else {
    MLA_TRY(run_cache_write(c, w, k, x, cache, st));
    MLA_TRY(prepare_queries(c, w, k, x, ws, st, true, nullptr));
  }
  if (w.w_b) {
    MLA_TRY(attend(c, w, k, cache, nullptr, ws, st));
    // y = sum_h B_h O_lat,h  (App. E Eq. 10-11): row (token) of O_lat is n_h * d_c wide
    const int64_t kb = (int64_t)c.n_heads * c.d_c;
    MLA_TRY(run_gemm(c, gemm(ws + L.o_lat, kb, 0, w.w_b, kb, 0, y, c.d_model, 0, d.M, c.d_model,
                             (int)kb, 1, 1.f),
                     false, st, "value-absorbed output projection"));
    return MLA_OK;
  }
  MLA_TRY(attend(c, w, k, cache, ws + L.out_heads, ws, st));
  // y = W_O out  (§3.3)
  MLA_TRY(run_gemm(c, gemm(ws + L.out_heads, (int64_t)c.n_heads * c.d_head, 0, w.w_o,
                           (int64_t)c.n_heads * c.d_head, 0, y, c.d_model, 0, d.M, c.d_model,
                           c.n_heads * c.d_head, 1, 1.f),
                   false, st, "output projection"));
  return MLA_OK;
}

}  // namespace

// ---------------------------------------------------------------- static scratch
// mla_step_static's scratch: one array in every device's memory, held until the
// process ends.  Host code must not use the array's name as a device address (it
// names the host-side stand-in): static_scratch() asks the runtime for the current
// device's copy once and keeps that address per device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char *g_scratch_ptr[kMaxDevices] = {};

int static_scratch(unsigned char **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "static scratch: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERR_UNSUPPORTED, "static scratch: device index beyond 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "static scratch: hipGetSymbolAddress");
    if (!p || ((uintptr_t)p & (kAlign - 1)) != 0)
      return fail(MLA_ERR_HIP, "static scratch: the runtime gave no 256-byte aligned address");
    g_scratch_ptr[dev] = (unsigned char *)p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_validate(const mla_config *cfg, const mla_chunk *chunk) {
  g_last_error.clear();
  return validate(cfg, chunk);
}

size_t mla_workspace_bytes(const mla_config *cfg, const mla_chunk *chunk) {
  if (validate(cfg, chunk) != MLA_OK) return 0;
  return carve(*cfg, *chunk).total;
}

size_t mla_cache_bytes(const mla_config *cfg, int32_t batch) {
  if (validate_config(cfg) != MLA_OK || batch <= 0) return 0;
  const size_t esz = cfg->dtype == MLA_BF16 ? 2 : 4;
  return (size_t)batch * ((size_t)cfg->sink_frames + cfg->window_frames) * cfg->grid_h *
         cfg->grid_w * (size_t)(cfg->d_c + cfg->d_rope) * esz;
}

int mla_cache_interleaved(const mla_config *cfg, int32_t batch, void *base, mla_cache *cache) {
  g_last_error.clear();
  MLA_TRY(validate_config(cfg));
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1");
  if (!base || !cache) return fail(MLA_ERR_INVALID_ARG, "base or cache is NULL");
  if (!aligned16(base)) return fail(MLA_ERR_ALIGNMENT, "base must be 16-byte aligned");
  const int64_t dk = (int64_t)cfg->d_c + cfg->d_rope, esz = cfg->dtype == MLA_BF16 ? 2 : 4;
  const int64_t rows = ((int64_t)cfg->sink_frames + cfg->window_frames) * cfg->grid_h * cfg->grid_w;
  cache->c_kv = base;
  cache->k_r = (unsigned char *)base + cfg->d_c * esz;
  cache->c_kv_row_stride = cache->k_r_row_stride = dk;
  cache->c_kv_batch_stride = cache->k_r_batch_stride = rows * dk;
  return MLA_OK;
}

int mla_cache_write(const mla_config *cfg, const mla_weights *w, const mla_chunk *chunk,
                    const void *x, const mla_cache *cache, void *stream) {
  g_last_error.clear();
  MLA_TRY(validate_config(cfg));
  MLA_TRY(validate_chunk_write(cfg, chunk));
  MLA_TRY(validate_weights(*cfg, w, true, false, false, false));
  if (!x) return fail(MLA_ERR_INVALID_ARG, "x is NULL");
  if (!aligned16(x)) return fail(MLA_ERR_ALIGNMENT, "x must be 16-byte aligned");
  MLA_TRY(validate_cache(*cfg, chunk->batch, cache));
  MLA_TRY(launch_gate());
  return run_cache_write(*cfg, *w, *chunk, x, *cache, (hipStream_t)stream);
}

int mla_chunk_attention(const mla_config *cfg, const mla_weights *w, const mla_chunk *chunk,
                        const void *x, const mla_cache *cache, void *out_heads, void *workspace,
                        size_t ws_bytes, void *stream) {
  g_last_error.clear();
  MLA_TRY(validate(cfg, chunk));
  MLA_TRY(validate_weights(*cfg, w, false, true, true, false));
  if (!x || !out_heads) return fail(MLA_ERR_INVALID_ARG, "x or out_heads is NULL");
  if (!aligned16(x) || !aligned16(out_heads))
    return fail(MLA_ERR_ALIGNMENT, "x and out_heads must be 16-byte aligned");
  MLA_TRY(validate_cache(*cfg, chunk->batch, cache));
  MLA_TRY(check_ws(*cfg, *chunk, workspace, ws_bytes));
  MLA_TRY(launch_gate());
  return run_chunk_attention(*cfg, *w, *chunk, x, *cache, out_heads, (unsigned char *)workspace,
                             (hipStream_t)stream);
}

int mla_step(const mla_config *cfg, const mla_weights *w, const mla_chunk *chunk, const void *x,
             const mla_cache *cache, void *y, void *workspace, size_t ws_bytes, void *stream) {
  g_last_error.clear();
  MLA_TRY(validate_step(cfg, w, chunk, x, cache, y));
  MLA_TRY(check_ws(*cfg, *chunk, workspace, ws_bytes));
  MLA_TRY(launch_gate());
  return run_step(*cfg, *w, *chunk, x, *cache, y, (unsigned char *)workspace,
                  (hipStream_t)stream);
}

int mla_step_static(const mla_config *cfg, const mla_weights *w, const mla_chunk *chunk,
                    const void *x, const mla_cache *cache, void *y, void *stream) {
  g_last_error.clear();
  MLA_TRY(validate_step(cfg, w, chunk, x, cache, y));
  const size_t need = carve(*cfg, *chunk).total;
  if (need > kStaticScratchBytes)
    return fail(MLA_ERR_WORKSPACE, "mla_step_static: this problem needs " + std::to_string(need) +
                                       " bytes of scratch; the static scratch holds " +
                                       std::to_string(kStaticScratchBytes) +
                                       " (use mla_step with a workspace)");
  MLA_TRY(launch_gate());
  unsigned char *ws = nullptr;
  MLA_TRY(static_scratch(&ws));
  return run_step(*cfg, *w, *chunk, x, *cache, y, ws, (hipStream_t)stream);
}

int mla_query_absorbed_weights(const mla_config *cfg, const mla_weights *w, void *w_qlat,
                               void *stream) {
  g_last_error.clear();
  MLA_TRY(validate_config(cfg));
  if (!w || !w->w_k_up || !w->w_q_up || !w->w_qr)
    return fail(MLA_ERR_INVALID_ARG, "need w_k_up, w_q_up and w_qr");
  if (!w_qlat) return fail(MLA_ERR_INVALID_ARG, "w_qlat is NULL");
  if (!aligned16(w->w_k_up) || !aligned16(w->w_q_up) || !aligned16(w->w_qr) || !aligned16(w_qlat))
    return fail(MLA_ERR_ALIGNMENT, "w_k_up, w_q_up, w_qr and w_qlat must be 16-byte aligned");
  MLA_TRY(launch_gate());
  MLA_HIP(mla::absorb_query(w->w_k_up, w->w_q_up, w->w_qr, w_qlat, cfg->n_heads, cfg->d_nope,
                            cfg->d_c, cfg->d_rope, cfg->d_q, cfg->dtype == MLA_BF16,
                            (hipStream_t)stream),
          "query absorption");
  return MLA_OK;
}

int mla_value_absorbed_weights(const mla_config *cfg, const mla_weights *w, void *w_b,
                               void *stream) {
  g_last_error.clear();
  MLA_TRY(validate_config(cfg));
  if (!w || !w->w_v_up || !w->w_o) return fail(MLA_ERR_INVALID_ARG, "need w_v_up and w_o");
  if (!w_b) return fail(MLA_ERR_INVALID_ARG, "w_b is NULL");
  if (!aligned16(w->w_v_up) || !aligned16(w->w_o) || !aligned16(w_b))
    return fail(MLA_ERR_ALIGNMENT, "w_v_up, w_o and w_b must be 16-byte aligned");
  MLA_TRY(launch_gate());
  MLA_HIP(mla::absorb_value(w->w_o, w->w_v_up, w_b, cfg->d_model, cfg->n_heads, cfg->d_head,
                            cfg->d_c, cfg->dtype == MLA_BF16, (hipStream_t)stream),
          "value absorption");
  return MLA_OK;
}

int mla_latent_attention(const mla_config *cfg, const mla_chunk *chunk, const void *q_lat,
                         const mla_cache *cache, void *o_lat, void *workspace, size_t ws_bytes,
                         void *stream) {
  g_last_error.clear();
  MLA_TRY(validate(cfg, chunk));
  if (cfg->rope_mode != MLA_ROPE_AT_WRITE || cfg->sink_frames != 0)
    return fail(MLA_ERR_UNSUPPORTED, "mla_latent_attention attends the cache as stored: "
                                     "needs MLA_ROPE_AT_WRITE and no sink");
  if (!q_lat || !o_lat) return fail(MLA_ERR_INVALID_ARG, "q_lat or o_lat is NULL");
  if (!aligned16(q_lat) || !aligned16(o_lat))
    return fail(MLA_ERR_ALIGNMENT, "q_lat and o_lat must be 16-byte aligned");
  MLA_TRY(validate_cache(*cfg, chunk->batch, cache));
  MLA_TRY(check_ws(*cfg, *chunk, workspace, ws_bytes));
  MLA_TRY(launch_gate());
  const Dims d = dims(*cfg, *chunk, cache_in_place(*cfg, chunk->batch, *cache));
  unsigned char *ws = (unsigned char *)workspace;
  hipStream_t st = (hipStream_t)stream;
  const void *keys = nullptr;
  MLA_TRY(attended_keys(*cfg, *chunk, d, *cache, ws, &keys, st));
  return run_latent_attention(*cfg, *chunk, d, q_lat, keys, o_lat, ws, false, st);
}

void mla_set_timing_events(void *ev_start, void *ev_stop) {
  if (ev_start && ev_stop) {
    g_ev_start = (hipEvent_t)ev_start;
    g_ev_stop = (hipEvent_t)ev_stop;
  } else {
    g_ev_start = nullptr;
    g_ev_stop = nullptr;
  }
}

int mla_attention_grid(const mla_config *cfg, const mla_chunk *chunk) {
  if (validate(cfg, chunk) != MLA_OK) return 0;
  const Dims d = dims(*cfg, *chunk);
  if (cfg->dtype != MLA_BF16) return (int)((d.M * cfg->n_heads + 3) / 4);
  const mla::AttnLayout al = mla::latent_attention_layout(cfg->d_c, cfg->d_rope);
  const int64_t t = mla::latent_attention_counts(attn_shape(*cfg, *chunk, d)).steps;
  const int64_t g = (int64_t)attn_grid_cus() * al.wgs_per_cu;
  return (int)(g < t ? g : t);
}

int mla_overflow_flags(const mla_config *cfg, const mla_chunk *chunk, size_t *offset,
                       int64_t *count) {
  g_last_error.clear();
  MLA_TRY(validate(cfg, chunk));
  if (!offset || !count) return fail(MLA_ERR_INVALID_ARG, "offset or count is NULL");
  const Workspace L = carve(*cfg, *chunk);
  *offset = L.flags;
  *count = L.n_flags;
  return MLA_OK;
}

const char *mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_ALIGNMENT: return "MLA_ERR_ALIGNMENT";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_UNKNOWN_STATUS";
  }
}

const char *mla_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
