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
//  * a workgroup is NW waves; each wave owns QT tiles of 32 query rows and keeps
//    their q_lat in registers as MFMA B operands for the whole window;
//  * key tiles of 64 ring rows are staged once per workgroup in LDS, key-major
//    only: the score contraction S^T = K Q^T reads 16-byte K fragments, and the
//    value contraction O^T = V^T P^T reads V^T fragments of the same rows with the
//    LDS transpose load ds_read_b64_tr_b16, so no transposed copy is written;
//  * k_latent_attn_w1 (the fast kernel): one wave per SIMD with 64 query rows (32
//    at d_c = 256, whose 64-row accumulators would not fit), tiles brought in by
//    buffer loads straight into an unpadded swizzled four-stage LDS ring, and the
//    softmax of one half tile interleaved with the score MFMAs of the next;
//  * S^T comes out of v_mfma_f32_32x32x16_bf16 with one query per lane column, so
//    the row max needs one cross-lane step (lane l and l^32) and the bf16
//    probabilities feed the next MFMA as its B operand without a shuffle;
//  * the fast kernel issues its score MFMAs as inline asm with architectural VGPR
//    destinations: O fills the accumulation registers, and with S there as well
//    the compiler moved every score in and out of them (two register moves per
//    score element, in blocks the matrix unit could not hide).  The compiler
//    cannot see these MFMAs, so wherever a VALU instruction may read S right
//    after them the score half ends with an explicit wait for their results;
//  * the K and V^T fragment rings run across the three steps of a tile (each
//    step's last MFMAs issue the next step's first LDS reads), and the output rows
//    leave through an LDS image of each wave's rows as contiguous wave-wide stores;
//  * fast path: each row's softmax reference is the max of the first key tile the
//    workgroup sees for it and is never moved, so O is never rescaled inside the
//    loop (a rescale would drag the AGPR-resident accumulators through VGPRs).
//    If a row's later scores exceed the reference by more than 64 (base 2), the
//    workgroup recomputes that piece at once against each row's exact maximum (a
//    pass for the maximum, then the softmax) and flags the row tile (a lower bound
//    can be set to exercise this on ordinary data).  Below that bound every weight
//    is at most 2^64, far inside fp32 and bf16 range;
//  * the fast grid is persistent: workgroup g takes the flat range
//    [gT/G, (g+1)T/G) of T = (row tiles) x (key tiles) tile steps, so every CU gets
//    the same work (with causal blocks, whose row tiles differ in length, each row
//    tile also counts a few steps for its fixed cost, so that a workgroup on many
//    short row tiles gets fewer key tiles).  A row tile finished by one workgroup is
//    written directly; one split across workgroups leaves normalised bf16 partials
//    plus (m, l) per row, merged in a fixed order (deterministic, no atomics): by
//    k_attn_merge, or by k_merge_vup while it loads the rows for the per-head value
//    up-projection.
#include <type_traits>

#include "mla_device.h"
#include "mla_launch.h"

namespace mla {
namespace {

constexpr int BN = kAttnKeyTile;       // keys per tile
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr float kFastSumLimit = 1.8446744e19f;  // 2^64: weights above it fall back
// Word 3 of a gfx9 buffer descriptor for raw byte-addressed loads (no format
// conversion, stride 0).
constexpr int kBufferConfig = 0x00020000;

// Work of one launch.  The rows of a request form nblk blocks of blk_rows rows
// (one block, all R rows, without a causal mask); block k attends the first
// min(nk0 + (k+1) blk_keys, nk) keys.  Each block is cut into blk_rt row tiles of
// RW rows (its last tile may be partial), and row tile rt has one step per key
// tile it attends, after ov steps that stand for its fixed cost (query load, first
// tile, output and record stores) and hold no key tile: the flat split then gives
// every workgroup the same time, not the same number of key tiles, where row tiles
// differ in length (causal blocks).  Steps are numbered request by request, block by
// block, row tile by row tile: T in all, Tb per request.
struct Sched {
  int B, R, RTb, RT;
  int nk, KT;
  int start0, len0;
  int64_t cache_rows;
  int64_t T, Tb;
  int G;
  int RW;
  int nblk, blk_rows, blk_rt, blk_keys, nk0;
  int ov;
  float sum_limit;  // row sums above it flag the row tile (at most kFastSumLimit)
};

__host__ __device__ __forceinline__ int wg_of(const Sched &s, int64_t flat) {
  return (int)(((flat + 1) * s.G - 1) / s.T);
}

__host__ __device__ __forceinline__ int blk_nk(const Sched &s, int k) {
  const int v = s.nk0 + (k + 1) * s.blk_keys;
  return v < s.nk ? v : s.nk;
}

__host__ __device__ __forceinline__ int blk_kt(const Sched &s, int k) {
  return (blk_nk(s, k) + BN - 1) / BN;
}

// One row tile: its request, rows [row0, row_end), keys attended, key tiles and
// the number of the step of its first key tile (its ov cost steps come before).
struct RowTile {
  int b, row0, row_end, nk, KT;
  int64_t f0;
};

__host__ __device__ __forceinline__ RowTile row_tile(const Sched &s, int rt) {
  RowTile t;
  t.b = rt / s.RTb;
  const int j = rt - t.b * s.RTb, k = j / s.blk_rt, i = j - k * s.blk_rt;
  int64_t f = (int64_t)t.b * s.Tb;
  for (int q = 0; q < k; ++q) f += (int64_t)s.blk_rt * (blk_kt(s, q) + s.ov);
  t.nk = blk_nk(s, k);
  t.KT = (t.nk + BN - 1) / BN;
  t.f0 = f + (int64_t)i * (t.KT + s.ov) + s.ov;
  t.row0 = k * s.blk_rows + i * s.RW;
  const int lim = min((k + 1) * s.blk_rows, s.R);
  t.row_end = min(t.row0 + s.RW, lim);
  return t;
}

// The row tile that step f belongs to (one of its cost steps or a key tile).
__host__ __device__ __forceinline__ int rt_of(const Sched &s, int64_t f) {
  const int b = (int)(f / s.Tb);
  int64_t r = f - (int64_t)b * s.Tb;
  int k = 0;
  for (; k + 1 < s.nblk; ++k) {
    const int64_t wk = (int64_t)s.blk_rt * (blk_kt(s, k) + s.ov);
    if (r < wk) break;
    r -= wk;
  }
  return b * s.RTb + k * s.blk_rt + (int)(r / (blk_kt(s, k) + s.ov));
}

// The key tiles [kt0, kt1) of row tile t that the steps [begin, end) hold (empty
// where they hold only its cost steps).
__host__ __device__ __forceinline__ void piece_of(const RowTile &t, int64_t begin, int64_t end,
                                                  int &kt0, int &kt1) {
  const int64_t a = begin - t.f0, e = end - t.f0;
  kt0 = (int)(a < 0 ? 0 : a > t.KT ? t.KT : a);
  kt1 = (int)(e < 0 ? 0 : e > t.KT ? t.KT : e);
}

// One wave per SIMD, QT x 32 query rows per wave, key tiles brought into an unpadded
// swizzled four-stage LDS ring by buffer loads into LDS (k_latent_attn_w1).
template <int DC_, int DR_, int QT_ = 2, bool BUILTIN_ = false>
struct CfgW {
  static constexpr int DC = DC_, DR = DR_, QT = QT_, NW = 4, WPC = 1, NBUF = 4;
  static constexpr int NT = NW * 64;
  static constexpr int DK = DC + DR;
  static constexpr int KB = DK / 16;
  static constexpr int FT = DC / 32;
  static constexpr int RW = NW * QT * 32;
  static constexpr int CPR = DK / 8;          // 16-byte chunks per ring row
  static constexpr int LOADS = CPR / NW;      // 64-chunk loads per wave per key tile
  static constexpr int STAGE = BN * DK;       // elements per LDS stage (no padding)
  static constexpr size_t LDS = (size_t)STAGE * 2 * NBUF;
  static constexpr size_t REC = (size_t)RW * DC * 2 + (size_t)RW * 8;
  // After a row tile's first key tile, its reference max enters the score MFMAs as
  // their initial accumulator (-m), so the exponentials need no subtraction.
  static constexpr bool FOLD_MAX = true;
  // LDS fragments read ahead of their MFMAs in the score and value contractions.
  static constexpr int DS = 3, DV = 3;
  // Score MFMAs issued so that S stays in architectural VGPRs (see TileW::scores),
  // where q_lat takes at most 112 of them (more would spill).  BUILTIN_ keeps the
  // compiler's own MFMA form, against which the asm form is checked bit for bit.
  static constexpr bool ASM_SCORES = !BUILTIN_ && DK * QT <= 448;
  static_assert(CPR % 4 == 0 && LOADS * NW * 64 == BN * CPR, "tile does not split into loads");
  static_assert(DK % 16 == 0 && DC % 32 == 0, "bad widths");
};

// Production configuration per (d_c, d_rope).
template <int DC, int DR>
struct Choice {
  using Fast = CfgW<DC, DR>;
  using FastBuiltin = CfgW<DC, DR, 2, true>;
};
// At d_c = 256 the 64-row O^T alone needs all 256 accumulation registers, so the
// one-wave kernel takes 32 rows per wave there.
template <>
struct Choice<256, 32> {
  using Fast = CfgW<256, 32, 1>;
  using FastBuiltin = CfgW<256, 32, 1, true>;
};

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

// The same values into an LDS image of the wave's rows (row-major, DC wide), 16-byte
// chunk k of row r at chunk position k ^ (r & 7), so that the lanes of one write
// (32 rows) spread over the banks; the rows then leave in contiguous wave-wide stores.
template <int FT, int QT, int DC>
__device__ __forceinline__ void stage_rows(bf16 *img, const f32x16 (&O)[FT][QT], int qt, int r,
                                           float inv, int g) {
  bf16 *row = img + r * DC;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16 v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] = (bf16)(O[ft][qt][4 * i + j] * inv);
      *(uint2 *)(row + (((ft * 4 + i) ^ (r & 7)) * 8) + g * 4) = *(const uint2 *)v4;
    }
}

// Chunk swizzle of the unpadded key tile: 16-byte chunk c of tile row r sits at
// chunk position c ^ swz4(r) of that row.  With it the 32-row K fragment reads and
// the V^T transpose reads below touch every LDS bank equally often.
__device__ __forceinline__ int swz4(int r) { return (r ^ (r >> 2)) & 3; }

// The compiler does not see the inline-asm score MFMAs, so it cannot space their
// consumers: where a VALU instruction may read S right after them, wait out their
// VGPR write latency first (24 wait states, tied to S so that no read of S moves
// above it).  Elsewhere the next read of S comes after a whole value step, or after
// a barrier and an LDS read wait, far more than that.
template <class C>
__device__ __forceinline__ void drain_scores(f32x16 (&S)[C::QT]) {
  if constexpr (C::ASM_SCORES) {
    static_assert(C::QT == 1 || C::QT == 2, "drain covers one or two query tiles");
    if constexpr (C::QT == 2)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(S[0]), "+v"(S[1]));
    else
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(S[0]));
  }
}

// Key tiles of the one-wave-per-SIMD kernel.  A tile is 64 ring rows of DK bf16,
// unpadded and swizzled, brought in by buffer_load_dwordx4 ... lds: each load puts
// 64 lanes' 16 bytes at consecutive LDS chunk positions, so the swizzle is applied
// on the global side (lane p of the tile fetches the chunk that belongs at position p).
template <class C>
struct TileW {
  static constexpr int DK = C::DK, KB = C::KB, FT = C::FT, QT = C::QT, LOADS = C::LOADS;
  bf16 *base;
  const bf16 *cb;
  int nk, start0, len0;
  unsigned boff[LOADS];  // byte offset, within the tile's rows, of this lane's chunks
  int dst0;              // element offset of this wave's first load in a stage

  __device__ __forceinline__ void init(int lane, int wave) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int p = (wave * LOADS + i) * 64 + lane;
      const int r = p / C::CPR;
      boff[i] = (unsigned)(r * DK + (((p % C::CPR) ^ swz4(r)) * 8)) * 2u;
    }
    dst0 = wave * LOADS * 64 * 8;
  }

  __device__ __forceinline__ bf16 *Ks(int buf) const { return base + buf * C::STAGE; }

  __device__ __forceinline__ int64_t key_row(int kk) const {
    return kk < len0 ? (int64_t)(start0 + kk) : (int64_t)(kk - len0);
  }

  // Loads of tile kt into stage buf (completion: vmcnt; LOADS per wave either way),
  // as buffer loads into LDS through rs, a descriptor of this request's ring
  // (byte offsets; anything past its end reads as zero).  A tile that is one run of
  // consecutive ring rows takes a uniform offset plus each lane's fixed offset, no
  // per-lane address arithmetic.  Otherwise (the window's last tile, or the tile
  // where the ring wraps) each lane finds its own row; keys past nk repeat key nk-1,
  // a finite row whose probability is zero.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int kt, int buf) const {
    typedef __attribute__((address_space(3))) void lds_void;
    const int k0 = kt * BN;
    bf16 *dst = Ks(buf) + dst0;
    if ((k0 + BN <= nk) && (k0 + BN <= len0 || k0 >= len0)) {
      const int tile_off = (int)(key_row(k0) * (DK * 2));
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + i * 512), 16, (int)boff[i],
                                                 tile_off, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int e = (int)(boff[i] / 2u), r = e / DK;
        const int off = (int)(key_row(min(k0 + r, nk - 1)) * (DK * 2)) + (e - r * DK) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + i * 512), 16, off, 0, 0, 0);
      }
    }
  }

  // K fragment kb of half T of stage buf (lane: key l32, features 8g..8g+7 of k-block
  // kb); the swizzle only flips the low two chunk bits.
  __device__ __forceinline__ bf16x8 kfrag_at(int buf, int T, int l32, int g, int kb) const {
    const bf16 *rb = Ks(buf) + (T * 32 + l32) * DK;
    return *(const bf16x8 *)(rb + ((2 * (kb & 1) + g) ^ swz4(l32)) * 8 + (kb >> 1) * 32);
  }

  // S^T of one 32-key half T of the tile for both query tiles.  K fragments run
  // C::DS k-blocks ahead of their MFMAs in the ring fr, fragment kb in slot
  // (BASE + kb) % (DS + 1); with PRE the first DS are already there.  After the MFMA
  // of (k-block kb, query tile qt) the caller's work(2kb + qt) is emitted, each group
  // fenced so the order stays MFMA / VALU / MFMA / VALU; where no fragment of this
  // half is left to fetch, tail(i) fetches fragment i of the next step instead.
  template <int T, bool ZERO, bool DRAIN, int BASE, bool PRE, class Work, class Tail>
  __device__ __forceinline__ void scores(f32x16 (&S)[QT], const bf16x8 (&Qr)[QT][KB],
                                         const f32x16 (&init)[QT], int buf, int l32, int g,
                                         bf16x8 (&fr)[C::DS + 1], Work &&work,
                                         Tail &&tail) const {
    // k-block kb is chunk 2kb + g of row T*32 + l32: even and odd k-blocks each have
    // one base address
    const int sw = swz4(l32);
    const bf16 *rb = Ks(buf) + (T * 32 + l32) * DK;
    const bf16 *kr[2] = {rb + ((g ^ sw) * 8), rb + (((2 + g) ^ sw) * 8)};
    auto kfrag = [&](int kb) { return *(const bf16x8 *)(kr[kb & 1] + (kb >> 1) * 32); };
    constexpr int D = C::DS, R = D + 1;
    if constexpr (!PRE) {
#pragma unroll
      for (int kb = 0; kb < D; ++kb) fr[(BASE + kb) % R] = kfrag(kb);
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      __builtin_amdgcn_sched_barrier(0);
      if (kb + D < KB)
        fr[(BASE + kb + D) % R] = kfrag(kb + D);
      else
        tail(kb + D - KB);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if constexpr (C::ASM_SCORES) {
          if (kb == 0 && ZERO)
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                         : "=&v"(S[qt])
                         : "v"(fr[(BASE + kb) % R]), "v"(Qr[qt][kb]));
          else if (kb == 0)
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3"
                         : "=&v"(S[qt])
                         : "v"(fr[(BASE + kb) % R]), "v"(Qr[qt][kb]), "v"(init[qt]));
          else
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                         : "+v"(S[qt])
                         : "v"(fr[(BASE + kb) % R]), "v"(Qr[qt][kb]));
        } else {
          S[qt] = mfma32(fr[(BASE + kb) % R], Qr[qt][kb], kb == 0 ? init[qt] : S[qt]);
        }
        work(kb * QT + qt);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (DRAIN) drain_scores<C>(S);
  }

  // The same with a ring of its own and nothing fetched for a next step.
  template <int T, bool ZERO = false, bool DRAIN = true, class Work>
  __device__ __forceinline__ void scores(f32x16 (&S)[QT], const bf16x8 (&Qr)[QT][KB],
                                         const f32x16 (&init)[QT], int buf, int l32, int g,
                                         Work &&work) const {
    bf16x8 fr[C::DS + 1];
    scores<T, ZERO, DRAIN, 0, false>(S, Qr, init, buf, l32, g, fr, work, [](int) {});
  }
};

// V^T fragment i of key blocks KB0 .. KB0+NKB-1 of stage buf (fragment i: key block
// KB0 + i % NKB, features 32 (i / NKB) .. +31).  For key block kb the A operand of
// lane l (16-lane group G = l/16, r = l%16, g = l/32) must hold feature
// 32 (i / NKB) + l%32 of keys 16kb + 4g + j (slots 0-3) and 16kb + 8 + 4g + j (slots
// 4-7).  ds_read_b64_tr_b16 hands lane r of a 16-lane group element r%4 of the
// 8-byte pieces addressed by lanes r/4 + 4j, so lane r addresses key
// 16kb + 8h + 4g + r/4 at feature 32 (i / NKB) + 16 (G%2) + 4 (r%4) (through the chunk
// swizzle), and no transposed copy of the latent is ever written.
template <class C, int KB0, int NKB>
__device__ __forceinline__ bf16x8 vfrag_at(const TileW<C> &tl, int buf, int lane, int i) {
  typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  constexpr int DK = C::DK;
  const int G = lane >> 4, r = lane & 15, g = lane >> 5;
  const int off = (KB0 + i % NKB) * 16 * DK + (i / NKB) * 32;
  s16x4 part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * h + 4 * g + (r >> 2);
    const int chunk = (2 * (G & 1) + ((r & 3) >> 1)) ^ swz4(row);
    part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4 *)(__attribute__((address_space(3))) bf16 *)(tl.Ks(buf) + row * DK +
                                                                 chunk * 8 + (r & 1) * 4 + off));
  }
  return __builtin_bit_cast(bf16x8,
                            (s16x8)__builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// O^T += V^T P^T over key blocks KB0 .. KB0+NKB-1 (16 keys each) of the tile, V^T
// fragments read with ds_read_b64_tr_b16 as in vfrag_at (addresses through the
// swizzle) C::DV ahead of their MFMAs in the ring fr (fragment i in slot i % (DV + 1);
// with PRE the first DV are already there); P holds packed bf16 pairs.  The caller's
// work(i) follows the MFMA of (fragment i / QT, query tile i % QT), each group fenced;
// where no fragment of this step is left to fetch, tail(j) fetches fragment j of the
// next step instead.
template <class C, int KB0, int NKB, bool PRE, class Work, class Tail>
__device__ __forceinline__ void values_part(const TileW<C> &tl, f32x16 (&O)[C::FT][C::QT],
                                            const u32x4 (&P)[BN / 16][C::QT], int buf, int lane,
                                            bf16x8 (&fr)[C::DV + 1], Work &&work, Tail &&tail) {
  typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  constexpr int DK = C::DK, FT = C::FT, QT = C::QT, NF = FT * NKB, D = C::DV, R = D + 1;
  static_assert(NF % R == 0, "each value step starts the ring at slot 0");
  const int G = lane >> 4, r = lane & 15, g = lane >> 5;
  const bf16 *vt[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * h + 4 * g + (r >> 2);
    const int chunk = (2 * (G & 1) + ((r & 3) >> 1)) ^ swz4(row);
    vt[h] = tl.Ks(buf) + row * DK + chunk * 8 + (r & 1) * 4;
  }
  auto vfrag = [&](int i) {
    const int off = (KB0 + i % NKB) * 16 * DK + (i / NKB) * 32;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4 *)(__attribute__((address_space(3))) bf16 *)(vt[0] + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4 *)(__attribute__((address_space(3))) bf16 *)(vt[1] + off));
    return __builtin_bit_cast(bf16x8,
                              (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  if constexpr (!PRE) {
#pragma unroll
    for (int i = 0; i < D; ++i) fr[i] = vfrag(i);
  }
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    if (i + D < NF)
      fr[(i + D) % R] = vfrag(i + D);
    else
      tail(i + D - NF);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      O[i / NKB][qt] = mfma32(fr[i % R],
                              __builtin_bit_cast(bf16x8, P[KB0 + i % NKB][qt]), O[i / NKB][qt]);
      work(i * QT + qt);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The same with a ring of its own and nothing fetched for a next step.
template <class C, int KB0, int NKB, class Work>
__device__ __forceinline__ void values_part(const TileW<C> &tl, f32x16 (&O)[C::FT][C::QT],
                                            const u32x4 (&P)[BN / 16][C::QT], int buf, int lane,
                                            Work &&work) {
  bf16x8 fr[C::DV + 1];
  values_part<C, KB0, NKB, false>(tl, O, P, buf, lane, fr, work, [](int) {});
}

// Keys of half T past nk get -inf (only the window's last tile has any).
template <int QT>
__device__ __forceinline__ void mask_half(f32x16 (&S)[QT], int key0, int nk, int g) {
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (key0 + (r >> 2) * 8 + g * 4 + (r & 3) >= nk)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) S[qt][r] = -INFINITY;
}

// Keeps v where the surrounding code put it: the value must exist at this point
// and the empty statement cannot move past the scheduling fences around it, so
// the arithmetic feeding it stays in its MFMA slot instead of being sunk towards
// its first use.
template <typename T>
__device__ __forceinline__ void pin(T &v) {
  asm volatile("" : "+v"(v));
}

// Softmax of one 32-key half T, split into NS slots so that it can be spread over
// the MFMAs of another step: slot i takes elements [i*16QT/NS, (i+1)*16QT/NS),
// element j being row j % 16 of query tile j / 16.  Block 2T + h of P takes S
// elements 8h..8h+7 (keys T*32 + 16h + 4g + e and T*32 + 16h + 8 + 4g + e) as
// packed bf16 pairs, as the V^T fragments expect.  SUB: S still holds raw scores
// (subtract the reference max), else the max was folded into the scores.  Row
// sums go to two partial sums per query tile; pend carries an even element to the
// element that completes its pair.  Each element's sum and packing run one element
// late (prev carries it), so no instruction waits on the exponential just issued.
template <int T, int QT, int NS, bool SUB>
__device__ __forceinline__ void exp_slot(int slot, const f32x16 (&S)[QT], u32x4 (&P)[BN / 16][QT],
                                         const float (&m)[QT], float (&ls)[QT][2],
                                         float (&pend)[QT], float &prev) {
  constexpr int NE = 16 * QT;
  auto finish = [&](int j, float p) {
    const int qt = j / 16, r = j % 16;
    ls[qt][r & 1] += p;
    pin(ls[qt][r & 1]);
    if (r & 1) {
      bf16x2 w2 = {(bf16)pend[qt], (bf16)p};
      unsigned w = __builtin_bit_cast(unsigned, w2);
      pin(w);
      P[2 * T + r / 8][qt][(r % 8) / 2] = w;
    } else {
      pend[qt] = p;
    }
  };
#pragma unroll
  for (int j = slot * NE / NS; j < (slot + 1) * NE / NS; ++j) {
    const int qt = j / 16, r = j % 16;
    float p = fast_exp2(SUB ? S[qt][r] - m[qt] : S[qt][r]);
    pin(p);
    if (j > 0) finish(j - 1, prev);
    prev = p;
    if (j == NE - 1) finish(j, p);
  }
}

template <int T, int QT, bool SUB>
__device__ __forceinline__ void exp_half(const f32x16 (&S)[QT], u32x4 (&P)[BN / 16][QT],
                                         const float (&m)[QT], float (&l)[QT]) {
  float ls[QT][2] = {}, pend[QT], prev = 0.f;
  exp_slot<T, QT, 1, SUB>(0, S, P, m, ls, pend, prev);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) l[qt] += ls[qt][0] + ls[qt][1];
}

// Wait until at most N vector-memory loads of this wave are outstanding (loads
// complete in order, so every older load has landed).
template <int N>
__device__ __forceinline__ void wait_loads() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Exact recomputation of one piece (key tiles kt0 .. kt1-1 of a row tile) for the
// workgroup's rows, taken only when the fast pass over that piece overflowed.  Two
// passes, one key tile at a time through stage 0: the first takes each row's true
// maximum score over the piece, the second the softmax against it, so every weight
// is at most 1 and O is never rescaled.  Leaves O, m and l as the fast pass would
// (O unnormalised, l the lane's partial row sum).  Every wave of the workgroup
// takes it together (it has barriers); on entry every wave is done with the LDS
// stages.
template <class C>
__device__ __forceinline__ void safe_piece(const TileW<C> &tl, __amdgpu_buffer_rsrc_t rs,
                                           const bf16x8 (&Qr)[C::QT][C::KB],
                                           f32x16 (&O)[C::FT][C::QT], float (&m)[C::QT],
                                           float (&l)[C::QT], int kt0, int kt1, int last_kt,
                                           int nk, int lane, int l32, int g) {
  constexpr int QT = C::QT, FT = C::FT;
  f32x16 S0[QT], S1[QT];
  const f32x16 zero[QT] = {};
  // scores of tile kt, both halves, keys past nk at -inf
  auto tile_scores = [&](int kt) {
    tl.load(rs, kt, 0);
    wait_loads<0>();
    __syncthreads();
    tl.template scores<0, true>(S0, Qr, zero, 0, l32, g, [](int) {});
    tl.template scores<1, true>(S1, Qr, zero, 0, l32, g, [](int) {});
    if (kt == last_kt) {
      mask_half<QT>(S0, kt * BN, nk, g);
      mask_half<QT>(S1, kt * BN + 32, nk, g);
    }
  };
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) m[qt] = -INFINITY;
  for (int kt = kt0; kt < kt1; ++kt) {
    tile_scores(kt);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) m[qt] = fmaxf(m[qt], fmaxf(S0[qt][r], S1[qt][r]));
    // every wave is done with stage 0 before the next tile goes there
    __syncthreads();
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = fmaxf(m[qt], __shfl_xor(m[qt], 32, 64));
    l[qt] = 0.f;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[ft][qt][r] = 0.f;
  }
  u32x4 P[BN / 16][QT];
  for (int kt = kt0; kt < kt1; ++kt) {
    tile_scores(kt);
    exp_half<0, QT, true>(S0, P, m, l);
    exp_half<1, QT, true>(S1, P, m, l);
    values_part<C, 0, BN / 16>(tl, O, P, 0, lane, [](int) {});
    __syncthreads();
  }
}

// Fast latent attention, one wave per SIMD.  Each wave owns QT x 32 query rows
// (64 at d_c <= 192, 32 at d_c = 256) whose q_lat stays in registers; O^T lives in
// the accumulation registers.  Key tile kt is handled in three steps:
//   1. S^T of keys 0-31 of kt, beside the softmax VALU work of keys 32-63 of kt-1;
//   2. O^T += V^T P^T of tile kt-1, then the loads of tile kt+2 are issued;
//   3. S^T of keys 32-63 of kt, beside the softmax VALU work of keys 0-31 of kt,
// so the wave's own MFMAs cover its exponentials.  Four LDS stages: at the end of
// step 3 tile kt+1 has landed (tile kt+2 may still be in flight), one barrier per
// tile.  A row tile whose piece covers all its key tiles is written directly; a
// piece of a split tile goes to its record (normalised bf16 rows plus m and l)
// for k_attn_merge.
template <class C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_latent_attn_w1(const bf16 *__restrict__ q, const bf16 *__restrict__ cache,
                      bf16 *__restrict__ o, unsigned char *__restrict__ part,
                      int *__restrict__ flags, Sched s) {
  constexpr int DC = C::DC, QT = C::QT, KB = C::KB, FT = C::FT, RW = C::RW, NB = C::NBUF;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  TileW<C> tl;
  tl.base = (bf16 *)lds;
  tl.start0 = s.start0;
  tl.len0 = s.len0;
  tl.init(lane, wave);

  const int wg = blockIdx.x;
  const int64_t begin = (int64_t)wg * s.T / s.G, end = (int64_t)(wg + 1) * s.T / s.G;

  bf16x8 Qr[QT][KB];
  f32x16 O[FT][QT];
  u32x4 P[BN / 16][QT];
  f32x16 S0[QT], S1[QT];
  float m[QT], l[QT], pend[QT];

  const int rt_first = rt_of(s, begin), rt_last = rt_of(s, end - 1);
  for (int rt = rt_last; rt >= rt_first; --rt) {
    const RowTile t = row_tile(s, rt);
    int kt0, kt1;
    piece_of(t, begin, end, kt0, kt1);
    if (kt0 >= kt1) continue;  // only cost steps of this row tile fall in the range
    const int last_kt = t.KT - 1, nk = t.nk;
    const int b = t.b, row0 = t.row0;
    tl.nk = nk;
    tl.cb = cache + (int64_t)b * s.cache_rows * C::DK;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)tl.cb, (short)0, (int)(s.cache_rows * C::DK * 2), kBufferConfig);

    tl.load(rs, kt0, kt0 % NB);
    load_queries<C::DK, QT, KB>(Qr, q, s, b, row0 + wave * QT * 32, l32, g);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      l[qt] = 0.f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[ft][qt][r] = 0.f;
    }
    wait_loads<0>();
    __syncthreads();
    if (kt0 + 1 < kt1) tl.load(rs, kt0 + 1, (kt0 + 1) % NB);

    // first tile: both halves, the fixed reference max, probabilities of keys 0-31
    constexpr bool FOLD = C::FOLD_MAX;
    f32x16 init[QT] = {};
    tl.template scores<0, true>(S0, Qr, init, kt0 % NB, l32, g, [](int) {});
    tl.template scores<1, true>(S1, Qr, init, kt0 % NB, l32, g, [](int) {});
    if (kt0 == last_kt) {
      mask_half<QT>(S0, kt0 * BN, nk, g);
      mask_half<QT>(S1, kt0 * BN + 32, nk, g);
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(S0[qt][r], S1[qt][r]));
      m[qt] = fmaxf(mx, __shfl_xor(mx, 32, 64));
    }
    exp_half<0, QT, true>(S0, P, m, l);
    if (FOLD) {
      // later tiles start their scores at -m; keys 32-63 of this tile catch up here
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          init[qt][r] = -m[qt];
          S1[qt][r] -= m[qt];
        }
    }
    wait_loads<0>();
    __syncthreads();
    if (kt0 + 2 < kt1) tl.load(rs, kt0 + 2, (kt0 + 2) % NB);

    // The K and V^T fragment rings run across the steps: the last MFMAs of each phase
    // issue the first reads of the next one, so no phase starts on an LDS latency.
    // Ring slots: the first score half starts at slot 0, the second at slot B1, so that
    // KB k-blocks later the next first half is back at 0; the value step at 0.  Reads
    // of a stage that holds no tile of this request (after the last step) are not used.
    // Only where the query fits 112 registers: otherwise the rings would spill.
    constexpr bool XP = C::ASM_SCORES;
    constexpr int R = C::DS + 1, B1 = (R - KB % R) % R;
    // A phase that runs d fragments ahead has d tail slots; the next phase wants dn
    // fragments: the last slot fetches any beyond d, slots beyond dn fetch nothing.
    auto cover = [](int j, int d, int dn, auto &&fetch) {
      if (j == d - 1) {
#pragma unroll
        for (int x = j; x < dn; ++x) fetch(x);
      } else if (j < dn) {
        fetch(j);
      }
    };
    bf16x8 kfr[R], vfr[C::DV + 1];
    if constexpr (XP) {
#pragma unroll
      for (int i = 0; i < C::DS; ++i) kfr[i] = tl.kfrag_at((kt0 + 1) % NB, 0, l32, g, i);
    }

    // One tile step.  Keys past nk exist only in the window's last key tile: MASK 1
    // masks them, 0 knows kt is not that tile, 2 checks.  Where registers allow,
    // the last tile is a step of its own, so that no branch splits the scores of
    // the others.
    auto tile_step = [&](const int kt, auto mask_tag) {
      constexpr int MASK = decltype(mask_tag)::value;
      const bool LAST = MASK == 1 || (MASK == 2 && kt == last_kt);
      const int cur = kt % NB, prev = (kt + NB - 1) % NB, next = (kt + 1) % NB;
      float ls[QT][2] = {}, late = 0.f;
      tl.template scores<0, false, false, 0, XP>(
          S0, Qr, init, cur, l32, g, kfr,
          [&](int i) { exp_slot<1, QT, KB * QT, !FOLD>(i, S1, P, m, ls, pend, late); },
          [&](int j) {
            if constexpr (XP)
              cover(j, C::DS, C::DV,
                    [&](int x) { vfr[x] = vfrag_at<C, 0, BN / 16>(tl, prev, lane, x); });
          });
      // Tile kt+1 (read from the end of the second half on) has landed for every wave,
      // and every wave is done with the stage tile kt+2 goes to.
      wait_loads<0>();
      __syncthreads();
      values_part<C, 0, BN / 16, XP>(
          tl, O, P, prev, lane, vfr, [](int) {}, [&](int j) {
            if constexpr (XP)
              cover(j, C::DV, C::DS,
                    [&](int x) { kfr[(B1 + x) % R] = tl.kfrag_at(cur, 1, l32, g, x); });
          });
      __builtin_amdgcn_sched_barrier(0);
      // Tile kt+2 is requested only now: the transpose reads of the value step would
      // otherwise make the compiler wait for these loads.
      if (kt + 2 < kt1) tl.load(rs, kt + 2, (kt + 2) % NB);
      if (LAST) mask_half<QT>(S0, kt * BN, nk, g);
      tl.template scores<1, false, MASK != 0, B1, XP>(
          S1, Qr, init, cur, l32, g, kfr,
          [&](int i) { exp_slot<0, QT, KB * QT, !FOLD>(i, S0, P, m, ls, pend, late); },
          [&](int j) {
            if constexpr (XP) kfr[j] = tl.kfrag_at(next, 0, l32, g, j);
          });
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) l[qt] += ls[qt][0] + ls[qt][1];
      if (LAST) mask_half<QT>(S1, kt * BN + 32, nk, g);
    };
    if constexpr (C::ASM_SCORES) {
      const int kt_mid = kt1 == t.KT ? kt1 - 1 : kt1;  // steps before the last key tile
      for (int kt = kt0 + 1; kt < kt_mid; ++kt) tile_step(kt, std::integral_constant<int, 0>{});
      if (kt_mid < kt1 && kt_mid > kt0) tile_step(kt_mid, std::integral_constant<int, 1>{});
    } else {
      for (int kt = kt0 + 1; kt < kt1; ++kt) tile_step(kt, std::integral_constant<int, 2>{});
    }
    drain_scores<C>(S1);  // the last step may have ended right after its scores
    exp_half<1, QT, !FOLD>(S1, P, m, l);
    values_part<C, 0, BN / 16>(tl, O, P, (kt1 - 1) % NB, lane, [](int) {});
    __syncthreads();

    const bool whole = (kt0 == 0 && kt1 == t.KT);
    unsigned char *rec = part + (size_t)(wg + rt) * C::REC;
    float *rec_m = (float *)(rec + (size_t)RW * DC * 2);
    float *rec_l = rec_m + RW;
    // Normalised rows go through an LDS image of the wave's rows (the key stages are
    // free: every wave is past its last read of them) and leave as whole 16-byte
    // chunks, consecutive lanes on consecutive addresses.
    constexpr int WR = QT * 32, CPR = DC / 8;
    static_assert(CPR % 8 == 0 && (size_t)C::NW * WR * DC * 2 <= C::LDS, "row image");
    bf16 *img = tl.base + wave * WR * DC;
    // The reference key of the first tile has weight 1, so a row sum is >= 1.  Any
    // weight above 2^64 (a score more than 64 above the reference) makes it exceed
    // 2^64, as does inf or NaN: then the whole workgroup recomputes this piece
    // exactly, and the row tile's flag records it.  Sums above 2^64 made only of
    // smaller weights take that path too (harmless).
    float lt[QT];
    int bad = 0;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      lt[qt] = l[qt] + __shfl_xor(l[qt], 32, 64);
      bad |= !(lt[qt] <= s.sum_limit);
    }
    if (__builtin_expect(__syncthreads_or(bad), 0)) {
      if (tid == 0) flags[rt] = 1;
      // the piece's bounds and ring are derived again here rather than kept live
      // through the tile loop
      int rt2 = rt;
      asm volatile("" : "+s"(rt2));
      const RowTile t2 = row_tile(s, rt2);
      int k0, k1;
      piece_of(t2, begin, end, k0, k1);
      tl.nk = t2.nk;
      tl.cb = cache + (int64_t)t2.b * s.cache_rows * C::DK;
      const __amdgpu_buffer_rsrc_t rs2 = __builtin_amdgcn_make_buffer_rsrc(
          (void *)tl.cb, (short)0, (int)(s.cache_rows * C::DK * 2), kBufferConfig);
      // the queries too: their registers are free after the tile loop
      load_queries<C::DK, QT, KB>(Qr, q, s, t2.b, t2.row0 + wave * QT * 32, l32, g);
      safe_piece<C>(tl, rs2, Qr, O, m, l, k0, k1, t2.KT - 1, t2.nk, lane, l32, g);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) lt[qt] = l[qt] + __shfl_xor(l[qt], 32, 64);
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      stage_rows<FT, QT, DC>(img, O, qt, qt * 32 + l32, 1.0f / lt[qt], g);
      const int lrow = wave * WR + qt * 32 + l32;
      if (!whole && g == 0 && row0 + lrow < t.row_end) {
        rec_m[lrow] = m[qt];
        rec_l[lrow] = lt[qt];
      }
    }
    // LDS operations of one wave complete in order; this keeps the compiler from
    // moving the reads above the writes of other lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
      const int wrow0 = row0 + wave * WR;  // the wave's first row
      bf16 *dst = whole ? o + ((int64_t)b * s.R + wrow0) * DC : (bf16 *)rec + (int64_t)wave * WR * DC;
      constexpr int UNR = C::ASM_SCORES ? 6 : 4;  // 6 spills beside a 128-register query
#pragma unroll UNR
      for (int it = 0; it < WR * CPR / 64; ++it) {
        const int c = it * 64 + lane, r = c / CPR, k = c % CPR;
        const uint4 v = *(const uint4 *)(img + r * DC + ((k ^ (r & 7)) * 8));
        if (wrow0 + r < t.row_end) *(uint4 *)(dst + r * DC + k * 8) = v;
      }
    }
    // the next row tile's first loads overwrite these images
    __syncthreads();
  }
}

// Merge the pieces of every row tile that more than one workgroup worked on.  The
// grid walks either the row tiles (unsplit ones exit at once) or, when there are
// more row tiles than workgroups, the workgroup boundaries: boundary w (the first
// step of workgroup w) falls inside at most one row tile, and a split tile is taken
// at the first boundary inside it, so every split tile is merged exactly once and
// the launch does not grow with the number of row tiles.  One thread per (row, 8
// latent columns): it weighs each piece's normalised partial by l_p * 2^(m_p - max
// m) and renormalises.
template <class C>
__global__ __launch_bounds__(256) void k_attn_merge(bf16 *__restrict__ o,
                                                    const unsigned char *__restrict__ part, Sched s,
                                                    int blocks_per_tile, int by_boundary) {
  constexpr int DC = C::DC, RW = C::RW, C8 = DC / 8;
  const int unit = blockIdx.x / blocks_per_tile;
  int rt, g0;
  if (by_boundary) {
    if (unit == 0) return;
    const int64_t f = (int64_t)unit * s.T / s.G;
    rt = rt_of(s, f);
    g0 = unit - 1;
  } else {
    rt = unit;
    g0 = -1;
  }
  const RowTile t = row_tile(s, rt);
  if (by_boundary) {
    // a boundary among the row tile's key tiles, the first one (the workgroup before
    // it took the first key tile)
    if ((int64_t)unit * s.T / s.G <= t.f0 || wg_of(s, t.f0) != g0) return;
  } else {
    g0 = wg_of(s, t.f0);
  }
  const int g1 = wg_of(s, t.f0 + t.KT - 1);
  if (g0 == g1) return;
  const int idx = (blockIdx.x % blocks_per_tile) * 256 + threadIdx.x;
  const int lrow = idx / C8, c8 = (idx % C8) * 8;
  const int b = t.b, row = t.row0 + lrow;
  if (lrow >= RW || row >= t.row_end) return;
  float mmax = -INFINITY;
  for (int gg = g0; gg <= g1; ++gg) {
    const float *rm = (const float *)(part + (size_t)(gg + rt) * C::REC + (size_t)RW * DC * 2);
    mmax = fmaxf(mmax, rm[lrow]);
  }
  float wsum = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int gg = g0; gg <= g1; ++gg) {
    const unsigned char *rec = part + (size_t)(gg + rt) * C::REC;
    const float *rm = (const float *)(rec + (size_t)RW * DC * 2);
    const float w = rm[RW + lrow] * fast_exp2(rm[lrow] - mmax);
    wsum += w;
    const bf16x8 v = *(const bf16x8 *)((const bf16 *)rec + (int64_t)lrow * DC + c8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += w * (float)v[e];
  }
  const float inv = 1.0f / wsum;
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (bf16)(acc[e] * inv);
  *(bf16x8 *)(o + ((int64_t)b * s.R + row) * DC + c8) = out;
}

// The per-head value up-projection of the chunk step (Eq. 2) with the merge of split
// row tiles folded into the loading of its A operand: one workgroup computes a
// 128-token x 128-column tile of out_heads for one head h,
//   out_heads[m][h*d_head + n] = sum_c W^V_up[h*d_head + n][c] O_lat[(m, h)][c].
// Row (m, h) of O_lat is read from o when its row tile was finished by one workgroup,
// else combined from the records of the pieces, in the same order and arithmetic as
// k_attn_merge (so the rows are the same bits), and never written back.  A and the
// head's W^V_up rows sit whole in LDS (K = d_c), 16-byte chunk c of row r at
// c ^ (r & 7); W^V_up arrives by direct loads while the rows are combined.  Four
// waves of 64 x 64, 32x32x16 MFMAs in k order, as the projections' GEMM tile.
struct VupArgs {
  const bf16 *w;  // W^V_up, (n_h * d_head) x d_c
  bf16 *out;      // out_heads, (B * T_q) x (n_h * d_head)
  int M, T_q, n_h, N, nbn;
};

template <class C>
struct VupTile {
  static constexpr int DC = C::DC, BM = 64, BN = 128, NT = 256, CH = DC / 8;
  static constexpr int TPR = NT / BM;  // threads per A row
  static constexpr int CPT = CH / TPR; // 16-byte chunks per thread
  static constexpr int NP = 3;         // pieces of a row whose loads are issued together
  static constexpr int MPW = 2;        // token tiles per workgroup (one W^V_up tile load)
  static constexpr size_t A_B = (size_t)BM * DC * 2, B_B = (size_t)BN * DC * 2;
  // the bf16 output tile (rows padded by 8) over the A tile where it fits, else past B
  static constexpr size_t T_B = (size_t)BM * (BN + 8) * 2;
  static constexpr size_t T_OFF = T_B <= A_B ? 0 : A_B + B_B;
  static constexpr size_t LDS = T_OFF + T_B > A_B + B_B ? T_OFF + T_B : A_B + B_B;
  static constexpr int B_LOADS = BN * CH / 64;  // 1 KB direct loads of the W^V_up tile
  static_assert(CH % 8 == 0 && CH % TPR == 0 && B_LOADS % (NT / 64) == 0, "tile shape");
};

// Row (r, h)'s combined latent, chunks c0 .. c0+CPT-1, into acc: the fixed-order
// combination of k_attn_merge (largest m first, weights l_p 2^(m_p - max m), sums in
// piece order, rounded to bf16), or the row itself when one workgroup finished its
// row tile.  Up to NP pieces have every load issued before the first use.
template <class C>
__device__ __forceinline__ void vup_row(float (&acc)[VupTile<C>::CPT][8], const bf16 *o,
                                        const unsigned char *part, const Sched &s, int b, int row,
                                        int c0) {
  using V = VupTile<C>;
  constexpr int DC = C::DC, RW = C::RW, CPT = V::CPT, NP = V::NP;
  const int k = row / s.blk_rows, j = row - k * s.blk_rows, i = j / s.RW;
  const int rt = b * s.RTb + k * s.blk_rt + i, lrow = j - i * s.RW;
  const RowTile t = row_tile(s, rt);
  const int g0 = wg_of(s, t.f0), g1 = wg_of(s, t.f0 + t.KT - 1);
  if (g0 == g1) {
    const bf16 *src = o + ((int64_t)b * s.R + row) * DC + c0 * 8;
    bf16x8 x[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) x[c] = *(const bf16x8 *)(src + c * 8);
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[c][e] = (float)x[c][e];
    return;
  }
  auto rec = [&](int gg) { return part + (size_t)(gg + rt) * C::REC; };
  auto mrec = [&](int gg) { return (const float *)(rec(gg) + (size_t)RW * DC * 2); };
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
  float wsum = 0.f;
  if (g1 - g0 < NP) {
    float mp[NP], lp[NP];
    bf16x8 x[NP][CPT];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int gg = min(g0 + p, g1);
      mp[p] = mrec(gg)[lrow];
      lp[p] = mrec(gg)[RW + lrow];
      const bf16 *src = (const bf16 *)rec(gg) + (int64_t)lrow * DC + c0 * 8;
#pragma unroll
      for (int c = 0; c < CPT; ++c) x[p][c] = *(const bf16x8 *)(src + c * 8);
    }
    float mmax = -INFINITY;
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (g0 + p <= g1) mmax = fmaxf(mmax, mp[p]);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (g0 + p > g1) break;
      const float w = lp[p] * fast_exp2(mp[p] - mmax);
      wsum += w;
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] += w * (float)x[p][c][e];
    }
  } else {
    float mmax = -INFINITY;
    for (int gg = g0; gg <= g1; ++gg) mmax = fmaxf(mmax, mrec(gg)[lrow]);
    for (int gg = g0; gg <= g1; ++gg) {
      const bf16 *src = (const bf16 *)rec(gg) + (int64_t)lrow * DC + c0 * 8;
      bf16x8 x[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) x[c] = *(const bf16x8 *)(src + c * 8);
      const float w = mrec(gg)[RW + lrow] * fast_exp2(mrec(gg)[lrow] - mmax);
      wsum += w;
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] += w * (float)x[c][e];
    }
  }
  const float inv = 1.0f / wsum;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = (float)(bf16)(acc[c][e] * inv);
}

template <class C>
__global__ __launch_bounds__(VupTile<C>::NT) void k_merge_vup(const bf16 *__restrict__ o,
                                                   const unsigned char *__restrict__ part, Sched s,
                                                   VupArgs v) {
  using V = VupTile<C>;
  constexpr int DC = C::DC, CH = V::CH, CPT = V::CPT, BM = V::BM, BN = V::BN, NT = V::NT;
  typedef __attribute__((address_space(3))) void lds_void;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  bf16 *As = (bf16 *)lds, *Bs = (bf16 *)(lds + V::A_B);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y, mt = blockIdx.x / v.nbn, nt = blockIdx.x % v.nbn;
  const int n0 = nt * BN;

  // W^V_up rows n0.. of head h (rows past N repeat row N-1; their columns are not
  // stored), once for the workgroup's MPW token tiles: lane p of load L fetches the
  // chunk that belongs at position L*64 + p.
  {
    constexpr int LPW = V::B_LOADS / (NT / 64);
    const bf16 *wb = v.w + (int64_t)h * v.N * DC;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int L = wave * LPW + i, p = L * 64 + lane;
      const int r = p / CH, c = (p % CH) ^ (r & 7);
      __builtin_amdgcn_global_load_lds((const void *)(wb + (int64_t)min(n0 + r, v.N - 1) * DC + c * 8),
                                       (lds_void *)((unsigned char *)Bs + L * 1024), 16, 0, 0);
    }
  }
  for (int t = 0; t < V::MPW; ++t) {
    const int m0 = (mt * V::MPW + t) * BM;
    if (m0 >= v.M) break;
    // A: thread (r, part) combines chunks part*CPT .. of row (m0 + r, h)
    {
      const int r = tid / V::TPR, c0 = (tid % V::TPR) * CPT, m = m0 + r;
      float acc[CPT][8];
      if (m < v.M) {
        const int b = m / v.T_q;
        vup_row<C>(acc, o, part, s, b, (m - b * v.T_q) * v.n_h + h, c0);
      } else {
#pragma unroll
        for (int c = 0; c < CPT; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        bf16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (bf16)acc[c][e];
        *(bf16x8 *)(As + r * DC + ((c0 + c) ^ (r & 7)) * 8) = x;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the W^V_up tile too, the first time
    __syncthreads();

    // waves of 32 x 64
    static_assert(NT / 64 == (BM / 32) * (BN / 64), "one 32 x 64 block per wave");
    const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, g8 = lane >> 5;
    f32x16 acc[2];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[jn][q] = 0.f;
#pragma unroll
    for (int ks = 0; ks < DC / 16; ++ks) {
      const int ra = wm * 32 + l32;
      const bf16x8 af = *(const bf16x8 *)(As + ra * DC + ((2 * ks + g8) ^ (ra & 7)) * 8);
      bf16x8 bfr[2];
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) {
        const int rb = wn * 64 + jn * 32 + l32;
        bfr[jn] = *(const bf16x8 *)(Bs + rb * DC + ((2 * ks + g8) ^ (rb & 7)) * 8);
      }
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) acc[jn] = mfma32(af, bfr[jn], acc[jn]);
    }
    // results through LDS (clear of the W^V_up rows) for 16-byte stores
    // (acc[j][4q + e]: row 8q + 4*g8 + e, column l32 of the 32x32 tile)
    constexpr int LDC = BN + 8;
    bf16 *tile = (bf16 *)(lds + V::T_OFF);
    __syncthreads();
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = wm * 32 + (q >> 2) * 8 + g8 * 4 + (q & 3);
        tile[row * LDC + wn * 64 + jn * 32 + l32] = (bf16)acc[jn][q];
      }
    __syncthreads();
    const int ldo = v.n_h * v.N;
    for (int id = tid; id < BM * (BN / 8); id += NT) {
      const int r = id / (BN / 8), c = (id % (BN / 8)) * 8;
      if (m0 + r < v.M && n0 + c < v.N)
        *(uint4 *)(v.out + (int64_t)(m0 + r) * ldo + h * v.N + n0 + c) = *(const uint4 *)(tile + r * LDC + c);
    }
    __syncthreads();  // the next token tile's rows go where this output tile was
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
  const int nk = blk_nk(s, (int)(row - (int64_t)b * s.R) / s.blk_rows);
  for (int kk = 0; kk < nk; ++kk) {
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

// Cost steps per row tile in the bf16 kernel's split where row tiles differ in length
// (causal blocks): a row tile's fixed cost (query load, first tile and its maximum,
// output and record stores) is about six key tiles' time.  Without blocks every row
// tile has the same length and the split counts key tiles only.
constexpr int kRowTileCostSteps = 6;

Sched make_sched(const AttnArgs &a, int rows_per_wg, int grid, int ov = 0) {
  Sched s;
  s.ov = ov;
  s.B = a.B;
  s.R = a.R;
  s.RW = rows_per_wg;
  s.nk = a.nk;
  s.KT = (a.nk + BN - 1) / BN;
  s.start0 = a.start0;
  s.len0 = a.len0;
  s.cache_rows = a.cache_rows;
  if (a.nblk > 1) {
    s.nblk = a.nblk;
    s.blk_rows = a.blk_rows;
    s.blk_keys = a.blk_keys;
    s.nk0 = a.nk0;
  } else {
    s.nblk = 1;
    s.blk_rows = a.R;
    s.blk_keys = a.nk;
    s.nk0 = 0;
  }
  s.blk_rt = (s.blk_rows + rows_per_wg - 1) / rows_per_wg;
  s.RTb = s.nblk * s.blk_rt;
  s.RT = s.B * s.RTb;
  s.Tb = 0;
  for (int k = 0; k < s.nblk; ++k) s.Tb += (int64_t)s.blk_rt * (blk_kt(s, k) + s.ov);
  s.T = (int64_t)s.B * s.Tb;
  s.G = (int)((int64_t)grid < s.T ? (int64_t)grid : s.T);
  if (s.G < 1) s.G = 1;
  s.sum_limit = a.sum_limit > 0.f && a.sum_limit < kFastSumLimit ? a.sum_limit : kFastSumLimit;
  return s;
}

template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <int DC, int DR>
hipError_t launch(const AttnArgs &a, hipEvent_t ev0, hipEvent_t ev1, hipStream_t st) {
  using F = typename Choice<DC, DR>::Fast;
  Sched s = make_sched(a, F::RW, a.grid * F::WPC, a.nblk > 1 ? kRowTileCostSteps : 0);
  if (s.T <= 0) return hipSuccess;
  auto fast = k_latent_attn_w1<F>;
  if constexpr (F::ASM_SCORES) {
    // the same kernel with the compiler's MFMA form for the scores (same layout,
    // records and results), on request
    using FB = typename Choice<DC, DR>::FastBuiltin;
    static_assert(FB::RW == F::RW && FB::REC == F::REC && FB::LDS == F::LDS, "same layout");
    if (a.builtin_scores) fast = k_latent_attn_w1<FB>;
  }
  hipError_t e = allow_lds(fast, F::LDS);
  if (e != hipSuccess) return e;
  if (!a.flags_zeroed) {
    hipLaunchKernelGGL(k_fill_i32, dim3((s.RT + 255) / 256), dim3(256), 0, st, a.flags, s.RT, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(fast, dim3(s.G), dim3(F::NT), F::LDS, st, (const bf16 *)a.q,
                     (const bf16 *)a.cache, (bf16 *)a.o, (unsigned char *)a.part, a.flags, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  if (a.out_heads) {
    using V = VupTile<F>;
    VupArgs v{(const bf16 *)a.w_v_up, (bf16 *)a.out_heads, a.B * a.T_q, a.T_q, a.n_h, a.d_head,
              (a.d_head + V::BN - 1) / V::BN};
    if ((e = allow_lds(k_merge_vup<F>, V::LDS)) != hipSuccess) return e;
    const int mtiles = (v.M + V::BM * V::MPW - 1) / (V::BM * V::MPW);
    hipLaunchKernelGGL(k_merge_vup<F>, dim3(mtiles * v.nbn, a.n_h), dim3(V::NT),
                       V::LDS, st, (const bf16 *)a.o, (const unsigned char *)a.part, s, v);
    return hipGetLastError();
  }
  const int merge_blocks = (F::RW * (DC / 8) + 255) / 256;
  const int by_boundary = s.RT > s.G;
  hipLaunchKernelGGL(k_attn_merge<F>, dim3((by_boundary ? s.G : s.RT) * merge_blocks), dim3(256), 0,
                     st, (bf16 *)a.o, (const unsigned char *)a.part, s, merge_blocks, by_boundary);
  return hipGetLastError();
}

template <int DC, int DR>
AttnLayout layout() {
  using F = typename Choice<DC, DR>::Fast;
  return AttnLayout{F::RW, F::WPC, F::REC};
}

}  // namespace

bool latent_attention_bf16_supported(int dc, int dr) {
  return (dc == 192 && dr == 32) || (dc == 128 && dr == 32) || (dc == 256 && dr == 32) ||
         (dc == 192 && dr == 64);
}

AttnCounts latent_attention_counts(const AttnArgs &a) {
  const AttnLayout al = latent_attention_layout(a.DC, a.DR);
  if (al.rows_per_wg <= 0) return AttnCounts{0, 0};
  const Sched s = make_sched(a, al.rows_per_wg, 1, a.nblk > 1 ? kRowTileCostSteps : 0);
  return AttnCounts{s.RT, s.T};
}

AttnLayout latent_attention_layout(int dc, int dr) {
  if (dc == 192 && dr == 32) return layout<192, 32>();
  if (dc == 128 && dr == 32) return layout<128, 32>();
  if (dc == 256 && dr == 32) return layout<256, 32>();
  if (dc == 192 && dr == 64) return layout<192, 64>();
  return AttnLayout{0, 0, 0};
}

hipError_t latent_attention_bf16(const AttnArgs &a, hipEvent_t ev0, hipEvent_t ev1,
                                 hipStream_t st) {
  if (a.DC == 192 && a.DR == 32) return launch<192, 32>(a, ev0, ev1, st);
  if (a.DC == 128 && a.DR == 32) return launch<128, 32>(a, ev0, ev1, st);
  if (a.DC == 256 && a.DR == 32) return launch<256, 32>(a, ev0, ev1, st);
  if (a.DC == 192 && a.DR == 64) return launch<192, 64>(a, ev0, ev1, st);
  return hipErrorInvalidValue;
}

hipError_t latent_attention_f32(const AttnArgs &a, hipEvent_t ev0, hipEvent_t ev1,
                                hipStream_t st) {
  if (a.DC + a.DR > 512 || a.DC > 512) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)a.B * a.R;
  if (rows <= 0 || a.nk <= 0) return hipSuccess;
  Sched s = make_sched(a, 1, 1);
  hipError_t e;
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_latent_attn_f32, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                     (const float *)a.q, (const float *)a.cache, (float *)a.o, s, a.DC, a.DR);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace mla
