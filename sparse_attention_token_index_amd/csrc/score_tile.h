// Index scores of one query row against a 32-key tile staged in LDS, on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fused with ReLU and the
// weighted reduction over heads.
//
// Score of key s for a query row (the lightning-indexer score; per-head
// weights reduce over heads after a per-head ReLU):
//     I[s] = sum_h w[h] * max(0, sum_d q[h, d] * k[s, d])
//
// Mapping: heads are the MFMA M dimension (M-tiles of 32 heads, heads past H
// are zero), the tile's 32 keys the N dimension and the head dim the K
// dimension (k-steps of 16).  The reduction index is permuted consistently
// for both operands: lane (c = l % 32, g = l / 32) supplies dims
// [g*D/2 + 8 j, g*D/2 + 8 j + 8) at k-step j, so every operand fragment is one
// 16-byte load and a lane's fragments cover one contiguous half of the head
// dim.  The accumulator lane (c, g) holds key c for 16 heads of each M-tile
// (rows 8 (r/4) + 4 g + r%4): ReLU, the head weights and the sum over M-tiles
// run in registers, and one shuffle adds the other half of the heads, leaving
// lanes l and l + 32 both holding the full score of key l % 32.
#pragma once

#include "device_common.h"

namespace dsai {

// Layout of staged key rows in LDS.  D = 128: rows are packed (256 bytes)
// and the 16-byte chunk x of row r is stored at chunk x ^ (r & 15), so the
// 16 keys a quarter-wave's ds_read_b128 gathers (same chunk of consecutive
// rows) land on distinct bank groups without padding.  Smaller D: rows are
// padded by 16 bytes instead.
template <int D>
struct TileGeom {
  static constexpr int kChunksPerRow = D / 8;  // 16-byte chunks
  static constexpr bool kSwizzle = D == 128;
  static constexpr int kRowBytes = kSwizzle ? 2 * D : 2 * D + 16;
  static constexpr int kTileKeys = 32;  // keys per matrix-core tile
  static constexpr int kTileBytes = kTileKeys * kRowBytes;
  static __device__ __forceinline__ uint32_t chunk_offset(int row, int x) {
    return (uint32_t)(row * kRowBytes + 16 * (kSwizzle ? (x ^ (row & 15)) : x));
  }
};

// Stages KEYS consecutive key rows (bf16, `row_stride` elements apart) from
// device memory into LDS, through registers so the next stage's loads
// overlap the current stage's math.  Loads go through a buffer resource whose
// range ends at the last valid key row: rows past it read as zero without a
// branch, and each thread's byte offsets within a stage are loop-invariant
// (the stage's row offset is a scalar).
template <int D, int NTHREADS, int KEYS = 32>
struct TileLoader {
  using G = TileGeom<D>;
  static constexpr int kChunks = KEYS * G::kChunksPerRow;
  static_assert(kChunks % NTHREADS == 0 || NTHREADS % kChunks == 0,
                "stage chunks must divide over the block (or the block over the chunks)");
  static constexpr int kPer = kChunks >= NTHREADS ? kChunks / NTHREADS : 1;
  static constexpr bool kSpare = kChunks < NTHREADS;  // some threads load nothing
  u32x4 r[kPer];
  uint32_t voff[kPer];
  uint32_t loff[kPer];
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t row_bytes;  // bytes between consecutive key rows in device memory

  // base: row 0 of the keys; valid_bytes: bytes from base through the end of
  // the last valid row (< 2^32).
  __device__ __forceinline__ void init(const uint16_t* base, uint32_t row_stride,
                                       uint32_t valid_bytes) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)valid_bytes, 0x00020000);
    row_bytes = row_stride * 2u;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = kSpare ? (int)threadIdx.x % kChunks : (int)threadIdx.x + i * NTHREADS;
      const int row = ch / G::kChunksPerRow;
      const int part = ch % G::kChunksPerRow;
      voff[i] = (uint32_t)row * row_bytes + (uint32_t)part * 16u;
      loff[i] = G::chunk_offset(row, part);
    }
  }

  __device__ __forceinline__ void load(uint32_t row0) {
    // the stage offset is wave-uniform; saying so keeps it scalar where the
    // compiler cannot prove it (a buffer load needs it in a scalar register)
    const uint32_t soff = __builtin_amdgcn_readfirstlane(row0 * row_bytes);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff[i], soff, 0));
  }

  __device__ __forceinline__ void store(lds_char* stage) const {
    if (kSpare && (int)threadIdx.x >= kChunks) return;
#pragma unroll
    for (int i = 0; i < kPer; ++i) *reinterpret_cast<DSAI_LDS u32x4*>(stage + loff[i]) = r[i];
  }
};

// NR query rows per wavefront share each key fragment read from LDS: every
// k-step feeds NR * MT independent accumulators, enough for one wavefront to
// keep the matrix core busy on its own.
template <int HP, int D, int NR = 1>
struct TileScorer {
  static_assert(HP == 32 || HP == 64, "padded heads: 32 or 64");
  static_assert(D % 16 == 0 && D >= 32 && D <= 128, "head dim: 32, 48, ... 128");
  static constexpr int MT = HP / 32;
  static constexpr int KS = D / 16;
  using G = TileGeom<D>;
  using Acc = floatx16[NR][MT];

  bf16x8 qf[NR][MT][KS];
  float wv[NR][MT][16];
  uint32_t boff0;  // LDS offset of this lane's key fragment at k-step 0

  __device__ __forceinline__ void init_offsets() {
    const int lane = lane_id();
    const int c = lane & 31, g = lane >> 5;
    boff0 = G::chunk_offset(c, g * KS);  // dims g*D/2 + 8j at k-step j
  }

  // Offset at k-step j: chunk g*KS + j of row c.  Swizzled rows: KS = 8 and
  // g*KS + j = 8g | j, so XOR-ing j into the chunk bits of the k-step-0
  // offset applies the row's swizzle; padded rows: consecutive chunks.
  __device__ __forceinline__ uint32_t frag_offset(int j) const {
    if constexpr (G::kSwizzle) {
      static_assert(KS == 8, "swizzled rows hold 16 chunks");
      return boff0 ^ ((uint32_t)j << 4);
    } else {
      return boff0 + 16u * (uint32_t)j;
    }
  }

  // Row `rr` of the wavefront: qrow [H, D] bf16, wrow [H] fp32.  Inactive rows
  // and heads past H load zeros (zero weight, zero query: no contribution).
  __device__ __forceinline__ void load_row(int rr, const uint16_t* __restrict__ qrow,
                                           const float* __restrict__ wrow, int H, bool active) {
    const int lane = lane_id();
    const int c = lane & 31, g = lane >> 5;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int h = 32 * m + c;
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        if (active && h < H) {
          qf[rr][m][j] =
              *reinterpret_cast<const bf16x8*>(qrow + (int64_t)h * D + g * (D / 2) + 8 * j);
        } else {
          qf[rr][m][j] = bf16x8{};
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hw = 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
        wv[rr][m][r] = (active && hw < H) ? wrow[hw] : 0.0f;
      }
    }
  }

  // LDS bytes load_row_staged needs: the padded query row as a tile of HP
  // key-row slots (the key tiles' layout).
  static constexpr int kStageBytes = HP * G::kRowBytes;

  // load_row through LDS.  Each fragment load instruction of load_row
  // gathers 16 bytes from each of 64 head rows, so it requests 64 cache
  // lines, and the 8 k-steps request each line again.  Here each load
  // instruction reads 64 consecutive 16-byte chunks of the row (whole cache
  // lines), the chunks go to `stage` (kStageBytes of LDS private to the
  // wavefront, free until the caller reuses it) in the key tiles' layout,
  // and the fragments are read back from there, conflict-free under that
  // layout's swizzle.  The weights are read as 16-byte groups of 4 heads when
  // `w4` holds (H a multiple of 4 and wrow 16-byte aligned).
  __device__ __forceinline__ void load_row_staged(int rr, const uint16_t* __restrict__ qrow,
                                                  const float* __restrict__ wrow, int H,
                                                  bool active, bool w4, lds_char* stage) {
    const int lane = lane_id();
    const int g = lane >> 5;
    constexpr int kCh = D / 8;
    constexpr int kPer = HP * kCh / kWave;
    u32x4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = i * kWave + lane;
      const int h = ch / kCh, x = ch % kCh;
      v[i] = (active && h < H) ? *reinterpret_cast<const u32x4*>(qrow + (int64_t)h * D + 8 * x)
                               : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (w4) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int h0 = 32 * m + 8 * a + 4 * g;
          const floatx4 f = (active && h0 < H) ? *reinterpret_cast<const floatx4*>(wrow + h0)
                                               : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) wv[rr][m][4 * a + e] = f[e];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int hw = 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
          wv[rr][m][r] = (active && hw < H) ? wrow[hw] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = i * kWave + lane;
      *reinterpret_cast<DSAI_LDS u32x4*>(stage + G::chunk_offset(ch / kCh, ch % kCh)) = v[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < KS; ++j)
        qf[rr][m][j] = *reinterpret_cast<const DSAI_LDS bf16x8*>(stage + 32 * m * G::kRowBytes +
                                                                 frag_offset(j));
  }

  // One-row form (NR == 1).
  __device__ __forceinline__ void load_query(const uint16_t* __restrict__ qrow,
                                             const float* __restrict__ wrow, int H, bool active) {
    init_offsets();
    load_row(0, qrow, wrow, H, active);
  }

  using Frag = bf16x8[KS];

  // This lane's key fragments of a staged tile (LDS reads only), so a caller
  // can fetch the next tile while the current one is on the matrix cores.
  __device__ __forceinline__ void fetch(const lds_char* tile, Frag& bf) const {
#pragma unroll
    for (int j = 0; j < KS; ++j) bf[j] = *reinterpret_cast<const DSAI_LDS bf16x8*>(tile + frag_offset(j));
  }

  // Products of a tile's 32 keys (fragments from fetch()) with the query
  // heads, on the matrix cores: acc[rr][m] holds row rr's M-tile m (lane
  // (c, g): key c, 16 heads).  reduce() consumes the result, so a caller can
  // overlap one tile's reduction with the next tile's products.
  __device__ __forceinline__ void mma(const Frag& bf, Acc& acc) const {
#pragma unroll
    for (int rr = 0; rr < NR; ++rr)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[rr][m] = floatx16{};
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int rr = 0; rr < NR; ++rr)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[rr][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[rr][m][j], bf[j], acc[rr][m], 0, 0, 0);
  }

  // mma() with a rolling fragment buffer: once k-step j's products have been
  // issued, bf[j] is refilled with k-step j of the tile at `next`, so the next
  // tile's reads overlap this tile's remaining products and one set of
  // fragment registers serves both tiles.
  __device__ __forceinline__ void mma_fetch(Frag& bf, const lds_char* next, Acc& acc) const {
#pragma unroll
    for (int rr = 0; rr < NR; ++rr)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[rr][m] = floatx16{};
#pragma unroll
    for (int j = 0; j < KS; ++j) {
#pragma unroll
      for (int rr = 0; rr < NR; ++rr)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[rr][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[rr][m][j], bf[j], acc[rr][m], 0, 0, 0);
      bf[j] = *reinterpret_cast<const DSAI_LDS bf16x8*>(next + frag_offset(j));
    }
  }

  // The last kSpare k-steps of each tile read a second set of fragment
  // registers, one set per tile parity.
  static constexpr int kSpare = KS >= 4 ? 2 : 1;
  using Spare = bf16x8[kSpare];

  // mma_fetch with the last kSpare k-steps double-buffered: the next tile's
  // fragments for those k-steps go into `spare_next` before this tile's
  // first product (its registers were last read by the previous tile's
  // products), so the step's last LDS read is issued kSpare k-steps before
  // its last product and has landed by the barrier that follows.
  __device__ __forceinline__ void mma_fetch_spare(Frag& bf, const Spare& spare_cur, Spare& spare_next,
                                                  const lds_char* next, Acc& acc) const {
#pragma unroll
    for (int rr = 0; rr < NR; ++rr)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[rr][m] = floatx16{};
#pragma unroll
    for (int s = 0; s < kSpare; ++s)
      spare_next[s] = *reinterpret_cast<const DSAI_LDS bf16x8*>(next + frag_offset(KS - kSpare + s));
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const bf16x8 b = j < KS - kSpare ? bf[j] : spare_cur[j - (KS - kSpare)];
#pragma unroll
      for (int rr = 0; rr < NR; ++rr)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[rr][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[rr][m][j], b, acc[rr][m], 0, 0, 0);
      if (j < KS - kSpare) bf[j] = *reinterpret_cast<const DSAI_LDS bf16x8*>(next + frag_offset(j));
    }
  }

  // fetch() for mma_fetch_spare: k-steps before the last kSpare into bf,
  // the last kSpare into spare.
  __device__ __forceinline__ void fetch_spare(const lds_char* tile, Frag& bf, Spare& spare) const {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const bf16x8 v = *reinterpret_cast<const DSAI_LDS bf16x8*>(tile + frag_offset(j));
      if (j < KS - kSpare) bf[j] = v;
      else spare[j - (KS - kSpare)] = v;
    }
  }

  __device__ __forceinline__ void mma(const lds_char* tile, Acc& acc) const {
    Frag bf;
    fetch(tile, bf);
    mma(bf, acc);
  }

  // ReLU, head weights and the sum over heads of row rr's products: the full
  // score of key lane % 32, in lanes l and l + 32 (four partial sums keep the
  // dependency chains short enough to interleave with matrix-core work).
  __device__ __forceinline__ float reduce(const Acc& acc, int rr) const {
    return combine(reduce_half(acc, rr));
  }

  // The part of reduce() over this lane's 16 heads per M-tile (lanes l and
  // l + 32 hold the two halves of key l % 32's heads) ...
  __device__ __forceinline__ float reduce_half(const Acc& acc, int rr) const {
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r & 3] = fmaf(wv[rr][m][r], fmaxf(acc[rr][m][r], 0.f), p[r & 3]);
    return (p[0] + p[1]) + (p[2] + p[3]);
  }

  // ... and the cross-half sum that completes it.  v_permlane32_swap trades
  // the upper half-wave of one copy for the lower half-wave of the other, so
  // r[0] + r[1] is (lane l % 32's half) + (lane l % 32 + 32's half) in every
  // lane (same operand order in both halves: identical bits), with no LDS
  // round trip.
  static __device__ __forceinline__ float combine(float half) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(half), __float_as_uint(half),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }

  // combine() of two tiles at once: lanes 0-31 get tile a's scores (key
  // l), lanes 32-63 tile b's (key l - 32), each with the operands in the
  // order combine() adds them (identical bits).
  static __device__ __forceinline__ float combine2(float half_a, float half_b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(half_a), __float_as_uint(half_b),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }

  // Full score of key `lane % 32` of the staged tile (in lanes l and l + 32).
  __device__ __forceinline__ float score(const lds_char* tile) const {
    Acc acc;
    mma(tile, acc);
    return reduce(acc, 0);
  }
};

}  // namespace dsai
