// Index scores of one query row against a 64-key tile staged in LDS, on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_bf16), fused with ReLU and the
// weighted reduction over heads.
//
// Score of key s for a query row (the lightning-indexer score; per-head
// weights reduce over heads after a per-head ReLU):
//     I[s] = sum_h w[h] * max(0, sum_d q[h, d] * k[s, d])
//
// Mapping: heads are the MFMA M dimension (M-tiles of 16 heads, heads past H
// are zero), keys the N dimension (four 16-key N-blocks per tile) and the
// head dim the K dimension (k-steps of 32).  The reduction index is permuted
// consistently for both operands: lane (c = l % 16, g = l / 16) supplies the
// 8 consecutive dims [32 j + 8 g, 32 j + 8 g + 8) at k-step j, so each operand
// fragment is one 16-byte load.  The accumulator lane (c, g) holds key c of an
// N-block for the 4 heads 4 g .. 4 g + 3 of each M-tile: ReLU, the head
// weights and the sum over M-tiles run in registers, and a 3-shuffle
// reduce-scatter over the four lane groups leaves lane l holding the full
// score of key l of the tile.
#pragma once

#include "device_common.h"

namespace dsai {

// Byte stride of one staged key row in LDS: 16 bytes of padding put the 16
// keys a ds_read_b128 gathers on distinct bank groups.
template <int D>
struct TileGeom {
  static constexpr int kRowBytes = 2 * D + 16;
  static constexpr int kTileKeys = 64;
  static constexpr int kTileBytes = kTileKeys * kRowBytes;
  static constexpr int kChunksPerRow = D / 8;               // 16-byte chunks
  static constexpr int kChunks = kTileKeys * kChunksPerRow;
};

// Stages 64 consecutive key rows (bf16, `row_stride` elements apart) from
// global memory into an LDS tile, through registers so the next tile's loads
// overlap the current tile's math.  Rows at or past `rows_valid` read as zero.
template <int D, int NTHREADS>
struct TileLoader {
  using G = TileGeom<D>;
  static_assert(G::kChunks % NTHREADS == 0, "tile chunks must divide over the block");
  static constexpr int kPer = G::kChunks / NTHREADS;
  u32x4 r[kPer];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t row_stride,
                                       int64_t row0, int64_t rows_valid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = (int)threadIdx.x + i * NTHREADS;
      const int row = ch / G::kChunksPerRow;
      const int part = ch % G::kChunksPerRow;
      const int64_t s = row0 + row;
      if (s < rows_valid) {
        r[i] = *reinterpret_cast<const u32x4*>(base + s * row_stride + part * 8);
      } else {
        r[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ __forceinline__ void store(lds_char* tile) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = (int)threadIdx.x + i * NTHREADS;
      const int row = ch / G::kChunksPerRow;
      const int part = ch % G::kChunksPerRow;
      *reinterpret_cast<DSAI_LDS u32x4*>(tile + row * G::kRowBytes + part * 16) = r[i];
    }
  }
};

template <int HP, int D>
struct TileScorer {
  static_assert(HP % 16 == 0 && HP >= 16 && HP <= 64, "padded heads: 16, 32, 48 or 64");
  static_assert(D % 32 == 0 && D >= 32 && D <= 128, "head dim: 32, 64, 96 or 128");
  static constexpr int MT = HP / 16;
  static constexpr int KS = D / 32;
  using G = TileGeom<D>;

  bf16x8 qf[MT][KS];
  float wv[MT][4];

  // qrow: [H, D] bf16 of this query row; wrow: [H] fp32.  Inactive rows and
  // heads past H load zeros (zero weight, zero query: no contribution).
  __device__ __forceinline__ void load_query(const uint16_t* __restrict__ qrow,
                                             const float* __restrict__ wrow, int H, bool active) {
    const int lane = lane_id();
    const int c = lane & 15, g = lane >> 4;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int h = 16 * m + c;
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        if (active && h < H) {
          qf[m][j] = *reinterpret_cast<const bf16x8*>(qrow + (int64_t)h * D + 32 * j + 8 * g);
        } else {
          qf[m][j] = bf16x8{};
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hw = 16 * m + 4 * g + i;
        wv[m][i] = (active && hw < H) ? wrow[hw] : 0.0f;
      }
    }
  }

  // Full score of key `lane` of the staged tile.
  __device__ __forceinline__ float score(const lds_char* tile) const {
    const int lane = lane_id();
    const int c = lane & 15, g = lane >> 4;
    floatx4 acc[4][MT];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[nb][m] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int j = 0; j < KS; ++j) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8 b = *reinterpret_cast<const DSAI_LDS bf16x8*>(
            tile + (nb * 16 + c) * G::kRowBytes + (32 * j + 8 * g) * 2);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[m][j], b, acc[nb][m], 0, 0, 0);
      }
    }

    float p[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(wv[m][i], fmaxf(acc[nb][m][i], 0.f), s);
      p[nb] = s;
    }

    // Reduce-scatter over the lane groups g = 0..3: lane group g ends with the
    // total of N-block g (key 16 g + c = lane).
    const bool h1 = (g >> 1) & 1, h0 = g & 1;
    const float keep0 = h1 ? p[2] : p[0], keep1 = h1 ? p[3] : p[1];
    const float send0 = h1 ? p[0] : p[2], send1 = h1 ? p[1] : p[3];
    const float q0 = keep0 + __shfl_xor(send0, 32);
    const float q1 = keep1 + __shfl_xor(send1, 32);
    const float keep = h0 ? q1 : q0, send = h0 ? q0 : q1;
    return keep + __shfl_xor(send, 16);
  }
};

}  // namespace dsai
