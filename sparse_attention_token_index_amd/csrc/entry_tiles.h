// A row of supplied key indices, walked 32 entries at a time with the key
// rows gathered into the fused indexer's fragment layout.  Used where a row
// names its keys explicitly: scores at supplied indices (the topk_indices
// form of the indexer) and the gradients of the selected scores.
#pragma once

#include "device_common.h"

namespace dsai {

// Entries j0 .. j0 + 31 of a row as loaded (lane c and c + 32: entry
// j0 + c): key and, with kGrad, incoming gradient.  The loads are clamped to
// the row's last entry and never skipped, so a loop that prefetches with
// them issues the same loads on every path and the compiler's wait counts
// stay exact; usability is decided when the tile is taken.
template <bool kGrad>
struct EntryIdx {
  int sv;
  float gv;
  bool in;  // j0 + c < n

  __device__ __forceinline__ void load(const int32_t* sup, const float* __restrict__ grad,
                                       int64_t orow, int n, int j0) {
    const int j = j0 + (lane_id() & 31);
    in = j < n;
    const int64_t e = orow + min(j, n - 1);
    sv = sup[e];
    gv = kGrad ? grad[e] : 0.f;
  }
};

// One 32-entry tile of a row: lane (c, g) holds entry c's key (-1 when not
// usable), incoming gradient (0 when not usable) and that key's fragments
// for the forward's tile layout (dims g*D/2 + 8x, x < D/16).  An unusable
// entry reads key 0 (the row sees at least one key, so it exists) and is
// discarded.
template <int D, bool kGrad>
struct EntryTile {
  int s;
  float g;
  bf16x8 f[D / 16];

  __device__ __forceinline__ void take(const EntryIdx<kGrad>& e, const uint16_t* __restrict__ k,
                                       int n_t, int B, int b) {
    const bool ok = e.in && e.sv >= 0 && e.sv < n_t;
    s = ok ? e.sv : -1;
    g = ok ? e.gv : 0.f;
    const uint16_t* src = k + ((int64_t)(ok ? e.sv : 0) * B + b) * D + (lane_id() >> 5) * (D / 2);
#pragma unroll
    for (int x = 0; x < D / 16; ++x) f[x] = *reinterpret_cast<const bf16x8*>(src + 8 * x);
  }
};

// Software pipeline over a row's ngroups >= 1 tiles of 32 entries (the row
// sees n_t >= 1 keys): while tile i is worked on by body(tile, i), the key
// rows of tile i + 1 and the indices of tile i + 2 are in flight.  Past the
// row's end the prefetches repeat its last tile, so every step issues the
// same loads, and the wait before a step covers only loads issued one step
// earlier.  Two register sets alternate, so no tile is copied.  The
// prefetches of tiles i + 1 and i + 2 are issued before body writes tile i's
// outputs, so `sup` may be the array body writes (in place).
template <int D, bool kGrad, class Body>
__device__ __forceinline__ void for_each_entry_tile(const int32_t* sup,
                                                    const float* __restrict__ grad,
                                                    const uint16_t* __restrict__ k, int64_t orow,
                                                    int n, int n_t, int B, int b, int ngroups,
                                                    Body&& body) {
  EntryTile<D, kGrad> ta, tb;
  EntryIdx<kGrad> ahead;
  ahead.load(sup, grad, orow, n, 0);
  ta.take(ahead, k, n_t, B, b);
  ahead.load(sup, grad, orow, n, min(1, ngroups - 1) * 32);
  auto step = [&](EntryTile<D, kGrad>& cur, EntryTile<D, kGrad>& nxt, int it) {
    nxt.take(ahead, k, n_t, B, b);
    ahead.load(sup, grad, orow, n, min(it + 2, ngroups - 1) * 32);
    body(cur, it);
  };
  for (int it = 0; it < ngroups; it += 2) {
    step(ta, tb, it);
    if (it + 1 < ngroups) step(tb, ta, it + 1);
  }
}

}  // namespace dsai
