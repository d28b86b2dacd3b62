// Wave-level top-k selection over an LDS candidate store (gfx950, wave64).
//
// One wavefront owns one output row.  Candidates are (key, idx) pairs where
// `key` is the order-preserving uint32 image of an fp32 score (ord_key) and
// `idx` the key/pool index (uint16 when every index fits, else uint32).
// Candidates enter the store in ascending index order and every step below
// keeps that order, so "lower index first among equal scores" needs no
// composite key:
//
//   wave_append        ballot + prefix count: appends the passing lanes in
//                      lane order after the current entries.
//   wave_radix_select  radix select of the k-th largest key value v and how
//                      many entries equal to v belong to the top k: a min/max
//                      pass, a 256-bin pass over the key range, then 8-bit
//                      passes inside the chosen bin.  Loads are batched and
//                      the histogram atomics return nothing.
//   wave_compact       stable in-place compaction to exactly the top k.
//   wave_emit          stable selection of the top k written straight to the
//                      output row (index order), then (-1, -inf) padding.
//
// All functions are called by every lane of the wave with wave-uniform scalar
// arguments.
#pragma once

#include "device_common.h"

namespace dsai {

template <typename IdxT>
struct RowStore {
  lds_u32* key;                       // [cap] order keys
  DSAI_LDS IdxT* idx;                 // [cap] indices
  lds_u32* hist;                      // [256] radix-select histogram (wave-private)
  lds_u32* side;                      // [side_cap] scratch keys for the select
  uint32_t side_cap;
};

__device__ __forceinline__ uint32_t uniform(uint32_t x) {
  return __builtin_amdgcn_readfirstlane(x);
}

template <typename IdxT>
__device__ __forceinline__ void wave_append(const RowStore<IdxT>& rs, uint32_t& count, bool pass,
                                            uint32_t u, uint32_t id) {
  const uint64_t m = ballot(pass);
  if (pass) {
    const uint32_t p = count + lanes_below(m);
    rs.key[p] = u;
    rs.idx[p] = (IdxT)id;
  }
  count = uniform(count + (uint32_t)__popcll(m));
}

// wave_append with no branch, so the compiler can interleave it with other
// work: every lane stores, the passing lanes after the current entries in
// lane order and the others into the slots right after those (slots past the
// count hold nothing), so the store needs 64 free slots past `count`.
template <typename IdxT>
__device__ __forceinline__ void wave_append_all(const RowStore<IdxT>& rs, uint32_t& count,
                                                bool pass, uint32_t u, uint32_t id) {
  const uint64_t m = ballot(pass);
  const uint32_t below = lanes_below(m);
  const uint32_t np = (uint32_t)__popcll(m);
  const uint32_t p = count + (pass ? below : np + (uint32_t)lane_id() - below);
  rs.key[p] = u;
  rs.idx[p] = (IdxT)id;
  count = uniform(count + np);
}

// LDS bytes per wavefront for the select: a 256-bin histogram and a 256-key
// side list.
constexpr int kSelScratchBytes = 2048;

// Keys per lane handled per batch of the store-scanning loops.
constexpr int kSelBatch = 8;

// Bin b (of 256) of the k-th largest key among `cnt` keys whose histogram
// sits in hist[0..255] (lane L owns bins 4L..4L+3); .y = number of keys in
// bins above b, so rank k falls at position k - .y inside bin b.
__device__ __forceinline__ uint2 find_bin(lds_u32* hist, uint32_t rem) {
  const int lane = lane_id();
  const u32x4 c = *reinterpret_cast<const DSAI_LDS u32x4*>(&hist[4 * lane]);
  const uint32_t s = c.x + c.y + c.z + c.w;
  const uint32_t a3 = wave_incl_suffix(s) - s;
  const uint32_t a2 = a3 + c.w, a1 = a2 + c.z, a0 = a1 + c.y;
  int found = -1;
  uint32_t above = 0u;
  if (a3 < rem && rem <= a3 + c.w) {
    found = 3; above = a3;
  } else if (a2 < rem && rem <= a2 + c.z) {
    found = 2; above = a2;
  } else if (a1 < rem && rem <= a1 + c.y) {
    found = 1; above = a1;
  } else if (a0 < rem && rem <= a0 + c.x) {
    found = 0; above = a0;
  }
  const uint64_t fm = ballot(found >= 0);
  const int src = (int)__ffsll((unsigned long long)fm) - 1;
  return make_uint2(lane_value((uint32_t)(4 * lane + found), src), lane_value(above, src));
}

__device__ __forceinline__ void clear_hist(lds_u32* hist) {
  const int lane = lane_id();
  *reinterpret_cast<DSAI_LDS u32x4*>(&hist[4 * lane]) = u32x4{0u, 0u, 0u, 0u};
  wave_lds_sync();
}

__device__ __forceinline__ void hist_add(lds_u32* hist, uint32_t bin) {
  __hip_atomic_fetch_add(&hist[bin], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// hist_add for lanes where `in` holds.  The branch is deliberate: behind it
// the compiler waits for each atomic before issuing the next, and that is
// faster here than straight-line atomics going out back to back (the keys
// of a store crowd into few bins; measured: a cut took 45K cycles with
// back-to-back atomics against 27K with this form).
__device__ __forceinline__ void hist_add_if(lds_u32* hist, uint32_t bin, bool in) {
  if (in) __hip_atomic_fetch_add(&hist[bin], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// Entry i of a store of n >= 1 entries, or entry 0 for i past the end (a
// load with no branch; the caller ignores those lanes).
__device__ __forceinline__ uint32_t load_clamped(const lds_u32* key, uint32_t i, uint32_t n) {
  return key[i < n ? i : 0u];
}

// One 64-entry chunk of an in-place compaction, with no branch: the kept
// lanes go to wpos.. in lane order, every other lane into the slots right
// after them (below wpos + 64: entries this pass has already read, since a
// chunk keeps at most what it read; the caller runs no chunk that starts
// past the store's entries, so those slots lie below the entry count
// rounded up to 64, within a store whose capacity is a multiple of 64).
template <typename IdxT>
__device__ __forceinline__ void compact_put(const RowStore<IdxT>& rs, uint32_t& wpos, bool keep,
                                            uint32_t u, uint32_t x) {
  const uint64_t mk = ballot(keep);
  const uint32_t below = lanes_below(mk);
  const uint32_t nk = (uint32_t)__popcll(mk);
  const uint32_t p = wpos + (keep ? below : nk + (uint32_t)lane_id() - below);
  rs.key[p] = u;
  rs.idx[p] = (IdxT)x;
  wpos = uniform(wpos + nk);
}

__device__ __forceinline__ uint32_t sat_add(uint32_t a, uint32_t b) {
  return a > 0xFFFFFFFFu - b ? 0xFFFFFFFFu : a + b;
}

// Radix select over a key range: finds the k-th largest of the keys in
// `key[0, n)` that lie in [lo, hi] (hi - lo < 2^bits; `m` of them, k <= m),
// resolving `bits` low bits 8 at a time with histograms of (u - lo) digits.
// FLOAT_KEYS: key[] holds fp32 scores (bits), mapped to order keys on load.
template <bool FLOAT_KEYS = false>
__device__ __forceinline__ uint2 select_in_range(const lds_u32* key, uint32_t n, lds_u32* hist,
                                                 uint32_t lo, uint32_t hi, int bits, uint32_t rem) {
  const int lane = lane_id();
  while (bits > 0) {
    const int shift = bits > 8 ? bits - 8 : 0;
    clear_hist(hist);
    for (uint32_t base = 0; base < n; base += kWave * kSelBatch) {
      uint32_t u[kSelBatch];
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) {
        u[j] = load_clamped(key, base + j * kWave + lane, n);
        if constexpr (FLOAT_KEYS) u[j] = ord_key(__uint_as_float(u[j]));
      }
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) {
        const uint32_t i = base + j * kWave + lane;
        hist_add_if(hist, (u[j] - lo) >> shift, (i < n) & (u[j] >= lo) & (u[j] <= hi));
      }
    }
    wave_lds_sync();
    const uint2 fb = find_bin(hist, rem);
    lo += fb.x << shift;
    rem -= fb.y;
    bits = shift;
    if (shift > 0 && hi - lo > (1u << shift) - 1u) hi = lo + ((1u << shift) - 1u);
    wave_lds_sync();
  }
  return make_uint2(lo, rem);
}

// k-th largest key value v among key[0, n), 1 <= k <= n (.x), and the number
// of entries equal to v that belong to the top k (.y).
//
// Pass 1 bins the keys by (u - min) scaled so the key range spans 256 bins,
// which spreads the histogram atomics over many addresses (raw high bytes of
// similar scores would all hit the same few bins).  The chosen bin is then
// resolved 8 bits at a time; when it holds few keys they are first copied to
// a side list so later passes touch only them.
__device__ __noinline__ uint2 wave_radix_select(lds_u32* key, lds_u32* hist, lds_u32* side,
                                                uint32_t side_cap, uint32_t n, uint32_t k) {
  const int lane = lane_id();
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (uint32_t base = 0; base < n; base += kWave * kSelBatch) {
    uint32_t u[kSelBatch];
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) u[j] = load_clamped(key, base + j * kWave + lane, n);
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) {  // lanes past n hold entry 0: no effect
      mn = min(mn, u[j]);
      mx = max(mx, u[j]);
    }
  }
  mn = uniform(wave_min(mn));
  mx = uniform(wave_max(mx));
  const uint32_t range = mx - mn;
  if (range == 0u) return make_uint2(mn, k);  // every key equal
  const int rbits = 32 - __clz(range);        // range < 2^rbits
  const int shift = rbits > 8 ? rbits - 8 : 0;
  clear_hist(hist);
  for (uint32_t base = 0; base < n; base += kWave * kSelBatch) {
    uint32_t u[kSelBatch];
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) u[j] = load_clamped(key, base + j * kWave + lane, n);
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j)
      hist_add_if(hist, (u[j] - mn) >> shift, base + j * kWave + lane < n);
  }
  wave_lds_sync();
  const uint2 fb = find_bin(hist, k);
  const uint32_t cnt_bin = uniform(hist[fb.x]);
  const uint32_t lo = mn + (fb.x << shift);
  uint32_t rem = k - fb.y;
  wave_lds_sync();
  if (shift == 0) return make_uint2(lo, rem);
  const uint32_t width = (1u << shift) - 1u;
  if (cnt_bin <= side_cap) {
    // gather the bin's keys (order is irrelevant for the value search)
    uint32_t nside = 0u;
    for (uint32_t base = 0; base < n; base += kWave) {
      const uint32_t i = base + lane;
      const uint32_t u = i < n ? key[i] : 0u;
      const bool in = i < n && u >= lo && (u - lo) <= width;
      const uint64_t m = ballot(in);
      if (in) side[nside + lanes_below(m)] = u;
      nside = uniform(nside + (uint32_t)__popcll(m));
    }
    wave_lds_sync();
    return select_in_range(side, nside, hist, lo, sat_add(lo, width), shift, rem);
  }
  return select_in_range(key, n, hist, lo, sat_add(lo, width), shift, rem);
}

// Keep, in store order, the entries with key > v and the first `take_eq`
// entries with key == v.  Returns the new count.
template <typename IdxT>
__device__ __noinline__ uint32_t wave_compact(RowStore<IdxT> rs, uint32_t n, uint32_t v,
                                              uint32_t take_eq) {
  const int lane = lane_id();
  uint32_t wpos = 0u, eq_seen = 0u;
  constexpr int kB = 4;
  for (uint32_t base = 0; base < n; base += kWave * kB) {
    uint32_t u[kB], x[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const uint32_t i = base + j * kWave + lane;
      const uint32_t ii = i < n ? i : 0u;
      u[j] = rs.key[ii];
      x[j] = (uint32_t)rs.idx[ii];
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      if (base + j * kWave >= n) break;  // (uniform) no chunk past the entries
      const uint32_t i = base + j * kWave + lane;
      const bool in = i < n;
      const bool eq = in & (u[j] == v);
      const uint64_t meq = ballot(eq);
      const bool keep = (in & (u[j] > v)) | (eq & ((eq_seen + lanes_below(meq)) < take_eq));
      compact_put(rs, wpos, keep, u[j], x[j]);
      eq_seen = uniform(eq_seen + (uint32_t)__popcll(meq));
    }
  }
  wave_lds_sync();
  return wpos;
}

// Keep, in store order, the entries with key >= t.  Returns the new count.
template <typename IdxT>
__device__ __noinline__ uint32_t wave_compact_ge(RowStore<IdxT> rs, uint32_t n, uint32_t t) {
  const int lane = lane_id();
  uint32_t wpos = 0u;
  constexpr int kB = 4;
  for (uint32_t base = 0; base < n; base += kWave * kB) {
    uint32_t u[kB], x[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const uint32_t i = base + j * kWave + lane;
      const uint32_t ii = i < n ? i : 0u;
      u[j] = rs.key[ii];
      x[j] = (uint32_t)rs.idx[ii];
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      if (base + j * kWave >= n) break;  // (uniform) no chunk past the entries
      const uint32_t i = base + j * kWave + lane;
      compact_put(rs, wpos, (i < n) & (u[j] >= t), u[j], x[j]);
    }
  }
  wave_lds_sync();
  return wpos;
}

// Bin-edge cut of a store holding n > k entries: a threshold t such that at
// least k entries have key >= t, found from one 256-bin histogram of the
// keys over [min, max] (and, when the bin holding rank k has more than
// kCutRefine keys, a second histogram inside that bin), then the entries
// with key >= t kept in store order.  Any t no larger than the k-th largest
// key keeps the row's top k; a later key equal to t can never displace one
// of the >= k kept keys (they are at least as large and come first), so t
// becomes the admission threshold (keys must exceed it).  That keeps k plus
// the part of t's bin below rank k - a few dozen entries more than an exact
// cut - for two passes over the store fewer and no side list.  When it would
// keep more than `max_keep` (many equal keys at the boundary), the exact cut
// runs instead (to exactly k, ties to the earlier entries), without a side
// list: `side` may be memory other wavefronts are using.  Returns (entries
// kept, new threshold), so the caller's threshold can stay in a register.
// [lo_bound, hi_bound], when lo_bound is not 0, is a range known to hold
// every key (the previous threshold and a running maximum), which saves the
// min/max pass.
constexpr uint32_t kCutRefine = 64;

template <typename IdxT>
__device__ __noinline__ uint2 wave_cut(RowStore<IdxT> rs, uint32_t n, uint32_t k,
                                       uint32_t max_keep, uint32_t lo_bound, uint32_t hi_bound) {
  const int lane = lane_id();
  wave_lds_sync();
  uint32_t mn = lo_bound, mx = hi_bound;
  if (lo_bound == 0u) {
    mn = 0xFFFFFFFFu;
    mx = 0u;
    for (uint32_t base = 0; base < n; base += kWave * kSelBatch) {
      uint32_t u[kSelBatch];
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) u[j] = load_clamped(rs.key, base + j * kWave + lane, n);
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) {  // lanes past n hold entry 0: no effect
        mn = min(mn, u[j]);
        mx = max(mx, u[j]);
      }
    }
  }
  const uint32_t lo = uniform(wave_min(mn));
  mx = uniform(wave_max(mx));
  const uint32_t range = mx - lo;
  uint32_t t = lo, kept = n;
  if (range != 0u) {
    const int rbits = 32 - __clz(range);
    const int shift = rbits > 8 ? rbits - 8 : 0;
    clear_hist(rs.hist);
    for (uint32_t base = 0; base < n; base += kWave * kSelBatch) {
      uint32_t u[kSelBatch];
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) u[j] = load_clamped(rs.key, base + j * kWave + lane, n);
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j)
        hist_add_if(rs.hist, (u[j] - lo) >> shift, base + j * kWave + lane < n);
    }
    wave_lds_sync();
    const uint2 fb = find_bin(rs.hist, k);
    const uint32_t cnt_bin = uniform(rs.hist[fb.x]);
    t = lo + (fb.x << shift);
    kept = fb.y + cnt_bin;
    wave_lds_sync();
    if (cnt_bin > kCutRefine && shift > 0) {
      // second round inside the bin: 8 more bits (or all that remain)
      const int shift2 = shift > 8 ? shift - 8 : 0;
      const uint32_t bin_hi = t + ((1u << shift) - 1u);  // no wrap: bin b lies in [lo, mx]
      clear_hist(rs.hist);
      for (uint32_t base = 0; base < n; base += kWave * kSelBatch) {
        uint32_t u[kSelBatch];
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) u[j] = load_clamped(rs.key, base + j * kWave + lane, n);
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
          const uint32_t i = base + j * kWave + lane;
          hist_add_if(rs.hist, (u[j] - t) >> shift2, (i < n) & (u[j] >= t) & (u[j] <= bin_hi));
        }
      }
      wave_lds_sync();
      const uint2 fb2 = find_bin(rs.hist, k - fb.y);
      t += fb2.x << shift2;
      kept = fb.y + fb2.y + uniform(rs.hist[fb2.x]);
      wave_lds_sync();
    }
  }
  if (kept > max_keep) {
    const uint2 sel = wave_radix_select(rs.key, rs.hist, rs.side, 0u, n, k);
    return make_uint2(wave_compact(rs, n, sel.x, sel.y), sel.x);
  }
  return make_uint2(wave_compact_ge(rs, n, t), t);
}

// Reduce the store to its top k (stable) if it holds more than k entries;
// *tau receives the k-th largest key (the new admission threshold).
template <typename IdxT>
__device__ __forceinline__ uint32_t wave_keep_topk(const RowStore<IdxT>& rs, uint32_t count,
                                                   uint32_t k, uint32_t* tau) {
  if (count <= k) return count;
  wave_lds_sync();
  const uint2 sel = wave_radix_select(rs.key, rs.hist, rs.side, rs.side_cap, count, k);
  *tau = sel.x;
  return wave_compact(rs, count, sel.x, sel.y);
}

// Write the row's top k in index order: the store's entries with key > v and
// the first `take_eq` entries with key == v (v = 0, take_eq = 0 keeps every
// entry: real keys are never 0), followed by (-1, -inf) up to `topk` slots.
template <typename IdxT>
__device__ __noinline__ void wave_emit(RowStore<IdxT> rs, uint32_t n, uint32_t v, uint32_t take_eq,
                                       int topk, int32_t* __restrict__ out_idx,
                                       float* __restrict__ out_score) {
  const int lane = lane_id();
  uint32_t wpos = 0u, eq_seen = 0u;
  for (uint32_t base = 0; base < n; base += kWave) {
    const uint32_t i = base + lane;
    const bool in = i < n;
    const uint32_t u = in ? rs.key[i] : 0u;
    const uint32_t x = in ? (uint32_t)rs.idx[i] : 0u;
    const bool eq = in && (u == v);
    const uint64_t meq = ballot(eq);
    const bool keep = (in && u > v) || (eq && (eq_seen + lanes_below(meq)) < take_eq);
    const uint64_t mk = ballot(keep);
    if (keep) {
      const uint32_t p = wpos + lanes_below(mk);
      out_idx[p] = (int32_t)x;
      out_score[p] = ord_to_float(u);
    }
    wpos = uniform(wpos + (uint32_t)__popcll(mk));
    eq_seen = uniform(eq_seen + (uint32_t)__popcll(meq));
  }
  for (uint32_t p = wpos + lane; p < (uint32_t)topk; p += kWave) {
    out_idx[p] = -1;
    out_score[p] = -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// Dense rows: key[i] is the order key of index i for i < n, the store is a
// multiple of 256 entries and 16-byte aligned.  Everything here is inlined so
// the row size and k stay scalar (uniform loops, no divergent bookkeeping).
// ---------------------------------------------------------------------------

// Float-linear histogram bin (0..255) of a score in the candidate range
// [a, b]: monotone non-decreasing in the score (halving, subtraction,
// scaling and the clamp are each monotone under round-to-nearest), so the
// bins partition [a, b] into consecutive intervals.  Halving keeps the
// difference of any two finite scores finite.
struct FloatBins {
  float base_h, scale;
  __device__ __forceinline__ FloatBins(float a, float b) {
    base_h = 0.5f * a;
    const float span = 0.5f * b - base_h;
    scale = span > 0.f ? fminf(256.f / span, 3.4e38f) : 0.f;
  }
  __device__ __forceinline__ uint32_t operator()(float x) const {
    const float d = __fmul_rn(__fsub_rn(__fmul_rn(0.5f, x), base_h), scale);
    return (uint32_t)fminf(fmaxf(d, 0.f), 255.f);
  }
};

// Dense row store: slot s holds the fp32 score of key s (-0 stored as +0,
// so equal scores have equal bits).  Slots up to the next multiple of 256 are
// readable.

// The dense store's final phase works on groups of 64 consecutive keys, key
// 64 g + lane in lane `lane`, four groups (one 256-key group of the store,
// which holds whole 256-key groups) at a time.  The phase runs beside the
// other wavefront of the SIMD, which is in its key loop, so it is bound by
// its own instruction count: a group's kept keys are placed by one ballot
// and the count of kept lanes below, with the running position in a scalar
// register (no wave scan); loads take immediate offsets from one address
// (no clamp: only the row's last 256 keys are masked); lanes that store
// nothing store to a dummy LDS word or with an offset past the output row's
// buffer range (the hardware drops such a store), so no group has a branch.
constexpr uint32_t kFinBatch = 4;

// Byte offset that puts a buffer store past any output row's range.
constexpr int kDropOffset = 0x7FFFFFF0;

// Scores of the 256 keys from slot `base` (a multiple of 256, below the
// store's capacity).
__device__ __forceinline__ void dense_load_batch(const lds_u32* key, uint32_t base,
                                                 float (&x)[kFinBatch]) {
  const lds_u32* p = key + base + (uint32_t)lane_id();
#pragma unroll
  for (uint32_t j = 0; j < kFinBatch; ++j) x[j] = __uint_as_float(p[j * kWave]);
}

// An output row of `topk` entries as two buffer resources whose range is
// the row, so a store with kDropOffset writes nothing.
struct RowOut {
  __amdgpu_buffer_rsrc_t idx, score;
  __device__ __forceinline__ RowOut(int32_t* out_idx, float* out_score, int topk) {
    idx = __builtin_amdgcn_make_buffer_rsrc((void*)out_idx, (short)0, topk * 4, 0x00020000);
    score = __builtin_amdgcn_make_buffer_rsrc((void*)out_score, (short)0, topk * 4, 0x00020000);
  }
  // entry p (dropped when `keep` is false)
  __device__ __forceinline__ void put(bool keep, uint32_t p, int32_t id, float x) const {
    const int off = keep ? (int)(p * 4u) : kDropOffset;
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)id, idx, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), score, off, 0, 0);
  }
};

// FloatBins with the clamp as one median instruction.
__device__ __forceinline__ uint32_t bin_of(const FloatBins& bins, float x) {
  const float d = __fmul_rn(__fsub_rn(__fmul_rn(0.5f, x), bins.base_h), bins.scale);
  return (uint32_t)__builtin_amdgcn_fmed3f(d, 0.f, 255.f);
}

// Histogram of the row's n scores over `bins` (level 0: every key counts).
__device__ __forceinline__ void dense_hist_all(const lds_u32* key, uint32_t n,
                                               const FloatBins& bins, lds_u32* hist) {
  const uint32_t lane = (uint32_t)lane_id();
  const uint32_t nfull = n & ~255u;
  for (uint32_t base = 0; base < nfull; base += kWave * kFinBatch) {
    float x[kFinBatch];
    dense_load_batch(key, base, x);
#pragma unroll
    for (uint32_t j = 0; j < kFinBatch; ++j)
      __hip_atomic_fetch_add(&hist[bin_of(bins, x[j])], 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WAVEFRONT);
  }
  if (nfull < n) {
    float x[kFinBatch];
    dense_load_batch(key, nfull, x);
#pragma unroll
    for (uint32_t j = 0; j < kFinBatch; ++j) {
      // lanes past the row add 0 to a bin of their own (no conflict)
      const bool in = nfull + j * kWave + lane < n;
      __hip_atomic_fetch_add(&hist[in ? bin_of(bins, x[j]) : lane], in ? 1u : 0u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    }
  }
}

// Gather the scores of bin `fb` into side[] (order irrelevant); the other
// lanes write to hist[lane] (no longer read).  Returns the count.
__device__ __forceinline__ uint32_t dense_gather_all(const lds_u32* key, uint32_t n,
                                                     const FloatBins& bins, uint32_t fb,
                                                     lds_u32* hist, lds_u32* side) {
  const uint32_t lane = (uint32_t)lane_id();
  uint32_t ns = 0u;
  for (uint32_t base = 0; base < n; base += kWave * kFinBatch) {
    float x[kFinBatch];
    dense_load_batch(key, base, x);
#pragma unroll
    for (uint32_t j = 0; j < kFinBatch; ++j) {
      const bool inb = (base + j * kWave + lane < n) & (bin_of(bins, x[j]) == fb);
      const uint64_t m = ballot(inb);
      *(inb ? &side[ns + lanes_below(m)] : &hist[lane]) = __float_as_uint(x[j]);
      ns = uniform(ns + (uint32_t)__popcll(m));
    }
  }
  return ns;
}

// The k-th largest score among the dense row's n > k scores (as fp32 bits,
// .x), how many scores equal to it belong to the top k (.y), and 1 in .z
// when that is every score equal to it (the top k is then exactly the
// scores >= .x).  [smin, smax]: the row's smallest and largest score.
// Histograms over float-linear bins of the candidate range spread a row's
// scores evenly, so the bin holding rank k usually has a few dozen keys:
// they are gathered into the side list and, up to 64 of them, each lane
// ranks one against the others (count greater, count equal); up to 256 go
// through a radix select.  A bin with more than 256 keys narrows the range
// to that bin and repeats; after three levels the exact radix select over
// the whole row finishes the search.
__device__ __forceinline__ uint3 dense_select(const lds_u32* key, uint32_t n, uint32_t k,
                                              float smin, float smax, lds_u32* hist,
                                              lds_u32* side) {
  const uint32_t lane = (uint32_t)lane_id();
  float a = smin, b = smax;
  uint32_t rem = k;
  for (int level = 0; level < 3; ++level) {
    if (!(a < b)) return make_uint3(__float_as_uint(a), rem, 0u);
    const FloatBins bins(a, b);
    const bool lvl0 = level == 0;  // [a, b] is the row's range: every key counts
    clear_hist(hist);
    if (lvl0) {
      dense_hist_all(key, n, bins, hist);
    } else {
      for (uint32_t base = 0; base < n; base += kWave * kFinBatch) {
        float x[kFinBatch];
        dense_load_batch(key, base, x);
#pragma unroll
        for (uint32_t j = 0; j < kFinBatch; ++j) {
          const bool in = (base + j * kWave + lane < n) & (x[j] >= a) & (x[j] <= b);
          __hip_atomic_fetch_add(&hist[in ? bin_of(bins, x[j]) : lane], in ? 1u : 0u,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        }
      }
    }
    wave_lds_sync();
    const uint2 fb = find_bin(hist, rem);
    const uint32_t cnt = uniform(hist[fb.x]);
    rem -= fb.y;  // rank inside the bin: 1 <= rem <= cnt
    wave_lds_sync();
    if (cnt <= 256u) {
      // gather the bin's scores into the side list (order is irrelevant);
      // the other lanes write to the histogram, which is no longer read
      // (the paths below clear it before they use it)
      uint32_t ns = 0u;
      if (lvl0) {
        ns = dense_gather_all(key, n, bins, fb.x, hist, side);
      } else {
        for (uint32_t base = 0; base < n; base += kWave * kFinBatch) {
          float x[kFinBatch];
          dense_load_batch(key, base, x);
#pragma unroll
          for (uint32_t j = 0; j < kFinBatch; ++j) {
            const bool inb = (base + j * kWave + lane < n) & (x[j] >= a) & (x[j] <= b) &
                             (bin_of(bins, x[j]) == fb.x);
            const uint64_t m = ballot(inb);
            *(inb ? &side[ns + lanes_below(m)] : &hist[lane]) = __float_as_uint(x[j]);
            ns = uniform(ns + (uint32_t)__popcll(m));
          }
        }
      }
      wave_lds_sync();
      if (ns <= (uint32_t)kWave) {
        // lane L ranks side entry L against all of them
        const bool own = lane < ns;
        const float o = __uint_as_float(side[own ? lane : 0u]);
        const DSAI_LDS u32x4* s4 = reinterpret_cast<const DSAI_LDS u32x4*>(side);
        uint32_t gt = 0u, eq = 0u;
#pragma unroll 4
        for (uint32_t j = 0; j < ns; j += 4u) {
          const u32x4 s = s4[j >> 2];  // the same address in every lane
#pragma unroll
          for (uint32_t e = 0; e < 4u; ++e) {
            const float y = __uint_as_float(s[e]);
            const bool ok = j + e < ns;
            gt += (ok & (y > o)) ? 1u : 0u;
            eq += (ok & (y == o)) ? 1u : 0u;
          }
        }
        // the rem-th largest value v: fewer than rem entries above it, at
        // least rem at or above it (every lane holding v qualifies)
        const uint64_t hm = ballot(own & (gt < rem) & (rem <= gt + eq));
        const int src = (int)__ffsll((unsigned long long)hm) - 1;
        const uint32_t vb = lane_value(__float_as_uint(o), src);
        const uint32_t take = rem - lane_value(gt, src);
        wave_lds_sync();  // the side list is read before anything reuses it
        return make_uint3(vb, take, take == lane_value(eq, src) ? 1u : 0u);
      }
      // more than 64: order keys, then a radix select inside the bin
      uint32_t lo = 0xFFFFFFFFu, hi = 0u;
      for (uint32_t i = lane; i < ns; i += kWave) {
        const uint32_t o = ord_key(__uint_as_float(side[i]));
        side[i] = o;
        lo = min(lo, o);
        hi = max(hi, o);
      }
      wave_lds_sync();
      lo = wave_min(lo);
      hi = wave_max(hi);
      uint2 r = make_uint2(lo, rem);
      if (lo != hi) r = select_in_range(side, ns, hist, lo, hi, 32 - __clz(hi - lo), rem);
      return make_uint3(__float_as_uint(ord_to_float(r.x)), r.y, 0u);
    }
    // narrow to the bin's score range
    float lo = 3.4e38f, hi = -3.4e38f;
    for (uint32_t base = 0; base < n; base += kWave * kFinBatch) {
      float x[kFinBatch];
      dense_load_batch(key, base, x);
#pragma unroll
      for (uint32_t j = 0; j < kFinBatch; ++j) {
        const bool inb = (base + j * kWave + lane < n) & (x[j] >= a) & (x[j] <= b) &
                         (bin_of(bins, x[j]) == fb.x);
        lo = fminf(lo, inb ? x[j] : 3.4e38f);
        hi = fmaxf(hi, inb ? x[j] : -3.4e38f);
      }
    }
    a = wave_fmin(lo);
    b = wave_fmax(hi);
  }
  if (!(a < b)) return make_uint3(__float_as_uint(a), rem, 0u);
  const uint32_t oa = ord_key(a), ob = ord_key(b);
  const uint2 r = select_in_range<true>(key, n, hist, oa, ob, 32 - __clz(ob - oa), rem);
  return make_uint3(__float_as_uint(ord_to_float(r.x)), r.y, 0u);
}

// Write the kept keys of the dense row in index order: keys with score > v,
// and the first `take_eq` keys with score == v (ALL_EQ: every key with score
// >= v).  Returns the number written.
template <bool ALL_EQ>
__device__ __forceinline__ uint32_t dense_emit(const lds_u32* key, uint32_t n, float v,
                                               uint32_t take_eq, const RowOut& out) {
  const uint32_t lane = (uint32_t)lane_id();
  uint32_t wpos = 0u, eq_seen = 0u;
  for (uint32_t base = 0; base < n; base += kWave * kFinBatch) {
    float x[kFinBatch];
    dense_load_batch(key, base, x);
    const uint32_t i0 = base + lane;
#pragma unroll
    for (uint32_t j = 0; j < kFinBatch; ++j) {
      const uint32_t i = i0 + j * kWave;
      const bool valid = i < n;
      bool keep;
      if constexpr (ALL_EQ) {
        keep = valid & (x[j] >= v);
      } else {
        const bool eqv = valid & (x[j] == v);
        const uint64_t meq = ballot(eqv);
        keep = (valid & (x[j] > v)) | (eqv & ((eq_seen + lanes_below(meq)) < take_eq));
        eq_seen = uniform(eq_seen + (uint32_t)__popcll(meq));
      }
      const uint64_t mk = ballot(keep);
      out.put(keep, wpos + lanes_below(mk), (int32_t)i, x[j]);
      wpos = uniform(wpos + (uint32_t)__popcll(mk));
    }
  }
  return wpos;
}

// Write the dense row's top k in index order, then (-1, -inf) padding up to
// `topk` slots.  With n <= k every visible key is written.  smin / smax:
// this lane's smallest and largest score (the wave's extremes are reduced
// here).
__device__ __forceinline__ void dense_finish(const lds_u32* key, uint32_t n, uint32_t k,
                                             float smin, float smax, lds_u32* hist,
                                             lds_u32* side, int topk,
                                             int32_t* __restrict__ out_idx,
                                             float* __restrict__ out_score) {
  const uint32_t lane = (uint32_t)lane_id();
  const RowOut out(out_idx, out_score, topk);
  uint32_t wpos = n;
  if (n <= k) {
    for (uint32_t base = 0; base < n; base += kWave * kFinBatch) {
      float x[kFinBatch];
      dense_load_batch(key, base, x);
#pragma unroll
      for (uint32_t j = 0; j < kFinBatch; ++j) {
        const uint32_t i = base + j * kWave + lane;
        out.put(i < n, i, (int32_t)i, x[j]);
      }
    }
  } else {
    wave_lds_sync();
    const uint3 sel = dense_select(key, n, k, wave_fmin(smin), wave_fmax(smax), hist, side);
    const float v = __uint_as_float(sel.x);
    wpos = sel.z ? dense_emit<true>(key, n, v, sel.y, out)
                 : dense_emit<false>(key, n, v, sel.y, out);
  }
  for (uint32_t p = wpos; p < (uint32_t)topk; p += kWave)
    out.put(p + lane < (uint32_t)topk, p + lane, -1, -__builtin_inff());
}

// The row's top k (index order) from a store holding `count` entries.
template <typename IdxT>
__device__ __forceinline__ void wave_finish_row(const RowStore<IdxT>& rs, uint32_t count, int topk,
                                                int32_t* __restrict__ out_idx,
                                                float* __restrict__ out_score) {
  uint32_t v = 0u, eq = 0u;
  if (count > (uint32_t)topk) {
    wave_lds_sync();
    const uint2 sel = wave_radix_select(rs.key, rs.hist, rs.side, rs.side_cap, count, (uint32_t)topk);
    v = sel.x;
    eq = sel.y;
  }
  wave_emit(rs, count, v, eq, topk, out_idx, out_score);
}

}  // namespace dsai
