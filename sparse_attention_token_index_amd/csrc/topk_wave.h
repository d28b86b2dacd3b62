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
//   wave_radix_select  8-bit MSD radix select of the k-th largest key value v
//                      (4 histogram passes over the store) and how many
//                      entries equal to v belong to the top k.  Loads are
//                      batched and the histogram atomics return nothing, so
//                      the passes run at LDS throughput, not latency.
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

// Keys per lane handled per batch of the histogram loop.
constexpr int kSelBatch = 8;

// k-th largest key value v among key[0, n), 1 <= k <= n (.x), and the number
// of entries equal to v that belong to the top k (.y).
__device__ __noinline__ uint2 wave_radix_select(lds_u32* key, lds_u32* hist, uint32_t n,
                                                uint32_t k) {
  const int lane = lane_id();
  uint32_t prefix = 0u, rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = lane; i < 256; i += kWave) hist[i] = 0u;
    wave_lds_sync();
    const uint32_t hi_mask = (shift == 24) ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (uint32_t base = 0; base < n; base += kWave * kSelBatch) {
      uint32_t u[kSelBatch];
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) {
        const uint32_t i = base + j * kWave + lane;
        u[j] = i < n ? key[i] : 0u;
      }
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) {
        const uint32_t i = base + j * kWave + lane;
        if (i < n && (u[j] & hi_mask) == prefix)
          __hip_atomic_fetch_add(&hist[(u[j] >> shift) & 255u], 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WAVEFRONT);
      }
    }
    wave_lds_sync();
    // lane L owns bins 4L .. 4L+3; count entries in higher bins
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
    const uint32_t digit = (uint32_t)__shfl(4 * lane + found, src);
    const uint32_t above_d = (uint32_t)__shfl((int)above, src);
    prefix = uniform(prefix | (digit << shift));
    rem = uniform(rem - above_d);
    wave_lds_sync();
  }
  return make_uint2(prefix, rem);
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
      u[j] = i < n ? rs.key[i] : 0u;
      x[j] = i < n ? (uint32_t)rs.idx[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const uint32_t i = base + j * kWave + lane;
      const bool in = i < n;
      const bool eq = in && (u[j] == v);
      const uint64_t meq = ballot(eq);
      const bool keep = (in && u[j] > v) || (eq && (eq_seen + lanes_below(meq)) < take_eq);
      const uint64_t mk = ballot(keep);
      if (keep) {
        const uint32_t p = wpos + lanes_below(mk);
        rs.key[p] = u[j];
        rs.idx[p] = (IdxT)x[j];
      }
      wpos = uniform(wpos + (uint32_t)__popcll(mk));
      eq_seen = uniform(eq_seen + (uint32_t)__popcll(meq));
    }
  }
  wave_lds_sync();
  return wpos;
}

// Reduce the store to its top k (stable) if it holds more than k entries;
// *tau receives the k-th largest key (the new admission threshold).
template <typename IdxT>
__device__ __forceinline__ uint32_t wave_keep_topk(const RowStore<IdxT>& rs, uint32_t count,
                                                   uint32_t k, uint32_t* tau) {
  if (count <= k) return count;
  wave_lds_sync();
  const uint2 sel = wave_radix_select(rs.key, rs.hist, count, k);
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

// The row's top k (index order) from a store holding `count` entries.
template <typename IdxT>
__device__ __forceinline__ void wave_finish_row(const RowStore<IdxT>& rs, uint32_t count, int topk,
                                                int32_t* __restrict__ out_idx,
                                                float* __restrict__ out_score) {
  uint32_t v = 0u, eq = 0u;
  if (count > (uint32_t)topk) {
    wave_lds_sync();
    const uint2 sel = wave_radix_select(rs.key, rs.hist, count, (uint32_t)topk);
    v = sel.x;
    eq = sel.y;
  }
  wave_emit(rs, count, v, eq, topk, out_idx, out_score);
}

}  // namespace dsai
