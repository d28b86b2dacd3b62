// Wave-level top-k machinery over an LDS candidate store (gfx950, wave64).
//
// One wavefront owns one output row.  Candidates are (key, idx) pairs where
// `key` is the order-preserving uint32 image of an fp32 score (ord_key) and
// `idx` the key/pool index.  Candidates enter the store in ascending index
// order and every step below is stable, so "lower index first among equal
// scores" holds without storing a composite key:
//
//   wave_append       ballot + prefix count: appends the passing lanes in lane
//                     order after the current entries.
//   wave_radix_select 8-bit MSD radix select of the k-th largest key value v
//                     (LDS histogram, 4 passes) and how many entries equal to
//                     v belong to the top k.
//   wave_compact      stable in-place compaction to exactly the top k.
//   wave_sort_desc    stable LSD radix sort (4-bit digits, descending) with
//                     per-lane private counters; digit positions where all
//                     keys agree are skipped.
//
// All functions must be called by every lane of the wave with wave-uniform
// scalar arguments.
#pragma once

#include "device_common.h"

namespace dsai {

struct RowStore {
  lds_u32* key;   // [cap] order keys
  lds_u32* idx;   // [cap] indices
  lds_u32* hist;  // [256] radix-select histogram (wave-private)
};

__device__ __forceinline__ uint32_t uniform(uint32_t x) {
  return __builtin_amdgcn_readfirstlane(x);
}

__device__ __forceinline__ void wave_append(RowStore rs, uint32_t& count, bool pass,
                                            uint32_t u, uint32_t id) {
  const uint64_t m = ballot(pass);
  if (pass) {
    const uint32_t p = count + lanes_below(m);
    rs.key[p] = u;
    rs.idx[p] = id;
  }
  count = uniform(count + (uint32_t)__popcll(m));
}

// k-th largest key value v among key[0, n), 1 <= k <= n (.x), and the number
// of entries equal to v that belong to the top k (.y).
__device__ __noinline__ uint2 wave_radix_select(RowStore rs, uint32_t n, uint32_t k) {
  const int lane = lane_id();
  uint32_t prefix = 0u, rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = lane; i < 256; i += kWave) rs.hist[i] = 0u;
    wave_lds_sync();
    const uint32_t hi_mask = (shift == 24) ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (uint32_t i = lane; i < n; i += kWave) {
      const uint32_t u = rs.key[i];
      if ((u & hi_mask) == prefix)
        __hip_atomic_fetch_add(&rs.hist[(u >> shift) & 255u], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WAVEFRONT);
    }
    wave_lds_sync();
    // lane L owns bins 4L .. 4L+3; count entries in higher bins
    const u32x4 c = *reinterpret_cast<const DSAI_LDS u32x4*>(&rs.hist[4 * lane]);
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
__device__ __noinline__ uint32_t wave_compact(RowStore rs, uint32_t n, uint32_t v,
                                              uint32_t take_eq) {
  const int lane = lane_id();
  uint32_t wpos = 0u, eq_seen = 0u;
  for (uint32_t base = 0; base < n; base += kWave) {
    const uint32_t i = base + lane;
    const bool in = i < n;
    const uint32_t u = in ? rs.key[i] : 0u;
    const uint32_t x = in ? rs.idx[i] : 0u;
    const bool eq = in && (u == v);
    const uint64_t meq = ballot(eq);
    const bool keep = (in && u > v) || (eq && (eq_seen + lanes_below(meq)) < take_eq);
    const uint64_t mk = ballot(keep);
    if (keep) {
      const uint32_t p = wpos + lanes_below(mk);
      rs.key[p] = u;
      rs.idx[p] = x;
    }
    wpos = uniform(wpos + (uint32_t)__popcll(mk));
    eq_seen = uniform(eq_seen + (uint32_t)__popcll(meq));
  }
  wave_lds_sync();
  return wpos;
}

// Reduce the store to its top k (stable) if it holds more than k entries.
__device__ __forceinline__ uint32_t wave_keep_topk(RowStore rs, uint32_t count, uint32_t k,
                                                   uint32_t* tau) {
  if (count <= k) return count;
  wave_lds_sync();
  const uint2 sel = wave_radix_select(rs, count, k);
  *tau = sel.x;
  return wave_compact(rs, count, sel.x, sel.y);
}

struct SortedView {
  const lds_u32* key;
  const lds_u32* idx;
  int lgm;     // block size exponent of the padded layout
  bool padded; // entries at pad_addr(i) rather than i
};

__device__ __forceinline__ uint32_t pad_addr(uint32_t p, int lgm) {
  return lgm > 0 ? p + (p >> lgm) : p;
}

// Stable descending sort of the first n entries of the store.  The region at
// [half, half + n + 64) of both arrays is the ping-pong buffer (half >= n + 64)
// and `cnt` holds 16 x 64 private counters.  Lane L handles the contiguous
// block [L*m, (L+1)*m) with m = 2^lgm >= n / 64; writes after the first pass
// use one pad word per block so the lanes' strided accesses hit distinct banks.
__device__ __noinline__ SortedView wave_sort_desc(RowStore rs, uint32_t n, uint32_t half,
                                                  lds_u32* cnt) {
  const int lane = lane_id();
  int lgm = 0;
  while ((64u << lgm) < n) ++lgm;
  const uint32_t m = 1u << lgm;

  uint32_t a = 0xFFFFFFFFu, o = 0u;
  for (uint32_t i = lane; i < n; i += kWave) {
    const uint32_t u = rs.key[i];
    a &= u;
    o |= u;
  }
  const uint32_t diff = uniform(wave_and(a) ^ wave_or(o));

  lds_u32* ks = rs.key;
  lds_u32* is = rs.idx;
  lds_u32* kd = rs.key + half;
  lds_u32* id = rs.idx + half;
  bool padded = false;
  const uint32_t p0 = (uint32_t)lane * m;

  for (int shift = 0; shift < 32; shift += 4) {
    if (((diff >> shift) & 15u) == 0u) continue;
#pragma unroll
    for (int d = 0; d < 16; ++d) cnt[d * kWave + lane] = 0u;
    for (uint32_t j = 0; j < m; ++j) {
      const uint32_t p = p0 + j;
      if (p < n) {
        const uint32_t u = ks[padded ? pad_addr(p, lgm) : p];
        const uint32_t d = 15u - ((u >> shift) & 15u);
        cnt[d * kWave + lane] += 1u;
      }
    }
    wave_lds_sync();
    // exclusive scan over the flat order f = d*64 + lane; lane L owns f in [16L, 16L+16)
    uint32_t v[16];
#pragma unroll
    for (int x = 0; x < 16; x += 4) {
      const u32x4 t = *reinterpret_cast<const DSAI_LDS u32x4*>(&cnt[16 * lane + x]);
      v[x] = t.x; v[x + 1] = t.y; v[x + 2] = t.z; v[x + 3] = t.w;
    }
    uint32_t run = 0u;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const uint32_t c = v[x];
      v[x] = run;
      run += c;
    }
    const uint32_t base = wave_incl_scan(run) - run;
#pragma unroll
    for (int x = 0; x < 16; x += 4) {
      *reinterpret_cast<DSAI_LDS u32x4*>(&cnt[16 * lane + x]) =
          u32x4{base + v[x], base + v[x + 1], base + v[x + 2], base + v[x + 3]};
    }
    wave_lds_sync();
    for (uint32_t j = 0; j < m; ++j) {
      const uint32_t p = p0 + j;
      if (p < n) {
        const uint32_t sa = padded ? pad_addr(p, lgm) : p;
        const uint32_t u = ks[sa];
        const uint32_t x = is[sa];
        const uint32_t d = 15u - ((u >> shift) & 15u);
        const uint32_t dst = cnt[d * kWave + lane];
        cnt[d * kWave + lane] = dst + 1u;
        const uint32_t ta = pad_addr(dst, lgm);
        kd[ta] = u;
        id[ta] = x;
      }
    }
    wave_lds_sync();
    lds_u32* t0 = ks; ks = kd; kd = t0;
    lds_u32* t1 = is; is = id; id = t1;
    padded = true;
  }
  return SortedView{ks, is, lgm, padded};
}

// Write the sorted top-k row: `count` entries, then (-1, -inf) padding.
__device__ __forceinline__ void wave_write_row(const SortedView& sv, uint32_t count, int topk,
                                               int32_t* __restrict__ out_idx,
                                               float* __restrict__ out_score) {
  for (int i = lane_id(); i < topk; i += kWave) {
    if ((uint32_t)i < count) {
      const uint32_t a = sv.padded ? pad_addr((uint32_t)i, sv.lgm) : (uint32_t)i;
      out_idx[i] = (int32_t)sv.idx[a];
      out_score[i] = ord_to_float(sv.key[a]);
    } else {
      out_idx[i] = -1;
      out_score[i] = -__builtin_inff();
    }
  }
}

}  // namespace dsai
