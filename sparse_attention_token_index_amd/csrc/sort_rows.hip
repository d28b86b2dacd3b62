// In-place sort of top-k rows by score descending, the lower index first among
// equal scores.  Padding slots (index -1, score -inf) end up at the tail.
//
// One workgroup (256 threads) sorts one row of up to 256 * ITEMS entries.
//
// Bucket path (the common case).  The row's real entries are spread over
// NB = 256 * ITEMS buckets by a monotone map of the score onto [0, NB)
// (BucketMap: higher scores land in lower buckets); a counting pass and a
// scan give every bucket its output range, the entries are scattered into
// their bucket's range, and
// each entry's final slot inside its bucket is its rank there under
// (score descending, index ascending), counted by comparing it with the
// bucket's other entries.  With about one entry per bucket this costs a few
// LDS operations per entry instead of a pass per digit.
//
// Radix path (rows with a bucket of more than kBucketLimit entries: many
// equal or nearly equal scores).  A stable block-wide LSD radix sort on the
// 32-bit order key with 3-bit digits; digit positions on which every real key
// agrees are skipped.  Stability gives the index order among equal scores
// because rows arrive in ascending index order (the selection kernels write
// them that way).
#include "internal.h"
#include "device_common.h"

namespace dsai {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr uint32_t kBucketLimit = 64;

// Radix path digits: 3 bits (11 passes at most, constant digits skipped).
constexpr int kRadixBits = 3;
constexpr int kRadixDigits = 1 << kRadixBits;

template <int ITEMS>
struct SortLayout {
  static constexpr int NB = kSortThreads * ITEMS;  // buckets (>= entries per row)
  // bucket path, in words: start[NB] (counts, then bucket starts, then bucket
  // ends) | pad | kv[NB] (key, index pairs)
  static constexpr int kStart = 0, kKV = NB + 4;
  static constexpr int kBucketWords = 3 * NB + 4;
  // radix path: cnt[digits][256] | xk[256 * (ITEMS + 1)] | xv[256 * (ITEMS + 1)]
  static constexpr int kRadixWords =
      kRadixDigits * kSortThreads + 2 * kSortThreads * (ITEMS + 1);
  static constexpr int kRed = kBucketWords > kRadixWords ? kBucketWords : kRadixWords;
  static constexpr int kWords = kRed + 4 * kSortWaves;
};

// Thread t's ITEMS consecutive words w[t*ITEMS ..]: 16-byte accesses when
// ITEMS is a multiple of 4 (word-strided accesses would hit the same banks).
template <int ITEMS>
__device__ __forceinline__ void load_run(const uint32_t* w, uint32_t (&v)[ITEMS]) {
  const int t = threadIdx.x;
  if constexpr (ITEMS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < ITEMS; j += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(&w[t * ITEMS + j]);
      v[j] = q.x; v[j + 1] = q.y; v[j + 2] = q.z; v[j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) v[j] = w[t * ITEMS + j];
  }
}

template <int ITEMS>
__device__ __forceinline__ void store_run(uint32_t* w, const uint32_t (&v)[ITEMS]) {
  const int t = threadIdx.x;
  if constexpr (ITEMS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < ITEMS; j += 4)
      *reinterpret_cast<uint4*>(&w[t * ITEMS + j]) = make_uint4(v[j], v[j + 1], v[j + 2], v[j + 3]);
  } else {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) w[t * ITEMS + j] = v[j];
  }
}

// Monotone non-increasing map of a row's scores onto [0, nb) buckets.  A top
// k's scores crowd just above the row's smallest (the selection threshold),
// the more so when a few large scores stretch the range, so the map is
// log-linear in the distance from the smallest: with d = s/2 - min/2 and
// c = (max - min) / 32, the bucket follows the float bits of d + c, counted
// from those of c and scaled onto the nb buckets: about linear (a fixed step)
// for d below c, logarithmic (equal buckets per octave) above it.  Each step
// (halving, subtracting, adding c, the bits of a non-negative float, the
// integer-to-float conversion, scaling, truncation, clamping) is monotone,
// so a higher score never lands in a higher bucket; halving keeps the
// difference of any two finite scores finite.  On top-k rows of the
// 65536-token workload (5 % of keys x4) a map linear in the score put 20-37
// entries in the fullest bucket, this one about 10; on rows nearer a
// Gaussian's upper half the two spread alike.
struct BucketMap {
  float hmin;     // min / 2
  float c;        // the offset: (max - min) / 32, halved like d
  float scale;    // buckets per unit of bits(d + c) - bits(c)
  uint32_t cbits;
  __device__ __forceinline__ BucketMap(float smin, float smax, uint32_t nb) {
    hmin = __fmul_rn(0.5f, smin);
    const float rh = __fsub_rn(__fmul_rn(0.5f, smax), hmin);
    c = __fmul_rn(rh, 0.0625f);  // exact: a power of two
    cbits = __float_as_uint(c);
    const uint32_t span = __float_as_uint(__fadd_rn(rh, c)) - cbits;
    scale = (float)nb / ((float)span + 1.0f);
  }
  // explicit roundings: both call sites must map a key to the same bucket
  __device__ __forceinline__ uint32_t operator()(uint32_t key, uint32_t nb) const {
    const float d = __fsub_rn(__fmul_rn(0.5f, ord_to_float(key)), hmin);
    const uint32_t b = __float_as_uint(__fadd_rn(d, c)) - cbits;
    const float x = __fmul_rn((float)b, scale);
    const uint32_t i = (uint32_t)fminf(x, (float)(nb - 1u));
    return nb - 1u - (i < nb ? i : nb - 1u);
  }
};

__device__ __forceinline__ uint32_t blocked_addr(uint32_t p, int items) {
  return p + p / (uint32_t)items;  // one pad word per thread block of items: odd stride
}

// Stable LSD radix sort of the row (reloaded in a blocked arrangement: thread
// t owns slots [t * ITEMS, (t + 1) * ITEMS)).
template <int ITEMS>
__device__ void radix_sort_row(int32_t* __restrict__ ri, float* __restrict__ rs, int topk,
                               uint32_t* smem) {
  using L = SortLayout<ITEMS>;
  uint32_t* cnt = smem;                                             // [digit][thread]
  uint32_t* xk = cnt + kRadixDigits * kSortThreads;                  // exchange keys
  int32_t* xv = (int32_t*)(xk + kSortThreads * (ITEMS + 1));         // exchange indices
  uint32_t* red = smem + L::kRed;
  const int t = threadIdx.x;
  const int lane = lane_id(), wave = t >> 6;

  uint32_t key[ITEMS];
  int32_t val[ITEMS];
  uint32_t a = 0xFFFFFFFFu, o = 0u;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int p = t * ITEMS + i;
    val[i] = p < topk ? ri[p] : -1;
    key[i] = 0xFFFFFFFFu;
    if (val[i] >= 0) {
      key[i] = ~ord_key(rs[p]);  // ascending on ~key = descending score
      a &= key[i];
      o |= key[i];
    }
  }
  a = wave_and(a);
  o = wave_or(o);
  __syncthreads();  // the bucket path's reads of `red` are done
  if (lane == 0) {
    red[wave] = a;
    red[kSortWaves + wave] = o;
  }
  __syncthreads();
  uint32_t ba = 0xFFFFFFFFu, bo = 0u;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) {
    ba &= red[w];
    bo |= red[kSortWaves + w];
  }
  const uint32_t diff = ba ^ bo;

  constexpr uint32_t kMask = (uint32_t)kRadixDigits - 1u;
  for (int shift = 0; shift < 32; shift += kRadixBits) {
    if (((diff >> shift) & kMask) == 0u) continue;
#pragma unroll
    for (int d = 0; d < kRadixDigits; ++d) cnt[d * kSortThreads + t] = 0u;
    uint32_t r[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint32_t d = (key[i] >> shift) & kMask;
      r[i] = cnt[d * kSortThreads + t];
      cnt[d * kSortThreads + t] = r[i] + 1u;
    }
    __syncthreads();
    // exclusive scan over f = d * 256 + thread; thread t owns f in
    // [kRadixDigits * t, kRadixDigits * (t + 1))
    uint32_t v[kRadixDigits];
#pragma unroll
    for (int x = 0; x < kRadixDigits; x += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(&cnt[kRadixDigits * t + x]);
      v[x] = q.x; v[x + 1] = q.y; v[x + 2] = q.z; v[x + 3] = q.w;
    }
    uint32_t run = 0u;
#pragma unroll
    for (int x = 0; x < kRadixDigits; ++x) {
      const uint32_t c = v[x];
      v[x] = run;
      run += c;
    }
    const uint32_t incl = wave_incl_scan(run);
    if (lane == kWave - 1) red[wave] = incl;
    __syncthreads();
    uint32_t base = incl - run;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w)
      if (w < wave) base += red[w];
#pragma unroll
    for (int x = 0; x < kRadixDigits; x += 4)
      *reinterpret_cast<uint4*>(&cnt[kRadixDigits * t + x]) =
          make_uint4(base + v[x], base + v[x + 1], base + v[x + 2], base + v[x + 3]);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint32_t d = (key[i] >> shift) & kMask;
      const uint32_t dst = blocked_addr(cnt[d * kSortThreads + t] + r[i], ITEMS);
      xk[dst] = key[i];
      xv[dst] = val[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint32_t s = blocked_addr((uint32_t)(t * ITEMS + i), ITEMS);
      key[i] = xk[s];
      val[i] = xv[s];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int p = t * ITEMS + i;
    if (p < topk) {
      ri[p] = val[i] >= 0 ? val[i] : -1;
      rs[p] = val[i] >= 0 ? ord_to_float(~key[i]) : -__builtin_huge_valf();
    }
  }
}

// Bucket path for one row (falls back to the radix path when a bucket is too
// full).  key/val: the row's entries in the striped arrangement (slot
// i * 256 + t), val < 0 for padding.  One array serves as the counts, then
// each bucket's first slot (scatter cursors), then, after the scatter, each
// bucket's end: bucket b spans [end[b-1], end[b]).
template <int ITEMS>
__device__ __forceinline__ void bucket_sort_row(int32_t* __restrict__ ri, float* __restrict__ rs,
                                                int topk, uint32_t* smem, uint32_t (&key)[ITEMS],
                                                int32_t (&val)[ITEMS]) {
  using L = SortLayout<ITEMS>;
  constexpr uint32_t NB = (uint32_t)L::NB;
  uint32_t* start = smem + L::kStart;
  uint2* kv = reinterpret_cast<uint2*>(smem + L::kKV);  // entries grouped by bucket
  uint32_t* red = smem + L::kRed;
  const int t = threadIdx.x;
  const int lane = lane_id(), wave = t >> 6;

  // Real entries, their key range.
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, nreal = 0u;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (val[i] >= 0) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
    nreal += (uint32_t)__popcll(ballot(val[i] >= 0));
  }
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  __syncthreads();  // the previous row's readers of `red` and `kv` are done
  if (lane == 0) {
    red[wave] = kmin;
    red[kSortWaves + wave] = kmax;
    red[2 * kSortWaves + wave] = nreal;
  }
  {
    uint32_t z[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) z[j] = 0u;
    store_run<ITEMS>(start, z);
  }
  __syncthreads();
  uint32_t nv = 0u;
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) {
    kmin = min(kmin, red[w]);
    kmax = max(kmax, red[kSortWaves + w]);
    nv += red[2 * kSortWaves + w];
  }
  const BucketMap bmap(ord_to_float(kmin), ord_to_float(kmax), NB);

  // Count entries per bucket.
  uint32_t bkt[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    bkt[i] = bmap(key[i], NB);
    if (val[i] >= 0) atomicAdd(&start[bkt[i]], 1u);
  }
  __syncthreads();

  // Exclusive scan of the counts (thread t owns buckets [t*ITEMS, (t+1)*ITEMS))
  // and the largest bucket.
  uint32_t c[ITEMS];
  load_run<ITEMS>(start, c);
  uint32_t run = 0u, big = 0u;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const uint32_t n = c[j];
    c[j] = run;
    run += n;
    big = max(big, n);
  }
  const uint32_t incl = wave_incl_scan(run);
  big = wave_max(big);
  if (lane == kWave - 1) {
    red[3 * kSortWaves + wave] = incl;
    red[wave] = big;  // every thread read red[0..3] before the last barrier
  }
  __syncthreads();
  uint32_t base = incl - run;
  big = 0u;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) {
    if (w < wave) base += red[3 * kSortWaves + w];
    big = max(big, red[w]);
  }
  if (big > kBucketLimit) {  // block-uniform
    radix_sort_row<ITEMS>(ri, rs, topk, smem);
    return;
  }
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) c[j] += base;
  store_run<ITEMS>(start, c);
  __syncthreads();

  // Scatter into the buckets' ranges (arbitrary order inside a bucket); the
  // cursors end at each bucket's end.
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (val[i] >= 0) {
      const uint32_t slot = atomicAdd(&start[bkt[i]], 1u);
      kv[slot] = make_uint2(key[i], (uint32_t)val[i]);
    }
  }
  __syncthreads();

  // Rank of each entry inside its bucket: entries with a higher key, or the
  // same key and a lower index, go first.  The comparison loops of the
  // thread's entries run side by side so their LDS reads overlap.
  uint32_t s0[ITEMS], cnt[ITEMS], rank[ITEMS];
  uint32_t maxc = 0u;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint32_t p = (uint32_t)(i * kSortThreads + t);
    s0[i] = p;
    cnt[i] = 0u;
    rank[i] = 0u;
    if (p < nv) {
      const uint2 e = kv[p];
      key[i] = e.x;
      val[i] = (int32_t)e.y;
      const uint32_t b = bmap(key[i], NB);
      const uint32_t lo = b > 0u ? start[b - 1u] : 0u, n = start[b] - lo;
      if (n > 1u) {
        s0[i] = lo;
        cnt[i] = n;
      }
    }
    maxc = max(maxc, cnt[i]);
  }
  // Two bucket entries per step (one paired LDS read); the second may lie
  // past the bucket (still inside the allocation) and is then ignored.
  for (uint32_t j = 0; j < maxc; j += 2) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (j < cnt[i]) {
        const uint2 e0 = kv[s0[i] + j];
        const uint2 e1 = kv[s0[i] + j + 1u];
        rank[i] += (e0.x > key[i] || (e0.x == key[i] && (int32_t)e0.y < val[i])) ? 1u : 0u;
        rank[i] += (j + 1u < cnt[i] &&
                    (e1.x > key[i] || (e1.x == key[i] && (int32_t)e1.y < val[i]))) ? 1u : 0u;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if ((uint32_t)(i * kSortThreads + t) < nv)
      kv[s0[i] + rank[i]] = make_uint2(key[i], (uint32_t)val[i]);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int p = i * kSortThreads + t;
    if (p < topk) {
      const bool real = (uint32_t)p < nv;
      const uint2 e = real ? kv[p] : make_uint2(0u, 0u);
      ri[p] = real ? (int32_t)e.y : -1;
      rs[p] = real ? ord_to_float(e.x) : -__builtin_huge_valf();
    }
  }
}

// Each workgroup sorts rows blockIdx.x, blockIdx.x + gridDim.x, ...; with PF
// the next row's entries are loaded while the current row is sorted (their
// registers cost one wavefront per SIMD at 2048-entry rows, which pays only
// where each workgroup has a second row).
template <int ITEMS, bool PF>
__global__ __launch_bounds__(kSortThreads) __attribute__((amdgpu_waves_per_eu(
    ITEMS <= 4 ? 6 : ITEMS <= 8 ? (PF ? 5 : 6) : 1))) void sort_rows_kernel(int32_t* __restrict__ idx,
                                                                    float* __restrict__ score,
                                                                    int topk, int rows) {
  extern __shared__ __align__(16) uint32_t sort_smem[];
  const int t = threadIdx.x;
  int32_t nval[ITEMS];
  float nsc[ITEMS];
  auto load = [&](int row) {
    const int32_t* ri = idx + (int64_t)row * topk;
    const float* rs = score + (int64_t)row * topk;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int p = i * kSortThreads + t;
      nval[i] = p < topk ? ri[p] : -1;
      nsc[i] = p < topk ? rs[p] : 0.f;
    }
  };
  int row = blockIdx.x;
  if (row < rows) load(row);
  for (; row < rows; row += gridDim.x) {
    uint32_t key[ITEMS];
    int32_t val[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      val[i] = nval[i];
      key[i] = val[i] >= 0 ? ord_key(nsc[i]) : 0u;
    }
    if (PF && row + (int)gridDim.x < rows) load(row + gridDim.x);
    bucket_sort_row<ITEMS>(idx + (int64_t)row * topk, score + (int64_t)row * topk, topk,
                           sort_smem, key, val);
    if (!PF && row + (int)gridDim.x < rows) load(row + gridDim.x);
  }
}

// The resident set R of a sort kernel: the runtime's occupancy for it (its
// registers and `lds` bytes of LDS) times the CUs.  The launch takes one
// workgroup per row up to 8 rows per slot, else one per two rows (each
// workgroup takes every grid-th row).  Workgroups that outlive the resident
// set are started by the dispatcher as slots free up, which balances the last
// round and keeps the workgroups of a CU out of step with each other.  Up to
// 8 rows per slot each workgroup sorts one row (a persistent grid of R would
// give some slots one row more than others: 3 against 2.67 at 4096 rows);
// beyond that each sorts two, the second row's loads in flight during the
// first's sort (the PF kernel).  Measured on MI355X: 4096 rows of 2048,
// 42 -> 37 us; 32768 rows of 512, 95 -> 80 us, against a persistent grid of
// R; 65536 rows of 2048, 0.570 -> 0.518 ms with the PF kernel at five
// wavefronts per SIMD (no spills) instead of six.
static int64_t sort_resident(const void* kern, size_t lds) {
  static int cus_cache[64];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < 64) cus = cus_cache[dev];
  if (cus <= 0) {
    if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                       hipSuccess || cus <= 0)
      cus = 256;
    if (dev >= 0 && dev < 64) cus_cache[dev] = cus;
  }
  // One cached answer per (kernel, device); each kernel instance always runs
  // with the same LDS size.
  static const void* kern_cache[64][6];
  static int per_cu_cache[64][6];
  int per_cu = 0, slot = -1;
  if (dev >= 0 && dev < 64) {
    for (int i = 0; i < 6 && slot < 0; ++i) {
      if (kern_cache[dev][i] == kern) {
        per_cu = per_cu_cache[dev][i];
        slot = i;
      } else if (kern_cache[dev][i] == nullptr) {
        slot = i;
      }
    }
  }
  if (per_cu <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kSortThreads, lds) !=
            hipSuccess || per_cu < 1)
      per_cu = 1;
    if (slot >= 0) {
      kern_cache[dev][slot] = kern;
      per_cu_cache[dev][slot] = per_cu;
    }
  }
  return (int64_t)cus * per_cu;
}

hipError_t launch_sort_rows(int32_t* idx, float* score, int64_t rows, int topk, hipStream_t st) {
  if (rows <= 0 || topk <= 1) return hipSuccess;
  if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
#define DSAI_ITEMS(n)                                                                          \
  if (topk <= kSortThreads * n) {                                                              \
    const size_t lds = 4 * (size_t)SortLayout<n>::kWords;                                      \
    const void* one = (const void*)sort_rows_kernel<n, false>;                                 \
    const void* two = (const void*)sort_rows_kernel<n, true>;                                  \
    hipError_t e = hipFuncSetAttribute(one, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    if (e == hipSuccess)                                                                       \
      e = hipFuncSetAttribute(two, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);      \
    if (e != hipSuccess) return e;                                                             \
    if (rows <= 8 * sort_resident(one, lds))                                                   \
      hipLaunchKernelGGL((sort_rows_kernel<n, false>), dim3((unsigned)rows), dim3(kSortThreads), \
                         lds, st, idx, score, topk, (int)rows);                                \
    else                                                                                       \
      hipLaunchKernelGGL((sort_rows_kernel<n, true>), dim3((unsigned)((rows + 1) / 2)),        \
                         dim3(kSortThreads), lds, st, idx, score, topk, (int)rows);            \
    return hipGetLastError();                                                                  \
  }
  DSAI_ITEMS(1) DSAI_ITEMS(2) DSAI_ITEMS(4) DSAI_ITEMS(8) DSAI_ITEMS(16) DSAI_ITEMS(32)
#undef DSAI_ITEMS
  return hipErrorInvalidValue;
}

}  // namespace dsai
