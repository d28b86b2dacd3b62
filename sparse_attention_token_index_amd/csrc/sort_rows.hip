// Stable in-place sort of top-k rows by score descending.
//
// Rows arrive in ascending index order (the selection kernels emit them that
// way), so a stable sort on the score alone yields the order "score
// descending, lower index first among equal scores".  Padding slots
// (index -1, score -inf) stay at the tail.
//
// One workgroup (256 threads) sorts one row with a block-wide LSD radix sort
// on the 32-bit order key (4-bit digits), the row held in registers in a
// blocked arrangement (thread t owns slots [t*ITEMS, (t+1)*ITEMS)):
//   count   each thread counts its items per digit in private LDS counters,
//   scan    exclusive scan over (digit, thread) gives every item its rank,
//   scatter items go to their rank in an LDS exchange buffer, then are
//           read back blocked.
// Digit positions on which every real key agrees are skipped.  The
// workgroup's LDS footprint is small, so several rows are sorted per CU at
// once and LDS latency is hidden by the other workgroups.
#include "internal.h"
#include "device_common.h"

namespace dsai {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / kWave;

__device__ __forceinline__ uint32_t blocked_addr(uint32_t p, int items) {
  return p + p / (uint32_t)items;  // one pad word per thread block of items: odd stride
}

template <int ITEMS>
__global__ __launch_bounds__(kSortThreads) void sort_rows_kernel(int32_t* __restrict__ idx,
                                                                 float* __restrict__ score,
                                                                 int topk) {
  extern __shared__ __align__(16) uint32_t sort_smem[];
  uint32_t* cnt = sort_smem;                                  // [digit][thread]
  uint32_t* xk = cnt + 16 * kSortThreads;                      // exchange keys
  int32_t* xv = (int32_t*)(xk + kSortThreads * (ITEMS + 1));   // exchange indices
  uint32_t* red = (uint32_t*)(xv + kSortThreads * (ITEMS + 1));

  const int t = threadIdx.x;
  const int lane = lane_id(), wave = t >> 6;
  int32_t* ri = idx + (int64_t)blockIdx.x * topk;
  float* rs = score + (int64_t)blockIdx.x * topk;

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
  const uint32_t diff = ba ^ bo;  // 0 when the row has no real entry

  for (int shift = 0; shift < 32; shift += 4) {
    if (((diff >> shift) & 15u) == 0u) continue;
#pragma unroll
    for (int d = 0; d < 16; ++d) cnt[d * kSortThreads + t] = 0u;
    uint32_t r[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint32_t d = (key[i] >> shift) & 15u;
      r[i] = cnt[d * kSortThreads + t];
      cnt[d * kSortThreads + t] = r[i] + 1u;
    }
    __syncthreads();
    // exclusive scan over f = d * 256 + thread; thread t owns f in [16t, 16t + 16)
    uint32_t v[16];
#pragma unroll
    for (int x = 0; x < 16; x += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(&cnt[16 * t + x]);
      v[x] = q.x; v[x + 1] = q.y; v[x + 2] = q.z; v[x + 3] = q.w;
    }
    uint32_t run = 0u;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
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
    for (int x = 0; x < 16; x += 4)
      *reinterpret_cast<uint4*>(&cnt[16 * t + x]) =
          make_uint4(base + v[x], base + v[x + 1], base + v[x + 2], base + v[x + 3]);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint32_t d = (key[i] >> shift) & 15u;
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
    if (p < topk && val[i] >= 0) {
      ri[p] = val[i];
      rs[p] = ord_to_float(~key[i]);
    }
  }
}

static size_t sort_lds_bytes(int items) {
  return 4 * ((size_t)16 * kSortThreads + 2 * (size_t)kSortThreads * (items + 1) + 2 * kSortWaves);
}

hipError_t launch_sort_rows(int32_t* idx, float* score, int64_t rows, int topk, hipStream_t st) {
  if (rows <= 0 || topk <= 1) return hipSuccess;
  if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)rows);
#define DSAI_ITEMS(n)                                                                          \
  if (topk <= kSortThreads * n) {                                                              \
    const size_t lds = sort_lds_bytes(n);                                                      \
    hipError_t e = hipFuncSetAttribute((const void*)sort_rows_kernel<n>,                       \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);  \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL(sort_rows_kernel<n>, grid, dim3(kSortThreads), lds, st, idx, score,     \
                       topk);                                                                  \
    return hipGetLastError();                                                                  \
  }
  DSAI_ITEMS(1) DSAI_ITEMS(2) DSAI_ITEMS(4) DSAI_ITEMS(8) DSAI_ITEMS(16) DSAI_ITEMS(32)
#undef DSAI_ITEMS
  return hipErrorInvalidValue;
}

}  // namespace dsai
