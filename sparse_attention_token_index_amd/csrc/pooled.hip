// Pooled decode selection: kpool_compress -> index_scores -> topk_pools ->
// expand_selection (page "Module glm5next_dsa", "Shape of the pipeline").
#include "internal.h"
#include "score_tile.h"
#include "topk_wave.h"

namespace dsai {

// ---------------------------------------------------------------------------
// kpool_compress (glm5next_dsa: kernel facts - the pool softmax runs over the
// pool-slot axis, per channel; pooling starts at first_key; a pool counts only
// if all of its slots are valid).  Streaming: one thread per (pool, 8-channel
// group); each reads KP x (32 B gate + 16 B keys) with 16-byte loads,
// consecutive threads covering consecutive channels of a token row.
// ---------------------------------------------------------------------------
template <int KP>
__global__ __launch_bounds__(256) void kpool_kernel(
    const uint16_t* __restrict__ kn, const float* __restrict__ gate,
    const uint8_t* __restrict__ valid, const float* __restrict__ ape, int D, int64_t first_key,
    int64_t P, int groups_log2, uint16_t* __restrict__ pool_k, int32_t* __restrict__ pool_tok,
    uint8_t* __restrict__ pool_valid) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t p = tid >> groups_log2;
  if (p >= P) return;
  const int cg = (int)(tid & ((1 << groups_log2) - 1));
  const int c0 = cg * 8;
  const int64_t tok0 = first_key + p * KP;

  float lg[KP][8];
  float kv[KP][8];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const int64_t row = (tok0 + j) * D + c0;
    const float4 g0 = *reinterpret_cast<const float4*>(gate + row);
    const float4 g1 = *reinterpret_cast<const float4*>(gate + row + 4);
    const float4 a0 = *reinterpret_cast<const float4*>(ape + j * D + c0);
    const float4 a1 = *reinterpret_cast<const float4*>(ape + j * D + c0 + 4);
    const uint4 kk = *reinterpret_cast<const uint4*>(kn + row);
    lg[j][0] = g0.x + a0.x; lg[j][1] = g0.y + a0.y; lg[j][2] = g0.z + a0.z; lg[j][3] = g0.w + a0.w;
    lg[j][4] = g1.x + a1.x; lg[j][5] = g1.y + a1.y; lg[j][6] = g1.z + a1.z; lg[j][7] = g1.w + a1.w;
    const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kv[j][2 * i] = __uint_as_float(kw[i] << 16);
      kv[j][2 * i + 1] = __uint_as_float(kw[i] & 0xFFFF0000u);
    }
  }
  uint32_t outw[4];
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    float r[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int c = i + cc;
      float mx = lg[0][c];
#pragma unroll
      for (int j = 1; j < KP; ++j) mx = fmaxf(mx, lg[j][c]);
      float den = 0.f, num = 0.f;
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const float e = expf(lg[j][c] - mx);
        den += e;
        num = fmaf(e, kv[j][c], num);
      }
      r[cc] = num / den;
    }
    outw[i / 2] = (uint32_t)f32_to_bf16_rne(r[0]) | ((uint32_t)f32_to_bf16_rne(r[1]) << 16);
  }
  *reinterpret_cast<uint4*>(pool_k + p * D + c0) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
  if (cg == 0) {
    uint8_t all = 1;
#pragma unroll
    for (int j = 0; j < KP; ++j) all &= (valid[tok0 + j] != 0) ? 1 : 0;
    pool_valid[p] = all;
    pool_tok[p] = (int32_t)tok0;
  }
}

hipError_t launch_kpool(const KpoolArgs& a, hipStream_t st) {
  if (a.P <= 0) return hipSuccess;
  const int groups = a.D / 8;
  int glog = 0;
  while ((1 << glog) < groups) ++glog;
  const int64_t threads = a.P << glog;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
#define DSAI_KP(kp)                                                                             \
  case kp:                                                                                      \
    hipLaunchKernelGGL(kpool_kernel<kp>, dim3(blocks), dim3(256), 0, st, a.k_normed, a.gate,    \
                       a.valid, a.ape, a.D, a.first_key, a.P, glog, a.pool_k, a.pool_tok,       \
                       a.pool_valid);                                                           \
    break;
  switch (a.KP) {
    DSAI_KP(1) DSAI_KP(2) DSAI_KP(3) DSAI_KP(4) DSAI_KP(5) DSAI_KP(6) DSAI_KP(7) DSAI_KP(8)
    default:
      return hipErrorInvalidValue;
  }
#undef DSAI_KP
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// index_scores: [Q, P] scores of decode queries against pool keys, -inf for
// invalid candidates (glm5next_dsa: "[Q, P] scores + candidate validity").
// One workgroup = 8 wavefronts = 8 query rows against a range of
// kPoolTilesPerBlock 32-pool tiles, so each staged tile serves 8 rows and
// each row's query stays in registers across the range.  The key loop is the
// fused indexer's: double-buffered LDS tiles, the next tile's fragments
// fetched right after the barrier, the head reduction of tile it - 1
// interleaved with tile it's products, and tile it - 2's scores stored.  With
// one workgroup per CU and little math per tile, the loop is bound by load
// latency, so two register stages (even and odd tiles) keep each tile's load
// in flight for two steps before it is staged.
// ---------------------------------------------------------------------------
constexpr int kPoolTilesPerBlock = 16;
constexpr int kPoolRows = 8;

template <int HP, int D>
struct PoolScoresLds {
  static constexpr int kStage = kPoolRows * TileScorer<HP, D>::kStageBytes;
  static constexpr int kTiles = 2 * TileGeom<D>::kTileBytes;
  static constexpr int kRegion = kStage > kTiles ? kStage : kTiles;
  static constexpr int kBytes = kRegion + kPoolTilesPerBlock * TileGeom<D>::kTileKeys;
};

template <int HP, int D>
__global__ __launch_bounds__(kPoolRows * 64) __attribute__((amdgpu_waves_per_eu(2))) void
pooled_scores_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                     const uint16_t* __restrict__ pool_k, const uint8_t* __restrict__ pool_valid,
                     const int32_t* __restrict__ limit, int Q, int P, int H, int pool_blocks,
                     float* __restrict__ scores) {
  using G = TileGeom<D>;
  using Scorer = TileScorer<HP, D>;
  using Acc = typename Scorer::Acc;
  using Frag = typename Scorer::Frag;
  using L = PoolScoresLds<HP, D>;
  constexpr int kPer = kPoolTilesPerBlock * G::kTileKeys;
  extern __shared__ __align__(16) char smem_raw[];
  lds_char* tiles = (lds_char*)smem_raw;
  DSAI_LDS uint8_t* valid_s = (DSAI_LDS uint8_t*)(tiles + L::kRegion);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = lane_id();
  const int pb = blockIdx.x % pool_blocks;  // consecutive blocks share a pool range
  const int row = (blockIdx.x / pool_blocks) * kPoolRows + wave;
  const bool active = row < Q;
  const int p0 = pb * kPer;
  const int np = min(kPer, P - p0);
  // the row's visible pools: p < its bound (clamped to [0, P]), all if none
  const int lim = (limit && active) ? min(max(limit[row], 0), P) : P;
  const int np_row = max(0, min(np, lim - p0));  // this block's pools the row sees
  const int ntiles = (np + G::kTileKeys - 1) / G::kTileKeys;

  TileLoader<D, kPoolRows * 64> lda, ldb;  // even and odd tiles
  lda.init(pool_k + (int64_t)p0 * D, (uint32_t)D, (uint32_t)((int64_t)np * D * 2));
  ldb.init(pool_k + (int64_t)p0 * D, (uint32_t)D, (uint32_t)((int64_t)np * D * 2));
  lda.load(0u);
  ldb.load((uint32_t)G::kTileKeys);
  Scorer sc;
  sc.init_offsets();
  const bool w4 = (H & 3) == 0 && ((uintptr_t)w & 15u) == 0;
  sc.load_row_staged(0, q + (int64_t)(active ? row : 0) * H * D,
                     w + (int64_t)(active ? row : 0) * H, H, active, w4,
                     tiles + wave * Scorer::kStageBytes);
  for (int i = threadIdx.x; i < kPer; i += kPoolRows * 64) valid_s[i] = i < np ? pool_valid[p0 + i] : 0;
  __syncthreads();
  float* srow = scores + (int64_t)row * P + p0;

  auto buf = [&](int it) { return tiles + (it & 1) * G::kTileBytes; };
  float part = 0.f;
  auto finish = [&](int it_rec) {
    const float s = Scorer::combine(part);
    const int i = it_rec * G::kTileKeys + (lane & 31);
    if (active && lane < 32 && i < np) srow[i] = (valid_s[i] && i < np_row) ? s : -__builtin_inff();
  };
  // ld holds tile it + 2 (loaded two steps earlier), then takes tile it + 4
  auto step = [&](int it, TileLoader<D, kPoolRows * 64>& ld, Frag& fcur, Frag& fnext, Acc& cur,
                  const Acc& old, bool fin, bool red) {
    __syncthreads();
    sc.fetch(buf(it + 1), fnext);
    if (fin) finish(it - 2);
    ld.store(buf(it + 2));
    ld.load((uint32_t)(it + 4) * G::kTileKeys);
    sc.mma(fcur, cur);
    if (red) part = sc.reduce_half(old, 0);
  };
  Acc acc0, acc1;
  Frag f0, f1;
  lda.store(buf(0));
  lda.load((uint32_t)(2 * G::kTileKeys));
  ldb.store(buf(1));
  ldb.load((uint32_t)(3 * G::kTileKeys));
  __syncthreads();
  sc.fetch(buf(0), f0);
  step(0, lda, f0, f1, acc0, acc1, false, false);
  if (ntiles > 1) {
    step(1, ldb, f1, f0, acc1, acc0, false, true);
    int it = 2;
    for (; it + 1 < ntiles; it += 2) {
      step(it, lda, f0, f1, acc0, acc1, true, true);
      step(it + 1, ldb, f1, f0, acc1, acc0, true, true);
    }
    if (it < ntiles) step(it, lda, f0, f1, acc0, acc1, true, true);
    finish(ntiles - 2);
  }
  part = sc.reduce_half(((ntiles - 1) & 1) ? acc1 : acc0, 0);
  finish(ntiles - 1);
}

template <int HP, int D>
static hipError_t launch_scores_t(const PooledScoresArgs& a, hipStream_t st) {
  const int per_block = kPoolTilesPerBlock * TileGeom<D>::kTileKeys;
  const int64_t pool_blocks = (a.P + per_block - 1) / per_block;
  const int64_t blocks = pool_blocks * ((a.Q + kPoolRows - 1) / kPoolRows);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  constexpr int lds = PoolScoresLds<HP, D>::kBytes;
  hipError_t e = hipFuncSetAttribute((const void*)pooled_scores_kernel<HP, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((pooled_scores_kernel<HP, D>), dim3((unsigned)blocks), dim3(kPoolRows * 64),
                     lds, st, a.q, a.w, a.pool_k, a.pool_valid, a.limit, (int)a.Q, (int)a.P, a.H,
                     (int)pool_blocks, a.scores);
  return hipGetLastError();
}

hipError_t launch_pooled_scores(const PooledScoresArgs& a, hipStream_t st) {
  if (a.Q <= 0 || a.P <= 0) return hipSuccess;
  const int HP = a.H <= 32 ? 32 : 64;
#define DSAI_CASE(hp, d) \
  if (HP == hp && a.D == d) return launch_scores_t<hp, d>(a, st);
  DSAI_CASE(32, 32) DSAI_CASE(32, 64) DSAI_CASE(32, 128)
  DSAI_CASE(64, 32) DSAI_CASE(64, 64) DSAI_CASE(64, 128)
#undef DSAI_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// topk_pools: one workgroup per row, NW wavefronts each streaming a
// contiguous slice of the row's P scores through the threshold filter and
// radix select of the fused indexer (-inf marks an invalid candidate and never
// enters a store).  The slices' survivors are concatenated in slice order
// (= index order) and one wavefront selects the row's top select_k from them;
// the row sort then orders them by score.
// ---------------------------------------------------------------------------
constexpr int kLoadBatch = 4;

__global__ __launch_bounds__(1024) void topk_rows_kernel(const float* __restrict__ scores, int P,
                                                         int sel, int cap, int NW,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ out_scores) {
  extern __shared__ __align__(16) char smem_raw[];
  lds_char* smem = (lds_char*)smem_raw;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int row = blockIdx.x;
  const size_t per_wave = (size_t)cap * 8 + kSelScratchBytes;
  lds_char* mine = smem + wave * per_wave;
  const RowStore<uint32_t> rs{(lds_u32*)mine, (lds_u32*)mine + cap, (lds_u32*)mine + 2 * cap,
                              (lds_u32*)mine + 2 * cap + 256, 256u};
  lds_u32* merged = (lds_u32*)(smem + NW * per_wave);   // [NW * sel] keys, then indices
  lds_u32* counts = merged + 2 * NW * sel;              // [NW]

  const float* srow = scores + (int64_t)row * P;
  const int per = ((P + NW - 1) / NW + kWave - 1) / kWave * kWave;
  const int p0 = wave * per;
  const int p1 = min(P, p0 + per);
  uint32_t count = 0u, tau = 0u;
  for (int base = p0; base < p1; base += kWave * kLoadBatch) {
    float v[kLoadBatch];
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int p = base + j * kWave + lane;
      v[j] = p < p1 ? srow[p] : -__builtin_inff();
    }
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int p = base + j * kWave + lane;
      const uint32_t u = ord_key(v[j]);
      wave_append(rs, count, p < p1 && v[j] != -__builtin_inff() && u > tau, u, (uint32_t)p);
      if (count > (uint32_t)(cap - kWave)) count = wave_keep_topk(rs, count, sel, &tau);
    }
  }
  int32_t* orow = ids + (int64_t)row * sel;
  float* osc = out_scores + (int64_t)row * sel;
  if (NW == 1) {
    wave_finish_row(rs, count, sel, orow, osc);
    return;
  }
  count = wave_keep_topk(rs, count, sel, &tau);
  if (lane == 0) counts[wave] = count;
  __syncthreads();
  uint32_t off = 0u, total = 0u;
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = counts[w];
    if (w < wave) off += c;
    total += c;
  }
  for (uint32_t i = lane; i < count; i += kWave) {
    merged[off + i] = rs.key[i];
    merged[NW * sel + off + i] = rs.idx[i];
  }
  __syncthreads();
  if (wave == 0) {
    const RowStore<uint32_t> all{merged, merged + NW * sel, rs.hist, rs.side, rs.side_cap};
    wave_finish_row(all, uniform(total), sel, orow, osc);
  }
}

// ---------------------------------------------------------------------------
// topk_pools for rows of at most 1024 * 32 pools: one 1024-thread workgroup
// per row holds the row in registers (thread t owns pools [t*ITEMS,
// (t+1)*ITEMS)) and finds the select_k-th largest key with a block-wide
// select: a histogram of the keys over 2048 float-linear bins of [min, max]
// (LDS atomics), a suffix search for the bin holding rank k, and the
// threshold among that bin's keys by direct counting (a crowded bin: at most
// three radix passes of 11 bits inside its range).  That gives the threshold
// key T and how many entries equal to T to keep (the lowest pool ids).  For
// the score order with select_k <= kRankSortMax, when the entries above T
// and every entry equal to T fit the LDS list, they are appended to it in
// any order and each one's rank under (score desc, pool id asc) is counted
// against the others; ranks past select_k (surplus equal keys) are dropped.
// Otherwise one block scan places the selected entries in pool-id order
// (ranked the same way for the score order, else written as they are).
// Each phase has LDS words of its own, so a barrier separates only a
// phase's writes from its reads.
// ---------------------------------------------------------------------------
constexpr int kBlockSelThreads = 1024;
constexpr int kBlockSelWaves = kBlockSelThreads / kWave;
constexpr int kBlockSelBinBits = 11;
constexpr int kBlockSelBins = 1 << kBlockSelBinBits;
constexpr int kRankSortMax = 512;

// Block-wide inclusive prefix sum of one value per thread; `red` holds
// kBlockSelWaves words that no thread reads after the last barrier before
// the call (one barrier inside).  Returns (inclusive, total).
__device__ __forceinline__ uint2 block_incl_scan(uint32_t x, uint32_t* red) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(x);
  if (lane == kWave - 1) red[wave] = incl;
  __syncthreads();
  uint32_t base = 0u, total = 0u;
#pragma unroll
  for (int w = 0; w < kBlockSelWaves; ++w) {
    const uint32_t c = red[w];
    base += w < wave ? c : 0u;
    total += c;
  }
  return make_uint2(base + incl, total);
}

template <int ITEMS>
__global__ __launch_bounds__(kBlockSelThreads) void block_select_kernel(
    const float* __restrict__ scores, int P, int sel, int score_order, int32_t* __restrict__ ids,
    float* __restrict__ out_scores, int32_t* __restrict__ tokens, int KP, int first_key) {
  __shared__ uint32_t hist[kBlockSelBins];
  __shared__ uint32_t red_mm[3 * kBlockSelWaves];  // per-wave min, max, count
  __shared__ uint32_t red_h[kBlockSelWaves];       // the histograms' scans
  __shared__ uint32_t red_s[kBlockSelWaves];       // the placement scan
  __shared__ uint32_t found[3];
  __shared__ uint2 staged[kRankSortMax];
  __shared__ uint32_t cand[kBlockSelThreads];
  __shared__ uint32_t ncand, nstage;
  const int t = threadIdx.x;
  const int lane = lane_id(), wave = t >> 6;
  const float* srow = scores + (int64_t)blockIdx.x * P;
  int32_t* orow = ids + (int64_t)blockIdx.x * sel;
  float* osc = out_scores + (int64_t)blockIdx.x * sel;
  // entry i of the row is pool `id` (-1: none); with `tokens`, its KP token
  // slots are written too (expand_selection fused into the selection)
  int32_t* trow = tokens ? tokens + (int64_t)blockIdx.x * sel * KP : nullptr;
  auto put = [&](uint32_t i, int32_t id, float v) {
    orow[i] = id;
    osc[i] = v;
    if (trow)
      for (int j = 0; j < KP; ++j) trow[(int64_t)i * KP + j] = id >= 0 ? first_key + id * KP + j : -1;
  };

  // The first histogram's bins and the append counters start at zero (the
  // barrier after the loads publishes them).
  hist[2 * t] = 0u;
  hist[2 * t + 1] = 0u;
  if (t == 0) {
    ncand = 0u;
    nstage = 0u;
  }

  // Load; -inf (an invalid pool) and slots past P never count.
  uint32_t u[ITEMS];
  uint32_t nloc = 0u, kmin = 0xFFFFFFFFu, kmax = 0u;
  const int p0 = t * ITEMS;
  if constexpr (ITEMS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < ITEMS; j += 4) {
      float4 v;
      if (p0 + j + 3 < P && (reinterpret_cast<uintptr_t>(srow) & 15u) == 0u) {
        v = *reinterpret_cast<const float4*>(srow + p0 + j);
      } else {
        v.x = p0 + j < P ? srow[p0 + j] : -__builtin_inff();
        v.y = p0 + j + 1 < P ? srow[p0 + j + 1] : -__builtin_inff();
        v.z = p0 + j + 2 < P ? srow[p0 + j + 2] : -__builtin_inff();
        v.w = p0 + j + 3 < P ? srow[p0 + j + 3] : -__builtin_inff();
      }
      u[j] = v.x == -__builtin_inff() ? 0u : ord_key(v.x);
      u[j + 1] = v.y == -__builtin_inff() ? 0u : ord_key(v.y);
      u[j + 2] = v.z == -__builtin_inff() ? 0u : ord_key(v.z);
      u[j + 3] = v.w == -__builtin_inff() ? 0u : ord_key(v.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const float v = p0 + j < P ? srow[p0 + j] : -__builtin_inff();
      u[j] = v == -__builtin_inff() ? 0u : ord_key(v);
    }
  }
  // Key 0 is below every finite score's key (ord_key(-inf) = 0x007FFFFF), so
  // it marks "not a candidate".
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    if (u[j] != 0u) {
      ++nloc;
      kmin = min(kmin, u[j]);
      kmax = max(kmax, u[j]);
    }
  }
  // Per-wave count / min / max, combined after one barrier.
  const uint32_t wcnt = wave_reduce(nloc, [](uint32_t x, uint32_t y) { return x + y; });
  const uint32_t wmin = wave_min(kmin), wmax = wave_max(kmax);
  if (lane == 0) {
    red_mm[wave] = wmin;
    red_mm[kBlockSelWaves + wave] = wmax;
    red_mm[2 * kBlockSelWaves + wave] = wcnt;
  }
  __syncthreads();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u, nvalid = 0u;
#pragma unroll
  for (int w = 0; w < kBlockSelWaves; ++w) {
    lo = min(lo, red_mm[w]);
    hi = max(hi, red_mm[kBlockSelWaves + w]);
    nvalid += red_mm[2 * kBlockSelWaves + w];
  }

  // Threshold key T, how many entries equal to T to keep, and (when known)
  // how many entries equal T in all.
  constexpr uint32_t kUnknown = 0xFFFFFFFFu;
  uint32_t T = 0u, need_eq = 0u, neq = kUnknown;
  const uint32_t k = (uint32_t)sel;
  bool resolved = false;
  uint32_t span = hi - lo, rem = k;
  if (nvalid > k && span != 0u) {
    // First round on float-linear bins of [min, max] (monotone in the score),
    // which spread a row's scores evenly: the bin holding rank k usually has
    // a few keys, and the threshold is found among them by direct counting.
    const float base_h = 0.5f * ord_to_float(lo);
    const float fspan = 0.5f * ord_to_float(hi) - base_h;
    const float scale = fspan > 0.f ? fminf((float)kBlockSelBins / fspan, 3.4e38f) : 0.f;
    uint32_t bn[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const float d = __fmul_rn(__fsub_rn(__fmul_rn(0.5f, ord_to_float(u[j])), base_h), scale);
      bn[j] = (uint32_t)fminf(fmaxf(d, 0.f), (float)(kBlockSelBins - 1));
      if (u[j] != 0u) atomicAdd(&hist[bn[j]], 1u);
    }
    __syncthreads();
    {
      const uint32_t h0 = hist[2 * t], h1 = hist[2 * t + 1];
      const uint2 sc = block_incl_scan(h0 + h1, red_h);
      const uint32_t after = sc.y - sc.x;
      if (h1 + after >= rem && after < rem) {
        found[0] = (uint32_t)(2 * t + 1);
        found[1] = after;
      } else if (h0 + h1 + after >= rem && h1 + after < rem) {
        found[0] = (uint32_t)(2 * t);
        found[1] = h1 + after;
      }
    }
    __syncthreads();
    const uint32_t fb = found[0];
    const uint32_t ncb = hist[fb];
    rem -= found[1];
    if (ncb <= (uint32_t)kBlockSelThreads) {
#pragma unroll
      for (int j = 0; j < ITEMS; ++j)
        if (u[j] != 0u && bn[j] == fb) cand[atomicAdd(&ncand, 1u)] = u[j];
      __syncthreads();
      if ((uint32_t)t < ncb) {
        const uint32_t me = cand[t];
        uint32_t gt = 0u, eq = 0u;
        for (uint32_t i = 0; i < ncb; ++i) {
          const uint32_t o = cand[i];
          gt += o > me ? 1u : 0u;
          eq += o == me ? 1u : 0u;
        }
        // every thread holding the threshold key agrees; its bin holds
        // every key equal to it, so eq counts them all
        if (gt < rem && rem <= gt + eq) {
          found[0] = me;
          found[1] = rem - gt;
          found[2] = eq;
        }
      }
      __syncthreads();
      T = found[0];
      need_eq = found[1];
      neq = found[2];
      resolved = true;
    } else {
      // many keys in one bin: continue with the radix rounds on its key range
      uint32_t bl = 0xFFFFFFFFu, bh = 0u;
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        if (u[j] != 0u && bn[j] == fb) {
          bl = min(bl, u[j]);
          bh = max(bh, u[j]);
        }
      }
      bl = wave_min(bl);
      bh = wave_max(bh);
      if (lane == 0) {  // red_mm's readers passed three barriers since
        red_mm[wave] = bl;
        red_mm[kBlockSelWaves + wave] = bh;
      }
      __syncthreads();
      lo = 0xFFFFFFFFu;
      hi = 0u;
#pragma unroll
      for (int w = 0; w < kBlockSelWaves; ++w) {
        lo = min(lo, red_mm[w]);
        hi = max(hi, red_mm[kBlockSelWaves + w]);
      }
      span = hi - lo;
    }
  }
  if (nvalid > k && !resolved) {
    while (true) {
      if (span == 0u) {
        T = lo;
        need_eq = rem;
        break;
      }
      const int bits = 32 - __builtin_clz(span);
      const int shift = bits > kBlockSelBinBits ? bits - kBlockSelBinBits : 0;
      __syncthreads();  // readers of hist / found from the last round are done
      hist[2 * t] = 0u;
      hist[2 * t + 1] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const uint32_t d = u[j] - lo;
        if (u[j] != 0u && u[j] >= lo && d <= span) atomicAdd(&hist[d >> shift], 1u);
      }
      __syncthreads();
      // suffix sums: S(b) = entries in bins >= b; find b with S(b) >= rem > S(b + 1)
      const uint32_t h0 = hist[2 * t], h1 = hist[2 * t + 1];
      const uint2 sc = block_incl_scan(h0 + h1, red_h);
      const uint32_t after = sc.y - sc.x;  // entries in bins above 2t + 1
      if (h1 + after >= rem && after < rem) {
        found[0] = (uint32_t)(2 * t + 1);
        found[1] = after;
      } else if (h0 + h1 + after >= rem && h1 + after < rem) {
        found[0] = (uint32_t)(2 * t);
        found[1] = h1 + after;
      }
      __syncthreads();
      const uint32_t b = found[0];
      rem -= found[1];
      lo += b << shift;
      if (shift == 0) {  // bins of one key: bin b holds every key equal to T
        T = lo;
        need_eq = rem;
        neq = hist[b];
        break;
      }
      const uint32_t width = (1u << shift) - 1u;
      span = min(span - (b << shift), width);
    }
  }

  // The row's entries: keys above T (every valid key if the row has at most
  // k), and the first need_eq keys equal to T (pool-id order).
  const bool cut = nvalid > k;
  const uint32_t nsel = cut ? k : nvalid;  // min(nvalid, sel)
  const bool rank_sort = score_order && sel <= kRankSortMax;
  const bool direct = rank_sort && (!cut || (neq != kUnknown && k - need_eq + neq <= kRankSortMax));
  uint32_t nst = nsel;  // entries on the ranking list
  if (direct) {
    // Append the keys above T and all keys equal to T, in any order (one
    // LDS atomic per wavefront); the ranks put the equal ones in pool-id
    // order and drop those past k.
    uint32_t mine = 0u;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) mine += (u[j] != 0u && (!cut || u[j] >= T)) ? 1u : 0u;
    const uint32_t incl = wave_incl_scan(mine);
    uint32_t base = 0u;
    if (lane == kWave - 1) base = atomicAdd(&nstage, incl);
    uint32_t pos = lane_value(base, kWave - 1) + incl - mine;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if (u[j] != 0u && (!cut || u[j] >= T)) staged[pos++] = make_uint2(u[j], (uint32_t)(p0 + j));
    nst = cut ? k - need_eq + neq : nvalid;
  } else {
    // Placement in pool-id order: one block scan of (equal count << 16 |
    // above count) gives every selected key its slot = keys above T before
    // it + min(keys equal to T before it, need_eq).  (Counts fit 16 bits:
    // at most 32768 pools.)
    uint32_t ab_loc = 0u, eq_loc = 0u;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      ab_loc += (u[j] != 0u && (!cut || u[j] > T)) ? 1u : 0u;
      eq_loc += (cut && u[j] == T) ? 1u : 0u;
    }
    const uint2 ss = block_incl_scan((eq_loc << 16) | ab_loc, red_s);
    const uint32_t ab_before = (ss.x - ((eq_loc << 16) | ab_loc)) & 0xFFFFu;
    uint32_t eq_before = (ss.x - ((eq_loc << 16) | ab_loc)) >> 16;
    uint32_t nab = 0u;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const bool above = u[j] != 0u && (!cut || u[j] > T);
      const bool eq = cut && u[j] == T;
      const bool s = above || (eq && eq_before < need_eq);
      if (s) {
        const uint32_t pos = ab_before + nab + min(eq_before, need_eq);
        if (rank_sort) {
          staged[pos] = make_uint2(u[j], (uint32_t)(p0 + j));
        } else {
          put(pos, p0 + j, ord_to_float(u[j]));
        }
      }
      nab += above ? 1u : 0u;
      eq_before += eq ? 1u : 0u;
    }
  }
  if (rank_sort) {
    // rank of each listed entry under (score desc, pool id asc): `tpe`
    // consecutive threads split the comparisons against the others, then
    // sum their counts; ranks below nsel are written
    __syncthreads();
    int tpe = kBlockSelThreads / kRankSortMax;
    while (tpe * 2 * (int)nst <= kBlockSelThreads && tpe < kWave) tpe *= 2;
    const uint32_t e = (uint32_t)(t / tpe), part = (uint32_t)(t % tpe);
    uint32_t r = 0u;
    uint2 me = make_uint2(0u, 0u);
    if (e < nst) {
      me = staged[e];
#pragma unroll 4
      for (uint32_t i = part; i < nst; i += (uint32_t)tpe) {
        const uint2 o = staged[i];
        r += (o.x > me.x || (o.x == me.x && o.y < me.y)) ? 1u : 0u;
      }
    }
    for (int off = 1; off < tpe; off <<= 1) r += (uint32_t)__shfl_xor((int)r, off);
    if (e < nst && part == 0u && r < nsel) {
      put(r, (int32_t)me.y, ord_to_float(me.x));
    }
  }
  for (int i = (int)nsel + t; i < sel; i += kBlockSelThreads) put((uint32_t)i, -1, -__builtin_inff());
}

// Waves per row and store capacity for select_k = sel within `lds_limit`.
TopkRowsPlan plan_topk_rows(int sel, int64_t P, size_t lds_limit) {
  TopkRowsPlan pl{};
  const int cap = ((sel + 4 * kWave) + kWave - 1) / kWave * kWave;
  for (int NW = 16; NW >= 1; NW /= 2) {
    if (NW > 1 && (int64_t)NW * kWave * 2 > P) continue;  // at least two loads per lane
    const size_t lds = (size_t)NW * ((size_t)cap * 8 + kSelScratchBytes) +
                       (NW > 1 ? (size_t)NW * sel * 8 + 16 * 4 : 0);
    if (lds <= lds_limit) {
      pl.waves = NW;
      pl.cap = cap;
      pl.lds_bytes = lds;
      return pl;
    }
  }
  return pl;
}

hipError_t launch_topk_pools(const TopkPoolsArgs& a, const TopkRowsPlan& pl, hipStream_t st) {
  if (a.Q <= 0) return hipSuccess;
  if (a.P <= (int64_t)kBlockSelThreads * 32) {
    const bool ranked = a.sort && a.sel <= kRankSortMax;
    // the rows are final when the kernel ends (no row sort follows): then
    // it writes the token ids as well
    int32_t* tok = (a.tokens && (!a.sort || ranked)) ? a.tokens : nullptr;
#define DSAI_ITEMS(n)                                                                          \
    if (a.P <= (int64_t)kBlockSelThreads * n) {                                                \
      hipLaunchKernelGGL(block_select_kernel<n>, dim3((unsigned)a.Q), dim3(kBlockSelThreads), \
                         0, st, a.scores, (int)a.P, a.sel, (int)a.sort, a.pool_ids,            \
                         a.pool_scores, tok, a.KP, a.first_key);                               \
    } else
    DSAI_ITEMS(1) DSAI_ITEMS(2) DSAI_ITEMS(4) DSAI_ITEMS(8) DSAI_ITEMS(16) DSAI_ITEMS(32) {}
#undef DSAI_ITEMS
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && a.sort && !ranked)
      e = launch_sort_rows(a.pool_ids, a.pool_scores, a.Q, a.sel, st);
    if (e != hipSuccess || !a.tokens || tok) return e;
    ExpandArgs x;
    x.pool_ids = a.pool_ids; x.Q = a.Q; x.sel = a.sel; x.KP = a.KP; x.first_key = a.first_key;
    x.tokens = a.tokens;
    return launch_expand(x, st);
  }
  hipError_t e = hipFuncSetAttribute((const void*)topk_rows_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl.lds_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)a.Q), dim3(pl.waves * kWave), pl.lds_bytes,
                     st, a.scores, (int)a.P, a.sel, pl.cap, pl.waves, a.pool_ids, a.pool_scores);
  e = hipGetLastError();
  if (e == hipSuccess && a.sort) e = launch_sort_rows(a.pool_ids, a.pool_scores, a.Q, a.sel, st);
  if (e != hipSuccess || !a.tokens) return e;
  ExpandArgs x;
  x.pool_ids = a.pool_ids; x.Q = a.Q; x.sel = a.sel; x.KP = a.KP; x.first_key = a.first_key;
  x.tokens = a.tokens;
  return launch_expand(x, st);
}

// ---------------------------------------------------------------------------
// expand_selection (glm5next_dsa: writes -1 over the whole index row before
// any index, so every slot is written).  One thread per (row, selected pool)
// writes the pool's KP slots: -1 for a missing pool, else the pool's token
// ids; each output slot is written exactly once, coalesced.  An id past
// max_id (its token ids would not fit int32) counts as missing.
// ---------------------------------------------------------------------------
template <int KP>
__global__ __launch_bounds__(256) void expand_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                     int first_key, int32_t max_id,
                                                     int32_t* __restrict__ tok) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int32_t p = ids[e];
  const bool ok = p >= 0 && p <= max_id;
  const int32_t t0 = ok ? first_key + p * KP : 0;  // no overflow: p <= max_id
  int32_t v[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) v[j] = ok ? t0 + j : -1;
  int32_t* o = tok + e * KP;
  if constexpr (KP == 4) {
    *reinterpret_cast<int4*>(o) = make_int4(v[0], v[1], v[2], v[3]);
  } else if constexpr (KP == 8) {
    reinterpret_cast<int4*>(o)[0] = make_int4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<int4*>(o)[1] = make_int4(v[4], v[5], v[6], v[7]);
  } else if constexpr (KP == 2) {
    *reinterpret_cast<int2*>(o) = make_int2(v[0], v[1]);
  } else {
#pragma unroll
    for (int j = 0; j < KP; ++j) o[j] = v[j];
  }
}

hipError_t launch_expand(const ExpandArgs& a, hipStream_t st) {
  const int64_t n = a.Q * a.sel;
  if (n <= 0) return hipSuccess;
  // largest pool id whose last token id, first_key + id * KP + KP - 1, fits int32
  const int64_t max_id64 = ((int64_t)2147483647 - a.first_key + 1) / a.KP - 1;
  const int32_t max_id = (int32_t)(max_id64 < 2147483647 ? max_id64 : 2147483647);
  const unsigned blocks = (unsigned)((n + 255) / 256);
#define DSAI_KP(kp)                                                                           \
  case kp:                                                                                    \
    hipLaunchKernelGGL(expand_kernel<kp>, dim3(blocks), dim3(256), 0, st, a.pool_ids, n,      \
                       a.first_key, max_id, a.tokens);                                        \
    break;
  switch (a.KP) {
    DSAI_KP(1) DSAI_KP(2) DSAI_KP(3) DSAI_KP(4) DSAI_KP(5) DSAI_KP(6) DSAI_KP(7) DSAI_KP(8)
    default:
      return hipErrorInvalidValue;
  }
#undef DSAI_KP
  return hipGetLastError();
}

}  // namespace dsai
