// Fused lightning-indexer score + causal/compressed mask + per-query top-k
// selection.
//
// Contract: NeMo AutoModel page
// "nemo_automodel.components.models.deepseek_v4.kernels.tilelang_indexer"
// (v4_lighting_indexer: index_q [seqlen, batch, heads, dim] bf16, index_k
// [seqlen_kv, batch, dim] bf16, weights [seqlen, batch, heads] fp32,
// compress_ratio, topk; result [batch, seqlen, topk]); causal masking per the
// module summary, with key s visible to query t iff s < floor((t+1)/ratio).
//
// One workgroup = 4 wavefronts, two workgroups per CU; each wavefront owns one
// query row of a block of up to 4 consecutive rows of one batch, so the rows
// of a block see nearly the same keys.  The block streams its keys through
// LDS in 32-key tiles (loaded once per block, shared by its rows); each wavefront
// scores the tile on the matrix cores (TileScorer) and records the scores in
// its LDS row store:
//   dense   when every visible key fits: the order key of key s goes to slot s
//           (no indices, no selection until the end);
//   filter  otherwise: keys beating the row's running threshold are appended
//           with their index; when the store fills, a radix select cuts it to
//           the top k and raises the threshold.
// After the last tile the row's top k is selected exactly and written in
// ascending index order; no score goes to device memory.  (Score-descending
// order is produced by the row sort.)  Blocks are numbered heaviest (largest
// t) first so the causal imbalance is absorbed by the dispatcher.
#include "internal.h"
#include "score_tile.h"
#include "topk_wave.h"

namespace dsai {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int HP, int D, bool DENSE, typename IdxT>
__global__ __launch_bounds__(kThreads) void score_select_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    int S, int Skv, int B, int H, int ratio, int topk, int row_begin, int row_end, int R, int cap,
    int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  extern __shared__ __align__(16) char smem_raw[];
  lds_char* smem = (lds_char*)smem_raw;
  using G = TileGeom<D>;
  constexpr int kScratch = DENSE ? 1024 : kSelScratchBytes;
  // Dense rows reuse the tile region for their side lists after the loop.
  constexpr int kTileRegion =
      (DENSE && G::kTileBytes < kWaves * 1024) ? kWaves * 1024 : G::kTileBytes;

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform
  const int lane = lane_id();
  const int row_bytes = DENSE ? cap * 4 : cap * 4 + ((cap * (int)sizeof(IdxT) + 15) & ~15);

  lds_char* tile = smem;
  lds_u32* scratch = (lds_u32*)(smem + kTileRegion + wave * kScratch);
  lds_char* mine = smem + kTileRegion + R * kScratch + wave * row_bytes;
  // Dense rows get their side list in the tile region once the loop is done.
  lds_u32* side = DENSE ? (lds_u32*)(smem + wave * 1024) : scratch + 256;
  const RowStore<IdxT> rs{(lds_u32*)mine, (DSAI_LDS IdxT*)(mine + cap * 4), scratch, side, 256u};

  const int nrow = row_end - row_begin;
  const int nrb = (nrow + R - 1) / R;
  const int j = blockIdx.x / B;
  const int b = blockIdx.x - j * B;
  const int t0 = row_begin + (nrb - 1 - j) * R;
  const int t = t0 + wave;
  const bool active = (wave < R) && (t < row_end);
  const int t_last = min(t0 + R, row_end) - 1;
  const int n_max = min(Skv, (t_last + 1) / ratio);
  const int n_t = active ? min(Skv, (t + 1) / ratio) : 0;
  const int ntiles = (n_max + G::kTileKeys - 1) / G::kTileKeys;

  TileScorer<HP, D> sc;
  const int64_t row = (int64_t)(active ? t : 0) * B + b;
  sc.load_query(q + row * H * D, w + row * H, H, active);

  uint32_t count = 0u, tau = 0u;
  TileLoader<D, kThreads> ld;
  const int64_t kbytes = ((int64_t)Skv * B - b) * D * 2;  // < 2^32 (checked on the host)
  ld.init(k + (int64_t)b * D, (uint32_t)(B * D), (uint32_t)(kbytes > 0 ? kbytes : 0));
  if (ntiles > 0) ld.load(0u);

  // Software pipeline: the products of tile `it` are issued before the
  // reduction and recording of tile it - 1, so the vector ALU work of one tile
  // overlaps the matrix-core work of the next.  The wave's tiles are a prefix
  // [0, nt_w) of the block's; the accumulators alternate between two register
  // sets (the loop body is unrolled twice so no copies are needed).
  constexpr int MT = TileScorer<HP, D>::MT;
  const int nt_w = (n_t + G::kTileKeys - 1) / G::kTileKeys;  // 0 when inactive
  auto record = [&](int it_rec, const floatx16 (&a)[MT]) {
    const float s = sc.reduce(a);  // lanes l and l + 32 hold key l % 32
    const uint32_t key = (uint32_t)(it_rec * G::kTileKeys + (lane & 31));
    const uint32_t u = ord_key(s);
    if constexpr (DENSE) {
      if (lane < 32) rs.key[key] = u;
    } else {
      wave_append(rs, count, lane < 32 && key < (uint32_t)n_t && u > tau, u, key);
      if (count > (uint32_t)(cap - G::kTileKeys)) count = wave_keep_topk(rs, count, topk, &tau);
    }
  };
  auto stage = [&](int it) {
    __syncthreads();
    ld.store(tile);
    __syncthreads();
    if (it + 1 < ntiles) ld.load((uint32_t)(it + 1) * G::kTileKeys);
  };
  auto step = [&](int it, floatx16 (&cur)[MT], const floatx16 (&old)[MT]) {
    stage(it);
    if (it < nt_w) {
      sc.mma(tile, cur);
      record(it - 1, old);
    } else if (it == nt_w) {
      record(it - 1, old);
    }
  };
  floatx16 acc0[MT], acc1[MT];
  if (ntiles > 0) {
    stage(0);
    if (nt_w > 0) sc.mma(tile, acc0);
  }
  for (int it = 1; it < ntiles; it += 2) {
    step(it, acc1, acc0);
    if (it + 1 < ntiles) step(it + 1, acc0, acc1);
  }
  if (nt_w > 0 && nt_w == ntiles) {
    if ((ntiles - 1) & 1) record(ntiles - 1, acc1);
    else record(ntiles - 1, acc0);
  }
  if constexpr (DENSE) __syncthreads();  // the tile region now holds the side lists
  if (!active) return;
  const int64_t orow = ((int64_t)b * S + t) * topk;
  if constexpr (DENSE) {
    dense_finish(rs.key, (uint32_t)n_t, (uint32_t)topk, rs.hist, rs.side, topk, out_idx + orow,
                 out_score + orow);
  } else {
    wave_finish_row(rs, count, topk, out_idx + orow, out_score + orow);
  }
}

namespace {

int store_row_bytes(int cap, int idx_bytes) { return cap * 4 + ((cap * idx_bytes + 15) & ~15); }

int tile_bytes_for(int D) { return 32 * (2 * D + 16); }

bool plan_dense(int D, int64_t Skv, int64_t budget, ScoreSelectPlan* p) {
  const int64_t tile = tile_bytes_for(D);
  const int64_t region = tile > kWaves * 1024 ? tile : kWaves * 1024;
  const int64_t cap = Skv > 0 ? ((Skv + 255) / 256) * 256 : 256;  // whole 256-key groups
  const int64_t lds = region + kWaves * 1024 + (int64_t)kWaves * cap * 4;
  if (lds > budget) return false;
  p->rows_per_block = kWaves;
  p->cap = (int)cap;
  p->dense = true;
  p->idx_bytes = 0;
  p->lds_bytes = (size_t)lds;
  return true;
}

bool plan_filter(int D, int topk, int64_t Skv, int64_t budget, int min_rows, ScoreSelectPlan* p) {
  const int64_t tile = tile_bytes_for(D);
  const int idx_bytes = Skv <= 65536 ? 2 : 4;
  const int need = topk + 8 * 32;
  for (int R = kWaves; R >= min_rows; --R) {
    const int64_t per_row = (budget - tile - (int64_t)R * kSelScratchBytes) / R;
    if (per_row <= 0) continue;
    int cap = (int)(per_row / (4 + idx_bytes)) & ~63;
    while (cap > 0 && store_row_bytes(cap, idx_bytes) > per_row) cap -= 64;
    if (cap < need) continue;
    p->rows_per_block = R;
    p->cap = cap;
    p->dense = false;
    p->idx_bytes = idx_bytes;
    p->lds_bytes = (size_t)(tile + (int64_t)R * kSelScratchBytes +
                            (int64_t)R * store_row_bytes(cap, idx_bytes));
    return true;
  }
  return false;
}

}  // namespace

// Launch geometry, in order of preference: two 4-row blocks per CU with a
// dense store (one slot per visible key), then with a filter store (the top
// k plus at least 8 tiles of candidates); then one block per CU, dense, then
// filter with as many rows as fit.
ScoreSelectPlan plan_score_select(int D, int topk, int64_t Skv, size_t lds_limit) {
  ScoreSelectPlan p{};
  const int64_t half = (int64_t)lds_limit / 2, full = (int64_t)lds_limit;
  if (plan_dense(D, Skv, half, &p)) return p;
  if (plan_filter(D, topk, Skv, half, kWaves, &p)) return p;
  if (plan_dense(D, Skv, full, &p)) return p;
  if (plan_filter(D, topk, Skv, full, 1, &p)) return p;
  return ScoreSelectPlan{};  // rows_per_block == 0: does not fit
}

template <int HP, int D, bool DENSE, typename IdxT>
static hipError_t launch_t(const ScoreTopkArgs& a, const ScoreSelectPlan& p, hipStream_t st) {
  auto kern = score_select_kernel<HP, D, DENSE, IdxT>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)p.lds_bytes);
  if (e != hipSuccess) return e;
  const int R = p.rows_per_block;
  const int64_t chunk = a.chunk_rows > 0 ? a.chunk_rows : a.S;
  for (int64_t r0 = 0; r0 < a.S; r0 += chunk) {
    const int64_t r1 = (r0 + chunk < a.S) ? r0 + chunk : a.S;
    const int64_t blocks = ((r1 - r0 + R - 1) / R) * a.B;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreads), p.lds_bytes, st, a.q, a.k,
                       a.w, (int)a.S, (int)a.Skv, (int)a.B, a.H, a.ratio, a.topk, (int)r0,
                       (int)r1, R, p.cap, a.out_idx, a.out_score);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.sort) return launch_sort_rows(a.out_idx, a.out_score, a.B * a.S, a.topk, st);
  return hipSuccess;
}

template <int HP, int D>
static hipError_t launch_hd(const ScoreTopkArgs& a, const ScoreSelectPlan& p, hipStream_t st) {
  if (p.dense) return launch_t<HP, D, true, uint16_t>(a, p, st);
  return p.idx_bytes == 2 ? launch_t<HP, D, false, uint16_t>(a, p, st)
                          : launch_t<HP, D, false, uint32_t>(a, p, st);
}

hipError_t launch_score_topk(const ScoreTopkArgs& a, const ScoreSelectPlan& p, hipStream_t st) {
  const int HP = a.H <= 32 ? 32 : 64;
#define DSAI_CASE(hp, d) \
  if (HP == hp && a.D == d) return launch_hd<hp, d>(a, p, st);
  DSAI_CASE(32, 32) DSAI_CASE(32, 64) DSAI_CASE(32, 128)
  DSAI_CASE(64, 32) DSAI_CASE(64, 64) DSAI_CASE(64, 128)
#undef DSAI_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsai
