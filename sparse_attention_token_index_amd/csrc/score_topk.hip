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
// One workgroup = 4 wavefronts; each wavefront owns one query row of a block
// of R consecutive rows (same batch), so the rows of a block see nearly the
// same keys.  The block streams its keys through LDS in 64-key tiles (loaded
// once per block, shared by its R rows); each wavefront scores the tile on
// the matrix cores (TileScorer) and appends the keys that beat its running
// threshold to its LDS candidate store.  When the store fills, a radix select
// cuts it to the top k and raises the threshold.  After the last tile the
// row's top k is written in ascending index order; no score ever goes to
// device memory.  (Score-descending order is produced by the row sort.)
// Blocks are numbered heaviest (largest t) first so the causal imbalance is
// absorbed by the dispatcher.
#include "internal.h"
#include "score_tile.h"
#include "topk_wave.h"

namespace dsai {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int HP, int D, typename IdxT>
__global__ __launch_bounds__(kThreads, 2) void score_select_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    int S, int Skv, int B, int H, int ratio, int topk, int row_begin, int row_end, int R, int cap,
    int stage_bytes, int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  extern __shared__ __align__(16) char smem_raw[];
  lds_char* smem = (lds_char*)smem_raw;
  using G = TileGeom<D>;

  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int row_bytes = cap * 4 + ((cap * (int)sizeof(IdxT) + 15) & ~15);

  lds_char* tile = smem;
  lds_char* mine = smem + stage_bytes + R * 1024 + wave * row_bytes;
  const RowStore<IdxT> rs{(lds_u32*)mine, (DSAI_LDS IdxT*)(mine + cap * 4),
                          (lds_u32*)(smem + stage_bytes) + wave * 256};

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
  const int64_t kstride = (int64_t)B * D;
  const uint16_t* kb = k + (int64_t)b * D;
  if (ntiles > 0) ld.load(kb, kstride, 0, Skv);

  for (int it = 0; it < ntiles; ++it) {
    __syncthreads();
    ld.store(tile);
    __syncthreads();
    if (it + 1 < ntiles) ld.load(kb, kstride, (int64_t)(it + 1) * G::kTileKeys, Skv);
    if (active && it * G::kTileKeys < n_t) {
      const float s = sc.score(tile);
      const uint32_t key = (uint32_t)(it * G::kTileKeys + lane);
      const uint32_t u = ord_key(s);
      wave_append(rs, count, key < (uint32_t)n_t && u > tau, u, key);
      if (count > (uint32_t)(cap - G::kTileKeys)) count = wave_keep_topk(rs, count, topk, &tau);
    }
  }
  if (!active) return;
  const int64_t orow = ((int64_t)b * S + t) * topk;
  wave_finish_row(rs, count, topk, out_idx + orow, out_score + orow);
}

namespace {

int store_row_bytes(int cap, int idx_bytes) { return cap * 4 + ((cap * idx_bytes + 15) & ~15); }

int stage_bytes_for(int D) { return 64 * (2 * D + 16); }

// Largest candidate-store capacity (a multiple of 64) for R rows in `budget`
// bytes of LDS.
int cap_for(int D, int R, int idx_bytes, size_t budget) {
  const long fixed = stage_bytes_for(D) + R * 1024;
  long per_row = ((long)budget - fixed) / R;
  if (per_row <= 0) return 0;
  int cap = (int)(per_row / (4 + idx_bytes)) & ~63;
  while (cap > 0 && store_row_bytes(cap, idx_bytes) > per_row) cap -= 64;
  return cap;
}

}  // namespace

// Pick rows per block and store capacity: prefer 4 rows and two blocks per
// CU (half the LDS each); the store must hold the top k plus room for at
// least 4 tiles of new candidates.  It never needs more than every visible
// key plus one tile.
ScoreSelectPlan plan_score_select(int D, int topk, int64_t Skv, size_t lds_limit) {
  ScoreSelectPlan p{};
  const int idx_bytes = Skv <= 65536 ? 2 : 4;
  const int need = topk + 4 * 64;
  const int64_t useful = ((Skv + 63) / 64) * 64 + 64;
  const size_t budgets[2] = {lds_limit / 2, lds_limit};
  for (size_t budget : budgets) {
    for (int R = kWaves; R >= 1; --R) {
      int cap = cap_for(D, R, idx_bytes, budget);
      if (cap < need) continue;
      if (cap > useful) cap = (int)useful;
      if (cap < need) cap = need;
      p.rows_per_block = R;
      p.cap = cap;
      p.idx_bytes = idx_bytes;
      p.lds_bytes = (size_t)stage_bytes_for(D) + R * 1024 + (size_t)R * store_row_bytes(cap, idx_bytes);
      return p;
    }
  }
  return p;  // rows_per_block == 0: does not fit
}

template <int HP, int D, typename IdxT>
static hipError_t launch_t(const ScoreTopkArgs& a, const ScoreSelectPlan& p, hipStream_t st) {
  auto kern = score_select_kernel<HP, D, IdxT>;
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
                       (int)r1, R, p.cap, stage_bytes_for(D), a.out_idx, a.out_score);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.sort) return launch_sort_rows(a.out_idx, a.out_score, a.B * a.S, a.topk, st);
  return hipSuccess;
}

hipError_t launch_score_topk(const ScoreTopkArgs& a, const ScoreSelectPlan& p, hipStream_t st) {
  const int HP = a.H <= 16 ? 16 : (a.H <= 32 ? 32 : 64);
#define DSAI_CASE(hp, d)                                                       \
  if (HP == hp && a.D == d)                                                    \
    return p.idx_bytes == 2 ? launch_t<hp, d, uint16_t>(a, p, st)              \
                            : launch_t<hp, d, uint32_t>(a, p, st);
  DSAI_CASE(16, 32) DSAI_CASE(16, 64) DSAI_CASE(16, 128)
  DSAI_CASE(32, 32) DSAI_CASE(32, 64) DSAI_CASE(32, 128)
  DSAI_CASE(64, 32) DSAI_CASE(64, 64) DSAI_CASE(64, 128)
#undef DSAI_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsai
