// Fused lightning-indexer score + causal/compressed mask + per-query top-k.
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
// row's top k is sorted (stable LSD radix) and written.  No score ever goes to
// device memory.  Blocks are numbered heaviest (largest t) first so the
// causal imbalance is absorbed by the dispatcher.
#include "internal.h"
#include "score_tile.h"
#include "topk_wave.h"

namespace dsai {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int HP, int D>
__global__ __launch_bounds__(kThreads) void score_topk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    int S, int Skv, int B, int H, int ratio, int topk, int row_begin, int row_end, int R, int cap,
    int stage_bytes, int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  extern __shared__ __align__(16) char smem_raw[];
  lds_char* smem = (lds_char*)smem_raw;
  using G = TileGeom<D>;

  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();

  lds_char* tile = smem;
  lds_u32* hist = (lds_u32*)(smem + stage_bytes) + wave * 256;
  lds_u32* rowkey = (lds_u32*)(smem + stage_bytes + R * 1024) + (size_t)wave * 2 * cap;
  const RowStore rs{rowkey, rowkey + cap, hist};

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
  __syncthreads();  // the tile region now holds the sort counters
  if (!active) return;
  wave_lds_sync();
  count = wave_keep_topk(rs, count, topk, &tau);
  lds_u32* cnt = (lds_u32*)smem + wave * 16 * kWave;
  const SortedView sv = wave_sort_desc(rs, count, (uint32_t)topk + 64u, cnt);
  const int64_t orow = ((int64_t)b * S + t) * topk;
  wave_write_row(sv, count, topk, out_idx + orow, out_score + orow);
}

// Candidate store entries per row: room for the top k plus at least one
// tile of new candidates, and for the sort's two padded halves.
static int store_cap(int topk) { return 2 * topk + 128; }

static size_t lds_bytes(int D, int R, int topk, int* stage_out) {
  const int row_bytes = 2 * D + 16;
  int stage = 64 * row_bytes;
  if (stage < R * 16 * kWave * 4) stage = R * 16 * kWave * 4;  // sort counters reuse it
  stage = (stage + 15) & ~15;
  if (stage_out) *stage_out = stage;
  return (size_t)stage + (size_t)R * 1024 + (size_t)R * store_cap(topk) * 8;
}

int score_topk_rows_per_block(int D, int topk, size_t lds_limit) {
  for (int R = kWaves; R >= 1; --R)
    if (lds_bytes(D, R, topk, nullptr) <= lds_limit) return R;
  return 0;
}

template <int HP, int D>
static hipError_t launch_t(const ScoreTopkArgs& a, int R, hipStream_t st) {
  int stage = 0;
  const size_t lds = lds_bytes(D, R, a.topk, &stage);
  auto kern = score_topk_kernel<HP, D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int cap = store_cap(a.topk);
  const int64_t chunk = a.chunk_rows > 0 ? a.chunk_rows : a.S;
  for (int64_t r0 = 0; r0 < a.S; r0 += chunk) {
    const int64_t r1 = (r0 + chunk < a.S) ? r0 + chunk : a.S;
    const int64_t nrb = (r1 - r0 + R - 1) / R;
    const int64_t blocks = nrb * a.B;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreads), lds, st, a.q, a.k, a.w,
                       (int)a.S, (int)a.Skv, (int)a.B, a.H, a.ratio, a.topk, (int)r0, (int)r1, R,
                       cap, stage, a.out_idx, a.out_score);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_score_topk(const ScoreTopkArgs& a, int R, hipStream_t st) {
  const int HP = a.H <= 16 ? 16 : (a.H <= 32 ? 32 : 64);
#define DSAI_CASE(hp, d) \
  if (HP == hp && a.D == d) return launch_t<hp, d>(a, R, st);
  DSAI_CASE(16, 32) DSAI_CASE(16, 64) DSAI_CASE(16, 128)
  DSAI_CASE(32, 32) DSAI_CASE(32, 64) DSAI_CASE(32, 128)
  DSAI_CASE(64, 32) DSAI_CASE(64, 64) DSAI_CASE(64, 128)
#undef DSAI_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsai
