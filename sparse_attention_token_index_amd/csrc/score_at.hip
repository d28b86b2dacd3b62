// Index scores at caller-supplied key indices: the topk_indices form of the
// indexer (NeMo AutoModel page "...deepseek_v4.kernels.tilelang_indexer":
// v4_lighting_indexer's optional topk_indices [batch, seqlen, topk] int32,
// and pytorch_extract_topk_scores, which gathers scores at given indices).
//
// One wavefront per (query row, batch); rows are independent, so there is
// no LDS and no barrier.  The supplied indices are consumed 32 at a time:
// lane (c, g) loads key idx[c]'s dims g*D/2 .. g*D/2 + D/2 - 1 straight into
// the B fragments of the fused indexer's tile scorer (128 contiguous bytes
// per lane at D = 128); the key rows of the next group and the indices of
// the one after are in flight while the current group is on the matrix
// cores (entry_tiles.h), and the score arithmetic
// (products, ReLU, head weights, cross-half sum) is the fused kernel's, so a
// key's score is bit-identical to the one the selection reports.  An entry
// outside [0, n_t) (padding -1, a masked or an out-of-range key) yields
// (-1, -inf); entries keep the supplied order.
#include "entry_tiles.h"
#include "internal.h"
#include "score_tile.h"

namespace dsai {

constexpr int kAtWaves = 4;

template <int HP, int D>
__global__ __launch_bounds__(kAtWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void
score_at_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const float* __restrict__ w, int S, int Skv, int B, int H, int ratio, int n,
                int row_begin, int row_end, const int32_t* sup, int32_t* out_idx,
                float* __restrict__ out_score) {
  using Scorer = TileScorer<HP, D>;
  using Frag = typename Scorer::Frag;
  using Acc = typename Scorer::Acc;
  constexpr int KS = D / 16;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = lane_id();
  const int64_t r = (int64_t)blockIdx.x * kAtWaves + wave;  // over (t - row_begin, b)
  const int64_t nrows = (int64_t)(row_end - row_begin) * B;
  if (r >= nrows) return;  // wave-uniform; no barriers below
  const int t = row_begin + (int)(r / B);
  const int b = (int)(r - (int64_t)(t - row_begin) * B);
  const int n_t = min(Skv, (t + 1) / ratio);

  Scorer sc;
  const int64_t qrow = (int64_t)t * B + b;
  sc.load_query(q + qrow * H * D, w + qrow * H, H, true);
  const int64_t orow = ((int64_t)b * S + t) * n;
  const int c = lane & 31, g = lane >> 5;

  if (n_t <= 0) {  // no visible key: every entry is (-1, -inf); nothing is read
    for (int j = lane; j < n; j += kWave) {
      out_idx[orow + j] = -1;
      out_score[orow + j] = -__builtin_inff();
    }
    return;
  }
  Acc acc;
  for_each_entry_tile<D, false>(sup, nullptr, k, orow, n, n_t, B, b, (n + 31) / 32,
                                [&](const EntryTile<D, false>& cur, int it) {
    sc.mma(cur.f, acc);
    const float x = sc.reduce(acc, 0) + 0.f;  // -0 -> +0
    const int j = it * 32 + c;
    if (g == 0 && j < n) {
      out_idx[orow + j] = cur.s;
      out_score[orow + j] = cur.s >= 0 ? x : -__builtin_inff();
    }
  });
}

template <int HP, int D>
static hipError_t launch_at_t(const ScoreAtArgs& a, hipStream_t st, hipStream_t st2) {
  const int64_t chunk = a.chunk_rows > 0 ? a.chunk_rows : a.S;
  int64_t ci = 0;
  for (int64_t r0 = 0; r0 < a.S; r0 += chunk, ++ci) {
    const int64_t r1 = (r0 + chunk < a.S) ? r0 + chunk : a.S;
    const int64_t blocks = ((r1 - r0) * a.B + kAtWaves - 1) / kAtWaves;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((score_at_kernel<HP, D>), dim3((unsigned)blocks), dim3(kAtWaves * 64), 0,
                       (st2 && (ci & 1)) ? st2 : st, a.q, a.k, a.w, (int)a.S, (int)a.Skv, (int)a.B, a.H, a.ratio, a.n,
                       (int)r0, (int)r1, a.sup, a.out_idx, a.out_score);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_score_at(const ScoreAtArgs& a, hipStream_t st, hipStream_t st2) {
  if (a.S <= 0 || a.B <= 0 || a.n <= 0) return hipSuccess;
  const int HP = a.H <= 32 ? 32 : 64;
#define DSAI_CASE(hp, d) \
  if (HP == hp && a.D == d) return launch_at_t<hp, d>(a, st, st2);
  DSAI_CASE(32, 32) DSAI_CASE(32, 64) DSAI_CASE(32, 128)
  DSAI_CASE(64, 32) DSAI_CASE(64, 64) DSAI_CASE(64, 128)
#undef DSAI_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsai
