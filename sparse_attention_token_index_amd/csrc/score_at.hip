// Index scores at caller-supplied key indices: the topk_indices form of the
// indexer (NeMo AutoModel page "...deepseek_v4.kernels.tilelang_indexer":
// v4_lighting_indexer's optional topk_indices [batch, seqlen, topk] int32,
// and pytorch_extract_topk_scores, which gathers scores at given indices).
//
// One wavefront per (query row, batch); rows are independent, so there is
// no LDS and no barrier.  The supplied indices are consumed 32 at a time:
// lane (c, g) loads key idx[c]'s dims g*D/2 .. g*D/2 + D/2 - 1 straight into
// the B fragments of the fused indexer's tile scorer (128 contiguous bytes
// per lane at D = 128), the next group's indices and fragments are loaded
// while the current group is on the matrix cores, and the score arithmetic
// (products, ReLU, head weights, cross-half sum) is the fused kernel's, so a
// key's score is bit-identical to the one the selection reports.  An entry
// outside [0, n_t) (padding -1, a masked or an out-of-range key) yields
// (-1, -inf); entries keep the supplied order.
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

  // Entry j0 + c of the row and its key's fragments (key 0, visible whenever
  // n_t > 0, stands in for an unusable entry; its products are discarded).
  auto fetch = [&](int j0, int& s, Frag& bf) {
    const int j = j0 + c;
    s = j < n ? sup[orow + j] : -1;
    if (n_t > 0) {  // wave-uniform; with no visible key nothing is read
      const int key = (s >= 0 && s < n_t) ? s : 0;
      const uint16_t* src = k + ((int64_t)key * B + b) * D + g * (D / 2);
#pragma unroll
      for (int x = 0; x < KS; ++x) bf[x] = *reinterpret_cast<const bf16x8*>(src + 8 * x);
    } else {
#pragma unroll
      for (int x = 0; x < KS; ++x) bf[x] = bf16x8{};
    }
  };
  const int ngroups = (n + 31) / 32;
  int s0 = -1, s1 = -1;
  Frag f0, f1;
  Acc acc;
  if (ngroups > 0) fetch(0, s0, f0);
  for (int it = 0; it < ngroups; ++it) {
    // the current group is in (s0, f0); load the next into (s1, f1)
    if (it + 1 < ngroups) fetch((it + 1) * 32, s1, f1);
    sc.mma(f0, acc);
    const float x = sc.reduce(acc, 0) + 0.f;  // -0 -> +0
    const int j = it * 32 + c;
    if (g == 0 && j < n) {
      const bool ok = s0 >= 0 && s0 < n_t;
      out_idx[orow + j] = ok ? s0 : -1;
      out_score[orow + j] = ok ? x : -__builtin_inff();
    }
    s0 = s1;
#pragma unroll
    for (int x2 = 0; x2 < KS; ++x2) f0[x2] = f1[x2];
  }
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
