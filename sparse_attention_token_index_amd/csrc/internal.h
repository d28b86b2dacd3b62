// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsai {

struct ScoreTopkArgs {
  const uint16_t* q;  // [S, B, H, D] bf16
  const uint16_t* k;  // [Skv, B, D] bf16
  const float* w;     // [S, B, H]
  int64_t S, Skv, B;
  int H, D, ratio, topk;
  int64_t chunk_rows;  // 0: all rows in one launch
  bool sort;           // score-descending rows (else ascending index order)
  bool est_cuts = true;  // filter store: cuts to an estimated rank (else to k)
  const int32_t* sup = nullptr;  // [B, S, topk] supplied indices (dense plan only;
                                 // may alias out_idx): their scores, no selection
  int32_t* out_idx;    // [B, S, topk]
  float* out_score;    // [B, S, topk]
};

// Launch geometry of the fused score + select kernel.
struct ScoreSelectPlan {
  int waves;           // wavefronts per workgroup
  int rows_per_wave;   // query rows per wavefront
  int rows_per_block;  // 0: the request does not fit in LDS
  int cap;             // store entries per row
  bool dense;          // one slot per visible key (index = slot)
  int idx_bytes;       // filter store: 2 (Skv <= 65536) or 4
  size_t lds_bytes;
};

struct KpoolArgs {
  const uint16_t* k_normed;  // [N, D]
  const float* gate;         // [N, D]
  const uint8_t* valid;      // [N]
  const float* ape;          // [KP, D]
  int D, KP;
  int64_t first_key, P;
  uint16_t* pool_k;  // [P, D]
  int32_t* pool_tok;
  uint8_t* pool_valid;
};

struct PooledScoresArgs {
  const uint16_t* q;  // [Q, H, D]
  const float* w;     // [Q, H]
  const uint16_t* pool_k;
  const uint8_t* pool_valid;
  const int32_t* limit;  // [Q] visible-pool bound per row, or null (all pools)
  int64_t Q, P;
  int H, D;
  float* scores;  // [Q, P]
};

struct TopkPoolsArgs {
  const float* scores;  // [Q, P]
  int64_t Q, P;
  int sel;
  int32_t* pool_ids;    // [Q, sel]
  float* pool_scores;   // [Q, sel]
  bool sort;            // score-descending rows (else ascending pool id)
  int32_t* tokens = nullptr;  // optional [Q, sel * KP]: the rows expanded to token ids
  int KP = 1, first_key = 0;
};

struct ExpandArgs {
  const int32_t* pool_ids;  // [Q, sel]
  int64_t Q;
  int sel, KP, first_key;
  int32_t* tokens;  // [Q, sel * KP]
};

// Launch geometry of the pooled top-k kernel.
struct TopkRowsPlan {
  int waves;  // wavefronts per row (0: does not fit)
  int cap;    // candidate-store entries per wavefront
  size_t lds_bytes;
};

ScoreSelectPlan plan_score_select(int HP, int D, int topk, int64_t Skv, size_t lds_limit);
TopkRowsPlan plan_topk_rows(int sel, int64_t P, size_t lds_limit);

// Packed sequences in one launch of the fused kernel: up to kPackedMax
// sequences, each the B = 1 problem on its own rows and keys (rows and keys
// counted from q0 / k0 of the packed tensors).  Workgroups blk_begin[i] ..
// blk_begin[i + 1] - 1 belong to sequence i; blk_begin[n] is the grid and
// the entries after it hold INT_MAX.  The table travels in the kernel
// arguments.
constexpr int kPackedMax = 64;
struct PackedSeqs {
  int n;
  int blk_begin[kPackedMax + 1];
  int q0[kPackedMax], k0[kPackedMax], S[kPackedMax], Skv[kPackedMax];
};
struct PackedTopkArgs {
  const uint16_t* q;  // [Tq, H, D] bf16
  const uint16_t* k;  // [Tk, D] bf16
  const float* w;     // [Tq, H]
  int H, D, ratio, topk;
  int32_t* out_idx;   // [Tq, topk], ascending index order
  float* out_score;
  bool est_cuts = true;  // filter store: cuts to an estimated rank (else to k)
};
hipError_t launch_score_topk_packed(const PackedTopkArgs& a, const PackedSeqs& seqs,
                                    const ScoreSelectPlan& p, hipStream_t st);

// Chunk launches (ScoreTopkArgs::chunk_rows) alternate between st and st2
// when st2 is not null (two chunks in flight); the score-order pass is the
// caller's (launch_sort_rows on the joined stream).
hipError_t launch_score_topk(const ScoreTopkArgs& a, const ScoreSelectPlan& p, hipStream_t st,
                             hipStream_t st2);

// Scores at supplied key indices (score_at.hip).
struct ScoreAtArgs {
  const uint16_t* q;   // [S, B, H, D] bf16
  const uint16_t* k;   // [Skv, B, D] bf16
  const float* w;      // [S, B, H]
  int64_t S, Skv, B;
  int H, D, ratio, n;  // n: supplied entries per row
  int64_t chunk_rows;  // 0: all rows in one launch
  const int32_t* sup;  // [B, S, n] supplied key indices (may alias out_idx)
  int32_t* out_idx;    // [B, S, n]
  float* out_score;    // [B, S, n]
};
hipError_t launch_score_at(const ScoreAtArgs& a, hipStream_t st, hipStream_t st2);

// k_norm: LayerNorm with a bias over rows of D channels (k_norm.hip).
struct KNormArgs {
  const uint16_t* x;      // [n, D] bf16
  const uint16_t* gamma;  // [D] bf16
  const uint16_t* beta;   // [D] bf16
  float eps;
  int64_t n;
  int D;
  uint16_t* y;            // [n, D] bf16
};
hipError_t launch_k_norm(const KNormArgs& a, hipStream_t st);
// Gradients of the selected scores (indexer_bwd.hip).  acc_k is an fp32
// [Skv, B, D] accumulator the launch clears and then converts into grad_k.
// The key gradients (clear, grouping, products, convert) go to st_keys and
// the per-row gradients (grad_q, grad_w) to st_rows; they share no output,
// so the two may run concurrently (st_rows may be st_keys).
#define DSAI_BWD_MAX_KEY_BLOCKS 1024
struct BackwardPlan {
  bool grouped;        // key-block kernels (else a per-entry atomic scatter)
  int nbk;             // key blocks of 256 keys
  int chunk_rows;      // query rows per key-block workgroup
  int nchunks;
  size_t bounds_off;   // workspace layout (bytes)
  size_t ent_off;
  size_t bytes;        // total workspace
};
BackwardPlan plan_backward(int64_t S, int64_t Skv, int64_t B, int D, int n, int ratio);

struct BackwardArgs {
  const uint16_t* q;    // [S, B, H, D] bf16
  const uint16_t* k;    // [Skv, B, D] bf16
  const float* w;       // [S, B, H]
  const int32_t* sup;   // [B, S, n] key indices
  const float* grad;    // [B, S, n] incoming gradient of the scores
  int64_t S, Skv, B;
  int H, D, ratio, n;
  uint16_t* grad_q;     // [S, B, H, D] bf16
  uint16_t* grad_k;     // [Skv, B, D] bf16
  float* grad_w;        // [S, B, H]
  void* ws;             // workspace of plan.bytes (acc_k at offset 0)
};
hipError_t launch_indexer_backward(const BackwardArgs& a, const BackwardPlan& p, hipStream_t st_keys,
                                   hipStream_t st_rows);
// Stable sort of `rows` rows of `topk` (idx, score) pairs, each in ascending
// index order with -1 padding at the tail, into score-descending order.
hipError_t launch_sort_rows(int32_t* idx, float* score, int64_t rows, int topk, hipStream_t st);
hipError_t launch_kpool(const KpoolArgs& a, hipStream_t st);
hipError_t launch_pooled_scores(const PooledScoresArgs& a, hipStream_t st);
hipError_t launch_topk_pools(const TopkPoolsArgs& a, const TopkRowsPlan& pl, hipStream_t st);
hipError_t launch_expand(const ExpandArgs& a, hipStream_t st);

}  // namespace dsai
