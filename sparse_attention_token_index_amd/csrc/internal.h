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
  int32_t* out_idx;    // [B, S, topk]
  float* out_score;    // [B, S, topk]
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
};

struct ExpandArgs {
  const int32_t* pool_ids;  // [Q, sel]
  int64_t Q;
  int sel, KP, first_key;
  int32_t* tokens;  // [Q, sel * KP]
};

// Rows per workgroup of the fused kernel for this head dim / topk within
// `lds_limit` bytes of LDS (0: does not fit).
int score_topk_rows_per_block(int D, int topk, size_t lds_limit);
size_t topk_rows_lds_bytes(int sel);

hipError_t launch_score_topk(const ScoreTopkArgs& a, int rows_per_block, hipStream_t st);
hipError_t launch_kpool(const KpoolArgs& a, hipStream_t st);
hipError_t launch_pooled_scores(const PooledScoresArgs& a, hipStream_t st);
hipError_t launch_topk_pools(const TopkPoolsArgs& a, hipStream_t st);
hipError_t launch_expand(const ExpandArgs& a, hipStream_t st);

}  // namespace dsai
