// The indexer's k_norm: a LayerNorm with a bias producing the cache's
// k_normed rows ("Module glm5next_dsa", "Checkpoint and kernel facts":
// indexer.k_norm is a LayerNorm with a bias; Constants: the BF16 LayerNorm
// module it runs).  Per row of D channels: mean and biased variance in fp32,
// y = (x - mean) / sqrt(var + eps) * gamma + beta, stored as bf16 (nearest
// even) - the rows kpool_compress later pools.
//
// Streaming: D / 8 lanes per row, each owning 8 channels (one 16-byte load
// and store), four rows per lane group with their loads issued together;
// the row sums are reduced across the row's lanes with xor shuffles.  Roofline: HBM, 4 * D bytes per row (read + write) plus the
// parameters.
#include "internal.h"
#include "device_common.h"

namespace dsai {

constexpr int kNormThreads = 256;
constexpr int kNormRowsPerLane = 4;  // rows per lane group, loads issued together

template <int D>
__global__ __launch_bounds__(kNormThreads) void k_norm_kernel(const uint16_t* x,
                                                              const uint16_t* __restrict__ gamma,
                                                              const uint16_t* __restrict__ beta,
                                                              float eps, int64_t n,
                                                              uint16_t* y) {  // may alias x
  constexpr int kTpr = D / 8;  // lanes per row (4, 8 or 16: inside one 16-lane DPP row)
  constexpr int kGroups = kNormThreads / kTpr;  // lane groups per block
  const int part = (int)threadIdx.x % kTpr;
  const int64_t group = (int64_t)blockIdx.x * kGroups + (int)threadIdx.x / kTpr;
  const u32x4 g4 = *reinterpret_cast<const u32x4*>(gamma + part * 8);
  const u32x4 b4 = *reinterpret_cast<const u32x4*>(beta + part * 8);
  // rows group, group + G, group + 2G, ... (G = lane groups in the grid):
  // consecutive lane groups take consecutive rows
  const int64_t stride = (int64_t)gridDim.x * kGroups;
  u32x4 raw[kNormRowsPerLane];
#pragma unroll
  for (int rr = 0; rr < kNormRowsPerLane; ++rr) {
    const int64_t row = group + rr * stride;
    raw[rr] = row < n ? *reinterpret_cast<const u32x4*>(x + row * D + part * 8)
                      : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int rr = 0; rr < kNormRowsPerLane; ++rr) {
    const int64_t row = group + rr * stride;  // whole lane groups are live or not
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(raw[rr][i] << 16);
      v[2 * i + 1] = __uint_as_float(raw[rr][i] & 0xFFFF0000u);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
#pragma unroll
    for (int m = 1; m < kTpr; m <<= 1) s += __shfl_xor(s, m);
    const float mean = s * (1.0f / (float)D);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] -= mean;
      q += v[i] * v[i];
    }
#pragma unroll
    for (int m = 1; m < kTpr; m <<= 1) q += __shfl_xor(q, m);
    const float rs = 1.0f / __fsqrt_rn(q * (1.0f / (float)D) + eps);
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g0 = __uint_as_float(g4[i] << 16), g1 = __uint_as_float(g4[i] & 0xFFFF0000u);
      const float b0 = __uint_as_float(b4[i] << 16), b1 = __uint_as_float(b4[i] & 0xFFFF0000u);
      const float y0 = fmaf(v[2 * i] * rs, g0, b0);
      const float y1 = fmaf(v[2 * i + 1] * rs, g1, b1);
      out[i] = (uint32_t)f32_to_bf16_rne(y0) | ((uint32_t)f32_to_bf16_rne(y1) << 16);
    }
    if (row < n) *reinterpret_cast<u32x4*>(y + row * D + part * 8) = out;
  }
}

hipError_t launch_k_norm(const KNormArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  const int groups = kNormThreads / (a.D / 8);
  const int64_t rows_per_block = (int64_t)groups * kNormRowsPerLane;
  const int64_t blocks = (a.n + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
#define DSAI_CASE(d)                                                                        \
  if (a.D == d) {                                                                           \
    hipLaunchKernelGGL(k_norm_kernel<d>, dim3((unsigned)blocks), dim3(kNormThreads), 0, st,  \
                       a.x, a.gamma, a.beta, a.eps, a.n, a.y);                              \
    return hipGetLastError();                                                               \
  }
  DSAI_CASE(32) DSAI_CASE(64) DSAI_CASE(128)
#undef DSAI_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsai
