// Gradients of the selected index scores: the backward of the V4 indexer's
// autograd function (NeMo AutoModel page "...deepseek_v4.kernels.
// tilelang_indexer": V4IndexerFunction.backward(grad_scores, grad_indices)).
// Only the returned scores carry a gradient; the indices are integers.  For a
// usable entry (key s with 0 <= s < n_t) of query row (t, b), incoming
// gradient g and per-head products d_h = q[t,b,h,:] . k[s,b,:]:
//
//   grad_w[t,b,h]   += g * ReLU(d_h)
//   grad_q[t,b,h,:] += g * w[t,b,h] * [d_h > 0] * k[s,b,:]
//   grad_k[s,b,:]   += g * sum_h w[t,b,h] * [d_h > 0] * q[t,b,h,:]
//
// ReLU's derivative is 0 at 0; an unusable entry (-1, masked, out of range)
// scores -inf in the forward and passes nothing back.
//
// Three products per 32-entry tile run on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16): the dot products d (as in the forward), then
// G^T-weighted sums of keys (grad_q) and of query heads (grad_k), with the
// gated weight G[h, s] = g * w_h * [d_h > 0] rounded to bf16 as the operand.
// The second and third products contract over an index that the row-major
// data keeps in its rows (keys, heads), so their B operands come from LDS
// through ds_read_b64_tr_b16, which hands each lane one column of four rows.
//
// keys kernel: one wavefront per query row; d in the forward's orientation
//   (lane = key, registers = heads), G straight into the A operand of
//   dK = G^T Q, and dK added to an fp32 [Skv, B, D] accumulator with global
//   atomics (the sum over rows is a scatter).
// queries kernel: one wavefront per (query row, 32-head group); d transposed
//   (lane = head, registers = keys) by swapping the operands, so G is the A
//   operand of grad_q = G K and the ReLU'd products sum into grad_w per lane.
#include "internal.h"
#include "score_tile.h"

namespace dsai {

namespace {

constexpr int kBwdWaves = 4;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Row pitch of the LDS matrices read with transposed loads: D bf16 padded so
// the pitch in dwords is 16 or 48 mod 64.  The four rows one 16-lane group
// reads then start 16 dwords apart, so the 32-byte pieces a half-wave reads
// (two column halves of four rows) fall on distinct banks.
template <int D>
struct TrPitch {
  static_assert(D == 32 || D == 64 || D == 128, "head dim 32, 64 or 128");
  static constexpr int kBytes = D == 32 ? 64 : (D == 64 ? 192 : 320);
};

// B fragment of a 32x32x16 product whose K index runs over rows of a
// row-major bf16 LDS matrix and whose N index runs over its columns: lane
// (n = l % 32, g = l / 32) receives, as elements e = 0..7, rows
// row0 + 8 (e / 4) + 4 g + e % 4 of column col0 + n.  ds_read_b64_tr_b16 gives
// lane i of each 16-lane group column c0 + i of four rows: the row its lanes
// 4j .. 4j + 3 point at is the group's j-th row (lane 4j + q names columns
// c0 + 4q .. c0 + 4q + 3 of it).
template <int PITCH>
__device__ __forceinline__ bf16x8 tr_frag(const lds_char* m, int row0, int col0) {
  const int lane = lane_id();
  const int s = lane & 15, nh = (lane >> 4) & 1, g = lane >> 5;
  const lds_char* p = m + (row0 + 4 * g + (s >> 2)) * PITCH + 2 * (col0 + 16 * nh + 4 * (s & 3));
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSAI_LDS s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSAI_LDS s16x4*)(p + 8 * PITCH));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Entry j0 + (lane % 32) of a row of supplied indices: its key (-1 when not
// usable), incoming gradient (0 when not usable) and that key's fragments
// for the forward's tile layout (lane (c, g): dims g*D/2 + 8x, x < D/16).
// An unusable entry reads key 0 (n_t > 0, so it exists) and is discarded.
template <int D>
struct EntryTile {
  int s;
  float g;
  bf16x8 f[D / 16];

  __device__ __forceinline__ void fetch(const int32_t* __restrict__ sup, const float* __restrict__ grad,
                                        const uint16_t* __restrict__ k, int64_t orow, int n, int j0,
                                        int n_t, int B, int b) {
    const int lane = lane_id();
    const int c = lane & 31, g2 = lane >> 5;
    const int j = j0 + c;
    const int sv = j < n ? sup[orow + j] : -1;
    const bool ok = sv >= 0 && sv < n_t;
    s = ok ? sv : -1;
    g = ok ? grad[orow + j] : 0.f;
    const uint16_t* src = k + ((int64_t)(ok ? sv : 0) * B + b) * D + g2 * (D / 2);
#pragma unroll
    for (int x = 0; x < D / 16; ++x) f[x] = *reinterpret_cast<const bf16x8*>(src + 8 * x);
  }
};

template <int HP, int D>
__global__ __launch_bounds__(kBwdWaves * 64) void bwd_keys_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    const int32_t* __restrict__ sup, const float* __restrict__ grad, int S, int Skv, int B, int H,
    int ratio, int n, float* __restrict__ gk) {
  using Scorer = TileScorer<HP, D>;
  using Acc = typename Scorer::Acc;
  constexpr int MT = HP / 32, NB = D / 32;
  constexpr int PITCH = TrPitch<D>::kBytes;
  constexpr int kStage = HP * PITCH;
  __shared__ __align__(16) char smem_raw[kBwdWaves][kStage + 128];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = lane_id();
  const int64_t r = (int64_t)blockIdx.x * kBwdWaves + wave;  // over (t, b)
  if (r >= (int64_t)S * B) return;  // wave-uniform; no block barriers below
  const int t = (int)(r / B);
  const int b = (int)(r - (int64_t)t * B);
  const int n_t = min(Skv, (t + 1) / ratio);
  if (n_t <= 0) return;  // no usable entry: nothing to add
  lds_char* qs = (lds_char*)smem_raw[wave];
  DSAI_LDS int32_t* slot_key = (DSAI_LDS int32_t*)(qs + kStage);
  const int c = lane & 31, g = lane >> 5;

  const int64_t qrow = (int64_t)t * B + b;
  Scorer sc;
  sc.load_query(q + qrow * H * D, w + qrow * H, H, true);
  // The query row again, row-major in LDS with heads past H zero: the source
  // of dK's transposed B fragments (rows = heads, columns = dims).
  for (int ch = lane; ch < HP * (D / 8); ch += kWave) {
    const int h = ch / (D / 8), part = ch % (D / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (h < H) v = *reinterpret_cast<const u32x4*>(q + (qrow * H + h) * D + part * 8);
    *reinterpret_cast<DSAI_LDS u32x4*>(qs + h * PITCH + part * 16) = v;
  }

  const int64_t orow = ((int64_t)b * S + t) * n;
  const int ngroups = (n + 31) / 32;
  EntryTile<D> cur, nxt;
  cur.fetch(sup, grad, k, orow, n, 0, n_t, B, b);
  for (int it = 0; it < ngroups; ++it) {
    if (it + 1 < ngroups) nxt.fetch(sup, grad, k, orow, n, (it + 1) * 32, n_t, B, b);
    if (ballot(cur.s >= 0) != 0) {  // wave-uniform: some entry of the tile is usable
      Acc acc;
      sc.mma(cur.f, acc);  // lane (c, g): key c, heads 32m + 8(r/4) + 4g + r%4
      // A operand of dK = G^T Q at K-step (m, p): lane (c, g) element e is
      // head 32m + 16p + 8(e/4) + 4g + e%4 of key c, i.e. register 8p + e.
      bf16x8 ga[MT][2];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          ga[m][rr >> 3][rr & 7] =
              (__bf16)(acc[0][m][rr] > 0.f ? cur.g * sc.wv[0][m][rr] : 0.f);
      wave_lds_sync();  // the query stage (first tile) and the last tile's slot reads
      if (g == 0) slot_key[c] = cur.s;
      wave_lds_sync();
      // dK lane (n, g) register r: key slot 8(r/4) + 4g + r%4, dim 32nb + n
      int key[16];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const i32x4 v = *reinterpret_cast<const DSAI_LDS i32x4*>(slot_key + 8 * rb + 4 * g);
        key[4 * rb + 0] = v.x; key[4 * rb + 1] = v.y; key[4 * rb + 2] = v.z; key[4 * rb + 3] = v.w;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        floatx16 dk = {};
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int p = 0; p < 2; ++p)
            dk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[m][p], tr_frag<PITCH>(qs, 32 * m + 16 * p, 32 * nb),
                                                         dk, 0, 0, 0);
        float* dst = gk + (int64_t)b * D + 32 * nb + c;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if (key[rr] >= 0) unsafeAtomicAdd(dst + (int64_t)key[rr] * B * D, dk[rr]);
      }
    }
    cur = nxt;
  }
}

template <int HP, int D>
__global__ __launch_bounds__(kBwdWaves * 64) void bwd_queries_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    const int32_t* __restrict__ sup, const float* __restrict__ grad, int S, int Skv, int B, int H,
    int ratio, int n, uint16_t* __restrict__ gq, float* __restrict__ gw) {
  using Scorer = TileScorer<HP, D>;
  constexpr int MT = HP / 32, KS = D / 16, NB = D / 32;
  constexpr int PITCH = TrPitch<D>::kBytes;
  constexpr int kTile = 32 * PITCH;
  __shared__ __align__(16) char smem_raw[kBwdWaves][kTile + 128];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = lane_id();
  const int64_t r = (int64_t)blockIdx.x * kBwdWaves + wave;  // over ((t, b), head group)
  if (r >= (int64_t)S * B * MT) return;  // wave-uniform; no block barriers below
  const int m = (int)(r % MT);
  const int64_t row = r / MT;
  const int t = (int)(row / B);
  const int b = (int)(row - (int64_t)t * B);
  const int n_t = min(Skv, (t + 1) / ratio);
  lds_char* kt = (lds_char*)smem_raw[wave];
  DSAI_LDS float* slot_g = (DSAI_LDS float*)(kt + kTile);
  const int c = lane & 31, g = lane >> 5;
  const int64_t qrow = (int64_t)t * B + b;
  const int h = 32 * m + c;  // this lane's head: the N index of d^T

  // B operand of d^T = K Q^T: lane (c, g) dims g*D/2 + 8x of head h (the
  // forward's query fragment, here on the other side of the product).
  bf16x8 qf[KS];
#pragma unroll
  for (int x = 0; x < KS; ++x)
    qf[x] = h < H ? *reinterpret_cast<const bf16x8*>(q + (qrow * H + h) * D + g * (D / 2) + 8 * x)
                  : bf16x8{};
  const float wh = h < H ? w[qrow * H + h] : 0.f;

  floatx16 acc_q[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc_q[nb] = floatx16{};
  float acc_w = 0.f;

  const int64_t orow = ((int64_t)b * S + t) * n;
  const int ngroups = n_t > 0 ? (n + 31) / 32 : 0;  // n_t == 0: no entry is usable
  EntryTile<D> cur, nxt;
  if (ngroups > 0) cur.fetch(sup, grad, k, orow, n, 0, n_t, B, b);
  for (int it = 0; it < ngroups; ++it) {
    if (it + 1 < ngroups) nxt.fetch(sup, grad, k, orow, n, (it + 1) * 32, n_t, B, b);
    if (ballot(cur.s >= 0) != 0) {  // wave-uniform
      floatx16 dt = {};  // lane (c, g): head h, key slots 8(r/4) + 4g + r%4
#pragma unroll
      for (int x = 0; x < KS; ++x) dt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.f[x], qf[x], dt, 0, 0, 0);
      wave_lds_sync();  // the last tile's transposed reads and slot reads are done
#pragma unroll
      for (int x = 0; x < KS; ++x)
        *reinterpret_cast<DSAI_LDS bf16x8*>(kt + c * PITCH + 2 * (g * (D / 2) + 8 * x)) = cur.f[x];
      if (g == 0) slot_g[c] = cur.g;
      wave_lds_sync();
      float gs[16];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const floatx4 v = *reinterpret_cast<const DSAI_LDS floatx4*>(slot_g + 8 * rb + 4 * g);
        gs[4 * rb + 0] = v.x; gs[4 * rb + 1] = v.y; gs[4 * rb + 2] = v.z; gs[4 * rb + 3] = v.w;
      }
      // A operand of grad_q = G K at K-step p: lane (c, g) element e is key
      // slot 16p + 8(e/4) + 4g + e%4 of head h, i.e. register 8p + e.
      bf16x8 ga[2];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        acc_w = fmaf(gs[rr], fmaxf(dt[rr], 0.f), acc_w);
        ga[rr >> 3][rr & 7] = (__bf16)(dt[rr] > 0.f ? gs[rr] * wh : 0.f);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          acc_q[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[p], tr_frag<PITCH>(kt, 16 * p, 32 * nb),
                                                              acc_q[nb], 0, 0, 0);
    }
    cur = nxt;
  }

  // grad_w: lanes c and c + 32 hold the two halves of head h's key slots
  const float tot_w = Scorer::combine(acc_w);
  if (g == 0 && h < H) gw[qrow * H + h] = tot_w;
  // grad_q lane (n, g) register r: head 32m + 8(r/4) + 4g + r%4, dim 32nb + n
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int hh = 32 * m + 8 * (rr >> 2) + 4 * g + (rr & 3);
    if (hh < H) {
      uint16_t* dst = gq + (qrow * H + hh) * D + c;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) dst[32 * nb] = f32_to_bf16_rne(acc_q[nb][rr]);
    }
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float4* __restrict__ p, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = float4{0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float4* __restrict__ src,
                                                          uint2* __restrict__ dst, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 v = src[i];
    dst[i] = uint2{(uint32_t)f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16),
                   (uint32_t)f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16)};
  }
}

unsigned stream_blocks(int64_t n4) {
  const int64_t b = (n4 + 255) / 256;
  return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

template <int HP, int D>
hipError_t launch_bwd_t(const BackwardArgs& a, hipStream_t st_keys, hipStream_t st_rows) {
  const int64_t rows = a.S * a.B;
  const int64_t n4 = a.Skv * a.B * a.D / 4;  // D is a multiple of 32
  const int64_t kb = (rows + kBwdWaves - 1) / kBwdWaves;
  const int64_t qb = (rows * (HP / 32) + kBwdWaves - 1) / kBwdWaves;
  if (kb > 0x7FFFFFFF || qb > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipError_t e;
  if (rows > 0) {
    hipLaunchKernelGGL((bwd_queries_kernel<HP, D>), dim3((unsigned)qb), dim3(kBwdWaves * 64), 0,
                       st_rows, a.q, a.k, a.w, a.sup, a.grad, (int)a.S, (int)a.Skv, (int)a.B, a.H,
                       a.ratio, a.n, a.grad_q, a.grad_w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(stream_blocks(n4)), dim3(256), 0, st_keys,
                     reinterpret_cast<float4*>(a.acc_k), n4);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (rows > 0) {
    hipLaunchKernelGGL((bwd_keys_kernel<HP, D>), dim3((unsigned)kb), dim3(kBwdWaves * 64), 0,
                       st_keys, a.q, a.k, a.w, a.sup, a.grad, (int)a.S, (int)a.Skv, (int)a.B, a.H,
                       a.ratio, a.n, a.acc_k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(stream_blocks(n4)), dim3(256), 0, st_keys,
                     reinterpret_cast<const float4*>(a.acc_k), reinterpret_cast<uint2*>(a.grad_k),
                     n4);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_backward(const BackwardArgs& a, hipStream_t st_keys, hipStream_t st_rows) {
  const int HP = a.H <= 32 ? 32 : 64;
#define DSAI_CASE(hp, d) \
  if (HP == hp && a.D == d) return launch_bwd_t<hp, d>(a, st_keys, st_rows);
  DSAI_CASE(32, 32) DSAI_CASE(32, 64) DSAI_CASE(32, 128)
  DSAI_CASE(64, 32) DSAI_CASE(64, 64) DSAI_CASE(64, 128)
#undef DSAI_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsai
