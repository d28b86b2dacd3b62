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
#include "entry_tiles.h"
#include "internal.h"
#include "score_tile.h"

namespace dsai {

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Elements e, e + 1 of a bf16 operand: the gated weights a (where d0 > 0)
// and b (where d1 > 0), else 0, rounded to nearest even in one paired
// conversion.
__device__ __forceinline__ void set_gate_pair(bf16x8& v, int e, float d0, float a, float d1,
                                              float b) {
  const bf16x2 p = __builtin_convertvector((floatx2){d0 > 0.f ? a : 0.f, d1 > 0.f ? b : 0.f}, bf16x2);
  v[e] = p[0];
  v[e + 1] = p[1];
}

namespace {

constexpr int kBwdWaves = 4;
constexpr int kMaxKeyBlocks = DSAI_BWD_MAX_KEY_BLOCKS;

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

// LDS image of a row-major bf16 matrix [rows][D] (a query row's heads, or a
// tile of key rows) read two ways: 16-byte row pieces (lane = row) and
// ds_read_b64_tr_b16 (lane = column: the B operand of dK = G^T Q or of
// grad_q = G K).  D = 128: rows
// packed (256 bytes), 16-byte chunk x of row r stored at chunk x ^ f(r) with
// f(r) = 4 (r & 3) + ((r >> 2) & 3): the 16 consecutive rows of a row-piece
// read, and the 4 rows x 4 chunks of a half-wave's transposed read, land on
// 16 distinct bank groups.  Smaller D: rows padded to the transposed reads'
// pitch instead.
template <int D>
struct QStage {
  static constexpr bool kSwizzle = D == 128;
  static constexpr int kPitch = kSwizzle ? 2 * D : TrPitch<D>::kBytes;
  static __device__ __forceinline__ uint32_t offset(int row, int byte_in_row) {
    if constexpr (kSwizzle) {
      const int f = 4 * (row & 3) + ((row >> 2) & 3);
      return (uint32_t)(row * kPitch + ((((byte_in_row >> 4) ^ f) << 4) | (byte_in_row & 15)));
    } else {
      return (uint32_t)(row * kPitch + byte_in_row);
    }
  }
  // B fragment of a 32x32x16 product whose K index runs over the image's
  // rows and whose N index over its columns: lane (n = l % 32, g = l / 32)
  // receives, as elements e = 0..7, rows row0 + 8 (e / 4) + 4 g + e % 4 of
  // column col0 + n.  ds_read_b64_tr_b16 gives lane i of each 16-lane group
  // column c0 + i of four rows: the row its lanes 4j .. 4j + 3 point at is
  // the group's j-th row (lane 4j + q names columns c0 + 4q .. c0 + 4q + 3).
  static __device__ __forceinline__ bf16x8 tr(const lds_char* m, int row0, int col0) {
    const int lane = lane_id();
    const int s = lane & 15, nh = (lane >> 4) & 1, g = lane >> 5;
    const int row = row0 + 4 * g + (s >> 2);
    const int byte = 2 * (col0 + 16 * nh + 4 * (s & 3));
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSAI_LDS s16x4*)(m + offset(row, byte)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSAI_LDS s16x4*)(m + offset(row + 8, byte)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
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
  using QS = QStage<D>;
  constexpr int kStage = HP * QS::kPitch;
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
    *reinterpret_cast<DSAI_LDS u32x4*>(qs + QS::offset(h, part * 16)) = v;
  }

  const int64_t orow = ((int64_t)b * S + t) * n;
  const int ngroups = (n + 31) / 32;
  for_each_entry_tile<D, true>(sup, grad, k, orow, n, n_t, B, b, ngroups, [&](const EntryTile<D, true>& cur, int) {
    if (ballot(cur.s >= 0) != 0) {  // wave-uniform: some entry of the tile is usable
      Acc acc;
      sc.mma(cur.f, acc);  // lane (c, g): key c, heads 32m + 8(r/4) + 4g + r%4
      // A operand of dK = G^T Q at K-step (m, p): lane (c, g) element e is
      // head 32m + 16p + 8(e/4) + 4g + e%4 of key c, i.e. register 8p + e.
      bf16x8 ga[MT][2];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int rr = 0; rr < 16; rr += 2)
          set_gate_pair(ga[m][rr >> 3], rr & 7, acc[0][m][rr], cur.g * sc.wv[0][m][rr],
                        acc[0][m][rr + 1], cur.g * sc.wv[0][m][rr + 1]);
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
            dk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[m][p], QS::tr(qs, 32 * m + 16 * p, 32 * nb),
                                                         dk, 0, 0, 0);
        float* dst = gk + (int64_t)b * D + 32 * nb + c;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if (key[rr] >= 0) unsafeAtomicAdd(dst + (int64_t)key[rr] * B * D, dk[rr]);
      }
    }
  });
}

template <int HP, int D>
__global__ __launch_bounds__(kBwdWaves * 64) void bwd_queries_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    const int32_t* __restrict__ sup, const float* __restrict__ grad, int S, int Skv, int B, int H,
    int ratio, int n, uint16_t* __restrict__ gq, float* __restrict__ gw) {
  using Scorer = TileScorer<HP, D>;
  using QS = QStage<D>;
  constexpr int MT = HP / 32, KS = D / 16, NB = D / 32;
  constexpr int kTile = 32 * QS::kPitch;
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
  if (n_t > 0)  // else no entry is usable
    for_each_entry_tile<D, true>(sup, grad, k, orow, n, n_t, B, b, (n + 31) / 32, [&](const EntryTile<D, true>& cur, int) {
      if (ballot(cur.s >= 0) != 0) {  // wave-uniform
        floatx16 dt = {};  // lane (c, g): head h, key slots 8(r/4) + 4g + r%4
#pragma unroll
        for (int x = 0; x < KS; ++x) dt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.f[x], qf[x], dt, 0, 0, 0);
        wave_lds_sync();  // the last tile's transposed reads and slot reads are done
#pragma unroll
        for (int x = 0; x < KS; ++x)
          *reinterpret_cast<DSAI_LDS bf16x8*>(kt + QS::offset(c, 2 * (g * (D / 2) + 8 * x))) = cur.f[x];
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
        for (int rr = 0; rr < 16; rr += 2) {
          acc_w = fmaf(gs[rr], fmaxf(dt[rr], 0.f), acc_w);
          acc_w = fmaf(gs[rr + 1], fmaxf(dt[rr + 1], 0.f), acc_w);
          set_gate_pair(ga[rr >> 3], rr & 7, dt[rr], gs[rr] * wh, dt[rr + 1], gs[rr + 1] * wh);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int p = 0; p < 2; ++p)
            acc_q[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[p], QS::tr(kt, 16 * p, 32 * nb),
                                                                acc_q[nb], 0, 0, 0);
      }
    });

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

// ---- key gradients grouped by key block (no per-entry scatter) -------------
//
// The entries of each query row are first bucketed by key block (kKeyBlock
// consecutive keys).  A workgroup then owns one key block of one batch and a
// chunk of query rows: wavefront w holds keys base + 64w .. base + 64w + 63
// as two 32-key tiles, their fragments (loaded once) and their dK rows (two
// 32 x D fp32 tiles in registers, accumulated over every row of the chunk).
// Per row, the block stages q_t, w_t and the row's incoming gradients for its
// keys (0 for keys the row did not select) in LDS; each wavefront computes d
// for its tiles that hold a nonzero gradient, the gated weights and
// dK += G^T Q_t on the matrix cores, reading q_t once for both tiles.  The
// tiles are added to the fp32 accumulator once per workgroup at the end.
constexpr int kKeyBlock = 256;
constexpr int kKeysPerWave = 32;
constexpr int kBlockWaves = kKeyBlock / kKeysPerWave;

// Per query row (b-major, as the index array): usable entries bucketed by
// key block.  bounds[row][i] = first bucketed entry of block i (relative to
// the row), bounds[row][nbk] = the row's usable entries; ent[row][e] =
// (key, incoming gradient bits).  One wavefront per row.
__global__ __launch_bounds__(4 * 64) void bwd_bucket_kernel(
    const int32_t* __restrict__ sup, const float* __restrict__ grad, int S, int Skv, int B,
    int ratio, int n, int nbk, int32_t* __restrict__ bounds, int2* __restrict__ ent) {
  __shared__ uint32_t cnt_raw[4][kMaxKeyBlocks];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = lane_id();
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= (int64_t)B * S) return;  // wave-uniform; no block barriers below
  const int t = (int)(r % S);
  const int n_t = min(Skv, (t + 1) / ratio);
  DSAI_LDS uint32_t* h = (DSAI_LDS uint32_t*)cnt_raw[wave];
  for (int i = lane; i < nbk; i += kWave) h[i] = 0u;
  wave_lds_sync();
  const int64_t off = r * n;
  // The row's entries go 8 per lane at a time, their loads issued together
  // (clamped to the row's last entry and masked), so a long row does not
  // wait on one load latency per 64 entries.
  constexpr int U = 8;
  for (int j0 = 0; j0 < n; j0 += U * kWave) {
    int sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) sv[u] = sup[off + min(j0 + u * kWave + lane, n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j0 + u * kWave + lane < n && sv[u] >= 0 && sv[u] < n_t)
        __hip_atomic_fetch_add(&h[sv[u] / kKeyBlock], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  wave_lds_sync();
  // exclusive scan of the bins; each lane takes a contiguous range of them
  const int per = (nbk + kWave - 1) / kWave;
  const int b0 = min(nbk, lane * per), b1 = min(nbk, b0 + per);
  uint32_t sum = 0;
  for (int i = b0; i < b1; ++i) sum += h[i];
  const uint32_t incl = wave_incl_scan(sum);
  uint32_t run = incl - sum;
  int32_t* bo = bounds + r * (nbk + 1);
  for (int i = b0; i < b1; ++i) {
    const uint32_t cnt = h[i];
    h[i] = run;
    bo[i] = (int32_t)run;
    run += cnt;
  }
  if (lane == kWave - 1) bo[nbk] = (int32_t)incl;
  wave_lds_sync();
  for (int j0 = 0; j0 < n; j0 += U * kWave) {
    int sv[U];
    float gv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = off + min(j0 + u * kWave + lane, n - 1);
      sv[u] = sup[j];
      gv[u] = grad[j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u * kWave + lane < n && sv[u] >= 0 && sv[u] < n_t) {
        const uint32_t pos = __hip_atomic_fetch_add(&h[sv[u] / kKeyBlock], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_WORKGROUP);
        ent[off + pos] = int2{sv[u], __float_as_int(gv[u])};
      }
    }
  }
}

// One query row's share of a key-block workgroup's staging, held in
// registers between its global loads and its LDS stores so that the loads of
// row i + 1 overlap the matrix-core work of row i: this thread's 16-byte
// pieces of q_t, one head weight and one bucketed entry.
template <int HP, int D>
struct RowStage {
  static constexpr int kThreads = kBlockWaves * 64;
  static constexpr int kChunks = HP * (D / 8);  // 16-byte pieces of a q row
  static constexpr int kPieces = (kChunks + kThreads - 1) / kThreads;
  static_assert(HP <= kThreads, "one head weight per thread");
  u32x4 qv[kPieces];
  float wv;
  int2 ev;
  bool has_e;

  __device__ __forceinline__ void load(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                       const int2* __restrict__ er, int64_t qrow, int H, int lo,
                                       int hi) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int ch = tid + i * kThreads;
      const int h = ch / (D / 8), part = ch % (D / 8);
      qv[i] = (ch < kChunks && h < H) ? *reinterpret_cast<const u32x4*>(q + (qrow * H + h) * D + part * 8)
                                      : u32x4{0u, 0u, 0u, 0u};
    }
    wv = tid < H ? w[qrow * H + tid] : 0.f;
    has_e = lo + tid < hi;
    if (has_e) ev = er[lo + tid];
  }

  // q_t into qs (QStage layout), w_t into ws, the row's incoming gradients
  // into gs (slot key - base; repeated keys add).  Entries past the first
  // kThreads of the row (only with repeated keys) load here.
  __device__ __forceinline__ void store(lds_char* qs, DSAI_LDS float* ws, DSAI_LDS float* gs,
                                        const int2* __restrict__ er, int lo, int hi, int base) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int ch = tid + i * kThreads;
      const int h = ch / (D / 8), part = ch % (D / 8);
      if (ch < kChunks) *reinterpret_cast<DSAI_LDS u32x4*>(qs + QStage<D>::offset(h, part * 16)) = qv[i];
    }
    if (tid < HP) ws[tid] = wv;
    if (has_e)
      __hip_atomic_fetch_add(gs + (ev.x - base), __int_as_float(ev.y), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int e = lo + tid + kThreads; e < hi; e += kThreads) {
      const int2 v = er[e];
      __hip_atomic_fetch_add(gs + (v.x - base), __int_as_float(v.y), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
};

constexpr int kRowWindow = 256;  // query rows whose bucket bounds sit in LDS at once

template <int HP, int D>
__global__ __launch_bounds__(kBlockWaves * 64) void bwd_keyblock_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    const int32_t* __restrict__ bounds, const int2* __restrict__ ent, int S, int Skv, int B, int H,
    int ratio, int n, int nbk, int chunk_rows, float* __restrict__ gk) {
  constexpr int MT = HP / 32, KS = D / 16, NB = D / 32, KT = kKeysPerWave / 32;
  using QS = QStage<D>;
  constexpr int kThreads = kBlockWaves * 64;
  __shared__ __align__(16) char qs_raw[2][HP * QS::kPitch];
  __shared__ __align__(16) float wst[2][HP];
  __shared__ float gst[2][kKeyBlock];
  __shared__ int2 win[kRowWindow];  // (lo, hi) of the window's rows in this key block
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = lane_id();
  const int c = lane & 31, g = lane >> 5;
  const int kb = blockIdx.x, b = blockIdx.y;
  const int base = kb * kKeyBlock;
  // first query row that sees key `base`: (t + 1) / ratio > base
  const int64_t t_first = (int64_t)(base + 1) * ratio - 1;
  const int64_t t0 = max((int64_t)blockIdx.z * chunk_rows, t_first);
  const int64_t t1 = min((int64_t)S, (int64_t)(blockIdx.z + 1) * chunk_rows);
  if (t0 >= t1) return;  // workgroup-uniform, before any barrier
  for (int i = threadIdx.x; i < 2 * kKeyBlock; i += kThreads) gst[i / kKeyBlock][i % kKeyBlock] = 0.f;

  // this wavefront's key tiles as B operands of d = Q K^T (lane (c, g): key
  // base + 64 wave + 32 tt + c, dims g*D/2 + 8x at k-step x); keys past Skv are zero
  bf16x8 kf[KT][KS];
#pragma unroll
  for (int tt = 0; tt < KT; ++tt) {
    const int key = base + kKeysPerWave * wave + 32 * tt + c;
#pragma unroll
    for (int x = 0; x < KS; ++x)
      kf[tt][x] = key < Skv ? *reinterpret_cast<const bf16x8*>(k + ((int64_t)key * B + b) * D + g * (D / 2) + 8 * x)
                            : bf16x8{};
  }
  floatx16 tab[KT][NB];
#pragma unroll
  for (int tt = 0; tt < KT; ++tt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) tab[tt][nb] = floatx16{};

  RowStage<HP, D> st;
  int par = 0;
  for (int64_t w0 = t0; w0 < t1; w0 += kRowWindow) {
    const int nw = (int)min((int64_t)kRowWindow, t1 - w0);
    __syncthreads();  // the previous window's last row is staged and every wave is past its reads of win
    for (int i = threadIdx.x; i < nw; i += kThreads) {
      const int32_t* bo = bounds + ((int64_t)b * S + w0 + i) * (nbk + 1) + kb;
      win[i] = int2{bo[0], bo[1]};
    }
    __syncthreads();
    // rows with no entry in this block are skipped (workgroup-uniform: win is shared)
    auto next_active = [&](int i) {
      while (i < nw && win[i].x == win[i].y) ++i;
      return i;
    };
    int cur = next_active(0);
    if (cur >= nw) continue;
    {
      const int64_t row = (int64_t)b * S + w0 + cur;
      st.load(q, w, ent + row * n, (w0 + cur) * B + b, H, win[cur].x, win[cur].y);
      st.store((lds_char*)qs_raw[par], (DSAI_LDS float*)wst[par], (DSAI_LDS float*)gst[par],
               ent + row * n, win[cur].x, win[cur].y, base);
    }
    __syncthreads();
    while (cur < nw) {
      const int nxt = next_active(cur + 1);
      if (nxt < nw)  // the next active row's loads, in flight during this row's products
        st.load(q, w, ent + ((int64_t)b * S + w0 + nxt) * n, (w0 + nxt) * B + b, H, win[nxt].x, win[nxt].y);
      const lds_char* qs = (const lds_char*)qs_raw[par];
      float gv[KT];
      bool on[KT];
#pragma unroll
      for (int tt = 0; tt < KT; ++tt) {
        gv[tt] = gst[par][kKeysPerWave * wave + 32 * tt + c];
        on[tt] = ballot(gv[tt] != 0.f) != 0;  // wave-uniform
      }
      if (on[0] || (KT > 1 && on[KT - 1])) {
        floatx16 acc[KT][MT];
#pragma unroll
        for (int tt = 0; tt < KT; ++tt)
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[tt][m] = floatx16{};
#pragma unroll
        for (int x = 0; x < KS; ++x)
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const bf16x8 a = *reinterpret_cast<const DSAI_LDS bf16x8*>(
                qs + QS::offset(32 * m + c, 2 * (g * (D / 2) + 8 * x)));
#pragma unroll
            for (int tt = 0; tt < KT; ++tt)
              if (on[tt]) acc[tt][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[tt][x], acc[tt][m], 0, 0, 0);
          }
        // lane (c, g) register r of M-tile m: key c of the tile, head
        // 32m + 8(r/4) + 4g + r%4; K-step (m, p) of dK = G^T Q takes
        // registers 8p .. 8p + 7
        bf16x8 ga[KT][MT][2];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const floatx4 w4 = *(const DSAI_LDS floatx4*)(&wst[par][32 * m + 8 * rb + 4 * g]);
#pragma unroll
            for (int tt = 0; tt < KT; ++tt)
#pragma unroll
              for (int i = 0; i < 4; i += 2) {
                const int rr = 4 * rb + i;
                set_gate_pair(ga[tt][m][rr >> 3], rr & 7, acc[tt][m][rr], gv[tt] * w4[i],
                              acc[tt][m][rr + 1], gv[tt] * w4[i + 1]);
              }
          }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const bf16x8 bq = QS::tr(qs, 32 * m + 16 * p, 32 * nb);
#pragma unroll
              for (int tt = 0; tt < KT; ++tt)
                if (on[tt]) tab[tt][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[tt][m][p], bq, tab[tt][nb], 0, 0, 0);
            }
      }
      if (g == 0) {  // clear for the row after next
#pragma unroll
        for (int tt = 0; tt < KT; ++tt) gst[par][kKeysPerWave * wave + 32 * tt + c] = 0.f;
      }
      if (nxt < nw)  // buffer par ^ 1 was last read two rows ago: every wave is past it
        st.store((lds_char*)qs_raw[par ^ 1], (DSAI_LDS float*)wst[par ^ 1], (DSAI_LDS float*)gst[par ^ 1],
                 ent + ((int64_t)b * S + w0 + nxt) * n, win[nxt].x, win[nxt].y, base);
      __syncthreads();
      par ^= 1;
      cur = nxt;
    }
  }
  // tab[tt][nb] lane (n, g) register r: key base + 64 wave + 32 tt + 8(r/4) + 4g + r%4, dim 32nb + n
#pragma unroll
  for (int tt = 0; tt < KT; ++tt)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int kk = base + kKeysPerWave * wave + 32 * tt + 8 * (rr >> 2) + 4 * g + (rr & 3);
      if (kk < Skv) {
        float* dst = gk + ((int64_t)kk * B + b) * D + c;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) unsafeAtomicAdd(dst + 32 * nb, tab[tt][nb][rr]);
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
hipError_t launch_bwd_t(const BackwardArgs& a, const BackwardPlan& p, hipStream_t st_keys,
                        hipStream_t st_rows) {
  const int64_t rows = a.S * a.B;
  const int64_t n4 = a.Skv * a.B * a.D / 4;  // D is a multiple of 32
  const int64_t kb = (rows + kBwdWaves - 1) / kBwdWaves;
  const int64_t qb = (rows * (HP / 32) + kBwdWaves - 1) / kBwdWaves;
  if (kb > 0x7FFFFFFF || qb > 0x7FFFFFFF) return hipErrorInvalidValue;
  float* acc_k = static_cast<float*>(a.ws);
  hipError_t e;
  if (rows > 0) {
    hipLaunchKernelGGL((bwd_queries_kernel<HP, D>), dim3((unsigned)qb), dim3(kBwdWaves * 64), 0,
                       st_rows, a.q, a.k, a.w, a.sup, a.grad, (int)a.S, (int)a.Skv, (int)a.B, a.H,
                       a.ratio, a.n, a.grad_q, a.grad_w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(stream_blocks(n4)), dim3(256), 0, st_keys,
                     reinterpret_cast<float4*>(acc_k), n4);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (rows > 0 && p.grouped) {
    char* ws = static_cast<char*>(a.ws);
    int32_t* bounds = reinterpret_cast<int32_t*>(ws + p.bounds_off);
    int2* ent = reinterpret_cast<int2*>(ws + p.ent_off);
    hipLaunchKernelGGL(bwd_bucket_kernel, dim3((unsigned)kb), dim3(4 * 64), 0, st_keys, a.sup,
                       a.grad, (int)a.S, (int)a.Skv, (int)a.B, a.ratio, a.n, p.nbk, bounds, ent);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_keyblock_kernel<HP, D>), dim3((unsigned)p.nbk, (unsigned)a.B, (unsigned)p.nchunks),
                       dim3(kBlockWaves * 64), 0, st_keys, a.q, a.k, a.w, bounds, ent, (int)a.S,
                       (int)a.Skv, (int)a.B, a.H, a.ratio, a.n, p.nbk, p.chunk_rows, acc_k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else if (rows > 0) {
    hipLaunchKernelGGL((bwd_keys_kernel<HP, D>), dim3((unsigned)kb), dim3(kBwdWaves * 64), 0,
                       st_keys, a.q, a.k, a.w, a.sup, a.grad, (int)a.S, (int)a.Skv, (int)a.B, a.H,
                       a.ratio, a.n, acc_k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(stream_blocks(n4)), dim3(256), 0, st_keys,
                     reinterpret_cast<const float4*>(acc_k), reinterpret_cast<uint2*>(a.grad_k),
                     n4);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

BackwardPlan plan_backward(int64_t S, int64_t Skv, int64_t B, int D, int n, int ratio) {
  BackwardPlan p{};
  p.bytes = align256((size_t)Skv * (size_t)B * (size_t)D * sizeof(float));
  const int64_t nbk = (Skv + kKeyBlock - 1) / kKeyBlock;
  p.grouped = S > 0 && Skv > 0 && B > 0 && B <= 65535 && nbk <= kMaxKeyBlocks;
  if (!p.grouped) return p;
  // The grouped form costs about one 32-key product unit per (row, 32 visible
  // keys), the scatter about D atomic adds per entry; measured on MI355X, a
  // unit costs as much as 5-6 entries.  With rows listing min(n, n_t) keys,
  // group when the entries outnumber the units 8 to 1 (a quarter of the
  // visible keys selected or more).
  int64_t units = 0, entries = 0;
  const int64_t vmax = Skv < S / ratio ? Skv : S / ratio;  // largest n_t
  for (int64_t v = 1; v <= vmax; ++v) {  // rows with n_t = v: t in [v r - 1, (v + 1) r - 1)
    const int64_t lo = v * ratio - 1;
    const int64_t hi = v == Skv ? S : ((v + 1) * ratio - 1 < S ? (v + 1) * ratio - 1 : S);
    if (hi <= lo) continue;
    units += (hi - lo) * ((v + 31) / 32);
    entries += (hi - lo) * (v < n ? v : n);
  }
  p.grouped = entries >= 8 * units;
  if (!p.grouped) return p;
  p.nbk = (int)nbk;
  // Rows that see some key of each block, summed, are the grouped kernel's
  // work.  The chunk is the smallest that leaves at most kBusyBlocks busy
  // workgroups (two rounds of one workgroup per CU), so the last round is
  // not a sliver of leftovers.
  constexpr int64_t kBusyBlocks = 512;
  int64_t visible = 0;
  for (int64_t i = 0; i < nbk; ++i) {
    const int64_t t_first = (i * kKeyBlock + 1) * (int64_t)ratio - 1;
    if (t_first < S) visible += S - t_first;
  }
  auto busy = [&](int64_t ch) {
    int64_t nblk = 0;
    for (int64_t i = 0; i < nbk; ++i) {
      const int64_t t_first = (i * kKeyBlock + 1) * (int64_t)ratio - 1;
      if (t_first < S) nblk += (S - 1) / ch - (t_first / ch) + 1;  // chunks meeting [t_first, S)
    }
    return nblk * B;
  };
  int64_t chunk = (visible * B + kBusyBlocks - 1) / kBusyBlocks;
  if (chunk < 32) chunk = 32;
  if (chunk < (S + 65534) / 65535) chunk = (S + 65534) / 65535;
  if (chunk > S) chunk = S;
  while (chunk < S && busy(chunk) > kBusyBlocks) chunk += (chunk + 15) / 16;
  if (chunk > S) chunk = S;
  p.chunk_rows = (int)chunk;
  p.nchunks = (int)((S + chunk - 1) / chunk);
  p.bounds_off = p.bytes;
  p.ent_off = p.bounds_off + align256((size_t)(B * S) * (size_t)(nbk + 1) * sizeof(int32_t));
  p.bytes = p.ent_off + align256((size_t)(B * S) * (size_t)n * 2 * sizeof(int32_t));
  return p;
}

hipError_t launch_indexer_backward(const BackwardArgs& a, const BackwardPlan& p, hipStream_t st_keys,
                                   hipStream_t st_rows) {
  const int HP = a.H <= 32 ? 32 : 64;
#define DSAI_CASE(hp, d) \
  if (HP == hp && a.D == d) return launch_bwd_t<hp, d>(a, p, st_keys, st_rows);
  DSAI_CASE(32, 32) DSAI_CASE(32, 64) DSAI_CASE(32, 128)
  DSAI_CASE(64, 32) DSAI_CASE(64, 64) DSAI_CASE(64, 128)
#undef DSAI_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsai
