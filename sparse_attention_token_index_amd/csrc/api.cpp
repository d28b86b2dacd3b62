// C ABI of the selection library: configuration validation, argument checks
// (all on the host, before any HIP call) and dispatch to the kernels.
#include "dsai.h"

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include <cmath>

#include "internal.h"

struct dsai_context {
  dsai_config cfg;
  int last_hip_error = 0;
  int device = -1;           // device the cached limits belong to
  size_t lds_limit = 0;      // max LDS bytes per workgroup on that device
  // Two streams (default priority) on which consecutive row chunks run,
  // forked from and joined back to the caller's stream, so that a chunk of
  // too few rows to fill the GPU on its own overlaps the next one.
  int side_device = -1;
  hipStream_t side[2] = {nullptr, nullptr};
  hipEvent_t fork = nullptr;
  hipEvent_t join[2] = {nullptr, nullptr};
};

namespace {

constexpr size_t kAlign = 16;

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

int select_k(const dsai_config& c) { return c.index_topk / c.kpool; }

// Config invariants: "Module glm5next_dsa" page (index_topk a nonzero
// multiple of index_kpool; index_kpool at most KERNEL_MAX_KPOOL, refused
// rather than truncated) plus the head/dim range the kernels are built for.
int check_config(const dsai_config& c) {
  if (c.heads < 1) return DSAI_ERR_INVALID_ARG;
  if (c.kpool < 1 || c.kpool > DSAI_MAX_KPOOL) return DSAI_ERR_INVALID_ARG;
  if (c.index_topk < 1 || c.index_topk % c.kpool != 0) return DSAI_ERR_INVALID_ARG;
  if (select_k(c) > DSAI_MAX_TOPK) return DSAI_ERR_INVALID_ARG;
  if (c.first_key < 0 || c.chunk_rows < 0) return DSAI_ERR_INVALID_ARG;
  if (c.order != DSAI_ORDER_SCORE && c.order != DSAI_ORDER_INDEX) return DSAI_ERR_INVALID_ARG;
  if (c.cuts != DSAI_CUTS_ESTIMATED && c.cuts != DSAI_CUTS_TOPK) return DSAI_ERR_INVALID_ARG;
  if (c.heads > DSAI_MAX_HEADS) return DSAI_ERR_UNSUPPORTED;
  if (c.dim != 32 && c.dim != 64 && c.dim != 128) return DSAI_ERR_UNSUPPORTED;
  return DSAI_OK;
}

int hip_status(dsai_context* h, hipError_t e) {
  if (e == hipSuccess) return DSAI_OK;
  h->last_hip_error = (int)e;
  return DSAI_ERR_HIP;
}

// LDS limit of the current device, queried once per device.
hipError_t device_limits(dsai_context* h) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev == h->device) return hipSuccess;
  int lds = 0;
  e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  h->device = dev;
  h->lds_limit = (size_t)lds;
  return hipSuccess;
}

constexpr int64_t kI32 = 2147483647;

void release_side(dsai_context* h) {
  for (int i = 0; i < 2; ++i) {
    if (h->join[i]) (void)hipEventDestroy(h->join[i]);
    if (h->side[i]) (void)hipStreamDestroy(h->side[i]);
    h->join[i] = nullptr;
    h->side[i] = nullptr;
  }
  if (h->fork) (void)hipEventDestroy(h->fork);
  h->fork = nullptr;
  h->side_device = -1;
}

hipError_t ensure_side(dsai_context* h) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (h->side_device == dev) return hipSuccess;
  release_side(h);
  for (int i = 0; i < 2; ++i) {
    if ((e = hipStreamCreateWithFlags(&h->side[i], hipStreamNonBlocking)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&h->join[i], hipEventDisableTiming)) != hipSuccess) {
      release_side(h);
      return e;
    }
  }
  if ((e = hipEventCreateWithFlags(&h->fork, hipEventDisableTiming)) != hipSuccess) {
    release_side(h);
    return e;
  }
  h->side_device = dev;
  return hipSuccess;
}

// launch(sa, sb) on the two side streams, ordered after the work already on
// `st` and before anything enqueued on `st` afterwards.  The join is
// recorded even when the launch fails, so `st` never runs ahead of work
// that did start.
template <class F>
hipError_t on_side_streams(dsai_context* h, hipStream_t st, F launch) {
  hipError_t e = ensure_side(h);
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(h->fork, st)) != hipSuccess) return e;
  for (int i = 0; i < 2; ++i)
    if ((e = hipStreamWaitEvent(h->side[i], h->fork, 0)) != hipSuccess) return e;
  const hipError_t le = launch(h->side[0], h->side[1]);
  for (int i = 0; i < 2; ++i) {
    if ((e = hipEventRecord(h->join[i], h->side[i])) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(st, h->join[i], 0)) != hipSuccess) return e;
  }
  return le;
}

// Packed-sequence offsets: nseq + 1 host int64 values per side, starting at
// 0 and never decreasing, totals below 2^31.  The totals go to *Tq, *Tk.
int check_offsets(int64_t nseq, const int64_t* cu_q, const int64_t* cu_k, int64_t* Tq,
                  int64_t* Tk) {
  if (nseq < 0) return DSAI_ERR_INVALID_ARG;
  *Tq = *Tk = 0;
  if (nseq == 0) return DSAI_OK;
  if (!cu_q || !cu_k) return DSAI_ERR_NULLPTR;
  if (cu_q[0] != 0 || cu_k[0] != 0) return DSAI_ERR_INVALID_ARG;
  for (int64_t i = 0; i < nseq; ++i)
    if (cu_q[i + 1] < cu_q[i] || cu_k[i + 1] < cu_k[i]) return DSAI_ERR_INVALID_ARG;
  if (cu_q[nseq] > kI32 || cu_k[nseq] > kI32) return DSAI_ERR_INVALID_ARG;
  *Tq = cu_q[nseq];
  *Tk = cu_k[nseq];
  return DSAI_OK;
}

// Visible (query, key) pairs of one batch: sum over t < S of
// min(Skv, floor((t + 1) / r)), in closed form.
int64_t visible_pairs(int64_t S, int64_t Skv, int64_t r) {
  const int64_t U = S < Skv * r ? S : Skv * r;  // u = t + 1 <= U: floor(u / r) <= Skv
  const int64_t q = U / r, rem = U % r;
  return r * q * (q - 1) / 2 + q * (rem + 1) + (S - U) * Skv;
}

// Scores at supplied indices by one of two kernels, both giving the
// selection's scores bit for bit.  Where a row's visible keys fit the fused
// kernel's dense store and the visible pairs are at most twice the supplied
// entries, the fused kernel scores every visible key (each 32-key tile
// staged once for a block of rows) and reads the entries from the row's
// store; otherwise each entry's key row is gathered (score_at_kernel), which
// costs about 2.5 times as much per pair (measured on MI355X).
hipError_t launch_scores_at(dsai_context* h, const dsai::ScoreAtArgs& a, hipStream_t st,
                            hipStream_t st2) {
  if (a.Skv > 0 && a.Skv * a.B * a.D * 2 <= (int64_t)0xFFFFFFFF &&
      visible_pairs(a.S, a.Skv, a.ratio) <= 2 * a.S * (int64_t)a.n) {
    hipError_t e = device_limits(h);
    if (e != hipSuccess) return e;
    const dsai::ScoreSelectPlan plan =
        dsai::plan_score_select(a.H <= 32 ? 32 : 64, a.D, a.n, a.Skv, h->lds_limit);
    if (plan.rows_per_block > 0 && plan.dense) {
      dsai::ScoreTopkArgs t;
      t.q = a.q; t.k = a.k; t.w = a.w;
      t.S = a.S; t.Skv = a.Skv; t.B = a.B;
      t.H = a.H; t.D = a.D; t.ratio = a.ratio; t.topk = a.n;
      t.chunk_rows = a.chunk_rows;
      t.sort = false;
      t.sup = a.sup;
      t.out_idx = a.out_idx; t.out_score = a.out_score;
      return dsai::launch_score_topk(t, plan, st, st2);
    }
  }
  return dsai::launch_score_at(a, st, st2);
}

}  // namespace


extern "C" {

int dsai_create(const dsai_config* cfg, dsai_handle* out) {
  if (!cfg || !out) return DSAI_ERR_NULLPTR;
  *out = nullptr;
  const int st = check_config(*cfg);
  if (st != DSAI_OK) return st;
  dsai_context* h = new (std::nothrow) dsai_context;
  if (!h) return DSAI_ERR_INVALID_ARG;
  h->cfg = *cfg;
  *out = h;
  return DSAI_OK;
}

int dsai_destroy(dsai_handle h) {
  if (h) release_side(h);
  delete h;
  return DSAI_OK;
}

const char* dsai_status_string(int status) {
  switch (status) {
    case DSAI_OK: return "ok";
    case DSAI_ERR_INVALID_ARG: return "invalid argument";
    case DSAI_ERR_UNSUPPORTED: return "unsupported";
    case DSAI_ERR_WORKSPACE: return "workspace missing or too small";
    case DSAI_ERR_NULLPTR: return "null pointer";
    case DSAI_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int dsai_last_hip_error(dsai_handle h) { return h ? h->last_hip_error : 0; }

// One per-sample problem (the body of dsai_score_topk); `sort`: score order.
static int score_topk_one(dsai_handle h, const void* index_q, const void* index_k,
                          const float* weights, int64_t S, int64_t Skv, int64_t B,
                          int compress_ratio, int topk, const int32_t* topk_indices,
                          int32_t* out_idx, float* out_score, void* stream, bool sort) {
  if (!h) return DSAI_ERR_NULLPTR;
  if (S < 0 || Skv < 0 || B < 0 || compress_ratio < 1) return DSAI_ERR_INVALID_ARG;
  if (topk < 1 || topk > DSAI_MAX_TOPK) return DSAI_ERR_INVALID_ARG;
  if (S > kI32 || Skv > kI32 || B > kI32 || S * B > kI32) return DSAI_ERR_INVALID_ARG;
  if (topk_indices) {
    // scores at the supplied indices: one [B, S, topk] entry per output slot
    if (S == 0 || B == 0) return DSAI_OK;
    if (!index_q || !weights || !out_idx || !out_score) return DSAI_ERR_NULLPTR;
    if (Skv > 0 && !index_k) return DSAI_ERR_NULLPTR;
    if (!aligned(index_q) || !aligned(index_k) || !aligned(out_idx) || !aligned(out_score) ||
        !aligned(topk_indices))
      return DSAI_ERR_INVALID_ARG;
    dsai::ScoreAtArgs a;
    a.q = static_cast<const uint16_t*>(index_q);
    a.k = static_cast<const uint16_t*>(index_k);
    a.w = weights;
    a.S = S; a.Skv = Skv; a.B = B;
    a.H = h->cfg.heads; a.D = h->cfg.dim; a.ratio = compress_ratio; a.n = topk;
    a.chunk_rows = h->cfg.chunk_rows;
    a.sup = topk_indices;
    a.out_idx = out_idx; a.out_score = out_score;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.chunk_rows > 0 && S > a.chunk_rows)
      return hip_status(h, on_side_streams(h, st, [&](hipStream_t s0, hipStream_t s1) {
                          return launch_scores_at(h, a, s0, s1);
                        }));
    return hip_status(h, launch_scores_at(h, a, st, nullptr));
  }
  // keys of one batch are addressed with 32-bit byte offsets
  if (Skv * B * h->cfg.dim * 2 > (int64_t)0xFFFFFFFF) return DSAI_ERR_UNSUPPORTED;
  if (S == 0 || B == 0) return DSAI_OK;
  if (!index_q || !weights || !out_idx || !out_score) return DSAI_ERR_NULLPTR;
  if (Skv > 0 && !index_k) return DSAI_ERR_NULLPTR;
  if (!aligned(index_q) || !aligned(index_k) || !aligned(out_idx) || !aligned(out_score))
    return DSAI_ERR_INVALID_ARG;
  hipError_t e = device_limits(h);
  if (e != hipSuccess) return hip_status(h, e);
  const dsai::ScoreSelectPlan plan =
      dsai::plan_score_select(h->cfg.heads <= 32 ? 32 : 64, h->cfg.dim, topk, Skv, h->lds_limit);
  if (plan.rows_per_block < 1) return DSAI_ERR_UNSUPPORTED;
  dsai::ScoreTopkArgs a;
  a.q = static_cast<const uint16_t*>(index_q);
  a.k = static_cast<const uint16_t*>(index_k);
  a.w = weights;
  a.S = S; a.Skv = Skv; a.B = B;
  a.H = h->cfg.heads; a.D = h->cfg.dim; a.ratio = compress_ratio; a.topk = topk;
  a.chunk_rows = h->cfg.chunk_rows;
  a.sort = sort;
  a.est_cuts = h->cfg.cuts == DSAI_CUTS_ESTIMATED;
  a.out_idx = out_idx; a.out_score = out_score;
  // one launch on the caller's stream whatever cfg.chunk_rows is
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t le = dsai::launch_score_topk(a, plan, st, nullptr);
  if (le != hipSuccess) return hip_status(h, le);
  if (a.sort) le = dsai::launch_sort_rows(out_idx, out_score, B * S, topk, st);
  return hip_status(h, le);
}

int dsai_score_topk(dsai_handle h, const void* index_q, const void* index_k, const float* weights,
                    int64_t S, int64_t Skv, int64_t B, int compress_ratio, int topk,
                    const int32_t* topk_indices, int32_t* out_idx, float* out_score,
                    void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  return score_topk_one(h, index_q, index_k, weights, S, Skv, B, compress_ratio, topk,
                        topk_indices, out_idx, out_score, stream,
                        h->cfg.order == DSAI_ORDER_SCORE);
}

int dsai_score_topk_packed(dsai_handle h, const void* index_q, const void* index_k,
                           const float* weights, int64_t nseq, const int64_t* cu_seqlens_q,
                           const int64_t* cu_seqlens_k, int compress_ratio, int topk,
                           const int32_t* topk_indices, int32_t* out_idx, float* out_score,
                           void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  if (nseq < 0 || compress_ratio < 1 || topk < 1 || topk > DSAI_MAX_TOPK || topk % 4 != 0)
    return DSAI_ERR_INVALID_ARG;
  int64_t Tq = 0, Tk = 0;
  const int so = check_offsets(nseq, cu_seqlens_q, cu_seqlens_k, &Tq, &Tk);
  if (so != DSAI_OK || Tq == 0) return so;
  if (!index_q || !weights || !out_idx || !out_score) return DSAI_ERR_NULLPTR;
  if (Tk > 0 && !index_k) return DSAI_ERR_NULLPTR;
  if (!aligned(index_q) || !aligned(index_k) || !aligned(out_idx) || !aligned(out_score) ||
      !aligned(topk_indices))
    return DSAI_ERR_INVALID_ARG;
  const int64_t H = h->cfg.heads, D = h->cfg.dim;
  const bool sort = h->cfg.order == DSAI_ORDER_SCORE && !topk_indices;
  if (!topk_indices) {  // every refusal before the first launch
    hipError_t e = device_limits(h);
    if (e != hipSuccess) return hip_status(h, e);
    for (int64_t i = 0; i < nseq; ++i) {
      const int64_t Skv = cu_seqlens_k[i + 1] - cu_seqlens_k[i];
      if (cu_seqlens_q[i + 1] == cu_seqlens_q[i]) continue;
      if (Skv * D * 2 > (int64_t)0xFFFFFFFF) return DSAI_ERR_UNSUPPORTED;
      if (dsai::plan_score_select(H <= 32 ? 32 : 64, (int)D, topk, Skv, h->lds_limit)
              .rows_per_block < 1)
        return DSAI_ERR_UNSUPPORTED;
    }
  }
  // Sequence i is the one-sample problem on its own rows and keys (topk % 4
  // == 0 keeps each sequence's output rows 16-byte aligned).
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t le = hipSuccess;
  if (topk_indices) {
    // Scores at supplied indices: one launch per sequence (per chunk of
    // cfg.chunk_rows rows), consecutive sequences alternating between the
    // handle's two streams so that two are in flight.
    le = on_side_streams(h, st, [&](hipStream_t s0, hipStream_t s1) {
      int64_t j = 0;
      for (int64_t i = 0; i < nseq; ++i) {
        const int64_t q0 = cu_seqlens_q[i], k0 = cu_seqlens_k[i];
        const int64_t S = cu_seqlens_q[i + 1] - q0, Skv = cu_seqlens_k[i + 1] - k0;
        if (S == 0) continue;
        const hipStream_t sj = (j++ & 1) ? s1 : s0;
        dsai::ScoreAtArgs a;
        a.q = static_cast<const uint16_t*>(index_q) + q0 * H * D;
        a.k = Skv > 0 ? static_cast<const uint16_t*>(index_k) + k0 * D : nullptr;
        a.w = weights + q0 * H;
        a.S = S; a.Skv = Skv; a.B = 1;
        a.H = (int)H; a.D = (int)D; a.ratio = compress_ratio; a.n = topk;
        a.chunk_rows = h->cfg.chunk_rows;
        a.sup = topk_indices + q0 * topk;
        a.out_idx = out_idx + q0 * topk; a.out_score = out_score + q0 * topk;
        const hipError_t e = launch_scores_at(h, a, sj, nullptr);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    });
  } else {
    // Selection: sequences in order of their longest row (most keys first,
    // stable), up to kPackedMax per launch of the fused kernel, all on
    // `stream`; each launch's plan is the one of its longest key range.
    std::vector<int64_t> order;
    order.reserve((size_t)nseq);
    for (int64_t i = 0; i < nseq; ++i)
      if (cu_seqlens_q[i + 1] > cu_seqlens_q[i]) order.push_back(i);
    auto heaviest = [&](int64_t i) {
      const int64_t S = cu_seqlens_q[i + 1] - cu_seqlens_q[i];
      const int64_t Skv = cu_seqlens_k[i + 1] - cu_seqlens_k[i];
      return std::min(Skv, S / compress_ratio);
    };
    std::stable_sort(order.begin(), order.end(),
                     [&](int64_t x, int64_t y) { return heaviest(x) > heaviest(y); });
    dsai::PackedTopkArgs a;
    a.q = static_cast<const uint16_t*>(index_q);
    a.k = static_cast<const uint16_t*>(index_k);
    a.w = weights;
    a.H = (int)H; a.D = (int)D; a.ratio = compress_ratio; a.topk = topk;
    a.out_idx = out_idx; a.out_score = out_score;
    a.est_cuts = h->cfg.cuts == DSAI_CUTS_ESTIMATED;
    for (size_t g0 = 0; g0 < order.size() && le == hipSuccess; g0 += dsai::kPackedMax) {
      const size_t g1 = std::min(order.size(), g0 + (size_t)dsai::kPackedMax);
      int64_t skv_max = 0;
      for (size_t j = g0; j < g1; ++j)
        skv_max = std::max(skv_max, cu_seqlens_k[order[j] + 1] - cu_seqlens_k[order[j]]);
      const dsai::ScoreSelectPlan plan =
          dsai::plan_score_select(H <= 32 ? 32 : 64, (int)D, topk, skv_max, h->lds_limit);
      dsai::PackedSeqs t;
      t.n = (int)(g1 - g0);
      for (int m = 0; m <= dsai::kPackedMax; ++m) t.blk_begin[m] = INT32_MAX;
      t.blk_begin[0] = 0;
      for (size_t j = g0; j < g1; ++j) {
        const int64_t i = order[j], m = (int64_t)(j - g0);
        t.q0[m] = (int)cu_seqlens_q[i];
        t.k0[m] = (int)cu_seqlens_k[i];
        t.S[m] = (int)(cu_seqlens_q[i + 1] - cu_seqlens_q[i]);
        t.Skv[m] = (int)(cu_seqlens_k[i + 1] - cu_seqlens_k[i]);
        t.blk_begin[m + 1] = t.blk_begin[m] + (t.S[m] + plan.rows_per_block - 1) / plan.rows_per_block;
      }
      le = dsai::launch_score_topk_packed(a, t, plan, st);
    }
  }
  if (le == hipSuccess && sort) le = dsai::launch_sort_rows(out_idx, out_score, Tq, topk, st);
  return hip_status(h, le);
}

int dsai_backward_workspace_size(dsai_handle h, int64_t S, int64_t Skv, int64_t B, int topk,
                                 int compress_ratio, size_t* bytes) {
  if (!h || !bytes) return DSAI_ERR_NULLPTR;
  if (S < 0 || Skv < 0 || B < 0 || topk < 1 || topk > DSAI_MAX_TOPK || compress_ratio < 1)
    return DSAI_ERR_INVALID_ARG;
  if (S > kI32 || Skv > kI32 || B > kI32 || S * B > kI32 || Skv * B > kI32)
    return DSAI_ERR_INVALID_ARG;
  *bytes = dsai::plan_backward(S, Skv, B, h->cfg.dim, topk, compress_ratio).bytes;
  return DSAI_OK;
}

int dsai_indexer_backward(dsai_handle h, const void* index_q, const void* index_k,
                          const float* weights, const int32_t* topk_indices,
                          const float* grad_scores, int64_t S, int64_t Skv, int64_t B,
                          int compress_ratio, int topk, void* grad_q, void* grad_k,
                          float* grad_weights, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  if (S < 0 || Skv < 0 || B < 0 || compress_ratio < 1) return DSAI_ERR_INVALID_ARG;
  if (topk < 1 || topk > DSAI_MAX_TOPK) return DSAI_ERR_INVALID_ARG;
  if (S > kI32 || Skv > kI32 || B > kI32 || S * B > kI32 || Skv * B > kI32)
    return DSAI_ERR_INVALID_ARG;
  if (B == 0 || (S == 0 && Skv == 0)) return DSAI_OK;
  const dsai::BackwardPlan plan = dsai::plan_backward(S, Skv, B, h->cfg.dim, topk, compress_ratio);
  if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes ||
                         reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
    return DSAI_ERR_WORKSPACE;
  if (Skv > 0 && (!index_k || !grad_k)) return DSAI_ERR_NULLPTR;
  if (S > 0 && (!index_q || !weights || !topk_indices || !grad_scores || !grad_q || !grad_weights))
    return DSAI_ERR_NULLPTR;
  if (!aligned(index_q) || !aligned(index_k) || !aligned(grad_q) || !aligned(grad_k) ||
      reinterpret_cast<uintptr_t>(topk_indices) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(grad_scores) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(weights) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(grad_weights) % 4 != 0)
    return DSAI_ERR_INVALID_ARG;
  dsai::BackwardArgs a;
  a.q = static_cast<const uint16_t*>(index_q);
  a.k = static_cast<const uint16_t*>(index_k);
  a.w = weights;
  a.sup = topk_indices;
  a.grad = grad_scores;
  a.S = S; a.Skv = Skv; a.B = B;
  a.H = h->cfg.heads; a.D = h->cfg.dim; a.ratio = compress_ratio; a.n = topk;
  a.grad_q = static_cast<uint16_t*>(grad_q);
  a.grad_k = static_cast<uint16_t*>(grad_k);
  a.grad_w = grad_weights;
  a.ws = workspace;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (S == 0 || Skv == 0) return hip_status(h, dsai::launch_indexer_backward(a, plan, st, st));
  // the key gradients and the matrix-core-bound per-row gradients overlap on
  // the handle's two streams
  return hip_status(h, on_side_streams(h, st, [&](hipStream_t s0, hipStream_t s1) {
                      return dsai::launch_indexer_backward(a, plan, s0, s1);
                    }));
}

int dsai_backward_packed_workspace_size(dsai_handle h, int64_t nseq, const int64_t* cu_seqlens_q,
                                        const int64_t* cu_seqlens_k, int topk,
                                        int compress_ratio, size_t* bytes) {
  if (!h || !bytes) return DSAI_ERR_NULLPTR;
  if (topk < 1 || topk > DSAI_MAX_TOPK || compress_ratio < 1) return DSAI_ERR_INVALID_ARG;
  int64_t Tq = 0, Tk = 0;
  const int so = check_offsets(nseq, cu_seqlens_q, cu_seqlens_k, &Tq, &Tk);
  if (so != DSAI_OK) return so;
  size_t most = 0;
  for (int64_t i = 0; i < nseq; ++i) {
    const size_t b = dsai::plan_backward(cu_seqlens_q[i + 1] - cu_seqlens_q[i],
                                         cu_seqlens_k[i + 1] - cu_seqlens_k[i], 1, h->cfg.dim,
                                         topk, compress_ratio).bytes;
    most = b > most ? b : most;
  }
  *bytes = most;
  return DSAI_OK;
}

int dsai_indexer_backward_packed(dsai_handle h, const void* index_q, const void* index_k,
                                 const float* weights, const int32_t* topk_indices,
                                 const float* grad_scores, int64_t nseq,
                                 const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k,
                                 int compress_ratio, int topk, void* grad_q, void* grad_k,
                                 float* grad_weights, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  if (compress_ratio < 1 || topk < 1 || topk > DSAI_MAX_TOPK) return DSAI_ERR_INVALID_ARG;
  int64_t Tq = 0, Tk = 0;
  int st = check_offsets(nseq, cu_seqlens_q, cu_seqlens_k, &Tq, &Tk);
  if (st != DSAI_OK || (Tq == 0 && Tk == 0)) return st;
  // every refusal before the first launch: the workspace must hold the
  // largest sequence's plan, and the base pointers pass the per-sample checks
  // (each sequence's slices are offsets of whole rows from them)
  size_t need = 0;
  st = dsai_backward_packed_workspace_size(h, nseq, cu_seqlens_q, cu_seqlens_k, topk,
                                           compress_ratio, &need);
  if (st != DSAI_OK) return st;
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
    return DSAI_ERR_WORKSPACE;
  if (Tk > 0 && (!index_k || !grad_k)) return DSAI_ERR_NULLPTR;
  if (Tq > 0 && (!index_q || !weights || !topk_indices || !grad_scores || !grad_q || !grad_weights))
    return DSAI_ERR_NULLPTR;
  if (!aligned(index_q) || !aligned(index_k) || !aligned(grad_q) || !aligned(grad_k) ||
      reinterpret_cast<uintptr_t>(topk_indices) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(grad_scores) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(weights) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(grad_weights) % 4 != 0)
    return DSAI_ERR_INVALID_ARG;
  const int64_t H = h->cfg.heads, D = h->cfg.dim;
  // One per-sample backward per sequence, in order on `stream` (they share
  // the workspace); a sequence with no rows still zeroes its keys' grad_k.
  for (int64_t i = 0; i < nseq; ++i) {
    const int64_t q0 = cu_seqlens_q[i], k0 = cu_seqlens_k[i];
    const int64_t S = cu_seqlens_q[i + 1] - q0, Skv = cu_seqlens_k[i + 1] - k0;
    if (S == 0 && Skv == 0) continue;
    st = dsai_indexer_backward(
        h, S > 0 ? static_cast<const uint16_t*>(index_q) + q0 * H * D : nullptr,
        Skv > 0 ? static_cast<const uint16_t*>(index_k) + k0 * D : nullptr,
        S > 0 ? weights + q0 * H : nullptr, S > 0 ? topk_indices + q0 * topk : nullptr,
        S > 0 ? grad_scores + q0 * topk : nullptr, S, Skv, 1, compress_ratio, topk,
        S > 0 ? static_cast<uint16_t*>(grad_q) + q0 * H * D : nullptr,
        Skv > 0 ? static_cast<uint16_t*>(grad_k) + k0 * D : nullptr,
        S > 0 ? grad_weights + q0 * H : nullptr, workspace, workspace_bytes, stream);
    if (st != DSAI_OK) return st;
  }
  return DSAI_OK;
}

int dsai_pool_count(dsai_handle h, int64_t N, int64_t* P) {
  if (!h || !P) return DSAI_ERR_NULLPTR;
  if (N < 0) return DSAI_ERR_INVALID_ARG;
  const int64_t avail = N - h->cfg.first_key;
  *P = avail > 0 ? avail / h->cfg.kpool : 0;
  return DSAI_OK;
}

int dsai_kpool_compress(dsai_handle h, const void* k_normed, const float* gate,
                        const uint8_t* valid, const float* ape, int64_t N, void* pool_k,
                        int32_t* pool_tok, uint8_t* pool_valid, void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  if (N < 0 || N > kI32) return DSAI_ERR_INVALID_ARG;
  int64_t P = 0;
  dsai_pool_count(h, N, &P);
  if (P == 0) return DSAI_OK;
  if (!k_normed || !gate || !valid || !ape || !pool_k || !pool_tok || !pool_valid)
    return DSAI_ERR_NULLPTR;
  if (!aligned(k_normed) || !aligned(gate) || !aligned(ape) || !aligned(pool_k))
    return DSAI_ERR_INVALID_ARG;
  dsai::KpoolArgs a;
  a.k_normed = static_cast<const uint16_t*>(k_normed);
  a.gate = gate; a.valid = valid; a.ape = ape;
  a.D = h->cfg.dim; a.KP = h->cfg.kpool; a.first_key = h->cfg.first_key; a.P = P;
  a.pool_k = static_cast<uint16_t*>(pool_k); a.pool_tok = pool_tok; a.pool_valid = pool_valid;
  return hip_status(h, dsai::launch_kpool(a, static_cast<hipStream_t>(stream)));
}

// Host checks of index_scores' arguments (no HIP call).
static int check_index_scores(dsai_handle h, const void* q, const float* w, const void* pool_k,
                              const uint8_t* pool_valid, const int32_t* pool_limit, int64_t Q,
                              int64_t P, const void* scores) {
  if (Q < 0 || P < 0 || Q > kI32 || P > kI32) return DSAI_ERR_INVALID_ARG;
  if (Q == 0 || P == 0) return DSAI_OK;
  if (P * h->cfg.dim * 2 > (int64_t)0xFFFFFFFF) return DSAI_ERR_UNSUPPORTED;  // 32-bit offsets
  if (!q || !w || !pool_k || !pool_valid || !scores) return DSAI_ERR_NULLPTR;
  if (!aligned(q) || !aligned(pool_k) || reinterpret_cast<uintptr_t>(pool_limit) % 4 != 0)
    return DSAI_ERR_INVALID_ARG;
  return DSAI_OK;
}

static hipError_t launch_index_scores(dsai_handle h, const void* q, const float* w,
                                      const void* pool_k, const uint8_t* pool_valid,
                                      const int32_t* pool_limit, int64_t Q, int64_t P,
                                      float* scores, hipStream_t st) {
  dsai::PooledScoresArgs a;
  a.q = static_cast<const uint16_t*>(q); a.w = w;
  a.pool_k = static_cast<const uint16_t*>(pool_k); a.pool_valid = pool_valid;
  a.limit = pool_limit;
  a.Q = Q; a.P = P; a.H = h->cfg.heads; a.D = h->cfg.dim; a.scores = scores;
  return dsai::launch_pooled_scores(a, st);
}

int dsai_index_scores(dsai_handle h, const void* q, const float* w, const void* pool_k,
                      const uint8_t* pool_valid, const int32_t* pool_limit, int64_t Q, int64_t P,
                      float* scores, void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  const int st = check_index_scores(h, q, w, pool_k, pool_valid, pool_limit, Q, P, scores);
  if (st != DSAI_OK || Q == 0 || P == 0) return st;
  return hip_status(h, launch_index_scores(h, q, w, pool_k, pool_valid, pool_limit, Q, P, scores,
                                           static_cast<hipStream_t>(stream)));
}

// Launch plan of topk_pools (queries the device's LDS limit once).
static int plan_pools(dsai_handle h, int64_t P, dsai::TopkRowsPlan* plan) {
  hipError_t e = device_limits(h);
  if (e != hipSuccess) return hip_status(h, e);
  *plan = dsai::plan_topk_rows(select_k(h->cfg), P, h->lds_limit);
  return plan->waves < 1 ? DSAI_ERR_UNSUPPORTED : DSAI_OK;
}

// topk_pools, and with `tokens` the rows expanded to token ids as well.
static hipError_t launch_pools(dsai_handle h, const dsai::TopkRowsPlan& plan, const float* scores,
                               int64_t Q, int64_t P, int32_t* pool_ids, float* pool_scores,
                               int32_t* tokens, hipStream_t st) {
  dsai::TopkPoolsArgs a;
  a.scores = scores; a.Q = Q; a.P = P; a.sel = select_k(h->cfg);
  a.pool_ids = pool_ids; a.pool_scores = pool_scores;
  a.sort = h->cfg.order == DSAI_ORDER_SCORE;
  a.tokens = tokens; a.KP = h->cfg.kpool; a.first_key = h->cfg.first_key;
  return dsai::launch_topk_pools(a, plan, st);
}

int dsai_topk_pools(dsai_handle h, const float* scores, int64_t Q, int64_t P, int32_t* pool_ids,
                    float* pool_scores, void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  if (Q < 0 || P < 0 || Q > kI32 || P > kI32) return DSAI_ERR_INVALID_ARG;
  if (Q == 0) return DSAI_OK;
  if (!pool_ids || !pool_scores || (P > 0 && !scores)) return DSAI_ERR_NULLPTR;
  dsai::TopkRowsPlan plan;
  const int st = plan_pools(h, P, &plan);
  if (st != DSAI_OK) return st;
  return hip_status(h, launch_pools(h, plan, scores, Q, P, pool_ids, pool_scores, nullptr,
                                    static_cast<hipStream_t>(stream)));
}

int dsai_select_workspace_size(dsai_handle h, int64_t Q, int64_t P, size_t* bytes) {
  if (!h || !bytes) return DSAI_ERR_NULLPTR;
  if (Q < 0 || P < 0) return DSAI_ERR_INVALID_ARG;
  *bytes = (size_t)Q * (size_t)P * sizeof(float);
  return DSAI_OK;
}

// index_scores into `scores` ([Q, P] fp32, device memory the caller
// provides), then topk_pools (with `tokens`: expanded as well).  Every
// refusal, the topk_pools plan included, comes before the first launch.
static int select_into(dsai_handle h, const void* q, const float* w, const void* pool_k,
                       const uint8_t* pool_valid, const int32_t* pool_limit, int64_t Q,
                       int64_t P, int32_t* pool_ids, float* pool_scores, int32_t* tokens,
                       float* scores, void* stream) {
  int st = check_index_scores(h, q, w, pool_k, pool_valid, pool_limit, Q, P, scores);
  if (st != DSAI_OK) return st;
  if (!pool_ids || !pool_scores) return DSAI_ERR_NULLPTR;
  dsai::TopkRowsPlan plan;
  if ((st = plan_pools(h, P, &plan)) != DSAI_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (P > 0) {
    const hipError_t e =
        launch_index_scores(h, q, w, pool_k, pool_valid, pool_limit, Q, P, scores, s);
    if (e != hipSuccess) return hip_status(h, e);
  }
  return hip_status(h, launch_pools(h, plan, scores, Q, P, pool_ids, pool_scores, tokens, s));
}

static int check_workspace(dsai_handle h, int64_t Q, int64_t P, const void* workspace,
                           size_t workspace_bytes) {
  size_t need = 0;
  dsai_select_workspace_size(h, Q, P, &need);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
    return DSAI_ERR_WORKSPACE;
  return DSAI_OK;
}

int dsai_select(dsai_handle h, const void* q, const float* w, const void* pool_k,
                const uint8_t* pool_valid, const int32_t* pool_limit, int64_t Q, int64_t P,
                int32_t* pool_ids, float* pool_scores, void* workspace, size_t workspace_bytes,
                void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  if (Q < 0 || P < 0 || Q > kI32 || P > kI32) return DSAI_ERR_INVALID_ARG;
  if (Q == 0) return DSAI_OK;
  const int st = check_workspace(h, Q, P, workspace, workspace_bytes);
  if (st != DSAI_OK) return st;
  return select_into(h, q, w, pool_k, pool_valid, pool_limit, Q, P, pool_ids, pool_scores,
                     nullptr, static_cast<float*>(workspace), stream);
}

// Token ids of the expanded rows are int32: the last token of the last pool,
// first_key + P * kpool - 1, must fit.
static bool tokens_fit(const dsai_config& c, int64_t P) {
  return (int64_t)c.first_key + P * (int64_t)c.kpool - 1 <= kI32;
}

static int check_select_expand(dsai_handle h, int64_t Q, int64_t P, const int32_t* pool_ids,
                               const float* pool_scores, const int32_t* tokens) {
  if (Q < 0 || P < 0 || Q > kI32 || P > kI32) return DSAI_ERR_INVALID_ARG;
  if (Q == 0) return DSAI_OK;
  if (!tokens || !pool_ids || !pool_scores) return DSAI_ERR_NULLPTR;
  if (!aligned(tokens) || !tokens_fit(h->cfg, P)) return DSAI_ERR_INVALID_ARG;
  return DSAI_OK;
}

int dsai_select_expand(dsai_handle h, const void* q, const float* w, const void* pool_k,
                       const uint8_t* pool_valid, const int32_t* pool_limit, int64_t Q,
                       int64_t P, int32_t* pool_ids, float* pool_scores, int32_t* tokens,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  int st = check_select_expand(h, Q, P, pool_ids, pool_scores, tokens);
  if (st != DSAI_OK || Q == 0) return st;
  if ((st = check_workspace(h, Q, P, workspace, workspace_bytes)) != DSAI_OK) return st;
  return select_into(h, q, w, pool_k, pool_valid, pool_limit, Q, P, pool_ids, pool_scores,
                     tokens, static_cast<float*>(workspace), stream);
}

// ---- dsai_select_expand_static: the [Q, P] scores in a static device array --
// One copy per device, held by the library until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device copy: the
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[DSAI_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch`.
hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

int dsai_select_expand_static(dsai_handle h, const void* q, const float* w, const void* pool_k,
                              const uint8_t* pool_valid, const int32_t* pool_limit, int64_t Q,
                              int64_t P, int32_t* pool_ids, float* pool_scores, int32_t* tokens,
                              void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  int st = check_select_expand(h, Q, P, pool_ids, pool_scores, tokens);
  if (st != DSAI_OK || Q == 0) return st;
  size_t need = 0;
  dsai_select_workspace_size(h, Q, P, &need);
  if (need > (size_t)DSAI_STATIC_SCRATCH_BYTES) return DSAI_ERR_WORKSPACE;
  void* buf = nullptr;
  const hipError_t e = static_scratch(&buf);
  if (e != hipSuccess) return hip_status(h, e);
  return select_into(h, q, w, pool_k, pool_valid, pool_limit, Q, P, pool_ids, pool_scores,
                     tokens, static_cast<float*>(buf), stream);
}

int dsai_expand(dsai_handle h, const int32_t* pool_ids, int64_t Q, int32_t* tokens,
                void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  if (Q < 0 || Q > kI32) return DSAI_ERR_INVALID_ARG;
  if (Q == 0) return DSAI_OK;
  if (!pool_ids || !tokens) return DSAI_ERR_NULLPTR;
  if (!aligned(tokens)) return DSAI_ERR_INVALID_ARG;
  dsai::ExpandArgs a;
  a.pool_ids = pool_ids; a.Q = Q; a.sel = select_k(h->cfg); a.KP = h->cfg.kpool;
  a.first_key = h->cfg.first_key; a.tokens = tokens;
  return hip_status(h, dsai::launch_expand(a, static_cast<hipStream_t>(stream)));
}

int dsai_k_norm(dsai_handle h, const void* k_raw, const void* gamma, const void* beta, float eps,
                int64_t N, void* k_normed, void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  if (N < 0 || !(eps > 0.0f) || !(eps < INFINITY)) return DSAI_ERR_INVALID_ARG;
  if (N == 0) return DSAI_OK;
  if (!k_raw || !gamma || !beta || !k_normed) return DSAI_ERR_NULLPTR;
  if (!aligned(k_raw) || !aligned(gamma) || !aligned(beta) || !aligned(k_normed))
    return DSAI_ERR_INVALID_ARG;
  dsai::KNormArgs a;
  a.x = static_cast<const uint16_t*>(k_raw);
  a.gamma = static_cast<const uint16_t*>(gamma);
  a.beta = static_cast<const uint16_t*>(beta);
  a.eps = eps; a.n = N; a.D = h->cfg.dim;
  a.y = static_cast<uint16_t*>(k_normed);
  return hip_status(h, dsai::launch_k_norm(a, static_cast<hipStream_t>(stream)));
}

int dsai_sort_rows(dsai_handle h, int32_t* idx, float* score, int64_t rows, int k, void* stream) {
  if (!h) return DSAI_ERR_NULLPTR;
  if (rows < 0 || rows > kI32 || k < 1 || k > DSAI_MAX_TOPK) return DSAI_ERR_INVALID_ARG;
  if (rows == 0 || k == 1) return DSAI_OK;
  if (!idx || !score) return DSAI_ERR_NULLPTR;
  if (reinterpret_cast<uintptr_t>(idx) % 4 != 0 || reinterpret_cast<uintptr_t>(score) % 4 != 0)
    return DSAI_ERR_INVALID_ARG;
  return hip_status(h, dsai::launch_sort_rows(idx, score, rows, k, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
