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
// One workgroup = NW wavefronts (4 or 8); each wavefront owns one query row of
// a block of up to NW consecutive rows of one batch, so the rows of a block
// see nearly the same keys.  The block streams its keys through two LDS
// buffers of 32-key tiles (loaded once per block, shared by its rows; the
// next tile is written while the current one is read, one barrier per tile).
// Each wavefront scores the tile on the matrix cores (TileScorer) and records
// the scores in its LDS row store:
//   dense   when every visible key fits: the fp32 score of key s goes to slot
//           s (no indices, no selection until the end);
//   filter  otherwise: keys beating the row's running threshold are appended
//           (order key and index); when a store fills, every wavefront of
//           the block whose store is past half its slack cuts it together
//           (a bin-edge cut to a rank: k, or by default the share of the top
//           k that the keys seen so far are expected to hold, with a margin;
//           every key dropped ranks below every key kept), which raises the
//           thresholds.  A row that ends with fewer than k entries although
//           it has k keys lost some of its top k to an estimated cut: its
//           block then runs its keys again with cuts to k.
// After the last tile the row's top k is selected exactly and written in
// ascending index order; no score goes to device memory.  With supplied
// indices (dense store only) the row's entries are read from its store
// instead of selected.  (Score-descending order is produced by the row
// sort.)  Blocks are numbered heaviest (largest t) first so the causal
// imbalance is absorbed by the dispatcher.
#include "internal.h"
#include "score_tile.h"
#include "topk_wave.h"

namespace dsai {

// LDS bytes per wavefront of the final select (histogram and side list);
// they live in the tile buffers once the key loop is done.
constexpr int kDenseScratch = 2048;

// LDS bytes per wavefront the filter store's cuts use during the key loop
// (one 256-bin histogram; the bin-edge cut needs no side list).
constexpr int kCutScratch = 1024;

// Static LDS of the filter-store kernels (cut requests, the short-row flag),
// rounded up.
constexpr int64_t kStaticLds = 128;

// A filter store asks for a cut once fewer than this many slots are free:
// the request is served within four more tiles (32 keys each) after the
// one that raised it.
constexpr int kCutRequest = 6 * 32;

// Rank a filter-store cut keeps when it estimates.  If the order of a row's
// N keys says nothing about their scores, the number of the row's final top
// k among the first n keys is hypergeometric: mean k n / N, variance at most
// that mean times (1 - n / N).  A cut to that mean plus six standard
// deviations and 32 loses none of the top k except with negligible
// probability; when it does, the row ends short and the block reruns
// exactly.  Exact cuts, and cuts once every key is seen, keep k.
__device__ __forceinline__ uint32_t cut_rank(uint32_t k, uint32_t n, uint32_t N, bool exact) {
  if (exact || n >= N) return k;
  const float f = (float)n / (float)N;
  const float mu = (float)k * f;
  const float m = mu + 6.f * __builtin_sqrtf(mu * (1.f - f)) + 32.f;
  return m < (float)k ? (uint32_t)m + 1u : k;
}

template <int D, int NW>
struct ScoreLds {
  static constexpr int kTileBytes = TileGeom<D>::kTileBytes;
  static constexpr int kTiles = 2 * kTileBytes;  // double buffer
  // dense: stage buffers (reused by the final select) | rows
  static constexpr int kDenseRegion = kTiles > NW * kDenseScratch ? kTiles : NW * kDenseScratch;
};

// The body of the kernels below: sup == nullptr selects, else the supplied
// entries are read from the dense store.  est: the filter store's cuts keep
// an estimated rank (cut_rank) instead of k.
template <int HP, int D, int NW, int NR, bool DENSE, typename IdxT>
__device__ __forceinline__ void score_select_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    int S, int Skv, int B, int H, int ratio, int topk, int row_begin, int row_end, int R, int cap,
    int32_t* __restrict__ out_idx, float* __restrict__ out_score, const int32_t* sup, int bid,
    bool est) {
  extern __shared__ __align__(16) char smem_raw[];
  // filter store: cut requests, one 8-byte word per tile modulo 3, byte w
  // written by wavefront w after recording that tile (1: its store is nearly
  // full)
  __shared__ uint64_t cut_req[3];
  // filter store with estimated cuts: set by a wavefront whose row ended
  // with fewer than k entries (the block then runs its keys again, exactly)
  __shared__ uint32_t short_rows;
  lds_char* smem = (lds_char*)smem_raw;
  using G = TileGeom<D>;
  using L = ScoreLds<D, NW>;
  using Scorer = TileScorer<HP, D, NR>;
  using Acc = typename Scorer::Acc;
  constexpr int kThreads = NW * 64;

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform
  const int lane = lane_id();
  const int row_bytes = DENSE ? cap * 4 : cap * 4 + ((cap * (int)sizeof(IdxT) + 15) & ~15);
  const int region = DENSE ? L::kDenseRegion : L::kTiles + NW * kCutScratch;

  // dense: the final select's histogram and side list, in the tile buffers;
  // filter: the cuts' histogram (its own region), and after the key loop the
  // final select's side list in the tile buffers (2 KB per wavefront)
  lds_u32* scratch = DENSE ? (lds_u32*)(smem + wave * kDenseScratch)
                           : (lds_u32*)(smem + L::kTiles + wave * kCutScratch);
  lds_u32* side = DENSE ? scratch + 256 : (lds_u32*)(smem + wave * (L::kTiles / NW));
  constexpr uint32_t kSideCap =
      DENSE ? 256u : ((L::kTiles / NW) / 4 < 256 ? (L::kTiles / NW) / 4 : 256u);

  // Rows of the block: t0 .. t0 + R - 1; wavefront `wave` owns rows
  // t0 + wave * NR + rr, rr < NR, each with its own LDS row store.
  const int nrow = row_end - row_begin;
  const int nrb = (nrow + R - 1) / R;
  const int jb = bid / B;
  const int b = bid - jb * B;
  const int t0 = row_begin + (nrb - 1 - jb) * R;
  const int t_last = min(t0 + R, row_end) - 1;
  const int n_max = min(Skv, (t_last + 1) / ratio);
  const int ntiles = (n_max + G::kTileKeys - 1) / G::kTileKeys;

  // The first two key tiles' loads go out before the query rows' loads, so
  // staging them waits for those two loads only, while the query rows are
  // still in flight.
  TileLoader<D, kThreads> ld, ld1;
  const int64_t kbytes = ((int64_t)Skv * B - b) * D * 2;  // < 2^32 (checked on the host)
  ld.init(k + (int64_t)b * D, (uint32_t)(B * D), (uint32_t)(kbytes > 0 ? kbytes : 0));
  ld1.init(k + (int64_t)b * D, (uint32_t)(B * D), (uint32_t)(kbytes > 0 ? kbytes : 0));
  if (ntiles > 0) {
    ld.load(0u);
    ld1.load((uint32_t)G::kTileKeys);
  }

  Scorer sc;
  sc.init_offsets();
  // 16-byte weight loads when every row's weights are 16-byte aligned
  const bool w4 = (H & 3) == 0 && ((uintptr_t)w & 15u) == 0;
  RowStore<IdxT> rs[NR];
  int t[NR], n_t[NR];
  bool active[NR];
  int n_w = 0;  // keys of the wave's longest row
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    const int slot = wave * NR + rr;
    t[rr] = t0 + slot;
    active[rr] = slot < R && t[rr] < row_end;
    n_t[rr] = active[rr] ? min(Skv, (t[rr] + 1) / ratio) : 0;
    n_w = max(n_w, n_t[rr]);
    lds_char* mine = smem + region + slot * row_bytes;
    rs[rr] = RowStore<IdxT>{(lds_u32*)mine, (DSAI_LDS IdxT*)(mine + cap * 4), scratch, side,
                            kSideCap};
    const int64_t row = (int64_t)(active[rr] ? t[rr] : 0) * B + b;
    // dense store: the query row comes in through the row's store (the key
    // loop writes it only after the row's fragments are in registers); the
    // filter kernels keep the direct loads (their registers are fuller)
    bool staged = false;
    if constexpr (DENSE) staged = row_bytes >= Scorer::kStageBytes;
    if (staged)
      sc.load_row_staged(rr, q + row * H * D, w + row * H, H, active[rr], w4, mine);
    else
      sc.load_row(rr, q + row * H * D, w + row * H, H, active[rr]);
  }

  if (!DENSE && threadIdx.x < 3) cut_req[threadIdx.x] = 0u;  // published by the loop's first barrier
  if (!DENSE && threadIdx.x == 3) short_rows = 0u;
  uint32_t count[NR], tau[NR];       // filter store: entries, running threshold
  uint32_t kmax[NR];                 // filter store: this lane's largest appended key
  // a bin-edge cut may keep a few entries past its rank; one that would keep
  // more than a quarter of the store's slack cuts exactly instead
  const uint32_t slack_keep = (uint32_t)(cap - topk) / 4u;
  float smin[NR], smax[NR];           // dense store: this lane's extreme scores
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    count[rr] = tau[rr] = kmax[rr] = 0u;
    smin[rr] = __builtin_inff();
    smax[rr] = -__builtin_inff();
  }

  // Keys stream in 32-key tiles through two LDS buffers, one barrier per
  // tile.  Every wavefront runs all of the block's tiles, so the
  // steady-state iteration has no branch: rows shorter than the block's
  // longest score a few keys past their n_t, which are never recorded;
  // stores and loads of tiles past the last one move unused data (rows past
  // the key range read as zero).  Iteration `it`, after the barrier that
  // publishes tile it + 1:
  //   fetch tile it + 1's fragments into registers (consumed next
  //   iteration, so no MFMA waits on LDS);
  //   record tile it - 2 (cross-half sum; dense: the score goes to its
  //   slot; filter: appended if it beats the row's threshold, the store cut
  //   to the top k when full);
  //   write tile it + 2 (loaded during the previous iteration) into buffer
  //   it & 1, whose last reader, the fetch of tile it, completed before
  //   this barrier; start the loads of tile it + 3;
  //   tile it's products on the matrix cores, interleaved with the head
  //   reduction of tile it - 1.
  // Every LDS access is issued early in its iteration, so the next barrier
  // does not wait on a recent one.
  using Frag = typename Scorer::Frag;
  // Buffer of a tile of parity p.  Every step knows the parity of its tile
  // at compile time (tile it's products go to acc0 when it is even, acc1
  // when odd, and a run of the filter loop starts at an even tile), so the
  // buffers' LDS addresses fold into the instructions' offsets.
  auto buf = [&](int p) { return smem + p * L::kTileBytes; };
  Acc acc0, acc1;
  Frag f0;  // one fragment buffer, refilled as each tile's products are issued
  typename Scorer::Spare sp0, sp1;  // the last k-steps' fragments of even / odd tiles
  float part[NR];    // reduce_half of the even tile of the pair awaiting its record
  float part_b[NR];  // ... and of its odd tile
  // Tiles are recorded two at a time: one cross-half exchange leaves tile
  // it_a's scores in lanes 0-31 and tile it_a + 1's in lanes 32-63, so every
  // lane of the record carries its own key (it_a * 32 + lane).
  // dense: the score goes to its key's slot (slots past the row's keys are
  // written but never read); filter: appended if it beats the threshold.
  auto record2 = [&](int it_a) {
    const uint32_t key = (uint32_t)(it_a * G::kTileKeys + lane);
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      const float x = Scorer::combine2(part[rr], part_b[rr]) + 0.f;  // -0 -> +0
      const bool vis = key < (uint32_t)n_t[rr];
      if constexpr (DENSE) {
        rs[rr].key[key] = __float_as_uint(x);
        smin[rr] = fminf(smin[rr], vis ? x : __builtin_inff());
        smax[rr] = fmaxf(smax[rr], vis ? x : -__builtin_inff());
      } else {
        const uint32_t u = ord_key_nz(x);  // x + 0 is never -0
        // (non-short-circuit: no branch)
        const bool pass = vis & (u > tau[rr]);
        wave_append_all(rs[rr], count[rr], pass, u, key);
        kmax[rr] = max(kmax[rr], pass ? u : 0u);  // running maximum of the store's keys
      }
    }
    if constexpr (!DENSE) {
      // Ask for a cut once a store has fewer than kCutRequest free slots:
      // every lane writes the wavefront's own byte, so no branch and no
      // clearing.
      bool need = false;
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) need |= count[rr] > (uint32_t)(cap - kCutRequest);
      ((DSAI_LDS uint8_t*)&cut_req[(it_a >> 1) % 3])[wave] = need ? 1u : 0u;
    }
  };
  // Head reduction of a tile's products: the even tile of a pair into part,
  // the odd one into part_b.
  auto reduce_into = [&](int par, const Acc& a) {
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      if (par == 0) part[rr] = sc.reduce_half(a, rr);
      else part_b[rr] = sc.reduce_half(a, rr);
    }
  };
  if (ntiles > 0) {
    ld.store(buf(0));
    ld1.store(buf(1));
    if constexpr (DENSE) {
      // Step `it` (parity par): tile it's products (the fragment registers
      // refilled with tile it + 1 as they are issued); the reduction of tile
      // it - 1; in odd steps the record of tiles it - 3 and it - 2.
      auto step = [&](int it, int par, Acc& cur, const Acc& old, const typename Scorer::Spare& spc,
                      typename Scorer::Spare& spn, bool fin, bool red) {
        __syncthreads();
        // Scheduling fences: the compiler may not hoist the next iteration's
        // products above this barrier or sink this one's below the next,
        // which would put a reduction right behind the products it reads.
        __builtin_amdgcn_sched_barrier(0);
        // The fragment reads come first: LDS operations issue in program
        // order, so behind the record's stores and the tile store (which
        // waits for the tile's global load) they would start late.
        sc.mma_fetch_spare(f0, spc, spn, buf(par ^ 1), cur);
        if (fin) record2(it - 3);
        ld.store(buf(par));
        ld.load((uint32_t)(it + 3) * G::kTileKeys);
        if (red) reduce_into(par ^ 1, old);
        __builtin_amdgcn_sched_barrier(0);
      };
      ld.load((uint32_t)(2 * G::kTileKeys));
      __syncthreads();
      sc.fetch_spare(buf(0), f0, sp0);
      step(0, 0, acc0, acc1, sp0, sp1, false, false);
      if (ntiles == 1) {
        reduce_into(0, acc0);
        reduce_into(1, acc0);  // the pair's odd half: keys past the row, never read
        record2(0);
      } else {
        step(1, 1, acc1, acc0, sp1, sp0, false, true);
        int it = 2;
        for (; it + 1 < ntiles; it += 2) {
          step(it, 0, acc0, acc1, sp0, sp1, false, true);
          step(it + 1, 1, acc1, acc0, sp1, sp0, true, true);
        }
        if (it < ntiles) {  // an odd number of tiles: tile it is the last
          step(it, 0, acc0, acc1, sp0, sp1, false, true);
          record2(it - 2);
          reduce_into(0, acc0);
          reduce_into(1, acc0);  // (slots past the last tile, within the store)
          record2(it);
        } else {
          reduce_into(1, acc1);
          record2(it - 2);
        }
      }
    } else {
      // Filter store: the same pipeline, run from tile s until a wavefront
      // of the block asks for a cut.  Tiles are recorded two at a time, in
      // the odd step of each pair: one cross-half exchange leaves tile
      // it - 2's scores in lanes 0-31 and tile it - 1's in lanes 32-63, so
      // every lane of the record carries a key.  The cut is a call and
      // needs registers the pipeline holds, so it never runs inside the
      // loop: every wavefront sees the request after the same barrier,
      // drains (records the last two tiles), and after one more barrier
      // cuts its store if it is past half its slack, or nearly full; then
      // the pipeline restarts at the next tile, whose tile and the one
      // after it are already staged in LDS.  After the record that raises
      // a request at most two more records (128 keys) run before the cut,
      // which kCutRequest leaves room for: a store holds at most cap - 64
      // entries before any record, the room wave_append_all needs.
      // Requests rotate over three words: the even step of tile `it` reads
      // the word of the record of tiles it - 4 and it - 3 (written in the
      // previous step, before this barrier); that word is written again
      // three records later; words of a finished run are not read.  The
      // steady-state steps have no branch, so the compiler interleaves the
      // record with the tile's products.
      int s = 0;  // first tile of the current run (always even)
      // One fragment buffer, refilled with tile it + 1 as tile it's products
      // are issued (registers for the store's bookkeeping).  Even steps
      // reduce the previous (odd) tile into part_b and read the request
      // word; odd steps record the previous pair and reduce the even tile
      // into part.
      auto step = [&](int it, int par, Frag& fcur, Acc& cur, const Acc& old,
                      const typename Scorer::Spare& spc, typename Scorer::Spare& spn, bool fin,
                      bool red) -> bool {
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        uint64_t req = 0;
        if (par == 0) req = cut_req[((it >> 1) + 1) % 3];  // used at the end of the step
        if (fin) record2(it - 3);
        ld.store(buf(par));
        ld.load((uint32_t)(it + 3) * G::kTileKeys);
        sc.mma_fetch_spare(fcur, spc, spn, buf(par ^ 1), cur);
        if (red) reduce_into(par ^ 1, old);
        // Issue order: each matrix-core product followed by a few vector
        // instructions (the record, the reduction), so that a wavefront
        // whose products wait for the matrix core still has vector work
        // queued behind them rather than in one block after the last.
        // (Pinning the fragment reads into the first half as well measured
        // slower: 28.9 against 28.2 ms.)
#pragma unroll
        for (int g = 0; g < Scorer::KS * Scorer::MT * NR; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // five VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        // (uniform and with no branch: `&`, not `&&`)
        return (it >= s + 4) & (uniform((uint32_t)req | (uint32_t)(req >> 32)) != 0u);
      };
      const uint32_t cut_full = (uint32_t)(cap - kCutRequest - 32);
      bool exact = !est;  // cuts to the top k (else to an estimated rank)
      for (;;) {
        ld.load((uint32_t)(s + 2) * G::kTileKeys);
        __syncthreads();
        sc.fetch_spare(buf(0), f0, sp0);  // s is even
        // Steps go in pairs (products in acc0, then acc1), so a run always
        // ends with its last products in acc1; a pair may run one tile past
        // the last (zero keys past the range, never recorded).  The first
        // pair of a run (nothing to record yet, no request to read) is
        // peeled, so the flags of the steady-state steps are constants.
        step(s, 0, f0, acc0, acc1, sp0, sp1, false, false);
        step(s + 1, 1, f0, acc1, acc0, sp1, sp0, false, true);
        int it = s + 2;
        while (it < ntiles) {
          const bool want = step(it, 0, f0, acc0, acc1, sp0, sp1, false, true);
          step(it + 1, 1, f0, acc1, acc0, sp1, sp0, true, true);
          it += 2;
          if (want) break;
        }
        // drain: record tiles it - 2 (reduced in the last step) and it - 1
        reduce_into(1, acc1);
        record2(it - 2);
        if (it >= ntiles) {
          if (exact) break;
          // Every key the estimated cuts dropped ranks below every entry
          // kept, so a store that ends with at least k entries (or with
          // all of its row's keys) holds the row's top k.  If a row of the
          // block ended short, the block runs its keys again with exact
          // cuts.
          bool short_row = false;
#pragma unroll
          for (int rr = 0; rr < NR; ++rr)
            short_row |= count[rr] < (uint32_t)min(topk, n_t[rr]);
          if (short_row) short_rows = 1u;
          __syncthreads();  // every wavefront is past its last tile
          if (short_rows == 0u) break;
          exact = true;
#pragma unroll
          for (int rr = 0; rr < NR; ++rr) count[rr] = tau[rr] = kmax[rr] = 0u;
          ld.load(0u);
          ld.store(buf(0));
          ld.load((uint32_t)G::kTileKeys);
          ld.store(buf(1));
          s = 0;
          continue;
        }
        __syncthreads();  // every wavefront drained; tiles it and it + 1 are staged
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) {
          // a store past half its slack over the cut's rank cuts (a nearly
          // full one always does)
          const uint32_t kc = cut_rank((uint32_t)topk, (uint32_t)min(n_t[rr], it * G::kTileKeys),
                                       (uint32_t)n_t[rr], exact);
          if (count[rr] > min((kc + (uint32_t)cap) / 2u, cut_full)) {
            // after the first cut every key lies in [threshold, running max]
            const uint2 c = wave_cut(rs[rr], count[rr], kc, kc + slack_keep, tau[rr], kmax[rr]);
            count[rr] = uniform(c.x);
            tau[rr] = uniform(c.y);
          }
        }
        s = it;
      }
    }
  }
  // The final select's scratch lies in the tile buffers, which the last
  // iteration of a slower wavefront may still be writing (its store of the
  // unused tile past the end).
  __syncthreads();

#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    if (!active[rr]) continue;
    const int64_t orow = ((int64_t)b * S + t[rr]) * topk;
    if constexpr (DENSE) {
      if (sup) {  // scores at supplied indices: the row's scores gathered from its store
        for (int j = lane; j < topk; j += kWave) {
          const int sj = sup[orow + j];
          const bool ok = sj >= 0 && sj < n_t[rr];
          out_idx[orow + j] = ok ? sj : -1;
          const float x = __uint_as_float(rs[rr].key[ok ? sj : 0]);
          out_score[orow + j] = ok ? x : -__builtin_inff();
        }
      } else {
        dense_finish(rs[rr].key, (uint32_t)n_t[rr], (uint32_t)topk, smin[rr], smax[rr],
                     rs[rr].hist, rs[rr].side, topk, out_idx + orow, out_score + orow);
      }
    } else {
      wave_finish_row(rs[rr], count[rr], topk, out_idx + orow, out_score + orow);
    }
  }
}

// Two wavefronts per SIMD (two 4-wave blocks or one 8-wave block per CU):
// at most 256 registers per lane.
template <int HP, int D, int NW, int NR, bool DENSE, typename IdxT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void score_select_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    int S, int Skv, int B, int H, int ratio, int topk, int row_begin, int row_end, int R, int cap,
    int32_t* __restrict__ out_idx, float* __restrict__ out_score, int est) {
  score_select_body<HP, D, NW, NR, DENSE, IdxT>(q, k, w, S, Skv, B, H, ratio, topk, row_begin,
                                                row_end, R, cap, out_idx, out_score, nullptr,
                                                (int)blockIdx.x, est != 0);
}

// Packed sequences: the workgroup's sequence is the number of sequence
// starts at or below its index (a fixed-length scan over the table, whose
// loads the compiler batches; starts past the last sequence hold INT_MAX),
// then the one-sample problem of that sequence.
template <int HP, int D, int NW, int NR, bool DENSE, typename IdxT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void score_select_packed_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    int H, int ratio, int topk, int R, int cap, int32_t* __restrict__ out_idx,
    float* __restrict__ out_score, const PackedSeqs seqs, int est) {
  const int bid = (int)blockIdx.x;
  int i = 0;
#pragma unroll
  for (int j = 1; j < kPackedMax; ++j) i += bid >= seqs.blk_begin[j] ? 1 : 0;
  const int64_t q0 = seqs.q0[i];
  score_select_body<HP, D, NW, NR, DENSE, IdxT>(
      q + q0 * H * D, k + (int64_t)seqs.k0[i] * D, w + q0 * H, seqs.S[i], seqs.Skv[i], 1, H, ratio,
      topk, 0, seqs.S[i], R, cap, out_idx + q0 * topk, out_score + q0 * topk, nullptr,
      bid - seqs.blk_begin[i], est != 0);
}

// Scores at supplied indices through the dense store (its own kernel, so
// profiles keep it apart from the selection).  sup may alias out_idx.
template <int HP, int D, int NW, int NR>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void score_at_dense_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w,
    int S, int Skv, int B, int H, int ratio, int topk, int row_begin, int row_end, int R, int cap,
    int32_t* out_idx, float* __restrict__ out_score, const int32_t* sup) {
  score_select_body<HP, D, NW, NR, true, uint16_t>(q, k, w, S, Skv, B, H, ratio, topk, row_begin,
                                                   row_end, R, cap, out_idx, out_score, sup,
                                                   (int)blockIdx.x, false);
}

namespace {

int store_row_bytes(int cap, int idx_bytes) { return cap * 4 + ((cap * idx_bytes + 15) & ~15); }

int tile_bytes_for(int D) { return 32 * (D == 128 ? 2 * D : 2 * D + 16); }

bool plan_dense(int D, int NW, int NR, int64_t Skv, int64_t budget, ScoreSelectPlan* p) {
  const int64_t tiles = 2 * (int64_t)tile_bytes_for(D);
  const int64_t region = tiles > (int64_t)NW * kDenseScratch ? tiles : (int64_t)NW * kDenseScratch;
  const int64_t cap = Skv > 0 ? ((Skv + 255) / 256) * 256 : 256;  // whole 256-key groups
  const int64_t lds = region + (int64_t)NW * NR * cap * 4;
  if (lds > budget) return false;
  p->waves = NW;
  p->rows_per_wave = NR;
  p->rows_per_block = NW * NR;
  p->cap = (int)cap;
  p->dense = true;
  p->idx_bytes = 0;
  p->lds_bytes = (size_t)lds;
  return true;
}

bool plan_filter(int D, int NW, int NR, int topk, int64_t Skv, int64_t budget, int min_rows,
                 ScoreSelectPlan* p) {
  const int64_t tiles = 2 * (int64_t)tile_bytes_for(D);
  const int idx_bytes = Skv <= 65536 ? 2 : 4;
  const int need = topk + 16 * 32;  // slack for a cut request and a bin-edge cut's extra entries
  for (int R = NW * NR; R >= min_rows; --R) {
    const int64_t per_row = (budget - tiles - (int64_t)NW * kCutScratch) / R;
    if (per_row <= 0) continue;
    int cap = (int)(per_row / (4 + idx_bytes)) & ~63;
    while (cap > 0 && store_row_bytes(cap, idx_bytes) > per_row) cap -= 64;
    if (cap < need) continue;
    p->waves = NW;
    p->rows_per_wave = NR;
    p->rows_per_block = R;
    p->cap = cap;
    p->dense = false;
    p->idx_bytes = idx_bytes;
    p->lds_bytes = (size_t)(tiles + (int64_t)NW * kCutScratch +
                            (int64_t)R * store_row_bytes(cap, idx_bytes));
    return true;
  }
  return false;
}

}  // namespace

// Launch geometry, in order of preference (one wavefront per row):
// dense store (one slot per visible key) with four wavefronts and two blocks
// per CU, then with eight wavefronts and one block per CU; filter store (the
// top k plus at least 8 tiles of candidates) with eight wavefronts and one
// block per CU (the larger stores need half the cuts), then four, then fewer
// rows per block.
ScoreSelectPlan plan_score_select(int HP, int D, int topk, int64_t Skv, size_t lds_limit) {
  ScoreSelectPlan p{};
  const int64_t full = (int64_t)lds_limit;
  const int64_t half = full / 2;
  // the filter kernels' static LDS (cut requests) comes out of their budget
  const int64_t full_f = full - kStaticLds, half_f = half - kStaticLds;
  (void)HP;
  if (plan_dense(D, 4, 1, Skv, half, &p)) return p;
  if (plan_dense(D, 8, 1, Skv, full, &p)) return p;
  if (plan_filter(D, 8, 1, topk, Skv, full_f, 8, &p)) return p;
  if (plan_filter(D, 4, 1, topk, Skv, half_f, 4, &p)) return p;
  if (plan_filter(D, 8, 1, topk, Skv, full_f, 1, &p)) return p;
  return ScoreSelectPlan{};  // rows_per_block == 0: does not fit
}

template <int HP, int D, int NW, int NR, bool DENSE, typename IdxT>
static hipError_t launch_t(const ScoreTopkArgs& a, const ScoreSelectPlan& p, hipStream_t st,
                           hipStream_t st2) {
  const bool at = DENSE && a.sup;  // scores at supplied indices
  const void* kern = at ? (const void*)score_at_dense_kernel<HP, D, NW, NR>
                        : (const void*)score_select_kernel<HP, D, NW, NR, DENSE, IdxT>;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)p.lds_bytes);
  if (e != hipSuccess) return e;
  const int R = p.rows_per_block;
  // The selection covers every row in one launch, workgroups numbered
  // heaviest rows first: no [chunk, Skv] scores exist, so a chunk would bound
  // no memory, and one launch has no per-chunk tail.  Scores at supplied
  // indices keep one launch per chunk_rows rows.
  const int64_t chunk = (at && a.chunk_rows > 0) ? a.chunk_rows : a.S;
  int64_t ci = 0;
  for (int64_t r0 = 0; r0 < a.S; r0 += chunk, ++ci) {
    const int64_t r1 = (r0 + chunk < a.S) ? r0 + chunk : a.S;
    const int64_t blocks = ((r1 - r0 + R - 1) / R) * a.B;
    const hipStream_t sc = (st2 && (ci & 1)) ? st2 : st;
    if (at)
      hipLaunchKernelGGL((score_at_dense_kernel<HP, D, NW, NR>), dim3((unsigned)blocks),
                         dim3(NW * 64), p.lds_bytes, sc, a.q, a.k, a.w, (int)a.S, (int)a.Skv,
                         (int)a.B, a.H, a.ratio, a.topk, (int)r0, (int)r1, R, p.cap, a.out_idx,
                         a.out_score, a.sup);
    else
      hipLaunchKernelGGL((score_select_kernel<HP, D, NW, NR, DENSE, IdxT>), dim3((unsigned)blocks),
                         dim3(NW * 64), p.lds_bytes, sc, a.q, a.k, a.w, (int)a.S, (int)a.Skv,
                         (int)a.B, a.H, a.ratio, a.topk, (int)r0, (int)r1, R, p.cap, a.out_idx,
                         a.out_score, a.est_cuts ? 1 : 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int HP, int D, int NW, int NR>
static hipError_t launch_w(const ScoreTopkArgs& a, const ScoreSelectPlan& p, hipStream_t st,
                           hipStream_t st2) {
  if (p.dense) return launch_t<HP, D, NW, NR, true, uint16_t>(a, p, st, st2);
  return p.idx_bytes == 2 ? launch_t<HP, D, NW, NR, false, uint16_t>(a, p, st, st2)
                          : launch_t<HP, D, NW, NR, false, uint32_t>(a, p, st, st2);
}

template <int HP, int D>
static hipError_t launch_hd(const ScoreTopkArgs& a, const ScoreSelectPlan& p, hipStream_t st,
                            hipStream_t st2) {
  return p.waves == 4 ? launch_w<HP, D, 4, 1>(a, p, st, st2) : launch_w<HP, D, 8, 1>(a, p, st, st2);
}

template <int HP, int D, int NW, int NR, bool DENSE, typename IdxT>
static hipError_t launch_packed_t(const PackedTopkArgs& a, const PackedSeqs& seqs,
                                  const ScoreSelectPlan& p, hipStream_t st) {
  const void* kern = (const void*)score_select_packed_kernel<HP, D, NW, NR, DENSE, IdxT>;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)p.lds_bytes);
  if (e != hipSuccess) return e;
  const int blocks = seqs.blk_begin[seqs.n];
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((score_select_packed_kernel<HP, D, NW, NR, DENSE, IdxT>), dim3((unsigned)blocks),
                     dim3(NW * 64), p.lds_bytes, st, a.q, a.k, a.w, a.H, a.ratio, a.topk,
                     p.rows_per_block, p.cap, a.out_idx, a.out_score, seqs, a.est_cuts ? 1 : 0);
  return hipGetLastError();
}

template <int HP, int D, int NW>
static hipError_t launch_packed_w(const PackedTopkArgs& a, const PackedSeqs& seqs,
                                  const ScoreSelectPlan& p, hipStream_t st) {
  if (p.dense) return launch_packed_t<HP, D, NW, 1, true, uint16_t>(a, seqs, p, st);
  return p.idx_bytes == 2 ? launch_packed_t<HP, D, NW, 1, false, uint16_t>(a, seqs, p, st)
                          : launch_packed_t<HP, D, NW, 1, false, uint32_t>(a, seqs, p, st);
}

hipError_t launch_score_topk_packed(const PackedTopkArgs& a, const PackedSeqs& seqs,
                                    const ScoreSelectPlan& p, hipStream_t st) {
  const int HP = a.H <= 32 ? 32 : 64;
#define DSAI_CASE(hp, d)                                                        \
  if (HP == hp && a.D == d)                                                     \
    return p.waves == 4 ? launch_packed_w<hp, d, 4>(a, seqs, p, st)             \
                        : launch_packed_w<hp, d, 8>(a, seqs, p, st);
  DSAI_CASE(32, 32) DSAI_CASE(32, 64) DSAI_CASE(32, 128)
  DSAI_CASE(64, 32) DSAI_CASE(64, 64) DSAI_CASE(64, 128)
#undef DSAI_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_score_topk(const ScoreTopkArgs& a, const ScoreSelectPlan& p, hipStream_t st,
                             hipStream_t st2) {
  const int HP = a.H <= 32 ? 32 : 64;
#define DSAI_CASE(hp, d) \
  if (HP == hp && a.D == d) return launch_hd<hp, d>(a, p, st, st2);
  DSAI_CASE(32, 32) DSAI_CASE(32, 64) DSAI_CASE(32, 128)
  DSAI_CASE(64, 32) DSAI_CASE(64, 64) DSAI_CASE(64, 128)
#undef DSAI_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsai
