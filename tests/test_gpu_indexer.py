"""GPU parity of the fused score + mask + top-k kernel against the CPU oracle.

Every case runs the HIP path through the C ABI (Python binding) on seeded
synthetic inputs and compares with the fp64 oracle under the rules in
tests/parity.py; integer-valued cases (exact in fp32) must match bit for
bit, ties and order included.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as SY
from parity import check_topk_rows, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsai():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import sparse_attention_token_index_amd as m
    m.load_library()
    return m


def to_gpu_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def run_gpu(dsai, case, inp, chunk_rows=None, out=None, cuts=0):
    ix = dsai.Indexer(heads=case.H, dim=case.D,
                      chunk_rows=case.chunk_rows if chunk_rows is None else chunk_rows, cuts=cuts)
    q = to_gpu_bf16(inp["q_bits"])
    k = to_gpu_bf16(inp["k_bits"])
    w = torch.from_numpy(inp["w"]).cuda()
    oi, os_ = (None, None) if out is None else out
    idx, sc = ix.score_topk(q, k, w, case.compress_ratio, case.topk, out_idx=oi, out_score=os_)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def oracle_rows(case, rows, q_bits_rows, k_bits, w_rows):
    q = SY.bf16_bits_to_f32(q_bits_rows).astype(np.float64)
    k = SY.bf16_bits_to_f32(k_bits).astype(np.float64)
    return oracle.score_topk(q, k, w_rows.astype(np.float64), case.compress_ratio, case.topk,
                             rows=rows, row_values=True)


def compare(case, gidx, gsc, rows, full):
    labels, gi, gs = [], [], []
    for b in range(case.B):
        for t in rows:
            labels.append(f"{case.name} b={b} t={t}")
            gi.append(gidx[b, t])
            gs.append(gsc[b, t])
    check_topk_rows(np.array(gi), np.array(gs), full, case.topk, labels)


MEDIUM = [
    SY.IndexerCase("h64d128_r1_k100", B=2, S=700, Skv=700, H=64, D=128, compress_ratio=1,
                   topk=100, w_var=1 / 64, seed=11),
    SY.IndexerCase("h32d64_r3_k64", B=1, S=1000, Skv=300, H=32, D=64, compress_ratio=3,
                   topk=64, w_var=1 / 32, seed=12),
    SY.IndexerCase("h4d32_r1_k16_compactions", B=1, S=1500, Skv=1500, H=4, D=32,
                   compress_ratio=1, topk=16, w_var=1 / 4, seed=13),
    SY.IndexerCase("h64d128_k2048_sortall", B=1, S=2300, Skv=2300, H=64, D=128,
                   compress_ratio=1, topk=2048, w_var=1 / 64, seed=14),
    SY.IndexerCase("h20d128_r4_pad_heads", B=3, S=900, Skv=200, H=20, D=128, compress_ratio=4,
                   topk=37, w_var=1 / 20, seed=15),
    SY.IndexerCase("topk_gt_skv", B=1, S=130, Skv=100, H=64, D=128, compress_ratio=1,
                   topk=200, w_var=1 / 64, seed=16),
    SY.IndexerCase("h64d32_k1", B=1, S=333, Skv=333, H=64, D=32, compress_ratio=1, topk=1,
                   w_var=1 / 64, seed=17),
    SY.IndexerCase("h16d64_r2_k300", B=2, S=777, Skv=500, H=16, D=64, compress_ratio=2,
                   topk=300, w_var=1 / 16, seed=18),
    SY.IndexerCase("h64d128_k4096", B=1, S=4200, Skv=4200, H=64, D=128, compress_ratio=1,
                   topk=4096, w_var=1 / 64, seed=19),
    # more keys than a dense row store holds: the filtering store with compactions
    SY.IndexerCase("filter_h32d64_k64", B=1, S=5000, Skv=5000, H=32, D=64, compress_ratio=1,
                   topk=64, w_var=1 / 32, seed=24),
    SY.IndexerCase("filter_h64d128_k2048", B=1, S=6000, Skv=6000, H=64, D=128,
                   compress_ratio=1, topk=2048, w_var=1 / 64, seed=25),
    SY.IndexerCase("filter_b2_r2_k300", B=2, S=9000, Skv=4500, H=16, D=128, compress_ratio=2,
                   topk=300, w_var=1 / 16, seed=26),
]


@pytest.mark.parametrize("case", MEDIUM, ids=[c.name for c in MEDIUM])
def test_medium_parity(dsai, case):
    log(f"[gpu] medium parity {case}")
    inp = SY.indexer_inputs(case)
    gidx, gsc = run_gpu(dsai, case, inp)
    rows = list(range(case.S))
    if case.S * case.B > 1500:  # keep the oracle to seconds: every row near the ends, a sample inside
        rng = np.random.default_rng(case.seed)
        rows = sorted(set(range(0, 40)) | set(range(case.S - 40, case.S)) |
                      set(rng.choice(case.S, 300, replace=False).tolist()))
    _, _, full = oracle_rows(case, rows, inp["q_bits"][rows], inp["k_bits"], inp["w"][rows])
    compare(case, gidx, gsc, rows, full)


INTEGER = [
    SY.IndexerCase("int_h64d128_r1", B=1, S=600, Skv=600, H=64, D=128, compress_ratio=1,
                   topk=50, w_var=0, integer=True, seed=21),
    SY.IndexerCase("int_h4d32_r2", B=2, S=400, Skv=300, H=4, D=32, compress_ratio=2, topk=40,
                   w_var=0, integer=True, seed=22),
    SY.IndexerCase("int_h32d128_k700", B=1, S=900, Skv=900, H=32, D=128, compress_ratio=1,
                   topk=700, w_var=0, integer=True, seed=23),
]


@pytest.mark.parametrize("case", INTEGER, ids=[c.name for c in INTEGER])
def test_integer_inputs_bit_exact(dsai, case):
    """Small-integer q, k and power-of-two weights: every fp32 step on the GPU
    is exact, so indices, order, ties and scores must equal the oracle's."""
    log(f"[gpu] integer bit-exact {case}")
    inp = SY.indexer_inputs(case)
    gidx, gsc = run_gpu(dsai, case, inp)
    oidx, ovals, _ = oracle_rows(case, list(range(case.S)), inp["q_bits"], inp["k_bits"], inp["w"])
    assert np.array_equal(gidx, oidx), np.argwhere(gidx != oidx)[:10]
    assert np.array_equal(gsc.astype(np.float64), ovals)   # -0.0 == +0.0


def _tie_inputs(case, lo, hi, w_zero=False):
    """Integer q, k drawn from [lo, hi] and weights from {+-1, +-1/2, +-1/4}
    (or all zero): every fp32 step of the GPU is exact, and the narrow range
    makes equal scores frequent."""
    rng = np.random.default_rng(case.seed + 500)
    q = rng.integers(lo, hi + 1, (case.S, case.B, case.H, case.D)).astype(np.float32)
    k = rng.integers(lo, hi + 1, (case.Skv, case.B, case.D)).astype(np.float32)
    w = (rng.choice([-1.0, -0.5, -0.25, 0.25, 0.5, 1.0], (case.S, case.B, case.H))
         .astype(np.float32))
    if w_zero:
        w[:] = 0.0
    return {"q_bits": SY.f32_to_bf16_bits(q), "k_bits": SY.f32_to_bf16_bits(k), "w": w}


def _exact_rows(case, gidx, gsc, inp, rows):
    oidx, ovals, _ = oracle_rows(case, rows, inp["q_bits"][rows], inp["k_bits"], inp["w"][rows])
    for b in range(case.B):
        g_i, g_s = gidx[b, rows], gsc[b, rows]
        bad = np.argwhere(g_i != oidx[b])
        assert bad.size == 0, f"b={b}: first differing (row, slot) {[(rows[r], c) for r, c in bad[:5]]}"
        assert np.array_equal(g_s.astype(np.float64), ovals[b])   # -0.0 == +0.0
        assert not np.any(g_s.view(np.uint32) == 0x80000000)       # the GPU writes +0


FILTER_TIES = [
    # rows longer than any dense store (D = 128: more than 4608 keys), topk =
    # 2048, integer inputs in [-4, 4]: the filter store fills and cuts
    # several times; 16-bit stored indices
    (SY.IndexerCase("filter_int_h64d128_k2048", B=1, S=6000, Skv=6000, H=64, D=128,
                    compress_ratio=1, topk=2048, w_var=0, seed=61), -4, 4, False),
    # the same with q, k in [-1, 1]: scores on a coarse grid, heavy ties at
    # the k-th value on every cut
    (SY.IndexerCase("filter_ties_h64d128_k2048", B=1, S=6000, Skv=6000, H=64, D=128,
                    compress_ratio=1, topk=2048, w_var=0, seed=62), -1, 1, False),
    # every score is zero: each cut keeps the lowest indices
    (SY.IndexerCase("filter_zero_h64d128_k2048", B=1, S=6000, Skv=6000, H=64, D=128,
                    compress_ratio=1, topk=2048, w_var=0, seed=63), -4, 4, True),
    # more than 65536 keys: 32-bit stored indices (H = 4, D = 32)
    (SY.IndexerCase("filter_ties_wide_h4d32_k1024", B=1, S=70000, Skv=70000, H=4, D=32,
                    compress_ratio=1, topk=1024, w_var=0, seed=64), -1, 1, False),
]


@pytest.mark.parametrize("case,lo,hi,w_zero", FILTER_TIES, ids=[c[0].name for c in FILTER_TIES])
def test_filter_store_ties_bit_exact(dsai, case, lo, hi, w_zero):
    """Exact-arithmetic inputs on rows long enough for the filtering store:
    indices, their order, scores and +-0 equal the oracle's bit for bit on
    every sampled row (ends, the rows where n_t crosses topk, every 13th
    row), so the lower-index-wins rule is pinned across repeated cuts, in
    score order and in index order."""
    log(f"[gpu] filter-store ties {case.name}")
    inp = _tie_inputs(case, lo, hi, w_zero)
    k = case.topk
    rows = sorted(set(range(0, 8)) | set(range(k - 4, k + 4)) | set(range(case.S - 8, case.S)) |
                  set(range(0, case.S, 13 if case.S < 10000 else 1750)) |
                  ({65534, 65535, 65536, 65537} if case.S > 65536 else set()))
    gidx, gsc = run_gpu(dsai, case, inp)
    if w_zero:   # closed form: the lowest min(topk, n_t) indices, score +0
        for t in rows:
            m = min(k, t + 1)
            assert gidx[0, t, :m].tolist() == list(range(m)), t
            assert np.all(gsc[0, t, :m].view(np.uint32) == 0)
    _exact_rows(case, gidx, gsc, inp, rows)
    # index order: the same set, ascending
    ix = dsai.Indexer(heads=case.H, dim=case.D, order=dsai.DSAI_ORDER_INDEX)
    ii, isc = ix.score_topk(to_gpu_bf16(inp["q_bits"]), to_gpu_bf16(inp["k_bits"]),
                            torch.from_numpy(inp["w"]).cuda(), case.compress_ratio, k)
    torch.cuda.synchronize()
    ii, isc = ii.cpu().numpy(), isc.cpu().numpy()
    for t in rows:
        m = int((gidx[0, t] >= 0).sum())
        order = np.argsort(gidx[0, t, :m], kind="stable")
        assert np.array_equal(ii[0, t, :m], gidx[0, t, :m][order]), t
        assert np.array_equal(isc[0, t, :m].view(np.uint32), gsc[0, t, :m][order].view(np.uint32)), t


def test_chunked_launches_match_single_launch(dsai):
    case = MEDIUM[0]
    log("[gpu] chunking")
    inp = SY.indexer_inputs(case)
    a = run_gpu(dsai, case, inp, chunk_rows=0)
    b = run_gpu(dsai, case, inp, chunk_rows=64)
    c = run_gpu(dsai, case, inp, chunk_rows=1)
    for x in (b, c):
        assert np.array_equal(a[0], x[0])
        assert np.array_equal(a[1].view(np.uint32), x[1].view(np.uint32))


def test_chunk_streams_join_the_callers_stream(dsai):
    """Scores at supplied indices in chunks run on the handle's two streams:
    work the caller enqueues on its own stream right after the call (no host
    sync) must see every chunk's output.  The selection (one launch whatever
    chunk_rows is) on the same non-default caller stream too."""
    case = MEDIUM[0]
    inp = SY.indexer_inputs(case)
    q, k = to_gpu_bf16(inp["q_bits"]), to_gpu_bf16(inp["k_bits"])
    w = torch.from_numpy(inp["w"]).cuda()
    ref = run_gpu(dsai, case, inp, chunk_rows=0)
    sup = torch.from_numpy(ref[0]).cuda()
    ix = dsai.Indexer(heads=case.H, dim=case.D, chunk_rows=50)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    shape = (case.B, case.S, case.topk)
    with torch.cuda.stream(side):
        for _ in range(3):   # the same outputs rewritten, each read right after
            oi = torch.full(shape, -7, dtype=torch.int32, device="cuda")
            os_ = torch.zeros(shape, dtype=torch.float32, device="cuda")
            ix.score_topk(q, k, w, case.compress_ratio, case.topk, out_idx=oi, out_score=os_)
            ci, cs = oi.clone(), os_.clone()   # enqueued on `side` after the call
            ai = torch.full(shape, -7, dtype=torch.int32, device="cuda")
            as_ = torch.zeros(shape, dtype=torch.float32, device="cuda")
            ix.score_topk(q, k, w, case.compress_ratio, case.topk, topk_indices=sup, out_idx=ai,
                          out_score=as_)
            di, ds = ai.clone(), as_.clone()
    torch.cuda.synchronize()
    assert np.array_equal(ci.cpu().numpy(), ref[0])
    assert np.array_equal(cs.cpu().numpy().view(np.uint32), ref[1].view(np.uint32))
    # the selection's own entries rescored: the same indices and score bits
    assert np.array_equal(di.cpu().numpy(), ref[0])
    assert np.array_equal(ds.cpu().numpy().view(np.uint32), ref[1].view(np.uint32))


def test_deterministic_and_every_slot_written(dsai):
    case = MEDIUM[3]
    log("[gpu] determinism + sentinel")
    inp = SY.indexer_inputs(case)
    shape = (case.B, case.S, case.topk)
    oi = torch.full(shape, -12345, dtype=torch.int32, device="cuda")
    os_ = torch.full(shape, 0, dtype=torch.int32, device="cuda").fill_(0x7FBFFFFF).view(torch.float32)
    a = run_gpu(dsai, case, inp, out=(oi, os_))
    assert not np.any(a[0] == -12345)
    assert not np.any(a[1].view(np.uint32) == 0x7FBFFFFF)
    b = run_gpu(dsai, case, inp)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


REPEAT_CASES = [
    # two 4-wave blocks per CU; odd and even tile counts per block
    SY.IndexerCase("c4_like_repeat", B=2, S=4096, Skv=1024, H=64, D=128, compress_ratio=4,
                   topk=512, w_var=1 / 64, seed=21),
    # one 8-wave block per CU (the dense store needs the whole LDS)
    SY.IndexerCase("wide_dense_repeat", B=1, S=4500, Skv=4500, H=64, D=128, compress_ratio=1,
                   topk=2048, w_var=1 / 64, seed=22),
]


@pytest.mark.parametrize("case", REPEAT_CASES, ids=lambda c: c.name)
def test_repeated_launches_bit_identical(dsai, case):
    """Back-to-back launches on the same inputs give identical bits (guards the
    hand-over of the tile buffers to the final select between wavefronts),
    and sampled rows keep parity with the oracle."""
    log(f"[gpu] repeated launches {case.name}")
    inp = SY.indexer_inputs(case)
    first = run_gpu(dsai, case, inp)
    for rep in range(4):
        again = run_gpu(dsai, case, inp)
        assert np.array_equal(first[0], again[0]), f"launch {rep + 1}: indices differ"
        assert np.array_equal(first[1].view(np.uint32), again[1].view(np.uint32))
    rows = sorted({0, case.S - 1, case.S // 2, case.S // 3, 2049, 4100} & set(range(case.S)))
    _, _, full = oracle_rows(case, rows, inp["q_bits"][rows], inp["k_bits"], inp["w"][rows])
    compare(case, first[0], first[1], rows, full)


def test_empty_and_degenerate_shapes(dsai):
    log("[gpu] degenerate shapes")
    ix = dsai.Indexer(heads=64, dim=128)
    dev = "cuda"
    # S == 0: nothing to do
    idx, sc = ix.score_topk(torch.zeros(0, 1, 64, 128, dtype=torch.bfloat16, device=dev),
                            torch.zeros(5, 1, 128, dtype=torch.bfloat16, device=dev),
                            torch.zeros(0, 1, 64, device=dev), 1, 8)
    assert idx.shape == (1, 0, 8)
    # Skv == 0: every row padded
    idx, sc = ix.score_topk(torch.ones(7, 2, 64, 128, dtype=torch.bfloat16, device=dev),
                            torch.zeros(0, 2, 128, dtype=torch.bfloat16, device=dev),
                            torch.ones(7, 2, 64, device=dev), 1, 5)
    torch.cuda.synchronize()
    assert (idx == -1).all() and torch.isneginf(sc).all()
    # rows t < r - 1 see nothing; r larger than S: every row empty
    case = SY.IndexerCase("r_large", B=1, S=20, Skv=20, H=64, D=128, compress_ratio=64, topk=4,
                          w_var=1 / 64, seed=30)
    gidx, gsc = run_gpu(dsai, case, SY.indexer_inputs(case))
    assert (gidx == -1).all() and np.isneginf(gsc).all()
    # all-zero queries: every visible score is 0 -> ties resolve to the lowest indices
    case = SY.IndexerCase("zeros", B=1, S=300, Skv=300, H=64, D=128, compress_ratio=1, topk=10,
                          w_var=1 / 64, seed=31)
    inp = SY.indexer_inputs(case)
    inp["q_bits"] = np.zeros_like(inp["q_bits"])
    gidx, gsc = run_gpu(dsai, case, inp)
    for t in range(case.S):
        m = min(10, t + 1)
        assert gidx[0, t, :m].tolist() == list(range(m)), t
        assert np.all(gsc[0, t, :m] == 0.0)


@pytest.mark.parametrize("heads,dim", [(64, 128), (20, 64)])
def test_filter_store_block_cuts(dsai, heads, dim):
    """Rows longer than any dense store (Skv = 6000 keys at D = 128) with
    topk = 2048: the filter store fills and every block cuts its rows
    together several times.  Sampled rows keep parity with the oracle, and a
    second launch gives the same bits (the cut requests pass between
    wavefronts through LDS)."""
    case = SY.IndexerCase(f"filter_cuts_h{heads}d{dim}", B=1, S=6000, Skv=6000, H=heads, D=dim,
                          compress_ratio=1, topk=2048, w_var=1 / heads, seed=41)
    log(f"[gpu] filter-store cuts {case.name}")
    inp = SY.indexer_inputs(case)
    first = run_gpu(dsai, case, inp)
    again = run_gpu(dsai, case, inp)
    assert np.array_equal(first[0], again[0])
    assert np.array_equal(first[1].view(np.uint32), again[1].view(np.uint32))
    rows = [0, 2047, 2048, 3001, 4799, 5998, 5999]
    _, _, full = oracle_rows(case, rows, inp["q_bits"][rows], inp["k_bits"], inp["w"][rows])
    compare(case, first[0], first[1], rows, full)


def _trend_inputs(case, falling):
    """Integer inputs whose scores follow the key position: key s is the
    trend (Skv - 1 - s) // 64 (falling) or s // 64 (rising) plus a random
    0..7, in every dimension plus a random 0 or 1; q in 0..2 and weights in
    {1/4, 1/2, 1}, all non-negative, so the score rises with the key's
    value.  Every fp32 step is exact (dot products below 2^14)."""
    rng = np.random.default_rng(case.seed + 700)
    s = np.arange(case.Skv)
    trend = (case.Skv - 1 - s) // 64 if falling else s // 64
    c = trend + rng.integers(0, 8, case.Skv)
    k = (c[:, None, None] + rng.integers(0, 2, (case.Skv, case.B, case.D))).astype(np.float32)
    q = rng.integers(0, 3, (case.S, case.B, case.H, case.D)).astype(np.float32)
    w = rng.choice([0.25, 0.5, 1.0], (case.S, case.B, case.H)).astype(np.float32)
    assert k.max() <= 256   # integers exact in bf16
    return {"q_bits": SY.f32_to_bf16_bits(q), "k_bits": SY.f32_to_bf16_bits(k), "w": w}


@pytest.mark.parametrize("trend", ["falling", "rising", "random"])
def test_filter_store_estimated_cuts(dsai, trend):
    """Rows longer than the dense store, cut to an estimated rank (the
    default) or to k: the same bits either way.  With scores that fall
    along the key sequence the estimated cuts drop part of the top k, the
    rows end short and their blocks run again with cuts to k; rising scores
    never do; random (Gaussian) inputs are the common case.  The integer
    cases also match the oracle bit for bit on sampled rows."""
    case = SY.IndexerCase(f"est_cuts_{trend}", B=1, S=8192, Skv=8192, H=4, D=32,
                          compress_ratio=1, topk=2048, w_var=1 / 4, seed=71)
    log(f"[gpu] estimated cuts, {trend} scores {case}")
    inp = SY.indexer_inputs(case) if trend == "random" else _trend_inputs(case, trend == "falling")
    q, k = to_gpu_bf16(inp["q_bits"]), to_gpu_bf16(inp["k_bits"])
    w = torch.from_numpy(inp["w"]).cuda()
    outs = []
    for cuts in (dsai.DSAI_CUTS_ESTIMATED, dsai.DSAI_CUTS_TOPK):
        ix = dsai.Indexer(heads=case.H, dim=case.D, cuts=cuts)
        idx, sc = ix.score_topk(q, k, w, 1, case.topk)
        torch.cuda.synchronize()
        outs.append((idx.cpu().numpy(), sc.cpu().numpy()))
    (ei, es), (ti, ts) = outs
    assert np.array_equal(ei, ti), np.argwhere(ei != ti)[:5]
    assert np.array_equal(es.view(np.uint32), ts.view(np.uint32))
    rows = sorted(set(range(0, 4)) | set(range(2044, 2052)) | set(range(0, case.S, 97)) |
                  set(range(case.S - 4, case.S)))
    if trend == "random":
        _, _, full = oracle_rows(case, rows, inp["q_bits"][rows], inp["k_bits"], inp["w"][rows])
        compare(case, ei, es, rows, full)
    else:
        _exact_rows(case, ei, es, inp, rows)


def test_filter_store_wide_indices(dsai):
    """Skv > 65536: the filtering store keeps 32-bit indices."""
    case = SY.IndexerCase("wide_idx", B=1, S=70000, Skv=70000, H=4, D=32, compress_ratio=1,
                          topk=16, w_var=1 / 4, seed=27)
    log(f"[gpu] wide indices {case}")
    inp = SY.indexer_inputs(case)
    gidx, gsc = run_gpu(dsai, case, inp)
    rows = [0, 15, 16, 65535, 65536, 65537, 69999] + list(range(1000, 70000, 7000))
    _, _, full = oracle_rows(case, rows, inp["q_bits"][rows], inp["k_bits"], inp["w"][rows])
    compare(case, gidx, gsc, rows, full)


def _sample_rows(case, extra=24, seed=0):
    rng = np.random.default_rng(seed + 1000)
    r, S, k = case.compress_ratio, case.S, case.topk
    cross = r * (k + 1) - 1   # first row with more than topk visible keys
    rows = {0, 1, 2, 3, r - 1, r, S - 1, S - 2, S // 2,
            max(0, cross - 1), min(S - 1, cross), min(S - 1, cross + 1)}
    rows |= set(rng.choice(S, extra, replace=False).tolist())
    return sorted(t for t in rows if 0 <= t < S)


@pytest.mark.parametrize("name", ["tiny", "prefill", "c4", "long"])
def test_config_parity(dsai, name):
    """The workloads at their full sizes, in the bench's launch configuration;
    the oracle checks all rows of the tiny case and sampled rows of the rest."""
    case = SY.CASES[name]
    log(f"[gpu] config parity {name}: generating inputs")
    inp = SY.indexer_inputs(case)
    log(f"[gpu] config parity {name}: running")
    gidx, gsc = run_gpu(dsai, case, inp)
    if name == "tiny":
        rows = list(range(case.S))
    elif name == "long":   # every 64th row as well
        rows = sorted(set(_sample_rows(case)) | set(range(0, case.S, 64)))
    else:
        rows = _sample_rows(case)
    if name == "long":   # estimated cuts (the default) and cuts to k: the same bits
        log(f"[gpu] config parity {name}: cuts to k")
        tidx, tsc = run_gpu(dsai, case, inp, cuts=dsai.DSAI_CUTS_TOPK)
        assert np.array_equal(tidx, gidx)
        assert np.array_equal(tsc.view(np.uint32), gsc.view(np.uint32))
        del tidx, tsc
    log(f"[gpu] config parity {name}: oracle on {len(rows)} rows x {case.B} batches")
    _, _, full = oracle_rows(case, rows, inp["q_bits"][rows], inp["k_bits"], inp["w"][rows])
    compare(case, gidx, gsc, rows, full)
    # properties that hold for every row: padding exactly where the row is short
    for b in range(case.B):
        n = np.minimum(case.Skv, (np.arange(case.S) + 1) // case.compress_ratio)
        npad = (gidx[b] == -1).sum(axis=1)
        assert np.array_equal(npad, np.maximum(0, case.topk - n))
        assert np.all(gidx[b] < n[:, None])


@pytest.mark.parametrize("case", [MEDIUM[0], MEDIUM[2], MEDIUM[3], MEDIUM[8]],
                         ids=lambda c: c.name)
def test_index_order_mode_and_row_sort(dsai, case):
    """order=DSAI_ORDER_INDEX returns the same top-k set in ascending index
    order; sorting it on the host by (score desc, index asc) must give the
    score-ordered output bit for bit (pins the row-sort kernel)."""
    log(f"[gpu] index-order mode {case.name}")
    inp = SY.indexer_inputs(case)
    q, k = to_gpu_bf16(inp["q_bits"]), to_gpu_bf16(inp["k_bits"])
    w = torch.from_numpy(inp["w"]).cuda()
    out = {}
    for order in (dsai.DSAI_ORDER_SCORE, dsai.DSAI_ORDER_INDEX):
        ix = dsai.Indexer(heads=case.H, dim=case.D, order=order)
        i, s = ix.score_topk(q, k, w, case.compress_ratio, case.topk)
        torch.cuda.synchronize()
        out[order] = (i.cpu().numpy(), s.cpu().numpy())
    si, ss = out[dsai.DSAI_ORDER_SCORE]
    ii, isc = out[dsai.DSAI_ORDER_INDEX]
    for b in range(case.B):
        for t in range(case.S):
            m = int((ii[b, t] >= 0).sum())
            assert np.all(ii[b, t, m:] == -1) and np.all(np.isneginf(isc[b, t, m:]))
            assert np.all(np.diff(ii[b, t, :m]) > 0), (b, t)
            order = np.lexsort((ii[b, t, :m], -isc[b, t, :m].astype(np.float64)))
            assert np.array_equal(ii[b, t, :m][order], si[b, t, :m]), (b, t)
            assert np.array_equal(isc[b, t, :m][order].view(np.uint32), ss[b, t, :m].view(np.uint32))
