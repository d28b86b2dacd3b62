"""GPU parity of the pooled decode path (kpool_compress, index_scores,
topk_pools, select, expand) against the CPU oracle.

Integer outputs (pool_tok, pool_valid, pool ids from exact fp32 inputs,
expanded token ids) must match bit for bit.  pool_k must match bit for bit
except where the oracle's fp64 value x lies within E = 2^-18 * max_j |k_j|
of a bf16 rounding midpoint (k_j the pool's slot keys in that channel); there
the GPU value may differ from x by at most E + one bf16 ulp of x.  The GPU
evaluates the softmax-weighted sum in fp32; its error is bounded by a few
fp32 ulps of the summands' magnitude (not of the result, which cancellation
between slots of opposite sign can make arbitrarily small), about
(KP + 2) * 2^-24 * max_j |k_j| <= E: only values that close to a midpoint
can round differently, and for a tiny (cancelled) result that error can span
several bf16 ulps of the result itself.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as SY
from parity import check_topk_rows, log, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsai():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import sparse_attention_token_index_amd as m
    m.load_library()
    return m


def bf16_gpu(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bits_of(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def f64(bits):
    return SY.bf16_bits_to_f32(bits).astype(np.float64)


def slot_magnitude(kn_f64, N, first_key, KP):
    """[P, D]: max_j |k_normed[tok_j, c]| over each pool's slots."""
    P = oracle.pool_count(N, first_key, KP)
    toks = first_key + np.arange(P)[:, None] * KP + np.arange(KP)[None, :]
    return np.abs(kn_f64[toks]).max(axis=1)


def check_pool_k(gpu_bits, oracle_f64, magnitude):
    _, ob = oracle.round_to_bf16(oracle_f64)
    diff = gpu_bits != ob
    if not np.any(diff):
        return
    x = oracle_f64[diff]
    _, e = np.frexp(x)
    ulp = np.ldexp(1.0, e - 8)
    mid = np.floor(x / ulp) * ulp + ulp / 2          # the midpoint between x's neighbours
    err = magnitude[diff] * 2.0 ** -18              # bound on the fp32 evaluation error
    near_mid = np.abs(x - mid) <= err
    g = f64(gpu_bits[diff])
    within = np.abs(g - x) <= err + ulp
    ok = near_mid & within
    assert np.all(ok), f"{int(np.sum(~ok))} pool_k elements differ away from a rounding midpoint"


def pooled_case_inputs(case):
    inp = SY.pooled_inputs(case)
    return inp


POOL_CASES = [
    SY.POOLED_CASES["pooled_decode"],
    SY.PooledCase("kp1_fk5_d64", N=3001, D=64, KP=1, first_key=5, H=16, Q=7, index_topk=40),
    SY.PooledCase("kp3_fk2_d32_h4", N=2000, D=32, KP=3, first_key=2, H=4, Q=9, index_topk=30),
    SY.PooledCase("kp8_d128_h64", N=5000, D=128, KP=8, first_key=0, H=64, Q=5, index_topk=64,
                  valid_p=0.999),
    SY.PooledCase("kp2_fk1_tail", N=1001, D=128, KP=2, first_key=1, H=32, Q=3, index_topk=2000,
                  valid_p=0.7, invalid_tail=100),   # select_k > valid pools: -1 padding
    SY.PooledCase("kp5_d64_h20", N=4099, D=64, KP=5, first_key=7, H=20, Q=66, index_topk=55),
]


@pytest.mark.parametrize("case", POOL_CASES, ids=[c.name for c in POOL_CASES])
def test_kpool_compress(dsai, case):
    log(f"[gpu] kpool {case}")
    inp = pooled_case_inputs(case)
    ix = dsai.Indexer(heads=case.H, dim=case.D, kpool=case.KP, index_topk=case.index_topk,
                      first_key=case.first_key)
    pk, pt, pv = ix.kpool_compress(bf16_gpu(inp["k_normed_bits"]), torch.from_numpy(inp["gate"]).cuda(),
                                   torch.from_numpy(inp["valid"]).cuda(),
                                   torch.from_numpy(inp["ape"]).cuda())
    torch.cuda.synchronize()
    ref = oracle.kpool_compress(f64(inp["k_normed_bits"]), inp["gate"], inp["valid"], inp["ape"],
                                case.first_key, case.KP)
    assert pk.shape[0] == ref["pool_k"].shape[0] == oracle.pool_count(case.N, case.first_key, case.KP)
    assert np.array_equal(pt.cpu().numpy(), ref["pool_tok"])
    assert np.array_equal(pv.cpu().numpy(), ref["pool_valid"])
    check_pool_k(bits_of(pk), ref["pool_k_f64"],
                 slot_magnitude(f64(inp["k_normed_bits"]), case.N, case.first_key, case.KP))


@pytest.mark.parametrize("case", POOL_CASES, ids=[c.name for c in POOL_CASES])
def test_index_scores_elementwise(dsai, case):
    """Stage-isolated: the GPU scores the oracle's own pool keys."""
    log(f"[gpu] index_scores {case}")
    inp = pooled_case_inputs(case)
    ref = oracle.kpool_compress(f64(inp["k_normed_bits"]), inp["gate"], inp["valid"], inp["ape"],
                                case.first_key, case.KP)
    ix = dsai.Indexer(heads=case.H, dim=case.D, kpool=case.KP, index_topk=case.index_topk,
                      first_key=case.first_key)
    sc = ix.index_scores(bf16_gpu(inp["q_bits"]), torch.from_numpy(inp["w"]).cuda(),
                         bf16_gpu(ref["pool_k_bits"]), torch.from_numpy(ref["pool_valid"]).cuda())
    torch.cuda.synchronize()
    g = sc.cpu().numpy().astype(np.float64)
    o = oracle.pooled_index_scores(f64(inp["q_bits"]), inp["w"], ref["pool_k"], ref["pool_valid"])
    inv = ~np.isfinite(o)
    assert np.array_equal(np.isneginf(g), inv)
    assert np.all(np.abs(g[~inv] - o[~inv]) <= tol(o[~inv]))


@pytest.mark.parametrize("Q,P,KP,index_topk", [
    (70, 16384, 4, 512),      # block select, ranked in LDS
    (9, 16384, 4, 4096),      # block select, then the row sort (select_k > 512)
    (6, 40000, 4, 512),       # more pools than one workgroup holds: streaming select
    (12, 1000, 1, 64),        # one pool per thread
    (5, 5001, 2, 64),         # rows not 16-byte aligned: scalar loads
    (4, 3, 1, 2),             # tiny rows
])
@pytest.mark.parametrize("order", ["score", "index"])
def test_topk_pools_exact_on_fp32_scores(dsai, Q, P, KP, index_topk, order):
    """topk_pools selects on the fp32 values it is given: with the oracle run on
    the same fp32 values, ids, order and scores must match exactly (index
    order: the oracle's selection sorted by pool id)."""
    log(f"[gpu] topk_pools exact Q={Q} P={P} KP={KP} index_topk={index_topk} order={order}")
    rng = np.random.default_rng(41 + P)
    s = rng.standard_normal((Q, P)).astype(np.float32)
    s[rng.random((Q, P)) < 0.08] = -np.inf                   # invalid candidates
    if Q > 4:
        s[1:3] = np.round(s[1:3] * 2).astype(np.float32)      # many exact ties
        s[3, :] = 0.0                                         # one big tie
        s[4, :] = -np.inf                                     # no valid pool
    if Q > 8:
        s[5, :] = -np.inf
        s[5, [0, P // 2, P - 1]] = [1.0, 2.0, 1.0]            # fewer valid than select_k
        s[6] = -np.abs(s[6])                                  # all negative
        s[7, ::2] = -0.0                                      # signed zeros tie with +0
        s[7, 1::2] = 0.0
        s[8, :] = 3.0e38                                      # the largest finite scores
        s[8, ::3] = -3.0e38
    if Q > 9:   # one outlier stretches the range: the rest crowd one bin (radix rounds), ties
        s[9] = (np.round(rng.standard_normal(P) * 64) / 64).astype(np.float32)
        s[9, P // 3] = 1.0e30
    ix = dsai.Indexer(heads=32, dim=128, kpool=KP, index_topk=index_topk,
                      order=dsai.DSAI_ORDER_SCORE if order == "score" else dsai.DSAI_ORDER_INDEX)
    ids, vals = ix.topk_pools(torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    gids, gvals = ids.cpu().numpy(), vals.cpu().numpy().astype(np.float64)
    oids, ovals = oracle.topk_pools(s.astype(np.float64), index_topk // KP)
    if order == "index":
        for r in range(Q):
            m = int((oids[r] >= 0).sum())
            o = np.argsort(oids[r, :m], kind="stable")
            oids[r, :m], ovals[r, :m] = oids[r, :m][o], ovals[r, :m][o]
    assert np.array_equal(gids, oids), np.argwhere(gids != oids)[:8]
    assert np.array_equal(gvals, ovals)


@pytest.mark.parametrize("case", POOL_CASES, ids=[c.name for c in POOL_CASES])
def test_select_and_expand_pipeline(dsai, case):
    """kpool -> select -> expand on the GPU; the oracle scores the GPU's pool
    keys (stage isolation) and expands the GPU's pool ids."""
    log(f"[gpu] select+expand {case}")
    inp = pooled_case_inputs(case)
    ix = dsai.Indexer(heads=case.H, dim=case.D, kpool=case.KP, index_topk=case.index_topk,
                      first_key=case.first_key)
    pk, pt, pv = ix.kpool_compress(bf16_gpu(inp["k_normed_bits"]), torch.from_numpy(inp["gate"]).cuda(),
                                   torch.from_numpy(inp["valid"]).cuda(),
                                   torch.from_numpy(inp["ape"]).cuda())
    q = bf16_gpu(inp["q_bits"])
    w = torch.from_numpy(inp["w"]).cuda()
    ids, vals = ix.select(q, w, pk, pv)
    tok = ix.expand(ids)
    torch.cuda.synchronize()
    gids, gvals, gtok = ids.cpu().numpy(), vals.cpu().numpy(), tok.cpu().numpy()
    pk64, pvv = f64(bits_of(pk)), pv.cpu().numpy()
    o = oracle.pooled_index_scores(f64(inp["q_bits"]), inp["w"], pk64, pvv)
    sel = case.index_topk // case.KP
    valid_idx = np.nonzero(pvv)[0]
    # parity rules over the valid pools (ids mapped into the valid subset)
    rows_scores = [o[i][valid_idx] for i in range(case.Q)]
    pos = -np.ones(max(1, o.shape[1]), dtype=np.int64)
    pos[valid_idx] = np.arange(len(valid_idx))
    mapped = np.where(gids >= 0, pos[np.maximum(gids, 0)], -1)
    assert np.all((gids < 0) | (pvv[np.maximum(gids, 0)] == 1)), "invalid pool selected"
    check_topk_rows(mapped, gvals, rows_scores, sel, [f"{case.name} q={i}" for i in range(case.Q)])
    assert np.array_equal(gtok, oracle.expand_selection(gids, case.first_key, case.KP))
    # the split calls give the same result as select
    sc = ix.index_scores(q, w, pk, pv)
    ids2, vals2 = ix.topk_pools(sc)
    torch.cuda.synchronize()
    assert np.array_equal(ids2.cpu().numpy(), gids)


@pytest.mark.parametrize("P,KP,index_topk,first_key", [
    (16384, 4, 512, 0),       # block select ranks its rows: tokens from the same kernel
    (16384, 4, 4096, 7),      # select_k > 512: row sort, then the expand kernel
    (40000, 2, 512, 3),       # streaming select, then the expand kernel
    (1000, 8, 64, 5),
    (0, 4, 64, 0),            # no pools: every row padding
])
@pytest.mark.parametrize("order", ["score", "index"])
def test_select_expand_fused(dsai, P, KP, index_topk, first_key, order):
    """dsai_select_expand gives the ids and scores of dsai_select and the
    tokens of dsai_expand on them, bit for bit, and the tokens equal the
    oracle's expansion of the ids."""
    log(f"[gpu] select_expand P={P} KP={KP} index_topk={index_topk} order={order}")
    rng = np.random.default_rng(7 + P + KP)
    Q, H, D = 11, 32, 128
    ix = dsai.Indexer(heads=H, dim=D, kpool=KP, index_topk=index_topk, first_key=first_key,
                      order=dsai.DSAI_ORDER_SCORE if order == "score" else dsai.DSAI_ORDER_INDEX)
    f = lambda shape: bf16_gpu(SY.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32)))
    q, pk = f((Q, H, D)), f((max(P, 1), D))[:P]
    w = torch.from_numpy((rng.standard_normal((Q, H)) / np.sqrt(H)).astype(np.float32)).cuda()
    pv = torch.from_numpy((rng.random(P) < 0.9).astype(np.uint8)).cuda()
    ids, vals = ix.select(q, w, pk, pv)
    tok = ix.expand(ids)
    fids, fvals, ftok = ix.select(q, w, pk, pv, expand=True)
    torch.cuda.synchronize()
    gids = ids.cpu().numpy()
    assert np.array_equal(fids.cpu().numpy(), gids)
    assert np.array_equal(fvals.cpu().numpy().view(np.uint32), vals.cpu().numpy().view(np.uint32))
    assert np.array_equal(ftok.cpu().numpy(), tok.cpu().numpy())
    assert np.array_equal(ftok.cpu().numpy(), oracle.expand_selection(gids, first_key, KP))


@pytest.mark.parametrize("KP", [1, 2, 3, 4, 5, 6, 7, 8])
def test_expand_bit_exact(dsai, KP):
    log(f"[gpu] expand KP={KP}")
    sel, Q, P, fk = 96, 37, 5000, 11
    ids = SY.random_pool_ids(KP, Q, sel, P, missing_frac=0.2)
    ix = dsai.Indexer(heads=32, dim=128, kpool=KP, index_topk=sel * KP, first_key=fk)
    out = torch.full((Q, sel * KP), -777, dtype=torch.int32, device="cuda")
    tok = ix.expand(torch.from_numpy(ids).cuda(), tokens=out)
    torch.cuda.synchronize()
    assert np.array_equal(tok.cpu().numpy(), oracle.expand_selection(ids, fk, KP))


def test_pooled_decode_full_size_counts(dsai):
    """The pooled decode workload: 16384 pools, the last 10 invalid."""
    case = SY.POOLED_CASES["pooled_decode"]
    inp = pooled_case_inputs(case)
    ix = dsai.Indexer(heads=case.H, dim=case.D, kpool=case.KP, index_topk=case.index_topk)
    _, _, pv = ix.kpool_compress(bf16_gpu(inp["k_normed_bits"]), torch.from_numpy(inp["gate"]).cuda(),
                                 torch.from_numpy(inp["valid"]).cuda(), torch.from_numpy(inp["ape"]).cuda())
    torch.cuda.synchronize()
    pvv = pv.cpu().numpy()
    assert pvv.shape == (16384,)
    assert not pvv[16374:].any()


def test_pooled_kp1_equals_unpooled(dsai):
    """Two GPU paths against each other: with KP = 1, ape = 0 and every token
    valid, a pool key is its token's key exactly (a one-slot softmax is 1), so
    the pooled selection of a decode query over N cached keys must equal the
    unpooled selection of a query row that sees all N keys (the row at
    position N - 1 of a causal batch): the same ids in the same order and
    equal scores."""
    N, H, D, Q, sel = 3000, 32, 128, 6, 256
    log(f"[gpu] pooled KP=1 vs unpooled N={N}")
    rng = np.random.default_rng(77)
    k_bits = SY.f32_to_bf16_bits(rng.standard_normal((N, D)).astype(np.float32))
    qd_bits = SY.f32_to_bf16_bits(rng.standard_normal((Q, H, D)).astype(np.float32))
    wd = (rng.standard_normal((Q, H)) / np.sqrt(H)).astype(np.float32)
    pix = dsai.Indexer(heads=H, dim=D, kpool=1, index_topk=sel)
    pk, pt, pv = pix.kpool_compress(bf16_gpu(k_bits),
                                    torch.from_numpy(rng.standard_normal((N, D)).astype(np.float32)).cuda(),
                                    torch.ones(N, dtype=torch.uint8, device="cuda"),
                                    torch.zeros((1, D), dtype=torch.float32, device="cuda"))
    ids, vals = pix.select(bf16_gpu(qd_bits), torch.from_numpy(wd).cuda(), pk, pv)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(pk), k_bits)
    # unpooled: S = N + Q - 1 rows, the last Q of them the decode queries
    S = N + Q - 1
    q_bits = np.zeros((S, 1, H, D), dtype=np.uint16)
    q_bits[N - 1:, 0] = qd_bits
    w = np.zeros((S, 1, H), dtype=np.float32)
    w[N - 1:, 0] = wd
    ix = dsai.Indexer(heads=H, dim=D)
    ui, us = ix.score_topk(bf16_gpu(q_bits), bf16_gpu(k_bits.reshape(N, 1, D)),
                           torch.from_numpy(w).cuda(), 1, sel)
    torch.cuda.synchronize()
    ui, us = ui.cpu().numpy()[0, N - 1:], us.cpu().numpy()[0, N - 1:]
    assert np.array_equal(ids.cpu().numpy(), ui)
    assert np.array_equal(vals.cpu().numpy().astype(np.float64), us.astype(np.float64))


@pytest.mark.parametrize("P,KP,index_topk", [(16384, 4, 512), (3001, 2, 64), (40000, 4, 512)])
@pytest.mark.parametrize("order", ["score", "index"])
def test_select_with_pool_limits(dsai, P, KP, index_topk, order):
    """Per-row visible-pool bounds (multi-token decode): each row selects only
    among its pools p < bound (bounds below 0 act as 0, above P as P).  The
    GPU's selection on the oracle's pool keys keeps the top-k parity rules
    against the oracle with the same bounds; the expanded token ids are the
    oracle's expansion of the GPU's ids; bounds of P for every row give the
    unbounded call's bits; a bound of 0 gives a padding row."""
    log(f"[gpu] pool limits P={P} KP={KP} order={order}")
    rng = np.random.default_rng(P + KP)
    Q, H, D = 13, 32, 128
    ix = dsai.Indexer(heads=H, dim=D, kpool=KP, index_topk=index_topk,
                      order=dsai.DSAI_ORDER_SCORE if order == "score" else dsai.DSAI_ORDER_INDEX)
    qb = SY.f32_to_bf16_bits(rng.standard_normal((Q, H, D)).astype(np.float32))
    pkb = SY.f32_to_bf16_bits(rng.standard_normal((P, D)).astype(np.float32))
    w = (rng.standard_normal((Q, H)) / np.sqrt(H)).astype(np.float32)
    pv = (rng.random(P) < 0.9).astype(np.uint8)
    lim = rng.integers(0, P + 1, size=Q).astype(np.int32)
    lim[:5] = [-3, 0, 1, P, P + 9]
    q, pk, wg, pvg = bf16_gpu(qb), bf16_gpu(pkb), torch.from_numpy(w).cuda(), torch.from_numpy(pv).cuda()
    limg = torch.from_numpy(lim).cuda()
    ids, vals, tok = ix.select(q, wg, pk, pvg, expand=True, pool_limit=limg)
    u_ids, u_vals = ix.select(q, wg, pk, pvg)
    f_ids, f_vals = ix.select(q, wg, pk, pvg, pool_limit=torch.full((Q,), P, dtype=torch.int32,
                                                                     device="cuda"))
    torch.cuda.synchronize()
    gids, gv = ids.cpu().numpy(), vals.cpu().numpy()
    assert np.array_equal(f_ids.cpu().numpy(), u_ids.cpu().numpy())
    assert np.array_equal(f_vals.cpu().numpy().view(np.uint32), u_vals.cpu().numpy().view(np.uint32))
    assert np.all(gids[1] == -1) and np.all(np.isneginf(gv[1]))      # bound 0
    assert np.all(gids[0] == -1)                                     # bound < 0
    assert np.array_equal(tok.cpu().numpy(), oracle.expand_selection(gids, 0, KP))
    sel = index_topk // KP
    o = oracle.pooled_index_scores(f64(qb), w, f64(pkb), pv, pool_limit=lim)
    for r in range(Q):
        vis = np.nonzero(np.isfinite(o[r]))[0]
        pos = np.full(P, -1, dtype=np.int64)
        pos[vis] = np.arange(vis.size)
        gi = np.where(gids[r] >= 0, pos[np.maximum(gids[r], 0)], -1)
        if order == "index":   # same set in pool-id order: compare in score order
            m = int((gids[r] >= 0).sum())
            srt = np.lexsort((gids[r][:m], -gv[r][:m].astype(np.float64)))
            gi = np.concatenate([gi[:m][srt], gi[m:]])
            gvr = np.concatenate([gv[r][:m][srt], gv[r][m:]])
        else:
            gvr = gv[r]
        check_topk_rows(gi[None], gvr[None], [o[r][vis]], sel, [f"row {r} bound {lim[r]}"])
