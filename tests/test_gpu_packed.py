"""GPU parity of dsai_score_topk_packed (packed sequences) against the fp64
oracle: each sequence is the one-sample problem on its own rows and keys,
with indices local to the sequence.  Ragged lengths, a sequence with no
query rows, one with no keys, the compressed mask, chunked launches inside
a sequence, the supplied-index form, and agreement with one dsai_score_topk
call per sequence."""
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


def bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def packed_inputs(name, cu_q, cu_k, H, D, r, topk, integer, seed):
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    case = SY.IndexerCase(name, B=1, S=Tq, Skv=Tk, H=H, D=D, compress_ratio=r, topk=topk,
                          w_var=1.0 / H, seed=seed, integer=integer)
    inp = SY.indexer_inputs(case)
    return (inp["q_bits"][:, 0], inp["k_bits"][:, 0], inp["w"][:, 0])


CASES = [
    # name, cu_q, cu_k, H, D, ratio, topk, integer inputs, chunk_rows
    ("exact_ragged", [0, 100, 100, 357, 600], [0, 100, 130, 130, 600], 4, 32, 1, 16, True, 0),
    ("exact_c4_chunked", [0, 300, 301, 700], [0, 75, 76, 176], 4, 64, 4, 12, True, 128),
    ("float_h64", [0, 257, 260, 900], [0, 257, 260, 643], 64, 128, 1, 64, False, 0),
]


@pytest.mark.parametrize("name,cu_q,cu_k,H,D,r,topk,integer,chunk", CASES)
def test_packed_matches_oracle(dsai, name, cu_q, cu_k, H, D, r, topk, integer, chunk):
    log(f"[gpu] packed {name}")
    cu_q, cu_k = np.array(cu_q, np.int64), np.array(cu_k, np.int64)
    qb, kb, w = packed_inputs(name, cu_q, cu_k, H, D, r, topk, integer, seed=len(name))
    ix = dsai.Indexer(heads=H, dim=D, chunk_rows=chunk)
    gi, gs = ix.score_topk_packed(bf16(qb), bf16(kb), torch.from_numpy(w).cuda(), cu_q, cu_k, r,
                                  topk)
    torch.cuda.synchronize()
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
    q64 = SY.bf16_bits_to_f32(qb).astype(np.float64)
    k64 = SY.bf16_bits_to_f32(kb).astype(np.float64)
    w64 = w.astype(np.float64)
    oi, ov = oracle.score_topk_packed(q64, k64, w64, cu_q, cu_k, r, topk)
    if integer:  # every step exact: the same indices, order and scores
        assert np.array_equal(gi, oi)
        assert np.array_equal(gs.astype(np.float64), ov.astype(np.float32).astype(np.float64))
    else:
        for i in range(len(cu_q) - 1):
            q0, q1, k0, k1 = (int(x) for x in (cu_q[i], cu_q[i + 1], cu_k[i], cu_k[i + 1]))
            if q1 == q0:
                continue
            _, _, full = oracle.score_topk(q64[q0:q1, None], k64[k0:k1, None], w64[q0:q1, None],
                                           r, topk, row_values=True)
            check_topk_rows(gi[q0:q1], gs[q0:q1], full, topk,
                            [f"{name} seq {i} t={t}" for t in range(q1 - q0)])

    # supplied indices: the rows' own selection rescored bit for bit
    ai, av = ix.score_topk_packed(bf16(qb), bf16(kb), torch.from_numpy(w).cuda(), cu_q, cu_k, r,
                                  topk, topk_indices=torch.from_numpy(gi).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(ai.cpu().numpy(), gi)
    assert np.array_equal(av.cpu().numpy().view(np.uint32), gs.view(np.uint32))

    # one dsai_score_topk call per sequence gives the same rows
    for i in range(len(cu_q) - 1):
        q0, q1, k0, k1 = (int(x) for x in (cu_q[i], cu_q[i + 1], cu_k[i], cu_k[i + 1]))
        if q1 == q0:
            continue
        si, ss = ix.score_topk(bf16(qb[q0:q1, None]), bf16(kb[k0:k1, None]),
                               torch.from_numpy(w[q0:q1, None]).cuda(), r, topk)
        torch.cuda.synchronize()
        assert np.array_equal(si.cpu().numpy()[0], gi[q0:q1]), (name, i)
        assert np.array_equal(ss.cpu().numpy()[0].view(np.uint32), gs[q0:q1].view(np.uint32))


def _ragged_offsets(rng, nseq, max_q, max_k):
    """Cumulative offsets of nseq sequences with 0..max_q rows and 0..max_k
    keys each (some sequences empty on one side or both)."""
    lq = rng.integers(0, max_q + 1, nseq)
    lk = rng.integers(0, max_k + 1, nseq)
    lq[rng.random(nseq) < 0.1] = 0
    lk[rng.random(nseq) < 0.1] = 0
    return (np.concatenate([[0], np.cumsum(lq)]).astype(np.int64),
            np.concatenate([[0], np.cumsum(lk)]).astype(np.int64))


PACKED_MANY = [
    # name, nseq, max rows, max keys, H, D, ratio, topk, extra long sequence
    ("many_256", 256, 40, 60, 4, 32, 1, 16, 0),
    ("many_c2", 150, 50, 40, 4, 64, 2, 12, 0),
    # one sequence past the dense store: its launch uses the filter store
    # for every sequence it holds
    ("long_and_short", 70, 30, 50, 4, 32, 1, 16, 6000),
]


@pytest.mark.parametrize("name,nseq,max_q,max_k,H,D,r,topk,extra", PACKED_MANY)
def test_packed_many_sequences(dsai, name, nseq, max_q, max_k, H, D, r, topk, extra):
    """Hundreds of ragged sequences (several launches of up to 64
    sequences, taken longest first), integer inputs: bit-exact against the
    packed oracle, order and ties included."""
    log(f"[gpu] packed many {name}")
    rng = np.random.default_rng(len(name) + nseq)
    cu_q, cu_k = _ragged_offsets(rng, nseq, max_q, max_k)
    if extra:
        at = nseq // 3  # the long sequence sits in the middle of the batch
        lq, lk = np.diff(cu_q), np.diff(cu_k)
        lq[at], lk[at] = extra, extra
        cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
        cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    qb, kb, w = packed_inputs(name, cu_q, cu_k, H, D, r, topk, True, seed=nseq)
    ix = dsai.Indexer(heads=H, dim=D)
    gi, gs = ix.score_topk_packed(bf16(qb), bf16(kb), torch.from_numpy(w).cuda(), cu_q, cu_k, r,
                                  topk)
    torch.cuda.synchronize()
    oi, ov = oracle.score_topk_packed(SY.bf16_bits_to_f32(qb).astype(np.float64),
                                      SY.bf16_bits_to_f32(kb).astype(np.float64),
                                      w.astype(np.float64), cu_q, cu_k, r, topk)
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
    bad = np.nonzero((gi != oi).any(axis=1))[0]
    assert bad.size == 0, f"{name}: {bad.size} rows differ, first {bad[:5]}"
    assert np.array_equal(gs.astype(np.float64), ov.astype(np.float32).astype(np.float64))


def test_packed_backward_exact(dsai):
    """dsai_indexer_backward_packed on integer inputs (every GPU step exact):
    bit-identical to the fp64 packed oracle rounded to bf16, and to one
    dsai_indexer_backward call per sequence.  A sequence with rows but no
    keys, one with keys but no rows, ragged lengths, the compressed mask."""
    log("[gpu] packed backward")
    H, D, r, n = 4, 32, 2, 12
    cu_q = np.array([0, 90, 90, 150, 400], np.int64)
    cu_k = np.array([0, 45, 70, 70, 195], np.int64)
    qb, kb, w = packed_inputs("bwd_packed", cu_q, cu_k, H, D, r, n, True, seed=41)
    sup = np.full((int(cu_q[-1]), n), -1, np.int32)
    for i in range(len(cu_q) - 1):
        q0, q1, k0, k1 = (int(x) for x in (cu_q[i], cu_q[i + 1], cu_k[i], cu_k[i + 1]))
        if q1 > q0 and k1 > k0:
            bound = [oracle.visible_keys(t, k1 - k0, r) for t in range(q1 - q0)]
            sup[q0:q1] = SY.key_lists(41 + i, 1, q1 - q0, n, k1 - k0, bound)[0]
    g = SY.score_grads(41, 1, int(cu_q[-1]), n, integer=True)[0]
    ix = dsai.Indexer(heads=H, dim=D)
    tq, tk, tw = bf16(qb), bf16(kb), torch.from_numpy(w).cuda()
    tsup, tg = torch.from_numpy(sup).cuda(), torch.from_numpy(g).cuda()
    gq, gk, gw = ix.indexer_backward_packed(tq, tk, tw, tsup, tg, cu_q, cu_k, r)
    torch.cuda.synchronize()
    ref = oracle.indexer_backward_packed(SY.bf16_bits_to_f32(qb).astype(np.float64),
                                         SY.bf16_bits_to_f32(kb).astype(np.float64),
                                         w.astype(np.float64), cu_q, cu_k, r, sup,
                                         g.astype(np.float64))

    def bits(t):
        b = t.cpu().view(torch.int16).numpy().view(np.uint16).copy()
        b[b == 0x8000] = 0
        return b

    for got, exact in ((gq, ref["grad_q"]), (gk, ref["grad_k"])):
        want = oracle.round_to_bf16(exact)[1].copy()
        want[want == 0x8000] = 0
        assert np.array_equal(bits(got), want)
    assert np.array_equal(gw.cpu().numpy().astype(np.float64), ref["grad_w"])
    assert np.any(ref["grad_k"] != 0) and np.any(ref["grad_q"] != 0)

    for i in range(len(cu_q) - 1):
        q0, q1, k0, k1 = (int(x) for x in (cu_q[i], cu_q[i + 1], cu_k[i], cu_k[i + 1]))
        if q1 == q0 and k1 == k0:
            continue
        sq, sk, sw = ix.indexer_backward(tq[q0:q1, None], tk[k0:k1, None], tw[q0:q1, None],
                                         tsup[None, q0:q1], tg[None, q0:q1], r)
        torch.cuda.synchronize()
        assert np.array_equal(bits(sq)[:, 0], bits(gq)[q0:q1]), i
        assert np.array_equal(bits(sk)[:, 0], bits(gk)[k0:k1]), i
        assert np.array_equal(sw.cpu().numpy()[:, 0], gw.cpu().numpy()[q0:q1]), i


def test_packed_estimated_cuts_rerun(dsai):
    """Sequences long enough for the filter store, with integer scores that
    fall (or rise) along their keys: in the packed launch the estimated cuts
    of the falling ones drop part of the top k, and those blocks run their
    keys again with cuts to k.  Every row equals one dsai_score_topk call per
    sequence with cuts to k, bit for bit."""
    log("[gpu] packed estimated cuts")
    rng = np.random.default_rng(77)
    lens = [7000, 50, 5200, 0, 300, 6100]
    H, D, topk = 4, 32, 2048
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    k = np.empty((T, D), np.float32)
    for i, n in enumerate(lens):
        s = np.arange(n)
        trend = (n - 1 - s) // 64 if i % 2 == 0 else s // 64
        c = trend + rng.integers(0, 8, n)
        k[cu[i]:cu[i + 1]] = c[:, None] + rng.integers(0, 2, (n, D))
    assert k.max() <= 256   # integers exact in bf16
    q = rng.integers(0, 3, (T, H, D)).astype(np.float32)
    w = rng.choice([0.25, 0.5, 1.0], (T, H)).astype(np.float32)
    qg, kg = bf16(SY.f32_to_bf16_bits(q)), bf16(SY.f32_to_bf16_bits(k))
    wg = torch.from_numpy(w).cuda()
    ix = dsai.Indexer(heads=H, dim=D)   # estimated cuts (the default)
    gi, gs = ix.score_topk_packed(qg, kg, wg, cu, cu, 1, topk)
    torch.cuda.synchronize()
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
    ref = dsai.Indexer(heads=H, dim=D, cuts=dsai.DSAI_CUTS_TOPK)
    for i in range(len(lens)):
        a, b = int(cu[i]), int(cu[i + 1])
        if a == b:
            continue
        si, ss = ref.score_topk(qg[a:b, None].contiguous(), kg[a:b, None].contiguous(),
                                wg[a:b, None].contiguous(), 1, topk)
        torch.cuda.synchronize()
        assert np.array_equal(si.cpu().numpy()[0], gi[a:b]), i
        assert np.array_equal(ss.cpu().numpy()[0].view(np.uint32), gs[a:b].view(np.uint32)), i
