"""GPU checks of scoring at supplied key indices (dsai_score_topk with
topk_indices, the page's optional precomputed-indices form).

The oracle is oracle.scores_at_indices (fp64 on the bf16 inputs); parity is
exact for indices and within abs 1e-3 + rel 1e-3 for scores.  Fed the fused
selection's own output, the gather must reproduce its scores bit for bit (the
same arithmetic on the same keys)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as SY
from parity import TOL_ABS, TOL_REL, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsai():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import sparse_attention_token_index_amd as m
    m.load_library()
    return m


def to_gpu_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def gpu_inputs(inp):
    return (to_gpu_bf16(inp["q_bits"]), to_gpu_bf16(inp["k_bits"]),
            torch.from_numpy(inp["w"]).cuda())


def oracle_at(case, inp, sup):
    q = SY.bf16_bits_to_f32(inp["q_bits"]).astype(np.float64)
    k = SY.bf16_bits_to_f32(inp["k_bits"]).astype(np.float64)
    return oracle.scores_at_indices(q, k, inp["w"].astype(np.float64), case.compress_ratio, sup)


CASES = [
    SY.IndexerCase("at_h64d128_r1", B=2, S=300, Skv=300, H=64, D=128, compress_ratio=1,
                   topk=77, w_var=1 / 64, seed=31),
    SY.IndexerCase("at_h20d64_r3", B=1, S=500, Skv=150, H=20, D=64, compress_ratio=3,
                   topk=40, w_var=1 / 20, seed=32),
    SY.IndexerCase("at_h4d32_r1", B=3, S=200, Skv=200, H=4, D=32, compress_ratio=1,
                   topk=33, w_var=1 / 4, seed=33),
    SY.IndexerCase("at_h64d32_r4", B=1, S=400, Skv=90, H=64, D=32, compress_ratio=4,
                   topk=1, w_var=1 / 64, seed=34),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_random_supplied_indices_match_oracle(dsai, case):
    """Indices drawn from [-3, Skv + 5): padding, out-of-range and masked
    entries, duplicates; the supplied order is kept."""
    log(f"[gpu] score at indices {case.name}")
    inp = SY.indexer_inputs(case)
    rng = np.random.default_rng(case.seed + 100)
    sup = rng.integers(-3, case.Skv + 5, size=(case.B, case.S, case.topk)).astype(np.int32)
    ix = dsai.Indexer(heads=case.H, dim=case.D)
    q, k, w = gpu_inputs(inp)
    gi, gs = ix.score_topk(q, k, w, case.compress_ratio, case.topk,
                           topk_indices=torch.from_numpy(sup).cuda())
    torch.cuda.synchronize()
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy().astype(np.float64)
    oi, ov = oracle_at(case, inp, sup)
    assert np.array_equal(gi, oi), np.argwhere(gi != oi)[:5]
    fin = np.isfinite(ov)
    assert np.array_equal(np.isfinite(gs), fin)
    assert np.all(gs[~fin] == -np.inf)
    err = np.abs(gs[fin] - ov[fin])
    assert np.all(err <= TOL_ABS + TOL_REL * np.abs(ov[fin])), err.max()


@pytest.mark.parametrize("order", [0, 1])
def test_selection_output_rescored_bit_exact_and_in_place(dsai, order):
    """Supplied = the fused selection's own rows (score or index order): the
    gather returns the same indices and bit-identical scores, also when
    out_idx is the supplied array itself."""
    case = SY.IndexerCase("at_consistency", B=2, S=700, Skv=700, H=64, D=128,
                          compress_ratio=2, topk=100, w_var=1 / 64, seed=35)
    inp = SY.indexer_inputs(case)
    q, k, w = gpu_inputs(inp)
    sel = dsai.Indexer(heads=64, dim=128, order=order)
    si, ss = sel.score_topk(q, k, w, case.compress_ratio, case.topk)
    ix = dsai.Indexer(heads=64, dim=128)
    gi, gs = ix.score_topk(q, k, w, case.compress_ratio, case.topk, topk_indices=si)
    inplace = si.clone()
    ii, is_ = ix.score_topk(q, k, w, case.compress_ratio, case.topk, topk_indices=inplace,
                            out_idx=inplace)
    torch.cuda.synchronize()
    assert torch.equal(gi, si) and torch.equal(gs.view(torch.int32), ss.view(torch.int32))
    assert ii.data_ptr() == inplace.data_ptr()
    assert torch.equal(ii, si) and torch.equal(is_.view(torch.int32), ss.view(torch.int32))


def test_prefill_selection_rescored_full_size(dsai):
    """The prefill workload at full size (B=1, S=Skv=4096, H=64, D=128,
    topk=2048): its own selection, rescored, is bit-identical; sampled rows
    against the oracle."""
    case = SY.CASES["prefill"]
    inp = SY.indexer_inputs(case)
    q, k, w = gpu_inputs(inp)
    sel = dsai.Indexer(heads=64, dim=128, order=1)
    si, ss = sel.score_topk(q, k, w, 1, case.topk)
    ix = dsai.Indexer(heads=64, dim=128)
    gi, gs = ix.score_topk(q, k, w, 1, case.topk, topk_indices=si)
    torch.cuda.synchronize()
    assert torch.equal(gi, si) and torch.equal(gs.view(torch.int32), ss.view(torch.int32))
    rows = [0, 1, 2047, 2048, 4095]
    sup = si.cpu().numpy()[:, rows]
    qb, wb = inp["q_bits"][rows], inp["w"][rows]
    qf = SY.bf16_bits_to_f32(qb).astype(np.float64)
    kf = SY.bf16_bits_to_f32(inp["k_bits"]).astype(np.float64)
    oi, ov = oracle.scores_at_indices(qf, kf, wb.astype(np.float64), 1, sup, rows=rows)
    g = gs.cpu().numpy()[:, rows].astype(np.float64)
    assert np.array_equal(gi.cpu().numpy()[:, rows], oi)
    fin = np.isfinite(ov)
    assert np.all(np.abs(g[fin] - ov[fin]) <= TOL_ABS + TOL_REL * np.abs(ov[fin]))
    assert np.all(g[~fin] == -np.inf)


def test_no_visible_keys_and_empty(dsai):
    ix = dsai.Indexer(heads=4, dim=32)
    S, B, n = 5, 2, 6
    q = torch.randn(S, B, 4, 32).to(torch.bfloat16).cuda()
    w = torch.randn(S, B, 4).cuda()
    sup = torch.arange(-1, n - 1, dtype=torch.int32).repeat(B, S, 1).contiguous().cuda()
    # Skv = 0: nothing is visible (the key pointer is never read)
    k0 = torch.zeros(0, B, 32, dtype=torch.bfloat16).cuda()
    gi, gs = ix.score_topk(q, k0, w, 1, n, topk_indices=sup)
    torch.cuda.synchronize()
    assert torch.all(gi == -1) and torch.all(gs == -float("inf"))
    # ratio larger than every t + 1: rows see no key either
    k = torch.randn(8, B, 32).to(torch.bfloat16).cuda()
    gi, gs = ix.score_topk(q, k, w, 100, n, topk_indices=sup)
    torch.cuda.synchronize()
    assert torch.all(gi == -1) and torch.all(gs == -float("inf"))
