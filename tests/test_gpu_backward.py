"""GPU checks of the backward (dsai_indexer_backward): gradients of the
selected scores with respect to index_q, index_k and weights.

The oracle is oracle.indexer_backward (fp64 on the bf16 inputs).  Indices and
incoming gradients are synthetic inputs (synthetic.key_lists /
noisy_key_lists / score_grads), never the GPU's own selection.

* Integer inputs (q, k small integers; weights and incoming gradients powers
  of two): every product and partial sum of the GPU path is exact in fp32 and
  every gated weight g * w is exact in bf16, so grad_q and grad_k equal the
  oracle rounded to bf16 (nearest even) bit for bit, and grad_weights equals
  it exactly.
* Gaussian inputs: the bound below, derived from the arithmetic.  The gated
  weight G = g * w * [d > 0] is rounded to bf16 (relative error <= 2^-8 per
  term), m terms (plus the 64-term head sums of grad_k) are accumulated in
  fp32 (<= (m + 64) 2^-24 of the sum of absolute terms A), gates whose
  product lies within fp32 reach of 0 may be decided either way (band: the
  sum of those absolute terms), and the result is rounded to bf16 once
  (<= 2^-8 of its magnitude):
      |gpu - exact| <= (2^-8 + (m + 64) 2^-24) A * 1.01 + 2^-8 |exact| + 1.01 band.
  grad_weights (fp32, no operand rounding; each product d carries <= D 2^-24
  sum_d |q_d k_d| of error):  |gpu - exact| <= (m + D + 8) 2^-24 A_w * 1.01.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as SY
from parity import log

pytestmark = pytest.mark.gpu

U8, U24 = 2.0 ** -8, 2.0 ** -24


@pytest.fixture(scope="module")
def dsai():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import sparse_attention_token_index_amd as m
    m.load_library()
    return m


def to_gpu_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def causal_bound(case):
    """Keys each query row may see (the bound used to draw realistic key lists)."""
    return [oracle.visible_keys(t, case.Skv, case.compress_ratio) for t in range(case.S)]


def run_backward(dsai, case, inp, sup, grad, ws_fill=None):
    ix = dsai.Indexer(heads=case.H, dim=case.D)
    q, k = to_gpu_bf16(inp["q_bits"]), to_gpu_bf16(inp["k_bits"])
    w = torch.from_numpy(inp["w"]).cuda()
    need = ix.backward_workspace_size(case.S, case.Skv, case.B, case.topk, case.compress_ratio)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    if ws_fill is not None:
        ws.fill_(ws_fill)  # stale contents the call must clear
    gq, gk, gw = ix.indexer_backward(q, k, w, torch.from_numpy(sup).cuda(),
                                     torch.from_numpy(grad).cuda(), case.compress_ratio,
                                     workspace=ws)
    torch.cuda.synchronize()
    return bf16_bits(gq), bf16_bits(gk), gw.cpu().numpy()


def oracle_backward(case, inp, sup, grad, rows=None, keys=None, with_bounds=False):
    q = SY.bf16_bits_to_f32(inp["q_bits"]).astype(np.float64)
    k = SY.bf16_bits_to_f32(inp["k_bits"]).astype(np.float64)
    return oracle.indexer_backward(q, k, inp["w"].astype(np.float64), case.compress_ratio, sup,
                                   grad.astype(np.float64), rows=rows, keys=keys,
                                   with_bounds=with_bounds)


def zero_normalised(bits):
    """bf16 bits with -0 mapped to +0."""
    b = bits.copy()
    b[b == 0x8000] = 0
    return b


def check_bf16_bound(name, got_bits, exact, A, band, m):
    got = SY.bf16_bits_to_f32(got_bits).astype(np.float64)
    tol = (U8 + (m + 64) * U24) * A * 1.01 + U8 * np.abs(exact) + 1.01 * band + 1e-30
    err = np.abs(got - exact)
    bad = err > tol
    assert not bad.any(), (name, int(bad.sum()), np.argwhere(bad)[:4], float((err - tol).max()))


def check_w_bound(got, exact, A_w, m, D):
    tol = (m + D + 8) * U24 * A_w * 1.01 + 1e-30
    err = np.abs(got.astype(np.float64) - exact)
    bad = err > tol
    assert not bad.any(), ("grad_w", int(bad.sum()), np.argwhere(bad)[:4])


INT_CASES = [
    SY.IndexerCase("bwd_int_h64d128_r1", B=2, S=150, Skv=150, H=64, D=128, compress_ratio=1,
                   topk=40, w_var=1 / 64, seed=51, integer=True),
    SY.IndexerCase("bwd_int_h20d64_r3", B=1, S=300, Skv=80, H=20, D=64, compress_ratio=3,
                   topk=33, w_var=1 / 20, seed=52, integer=True),
    SY.IndexerCase("bwd_int_h4d32_r1", B=3, S=100, Skv=100, H=4, D=32, compress_ratio=1,
                   topk=7, w_var=1 / 4, seed=53, integer=True),
    SY.IndexerCase("bwd_int_h40d128_r2", B=1, S=200, Skv=120, H=40, D=128, compress_ratio=2,
                   topk=64, w_var=1 / 40, seed=54, integer=True),
]


@pytest.mark.parametrize("case", INT_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("noisy", [False, True], ids=["selection", "noisy"])
def test_integer_inputs_bit_exact(dsai, case, noisy):
    """Integer data: grad_q / grad_k bits = bf16(oracle), grad_weights = oracle.
    noisy: entries with -1/-2 padding, out-of-range, masked and repeated keys;
    selection: distinct usable keys per row (-1 padded where fewer are visible)."""
    log(f"[gpu] backward integer {case.name} noisy={noisy}")
    inp = SY.indexer_inputs(case)
    if noisy:
        sup = SY.noisy_key_lists(case.seed, case.B, case.S, case.topk, case.Skv)
    else:
        sup = SY.key_lists(case.seed, case.B, case.S, case.topk, case.Skv, causal_bound(case))
    grad = SY.score_grads(case.seed, case.B, case.S, case.topk, integer=True)
    gq, gk, gw = run_backward(dsai, case, inp, sup, grad, ws_fill=0x7F)
    ref = oracle_backward(case, inp, sup, grad)
    _, rq = oracle.round_to_bf16(ref["grad_q"])
    _, rk = oracle.round_to_bf16(ref["grad_k"])
    assert np.array_equal(zero_normalised(gq), zero_normalised(rq)), np.argwhere(gq != rq)[:5]
    assert np.array_equal(zero_normalised(gk), zero_normalised(rk)), np.argwhere(gk != rk)[:5]
    assert np.array_equal(gw.astype(np.float64), ref["grad_w"]), np.argwhere(gw != ref["grad_w"])[:5]
    assert np.count_nonzero(ref["grad_k"]) > 0 and np.count_nonzero(ref["grad_q"]) > 0


GAUSS_CASES = [
    SY.IndexerCase("bwd_h64d128_r1", B=2, S=200, Skv=200, H=64, D=128, compress_ratio=1,
                   topk=75, w_var=1 / 64, seed=61),
    SY.IndexerCase("bwd_h20d64_r3", B=1, S=400, Skv=120, H=20, D=64, compress_ratio=3,
                   topk=40, w_var=1 / 20, seed=62),
    SY.IndexerCase("bwd_h4d32_r1", B=3, S=150, Skv=150, H=4, D=32, compress_ratio=1,
                   topk=16, w_var=1 / 4, seed=63),
    SY.IndexerCase("bwd_h64d64_r4", B=1, S=600, Skv=150, H=64, D=64, compress_ratio=4,
                   topk=1, w_var=1 / 64, seed=64),
]


@pytest.mark.parametrize("case", GAUSS_CASES, ids=lambda c: c.name)
def test_gaussian_inputs_within_bound(dsai, case):
    log(f"[gpu] backward gaussian {case.name}")
    inp = SY.indexer_inputs(case)
    sup = SY.key_lists(case.seed, case.B, case.S, case.topk, case.Skv, causal_bound(case))
    grad = SY.score_grads(case.seed, case.B, case.S, case.topk)
    gq, gk, gw = run_backward(dsai, case, inp, sup, grad)
    ref = oracle_backward(case, inp, sup, grad, with_bounds=True)
    check_bf16_bound("grad_q", gq, ref["grad_q"], ref["abs_q"], ref["band_q"], case.topk)
    check_bf16_bound("grad_k", gk, ref["grad_k"], ref["abs_k"], ref["band_k"],
                     ref["count_k"][:, :, None])
    check_w_bound(gw, ref["grad_w"], ref["abs_w"], case.topk, case.D)
    # aggregate accuracy: bf16 operands and outputs keep the relative RMS
    # error near 2^-8 (a dropped or misplaced term would not)
    for name, got in (("grad_q", gq), ("grad_k", gk)):
        ex = ref[name]
        e = SY.bf16_bits_to_f32(got).astype(np.float64) - ex
        rel = np.sqrt(np.sum(e * e) / max(np.sum(ex * ex), 1e-300))
        assert rel < 2.0 ** -7, (name, rel)


FULL_CASES = {
    "prefill": SY.CASES["prefill"],   # key-block grouping
    "c4": SY.CASES["c4"],             # sparse selection: per-entry scatter
    # 16384 rows over 4096 keys, half selected: key-block workgroups of
    # several hundred rows (more than one window of bucket bounds)
    "dense_16k": SY.IndexerCase("dense_16k", B=1, S=16384, Skv=4096, H=64, D=128,
                                compress_ratio=1, topk=2048, w_var=1 / 64, seed=67),
}


@pytest.mark.parametrize("name", sorted(FULL_CASES))
def test_full_size_sampled(dsai, name):
    """The benchmark's shapes: every row's grad_q / grad_weights computed on
    the GPU, the oracle on sampled rows; grad_k on sampled keys (the oracle
    sums every row's entries that name them)."""
    case = FULL_CASES[name]
    log(f"[gpu] backward full size {name}")
    inp = SY.indexer_inputs(case)
    sup = SY.key_lists(case.seed + 7, case.B, case.S, case.topk, case.Skv, causal_bound(case))
    grad = SY.score_grads(case.seed + 7, case.B, case.S, case.topk)
    gq, gk, gw = run_backward(dsai, case, inp, sup, grad)
    rng = np.random.default_rng(5)
    rows = sorted({0, 1, 2, 3, case.S - 1, case.S // 2} | set(rng.choice(case.S, 10, replace=False).tolist()))
    keys = sorted({0, 1, case.Skv - 1, case.Skv // 3} | set(rng.choice(case.Skv, 8, replace=False).tolist()))
    sub = {"q_bits": inp["q_bits"][rows], "k_bits": inp["k_bits"], "w": inp["w"][rows]}
    ref = oracle_backward(case, sub, np.ascontiguousarray(sup[:, rows]),
                          np.ascontiguousarray(grad[:, rows]), rows=rows, with_bounds=True)
    check_bf16_bound("grad_q", gq[rows], ref["grad_q"], ref["abs_q"], ref["band_q"], case.topk)
    check_w_bound(gw[rows], ref["grad_w"], ref["abs_w"], case.topk, case.D)
    refk = oracle_backward(case, inp, sup, grad, keys=keys, with_bounds=True)
    check_bf16_bound("grad_k", gk[keys], refk["grad_k"][keys], refk["abs_k"][keys],
                     refk["band_k"][keys], refk["count_k"][keys][:, :, None])


def test_many_repeated_keys_in_one_block(dsai):
    """2048 entries per row drawn from 40 keys: far more entries per key
    block than threads per workgroup, each key repeated ~50 times (their
    gradients add).  Integer data: grad_q and grad_weights are exact; the
    key gradients sum a key's repeated gradients before the product with
    the head weights, and that sum times w need not fit bf16, so grad_k is
    held to the bound."""
    case = SY.IndexerCase("bwd_repeats", B=2, S=48, Skv=300, H=64, D=128, compress_ratio=1,
                          topk=2048, w_var=1 / 64, seed=66, integer=True)
    log(f"[gpu] backward {case.name}")
    inp = SY.indexer_inputs(case)
    sup = SY.noisy_key_lists(case.seed, case.B, case.S, case.topk, 38)   # entries in [-2, 41)
    grad = SY.score_grads(case.seed, case.B, case.S, case.topk, integer=True)
    gq, gk, gw = run_backward(dsai, case, inp, sup, grad, ws_fill=0x33)
    ref = oracle_backward(case, inp, sup, grad, with_bounds=True)
    _, rq = oracle.round_to_bf16(ref["grad_q"])
    assert np.array_equal(zero_normalised(gq), zero_normalised(rq)), np.argwhere(gq != rq)[:5]
    assert np.array_equal(gw.astype(np.float64), ref["grad_w"])
    check_bf16_bound("grad_k", gk, ref["grad_k"], ref["abs_k"], ref["band_k"],
                     ref["count_k"][:, :, None])
    assert np.count_nonzero(ref["grad_k"][:41]) > 0


def test_more_than_1024_key_blocks(dsai):
    """Skv = 300000 (over 1024 blocks of 256 keys): the per-entry atomic
    scatter instead of the key-block grouping; same bound."""
    case = SY.IndexerCase("bwd_wide_keys", B=1, S=96, Skv=300000, H=20, D=64, compress_ratio=1,
                          topk=40, w_var=1 / 20, seed=65)
    log(f"[gpu] backward {case.name}")
    inp = SY.indexer_inputs(case)
    sup = SY.noisy_key_lists(case.seed, case.B, case.S, case.topk, 120)   # keys near the rows
    grad = SY.score_grads(case.seed, case.B, case.S, case.topk)
    gq, gk, gw = run_backward(dsai, case, inp, sup, grad, ws_fill=0x55)
    ref = oracle_backward(case, inp, sup, grad, with_bounds=True)
    check_bf16_bound("grad_q", gq, ref["grad_q"], ref["abs_q"], ref["band_q"], case.topk)
    check_bf16_bound("grad_k", gk, ref["grad_k"], ref["abs_k"], ref["band_k"],
                     ref["count_k"][:, :, None])
    check_w_bound(gw, ref["grad_w"], ref["abs_w"], case.topk, case.D)
    assert np.count_nonzero(ref["grad_k"]) > 0


def test_edge_sizes(dsai):
    """S == 0 (grad_k all zero), Skv == 0 (grad_q / grad_weights zero), rows
    with no visible key, topk == 1, and no usable entry at all."""
    H, D = 8, 32
    ix = dsai.Indexer(heads=H, dim=D)
    dev = "cuda"
    # S == 0: grad_k must still be written (zeros over stale memory)
    k = torch.randn(9, 2, D, device=dev).to(torch.bfloat16)
    gk = torch.full((9, 2, D), 7.0, device=dev).to(torch.bfloat16)
    q0 = torch.empty((0, 2, H, D), dtype=torch.bfloat16, device=dev)
    ix.indexer_backward(q0, k, torch.empty((0, 2, H), device=dev),
                        torch.empty((2, 0, 3), dtype=torch.int32, device=dev),
                        torch.empty((2, 0, 3), device=dev), 1, grad_k=gk)
    torch.cuda.synchronize()
    assert torch.count_nonzero(gk.float()).item() == 0
    # Skv == 0 and a ratio larger than S: nothing usable, zeros everywhere
    for Skv, r in ((0, 1), (5, 100)):
        S, B, n = 37, 2, 5
        q = torch.randn(S, B, H, D, device=dev).to(torch.bfloat16)
        kk = torch.randn(Skv, B, D, device=dev).to(torch.bfloat16)
        w = torch.randn(S, B, H, device=dev)
        sup = torch.randint(-1, 6, (B, S, n), dtype=torch.int32, device=dev)
        g = torch.randn(B, S, n, device=dev)
        gq, gkk, gw = ix.indexer_backward(
            q, kk, w, sup, g, r,
            grad_q=torch.full((S, B, H, D), 3.0, device=dev).to(torch.bfloat16),
            grad_weights=torch.full((S, B, H), 3.0, device=dev))
        torch.cuda.synchronize()
        assert torch.count_nonzero(gq.float()).item() == 0
        assert torch.count_nonzero(gw).item() == 0
        assert torch.count_nonzero(gkk.float()).item() == 0


def test_autograd_function(dsai):
    """IndexerFunction: forward = score_topk's (scores, indices); backward of
    sum(scores * G) = indexer_backward at those indices (integer data: the
    same bits whatever the order of the atomic adds)."""
    case = INT_CASES[0]
    inp = SY.indexer_inputs(case)
    ix = dsai.Indexer(heads=case.H, dim=case.D)
    q = to_gpu_bf16(inp["q_bits"]).requires_grad_(True)
    k = to_gpu_bf16(inp["k_bits"]).requires_grad_(True)
    w = torch.from_numpy(inp["w"]).cuda().requires_grad_(True)
    scores, idx = dsai.IndexerFunction.apply(ix, q, k, w, case.compress_ratio, case.topk)
    ri, rs = ix.score_topk(q.detach(), k.detach(), w.detach(), case.compress_ratio, case.topk)
    assert torch.equal(idx, ri) and torch.equal(scores, rs)
    g = torch.from_numpy(SY.score_grads(case.seed, case.B, case.S, case.topk, integer=True)).cuda()
    fin = torch.isfinite(scores)
    (torch.where(fin, scores, torch.zeros_like(scores)) * g).sum().backward()
    gq, gk, gw = ix.indexer_backward(q.detach(), k.detach(), w.detach(), idx,
                                     torch.where(fin, g, torch.zeros_like(g)), case.compress_ratio)
    torch.cuda.synchronize()
    assert torch.equal(q.grad.view(torch.int16), gq.view(torch.int16))
    assert torch.equal(k.grad.view(torch.int16), gk.view(torch.int16))
    assert torch.equal(w.grad, gw)
    # with supplied indices (padding, masked and repeated keys among them)
    sup = torch.from_numpy(SY.noisy_key_lists(case.seed, case.B, case.S, case.topk, case.Skv)).cuda()
    for t in (q, k, w):
        t.grad = None
    scores, idx = dsai.IndexerFunction.apply(ix, q, k, w, case.compress_ratio, case.topk, sup)
    fin = torch.isfinite(scores)
    (torch.where(fin, scores, torch.zeros_like(scores)) * g).sum().backward()
    gq, gk, gw = ix.indexer_backward(q.detach(), k.detach(), w.detach(), sup,
                                     torch.where(fin, g, torch.zeros_like(g)), case.compress_ratio)
    torch.cuda.synchronize()
    assert torch.equal(q.grad.view(torch.int16), gq.view(torch.int16))
    assert torch.equal(k.grad.view(torch.int16), gk.view(torch.int16))
    assert torch.equal(w.grad, gw)


def test_repeat_calls_and_stale_workspace(dsai):
    """Two calls on one workspace (the second over the first's sums): grad_q
    and grad_weights repeat bit for bit (no atomics there), grad_k within
    the bound (the atomic order may differ)."""
    case = GAUSS_CASES[0]
    inp = SY.indexer_inputs(case)
    sup = SY.key_lists(case.seed, case.B, case.S, case.topk, case.Skv, causal_bound(case))
    grad = SY.score_grads(case.seed, case.B, case.S, case.topk)
    ix = dsai.Indexer(heads=case.H, dim=case.D)
    q, k = to_gpu_bf16(inp["q_bits"]), to_gpu_bf16(inp["k_bits"])
    w = torch.from_numpy(inp["w"]).cuda()
    ws = torch.empty(ix.backward_workspace_size(case.S, case.Skv, case.B, case.topk, case.compress_ratio),
                     dtype=torch.uint8, device="cuda")
    tsup, tg = torch.from_numpy(sup).cuda(), torch.from_numpy(grad).cuda()
    a = [t.clone() for t in ix.indexer_backward(q, k, w, tsup, tg, case.compress_ratio, workspace=ws)]
    b = ix.indexer_backward(q, k, w, tsup, tg, case.compress_ratio, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[2], b[2])
    ref = oracle_backward(case, inp, sup, grad, with_bounds=True)
    check_bf16_bound("grad_k", bf16_bits(b[1]), ref["grad_k"], ref["abs_k"], ref["band_k"],
                     ref["count_k"][:, :, None])
