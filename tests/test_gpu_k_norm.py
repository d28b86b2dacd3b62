"""GPU checks of dsai_k_norm, the indexer's LayerNorm with a bias (the cache
write that produces k_normed).

The GPU value must be the bf16 rounding (nearest even) of some value within
E of the exact fp64 result y: round(y - E) <= gpu <= round(y + E).  That
fixes every bit except where y lies within E of a rounding midpoint, or
where the terms cancel to a result much smaller than themselves.  E bounds
the fp32 evaluation's error relative to the size of its terms:
E = 2^-16 * (|gamma_c| * (max_c' |x_c' - mean| + |mean|) / sqrt(var + eps)
+ |beta_c|), about 64 times a few fp32 roundings of terms that size (the
|mean| part covers the error of the fp32 mean on rows far from zero)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as SY

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsai():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import sparse_attention_token_index_amd as m
    m.load_library()
    return m


def bf16_bits(x):
    return SY.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def to_gpu(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def make(rng, N, D):
    """Rows with their own offset and spread (what a LayerNorm input looks like)."""
    x = rng.standard_normal((N, D)) * rng.uniform(0.2, 6.0, (N, 1)) + rng.normal(0, 3, (N, 1))
    g = 1.0 + rng.normal(0, 0.2, D)
    b = rng.normal(0, 0.2, D)
    return bf16_bits(x), bf16_bits(g), bf16_bits(b)


def check(gpu_bits, xb, gb, bb, eps):
    x = SY.bf16_bits_to_f32(xb).astype(np.float64)
    g = SY.bf16_bits_to_f32(gb).astype(np.float64)
    b = SY.bf16_bits_to_f32(bb).astype(np.float64)
    ref = oracle.k_norm(x, g, b, eps)
    y, want = ref["k_normed_f64"], ref["k_normed_bits"]
    same = gpu_bits == want
    if same.all():
        return
    mu = x.mean(axis=1, keepdims=True)
    sd = np.sqrt(x.var(axis=1, keepdims=True) + eps)
    r = (np.abs(x - mu).max(axis=1, keepdims=True) + np.abs(mu)) / sd
    E = 2.0 ** -16 * (np.abs(g)[None, :] * r + np.abs(b)[None, :])
    lo = oracle.round_to_bf16(y - E)[0]
    hi = oracle.round_to_bf16(y + E)[0]
    gv = SY.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    bad = ~same & ~((gv >= lo) & (gv <= hi))
    assert not bad.any(), (np.argwhere(bad)[:5], gv[bad][:5], y[bad][:5])
    # the allowance is narrow: almost every element is bit-exact
    assert same.mean() > 0.999, same.mean()


@pytest.mark.parametrize("N,D", [(65536, 128), (1, 128), (17, 64), (1000, 64), (333, 32)])
def test_k_norm_matches_oracle(dsai, N, D):
    rng = np.random.default_rng(N + D)
    xb, gb, bb = make(rng, N, D)
    ix = dsai.Indexer(heads=4, dim=D)
    out = ix.k_norm(to_gpu(xb), to_gpu(gb), to_gpu(bb), eps=1e-5)
    torch.cuda.synchronize()
    check(out.view(torch.int16).cpu().numpy().view(np.uint16), xb, gb, bb, 1e-5)


def test_k_norm_in_place_and_constant_rows(dsai):
    rng = np.random.default_rng(3)
    xb, gb, bb = make(rng, 300, 128)
    xb[5] = xb[5, 0]           # a constant row: the output is beta exactly
    x = to_gpu(xb)
    ix = dsai.Indexer(heads=4, dim=128)
    out = ix.k_norm(x, to_gpu(gb), to_gpu(bb), eps=1e-6, out=x)
    torch.cuda.synchronize()
    assert out.data_ptr() == x.data_ptr()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[5], bb)
    check(got, xb, gb, bb, 1e-6)
