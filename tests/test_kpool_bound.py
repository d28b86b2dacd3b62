"""The pool-key tolerance, as evidence rather than prose (CPU only).

The pool-key parity rule lets the GPU's bf16 pool key differ from the
oracle's rounding only where the exact value lies within
E = 2^-18 * max_j |k_normed[tok_j, c]| of a bf16 rounding midpoint.  That
rests on the claim that an fp32 evaluation of the slot softmax and the
weighted sum stays within E of the exact value for KP <= 8.  Here the same
steps the kernel takes (fp32 logits gate + ape, max subtraction, exp, a
running sum of the weights, a running weighted sum, one division) are
evaluated in numpy float32 - with the weighted sum rounded twice per step,
which errs more than the kernel's fused multiply-add - and compared with the
fp64 oracle on the pooled decode cache and on adversarial pools (slots of
opposite sign that cancel, logits far apart, equal logits).
"""
import numpy as np
import pytest

import oracle
import synthetic as SY

E_SCALE = 2.0 ** -18


def fp32_pool_keys(kn, gate, ape, first_key, KP):
    P = oracle.pool_count(kn.shape[0], first_key, KP)
    toks = first_key + np.arange(P)[:, None] * KP + np.arange(KP)[None, :]
    lg = (gate[toks].astype(np.float32) + ape[None, :KP].astype(np.float32)).astype(np.float32)
    kv = kn[toks].astype(np.float32)
    mx = lg.max(axis=1)
    den = np.zeros(mx.shape, dtype=np.float32)
    num = np.zeros(mx.shape, dtype=np.float32)
    for j in range(KP):
        e = np.exp((lg[:, j] - mx).astype(np.float32)).astype(np.float32)
        den = (den + e).astype(np.float32)
        num = (num + (e * kv[:, j]).astype(np.float32)).astype(np.float32)
    return (num / den).astype(np.float32), np.abs(kv).max(axis=1)


def check_bound(kn_bits, gate, ape, first_key, KP):
    kn = SY.bf16_bits_to_f32(kn_bits).astype(np.float64)
    ref = oracle.kpool_compress(kn, gate, np.ones(kn.shape[0], np.uint8), ape, first_key, KP)
    got, mag = fp32_pool_keys(kn, gate, ape, first_key, KP)
    err = np.abs(got.astype(np.float64) - ref["pool_k_f64"])
    bound = E_SCALE * mag
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-300)).max())
    return float((err / np.maximum(bound, 1e-300)).max())


def test_pooled_decode_cache_within_bound():
    pc = SY.POOLED_CASES["pooled_decode"]
    inp = SY.pooled_inputs(pc)
    ratio = check_bound(inp["k_normed_bits"], inp["gate"], inp["ape"], pc.first_key, pc.KP)
    assert ratio < 0.5   # the bound holds with room to spare


@pytest.mark.parametrize("KP", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("kind", ["cancel", "spread", "equal"])
def test_adversarial_pools_within_bound(KP, kind):
    rng = np.random.default_rng(100 + KP)
    N, D = 4096 * KP, 128
    k = rng.standard_normal((N, D)).astype(np.float32)
    if kind == "cancel":        # slot pairs of opposite sign: the result is tiny
        k = k.reshape(-1, KP, D)
        k[:, 1::2] = -k[:, 0::2][:, : k[:, 1::2].shape[1]] * (1 + 2.0 ** -7)
        k = k.reshape(N, D)
        gate = np.zeros((N, D), np.float32)
    elif kind == "spread":      # logits far apart: weights from 1 down to ~e^-60
        gate = (rng.standard_normal((N, D)) * 20).astype(np.float32)
    else:                       # equal logits: the plain slot mean
        gate = np.full((N, D), 3.0, np.float32)
    ape = rng.standard_normal((KP, D)).astype(np.float32) * (0.0 if kind == "equal" else 0.3)
    check_bound(SY.f32_to_bf16_bits(k), gate, ape, 0, KP)
