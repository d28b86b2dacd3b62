"""The estimated rank of the filter store's cuts (cut_rank in
csrc/score_topk.hip), checked against its statistical claim on the CPU.

A cut after n of a row's N visible keys keeps kc = k n / N plus six standard
deviations of that count and 32 (at most k).  If key order says nothing
about the scores, the number X of the row's final top k among the first n
keys is hypergeometric (N keys, k marked, n drawn), and a cut loses one of
the final top k only when X > kc.  Results never depend on this (a row that
ends short is recomputed with cuts to k); the rate at which the fast path
holds does."""
import math

import numpy as np
import pytest
from scipy.stats import hypergeom


def cut_rank(k, n, N):
    """The kernel's rule, in float32 arithmetic as on the GPU."""
    if n >= N:
        return k
    f = np.float32(n) / np.float32(N)
    mu = np.float32(k) * f
    m = mu + np.float32(6.0) * np.sqrt(mu * (np.float32(1.0) - f)) + np.float32(32.0)
    return int(m) + 1 if m < np.float32(k) else k


@pytest.mark.parametrize("k", [16, 512, 2048, 8192])
@pytest.mark.parametrize("N", [3000, 8192, 65536, 1 << 20])
def test_cut_loses_top_k_with_negligible_probability(k, N):
    if k >= N:
        pytest.skip("rows with at most k keys are never cut")
    worst = 0.0
    for frac in np.linspace(0.02, 0.98, 49):
        n = max(1, int(frac * N))
        kc = cut_rank(k, n, N)
        assert 1 <= kc <= k
        p = hypergeom.sf(kc, N, k, n)   # P(X > kc)
        worst = max(worst, p)
    assert worst < 1e-9, worst


def test_cut_rank_is_k_once_every_key_is_seen_and_never_above_k():
    for k, N in [(2048, 65536), (512, 4096), (16, 70000)]:
        assert cut_rank(k, N, N) == k
        assert all(cut_rank(k, n, N) <= k for n in range(1, N, max(1, N // 97)))


def test_cuts_shrink_the_store_on_long_rows():
    """On a 65536-key row with k = 2048 the first cut (about 2.7K keys seen)
    keeps under a tenth of k, so the store fills far more slowly than with
    cuts to k."""
    kc = cut_rank(2048, 2700, 65536)
    assert kc < 205
    assert kc > 2048 * 2700 / 65536   # never below the expected count
    assert math.isclose(cut_rank(2048, 32768, 65536), 1024 + 6 * math.sqrt(512) + 32, abs_tol=2)
