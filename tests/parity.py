"""Parity rules between the HIP path and the CPU oracle (helpers for tests).

Rules (scores: abs 1e-3 + rel 1e-3; indices exact wherever the oracle's
ordering is decided by more than that tolerance):

* every output slot is written; rows with fewer visible keys than topk hold
  exactly the visible keys followed by (-1, -inf);
* no duplicate index, none outside the visible range;
* the GPU's reported score of each selected index matches the oracle's
  score of that index within tolerance, and the GPU row is non-increasing;
* if the oracle's k-th and (k+1)-th scores differ by more than the
  tolerance, the selected index SET equals the oracle's; otherwise every
  selected index scores >= s_k - tol and every unselected one <= s_k + tol;
* at each position whose oracle value is separated from both neighbours by
  more than the tolerance, the index equals the oracle's exactly, and at
  every position the selected value is within 2 tol of the oracle's i-th.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

TOL_ABS = 1e-3
TOL_REL = 1e-3


def tol(x):
    return TOL_ABS + TOL_REL * np.abs(x)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_topk_row(gidx: np.ndarray, gsc: np.ndarray, scores: np.ndarray, topk: int,
                   pad_score=-np.inf) -> list:
    """Problems found in one GPU row (empty list = parity)."""
    n = int(scores.shape[0])
    m = min(topk, n)
    errs = []
    if gidx.shape[0] != topk:
        return [f"row length {gidx.shape[0]} != {topk}"]
    if not np.all(gidx[m:] == -1):
        errs.append(f"padding indices {gidx[m:][:8]}")
    if not np.all(gsc[m:] == pad_score):
        errs.append(f"padding scores {gsc[m:][:8]}")
    sel = gidx[:m].astype(np.int64)
    if np.any(sel < 0) or np.any(sel >= n):
        errs.append(f"index outside [0,{n}): {sel[(sel < 0) | (sel >= n)][:8]}")
        return errs
    if np.unique(sel).shape[0] != m:
        errs.append("duplicate indices")
    ref = scores[sel]
    bad = np.abs(gsc[:m].astype(np.float64) - ref) > tol(ref)
    if np.any(bad):
        i = int(np.argmax(bad))
        errs.append(f"score[{i}] idx {sel[i]}: gpu {gsc[i]!r} oracle {ref[i]!r}")
    if m > 1 and np.any(gsc[: m - 1] < gsc[1:m]):
        errs.append("GPU row not non-increasing")
    order = oracle.rank_desc(scores)
    if n <= topk:
        if set(sel.tolist()) != set(range(n)):
            errs.append("row with n <= topk does not hold every visible key")
    else:
        sk, sk1 = scores[order[topk - 1]], scores[order[topk]]
        if sk - sk1 > tol(sk):
            if set(sel.tolist()) != set(order[:topk].tolist()):
                errs.append(f"selected set differs (gap {sk - sk1:.3g})")
        else:
            rest = np.setdiff1d(np.arange(n), sel)
            if ref.min() < sk - tol(sk) or scores[rest].max() > sk + tol(sk):
                errs.append("near-tie boundary rule violated")
    os_ = scores[order[:m]]
    nxt = np.append(os_[1:], scores[order[m]] if n > m else -np.inf)
    prv = np.insert(os_[:-1], 0, np.inf)
    isolated = ((prv - os_) > tol(os_)) & ((os_ - nxt) > tol(os_))
    if np.any(gidx[:m][isolated] != order[:m][isolated]):
        i = int(np.argmax(gidx[:m][isolated] != order[:m][isolated]))
        errs.append(f"isolated position {np.nonzero(isolated)[0][i]} index differs")
    if np.any(np.abs(ref - os_) > 2 * tol(os_)):
        errs.append("i-th selected value far from oracle's i-th value")
    return errs


def check_topk_rows(gidx: np.ndarray, gsc: np.ndarray, rows_scores, topk: int, labels,
                    max_report=5):
    """Check many rows; raise AssertionError listing the first failures."""
    fails = []
    for i, (s, lab) in enumerate(zip(rows_scores, labels)):
        e = check_topk_row(gidx[i], gsc[i], s, topk)
        if e:
            fails.append(f"{lab}: {'; '.join(e)}")
            if len(fails) >= max_report:
                break
    assert not fails, "parity failures:\n" + "\n".join(fails)
