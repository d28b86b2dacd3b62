"""Seeded synthetic inputs for the DSA lightning-indexer selection path.

This module is the only code shared by the HIP path's tests/benchmark and by
the CPU oracle.  It draws random numbers and encodes them in the input
formats (bf16 bit patterns, fp32, bool bytes); it holds none of the method's
arithmetic (no scores, masks, softmax, selection or expansion).

Every tensor is drawn from its own PCG64 stream, keyed by
``SeedSequence([seed, tensor_id, block])``.  Row-major tensors are drawn in
blocks of ``BLOCK`` leading-dimension rows, so any subset of rows (say the
query rows a parity test samples at full size) can be regenerated without
drawing the whole tensor, and the values never depend on which subset was
asked for.

Value distributions follow the workloads described on the pages' sources:
index queries/keys ~ N(0, 1) rounded to bf16 (round-to-nearest-even),
per-head weights fp32 ~ N(0, 1/H) (the second argument of N(.,.) is read as
the variance), and for the pooled decode cache gate ~ N(0, 1) fp32,
valid ~ Bernoulli(0.98) plus an invalid tail, ape ~ N(0, 0.1) fp32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

BLOCK = 1024  # leading-dimension rows per random stream block

# Stream identifiers: one per tensor, fixed forever (changing one changes data).
TID_Q, TID_K, TID_W, TID_HEAVY = 1, 2, 3, 4
TID_KNORM, TID_GATE, TID_VALID, TID_APE, TID_PQ, TID_PW = 5, 6, 7, 8, 9, 10
TID_INT_Q, TID_INT_K, TID_INT_W = 11, 12, 13
TID_KEYS, TID_GRAD = 14, 15


def _stream(seed: int, tid: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, block])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode fp32 values as bf16 bit patterns, rounding to nearest even.

    Inputs are finite by construction, so the uint32 sum cannot wrap.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns to the fp32 values they denote (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rows_blocked(seed, tid, n_rows, row_shape, draw, rows=None, post=None):
    """Draw a [n_rows, *row_shape] tensor block by block; return `rows` of it.

    `post` (optional) encodes each drawn block (e.g. to bf16 bits) so large
    tensors never exist in fp32 all at once."""
    row_elems = int(np.prod(row_shape)) if row_shape else 1
    if rows is None:
        rows = np.arange(n_rows)
    rows = np.asarray(rows, dtype=np.int64)
    out = None
    for blk in np.unique(rows // BLOCK):
        lo = int(blk) * BLOCK
        hi = min(n_rows, lo + BLOCK)
        vals = draw(_stream(seed, tid, int(blk)), (hi - lo) * row_elems)
        vals = vals.reshape((hi - lo,) + tuple(row_shape))
        sel = rows[(rows // BLOCK) == blk]
        if post is not None:
            vals = post(vals[sel - lo])
            sel = np.arange(len(sel)) + lo
        if out is None:
            out = np.empty((len(rows),) + tuple(row_shape), dtype=vals.dtype)
        out[np.nonzero((rows // BLOCK) == blk)[0]] = vals[sel - lo]
    if out is None:  # empty selection
        return np.empty((0,) + tuple(row_shape), dtype=np.uint16 if post else np.float32)
    return out


def _normal(std):
    return lambda g, n: (g.standard_normal(n, dtype=np.float32) * np.float32(std))


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class IndexerCase:
    """Unpooled indexer workload: q [S,B,H,D] bf16, k [Skv,B,D] bf16, w [S,B,H] fp32."""
    name: str
    B: int
    S: int
    Skv: int
    H: int
    D: int
    compress_ratio: int
    topk: int
    w_var: float
    heavy_frac: float = 0.0   # fraction of keys scaled by heavy_scale
    heavy_scale: float = 1.0
    chunk_rows: int = 0       # query rows per launch (0 = whole batch at once)
    seed: int = 0
    integer: bool = False     # small-integer q/k and power-of-two w (exact in fp32)


@dataclasses.dataclass(frozen=True)
class PooledCase:
    """Pooled decode selection over one indexer cache."""
    name: str
    N: int            # cached tokens
    D: int
    KP: int           # index_kpool
    first_key: int
    H: int
    Q: int            # decode query rows
    index_topk: int   # tokens selected per row (select_k = index_topk / KP pools)
    valid_p: float = 0.98
    invalid_tail: int = 37
    ape_var: float = 0.1
    seed: int = 0


CASES = {
    # B=1, S=Skv=256, H=4, D=32, w ~ N(0, 1/H), causal, topk=16.
    "tiny": IndexerCase("tiny", B=1, S=256, Skv=256, H=4, D=32, compress_ratio=1,
                        topk=16, w_var=1.0 / 4),
    # DSA prefill indexer: S=Skv=4096, H=64, D=128, topk=2048.
    "prefill": IndexerCase("prefill", B=1, S=4096, Skv=4096, H=64, D=128,
                           compress_ratio=1, topk=2048, w_var=1.0 / 64),
    # C4 compressed-KV indexer: B=2, S=16384 queries, Skv=4096 keys, ratio 4, topk=512.
    "c4": IndexerCase("c4", B=2, S=16384, Skv=4096, H=64, D=128, compress_ratio=4,
                      topk=512, w_var=1.0 / 64),
    # Long-context stress: S=Skv=65536, 5% of keys x4, topk=2048, 1024-row chunks
    # (chunk_rows bounds the launches of scores at supplied indices; the fused
    # selection forms no score matrix and runs as one launch).
    "long": IndexerCase("long", B=1, S=65536, Skv=65536, H=64, D=128, compress_ratio=1,
                        topk=2048, w_var=1.0 / 64, heavy_frac=0.05, heavy_scale=4.0,
                        chunk_rows=1024),
}

POOLED_CASES = {
    # Pooled decode selection: 64 query rows against a 65536-token cache.
    "pooled_decode": PooledCase("pooled_decode", N=65536, D=128, KP=4, first_key=0,
                                H=32, Q=64, index_topk=512),
}


# ---------------------------------------------------------------------------
# Unpooled indexer inputs
# ---------------------------------------------------------------------------

def indexer_q_bits(case: IndexerCase, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """index_q as bf16 bits, [len(rows) or S, B, H, D] (rows = query positions t)."""
    shape = (case.B, case.H, case.D)
    if case.integer:
        draw = lambda g, n: g.integers(-4, 5, n).astype(np.float32)
        return _rows_blocked(case.seed, TID_INT_Q, case.S, shape, draw, rows, f32_to_bf16_bits)
    return _rows_blocked(case.seed, TID_Q, case.S, shape, _normal(1.0), rows, f32_to_bf16_bits)


def indexer_w(case: IndexerCase, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Per-head weights fp32, [len(rows) or S, B, H]."""
    shape = (case.B, case.H)
    if case.integer:
        choices = np.array([1.0, -1.0, 0.5, -0.5, 0.25, -0.25], dtype=np.float32)
        draw = lambda g, n: choices[g.integers(0, len(choices), n)]
        return _rows_blocked(case.seed, TID_INT_W, case.S, shape, draw, rows)
    return _rows_blocked(case.seed, TID_W, case.S, shape, _normal(np.sqrt(case.w_var)), rows)


def indexer_k_bits(case: IndexerCase) -> np.ndarray:
    """index_k as bf16 bits, [Skv, B, D]; a seeded fraction of keys scaled exactly."""
    shape = (case.B, case.D)
    if case.integer:
        draw = lambda g, n: g.integers(-4, 5, n).astype(np.float32)
        return f32_to_bf16_bits(_rows_blocked(case.seed, TID_INT_K, case.Skv, shape, draw))
    k = _rows_blocked(case.seed, TID_K, case.Skv, shape, _normal(1.0))
    bits = f32_to_bf16_bits(k)
    if case.heavy_frac > 0.0:
        heavy = _rows_blocked(case.seed, TID_HEAVY, case.Skv, (case.B,),
                              lambda g, n: (g.random(n) < case.heavy_frac))
        vals = bf16_bits_to_f32(bits)
        vals[heavy.astype(bool)] *= np.float32(case.heavy_scale)  # power of two: exact
        bits = f32_to_bf16_bits(vals)
    return bits


def heavy_key_mask(case: IndexerCase) -> np.ndarray:
    """[Skv, B] bool: which keys were scaled (for reporting only)."""
    if case.heavy_frac <= 0.0:
        return np.zeros((case.Skv, case.B), dtype=bool)
    return _rows_blocked(case.seed, TID_HEAVY, case.Skv, (case.B,),
                         lambda g, n: (g.random(n) < case.heavy_frac)).astype(bool)


def indexer_inputs(case: IndexerCase, rows: Optional[Sequence[int]] = None) -> dict:
    """q_bits [R,B,H,D] u16, k_bits [Skv,B,D] u16, w [R,B,H] f32 (R = S or len(rows))."""
    return {"q_bits": indexer_q_bits(case, rows), "k_bits": indexer_k_bits(case),
            "w": indexer_w(case, rows)}


# ---------------------------------------------------------------------------
# Pooled decode inputs
# ---------------------------------------------------------------------------

def pooled_inputs(case: PooledCase) -> dict:
    """Indexer cache rows and decode queries for the pooled selection path.

    k_normed [N,D] bf16 bits, gate [N,D] fp32, valid [N] uint8 (0/1),
    ape [KP,D] fp32, q [Q,H,D] bf16 bits, w [Q,H] fp32 ~ N(0, 1/H).
    """
    kn = f32_to_bf16_bits(_rows_blocked(case.seed, TID_KNORM, case.N, (case.D,), _normal(1.0)))
    gate = _rows_blocked(case.seed, TID_GATE, case.N, (case.D,), _normal(1.0))
    valid = _rows_blocked(case.seed, TID_VALID, case.N, (),
                          lambda g, n: (g.random(n) < case.valid_p)).astype(np.uint8)
    if case.invalid_tail > 0:
        valid[max(0, case.N - case.invalid_tail):] = 0
    ape = _rows_blocked(case.seed, TID_APE, case.KP, (case.D,), _normal(np.sqrt(case.ape_var)))
    q = f32_to_bf16_bits(_rows_blocked(case.seed, TID_PQ, case.Q, (case.H, case.D), _normal(1.0)))
    w = _rows_blocked(case.seed, TID_PW, case.Q, (case.H,), _normal(np.sqrt(1.0 / case.H)))
    return {"k_normed_bits": kn, "gate": gate, "valid": valid, "ape": ape,
            "q_bits": q, "w": w}


def random_pool_ids(seed: int, Q: int, select_k: int, P: int, missing_frac: float = 0.1) -> np.ndarray:
    """[Q, select_k] int32 pool ids in [0, P) with a seeded fraction replaced by -1.

    An input generator for testing expand_selection in isolation.
    """
    g = _stream(seed, 99, 0)
    ids = g.integers(0, max(P, 1), (Q, select_k)).astype(np.int32)
    ids[g.random((Q, select_k)) < missing_frac] = -1
    return ids


# ---------------------------------------------------------------------------
# Backward inputs: key lists and incoming gradients of their scores
# ---------------------------------------------------------------------------

def key_lists(seed: int, B: int, R: int, n: int, Skv: int, bound=None) -> np.ndarray:
    """[B, R, n] int32: row r of batch b lists min(n, m) distinct keys drawn
    uniformly from [0, m) in random order, then -1, where m = bound[r]
    (default Skv).  A stand-in for a selection's index rows."""
    out = np.full((B, R, n), -1, dtype=np.int32)
    for b in range(B):
        g = _stream(seed, TID_KEYS, b)
        for r in range(R):
            m = Skv if bound is None else int(bound[r])
            if m <= 0:
                continue
            c = min(n, m)
            out[b, r, :c] = g.permutation(m)[:c]
    return out


def noisy_key_lists(seed: int, B: int, R: int, n: int, Skv: int) -> np.ndarray:
    """[B, R, n] int32 entries uniform in [-2, Skv + 3): padding, out-of-range
    and (for any row bound) masked entries, and repeats."""
    return _rows_blocked(seed, TID_KEYS, B, (R, n),
                         lambda g, k: g.integers(-2, Skv + 3, k).astype(np.int32))


def score_grads(seed: int, B: int, R: int, n: int, integer: bool = False) -> np.ndarray:
    """[B, R, n] fp32 incoming gradients of selected scores: N(0, 1), or
    (integer=True) drawn from {+-1/4, +-1/2, +-1, +-2} so products with
    power-of-two weights stay exact."""
    if integer:
        choices = np.array([0.25, -0.25, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0], dtype=np.float32)
        draw = lambda g, k: choices[g.integers(0, len(choices), k)]
    else:
        draw = _normal(1.0)
    return _rows_blocked(seed, TID_GRAD, B, (R, n), draw)
