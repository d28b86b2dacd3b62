"""fp64 CPU oracle of the lightning-indexer selection path.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  Plain definitions, no
blocking, fusion or reordering beyond what each definition states.

Sources (the pages this follows, cited by title and section):

* "nemo_automodel.components.models.deepseek_v4.kernels.tilelang_indexer"
  (NeMo AutoModel API page; "V4IndexerFunction" and "v4_lighting_indexer"):
  SBHD tensor contracts - index_q [seqlen, batch, heads, dim] bf16,
  index_k [seqlen_kv, batch, dim] bf16, weights [seqlen, batch, heads] fp32,
  compress_ratio (4 for C4 layers), topk, result [batch, seqlen, topk].
  The module summary says the indexer applies causal masking.
* "Module glm5next_dsa" (metrale API page): "Shape of the pipeline"
  (kpool_compress -> index_scores -> topk_pools -> expand_selection),
  "Checkpoint and kernel facts the code depends on" (slot-axis softmax per
  channel, pooling starts at first_key, a pool counts only if all of its
  slots are valid, expand writes -1 over the row before any index), the
  config invariants (index_topk a nonzero multiple of index_kpool,
  index_kpool at most KERNEL_MAX_KPOOL = 8).

Readings where the pages are silent (each also listed in the design notes):

* Score: I[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . k[s,:]) - ReLU per head,
  then the fp32 per-head weights reduce over heads; no extra scale.
* Causal mask under compression: key s is visible to query t (0-based)
  iff s < n_t = min(Skv, floor((t+1)/r)).
* Top-k order: score descending, lower key index first on equal scores
  (+0.0 and -0.0 are equal); rows with fewer visible keys than topk are
  padded with index -1 and score -inf.
* kpool: logits gate[tok,c] + ape[j,c] for slot j; softmax over the slots
  per channel; pool key = softmax-weighted sum of the slots' k_normed,
  rounded to bf16 (nearest even); pool p covers tokens
  first_key + p*KP ... first_key + p*KP + KP - 1, and P = floor(max(0, N -
  first_key) / KP) so a trailing partial pool is not a pool.
* Pooled scores use the same formula over pool keys, with no causal mask
  (the cache precedes the decode query) and invalid pools excluded;
  select_k = index_topk / KP pools per row, ties to the lower pool id.
* expand: slot i*KP + j of a row holds first_key + p_i*KP + j for the i-th
  selected pool p_i, and -1 where the pool id is -1.
* Backward (V4IndexerFunction.backward(grad_scores, grad_indices)): the
  gradient of the returned scores only (indices are integers); ReLU's
  derivative is taken as 0 at 0; unusable entries (score -inf) get none.
* Packed sequences ("packed-sequence dispatch" among the local modifications
  on the "nemo_automodel.components.models.deepseek_v4.kernels" page, which
  gives it no layout): independent samples laid end to end, each the
  one-sample problem on its own rows and keys (positions and key indices
  local to the sample), split by cumulative offsets cu_q / cu_k.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Unpooled lightning indexer (tilelang_indexer page)
# ---------------------------------------------------------------------------

def visible_keys(t: int, Skv: int, compress_ratio: int) -> int:
    """Number of keys query position t may see: min(Skv, floor((t+1)/r)).

    Causal masking (tilelang_indexer module summary) under the compression
    ratio (v4_lighting_indexer parameter compress_ratio, 4 for C4 layers):
    a compressed key summarises r consecutive tokens, so it is visible once
    all r of them are at or before t.  r = 1 is the plain causal mask s <= t.
    """
    return min(Skv, (t + 1) // compress_ratio)


def _dot_products(q_row: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """[H, n]: q_row [H, D] times keys [n, D] transposed, in fp64."""
    return q_row @ keys.T


def _relu(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0)


def _weighted_head_sum(w_row: np.ndarray, per_head: np.ndarray) -> np.ndarray:
    """sum_h w[h] * per_head[h, :] in fp64 -> [n]."""
    return (w_row[:, None] * per_head).sum(axis=0)


def head_scores(q_row: np.ndarray, keys: np.ndarray, w_row: np.ndarray) -> np.ndarray:
    """Index scores of one query row against `keys`.

    I[s] = sum_h w[h] * ReLU(q[h,:] . k[s,:]): per-head dot products of the
    bf16 index query with each bf16 index key, ReLU per head, then the fp32
    per-head weights reduce over heads (v4_lighting_indexer: index_q, index_k,
    weights [seqlen, batch, heads] fp32).
    q_row [H, D], keys [n, D], w_row [H]; all converted to fp64.
    """
    q64 = np.asarray(q_row, dtype=np.float64)
    k64 = np.asarray(keys, dtype=np.float64).reshape(-1, q64.shape[1])
    w64 = np.asarray(w_row, dtype=np.float64)
    if k64.shape[0] == 0:
        return np.zeros(0, dtype=np.float64)
    return _weighted_head_sum(w64, _relu(_dot_products(q64, k64)))


def rank_desc(scores: np.ndarray) -> np.ndarray:
    """Positions of `scores` ordered by (score descending, position ascending).

    A stable lexicographic sort; +0.0 and -0.0 compare equal.
    """
    scores = np.asarray(scores, dtype=np.float64)
    return np.lexsort((np.arange(scores.shape[0]), -scores))


def select_topk(scores: np.ndarray, topk: int):
    """First `topk` of rank_desc(scores); pad with (-1, -inf).

    Returns (idx int32 [topk], vals float64 [topk]).
    """
    order = rank_desc(scores)[:topk]
    idx = np.full(topk, -1, dtype=np.int32)
    vals = np.full(topk, NEG_INF, dtype=np.float64)
    idx[: order.shape[0]] = order
    vals[: order.shape[0]] = np.asarray(scores, dtype=np.float64)[order]
    return idx, vals


def score_topk(q: np.ndarray, k: np.ndarray, w: np.ndarray, compress_ratio: int, topk: int,
               rows=None, row_values=False):
    """Top-k key indices and scores per query (v4_lighting_indexer forward).

    q [S, B, H, D], k [Skv, B, D], w [S, B, H] (SBHD layout) as float arrays
    holding the bf16 / fp32 input values.  Returns (idx int32 [B, S, topk],
    vals float64 [B, S, topk]).

    If `rows` (a sequence of query positions t) is given, q and w hold only
    those rows, in that order ([len(rows), B, ...]); the result is then
    [B, len(rows), topk].  With `row_values=True` the full score rows are
    also returned (a list over (b, row) of fp64 arrays of length n_t).
    """
    R, B = q.shape[0], q.shape[1]
    Skv = k.shape[0]
    positions = list(range(R)) if rows is None else [int(t) for t in rows]
    assert len(positions) == R
    idx = np.empty((B, R, topk), dtype=np.int32)
    vals = np.empty((B, R, topk), dtype=np.float64)
    full = []
    for b in range(B):
        for i, t in enumerate(positions):
            n_t = visible_keys(t, Skv, compress_ratio)
            s = head_scores(q[i, b], k[:n_t, b], w[i, b])
            idx[b, i], vals[b, i] = select_topk(s, topk)
            if row_values:
                full.append(s)
    if row_values:
        return idx, vals, full
    return idx, vals


def _sequence_spans(cu_q, cu_k):
    """(first row, end row, first key, end key) of each packed sequence."""
    return [(int(cu_q[i]), int(cu_q[i + 1]), int(cu_k[i]), int(cu_k[i + 1]))
            for i in range(len(cu_q) - 1)]


def score_topk_packed(q: np.ndarray, k: np.ndarray, w: np.ndarray, cu_q, cu_k,
                      compress_ratio: int, topk: int, topk_indices=None):
    """Packed sequences: q [Tq, H, D], k [Tk, D], w [Tq, H], and nseq + 1
    cumulative offsets cu_q, cu_k.  Sequence i is the one-sample problem
    (B = 1) on rows cu_q[i]:cu_q[i+1] and keys cu_k[i]:cu_k[i+1], answered by
    score_topk (or scores_at_indices with that sequence's rows of
    topk_indices [Tq, topk], indices local to the sequence); the rows are
    concatenated.  Returns (idx int32 [Tq, topk], vals float64 [Tq, topk])."""
    Tq = q.shape[0]
    idx = np.empty((Tq, topk), dtype=np.int32)
    vals = np.empty((Tq, topk), dtype=np.float64)
    for q0, q1, k0, k1 in _sequence_spans(cu_q, cu_k):
        if q1 == q0:
            continue
        qs, ks, ws = q[q0:q1, None], k[k0:k1, None], w[q0:q1, None]
        if topk_indices is None:
            oi, ov = score_topk(qs, ks, ws, compress_ratio, topk)
        else:
            oi, ov = scores_at_indices(qs, ks, ws, compress_ratio, topk_indices[None, q0:q1])
        idx[q0:q1], vals[q0:q1] = oi[0], ov[0]
    return idx, vals


def indexer_backward_packed(q: np.ndarray, k: np.ndarray, w: np.ndarray, cu_q, cu_k,
                            compress_ratio: int, topk_indices: np.ndarray,
                            grad_scores: np.ndarray):
    """Gradients of the selected scores for packed sequences (the reading of
    score_topk_packed): q [Tq, H, D], k [Tk, D], w [Tq, H], topk_indices /
    grad_scores [Tq, n] with key indices local to each sequence.  Sequence
    i's slices get indexer_backward of the one-sample problem on its rows
    and keys; keys of a sequence with no rows get zero.  Returns a dict with
    grad_q [Tq, H, D], grad_k [Tk, D], grad_w [Tq, H]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    out = {"grad_q": np.zeros(q.shape), "grad_k": np.zeros(k.shape), "grad_w": np.zeros(w.shape)}
    for q0, q1, k0, k1 in _sequence_spans(cu_q, cu_k):
        if q1 == q0 or k1 == k0:
            continue
        r = indexer_backward(q[q0:q1, None], k[k0:k1, None], w[q0:q1, None], compress_ratio,
                             np.asarray(topk_indices)[None, q0:q1],
                             np.asarray(grad_scores, dtype=np.float64)[None, q0:q1])
        out["grad_q"][q0:q1] = r["grad_q"][:, 0]
        out["grad_k"][k0:k1] = r["grad_k"][:, 0]
        out["grad_w"][q0:q1] = r["grad_w"][:, 0]
    return out


def _usable_keys(s: np.ndarray, n_t: int) -> np.ndarray:
    """Supplied key indices that name a key the row may see: 0 <= s < n_t."""
    return (s >= 0) & (s < n_t)


def scores_at_indices(q: np.ndarray, k: np.ndarray, w: np.ndarray, compress_ratio: int,
                      topk_indices: np.ndarray, rows=None):
    """Index scores at supplied key indices (v4_lighting_indexer with its
    optional topk_indices [batch, seqlen, topk] int32, and
    pytorch_extract_topk_scores: the scores gathered at given indices along
    the key axis).

    q [R, B, H, D], k [Skv, B, D], w [R, B, H] as in score_topk (with `rows`
    the query positions of q's R rows, else 0..R-1); topk_indices [B, R, n]
    integers.  Entry s of row (b, t) is usable when 0 <= s < n_t, the row's
    causal/compressed bound: the result there is (s, I[t, s]).  Any other
    entry (-1 padding, a masked or an out-of-range key) gives (-1, -inf).
    Entries keep the supplied order; duplicates are scored each time.
    Returns (idx int32 [B, R, n], vals float64 [B, R, n]).
    """
    R, B = q.shape[0], q.shape[1]
    Skv = k.shape[0]
    positions = list(range(R)) if rows is None else [int(t) for t in rows]
    assert len(positions) == R
    sup = np.asarray(topk_indices)
    n = sup.shape[2]
    idx = np.full((B, R, n), -1, dtype=np.int32)
    vals = np.full((B, R, n), NEG_INF, dtype=np.float64)
    for b in range(B):
        for i, t in enumerate(positions):
            n_t = visible_keys(t, Skv, compress_ratio)
            s = sup[b, i].astype(np.int64)
            ok = _usable_keys(s, n_t)
            if np.any(ok):
                vals[b, i, ok] = head_scores(q[i, b], k[s[ok], b], w[i, b])
                idx[b, i, ok] = s[ok]
    return idx, vals


def _pair_dots(qp: np.ndarray, kp: np.ndarray) -> np.ndarray:
    """Per entry p and head h: d[p, h] = q_p[h, :] . k_p[:] (qp [P, H, D], kp [P, D])."""
    return np.einsum("phd,pd->ph", qp, kp)


def _gate_coef(g: np.ndarray, wp: np.ndarray, on: np.ndarray) -> np.ndarray:
    """dI/dd_h times the incoming gradient: g[p] * w[p, h] * gate[p, h]."""
    return g[:, None] * wp * on


def _relu_gate(d: np.ndarray) -> np.ndarray:
    """Derivative of ReLU used by the backward: 1 where d > 0, else 0 (the
    subgradient 0 at d == 0)."""
    return (d > 0).astype(np.float64)


def _usable_entries(sup: np.ndarray, positions, Skv: int, compress_ratio: int, keys=None):
    """(b, i, j, s) of every usable entry of supplied indices sup [B, R, n]:
    row i of the batch-b block holds query position positions[i], and entry
    j names key s with 0 <= s < n_t (optionally also s in `keys`)."""
    B, R, n = sup.shape
    n_t = np.array([visible_keys(t, Skv, compress_ratio) for t in positions], dtype=np.int64)
    s = sup.astype(np.int64)
    ok = _usable_keys(s, n_t[None, :, None])
    if keys is not None:
        ok &= np.isin(s, np.asarray(list(keys), dtype=np.int64))
    b, i, j = np.nonzero(ok)
    return b, i, j, s[b, i, j]


def indexer_backward(q: np.ndarray, k: np.ndarray, w: np.ndarray, compress_ratio: int,
                     topk_indices: np.ndarray, grad_scores: np.ndarray, rows=None, keys=None,
                     with_bounds=False, chunk=512):
    """Gradients of the selected index scores (V4IndexerFunction.backward,
    whose inputs are grad_scores [batch, seqlen, topk] and grad_indices; the
    returned indices are integers and carry no gradient, so only grad_scores
    flows back).

    The forward value of usable entry j of row (b, t), key s = idx[b, t, j],
    is I = sum_h w[t,b,h] * ReLU(d_h) with d_h = q[t,b,h,:] . k[s,b,:]; an
    unusable entry (-1, masked or out of range) is the constant -inf and has
    no gradient.  With g = grad_scores[b, t, j] each usable entry adds

      grad_w[t,b,h]   += g * ReLU(d_h)
      grad_q[t,b,h,:] += g * w[t,b,h] * [d_h > 0] * k[s,b,:]
      grad_k[s,b,:]   += g * sum_h w[t,b,h] * [d_h > 0] * q[t,b,h,:]

    Repeated entries add once each.  q [R, B, H, D], k [Skv, B, D], w [R, B, H],
    topk_indices / grad_scores [B, R, n]; `rows` lists the query positions of
    the R rows (else 0..R-1).  `keys` restricts the sums to entries naming
    those keys: then only grad_k at those key rows is complete.  fp64 on the
    given values.

    Returns a dict with grad_q, grad_k, grad_w; with_bounds=True adds, per
    element, the sum of absolute values of its terms (abs_q, abs_k: the
    products above; abs_w: |g| * sum_d |q_d k_d|), the number of terms summed
    into each key row (count_k), and band_q / band_k: the absolute terms whose
    gate is undecided in fp32 arithmetic, |d_h| <= D * 2^-24 * sum_d |q_d k_d|.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    g_all = np.asarray(grad_scores, dtype=np.float64)
    R, B, H, D = q.shape
    Skv = k.shape[0]
    positions = list(range(R)) if rows is None else [int(t) for t in rows]
    assert len(positions) == R
    b_e, i_e, j_e, s_e = _usable_entries(np.asarray(topk_indices), positions, Skv,
                                         compress_ratio, keys)
    out = {"grad_q": np.zeros((R, B, H, D)), "grad_k": np.zeros((Skv, B, D)),
           "grad_w": np.zeros((R, B, H))}
    if with_bounds:
        for name, shape in (("abs_q", (R, B, H, D)), ("band_q", (R, B, H, D)),
                            ("abs_k", (Skv, B, D)), ("band_k", (Skv, B, D)),
                            ("abs_w", (R, B, H))):
            out[name] = np.zeros(shape)
        out["count_k"] = np.zeros((Skv, B), dtype=np.int64)
    for c0 in range(0, b_e.shape[0], chunk):
        b, i, s = b_e[c0:c0 + chunk], i_e[c0:c0 + chunk], s_e[c0:c0 + chunk]
        g = g_all[b, i, j_e[c0:c0 + chunk]]                      # [P]
        qp = q[i, b]                                             # [P, H, D]
        kp = k[s, b]                                             # [P, D]
        wp = w[i, b]                                             # [P, H]
        d = _pair_dots(qp, kp)                                   # [P, H]
        on = _relu_gate(d)
        np.add.at(out["grad_w"], (i, b), g[:, None] * _relu(d))
        coef = _gate_coef(g, wp, on)                             # [P, H]
        np.add.at(out["grad_q"], (i, b), coef[:, :, None] * kp[:, None, :])
        np.add.at(out["grad_k"], (s, b), np.einsum("ph,phd->pd", coef, qp))
        if with_bounds:
            mag = np.einsum("phd,pd->ph", np.abs(qp), np.abs(kp))  # sum_d |q_d k_d|
            undecided = np.abs(d) <= D * 2.0 ** -24 * mag
            acoef = np.abs(g[:, None] * wp)
            np.add.at(out["abs_w"], (i, b), np.abs(g)[:, None] * mag)
            np.add.at(out["abs_q"], (i, b), (acoef * on)[:, :, None] * np.abs(kp)[:, None, :])
            np.add.at(out["band_q"], (i, b),
                      (acoef * undecided)[:, :, None] * np.abs(kp)[:, None, :])
            np.add.at(out["abs_k"], (s, b), np.einsum("ph,phd->pd", acoef * on, np.abs(qp)))
            np.add.at(out["band_k"], (s, b), np.einsum("ph,phd->pd", acoef * undecided, np.abs(qp)))
            np.add.at(out["count_k"], (s, b), 1)
    return out


# ---------------------------------------------------------------------------
# Pooled decode selection (glm5next_dsa page)
# ---------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray):
    """Round fp64 values to bf16, nearest with ties to even, directly.

    bf16 keeps 8 significant bits.  Writing x = m * 2**e with 0.5 <= |m| < 1,
    the rounded value is rint(m * 256) * 2**(e - 8), where rint rounds half
    to even and every step is exact in fp64 (no double rounding through
    fp32).  Returns (values fp64, bits uint16).  Inputs are finite and far
    from the bf16 subnormal range.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return r, bits


def _row_moments(x: np.ndarray):
    """Per-row mean and biased variance (divide by the row length) of [N, D]."""
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    return mu, var


def _inv_std(var: np.ndarray, eps: float) -> np.ndarray:
    """1 / sqrt(var + eps): eps inside the square root."""
    return 1.0 / np.sqrt(var + eps)


def k_norm(k_raw: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float):
    """The indexer's k_norm, the producer of the cache's k_normed rows
    (glm5next_dsa: "indexer.k_norm is a LayerNorm with a bias"; the BF16
    LayerNorm-with-bias module of its Constants).  Per row n of [N, D]:

      mu = mean_c x[n, c],  var = mean_c (x[n, c] - mu)^2   (biased)
      y[n, c] = (x[n, c] - mu) / sqrt(var + eps) * gamma[c] + beta[c]

    rounded to bf16 (nearest even).  k_raw [N, D] bf16 values, gamma / beta
    [D] bf16 values (the checkpoint's dtype), eps > 0.  Returns dict with
    k_normed_f64 [N, D] (before rounding), k_normed (bf16 values as fp64) and
    k_normed_bits uint16.
    """
    x = np.asarray(k_raw, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    b = np.asarray(beta, dtype=np.float64)
    mu, var = _row_moments(x)
    y = (x - mu) * _inv_std(var, float(eps)) * g[None, :] + b[None, :]
    rv, rb = round_to_bf16(y)
    return {"k_normed_f64": y, "k_normed": rv, "k_normed_bits": rb}


def _slot_softmax(logits: np.ndarray) -> np.ndarray:
    """Softmax over the pool-slot axis (axis 0) of [KP, D] logits, per channel,
    with the per-channel maximum subtracted first (exact shift invariance)."""
    ex = np.exp(logits - logits.max(axis=0, keepdims=True))
    return ex / ex.sum(axis=0, keepdims=True)


def pool_count(N: int, first_key: int, kpool: int) -> int:
    """P = floor(max(0, N - first_key) / KP): pooling starts at first_key and a
    trailing partial pool is not a pool (glm5next_dsa, kernel facts)."""
    return max(0, N - first_key) // kpool


def kpool_compress(k_normed: np.ndarray, gate: np.ndarray, valid: np.ndarray,
                   ape: np.ndarray, first_key: int, kpool: int):
    """Compress index keys into pool keys (glm5next_dsa: kpool_compress).

    For pool p (tokens tok_j = first_key + p*KP + j, j < KP) and channel c:
      logits lg_j = gate[tok_j, c] + ape[j, c]
      a_j = softmax over the slot axis j of lg (per channel)
      pool_k[p, c] = bf16( sum_j a_j * k_normed[tok_j, c] )
    pool_valid[p] = all(valid[tok_j]);  pool_tok[p] = tok_0.

    k_normed [N, D] (bf16 values), gate [N, D] fp32, valid [N] (0/1),
    ape [KP, D] fp32.  Returns dict with pool_k_f64 [P, D] (before rounding),
    pool_k [P, D] (bf16 values as fp64), pool_k_bits [P, D] uint16,
    pool_tok [P] int32, pool_valid [P] uint8.
    """
    N, D = k_normed.shape
    KP = kpool
    P = pool_count(N, first_key, KP)
    kn = np.asarray(k_normed, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    a = np.asarray(ape, dtype=np.float64)
    pk = np.empty((P, D), dtype=np.float64)
    pv = np.empty(P, dtype=np.uint8)
    pt = np.empty(P, dtype=np.int32)
    for p in range(P):
        toks = first_key + p * KP + np.arange(KP)
        lg = g[toks, :] + a[:KP, :]      # [KP, D] slot logits
        wts = _slot_softmax(lg)
        pk[p] = (wts * kn[toks, :]).sum(axis=0)
        pv[p] = 1 if np.all(np.asarray(valid)[toks] != 0) else 0
        pt[p] = toks[0]
    rv, rb = round_to_bf16(pk)
    return {"pool_k_f64": pk, "pool_k": rv, "pool_k_bits": rb,
            "pool_tok": pt, "pool_valid": pv}


def visible_pools(P: int, limit) -> np.ndarray:
    """Pools a decode row may select under a per-row visible-pool bound:
    p < limit, the bound clamped to [0, P] (None: every pool).  Reading for
    multi-token decode, where rows of one step sit at different positions:
    the "Module glm5next_dsa" page has index_scores return [Q, P] scores
    plus candidate validity, and its topk_pools select from valid
    candidates; a row's bound makes the pools at or past it invalid
    candidates for that row only."""
    if limit is None:
        return np.ones(P, dtype=bool)
    lim = min(max(int(limit), 0), P)
    return np.arange(P) < lim


def pooled_index_scores(q: np.ndarray, w: np.ndarray, pool_k: np.ndarray,
                        pool_valid: np.ndarray, pool_limit=None) -> np.ndarray:
    """[Q, P] scores of decode queries against pool keys (glm5next_dsa: index_scores).

    S[q, p] = sum_h w[q, h] * ReLU(q[q, h, :] . pool_k[p, :]) for valid pools;
    -inf marks an invalid candidate.  No causal mask.  With pool_limit
    ([Q] ints), row i's pools at or past pool_limit[i] are invalid
    candidates too (visible_pools).
    q [Q, H, D], w [Q, H], pool_k [P, D], pool_valid [P].
    """
    Q = q.shape[0]
    P = pool_k.shape[0]
    out = np.empty((Q, P), dtype=np.float64)
    for i in range(Q):
        out[i] = head_scores(q[i], pool_k, w[i])
        out[i, ~visible_pools(P, None if pool_limit is None else pool_limit[i])] = NEG_INF
    out[:, np.asarray(pool_valid) == 0] = NEG_INF
    return out


def topk_pools(scores: np.ndarray, select_k: int):
    """Keep select_k pool ids per row (glm5next_dsa: topk_pools).

    Valid pools (score > -inf) ranked by (score desc, pool id asc); rows with
    fewer valid pools are padded with (-1, -inf).  Returns (ids int32
    [Q, select_k], vals float64 [Q, select_k]).
    """
    Q = scores.shape[0]
    ids = np.full((Q, select_k), -1, dtype=np.int32)
    vals = np.full((Q, select_k), NEG_INF, dtype=np.float64)
    for i in range(Q):
        cand = np.nonzero(np.isfinite(scores[i]))[0]
        order = cand[rank_desc(scores[i][cand])][:select_k]
        ids[i, : order.shape[0]] = order
        vals[i, : order.shape[0]] = scores[i][order]
    return ids, vals


def expand_selection(pool_ids: np.ndarray, first_key: int, kpool: int) -> np.ndarray:
    """Pool ids -> token ids (glm5next_dsa: expand_selection).

    The row is first filled with -1 (every slot written); then for each
    selected pool p_i != -1, slots i*KP + j receive first_key + p_i*KP + j.
    pool_ids [Q, select_k] -> [Q, select_k * KP] int32.
    """
    Q, K = pool_ids.shape
    out = np.full((Q, K * kpool), -1, dtype=np.int32)
    for q in range(Q):
        for i in range(K):
            p = int(pool_ids[q, i])
            if p != -1:
                for j in range(kpool):
                    out[q, i * kpool + j] = first_key + p * kpool + j
    return out
