"""GPU checks of dsai_sort_rows, the score-order pass of the top-k rows.

Input rows are built the way the selection kernels write them in index order
(real entries in ascending index order, padding (-1, -inf) at the tail); the
expected order (score descending, lower index first among equal scores,
padding last) comes from a plain stable sort on the host.  Both code paths of
the kernel are covered: spread-out float scores (bucket path) and rows with
many equal scores (radix path).  All comparisons are exact.
"""
import numpy as np
import pytest
import torch

from parity import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ix():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import sparse_attention_token_index_amd as m
    m.load_library()
    return m.Indexer(heads=4, dim=32)


def make_rows(rng, rows, k, kind):
    idx = np.full((rows, k), -1, np.int32)
    sc = np.full((rows, k), -np.inf, np.float32)
    for r in range(rows):
        nv = k if r % 3 == 0 else int(rng.integers(0, k + 1))
        ids = np.sort(rng.choice(max(4 * k, 16), size=nv, replace=False)).astype(np.int32)
        if kind == "normal":
            v = rng.standard_normal(nv).astype(np.float32) * 8
        elif kind == "ties":
            v = rng.integers(-3, 4, size=nv).astype(np.float32) * 0.25
        elif kind == "equal":
            v = np.full(nv, 1.5, np.float32)
        elif kind == "zeros":
            v = np.where(rng.random(nv) < 0.5, 0.0, -0.0).astype(np.float32)
        elif kind == "wide":
            v = (rng.standard_normal(nv) * 1e37).astype(np.float32)
            if nv >= 2:
                v[0], v[-1] = np.float32(3.4e38), np.float32(-3.4e38)
        elif kind == "clustered":  # one outlier stretches the range; the rest nearly equal
            v = (1.0 + rng.standard_normal(nv) * 1e-6).astype(np.float32)
            if nv:
                v[int(rng.integers(0, nv))] = 1e30
        else:
            raise ValueError(kind)
        idx[r, :nv] = ids
        sc[r, :nv] = v
    return idx, sc


def expected(idx, sc):
    ei, es = np.full_like(idx, -1), np.full_like(sc, -np.inf)
    for r in range(idx.shape[0]):
        real = idx[r] >= 0
        ids, v = idx[r][real], sc[r][real].astype(np.float64)
        v = np.where(v == 0, 0.0, v)  # -0 and +0 are equal scores
        order = np.lexsort((ids, -v))
        n = len(ids)
        ei[r, :n] = ids[order]
        es[r, :n] = v[order]
    return ei, es


@pytest.mark.parametrize("k,kind", [
    (2, "normal"), (64, "normal"), (256, "normal"), (257, "normal"), (512, "normal"),
    (2048, "normal"), (2049, "normal"), (8192, "normal"),
    (512, "ties"), (2048, "ties"), (2048, "equal"), (300, "zeros"), (2048, "wide"),
    (2048, "clustered"), (8192, "ties"),
    # rows of at most 512 entries (one wavefront per row): its tie fallback
    # (a bucket of more than 64 entries) and the range extremes
    (512, "equal"), (100, "equal"), (512, "wide"), (200, "clustered"), (33, "ties"),
    (129, "zeros"), (65, "normal"),
])
def test_sort_rows_matches_stable_host_sort(ix, k, kind):
    rng = np.random.default_rng(1000 + k + len(kind))
    rows = 24 if k <= 2048 else 6
    idx, sc = make_rows(rng, rows, k, kind)
    gi, gs = torch.from_numpy(idx).cuda(), torch.from_numpy(sc).cuda()
    ix.sort_rows(gi, gs)
    torch.cuda.synchronize()
    ei, es = expected(idx, sc)
    got_i, got_s = gi.cpu().numpy(), gs.cpu().numpy()
    for r in range(rows):
        assert np.array_equal(got_i[r], ei[r]), f"k={k} {kind} row {r}: indices differ"
        assert np.array_equal(np.where(got_s[r] == 0, 0.0, got_s[r]), es[r]), \
            f"k={k} {kind} row {r}: scores differ"


def test_sort_rows_is_idempotent_and_k1_is_a_noop(ix):
    rng = np.random.default_rng(7)
    idx, sc = make_rows(rng, 8, 1024, "normal")
    gi, gs = torch.from_numpy(idx).cuda(), torch.from_numpy(sc).cuda()
    ix.sort_rows(gi, gs)
    once = (gi.clone(), gs.clone())
    ix.sort_rows(gi, gs)
    torch.cuda.synchronize()
    assert torch.equal(once[0], gi) and torch.equal(once[1], gs)
    one_i = torch.tensor([[5], [-1]], dtype=torch.int32, device="cuda")
    one_s = torch.tensor([[2.0], [-np.inf]], dtype=torch.float32, device="cuda")
    ix.sort_rows(one_i, one_s)
    torch.cuda.synchronize()
    assert one_i.cpu().tolist() == [[5], [-1]]


@pytest.mark.parametrize("k,rows", [(64, 40001), (512, 20001)])
def test_sort_many_rows(ix, k, rows):
    """More rows than 8 per resident workgroup slot, so each workgroup sorts
    two rows (the second's loads in flight during the first's sort), with an
    odd row count (the last workgroup has one row).  Tied scores, partly
    padded rows and fully padded rows; checked against one host lexsort."""
    log(f"[gpu] sort many rows k={k} rows={rows}")
    rng = np.random.default_rng(31 + k)
    idx = (np.cumsum(rng.integers(1, 5, size=(rows, k)), axis=1) - 1).astype(np.int32)
    sc = (np.round(rng.standard_normal((rows, k)) * 8.0) / 8.0).astype(np.float32) + np.float32(0)
    n = np.full(rows, k)
    short = rng.random(rows) < 0.3
    n[short] = rng.integers(0, k, size=int(short.sum()))
    pad = np.arange(k)[None, :] >= n[:, None]
    idx[pad] = -1
    sc[pad] = -np.inf
    gi, gs = torch.from_numpy(idx).cuda(), torch.from_numpy(sc).cuda()
    ix.sort_rows(gi, gs)
    torch.cuda.synchronize()
    r = np.repeat(np.arange(rows), k)
    order = np.lexsort((idx.ravel(), -sc.ravel().astype(np.float64), r))
    ei, es = idx.ravel()[order].reshape(rows, k), sc.ravel()[order].reshape(rows, k)
    got_i, got_s = gi.cpu().numpy(), gs.cpu().numpy()
    bad = np.flatnonzero(~(got_i == ei).all(axis=1))
    assert bad.size == 0, f"rows {bad[:5]} differ in indices"
    z = np.float32(0)
    assert np.array_equal(np.where(got_s == 0, z, got_s).view(np.uint32),
                          np.where(es == 0, z, es).view(np.uint32))
