"""dsai_select_expand_static (the entry point for callers that cannot
allocate: its [Q, P] scores live in the library's static device array)
against dsai_select_expand with a caller workspace, through the C ABI.

Two calls in a row on one handle, the second smaller than the first, must
each return the ids, scores and token ids of dsai_select_expand on the same
inputs bit for bit: the array keeps the first call's scores, and the second
call must not read any of them.  The pooled decode workload's own size
(64 rows over 16384 pools, 4 MiB of scores) and a row wider than the block
select's limit (the streaming select, then the expand kernel) are covered,
in both row orders.
"""
import numpy as np
import pytest
import torch

import synthetic as SY

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsai():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import sparse_attention_token_index_amd as m
    m.load_library()
    return m


def _inputs(rng, Q, P, H, D):
    f = lambda shape: torch.from_numpy(
        SY.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32)).view(np.int16)
    ).view(torch.bfloat16).cuda()
    q, pk = f((Q, H, D)), f((max(P, 1), D))[:P]
    w = torch.from_numpy((rng.standard_normal((Q, H)) / np.sqrt(H)).astype(np.float32)).cuda()
    pv = torch.from_numpy((rng.random(P) < 0.92).astype(np.uint8)).cuda()
    return q, w, pk, pv


def _static(ix, q, w, pk, pv):
    Q, K = q.shape[0], ix.select_k
    ids = torch.full((Q, K), -777, dtype=torch.int32, device="cuda")
    sc = torch.full((Q, K), 7.0, dtype=torch.float32, device="cuda")
    tok = torch.full((Q, K * ix.cfg.kpool), -777, dtype=torch.int32, device="cuda")
    return ix.select_expand_static(q, w, pk, pv, ids, sc, tok)


@pytest.mark.parametrize("order", ["score", "index"])
@pytest.mark.parametrize("KP,index_topk,first_key,sizes", [
    (4, 512, 0, [(64, 16384), (5, 3000)]),     # pooled decode size, then smaller
    (2, 256, 3, [(8, 40000), (3, 35001)]),     # streaming select + expand kernel
])
def test_static_matches_workspace_form(dsai, order, KP, index_topk, first_key, sizes):
    H, D = 32, 128
    ix = dsai.Indexer(heads=H, dim=D, kpool=KP, index_topk=index_topk, first_key=first_key,
                      order=dsai.DSAI_ORDER_SCORE if order == "score" else dsai.DSAI_ORDER_INDEX)
    rng = np.random.default_rng(11 + KP)
    for Q, P in sizes:
        print(f"[gpu] select_expand_static Q={Q} P={P} KP={KP} order={order}", flush=True)
        assert Q * P * 4 <= dsai.DSAI_STATIC_SCRATCH_BYTES
        q, w, pk, pv = _inputs(rng, Q, P, H, D)
        ids, sc, tok = ix.select(q, w, pk, pv, expand=True)
        sids, ssc, stok = _static(ix, q, w, pk, pv)
        torch.cuda.synchronize()
        assert np.array_equal(sids.cpu().numpy(), ids.cpu().numpy())
        assert np.array_equal(ssc.cpu().numpy().view(np.uint32), sc.cpu().numpy().view(np.uint32))
        assert np.array_equal(stok.cpu().numpy(), tok.cpu().numpy())


def test_static_refuses_past_its_array(dsai):
    """Q * P * 4 above the array's size is refused before any launch, and
    the outputs stay untouched."""
    ix = dsai.Indexer(heads=32, dim=128, kpool=4, index_topk=512)
    Q = 64
    P = dsai.DSAI_STATIC_SCRATCH_BYTES // (4 * Q) + 1
    rng = np.random.default_rng(5)
    q, w, pk, pv = _inputs(rng, Q, P, 32, 128)
    with pytest.raises(dsai.DsaiError) as e:
        _static(ix, q, w, pk, pv)
    assert e.value.status == -3  # DSAI_ERR_WORKSPACE
