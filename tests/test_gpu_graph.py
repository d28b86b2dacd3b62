"""GPU checks that the single-stream calls can be captured in a HIP graph
(torch.cuda.graph) and replayed: the pooled decode pipeline
(kpool_compress -> select -> expand, and select with expand in one call),
the cache write's k_norm, and the fused score + top-k with its row sort.  Every replay, with eager work and
synchronisations between replays, must reproduce the eager results bit for
bit.  (No call here clears memory with hipMemsetAsync, which graphs do not
replay reliably on this hardware.)"""
import numpy as np
import pytest
import torch

import synthetic as SY
from parity import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsai():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import sparse_attention_token_index_amd as m
    m.load_library()
    return m


def bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def replay_and_compare(graph, outputs, eager, n=3):
    for rep in range(n):
        for t in outputs:  # stale values the replay must overwrite
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        scratch = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for got, want in zip(outputs, eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), rep


def test_pooled_pipeline_graph(dsai):
    log("[gpu] graph: pooled pipeline")
    pc = SY.PooledCase("graph_pooled", N=8195, D=128, KP=4, first_key=3, H=32, Q=16,
                       index_topk=128)
    pin = SY.pooled_inputs(pc)
    ix = dsai.Indexer(heads=pc.H, dim=pc.D, kpool=pc.KP, index_topk=pc.index_topk,
                      first_key=pc.first_key)
    kn, gate = bf16(pin["k_normed_bits"]), torch.from_numpy(pin["gate"]).cuda()
    valid, ape = torch.from_numpy(pin["valid"]).cuda(), torch.from_numpy(pin["ape"]).cuda()
    q, w = bf16(pin["q_bits"]), torch.from_numpy(pin["w"]).cuda()
    P = ix.pool_count(pc.N)
    K = ix.select_k
    pool_k = torch.empty((P, pc.D), dtype=torch.bfloat16, device="cuda")
    pool_tok = torch.empty((P,), dtype=torch.int32, device="cuda")
    pool_valid = torch.empty((P,), dtype=torch.uint8, device="cuda")
    ws = torch.empty(ix.select_workspace_size(pc.Q, P), dtype=torch.uint8, device="cuda")
    ids = torch.empty((pc.Q, K), dtype=torch.int32, device="cuda")
    sc = torch.empty((pc.Q, K), dtype=torch.float32, device="cuda")
    tok = torch.empty((pc.Q, K * pc.KP), dtype=torch.int32, device="cuda")
    ids2, sc2, tok2 = torch.empty_like(ids), torch.empty_like(sc), torch.empty_like(tok)

    def run():
        ix.kpool_compress(kn, gate, valid, ape, pool_k, pool_tok, pool_valid)
        ix.select(q, w, pool_k, pool_valid, ws, ids, sc)
        ix.expand(ids, tok)
        ix.select(q, w, pool_k, pool_valid, ws, ids2, sc2, tokens=tok2, expand=True)

    outs = [pool_k, pool_tok, pool_valid, ids, sc, tok, ids2, sc2, tok2]
    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    replay_and_compare(g, outs, eager)
    for fused, split in ((ids2, ids), (sc2, sc), (tok2, tok)):  # select with expand = the two calls
        assert torch.equal(fused.view(torch.uint8), split.view(torch.uint8))


def test_score_topk_and_k_norm_graph(dsai):
    log("[gpu] graph: score_topk + sort, k_norm")
    case = SY.IndexerCase("graph_idx", B=2, S=300, Skv=300, H=64, D=128, compress_ratio=1,
                          topk=100, w_var=1 / 64, seed=71)
    inp = SY.indexer_inputs(case)
    q, k, w = bf16(inp["q_bits"]), bf16(inp["k_bits"]), torch.from_numpy(inp["w"]).cuda()
    ix = dsai.Indexer(heads=case.H, dim=case.D)  # score order: fused kernel + row sort
    oi = torch.empty((case.B, case.S, case.topk), dtype=torch.int32, device="cuda")
    os_ = torch.empty((case.B, case.S, case.topk), dtype=torch.float32, device="cuda")
    kraw = bf16(SY.f32_to_bf16_bits(np.random.default_rng(5).standard_normal((777, 128)).astype(np.float32)))
    gamma = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    beta = torch.zeros(128, dtype=torch.bfloat16, device="cuda")
    kn = torch.empty_like(kraw)

    def run():
        ix.score_topk(q, k, w, case.compress_ratio, case.topk, out_idx=oi, out_score=os_)
        ix.k_norm(kraw, gamma, beta, 1e-5, out=kn)

    outs = [oi, os_, kn]
    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    replay_and_compare(g, outs, eager)
