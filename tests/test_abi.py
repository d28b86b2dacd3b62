"""Host-side checks of the C ABI (CPU only: no compute call reaches the GPU).

The library must load, export every entry point include/dsai.h declares, and
refuse bad configurations and arguments with the documented status codes
before any HIP call is made.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsai.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, NULLPTR = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def lib():
    import sparse_attention_token_index_amd as dsai
    if not os.path.exists(dsai.library_path()):
        import sparse_attention_token_index_amd.build as b
        b.build()
    return dsai.load_library()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsai_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    import sparse_attention_token_index_amd as dsai
    assert declared_symbols() == sorted(dsai.EXPORTS)


def test_config_struct_matches_the_header():
    """The binding's ctypes mirror of dsai_config has the header's int
    fields, in the header's order."""
    import sparse_attention_token_index_amd as dsai
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct dsai_config \{(.*?)\} dsai_config;", text, re.S).group(1)
    fields = re.findall(r"\bint\s+([a-z_]+)\s*;", body)
    assert fields == [f for f, _ in dsai._Config._fields_]
    assert all(t is ctypes.c_int for _, t in dsai._Config._fields_)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_exports_are_c_symbols():
    import subprocess
    import sparse_attention_token_index_amd as dsai
    out = subprocess.run(["nm", "-D", "--defined-only", dsai.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dsai_[a-z_]+)\b", out))
    assert set(declared_symbols()) <= exported


def _cfg(heads=64, dim=128, kpool=4, index_topk=512, first_key=0, chunk_rows=0, order=0, cuts=0):
    import sparse_attention_token_index_amd as dsai
    return dsai._Config(heads, dim, kpool, index_topk, first_key, chunk_rows, order, cuts)


def _create(lib, **kw):
    h = ctypes.c_void_p()
    st = lib.dsai_create(ctypes.byref(_cfg(**kw)), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    ({}, OK),
    ({"heads": 4, "dim": 32, "kpool": 1, "index_topk": 1}, OK),
    ({"kpool": 8, "index_topk": 8}, OK),
    ({"kpool": 0}, INVALID),
    ({"kpool": 9, "index_topk": 18}, INVALID),            # above KERNEL_MAX_KPOOL: refused
    ({"kpool": 4, "index_topk": 510}, INVALID),           # not a multiple of kpool
    ({"kpool": 4, "index_topk": 0}, INVALID),             # zero is not allowed
    ({"kpool": 1, "index_topk": 8193}, INVALID),          # select_k above the max
    ({"heads": 0}, INVALID),
    ({"first_key": -1}, INVALID),
    ({"chunk_rows": -5}, INVALID),
    ({"order": 1}, OK),
    ({"order": 2}, INVALID),
    ({"order": -1}, INVALID),
    ({"cuts": 1}, OK),
    ({"cuts": 2}, INVALID),
    ({"cuts": -1}, INVALID),
    ({"heads": 65}, UNSUPPORTED),
    ({"dim": 96}, UNSUPPORTED),
    ({"dim": 256}, UNSUPPORTED),
])
def test_create_validation(lib, kw, status):
    st, h = _create(lib, **kw)
    assert st == status
    if st == OK:
        assert h.value
        assert lib.dsai_destroy(h) == OK
    else:
        assert not h.value


def test_create_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.dsai_create(None, ctypes.byref(h)) == NULLPTR
    assert lib.dsai_create(ctypes.byref(_cfg()), None) == NULLPTR
    assert lib.dsai_destroy(None) == OK


def test_status_strings(lib):
    for st in (OK, INVALID, UNSUPPORTED, WORKSPACE, NULLPTR, -5, 42):
        assert isinstance(lib.dsai_status_string(st), bytes)


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def test_score_topk_argument_errors(lib):
    st, h = _create(lib)
    assert st == OK
    call = lambda S=8, Skv=8, B=1, r=1, topk=4, tki=None, q=FAKE, k=FAKE, w=FAKE, oi=FAKE, os_=FAKE: \
        lib.dsai_score_topk(h, q, k, w, S, Skv, B, r, topk, tki, oi, os_, None)
    assert call(S=-1) == INVALID
    assert call(Skv=-1) == INVALID
    assert call(B=-1) == INVALID
    assert call(r=0) == INVALID
    assert call(topk=0) == INVALID
    assert call(topk=8193) == INVALID
    assert call(S=2 ** 31) == INVALID
    # supplied indices: the same argument rules, plus an aligned index array
    assert call(tki=FAKE, S=0) == OK
    assert call(tki=FAKE, q=None) == NULLPTR
    assert call(tki=FAKE, k=None) == NULLPTR
    assert call(tki=FAKE, oi=None) == NULLPTR
    assert call(tki=ctypes.c_void_p(0x10004)) == INVALID  # misaligned index array
    assert call(tki=FAKE, topk=0) == INVALID
    assert call(S=0) == OK                        # empty: nothing launched
    assert call(B=0) == OK
    assert call(q=None) == NULLPTR
    assert call(w=None) == NULLPTR
    assert call(oi=None) == NULLPTR
    assert call(os_=None) == NULLPTR
    assert call(k=None) == NULLPTR                # Skv > 0 needs keys
    assert call(q=ctypes.c_void_p(0x10002)) == INVALID  # misaligned
    assert lib.dsai_score_topk(None, FAKE, FAKE, FAKE, 8, 8, 1, 1, 4, None, FAKE, FAKE, None) == NULLPTR
    lib.dsai_destroy(h)


def test_score_topk_packed_argument_errors(lib):
    st, h = _create(lib)
    assert st == OK
    offs = lambda *v: (ctypes.c_int64 * len(v))(*v)

    def call(n=2, cq=None, ck=None, r=1, topk=4, tki=None, q=FAKE, k=FAKE, w=FAKE, oi=FAKE,
             os_=FAKE):
        cq = offs(0, 3, 8) if cq is None else cq
        ck = offs(0, 5, 9) if ck is None else ck
        return lib.dsai_score_topk_packed(h, q, k, w, n, cq, ck, r, topk, tki, oi, os_, None)
    assert call(n=-1) == INVALID
    assert call(r=0) == INVALID
    assert call(topk=0) == INVALID
    assert call(topk=6) == INVALID                          # not a multiple of 4
    assert call(topk=8196) == INVALID
    assert call(n=0) == OK                                  # no sequence: nothing launched
    assert lib.dsai_score_topk_packed(h, FAKE, FAKE, FAKE, 2, None, offs(0, 5, 9), 1, 4, None,
                                      FAKE, FAKE, None) == NULLPTR
    assert call(cq=offs(1, 3, 8)) == INVALID                # offsets start at 0
    assert call(ck=offs(0, 5, 4)) == INVALID                # and never decrease
    assert call(cq=offs(0, 0, 2 ** 31)) == INVALID
    assert call(cq=offs(0, 0, 0)) == OK                     # every sequence empty
    assert call(q=None) == NULLPTR
    assert call(w=None) == NULLPTR
    assert call(oi=None) == NULLPTR
    assert call(os_=None) == NULLPTR
    assert call(k=None) == NULLPTR                          # keys present, pointer missing
    assert call(q=ctypes.c_void_p(0x10002)) == INVALID      # misaligned, refused before any HIP call
    assert call(oi=ctypes.c_void_p(0x10004)) == INVALID
    assert lib.dsai_score_topk_packed(None, FAKE, FAKE, FAKE, 2, offs(0, 3, 8), offs(0, 5, 9),
                                      1, 4, None, FAKE, FAKE, None) == NULLPTR
    lib.dsai_destroy(h)


def test_backward_packed_argument_errors(lib):
    st, h = _create(lib)
    assert st == OK
    offs = lambda *v: (ctypes.c_int64 * len(v))(*v)
    cq, ck = offs(0, 40, 100), offs(0, 64, 300)
    need = ctypes.c_size_t()
    assert lib.dsai_backward_packed_workspace_size(h, 2, cq, ck, 8, 1, ctypes.byref(need)) == OK
    single = [ctypes.c_size_t(), ctypes.c_size_t()]
    assert lib.dsai_backward_workspace_size(h, 40, 64, 1, 8, 1, ctypes.byref(single[0])) == OK
    assert lib.dsai_backward_workspace_size(h, 60, 236, 1, 8, 1, ctypes.byref(single[1])) == OK
    assert need.value == max(s.value for s in single)       # the largest sequence's need
    assert lib.dsai_backward_packed_workspace_size(h, 2, cq, ck, 0, 1, ctypes.byref(need)) == INVALID
    assert lib.dsai_backward_packed_workspace_size(h, 2, None, ck, 8, 1, ctypes.byref(need)) == NULLPTR
    ws_ok = need.value

    def call(n=2, cq=cq, ck=ck, r=1, topk=8, ws=FAKE, wsb=None, q=FAKE, k=FAKE, w=FAKE, sup=FAKE,
             g=FAKE, gq=FAKE, gk=FAKE, gw=FAKE):
        return lib.dsai_indexer_backward_packed(h, q, k, w, sup, g, n, cq, ck, r, topk, gq, gk, gw,
                                                ws, ws_ok if wsb is None else wsb, None)
    assert call(r=0) == INVALID
    assert call(topk=0) == INVALID
    assert call(n=-1) == INVALID
    assert call(cq=offs(0, 50, 40)) == INVALID
    assert call(cq=None) == NULLPTR
    assert call(n=0) == OK
    assert call(cq=offs(0, 0, 0), ck=offs(0, 0, 0)) == OK   # nothing to do
    assert call(wsb=ws_ok - 1) == WORKSPACE
    assert call(ws=ctypes.c_void_p(0x10010)) == WORKSPACE    # not 256-byte aligned
    assert call(ws=None) == WORKSPACE
    assert call(k=None) == NULLPTR
    assert call(gk=None) == NULLPTR
    assert call(sup=None) == NULLPTR
    assert call(gq=None) == NULLPTR
    assert call(q=ctypes.c_void_p(0x10002)) == INVALID
    lib.dsai_destroy(h)


def test_k_norm_argument_errors(lib):
    st, h = _create(lib)
    assert st == OK
    f = lib.dsai_k_norm
    f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_float, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p]
    call = lambda N=8, eps=1e-5, x=FAKE, g=FAKE, b=FAKE, y=FAKE: f(h, x, g, b, eps, N, y, None)
    assert call(N=-1) == INVALID
    assert call(eps=0.0) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(eps=float("inf")) == INVALID
    assert call(N=0) == OK                       # nothing launched
    assert call(x=None) == NULLPTR
    assert call(g=None) == NULLPTR
    assert call(b=None) == NULLPTR
    assert call(y=None) == NULLPTR
    assert call(y=ctypes.c_void_p(0x10008)) == INVALID  # misaligned
    assert f(None, FAKE, FAKE, FAKE, 1e-5, 8, FAKE, None) == NULLPTR
    lib.dsai_destroy(h)


def test_backward_argument_errors(lib):
    """Every check of dsai_indexer_backward returns before any HIP call."""
    st, h = _create(lib, heads=64, dim=128)
    assert st == OK
    n = ctypes.c_size_t()
    # dense selection (half the visible keys): grouped by key block, so the
    # accumulator + bucket bounds (2 blocks + 1 per row) + bucketed entries
    assert lib.dsai_backward_workspace_size(h, 512, 512, 2, 256, 1, ctypes.byref(n)) == OK
    assert n.value == 512 * 2 * 128 * 4 + 2 * 512 * 3 * 4 + 2 * 512 * 256 * 8
    # sparse selection (4 of up to 4096 keys): per-entry scatter, accumulator only
    assert lib.dsai_backward_workspace_size(h, 8, 4096, 2, 4, 1, ctypes.byref(n)) == OK
    assert n.value == 4096 * 2 * 128 * 4
    ws_ok = n.value
    # past 1024 key blocks: the accumulator only (per-entry atomic scatter)
    assert lib.dsai_backward_workspace_size(h, 8, 300000, 1, 4, 1, ctypes.byref(n)) == OK
    assert n.value == 300000 * 128 * 4
    for args in ((-1, 4096, 2, 4, 1), (8, -1, 2, 4, 1), (8, 4096, -1, 4, 1), (8, 4096, 2, 0, 1),
                 (8, 4096, 2, 8193, 1), (8, 4096, 2, 4, 0)):
        assert lib.dsai_backward_workspace_size(h, *args, ctypes.byref(n)) == INVALID, args
    assert lib.dsai_backward_workspace_size(h, 8, 4, 2, 4, 1, None) == NULLPTR
    WS = ctypes.c_void_p(0x100000)  # 256-byte aligned, never dereferenced

    def call(S=8, Skv=4096, B=2, r=1, topk=4, q=FAKE, k=FAKE, w=FAKE, idx=FAKE, g=FAKE,
             gq=FAKE, gk=FAKE, gw=FAKE, ws=WS, ws_bytes=ws_ok, handle=h):
        return lib.dsai_indexer_backward(handle, q, k, w, idx, g, S, Skv, B, r, topk, gq, gk, gw,
                                         ws, ws_bytes, None)

    assert call(handle=None) == NULLPTR
    for kw in ({"S": -1}, {"Skv": -1}, {"B": -1}, {"r": 0}, {"topk": 0}, {"topk": 8193},
               {"S": 1 << 31}, {"S": 1 << 20, "B": 1 << 12}, {"Skv": 1 << 20, "B": 1 << 12}):
        assert call(**kw) == INVALID, kw
    assert call(B=0) == OK                  # nothing to write
    assert call(S=0, Skv=0) == OK
    assert call(ws=None) == WORKSPACE
    assert call(ws_bytes=ws_ok - 1) == WORKSPACE
    assert call(ws=ctypes.c_void_p(0x100080)) == WORKSPACE   # not 256-byte aligned
    for name in ("q", "k", "w", "idx", "g", "gq", "gk", "gw"):
        assert call(**{name: None}) == NULLPTR, name
    for name in ("q", "k", "gq", "gk"):
        assert call(**{name: ctypes.c_void_p(0x10008)}) == INVALID, name
    for name in ("w", "idx", "g", "gw"):
        assert call(**{name: ctypes.c_void_p(0x10002)}) == INVALID, name
    # S == 0 needs only the key side; Skv == 0 only the query side
    assert call(S=0, q=None, w=None, idx=None, g=None, gq=None, gw=None, k=None) == NULLPTR
    assert call(Skv=0, ws=None, ws_bytes=0, k=None, gk=None, q=None) == NULLPTR
    lib.dsai_destroy(h)


def test_pooled_argument_errors(lib):
    st, h = _create(lib, kpool=4, index_topk=512, first_key=3)
    assert st == OK
    P = ctypes.c_int64()
    assert lib.dsai_pool_count(h, 65536, ctypes.byref(P)) == OK and P.value == (65536 - 3) // 4
    assert lib.dsai_pool_count(h, 2, ctypes.byref(P)) == OK and P.value == 0
    assert lib.dsai_pool_count(h, 6, ctypes.byref(P)) == OK and P.value == 0   # partial pool only
    assert lib.dsai_pool_count(h, 7, ctypes.byref(P)) == OK and P.value == 1
    assert lib.dsai_pool_count(h, -1, ctypes.byref(P)) == INVALID
    assert lib.dsai_pool_count(h, 5, None) == NULLPTR
    # kpool_compress
    kp = lambda N=64, *ptrs: lib.dsai_kpool_compress(h, *(ptrs or (FAKE,) * 4), N, FAKE, FAKE, FAKE, None)
    assert kp(-1) == INVALID
    assert kp(3) == OK                                 # no pool: nothing launched
    assert lib.dsai_kpool_compress(h, None, FAKE, FAKE, FAKE, 64, FAKE, FAKE, FAKE, None) == NULLPTR
    assert lib.dsai_kpool_compress(h, FAKE, FAKE, FAKE, FAKE, 64, None, FAKE, FAKE, None) == NULLPTR
    # index_scores
    assert lib.dsai_index_scores(h, FAKE, FAKE, FAKE, FAKE, None, -1, 5, FAKE, None) == INVALID
    assert lib.dsai_index_scores(h, FAKE, FAKE, FAKE, FAKE, None, 0, 5, FAKE, None) == OK
    assert lib.dsai_index_scores(h, None, FAKE, FAKE, FAKE, None, 2, 5, FAKE, None) == NULLPTR
    # pool_limit: an int32 array (4-byte aligned) or NULL
    assert lib.dsai_index_scores(h, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x10002), 2, 5, FAKE,
                                 None) == INVALID
    # topk_pools
    assert lib.dsai_topk_pools(h, FAKE, -2, 5, FAKE, FAKE, None) == INVALID
    assert lib.dsai_topk_pools(h, FAKE, 0, 5, FAKE, FAKE, None) == OK
    assert lib.dsai_topk_pools(h, FAKE, 2, 5, None, FAKE, None) == NULLPTR
    # select: workspace
    need = ctypes.c_size_t()
    assert lib.dsai_select_workspace_size(h, 64, 16384, ctypes.byref(need)) == OK
    assert need.value == 64 * 16384 * 4
    assert lib.dsai_select(h, FAKE, FAKE, FAKE, FAKE, None, 64, 16384, FAKE, FAKE, None, 0, None) == WORKSPACE
    assert lib.dsai_select(h, FAKE, FAKE, FAKE, FAKE, None, 64, 16384, FAKE, FAKE, FAKE, need.value - 1,
                           None) == WORKSPACE
    assert lib.dsai_select(h, FAKE, FAKE, FAKE, FAKE, None, 64, 16384, FAKE, FAKE,
                           ctypes.c_void_p(0x10010), need.value, None) == WORKSPACE   # not 256-aligned
    assert lib.dsai_select(h, FAKE, FAKE, FAKE, FAKE, None, -1, 16384, FAKE, FAKE, FAKE, 0, None) == INVALID
    # select with expand: select's rules plus the token array
    se = lambda Q=64, tok=FAKE, ws=FAKE, wsb=need.value: lib.dsai_select_expand(
        h, FAKE, FAKE, FAKE, FAKE, None, Q, 16384, FAKE, FAKE, tok, ws, wsb, None)
    assert se(Q=-1) == INVALID
    assert se(Q=0) == OK
    assert se(tok=None) == NULLPTR
    assert se(tok=ctypes.c_void_p(0x10004)) == INVALID     # tokens 16-byte aligned
    assert se(wsb=need.value - 1) == WORKSPACE
    assert se(ws=None) == WORKSPACE
    # select with expand from the static array: its rules, and no more
    # scores than the array holds (refused before any HIP call)
    sst = lambda Q=64, P=16384, tok=FAKE: lib.dsai_select_expand_static(
        h, FAKE, FAKE, FAKE, FAKE, None, Q, P, FAKE, FAKE, tok, None)
    assert sst(Q=-1) == INVALID
    assert sst(Q=0) == OK
    assert sst(tok=None) == NULLPTR
    assert sst(tok=ctypes.c_void_p(0x10004)) == INVALID
    assert sst(Q=64, P=(16 << 20) // (4 * 64) + 1) == WORKSPACE
    assert sst(Q=1, P=(16 << 20) // 4 + 1) == WORKSPACE
    assert lib.dsai_select_expand_static(None, FAKE, FAKE, FAKE, FAKE, None, 1, 1, FAKE, FAKE, FAKE,
                                         None) == NULLPTR
    # expand
    assert lib.dsai_expand(h, FAKE, -1, FAKE, None) == INVALID
    assert lib.dsai_expand(h, FAKE, 0, FAKE, None) == OK
    assert lib.dsai_expand(h, None, 3, FAKE, None) == NULLPTR
    assert lib.dsai_expand(h, FAKE, 3, None, None) == NULLPTR
    lib.dsai_destroy(h)


def test_expanded_token_ids_must_fit_int32(lib):
    """first_key + P * kpool - 1 above 2^31 - 1 would overflow the int32
    token ids: select with expand (either form) refuses it before any HIP
    call; one pool fewer passes the check (and then needs a device, so the
    workspace check is what answers here)."""
    KP, fk = 8, 2 ** 31 - 1 - 8 * 1000
    st, h = _create(lib, kpool=KP, index_topk=64, first_key=fk)
    assert st == OK
    P_ok = (2 ** 31 - 1 - fk + 1) // KP          # last token = 2^31 - 1
    se = lambda P, ws=None: lib.dsai_select_expand(h, FAKE, FAKE, FAKE, FAKE, None, 2, P, FAKE, FAKE,
                                                   FAKE, ws, 0, None)
    assert se(P_ok + 1) == INVALID
    assert se(P_ok) == WORKSPACE                 # past the token check: no workspace given
    assert lib.dsai_select_expand_static(h, FAKE, FAKE, FAKE, FAKE, None, 2, P_ok + 1, FAKE, FAKE,
                                         FAKE, None) == INVALID
    lib.dsai_destroy(h)


def test_sort_rows_argument_errors(lib):
    st, h = _create(lib)
    assert st == OK
    assert lib.dsai_sort_rows(h, FAKE, FAKE, -1, 8, None) == INVALID
    assert lib.dsai_sort_rows(h, FAKE, FAKE, 2 ** 31, 8, None) == INVALID
    assert lib.dsai_sort_rows(h, FAKE, FAKE, 4, 0, None) == INVALID
    assert lib.dsai_sort_rows(h, FAKE, FAKE, 4, 8193, None) == INVALID
    assert lib.dsai_sort_rows(h, FAKE, FAKE, 0, 8, None) == OK       # nothing to do
    assert lib.dsai_sort_rows(h, FAKE, FAKE, 4, 1, None) == OK       # one entry per row
    assert lib.dsai_sort_rows(h, None, FAKE, 4, 8, None) == NULLPTR
    assert lib.dsai_sort_rows(h, FAKE, None, 4, 8, None) == NULLPTR
    assert lib.dsai_sort_rows(h, ctypes.c_void_p(0x10002), FAKE, 4, 8, None) == INVALID
    assert lib.dsai_sort_rows(None, FAKE, FAKE, 4, 8, None) == NULLPTR
    lib.dsai_destroy(h)


def test_binding_refuses_cpu_tensors(lib):
    import torch
    import sparse_attention_token_index_amd as dsai
    ix = dsai.Indexer(heads=4, dim=32)
    q = torch.zeros(8, 1, 4, 32, dtype=torch.bfloat16)
    k = torch.zeros(8, 1, 32, dtype=torch.bfloat16)
    w = torch.zeros(8, 1, 4)
    with pytest.raises(dsai.DsaiError):
        ix.score_topk(q, k, w, 1, 4)
