"""MI355X (gfx950) DSA lightning-indexer token selection.

A thin ctypes binding over the C ABI in ``include/dsai.h`` (``libdsai.so``,
built in-tree by ``python -m sparse_attention_token_index_amd.build``).  This
module only checks and marshals arguments: every step of the selection path
runs in the library's HIP kernels, on the current PyTorch stream.  PyTorch
provides device memory and streams.  There is no CPU fallback: without the
built library, or without tensors on a ROCm GPU, every call raises.

Names follow the C entry points: ``score_topk`` (lightning-indexer score +
causal/compressed mask + top-k, or scores at supplied indices),
``indexer_backward`` (gradients of the selected scores; ``IndexerFunction``
is the autograd pairing of the two), ``k_norm``
(the cache write's LayerNorm), and the pooled decode pipeline
``kpool_compress`` -> ``index_scores`` -> ``topk_pools`` -> ``expand``
(``select`` = ``index_scores`` + ``topk_pools``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

__all__ = ["DsaiError", "Indexer", "IndexerFunction", "load_library", "library_path", "EXPORTS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdsai.so")

# Every symbol include/dsai.h declares.
EXPORTS = (
    "dsai_create", "dsai_destroy", "dsai_status_string", "dsai_last_hip_error",
    "dsai_score_topk", "dsai_score_topk_packed", "dsai_backward_packed_workspace_size",
    "dsai_indexer_backward_packed", "dsai_select_expand", "dsai_pool_count", "dsai_kpool_compress", "dsai_index_scores",
    "dsai_topk_pools", "dsai_select_workspace_size", "dsai_select", "dsai_expand",
    "dsai_sort_rows", "dsai_k_norm", "dsai_backward_workspace_size", "dsai_indexer_backward",
    "dsai_select_expand_static",
)

DSAI_OK = 0
DSAI_ORDER_SCORE = 0  # rows by score descending, lower index first on ties
DSAI_ORDER_INDEX = 1  # rows by ascending index (same set, no sorting pass)
DSAI_CUTS_ESTIMATED = 0  # filter-store cuts keep an estimated rank (rerun if short)
DSAI_CUTS_TOPK = 1  # filter-store cuts keep k (key order that predicts the scores)
DSAI_MAX_KPOOL = 8
DSAI_MAX_TOPK = 8192
DSAI_STATIC_SCRATCH_BYTES = 16 << 20  # scores array of dsai_select_expand_static


class DsaiError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        super().__init__(f"{what}: {detail} (status {status})")


class _Config(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int), ("dim", ctypes.c_int), ("kpool", ctypes.c_int),
                ("index_topk", ctypes.c_int), ("first_key", ctypes.c_int),
                ("chunk_rows", ctypes.c_int), ("order", ctypes.c_int), ("cuts", ctypes.c_int)]


_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return _LIB_PATH


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libdsai.so once and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise DsaiError(-2, "libdsai.so is not built",
                        f"{p} missing; run `python -m sparse_attention_token_index_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "dsai_create": [ctypes.POINTER(_Config), ctypes.POINTER(vp)],
        "dsai_destroy": [vp],
        "dsai_status_string": [c_int],
        "dsai_last_hip_error": [vp],
        "dsai_score_topk": [vp, vp, vp, vp, i64, i64, i64, c_int, c_int, vp, vp, vp, vp],
        "dsai_score_topk_packed": [vp, vp, vp, vp, i64, vp, vp, c_int, c_int, vp, vp, vp, vp],
        "dsai_backward_packed_workspace_size": [vp, i64, vp, vp, c_int, c_int, vp],
        "dsai_select_expand": [vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, ctypes.c_size_t,
                               vp],
        "dsai_select_expand_static": [vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp],
        "dsai_indexer_backward_packed": [vp, vp, vp, vp, vp, vp, i64, vp, vp, c_int, c_int, vp, vp,
                                         vp, vp, ctypes.c_size_t, vp],
        "dsai_pool_count": [vp, i64, ctypes.POINTER(i64)],
        "dsai_kpool_compress": [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp],
        "dsai_index_scores": [vp, vp, vp, vp, vp, vp, i64, i64, vp, vp],
        "dsai_topk_pools": [vp, vp, i64, i64, vp, vp, vp],
        "dsai_select_workspace_size": [vp, i64, i64, ctypes.POINTER(ctypes.c_size_t)],
        "dsai_select": [vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, ctypes.c_size_t, vp],
        "dsai_expand": [vp, vp, i64, vp, vp],
        "dsai_sort_rows": [vp, vp, vp, i64, c_int, vp],
        "dsai_k_norm": [vp, vp, vp, vp, ctypes.c_float, i64, vp, vp],
        "dsai_backward_workspace_size": [vp, i64, i64, i64, c_int, c_int,
                                         ctypes.POINTER(ctypes.c_size_t)],
        "dsai_indexer_backward": [vp, vp, vp, vp, vp, vp, i64, i64, i64, c_int, c_int, vp, vp, vp,
                                  vp, ctypes.c_size_t, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "dsai_status_string" else c_int
    if path is None:
        _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _offsets(cu_q, cu_k):
    """Host int64 copies of packed-sequence offsets and the sequence count."""
    cq = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int64))
    ck = np.ascontiguousarray(np.asarray(cu_k, dtype=np.int64))
    if cq.ndim != 1 or ck.shape != cq.shape or cq.size < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k: equal-length 1-D offset lists")
    return cq, ck, cq.size - 1


def _host(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise DsaiError(-2, name, "must be a GPU tensor (the HIP path has no CPU fallback)")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


class Indexer:
    """One configured handle of the selection library (dsai_create)."""

    def __init__(self, heads: int, dim: int, kpool: int = 1, index_topk: int = 1,
                 first_key: int = 0, chunk_rows: int = 0, order: int = DSAI_ORDER_SCORE,
                 cuts: int = DSAI_CUTS_ESTIMATED):
        self._lib = load_library()
        self.cfg = _Config(heads, dim, kpool, index_topk, first_key, chunk_rows, order, cuts)
        h = ctypes.c_void_p()
        st = self._lib.dsai_create(ctypes.byref(self.cfg), ctypes.byref(h))
        self._check(st, "dsai_create")
        self._h = h

    # -- plumbing ---------------------------------------------------------
    def _check(self, st: int, what: str):
        if st != DSAI_OK:
            msg = self._lib.dsai_status_string(st).decode()
            if st == -5 and getattr(self, "_h", None):
                msg += f" (hipError {self._lib.dsai_last_hip_error(self._h)})"
            raise DsaiError(st, what, msg)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.dsai_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def heads(self):
        return self.cfg.heads

    @property
    def dim(self):
        return self.cfg.dim

    @property
    def select_k(self):
        return self.cfg.index_topk // self.cfg.kpool

    # -- unpooled lightning indexer ----------------------------------------
    def score_topk(self, index_q: torch.Tensor, index_k: torch.Tensor, weights: torch.Tensor,
                   compress_ratio: int, topk: int, topk_indices=None,
                   out_idx: Optional[torch.Tensor] = None,
                   out_score: Optional[torch.Tensor] = None):
        """index_q [S,B,H,D] bf16, index_k [Skv,B,D] bf16, weights [S,B,H] fp32 ->
        (idx [B,S,topk] int32, score [B,S,topk] fp32).

        With topk_indices [B,S,topk] int32 the keys are not selected: each
        supplied index s with 0 <= s < n_t gets its score, any other entry
        (-1, -inf); entries keep the supplied order (out_idx may be
        topk_indices itself)."""
        S, B = index_q.shape[0], index_q.shape[1]
        Skv = index_k.shape[0]
        H, D = self.cfg.heads, self.cfg.dim
        dev = index_q.device
        _need(index_q, "index_q", torch.bfloat16, (S, B, H, D))
        _need(index_k, "index_k", torch.bfloat16, (Skv, B, D), dev)
        _need(weights, "weights", torch.float32, (S, B, H), dev)
        if topk_indices is not None:
            _need(topk_indices, "topk_indices", torch.int32, (B, S, topk), dev)
        if out_idx is None:
            out_idx = torch.empty((B, S, topk), dtype=torch.int32, device=dev)
        if out_score is None:
            out_score = torch.empty((B, S, topk), dtype=torch.float32, device=dev)
        _need(out_idx, "out_idx", torch.int32, (B, S, topk), dev)
        _need(out_score, "out_score", torch.float32, (B, S, topk), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_score_topk(self._h, _ptr(index_q), _ptr(index_k), _ptr(weights),
                                           S, Skv, B, int(compress_ratio), int(topk),
                                           _ptr(topk_indices), _ptr(out_idx), _ptr(out_score),
                                           _stream(dev))
        self._check(st, "dsai_score_topk")
        return out_idx, out_score

    def score_topk_packed(self, index_q: torch.Tensor, index_k: torch.Tensor,
                          weights: torch.Tensor, cu_seqlens_q, cu_seqlens_k,
                          compress_ratio: int, topk: int, topk_indices=None,
                          out_idx: Optional[torch.Tensor] = None,
                          out_score: Optional[torch.Tensor] = None):
        """Packed sequences: index_q [Tq,H,D] bf16, index_k [Tk,D] bf16,
        weights [Tq,H] fp32, cu_seqlens_q / cu_seqlens_k nseq + 1 offsets
        (a sequence of ints or a CPU tensor; they are read on the host) ->
        (idx [Tq,topk] int32, score [Tq,topk] fp32).  Each sequence is the
        one-sample problem on its own rows and keys; indices are local to it.
        topk must be a multiple of 4."""
        cq, ck, nseq = _offsets(cu_seqlens_q, cu_seqlens_k)
        Tq, Tk = index_q.shape[0], index_k.shape[0]
        H, D = self.cfg.heads, self.cfg.dim
        dev = index_q.device
        _need(index_q, "index_q", torch.bfloat16, (Tq, H, D))
        _need(index_k, "index_k", torch.bfloat16, (Tk, D), dev)
        _need(weights, "weights", torch.float32, (Tq, H), dev)
        if int(cq[-1]) != Tq or int(ck[-1]) != Tk:
            raise ValueError("the last offsets must equal the row counts of index_q and index_k")
        if topk_indices is not None:
            _need(topk_indices, "topk_indices", torch.int32, (Tq, topk), dev)
        if out_idx is None:
            out_idx = torch.empty((Tq, topk), dtype=torch.int32, device=dev)
        if out_score is None:
            out_score = torch.empty((Tq, topk), dtype=torch.float32, device=dev)
        _need(out_idx, "out_idx", torch.int32, (Tq, topk), dev)
        _need(out_score, "out_score", torch.float32, (Tq, topk), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_score_topk_packed(
                self._h, _ptr(index_q), _ptr(index_k), _ptr(weights), nseq,
                _host(cq), _host(ck),
                int(compress_ratio), int(topk), _ptr(topk_indices), _ptr(out_idx),
                _ptr(out_score), _stream(dev))
        self._check(st, "dsai_score_topk_packed")
        return out_idx, out_score

    # -- backward ------------------------------------------------------------
    def backward_workspace_size(self, S: int, Skv: int, B: int, topk: int,
                                compress_ratio: int) -> int:
        n = ctypes.c_size_t()
        self._check(self._lib.dsai_backward_workspace_size(self._h, int(S), int(Skv), int(B),
                                                           int(topk), int(compress_ratio),
                                                           ctypes.byref(n)),
                    "dsai_backward_workspace_size")
        return n.value

    def indexer_backward(self, index_q: torch.Tensor, index_k: torch.Tensor,
                         weights: torch.Tensor, topk_indices: torch.Tensor,
                         grad_scores: torch.Tensor, compress_ratio: int,
                         workspace: Optional[torch.Tensor] = None,
                         grad_q: Optional[torch.Tensor] = None,
                         grad_k: Optional[torch.Tensor] = None,
                         grad_weights: Optional[torch.Tensor] = None):
        """Gradients of the scores at topk_indices [B,S,topk] int32 given their
        incoming gradient grad_scores [B,S,topk] fp32 -> (grad_q [S,B,H,D] bf16,
        grad_k [Skv,B,D] bf16, grad_weights [S,B,H] fp32).  Entries that are
        -1, masked or out of range pass nothing back.  `workspace` (uint8,
        backward_workspace_size(S, Skv, B, topk, compress_ratio) bytes) is
        allocated when not given."""
        S, B = index_q.shape[0], index_q.shape[1]
        Skv = index_k.shape[0]
        H, D = self.cfg.heads, self.cfg.dim
        dev = index_q.device
        _need(index_q, "index_q", torch.bfloat16, (S, B, H, D))
        _need(index_k, "index_k", torch.bfloat16, (Skv, B, D), dev)
        _need(weights, "weights", torch.float32, (S, B, H), dev)
        if topk_indices.dim() != 3:
            raise ValueError("topk_indices: expected [B, S, topk]")
        topk = topk_indices.shape[2]
        _need(topk_indices, "topk_indices", torch.int32, (B, S, topk), dev)
        _need(grad_scores, "grad_scores", torch.float32, (B, S, topk), dev)
        need = self.backward_workspace_size(S, Skv, B, topk, compress_ratio)
        if workspace is None:
            workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
        if grad_q is None:
            grad_q = torch.empty((S, B, H, D), dtype=torch.bfloat16, device=dev)
        if grad_k is None:
            grad_k = torch.empty((Skv, B, D), dtype=torch.bfloat16, device=dev)
        if grad_weights is None:
            grad_weights = torch.empty((S, B, H), dtype=torch.float32, device=dev)
        _need(grad_q, "grad_q", torch.bfloat16, (S, B, H, D), dev)
        _need(grad_k, "grad_k", torch.bfloat16, (Skv, B, D), dev)
        _need(grad_weights, "grad_weights", torch.float32, (S, B, H), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_indexer_backward(
                self._h, _ptr(index_q), _ptr(index_k), _ptr(weights), _ptr(topk_indices),
                _ptr(grad_scores), S, Skv, B, int(compress_ratio), int(topk), _ptr(grad_q),
                _ptr(grad_k), _ptr(grad_weights), _ptr(workspace),
                workspace.numel() * workspace.element_size(), _stream(dev))
        self._check(st, "dsai_indexer_backward")
        return grad_q, grad_k, grad_weights

    def backward_packed_workspace_size(self, cu_seqlens_q, cu_seqlens_k, topk: int,
                                       compress_ratio: int) -> int:
        cq, ck, nseq = _offsets(cu_seqlens_q, cu_seqlens_k)
        n = ctypes.c_size_t()
        self._check(self._lib.dsai_backward_packed_workspace_size(
            self._h, nseq, _host(cq), _host(ck), int(topk), int(compress_ratio), ctypes.byref(n)),
            "dsai_backward_packed_workspace_size")
        return n.value

    def indexer_backward_packed(self, index_q: torch.Tensor, index_k: torch.Tensor,
                                weights: torch.Tensor, topk_indices: torch.Tensor,
                                grad_scores: torch.Tensor, cu_seqlens_q, cu_seqlens_k,
                                compress_ratio: int, workspace: Optional[torch.Tensor] = None,
                                grad_q: Optional[torch.Tensor] = None,
                                grad_k: Optional[torch.Tensor] = None,
                                grad_weights: Optional[torch.Tensor] = None):
        """Packed sequences: index_q [Tq,H,D], index_k [Tk,D], weights [Tq,H],
        topk_indices / grad_scores [Tq,topk] (indices local to each sequence)
        -> (grad_q [Tq,H,D] bf16, grad_k [Tk,D] bf16, grad_weights [Tq,H]
        fp32); each sequence gets its one-sample gradients."""
        cq, ck, nseq = _offsets(cu_seqlens_q, cu_seqlens_k)
        Tq, Tk = index_q.shape[0], index_k.shape[0]
        H, D = self.cfg.heads, self.cfg.dim
        dev = index_q.device
        _need(index_q, "index_q", torch.bfloat16, (Tq, H, D))
        _need(index_k, "index_k", torch.bfloat16, (Tk, D), dev)
        _need(weights, "weights", torch.float32, (Tq, H), dev)
        if int(cq[-1]) != Tq or int(ck[-1]) != Tk:
            raise ValueError("the last offsets must equal the row counts of index_q and index_k")
        if topk_indices.dim() != 2:
            raise ValueError("topk_indices: expected [Tq, topk]")
        topk = topk_indices.shape[1]
        _need(topk_indices, "topk_indices", torch.int32, (Tq, topk), dev)
        _need(grad_scores, "grad_scores", torch.float32, (Tq, topk), dev)
        need = self.backward_packed_workspace_size(cq, ck, topk, compress_ratio)
        if workspace is None:
            workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
        if grad_q is None:
            grad_q = torch.empty((Tq, H, D), dtype=torch.bfloat16, device=dev)
        if grad_k is None:
            grad_k = torch.empty((Tk, D), dtype=torch.bfloat16, device=dev)
        if grad_weights is None:
            grad_weights = torch.empty((Tq, H), dtype=torch.float32, device=dev)
        _need(grad_q, "grad_q", torch.bfloat16, (Tq, H, D), dev)
        _need(grad_k, "grad_k", torch.bfloat16, (Tk, D), dev)
        _need(grad_weights, "grad_weights", torch.float32, (Tq, H), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_indexer_backward_packed(
                self._h, _ptr(index_q), _ptr(index_k), _ptr(weights), _ptr(topk_indices),
                _ptr(grad_scores), nseq, _host(cq), _host(ck), int(compress_ratio), int(topk),
                _ptr(grad_q), _ptr(grad_k), _ptr(grad_weights), _ptr(workspace),
                workspace.numel() * workspace.element_size(), _stream(dev))
        self._check(st, "dsai_indexer_backward_packed")
        return grad_q, grad_k, grad_weights

    # -- cache write ---------------------------------------------------------
    def k_norm(self, k_raw: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor,
               eps: float = 1e-5, out: Optional[torch.Tensor] = None):
        """k_raw [N,D] bf16, gamma/beta [D] bf16 -> k_normed [N,D] bf16 (LayerNorm with a
        bias, fp32 inside); `out` may be k_raw itself."""
        N, D = k_raw.shape[0], self.cfg.dim
        dev = k_raw.device
        _need(k_raw, "k_raw", torch.bfloat16, (N, D))
        _need(gamma, "gamma", torch.bfloat16, (D,), dev)
        _need(beta, "beta", torch.bfloat16, (D,), dev)
        if out is None:
            out = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
        _need(out, "out", torch.bfloat16, (N, D), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_k_norm(self._h, _ptr(k_raw), _ptr(gamma), _ptr(beta),
                                       float(eps), N, _ptr(out), _stream(dev))
        self._check(st, "dsai_k_norm")
        return out

    # -- pooled decode pipeline ---------------------------------------------
    def pool_count(self, N: int) -> int:
        P = ctypes.c_int64()
        self._check(self._lib.dsai_pool_count(self._h, int(N), ctypes.byref(P)), "dsai_pool_count")
        return P.value

    def kpool_compress(self, k_normed, gate, valid, ape, pool_k=None, pool_tok=None,
                       pool_valid=None):
        """k_normed [N,D] bf16, gate [N,D] fp32, valid [N] bool/uint8, ape [KP,D] fp32 ->
        (pool_k [P,D] bf16, pool_tok [P] int32, pool_valid [P] uint8)."""
        N, D, KP = k_normed.shape[0], self.cfg.dim, self.cfg.kpool
        dev = k_normed.device
        if valid.dtype == torch.bool:
            valid = valid.view(torch.uint8)
        _need(k_normed, "k_normed", torch.bfloat16, (N, D))
        _need(gate, "gate", torch.float32, (N, D), dev)
        _need(valid, "valid", torch.uint8, (N,), dev)
        _need(ape, "ape", torch.float32, (KP, D), dev)
        P = self.pool_count(N)
        if pool_k is None:
            pool_k = torch.empty((P, D), dtype=torch.bfloat16, device=dev)
        if pool_tok is None:
            pool_tok = torch.empty((P,), dtype=torch.int32, device=dev)
        if pool_valid is None:
            pool_valid = torch.empty((P,), dtype=torch.uint8, device=dev)
        _need(pool_k, "pool_k", torch.bfloat16, (P, D), dev)
        _need(pool_tok, "pool_tok", torch.int32, (P,), dev)
        _need(pool_valid, "pool_valid", torch.uint8, (P,), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_kpool_compress(self._h, _ptr(k_normed), _ptr(gate), _ptr(valid),
                                               _ptr(ape), N, _ptr(pool_k), _ptr(pool_tok),
                                               _ptr(pool_valid), _stream(dev))
        self._check(st, "dsai_kpool_compress")
        return pool_k, pool_tok, pool_valid

    def index_scores(self, q, w, pool_k, pool_valid, out=None, pool_limit=None):
        """q [Q,H,D] bf16, w [Q,H] fp32, pool_k [P,D] bf16, pool_valid [P] uint8 -> [Q,P] fp32.
        pool_limit: optional [Q] int32 per-row bound; row q's pools p >= it are
        invalid candidates (-inf) for that row."""
        Q, P = q.shape[0], pool_k.shape[0]
        H, D = self.cfg.heads, self.cfg.dim
        dev = q.device
        if pool_valid.dtype == torch.bool:
            pool_valid = pool_valid.view(torch.uint8)
        _need(q, "q", torch.bfloat16, (Q, H, D))
        _need(w, "w", torch.float32, (Q, H), dev)
        _need(pool_k, "pool_k", torch.bfloat16, (P, D), dev)
        _need(pool_valid, "pool_valid", torch.uint8, (P,), dev)
        if pool_limit is not None:
            _need(pool_limit, "pool_limit", torch.int32, (Q,), dev)
        if out is None:
            out = torch.empty((Q, P), dtype=torch.float32, device=dev)
        _need(out, "scores", torch.float32, (Q, P), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_index_scores(self._h, _ptr(q), _ptr(w), _ptr(pool_k),
                                             _ptr(pool_valid), _ptr(pool_limit), Q, P, _ptr(out),
                                             _stream(dev))
        self._check(st, "dsai_index_scores")
        return out

    def topk_pools(self, scores, pool_ids=None, pool_scores=None):
        """scores [Q,P] fp32 -> (pool_ids [Q,select_k] int32, pool_scores [Q,select_k] fp32)."""
        Q, P = scores.shape
        dev = scores.device
        K = self.select_k
        _need(scores, "scores", torch.float32, (Q, P))
        if pool_ids is None:
            pool_ids = torch.empty((Q, K), dtype=torch.int32, device=dev)
        if pool_scores is None:
            pool_scores = torch.empty((Q, K), dtype=torch.float32, device=dev)
        _need(pool_ids, "pool_ids", torch.int32, (Q, K), dev)
        _need(pool_scores, "pool_scores", torch.float32, (Q, K), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_topk_pools(self._h, _ptr(scores), Q, P, _ptr(pool_ids),
                                           _ptr(pool_scores), _stream(dev))
        self._check(st, "dsai_topk_pools")
        return pool_ids, pool_scores

    def select_workspace_size(self, Q: int, P: int) -> int:
        n = ctypes.c_size_t()
        self._check(self._lib.dsai_select_workspace_size(self._h, int(Q), int(P), ctypes.byref(n)),
                    "dsai_select_workspace_size")
        return n.value

    def select(self, q, w, pool_k, pool_valid, workspace=None, pool_ids=None, pool_scores=None,
               tokens=None, expand=False, pool_limit=None):
        """index_scores + topk_pools with the [Q,P] scores in `workspace` (uint8
        tensor) -> (pool_ids, pool_scores); with expand=True also the token ids
        [Q, select_k*kpool] (dsai_select_expand) -> (pool_ids, pool_scores,
        tokens)."""
        Q, P = q.shape[0], pool_k.shape[0]
        H, D = self.cfg.heads, self.cfg.dim
        dev = q.device
        K = self.select_k
        if pool_valid.dtype == torch.bool:
            pool_valid = pool_valid.view(torch.uint8)
        _need(q, "q", torch.bfloat16, (Q, H, D))
        _need(w, "w", torch.float32, (Q, H), dev)
        _need(pool_k, "pool_k", torch.bfloat16, (P, D), dev)
        _need(pool_valid, "pool_valid", torch.uint8, (P,), dev)
        if pool_limit is not None:
            _need(pool_limit, "pool_limit", torch.int32, (Q,), dev)
        need = self.select_workspace_size(Q, P)
        if workspace is None:
            workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
        if pool_ids is None:
            pool_ids = torch.empty((Q, K), dtype=torch.int32, device=dev)
        if pool_scores is None:
            pool_scores = torch.empty((Q, K), dtype=torch.float32, device=dev)
        _need(pool_ids, "pool_ids", torch.int32, (Q, K), dev)
        _need(pool_scores, "pool_scores", torch.float32, (Q, K), dev)
        if expand:
            if tokens is None:
                tokens = torch.empty((Q, K * self.cfg.kpool), dtype=torch.int32, device=dev)
            _need(tokens, "tokens", torch.int32, (Q, K * self.cfg.kpool), dev)
            with torch.cuda.device(dev):
                st = self._lib.dsai_select_expand(
                    self._h, _ptr(q), _ptr(w), _ptr(pool_k), _ptr(pool_valid), _ptr(pool_limit), Q, P,
                    _ptr(pool_ids), _ptr(pool_scores), _ptr(tokens), _ptr(workspace),
                    workspace.numel() * workspace.element_size(), _stream(dev))
            self._check(st, "dsai_select_expand")
            return pool_ids, pool_scores, tokens
        with torch.cuda.device(dev):
            st = self._lib.dsai_select(self._h, _ptr(q), _ptr(w), _ptr(pool_k), _ptr(pool_valid),
                                       _ptr(pool_limit), Q, P, _ptr(pool_ids), _ptr(pool_scores), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(dev))
        self._check(st, "dsai_select")
        return pool_ids, pool_scores

    def select_expand_static(self, q, w, pool_k, pool_valid, pool_ids, pool_scores, tokens,
                             pool_limit=None):
        """dsai_select_expand_static: select with expand whose [Q,P] scores live
        in the library's static device array (no workspace; the output
        tensors are the caller's, so the call allocates nothing).  Calls that
        overlap on one GPU share that array and race."""
        Q, P = q.shape[0], pool_k.shape[0]
        H, D, K = self.cfg.heads, self.cfg.dim, self.select_k
        dev = q.device
        if pool_valid.dtype == torch.bool:
            pool_valid = pool_valid.view(torch.uint8)
        _need(q, "q", torch.bfloat16, (Q, H, D))
        _need(w, "w", torch.float32, (Q, H), dev)
        _need(pool_k, "pool_k", torch.bfloat16, (P, D), dev)
        _need(pool_valid, "pool_valid", torch.uint8, (P,), dev)
        _need(pool_ids, "pool_ids", torch.int32, (Q, K), dev)
        _need(pool_scores, "pool_scores", torch.float32, (Q, K), dev)
        _need(tokens, "tokens", torch.int32, (Q, K * self.cfg.kpool), dev)
        if pool_limit is not None:
            _need(pool_limit, "pool_limit", torch.int32, (Q,), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_select_expand_static(
                self._h, _ptr(q), _ptr(w), _ptr(pool_k), _ptr(pool_valid), _ptr(pool_limit), Q, P,
                _ptr(pool_ids), _ptr(pool_scores), _ptr(tokens), _stream(dev))
        self._check(st, "dsai_select_expand_static")
        return pool_ids, pool_scores, tokens

    def expand(self, pool_ids, tokens=None):
        """pool_ids [Q,select_k] int32 -> token ids [Q, select_k*kpool] int32 (-1 = invalid)."""
        Q = pool_ids.shape[0]
        dev = pool_ids.device
        K, KP = self.select_k, self.cfg.kpool
        _need(pool_ids, "pool_ids", torch.int32, (Q, K))
        if tokens is None:
            tokens = torch.empty((Q, K * KP), dtype=torch.int32, device=dev)
        _need(tokens, "tokens", torch.int32, (Q, K * KP), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_expand(self._h, _ptr(pool_ids), Q, _ptr(tokens), _stream(dev))
        self._check(st, "dsai_expand")
        return tokens

    def sort_rows(self, idx, score):
        """In place: each row of idx/score [..., k] (ascending-index top-k rows,
        as written in DSAI_ORDER_INDEX order) reordered by score descending,
        lower index first among equal scores, padding (-1, -inf) last."""
        if idx.dim() < 1:
            raise ValueError("idx: needs a last (row) dimension")
        k = idx.shape[-1]
        rows = idx.numel() // k if k else 0
        dev = idx.device
        _need(idx, "idx", torch.int32, tuple(idx.shape))
        _need(score, "score", torch.float32, tuple(idx.shape), dev)
        with torch.cuda.device(dev):
            st = self._lib.dsai_sort_rows(self._h, _ptr(idx), _ptr(score), rows, int(k), _stream(dev))
        self._check(st, "dsai_sort_rows")
        return idx, score


class IndexerFunction(torch.autograd.Function):
    """Autograd pairing of score_topk and indexer_backward (the V4 indexer's
    autograd function): apply(indexer, index_q, index_k, weights,
    compress_ratio, topk, topk_indices=None) -> (scores, indices), both
    [B,S,topk]; scores fp32 (-inf padding), indices int32 (-1 padding).
    The indices take no gradient; the scores pass theirs to index_q,
    index_k and weights."""

    @staticmethod
    def forward(ctx, indexer: Indexer, index_q, index_k, weights, compress_ratio: int, topk: int,
                topk_indices=None):
        idx, score = indexer.score_topk(index_q.detach(), index_k.detach(), weights.detach(),
                                        compress_ratio, topk, topk_indices=topk_indices)
        ctx.indexer = indexer
        ctx.compress_ratio = int(compress_ratio)
        ctx.save_for_backward(index_q, index_k, weights, idx)
        ctx.mark_non_differentiable(idx)
        return score, idx

    @staticmethod
    def backward(ctx, grad_scores, grad_indices):
        index_q, index_k, weights, idx = ctx.saved_tensors
        if grad_scores is None:
            return None, None, None, None, None, None, None
        gq, gk, gw = ctx.indexer.indexer_backward(index_q.detach(), index_k.detach(),
                                                  weights.detach(), idx,
                                                  grad_scores.float().contiguous(),
                                                  ctx.compress_ratio)
        return None, gq, gk, gw, None, None, None
