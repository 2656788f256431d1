"""Python binding of ``libqsa.so`` (the C ABI of include/qsa.h).

Argument marshalling only: every step of the indexer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  The binding
fails loudly when the library is missing or the tensors are not what the C
ABI expects; it never computes a result itself and has no fallback.

Function names are those of the C entry points.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

QSA_OK = 0
QSA_ERR_INVALID_ARGUMENT = 1
QSA_ERR_UNSUPPORTED = 2
QSA_ERR_WORKSPACE_TOO_SMALL = 3
QSA_ERR_DEVICE = 4

QSA_SCORE_RELU = 0x1
QSA_OUT_KEYS = 0x2
QSA_STREAM_SELECT = 0x8
QSA_ROPE_INTERLEAVED = 0x4
QSA_MAX_SELECT = 4096

QSA_NOALLOC_SCRATCH_BYTES = 96 << 20

QSA_DEBUG_FORCE_TWO_PASS = 0x1
QSA_DEBUG_FORCE_FUSED = 0x2
QSA_DEBUG_FORCE_FALLBACK = 0x4
QSA_DEBUG_FORCE_TILES = 0x8
QSA_DEBUG_FORCE_GROUPS = 0x10
QSA_DEBUG_FORCE_REDO = 0x20
QSA_DEBUG_FORCE_STREAM = 0x40

EXPORTED = (
    "qsa_score_paged", "qsa_topk_rows", "qsa_topk_rows_workspace_size",
    "qsa_select_paged_tokens", "qsa_select_paged_tokens_workspace_size", "qsa_select_paged_tokens_noalloc",
    "qsa_sparse_attention",
    "qsa_sparse_attention_workspace_size", "qsa_compress_keys", "qsa_last_error", "qsa_last_path", "qsa_version",
    "qsa_debug_record_events", "qsa_debug_events_recorded", "qsa_debug_force", "qsa_debug_forced",
)


class QSAError(RuntimeError):
    """A non-zero qsa_status; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"qsa status {status}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with paged_block_scoring_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    L.qsa_score_paged.argtypes = [P, P, P, i64, i32, i32, P, P, i32, i32, i32, i32, i32, i32, u32, P, i64, P]
    L.qsa_score_paged.restype = ctypes.c_int
    L.qsa_topk_rows.argtypes = [P, i64, P, i32, i32, i32, P, P, sz, P]
    L.qsa_topk_rows.restype = ctypes.c_int
    L.qsa_topk_rows_workspace_size.argtypes = [i32, i32, i32]
    L.qsa_topk_rows_workspace_size.restype = sz
    L.qsa_select_paged_tokens.argtypes = [P, P, P, i64, i32, i32, P, P, i32, i32, i32, i32, i32, i32, i32, u32,
                                          P, P, sz, P]
    L.qsa_select_paged_tokens.restype = ctypes.c_int
    L.qsa_select_paged_tokens_noalloc.argtypes = [P, P, P, i64, i32, i32, P, P, i32, i32, i32, i32, i32, i32,
                                                  i32, u32, P, P]
    L.qsa_select_paged_tokens_noalloc.restype = ctypes.c_int
    L.qsa_select_paged_tokens_workspace_size.argtypes = [i32, i32, i32, i32, i32, u32]
    L.qsa_select_paged_tokens_workspace_size.restype = sz
    L.qsa_sparse_attention.argtypes = [P, P, P, P, i64, i32, i32, P, P, i32, i32, i32, i32, i32, i32,
                                       ctypes.c_float, P, P, sz, P]
    L.qsa_sparse_attention_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.qsa_sparse_attention_workspace_size.restype = sz
    L.qsa_sparse_attention.restype = ctypes.c_int
    L.qsa_compress_keys.argtypes = [P, P, P, i32, i32, P, ctypes.c_float, i32, ctypes.c_double, u32, P, P, P,
                                    i64, i32, i32, i32, i32, P]
    L.qsa_compress_keys.restype = ctypes.c_int
    L.qsa_debug_record_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), i32]
    L.qsa_debug_record_events.restype = ctypes.c_int
    L.qsa_debug_events_recorded.argtypes = []
    L.qsa_debug_events_recorded.restype = i32
    L.qsa_debug_force.argtypes = [u32]
    L.qsa_debug_force.restype = ctypes.c_int
    L.qsa_debug_forced.argtypes = []
    L.qsa_debug_forced.restype = u32
    for name in ("qsa_last_error", "qsa_last_path", "qsa_version"):
        getattr(L, name).argtypes = []
        getattr(L, name).restype = ctypes.c_char_p
    _lib = L
    return L


def qsa_last_error() -> str:
    return lib().qsa_last_error().decode()


def qsa_last_path() -> str:
    return lib().qsa_last_path().decode()


def qsa_version() -> str:
    return lib().qsa_version().decode()


def qsa_debug_force(mask: int) -> None:
    """Process-wide arm / scorer override (QSA_DEBUG_FORCE_* bits; 0 clears)."""
    _check(lib().qsa_debug_force(int(mask)))


def qsa_debug_forced() -> int:
    return int(lib().qsa_debug_forced())


class record_events:
    """Arms the next qsa_select_paged_tokens or qsa_compress_keys call on this thread to record
    the given torch.cuda.Event objects between its kernels (see
    qsa_debug_record_events in include/qsa.h).  Keep the object alive until
    that call has returned."""

    def __init__(self, events):
        self.events = list(events)
        for e in self.events:
            if not e.cuda_event:   # torch creates the HIP event on its first record
                e.record()
        self._arr = (ctypes.c_void_p * len(self.events))(*[e.cuda_event for e in self.events])
        _check(lib().qsa_debug_record_events(self._arr, len(self.events)))

    @staticmethod
    def recorded() -> int:
        return int(lib().qsa_debug_events_recorded())


def _check(status: int):
    if status != QSA_OK:
        raise QSAError(status, qsa_last_error())


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _want(t, name, dtype, ndim):
    """Type, dtype, rank and layout of one tensor argument (no device check:
    _on_device runs after every shape relation has been checked, so that a
    mis-shaped argument is reported as such wherever it lives)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(**tensors):
    """Every given tensor (None entries skipped) is a device tensor on the
    first one's device; returns that device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    return dev


def _want_shape(t, name, shape):
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")


def _paged_inputs(q, kcache, page_table, pos, row_req):
    """Structure of the paged inputs shared by the scorer and the indexer."""
    _want(q, "q", torch.float16, 3)
    _want(kcache, "kcache", torch.float16, 3)
    if kcache.shape[2] != q.shape[2]:
        raise ValueError(f"kcache head_dim ({kcache.shape[2]}) differs from q's ({q.shape[2]})")
    _want(page_table, "page_table", torch.int32, 2)
    _want(pos, "pos", torch.int32, 1)
    if row_req is not None:
        _want(row_req, "row_req", torch.int32, 1)
        if row_req.numel() != q.shape[0]:
            raise ValueError("row_req must have one entry per row")
    if pos.numel() != q.shape[0]:
        raise ValueError("pos must have one entry per row")


def _workspace(workspace, need, dev):
    """The caller's workspace (any contiguous device tensor; its bytes count)
    or, when none is given, a fresh allocation of `need` bytes."""
    if workspace is None:
        return (torch.empty(need, dtype=torch.uint8, device=dev), need) if need > 0 else (None, 0)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    _on_device(workspace=workspace)
    if workspace.device != dev:
        raise ValueError(f"workspace is on {workspace.device}, expected {dev}")
    return workspace, workspace.numel() * workspace.element_size()


def qsa_score_paged(q, kcache, page_table, pos, compress_ratio, *, max_visible, row_req=None, flags=0,
                    scores=None, ld_scores=None) -> torch.Tensor:
    """fp32 scores [rows][ld_scores]; entry (r, j) is written for j < V_r only.

    q fp16 [rows, heads, head_dim]; kcache fp16 [num_pages, page_size/cr, head_dim];
    page_table int32 [num_reqs, pt_stride]; pos int32 [rows]; row_req int32 [rows] or None.
    ``max_visible`` is the caller's bound on every row's visible key count
    (the C ABI's argument of that name).  A freshly allocated ``scores`` is
    uninitialised past each row's V_r.
    """
    _paged_inputs(q, kcache, page_table, pos, row_req)
    rows, heads, head_dim = q.shape
    if ld_scores is None:
        ld_scores = max(1, int(max_visible))
    if scores is not None:
        _want(scores, "scores", torch.float32, 2)
        _want_shape(scores, "scores", (rows, ld_scores))
    dev = _on_device(q=q, kcache=kcache, page_table=page_table, pos=pos, row_req=row_req, scores=scores)
    if scores is None:
        scores = torch.empty((rows, ld_scores), dtype=torch.float32, device=dev)
    page_size = kcache.shape[1] * int(compress_ratio)
    _check(lib().qsa_score_paged(
        _ptr(q), _ptr(kcache), _ptr(page_table), page_table.shape[1], kcache.shape[0], page_table.shape[0],
        _ptr(row_req), _ptr(pos), rows, heads, head_dim, page_size, int(compress_ratio), int(max_visible),
        int(flags), _ptr(scores), int(ld_scores), _stream(dev)))
    return scores


def qsa_topk_rows_workspace_size(rows, max_visible, k) -> int:
    return int(lib().qsa_topk_rows_workspace_size(int(rows), int(max_visible), int(k)))


def qsa_topk_rows(scores, k, *, visible=None, max_visible=None, out=None, workspace=None) -> torch.Tensor:
    """Exact top-k key indices per row of ``scores`` [rows, ld] (rank order,
    -1 padded); ``max_visible`` defaults to the width ld."""
    _want(scores, "scores", torch.float32, 2)
    rows, ld = scores.shape
    if visible is not None:
        _want(visible, "visible", torch.int32, 1)
        if visible.numel() != rows:
            raise ValueError("visible must have one entry per row")
    if out is not None:
        _want(out, "out", torch.int32, 2)
        _want_shape(out, "out", (rows, k))
    dev = _on_device(scores=scores, visible=visible, out=out)
    if max_visible is None:
        max_visible = ld
    if out is None:
        out = torch.empty((rows, int(k)), dtype=torch.int32, device=dev)
    workspace, wbytes = _workspace(workspace, qsa_topk_rows_workspace_size(rows, max_visible, k), dev)
    _check(lib().qsa_topk_rows(_ptr(scores), ld, _ptr(visible), rows, int(max_visible), int(k), _ptr(out),
                               _ptr(workspace), wbytes, _stream(dev)))
    return out


def qsa_sparse_attention_workspace_size(rows, q_heads, kv_heads, head_dim, k) -> int:
    return int(lib().qsa_sparse_attention_workspace_size(int(rows), int(q_heads), int(kv_heads), int(head_dim),
                                                         int(k)))


def qsa_sparse_attention(q, k_cache, v_cache, page_table, tokens, *, row_req=None, scale=None,
                         out=None, workspace=None) -> torch.Tensor:
    """Softmax attention of every query head over the tokens listed per row
    (entries < 0 skipped), K/V gathered from the paged main cache
    [pages][page_size][kv_heads][head_dim]; fp32 [rows, q_heads, head_dim].
    ``scale`` defaults to 1/sqrt(head_dim)."""
    _want(q, "q", torch.float16, 3)
    _want(k_cache, "k_cache", torch.float16, 4)
    _want(v_cache, "v_cache", torch.float16, 4)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    _want(page_table, "page_table", torch.int32, 2)
    _want(tokens, "tokens", torch.int32, 2)
    rows, q_heads, head_dim = q.shape
    if tokens.shape[0] != rows:
        raise ValueError("tokens must have one row per query row")
    if row_req is not None:
        _want(row_req, "row_req", torch.int32, 1)
        if row_req.numel() != rows:
            raise ValueError("row_req must have one entry per row")
    num_pages, page_size, kv_heads, kd = k_cache.shape
    if kd != head_dim:
        raise ValueError("k_cache head_dim differs from q's")
    if out is not None:
        _want(out, "out", torch.float32, 3)
        _want_shape(out, "out", (rows, q_heads, head_dim))
    dev = _on_device(q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table, tokens=tokens, row_req=row_req,
                     out=out)
    if scale is None:
        scale = 1.0 / float(head_dim) ** 0.5
    if out is None:
        out = torch.empty((rows, q_heads, head_dim), dtype=torch.float32, device=dev)
    need = qsa_sparse_attention_workspace_size(rows, q_heads, kv_heads, head_dim, tokens.shape[1])
    workspace, wbytes = _workspace(workspace, need, dev)
    _check(lib().qsa_sparse_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), page_table.shape[1], num_pages,
        page_table.shape[0], _ptr(row_req), _ptr(tokens), tokens.shape[1], rows, q_heads, kv_heads, head_dim,
        page_size, float(scale), _ptr(out), _ptr(workspace), wbytes, _stream(dev)))
    return out


def qsa_compress_keys(k_tok, tok_pos, state, kcache, page_table, compress_ratio, *, tok_req=None, norm_w=None,
                      eps=1e-6, rope_dim=128, rope_base=10000.0, interleaved=False) -> None:
    """Compressed-key producer: finishes every block of compress_ratio tokens
    whose last token is in this call (mean pool, RMSNorm, RoPE at the block
    start, fp16) into its slot of kcache [pages][page_size/cr][128], and keeps
    the raw keys of blocks left open in state [num_reqs][cr][128]."""
    _want(k_tok, "k_tok", torch.float16, 2)
    tokens, head_dim = k_tok.shape
    _want(tok_pos, "tok_pos", torch.int32, 1)
    if tok_pos.numel() != tokens:
        raise ValueError("tok_pos must have one entry per token")
    if tok_req is not None:
        _want(tok_req, "tok_req", torch.int32, 1)
        if tok_req.numel() != tokens:
            raise ValueError("tok_req must have one entry per token")
    _want(kcache, "kcache", torch.float16, 3)
    _want(page_table, "page_table", torch.int32, 2)
    if state is not None:
        _want(state, "state", torch.float16, 3)
        if state.shape != (page_table.shape[0], int(compress_ratio), head_dim):
            raise ValueError("state must be [num_reqs, compress_ratio, head_dim]")
    if norm_w is not None:
        _want(norm_w, "norm_w", torch.float32, 1)
        if norm_w.numel() != head_dim:
            raise ValueError("norm_w must have head_dim entries")
    if kcache.shape[2] != head_dim:
        raise ValueError("kcache head_dim differs from k_tok's")
    dev = _on_device(k_tok=k_tok, tok_pos=tok_pos, tok_req=tok_req, kcache=kcache, page_table=page_table,
                     state=state, norm_w=norm_w)
    page_size = kcache.shape[1] * int(compress_ratio)
    flags = QSA_ROPE_INTERLEAVED if interleaved else 0
    _check(lib().qsa_compress_keys(
        _ptr(k_tok), _ptr(tok_req), _ptr(tok_pos), tokens, head_dim, _ptr(norm_w), float(eps), int(rope_dim),
        float(rope_base), flags, _ptr(state), _ptr(kcache), _ptr(page_table), page_table.shape[1], kcache.shape[0],
        page_table.shape[0], page_size, int(compress_ratio), _stream(dev)))


def qsa_select_paged_tokens_workspace_size(rows, num_reqs, max_visible, compress_ratio, k, flags=0) -> int:
    return int(lib().qsa_select_paged_tokens_workspace_size(int(rows), int(num_reqs), int(max_visible),
                                                            int(compress_ratio), int(k), int(flags)))


def qsa_select_paged_tokens(q, kcache, page_table, pos, compress_ratio, k, *, max_visible, row_req=None,
                            flags=0, out=None, workspace=None) -> torch.Tensor:
    """The whole indexer: int32 [rows, k] token indices (or key indices with
    QSA_OUT_KEYS), rank order, -1 padded.  ``max_visible`` is the caller's
    bound on every row's visible key count (the C ABI's argument)."""
    _paged_inputs(q, kcache, page_table, pos, row_req)
    rows, heads, head_dim = q.shape
    num_reqs = page_table.shape[0]
    if out is not None:
        _want(out, "out", torch.int32, 2)
        _want_shape(out, "out", (rows, k))
    dev = _on_device(q=q, kcache=kcache, page_table=page_table, pos=pos, row_req=row_req, out=out)
    if out is None:
        out = torch.empty((rows, int(k)), dtype=torch.int32, device=dev)
    need = qsa_select_paged_tokens_workspace_size(rows, num_reqs, max_visible, compress_ratio, k, flags)
    workspace, wbytes = _workspace(workspace, need, dev)
    page_size = kcache.shape[1] * int(compress_ratio)
    _check(lib().qsa_select_paged_tokens(
        _ptr(q), _ptr(kcache), _ptr(page_table), page_table.shape[1], kcache.shape[0], num_reqs,
        _ptr(row_req), _ptr(pos), rows, heads, head_dim, page_size, int(compress_ratio), int(max_visible),
        int(k), int(flags), _ptr(out), _ptr(workspace), wbytes, _stream(dev)))
    return out


def qsa_select_paged_tokens_noalloc(q, kcache, page_table, pos, compress_ratio, k, *, max_visible, out,
                                    row_req=None, flags=0) -> torch.Tensor:
    """qsa_select_paged_tokens without a workspace (the library's static
    per-device scratch of QSA_NOALLOC_SCRATCH_BYTES); the caller passes
    ``out`` int32 [rows, k], so nothing is allocated.  Calls that overlap on
    one device race on the shared scratch."""
    _paged_inputs(q, kcache, page_table, pos, row_req)
    rows, heads, head_dim = q.shape
    _want(out, "out", torch.int32, 2)
    _want_shape(out, "out", (rows, k))
    dev = _on_device(q=q, kcache=kcache, page_table=page_table, pos=pos, row_req=row_req, out=out)
    page_size = kcache.shape[1] * int(compress_ratio)
    _check(lib().qsa_select_paged_tokens_noalloc(
        _ptr(q), _ptr(kcache), _ptr(page_table), page_table.shape[1], kcache.shape[0], page_table.shape[0],
        _ptr(row_req), _ptr(pos), rows, heads, head_dim, page_size, int(compress_ratio), int(max_visible),
        int(k), int(flags), _ptr(out), _stream(dev)))
    return out
