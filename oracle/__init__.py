"""ctypes front end of the CPU oracle (``qsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The GPU library and its Python
binding never import this package; the two implementations share no code.

Every function takes NumPy arrays (fp16 data as ``np.float16``), copies them to
contiguous buffers of the exact C types and calls the plain C oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

SCORE_RELU = 1
OUT_KEYS = 2

_lib = None


def build() -> str:
    """Compile the oracle with gcc: no fast-math, no FMA contraction."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-o", _LIB + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, u32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    lib.oracle_half_to_float.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_float.restype = ctypes.c_float
    lib.oracle_visible_keys.argtypes = [i32, i32]
    lib.oracle_visible_keys.restype = i32
    lib.oracle_score_paged.argtypes = [P, P, P, i64, P, P, i32, i32, i32, i32, i32, u32, P, i64, i32]
    lib.oracle_score_paged.restype = None
    lib.oracle_select_rows.argtypes = [P, i64, P, i32, i32, P, i32]
    lib.oracle_select_rows.restype = None
    lib.oracle_select_paged_tokens.argtypes = [P, P, P, i64, P, P, i32, i32, i32, i32, i32, i32, u32, P, i32]
    lib.oracle_select_paged_tokens.restype = None
    _lib = lib
    return lib


def _threads(nthreads):
    return int(nthreads) if nthreads else (os.cpu_count() or 1)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def half_to_float(bits: int) -> float:
    return float(_load().oracle_half_to_float(int(bits) & 0xFFFF))


def visible_keys(pos: int, compress_ratio: int) -> int:
    return int(_load().oracle_visible_keys(int(pos), int(compress_ratio)))


def _paged_args(q, kcache, page_table, row_req, pos):
    q = _c(q, np.float16)
    kcache = _c(kcache, np.float16)
    page_table = _c(page_table, np.int32)
    if page_table.ndim == 1:
        page_table = page_table[None, :]
    row_req = None if row_req is None else _c(row_req, np.int32)
    pos = _c(pos, np.int32)
    rows, heads, head_dim = q.shape
    return q, kcache, page_table, row_req, pos, rows, heads, head_dim


def score_paged(q, kcache, page_table, pos, compress_ratio, row_req=None, flags=0,
                ld=None, nthreads=None):
    """fp32 scores [rows][ld]; entries j >= visible count are NaN-filled here
    (the oracle itself leaves them untouched)."""
    q, kcache, page_table, row_req, pos, rows, heads, head_dim = _paged_args(
        q, kcache, page_table, row_req, pos)
    page_size = kcache.shape[1] * compress_ratio
    vmax = int(max([visible_keys(p, compress_ratio) for p in pos] + [0]))
    ld = int(ld) if ld is not None else max(vmax, 1)
    out = np.full((rows, ld), np.nan, dtype=np.float32)
    _load().oracle_score_paged(
        _ptr(q), _ptr(kcache), _ptr(page_table), page_table.shape[1], _ptr(row_req), _ptr(pos),
        rows, heads, head_dim, page_size, compress_ratio, flags, _ptr(out), ld, _threads(nthreads))
    return out


def select_rows(scores, visible, k, nthreads=None):
    """Exact lexicographic top-k key indices per row, rank order, -1 padded."""
    scores = _c(scores, np.float32)
    rows, ld = scores.shape
    visible = _c(visible, np.int32)
    assert visible.shape == (rows,)
    assert int(visible.max(initial=0)) <= ld
    out = np.empty((rows, k), dtype=np.int32)
    _load().oracle_select_rows(_ptr(scores), ld, _ptr(visible), rows, k, _ptr(out), _threads(nthreads))
    return out


def select_paged_tokens(q, kcache, page_table, pos, compress_ratio, k, row_req=None,
                        flags=0, nthreads=None):
    """The whole indexer: int32 [rows][k], -1 padded."""
    q, kcache, page_table, row_req, pos, rows, heads, head_dim = _paged_args(
        q, kcache, page_table, row_req, pos)
    page_size = kcache.shape[1] * compress_ratio
    out = np.empty((rows, k), dtype=np.int32)
    _load().oracle_select_paged_tokens(
        _ptr(q), _ptr(kcache), _ptr(page_table), page_table.shape[1], _ptr(row_req), _ptr(pos),
        rows, heads, head_dim, page_size, compress_ratio, k, flags, _ptr(out), _threads(nthreads))
    return out
