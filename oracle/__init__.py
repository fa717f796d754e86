"""Sink-attention oracle (fp64, CPU).  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library and neither
imports the other.

Two independent formulations of one definition (GPT-OSS on Day 0,
Perplexity; section "Sink attention" under "Kernels for GPT-OSS" and the
"Attention: GQA with attention sinks" list):

* ``attend`` / ``partial`` / ``attend_rows`` / ``row_weights`` / ``merge``:
  the C file ``sink_attn_oracle.c``, three literal passes per row in fp64,
  OpenMP over rows;
* ``brute`` (``brute.py``): numpy, per request and head, concatenates the
  sink as one extra logit column, takes a textbook softmax, drops that
  column and multiplies by V.

Batches are duck-typed: any object with the attributes q, qo_indptr, k, v,
kv_indptr, page_indices, kv_len, sinks, num_qo_heads, num_kv_heads,
head_dim, page_size, sm_scale and causal, and optionally draft_mask (uint64
per query row; layouts in the C file's header).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

from .brute import brute  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sink_attn_oracle.c")
_LIB = os.path.join(_HERE, "libsink_attn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle (gcc, -O2, OpenMP) next to its source."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        ctx = [P, P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
               ctypes.c_int, ctypes.c_double, ctypes.c_int, P]
        L.sa_oracle_partial.argtypes = ctx + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                              P, P, ctypes.c_int]
        L.sa_oracle_attend.argtypes = ctx + [P, P, ctypes.c_int]
        L.sa_oracle_attend_rows.argtypes = ctx + [P, P, ctypes.c_int64, P, P, ctypes.c_int]
        L.sa_oracle_row_weights.argtypes = ctx + [ctypes.c_int64, ctypes.c_int, P, P, P, P, P, P]
        L.sa_oracle_merge.argtypes = [P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, P, P]
        for f in ("sa_oracle_partial", "sa_oracle_attend", "sa_oracle_attend_rows",
                  "sa_oracle_row_weights", "sa_oracle_merge"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _ctx(b):
    """Marshal a batch; returns (argument tuple, arrays kept alive)."""
    keep = []

    def arr(x, dt):
        if x is None:
            return None
        a = np.ascontiguousarray(x, dtype=dt)
        keep.append(a)
        return a

    q = arr(b.q, np.uint16)
    qo = arr(b.qo_indptr, np.int32)
    k = arr(b.k, np.uint16)
    v = arr(b.v, np.uint16)
    kvi = arr(b.kv_indptr, np.int32)
    pi = arr(b.page_indices, np.int32)
    kl = arr(b.kv_len, np.int32)
    s = arr(b.sinks, np.float32)
    dm = arr(getattr(b, "draft_mask", None), np.uint64)
    args = (_ptr(q), _ptr(qo), _ptr(k), _ptr(v), _ptr(kvi), _ptr(pi), _ptr(kl), _ptr(s),
            int(qo.shape[0] - 1), int(b.num_qo_heads), int(b.num_kv_heads), int(b.head_dim),
            int(b.page_size), float(b.sm_scale), int(bool(b.causal)), _ptr(dm))
    return args, keep, int(qo[-1])


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def partial(b, key_begin: int, key_end: int, include_sink: bool,
            nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Attention restricted to keys [key_begin, key_end) of each row's allowed
    set, with the sink iff include_sink.  Returns out [total_q, Hq, D] and
    lse [total_q, Hq] (fp64, natural log)."""
    args, keep, total_q = _ctx(b)
    out = np.zeros((total_q, b.num_qo_heads, b.head_dim), dtype=np.float64)
    lse = np.zeros((total_q, b.num_qo_heads), dtype=np.float64)
    rc = lib().sa_oracle_partial(*args, int(key_begin), int(key_end), int(bool(include_sink)),
                                 _ptr(out), _ptr(lse), int(nthreads))
    _check(rc, "partial")
    return out, lse


def attend(b, nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """The full method over every (query row, head)."""
    args, keep, total_q = _ctx(b)
    out = np.zeros((total_q, b.num_qo_heads, b.head_dim), dtype=np.float64)
    lse = np.zeros((total_q, b.num_qo_heads), dtype=np.float64)
    rc = lib().sa_oracle_attend(*args, _ptr(out), _ptr(lse), int(nthreads))
    _check(rc, "attend")
    return out, lse


def attend_rows(b, rows, heads, nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """The full method on sampled (query row, head) pairs: out [n, D], lse [n]."""
    args, keep, _ = _ctx(b)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    n = rows.shape[0]
    out = np.zeros((n, b.head_dim), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    rc = lib().sa_oracle_attend_rows(*args, _ptr(rows), _ptr(heads), n, _ptr(out), _ptr(lse),
                                     int(nthreads))
    _check(rc, "attend_rows")
    return out, lse


def row_weights(b, row: int, head: int):
    """Softmax weights of one (row, head): (weights over allowed keys j0..j1-1,
    sink weight, j0, j1, o, lse)."""
    args, keep, _ = _ctx(b)
    L = int(np.max(b.kv_len)) if b.kv_len is not None else int(np.max(np.diff(b.kv_indptr)))
    w = np.zeros(max(L, 1), dtype=np.float64)
    ws = np.zeros(1, dtype=np.float64)
    j0 = np.zeros(1, dtype=np.int64)
    j1 = np.zeros(1, dtype=np.int64)
    o = np.zeros(b.head_dim, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    rc = lib().sa_oracle_row_weights(*args, int(row), int(head), _ptr(w), _ptr(ws), _ptr(j0),
                                     _ptr(j1), _ptr(o), _ptr(lse))
    _check(rc, "row_weights")
    n = int(j1[0] - j0[0])
    return w[:n].copy(), float(ws[0]), int(j0[0]), int(j1[0]), o, float(lse[0])


def merge(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """LSE merge of normalised partials o_parts [N, H, S, D], lse_parts
    [N, H, S] -> out [N, H, D], lse [N, H]."""
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    N, H, S, D = o_parts.shape
    assert lse_parts.shape == (N, H, S)
    out = np.zeros((N, H, D), dtype=np.float64)
    lse = np.zeros((N, H), dtype=np.float64)
    rc = lib().sa_oracle_merge(_ptr(o_parts), _ptr(lse_parts), N, H, S, D, _ptr(out), _ptr(lse))
    _check(rc, "merge")
    return out, lse
