"""Brute-force sink attention in numpy (fp64).  TEST INFRASTRUCTURE ONLY.

A second, independent formulation of the definition the C oracle computes
(GPT-OSS on Day 0, Perplexity; "Attention: GQA with attention sinks" and
"Sink attention" under "Kernels for GPT-OSS"): for each request and query
head, build the full score matrix, append the head's sink as one extra
column of logits, take a textbook softmax over each row, drop the sink
column (it has no value vector) and multiply by V.  Meant for small shapes.

With a draft mask ("Accelerating Sonar Through Speculation", Perplexity,
section "EAGLE": tree drafts are verified under custom attention masks) the
allowed-key matrix is built from the bits directly: prefix keys always,
drafted key i of the request when bit i of the row's mask is set.
"""
from __future__ import annotations

import numpy as np


def _f(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) \
        .view(np.float32).astype(np.float64)


def _gather_kv(b, req: int):
    """K and V of one request as [L, Hkv, D] float64 arrays."""
    L = int(b.kv_len[req]) if b.kv_len is not None else int(b.kv_indptr[req + 1] - b.kv_indptr[req])
    if b.page_indices is None:
        s = int(b.kv_indptr[req])
        return _f(b.k[s:s + L]), _f(b.v[s:s + L])
    ps = b.page_size
    pages = b.page_indices[b.kv_indptr[req]:b.kv_indptr[req + 1]]
    # [n_pages, Hkv, ps, D] -> [n_pages*ps, Hkv, D] -> first L tokens
    k = _f(b.k[pages]).transpose(0, 2, 1, 3).reshape(-1, b.num_kv_heads, b.head_dim)[:L]
    v = _f(b.v[pages]).transpose(0, 2, 1, 3).reshape(-1, b.num_kv_heads, b.head_dim)[:L]
    return k, v


def brute(b, key_begin: int = 0, key_end: int | None = None, include_sink: bool = True):
    """Returns out [total_q, Hq, D], lse [total_q, Hq] in float64."""
    Hq, Hkv, D = b.num_qo_heads, b.num_kv_heads, b.head_dim
    G = Hq // Hkv
    total_q = int(b.qo_indptr[-1])
    out = np.zeros((total_q, Hq, D))
    lse = np.zeros((total_q, Hq))
    B = len(b.qo_indptr) - 1
    for r in range(B):
        q0, q1 = int(b.qo_indptr[r]), int(b.qo_indptr[r + 1])
        n = q1 - q0
        if n == 0:
            continue
        k, v = _gather_kv(b, r)
        L = k.shape[0]
        q = _f(b.q[q0:q1])                       # [n, Hq, D]
        pos = L - n + np.arange(n)               # absolute query positions
        keys = np.arange(L)
        allowed = np.ones((n, L), dtype=bool)
        dmask = getattr(b, "draft_mask", None)
        if dmask is not None:
            bits = np.array([[(int(dmask[q0 + t]) >> i) & 1 for i in range(n)]
                             for t in range(n)], dtype=bool)          # [n, n]
            allowed[:, L - n:] = bits
        elif b.causal:
            allowed &= keys[None, :] <= pos[:, None]
        allowed &= keys[None, :] >= key_begin
        if key_end is not None:
            allowed &= keys[None, :] < key_end
        for h in range(Hq):
            g = h // G
            s = b.sm_scale * (q[:, h, :] @ k[:, g, :].T)        # [n, L]
            s = np.where(allowed, s, -np.inf)
            sig = float(b.sinks[h]) if (include_sink and b.sinks is not None) else -np.inf
            z = np.concatenate([s, np.full((n, 1), sig)], axis=1)  # sink = extra column
            m = z.max(axis=1, keepdims=True)
            for i in range(n):
                if m[i, 0] == -np.inf:
                    out[q0 + i, h] = 0.0
                    lse[q0 + i, h] = -np.inf
                    continue
                if m[i, 0] == np.inf:
                    out[q0 + i, h] = 0.0
                    lse[q0 + i, h] = np.inf
                    continue
                e = np.exp(z[i] - m[i, 0])
                p = e / e.sum()
                out[q0 + i, h] = p[:-1] @ v[:, g, :]             # sink column dropped
                lse[q0 + i, h] = m[i, 0] + np.log(e.sum())
    return out, lse
