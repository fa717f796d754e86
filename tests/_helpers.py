"""Small shared helpers for the tests (no attention arithmetic here)."""
from __future__ import annotations

import numpy as np

from workloads import Batch, to_bf16_bits

# (case name, elements compared, max-abs error, relative L2 error) of every
# parity check of the session, for the terminal summary.
PARITY_RECORD: list = []


def batch_from_values(q, k, v, *, qlens, kv_lens, hq, hkv, d, sinks, sm_scale, causal,
                      kind="prefill") -> Batch:
    """Contiguous batch from explicit (bf16-exact) float values.
    q [total_q, Hq, D], k/v [total_kv, Hkv, D]."""
    q = np.asarray(q, dtype=np.float32).reshape(-1, hq, d)
    k = np.asarray(k, dtype=np.float32).reshape(-1, hkv, d)
    v = np.asarray(v, dtype=np.float32).reshape(-1, hkv, d)
    qb, kb, vb = to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)
    assert np.array_equal((qb.astype(np.uint32) << 16).view(np.float32), q), "q not bf16-exact"
    if k.size == 0:
        kb = np.zeros((1, hkv, d), np.uint16)
        vb = np.zeros((1, hkv, d), np.uint16)
    qo = np.zeros(len(qlens) + 1, np.int32)
    qo[1:] = np.cumsum(qlens)
    kvi = np.zeros(len(kv_lens) + 1, np.int32)
    kvi[1:] = np.cumsum(kv_lens)
    s = None if sinks is None else np.asarray(sinks, dtype=np.float32).reshape(hq)
    return Batch(kind=kind, q=qb, qo_indptr=qo, k=kb, v=vb, kv_indptr=kvi, page_indices=None,
                 kv_len=np.asarray(kv_lens, np.int32), sinks=s, num_qo_heads=hq,
                 num_kv_heads=hkv, head_dim=d, page_size=16, sm_scale=sm_scale, causal=causal)


def to_paged(b: Batch, page_size: int, rng=None) -> Batch:
    """Re-lay a contiguous batch as a paged cache (optionally permuted pages)."""
    assert b.page_indices is None
    B = b.batch
    L = b.kv_len.astype(np.int64)
    pages_per = (L + page_size - 1) // page_size
    indptr = np.zeros(B + 1, np.int32)
    indptr[1:] = np.cumsum(pages_per)
    P = int(indptr[-1])
    perm = np.arange(P) if rng is None else rng.permutation(P)
    perm = perm.astype(np.int32)
    kp = np.full((max(P, 1), b.num_kv_heads, page_size, b.head_dim), 0x4100, np.uint16)  # 8.0
    vp = np.full_like(kp, 0x42C8)  # 100.0
    for r in range(B):
        s = int(b.kv_indptr[r])
        for j in range(int(L[r])):
            page = perm[indptr[r] + j // page_size]
            kp[page, :, j % page_size, :] = b.k[s + j]
            vp[page, :, j % page_size, :] = b.v[s + j]
    return Batch(kind=b.kind, q=b.q, qo_indptr=b.qo_indptr, k=kp, v=vp, kv_indptr=indptr,
                 page_indices=perm, kv_len=b.kv_len, sinks=b.sinks, num_qo_heads=b.num_qo_heads,
                 num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, page_size=page_size,
                 sm_scale=b.sm_scale, causal=b.causal, out_dtype=b.out_dtype,
                 num_splits=b.num_splits)


def rel_l2(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((a - ref).ravel())
    return float(num / den) if den > 0 else float(num)
