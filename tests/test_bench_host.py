"""Host-side accounting of bench.py (CPU only): the algorithmic work every
roofline figure divides by, counted here by brute force over small batches.

- prefill: 4 * D flops per unmasked (query row, head, key) triple; a causal
  query t of a request with qlen new tokens and kv_len keys sees keys
  0 .. kv_len - qlen + t (the bottom-right alignment of the causal mask), a
  non-causal one sees all kv_len keys;
- decode: every KV token's K and V row of every KV head read once, the
  queries read and the output rows and LSE written once, plus page ids,
  lengths, offsets and sinks.
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import pytest

import bench
import workloads as W


def brute_pairs(qlens, kv_lens, hq, causal):
    n = 0
    for ql, kl in zip(qlens, kv_lens):
        for t in range(ql):
            for j in range(kl):
                if not causal or j <= kl - ql + t:
                    n += 1
    return n * hq


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("qlens,kv_lens", [([1], [1]), ([5, 0, 17], [5, 9, 40]),
                                           ([64, 3], [64, 200]), ([33], [33])])
def test_prefill_pairs_count_the_unmasked_triples(qlens, kv_lens, causal):
    b = W.make_batch(3, kind="prefill", qlens=qlens, kv_lens=kv_lens, hq=4, hkv=2,
                     causal=causal)
    assert bench.prefill_pairs(b) == brute_pairs(qlens, kv_lens, 4, causal)
    assert bench.prefill_flops(b) == 4 * 64 * brute_pairs(qlens, kv_lens, 4, causal)


def test_causal_workload_pair_count_closed_form():
    # 8 requests of 4,096 tokens, 64 heads: 64 * 8 * 4096 * 4097 / 2 triples
    # (only the lengths are needed, not the tensors)
    b = SimpleNamespace(qo_indptr=np.arange(9, dtype=np.int32) * 4096,
                        kv_len=np.full(8, 4096, np.int32), num_qo_heads=64, head_dim=64,
                        causal=True)
    assert bench.prefill_pairs(b) == 64 * 8 * 4096 * 4097 // 2
    assert bench.prefill_flops(b) == 1_099_780_063_232


def test_decode_bytes_by_enumeration():
    L = [1, 16, 17, 300]
    b = W.make_batch(5, kind="decode", qlens=[1] * 4, kv_lens=L, hq=8, hkv=2, paged=True)
    kv = sum(L) * 2 * 2 * 64 * 2                       # K and V, 2 KV heads, 64 dims, bf16
    q = 4 * 8 * 64 * 2                                 # one bf16 query row per head
    out = 4 * 8 * 64 * 4 + 4 * 8 * 4                   # fp32 rows and their LSE
    pages = sum((l + 15) // 16 for l in L) * 4
    meta = 4 * 4 + 5 * 4 + 8 * 4                       # lengths, page offsets, sinks
    assert bench.decode_algorithmic_bytes(b) == kv + q + out + pages + meta
    assert bench.kv_bytes_of(b) == kv
