"""Pins of the oracle's draft (tree) mask, on the CPU.

"Accelerating Sonar Through Speculation" (Perplexity), section "EAGLE": a
tree of drafted tokens is verified in one target pass under a custom
attention mask.  The oracle's reading: row t of a request with qlen drafted
tokens sees every prefix key (j < P = kv_len - qlen) and drafted key P + i
exactly when bit i of its mask word is set.

Each pin ties the masked oracle to something other than itself: the causal
path (a linear draft), a single-query decode over the keys of the row's
tree path gathered into a fresh cache, the key-window partial (no drafted
key visible), and the numpy brute force, which builds the allowed matrix
from the bits independently.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from tests._helpers import batch_from_values
from workloads import bf16_bits_to_f32, make_batch


def _with_mask(b, mask):
    b.draft_mask = np.asarray(mask, dtype=np.uint64)
    return b


def _tree_masks(rng, qlens):
    return np.concatenate([W.tree_mask(W.draft_tree(rng, int(n))) if n else
                           np.zeros(0, np.uint64) for n in qlens])


@pytest.mark.parametrize("paged", [False, True])
def test_linear_draft_equals_causal(paged):
    """A chain mask (token t sees drafted tokens 0..t) is causal attention."""
    qlens, kvl = [1, 7, 16, 3], [1, 40, 16, 90]
    b = make_batch(901, kind="prefill", qlens=qlens, kv_lens=kvl, hq=8, hkv=2, paged=paged,
                   sinks="normal", causal=True)
    o, l = oracle.attend(b)
    m = _with_mask(b, np.concatenate([W.chain_mask(n) for n in qlens]))
    om, lm = oracle.attend(m)
    np.testing.assert_array_equal(om, o)
    np.testing.assert_array_equal(lm, l)


def test_tree_row_equals_decode_over_its_path():
    """Row t equals one decode query over the prefix followed by the keys of
    t's ancestors and t itself (in cache order), gathered into a new cache."""
    rng = np.random.default_rng(902)
    n, P, hq, hkv = 12, 37, 8, 2
    parents = W.draft_tree(rng, n, max_children=3)
    b = make_batch(rng, kind="prefill", qlens=[n], kv_lens=[P + n], hq=hq, hkv=hkv,
                   sinks="normal", causal=True)
    _with_mask(b, W.tree_mask(parents))
    o, l = oracle.attend(b)
    k, v = bf16_bits_to_f32(b.k), bf16_bits_to_f32(b.v)
    for t in range(n):
        path = []
        j = t
        while j >= 0:
            path.append(j)
            j = int(parents[j])
        keys = list(range(P)) + [P + j for j in sorted(path)]
        dec = batch_from_values(bf16_bits_to_f32(b.q[t:t + 1]), k[keys], v[keys], qlens=[1],
                                kv_lens=[len(keys)], hq=hq, hkv=hkv, d=64, sinks=b.sinks,
                                sm_scale=b.sm_scale, causal=True, kind="decode")
        od, ld = oracle.attend(dec)
        np.testing.assert_allclose(o[t], od[0], rtol=0, atol=1e-14, err_msg=f"token {t}")
        np.testing.assert_allclose(l[t], ld[0], rtol=0, atol=1e-14)
    # a transposed mask (descendants instead of ancestors) is a different result
    mt = np.zeros(n, np.uint64)
    for i in range(n):
        for j in range(n):
            if (int(b.draft_mask[j]) >> i) & 1:
                mt[i] |= np.uint64(1 << j)
    assert not np.array_equal(mt, b.draft_mask)
    ot, _ = oracle.attend(_with_mask(b, mt))
    assert np.max(np.abs(ot - o)) > 1e-3


def test_no_visible_draft_equals_prefix_window():
    """All-zero bits: each row sees only the prefix, i.e. the key-window
    partial over [0, P) with the sink."""
    for qlen, L in [(5, 50), (1, 1), (9, 9)]:
        b = make_batch(903 + L, kind="prefill", qlens=[qlen], kv_lens=[L], hq=4, hkv=1,
                       sinks="normal", causal=False)
        ref_o, ref_l = oracle.partial(b, 0, L - qlen, include_sink=True)
        o, l = oracle.attend(_with_mask(b, np.zeros(qlen, np.uint64)))
        np.testing.assert_array_equal(o, ref_o)
        np.testing.assert_array_equal(l, ref_l)


def test_bits_at_or_above_qlen_are_ignored():
    rng = np.random.default_rng(904)
    qlens, kvl = [6, 2, 33], [20, 2, 70]
    b = make_batch(rng, kind="prefill", qlens=qlens, kv_lens=kvl, hq=8, hkv=4, paged=True,
                   sinks="normal", causal=True)
    m = _tree_masks(rng, qlens)
    o, l = oracle.attend(_with_mask(b, m))
    junk = m.copy()
    r = 0
    for n in qlens:
        for t in range(n):
            noise = int(rng.integers(0, 1 << 63, dtype=np.int64))
            junk[r + t] |= np.uint64(noise & ~((1 << n) - 1))
        r += n
    oj, lj = oracle.attend(_with_mask(b, junk))
    np.testing.assert_array_equal(oj, o)
    np.testing.assert_array_equal(lj, l)


def test_masked_weights_are_zero_and_sum_to_one():
    rng = np.random.default_rng(905)
    n, P = 10, 23
    b = make_batch(rng, kind="prefill", qlens=[n], kv_lens=[P + n], hq=4, hkv=1,
                   sinks="normal", causal=True)
    _with_mask(b, W.tree_mask(W.draft_tree(rng, n)))
    for t in range(n):
        w, ws, j0, j1, o, lse = oracle.row_weights(b, t, 1)
        bits = int(b.draft_mask[t])
        for j in range(j0, j1):
            seen = j < P or (bits >> (j - P)) & 1
            assert (w[j - j0] > 0) == bool(seen), (t, j)
        assert abs(w.sum() + ws - 1.0) < 1e-13


def test_draft_mask_c_oracle_agrees_with_brute_force():
    """Arbitrary bit patterns (not only trees), sinks including +-inf."""
    rng = np.random.default_rng(906)
    for case in range(40):
        B = int(rng.integers(1, 4))
        hkv = int(rng.choice([1, 2]))
        hq = hkv * int(rng.choice([1, 2, 4]))
        d = int(rng.choice([4, 64]))
        qlens = rng.integers(0, 9, size=B)
        kvl = qlens + rng.integers(0, 30, size=B)
        kvl[kvl == 0] = 1
        qlens = np.minimum(qlens, kvl)
        sinks = "normal" if case % 3 else np.array(
            rng.choice([-np.inf, np.inf, -1e4, 10.0, 0.0], size=hq), np.float32)
        b = make_batch(int(rng.integers(1 << 30)), kind="prefill", qlens=qlens, kv_lens=kvl,
                       hq=hq, hkv=hkv, d=d, paged=bool(case % 2),
                       page_size=int(rng.choice([1, 4, 16])), sinks=sinks, sink_std=3.0,
                       causal=bool(rng.integers(0, 2)))
        total = int(qlens.sum())
        m = rng.integers(0, 1 << 63, size=total, dtype=np.int64).astype(np.uint64)
        if case % 4 == 0:
            m = _tree_masks(rng, qlens)
        _with_mask(b, m)
        o, l = oracle.attend(b)
        bo, bl = oracle.brute(b)
        np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12, err_msg=str(case))
        fin = np.isfinite(bl)
        assert np.array_equal(np.isfinite(l), fin)
        np.testing.assert_allclose(l[fin], bl[fin], rtol=0, atol=1e-12)
        assert np.array_equal(l[~fin], bl[~fin])


def test_tree_generator_structure():
    """Input recipe: parents precede children, trees are breadth-first
    consistent, and every token sees itself and its parent's bits."""
    rng = np.random.default_rng(907)
    for n in (1, 2, 16, 64):
        p = W.draft_tree(rng, n)
        assert p[0] == -1 and np.all(p < np.arange(n))
        m = W.tree_mask(p)
        for i in range(n):
            w = int(m[i])
            assert (w >> i) & 1 and w < (1 << (i + 1))
            if p[i] >= 0:
                assert w == int(m[p[i]]) | (1 << i)
            else:
                assert w == 1 << i
