"""Pins for the fp64 oracle (CPU only).

The pages print no numeric example, so every pin here comes from the
definition (GPT-OSS on Day 0, "Attention: GQA with attention sinks" and
"Sink attention"): hand-worked closed forms, a special case that reduces to
a library routine (torch SDPA), identities of the softmax, and a second,
independent formulation (numpy brute force).  Each is chosen so that a
plausible slip in the oracle (a dropped sink term, a sink with a value, a
scaled sink, a wrong GQA head map, a mis-aligned causal mask, a wrong page
index, a sink in every split chunk) fails at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests._helpers import batch_from_values, rel_l2, to_paged
from workloads import bf16_bits_to_f32, make_batch, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _sdpa_std(b, req):
    """Standard (sink-free) attention of one contiguous request via torch SDPA
    in fp64 on the CPU, with the bottom-right causal alignment as a mask."""
    q0, q1 = int(b.qo_indptr[req]), int(b.qo_indptr[req + 1])
    k0, k1 = int(b.kv_indptr[req]), int(b.kv_indptr[req + 1])
    q = torch.from_numpy(bf16_bits_to_f32(b.q[q0:q1]).astype(np.float64)).permute(1, 0, 2)[None]
    k = torch.from_numpy(bf16_bits_to_f32(b.k[k0:k1]).astype(np.float64)).permute(1, 0, 2)[None]
    v = torch.from_numpy(bf16_bits_to_f32(b.v[k0:k1]).astype(np.float64)).permute(1, 0, 2)[None]
    n, L = q1 - q0, k1 - k0
    mask = None
    if b.causal:
        pos = torch.arange(n) + (L - n)
        mask = torch.arange(L)[None, :] <= pos[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.contiguous(), v.contiguous(), attn_mask=mask, scale=b.sm_scale, enable_gqa=True)
    # log-sum-exp of the masked scores, from torch's own matmul/logsumexp
    G = b.num_qo_heads // b.num_kv_heads
    kr = k.repeat_interleave(G, dim=1)
    s = b.sm_scale * torch.matmul(q, kr.transpose(-1, -2).contiguous())
    if mask is not None:
        s = s.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    return o[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


# ---------------------------------------------------------------- closed forms

def test_golden_closed_form_cases():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 5
    for c in cases:
        d = c["head_dim"]
        nq = len(c["q"])
        nk = len(c["k"])
        b = batch_from_values(c["q"], c["k"] if nk else np.zeros((0, d)),
                              c["v"] if nk else np.zeros((0, d)),
                              qlens=[nq], kv_lens=[nk], hq=1, hkv=1, d=d,
                              sinks=None if c["sink"] is None else [c["sink"]],
                              sm_scale=c["sm_scale"], causal=c["causal"])
        out, lse = oracle.attend(b)
        np.testing.assert_allclose(out[:, 0, :], np.array(c["expect_o"]), rtol=0, atol=1e-15,
                                   err_msg=c["name"])
        np.testing.assert_allclose(lse[:, 0], np.array(c["expect_lse"]), rtol=0, atol=1e-15,
                                   err_msg=c["name"])
        for i in range(nq):
            w, ws, j0, j1, o, l = oracle.row_weights(b, i, 0)
            assert abs(ws - c["expect_w_sink"][i]) <= 1e-15, c["name"]
        bo, bl = oracle.brute(b)
        np.testing.assert_allclose(bo, out, rtol=0, atol=1e-15)
        np.testing.assert_allclose(bl, lse, rtol=0, atol=1e-15)


def test_single_key_closed_form_random():
    """L = 1: o = v0 * sigmoid(s0 - sigma), lse = logaddexp(s0, sigma)."""
    rng = np.random.default_rng(7)
    for trial in range(20):
        d = int(rng.choice([4, 8, 64]))
        q = bf16_bits_to_f32(to_bf16_bits(rng.standard_normal((1, 1, d)).astype(np.float32)))
        k = bf16_bits_to_f32(to_bf16_bits(rng.standard_normal((1, 1, d)).astype(np.float32)))
        v = bf16_bits_to_f32(to_bf16_bits(rng.standard_normal((1, 1, d)).astype(np.float32)))
        sig = np.float32(rng.standard_normal() * 3)
        tau = 1.0 / math.sqrt(d)
        b = batch_from_values(q, k, v, qlens=[1], kv_lens=[1], hq=1, hkv=1, d=d, sinks=[sig],
                              sm_scale=tau, causal=True)
        out, lse = oracle.attend(b)
        s0 = tau * float(np.dot(q.astype(np.float64).ravel(), k.astype(np.float64).ravel()))
        w = 1.0 / (1.0 + math.exp(float(sig) - s0))
        np.testing.assert_allclose(out[0, 0], w * v.astype(np.float64).ravel(), rtol=1e-14,
                                   atol=1e-15)
        assert abs(lse[0, 0] - np.logaddexp(s0, float(sig))) <= 1e-14


# ------------------------------------------------- special case -> library routine

@pytest.mark.parametrize("qlen,kvlen,hq,hkv", [(37, 37, 8, 2), (5, 29, 4, 1), (1, 33, 8, 8),
                                                (16, 16, 64, 8)])
def test_no_sink_equals_torch_sdpa(qlen, kvlen, hq, hkv):
    """sink = -inf (NULL) is standard softmax attention: torch SDPA in fp64."""
    b = make_batch(11 + qlen, kind="prefill", qlens=[qlen], kv_lens=[kvlen], hq=hq, hkv=hkv,
                   d=64, sinks=None, causal=True)
    out, lse = oracle.attend(b)
    o_ref, lse_ref = _sdpa_std(b, 0)
    np.testing.assert_allclose(out, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("sink_std", [0.5, 2.0, 6.0])
def test_sink_closed_form_against_sdpa(sink_std):
    """With a sink: o = o_std * sigmoid(lse_std - sigma),
    lse = logaddexp(lse_std, sigma), where o_std/lse_std come from torch."""
    b = make_batch(23, kind="prefill", qlens=[20, 9], kv_lens=[20, 31], hq=8, hkv=2, d=64,
                   sinks="normal", sink_std=sink_std, causal=True)
    out, lse = oracle.attend(b)
    for r in range(2):
        q0, q1 = int(b.qo_indptr[r]), int(b.qo_indptr[r + 1])
        o_std, l_std = _sdpa_std(b, r)
        sig = b.sinks.astype(np.float64)[None, :]
        w = 1.0 / (1.0 + np.exp(sig - l_std))
        np.testing.assert_allclose(out[q0:q1], o_std * w[..., None], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[q0:q1], np.logaddexp(l_std, sig), rtol=0, atol=1e-12)


# ------------------------------------------------------------------- invariants

def test_large_sink_drives_output_to_zero():
    b = make_batch(31, kind="prefill", qlens=[12], kv_lens=[12], hq=4, hkv=1, d=64,
                   sinks=None, causal=True)
    o_std, l_std = oracle.attend(b)
    vmax = np.abs(bf16_bits_to_f32(b.v)).max()
    prev = None
    for sig in [0.0, 5.0, 20.0, 80.0]:
        b.sinks = np.full(4, sig, np.float32)
        o, l = oracle.attend(b)
        bound = vmax / (1.0 + np.exp(sig - l_std))
        assert np.all(np.abs(o).max(axis=-1) <= bound + 1e-15)
        norm = np.abs(o).max()
        if prev is not None:
            assert norm < prev
        prev = norm
    assert prev < 1e-25
    # a very negative sink leaves standard attention (its weight underflows)
    b.sinks = np.full(4, -1e4, np.float32)
    o, l = oracle.attend(b)
    np.testing.assert_array_equal(o, o_std)
    np.testing.assert_array_equal(l, l_std)
    # +inf sink: all mass on the sink
    b.sinks = np.full(4, np.inf, np.float32)
    o, l = oracle.attend(b)
    assert np.all(o == 0) and np.all(l == np.inf)


def test_shift_invariance_via_extra_dimension():
    """Adding c to every score and to the sink leaves o unchanged and adds c
    to lse.  Realised on inputs: q' = [q, c/tau], k' = [k, 1], sigma' = sigma + c."""
    d = 64
    tau = 1.0 / math.sqrt(d)
    b = make_batch(41, kind="prefill", qlens=[13, 1], kv_lens=[13, 27], hq=8, hkv=2, d=d,
                   sinks="normal", causal=True)
    # sinks with few mantissa bits, so that sigma + c is exact in fp32
    b.sinks = bf16_bits_to_f32(to_bf16_bits(b.sinks))
    o, l = oracle.attend(b)
    for c in [1.0, -3.0, 8.0]:
        qf = bf16_bits_to_f32(b.q)
        kf = bf16_bits_to_f32(b.k)
        q2 = np.concatenate([qf, np.full(qf.shape[:-1] + (1,), c / tau, np.float32)], axis=-1)
        k2 = np.concatenate([kf, np.ones(kf.shape[:-1] + (1,), np.float32)], axis=-1)
        v2 = bf16_bits_to_f32(b.v)
        v2 = np.concatenate([v2, np.zeros(v2.shape[:-1] + (1,), np.float32)], axis=-1)
        b2 = batch_from_values(q2, k2, v2, qlens=b.qlens, kv_lens=b.kv_len, hq=8, hkv=2, d=d + 1,
                               sinks=b.sinks + np.float32(c), sm_scale=tau, causal=True)
        o2, l2 = oracle.attend(b2)
        np.testing.assert_allclose(o2[..., :d], o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, l + c, rtol=0, atol=1e-12)


def test_weights_sum_to_one():
    b = make_batch(51, kind="prefill", qlens=[7, 19], kv_lens=[30, 19], hq=4, hkv=2, d=64,
                   sinks="normal", sink_std=2.0, causal=True)
    for row in range(b.total_q):
        for h in range(4):
            w, ws, j0, j1, o, l = oracle.row_weights(b, row, h)
            assert np.all(w >= 0) and 0 <= ws <= 1
            assert abs(w.sum() + ws - 1.0) <= 1e-14
            # the weights reproduce the output: o = sum_j w_j v_j
            req = 0 if row < b.qo_indptr[1] else 1
            kv0 = int(b.kv_indptr[req])
            g = h // 2
            vv = bf16_bits_to_f32(b.v[kv0 + j0:kv0 + j1, g, :]).astype(np.float64)
            np.testing.assert_allclose(w @ vv, o, rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads():
    b = make_batch(61, kind="prefill", qlens=[11, 4], kv_lens=[11, 20], hq=8, hkv=2, d=64,
                   sinks="normal", causal=True)
    o, l = oracle.attend(b)
    G = 4
    k_rep = np.repeat(b.k, G, axis=1)
    v_rep = np.repeat(b.v, G, axis=1)
    b2 = batch_from_values(bf16_bits_to_f32(b.q), bf16_bits_to_f32(k_rep), bf16_bits_to_f32(v_rep),
                           qlens=b.qlens, kv_lens=b.kv_len, hq=8, hkv=8, d=64, sinks=b.sinks,
                           sm_scale=b.sm_scale, causal=True)
    o2, l2 = oracle.attend(b2)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)
    # and a different map (h % Hkv) would differ: the convention is observable
    k_tile = np.tile(b.k, (1, G, 1))
    v_tile = np.tile(b.v, (1, G, 1))
    b3 = batch_from_values(bf16_bits_to_f32(b.q), bf16_bits_to_f32(k_tile), bf16_bits_to_f32(v_tile),
                           qlens=b.qlens, kv_lens=b.kv_len, hq=8, hkv=8, d=64, sinks=b.sinks,
                           sm_scale=b.sm_scale, causal=True)
    o3, _ = oracle.attend(b3)
    assert np.abs(o3 - o).max() > 1e-3


def test_causal_alignment_prefill_row_equals_decode():
    """Row t of a chunked prefill on prefix P equals a decode over the first
    P+t+1 keys, and equals row P+t of the full prefill."""
    P, n = 9, 6
    full = make_batch(71, kind="prefill", qlens=[P + n], kv_lens=[P + n], hq=8, hkv=2, d=64,
                      sinks="normal", causal=True)
    of, lf = oracle.attend(full)
    chunk = batch_from_values(bf16_bits_to_f32(full.q[P:]), bf16_bits_to_f32(full.k),
                              bf16_bits_to_f32(full.v), qlens=[n], kv_lens=[P + n], hq=8, hkv=2,
                              d=64, sinks=full.sinks, sm_scale=full.sm_scale, causal=True)
    oc, lc = oracle.attend(chunk)
    np.testing.assert_array_equal(oc, of[P:])
    np.testing.assert_array_equal(lc, lf[P:])
    for t in range(n):
        L = P + t + 1
        dec = batch_from_values(bf16_bits_to_f32(full.q[P + t:P + t + 1]),
                                bf16_bits_to_f32(full.k[:L]), bf16_bits_to_f32(full.v[:L]),
                                qlens=[1], kv_lens=[L], hq=8, hkv=2, d=64, sinks=full.sinks,
                                sm_scale=full.sm_scale, causal=True, kind="decode")
        od, ld = oracle.attend(dec)
        np.testing.assert_array_equal(od[0], oc[t])
        np.testing.assert_array_equal(ld[0], lc[t])


def test_paged_layout_and_page_permutation_are_bitwise_invariant():
    b = make_batch(81, kind="prefill", qlens=[5, 17, 1], kv_lens=[40, 17, 33], hq=8, hkv=2,
                   d=64, sinks="normal", causal=True)
    o, l = oracle.attend(b)
    for ps, seed in [(16, None), (16, 3), (4, 5), (1, 7)]:
        rng = None if seed is None else np.random.default_rng(seed)
        bp = to_paged(b, ps, rng)
        op, lp = oracle.attend(bp)
        np.testing.assert_array_equal(op, o)
        np.testing.assert_array_equal(lp, l)
        bo, bl = oracle.brute(bp)
        np.testing.assert_allclose(bo, o, rtol=0, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 5, 16, 40, 64])
def test_split_then_merge_equals_unsplit(chunk):
    """Partials over key chunks, the sink in chunk 0 only, merged by LSE,
    equal the unsplit result; chunks past a row's keys are empty."""
    b = make_batch(91, kind="decode", qlens=[1] * 5, kv_lens=[1, 16, 37, 64, 100], hq=8, hkv=2,
                   d=64, paged=True, sinks="normal", sink_std=2.0, causal=True)
    o, l = oracle.attend(b)
    S = (100 + chunk - 1) // chunk
    parts = [oracle.partial(b, c * chunk, (c + 1) * chunk, include_sink=(c == 0))
             for c in range(S)]
    op = np.stack([p[0] for p in parts], axis=2)   # [N, H, S, D]
    lp = np.stack([p[1] for p in parts], axis=2)   # [N, H, S]
    om, lm = oracle.merge(op, lp)
    np.testing.assert_allclose(om, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, l, rtol=0, atol=1e-12)
    # empty chunks: lse = -inf and o = 0, except chunk 0 which holds the sink
    for r in range(5):
        for c in range(S):
            if c * chunk >= b.kv_len[r]:
                if c == 0:
                    np.testing.assert_array_equal(lp[r, :, c], b.sinks.astype(np.float64))
                else:
                    assert np.all(lp[r, :, c] == -np.inf) and np.all(op[r, :, c] == 0)
    if S >= 2:
        # negative control: the sink in every chunk is a different (wrong) result
        bad = [oracle.partial(b, c * chunk, (c + 1) * chunk, include_sink=True) for c in range(S)]
        ob, lb = oracle.merge(np.stack([p[0] for p in bad], 2), np.stack([p[1] for p in bad], 2))
        assert np.abs(ob - o).max() > 1e-3


def test_merge_edge_cases():
    o = np.zeros((1, 2, 3, 4))
    l = np.full((1, 2, 3), -np.inf)
    om, lm = oracle.merge(o, l)
    assert np.all(om == 0) and np.all(lm == -np.inf)
    # one live chunk passes through unchanged
    rng = np.random.default_rng(0)
    o = rng.standard_normal((2, 3, 4, 8))
    l = np.full((2, 3, 4), -np.inf)
    l[:, :, 2] = 1.25
    om, lm = oracle.merge(o, l)
    np.testing.assert_array_equal(om, o[:, :, 2])
    np.testing.assert_array_equal(lm, l[:, :, 2])
    # two equal-lse chunks average
    l = np.zeros((2, 3, 4))
    om, lm = oracle.merge(o, l)
    np.testing.assert_allclose(om, o.mean(axis=2), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lm, np.log(4.0), rtol=0, atol=1e-15)


def test_empty_rows():
    """A non-causal request with no keys: o = 0, lse = sigma (or -inf)."""
    b = batch_from_values(np.ones((2, 4, 8)), np.zeros((0, 1, 8)), np.zeros((0, 1, 8)),
                          qlens=[1, 1], kv_lens=[0, 0], hq=4, hkv=1, d=8,
                          sinks=[0.5, -2.0, 3.0, 0.0], sm_scale=0.5, causal=False)
    o, l = oracle.attend(b)
    assert np.all(o == 0)
    np.testing.assert_array_equal(l, np.tile(np.array([0.5, -2.0, 3.0, 0.0]), (2, 1)))
    b.sinks = None
    o, l = oracle.attend(b)
    assert np.all(o == 0) and np.all(l == -np.inf)


# ----------------------------------------------------- brute force, tiny shapes

def _random_small(rng, case):
    B = int(rng.integers(1, 4))
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4]))
    hq = hkv * G
    d = int(rng.choice([4, 8, 64]))
    causal = bool(rng.integers(0, 2))
    kv = rng.integers(1, 41, size=B)
    q = np.array([int(rng.integers(1, kv_b + 1)) for kv_b in kv]) if causal else \
        rng.integers(1, 6, size=B)
    mode = case % 4
    sinks = "normal" if mode == 0 else (None if mode == 1 else
                                        np.array(rng.choice([-np.inf, np.inf, -1e4, 10.0, 0.0],
                                                            size=hq), np.float32))
    paged = bool(rng.integers(0, 2))
    return make_batch(int(rng.integers(1 << 30)), kind="prefill", qlens=q, kv_lens=kv, hq=hq,
                      hkv=hkv, d=d, paged=paged, page_size=int(rng.choice([1, 4, 16])),
                      sinks=sinks, sink_std=3.0, causal=causal)


def test_c_oracle_agrees_with_numpy_brute_force():
    rng = np.random.default_rng(2024)
    for case in range(60):
        b = _random_small(rng, case)
        o, l = oracle.attend(b)
        bo, bl = oracle.brute(b)
        np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12, err_msg=str(case))
        fin = np.isfinite(bl)
        assert np.array_equal(np.isfinite(l), fin)
        np.testing.assert_allclose(l[fin], bl[fin], rtol=0, atol=1e-12)
        assert np.array_equal(l[~fin], bl[~fin])


def test_sampled_rows_match_full():
    b = make_batch(5, kind="prefill", qlens=[30, 7], kv_lens=[30, 50], hq=8, hkv=2, d=64,
                   paged=True, sinks="normal", causal=True)
    o, l = oracle.attend(b)
    rng = np.random.default_rng(1)
    rows = rng.integers(0, b.total_q, 25)
    heads = rng.integers(0, 8, 25)
    os_, ls_ = oracle.attend_rows(b, rows, heads)
    np.testing.assert_array_equal(os_, o[rows, heads])
    np.testing.assert_array_equal(ls_, l[rows, heads])


def test_oracle_rejects_bad_arguments():
    b = make_batch(5, kind="prefill", qlens=[3], kv_lens=[3], hq=4, hkv=2, d=8, sinks=None)
    b.num_kv_heads = 3   # Hq % Hkv != 0
    with pytest.raises(ValueError):
        oracle.attend(b)


# --------------------------------------------------------------- input module

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39, 65504.0],
                                 np.float32)])
    ours = to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_paged_recipe_structure():
    b = make_batch(9, kind="decode", qlens=[1] * 6, kv_lens=[1, 15, 16, 17, 33, 64], hq=8, hkv=2,
                   d=64, paged=True, sinks="normal")
    pages = np.diff(b.kv_indptr)
    np.testing.assert_array_equal(pages, [1, 1, 1, 2, 3, 4])
    assert sorted(b.page_indices.tolist()) == list(range(12))
    assert b.k.shape == (12, 2, 16, 64)
    # poison in the unused slots of each last page
    for r, L in enumerate(b.kv_len):
        last = b.page_indices[b.kv_indptr[r + 1] - 1]
        used = L % 16
        if used:
            assert np.all(bf16_bits_to_f32(b.k[last, :, used:]) == 8.0)
            assert np.all(bf16_bits_to_f32(b.v[last, :, used:]) == 100.0)
    # a rel_l2 sanity check of the helper used by the parity tests
    assert rel_l2(np.ones(4), np.ones(4)) == 0.0


def test_planted_mistakes_still_apply():
    """The planted-mistake list (tests/oracle_mutations.py, run by hand: every
    mistake must fail a pin) still applies to the current oracle sources."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "oracle_mutations", os.path.join(os.path.dirname(__file__), "oracle_mutations.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.check_applicable()
    assert len(mod.MUTATIONS) >= 30
