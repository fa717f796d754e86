"""Pins of the projection-side oracle (oracle/rope.py): QKV bias, YaRN rotary
encoding and the paged append, on the CPU.

Each pin ties the oracle to something other than itself: the ramp
boundaries derived by hand from the wavelength bounds (tests/golden), the
closed-form temperature, a complex-number formulation of the rotation, the
relative-position property of rotary encoding, and the attention oracle's
own reading of the paged layout (oracle/brute.py gathers a request's keys).
"""
from __future__ import annotations

import cmath
import json
import math
import os

import numpy as np
import pytest

from oracle import rope
from oracle.brute import _gather_kv
import workloads as W
from workloads import bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "yarn_ramp_boundaries.json")


def test_golden_ramp_boundaries_and_temperature():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        D, base, s = c["head_dim"], c["base"], c["factor"]
        f = rope.yarn_frequencies(D, base, s, c["original_max_pos"], c["beta_fast"],
                                  c["beta_slow"])
        theta = base ** (-2.0 * np.arange(D // 2) / D)
        k0, k1 = c["kept"]
        r0, r1 = c["ramped"]
        i0, i1 = c["interpolated"]
        assert (k0, k1 + 1, r1 + 1, i1 + 1) == (0, r0, i0, D // 2)
        np.testing.assert_allclose(f[k0:k1 + 1], theta[k0:k1 + 1], rtol=1e-15, atol=0)
        np.testing.assert_allclose(f[i0:i1 + 1], theta[i0:i1 + 1] / s, rtol=1e-15, atol=0)
        mid = slice(r0, r1 + 1)
        assert np.all(f[mid] > theta[mid] / s) and np.all(f[mid] < theta[mid])
        assert abs(rope.yarn_temperature(s) - c["temperature"]) < 1e-15
        assert abs(rope.yarn_temperature(s) - (0.5 * math.log(2) + 1)) < 1e-15


def test_ramp_is_continuous_and_frequencies_decrease():
    """Frequencies fall with the pair index and the interpolated fraction
    rises: no jump at either bound of the ramp."""
    for base in (1e4, 1.5e5, 5e5):
        f = rope.yarn_frequencies(64, base, 32.0, 4096, 32.0, 1.0)
        theta = base ** (-2.0 * np.arange(32) / 64)
        assert np.all(np.diff(f) < 0)
        keep = (f - theta / 32) / (theta - theta / 32)   # 1 = kept, 0 = interpolated
        assert np.all(np.diff(keep) <= 1e-12)
        assert np.all((keep >= -1e-12) & (keep <= 1 + 1e-12))
        # a ramp of the rotation count cannot move by more than one step
        # between neighbouring pairs: r shrinks by base^(2/64) per pair
        assert np.max(np.abs(np.diff(keep))) < 1.0


def test_no_scaling_is_plain_rotary():
    for D in (8, 64):
        f = rope.yarn_frequencies(D, 10000.0, 1.0, 4096, 32.0, 1.0)
        np.testing.assert_allclose(f, 10000.0 ** (-2.0 * np.arange(D // 2) / D), rtol=1e-15)
    assert rope.yarn_temperature(1.0) == 1.0


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_equals_complex_multiplication(interleaved):
    """Pair (a, b) as a + ib, times m e^{i p f}: an independent formulation."""
    rng = np.random.default_rng(11)
    D = 64
    tab = rope.rope_table(50, D, 150000.0, 32.0, 4096, 32.0, 1.0)
    f = rope.yarn_frequencies(D, 150000.0, 32.0, 4096, 32.0, 1.0)
    m = rope.yarn_temperature(32.0)
    for p in (0, 1, 7, 49):
        x = rng.standard_normal(D)
        y = rope.rotate(x, tab[p, :D // 2], tab[p, D // 2:], interleaved)
        for d in range(D // 2):
            i, j = (2 * d, 2 * d + 1) if interleaved else (d, d + D // 2)
            z = complex(x[i], x[j]) * m * cmath.exp(1j * p * f[d])
            assert abs(y[i] - z.real) < 1e-12 and abs(y[j] - z.imag) < 1e-12
    # position 0 only scales by the temperature
    x = rng.standard_normal(D)
    np.testing.assert_allclose(rope.rotate(x, tab[0, :32], tab[0, 32:], interleaved), m * x,
                               rtol=0, atol=1e-15)


def test_scores_depend_on_relative_position_only():
    """<R_m q, R_n k> = T^2 <R_{m-n} q, k>: rotary encoding's defining property,
    with the temperature T applied to both sides."""
    rng = np.random.default_rng(12)
    D = 64
    tab = rope.rope_table(300, D, 10000.0, 8.0, 64, 32.0, 1.0)
    T = rope.yarn_temperature(8.0)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for inter in (False, True):
        rot = lambda x, p: rope.rotate(x, tab[p, :32], tab[p, 32:], inter)  # noqa: E731
        for m, n in [(5, 3), (200, 198), (17, 17), (299, 0)]:
            a = rot(q, m) @ rot(k, n)
            b = T * T * (rope.rotate(q, tab[m - n, :32] / T, tab[m - n, 32:] / T, inter) @ k)
            assert abs(a - b) < 1e-9 * (1 + abs(a))
        # the two pairings are different encodings
        assert abs(rot(q, 5) @ rot(k, 3) - rope.rotate(q, tab[5, :32], tab[5, 32:], not inter)
                   @ rope.rotate(k, tab[3, :32], tab[3, 32:], not inter)) > 1e-6


def test_table_entries_have_the_temperature_as_norm():
    tab = rope.rope_table(64, 64, 150000.0, 32.0, 4096, 32.0, 1.0)
    n = tab[:, :32] ** 2 + tab[:, 32:] ** 2
    np.testing.assert_allclose(n, rope.yarn_temperature(32.0) ** 2, rtol=1e-14)
    t1 = rope.rope_table(8, 64, 150000.0, 32.0, 4096, 32.0, 1.0, attn_factor=1.0)
    np.testing.assert_allclose(t1[:, :32] ** 2 + t1[:, 32:] ** 2, 1.0, rtol=1e-14)


@pytest.mark.parametrize("interleaved", [False, True])
def test_append_lands_where_the_attention_oracle_reads(interleaved):
    """The attention oracle's own paged reader (brute force) is pointed at a
    cache whose slots hold their own (page, slot) address; at each new
    token's position it names the slot where the append must have put that
    token's biased, rotated key and biased value.  Every other slot keeps its
    old contents."""
    qlens, kvl = [1, 5, 17, 3], [1, 40, 17, 33]
    ab = W.make_append_batch(21, qlens=qlens, kv_lens=kvl, hq=8, hkv=2)
    tab = rope.rope_table(64, 64, 150000.0, 32.0, 4096, 32.0, 1.0)
    q, kc, vc = rope.qkv_rope_append(ab.qkv, ab.bias, tab, ab.qo_indptr, ab.kv_len,
                                     ab.page_indptr, ab.page_indices, ab.k_pages, ab.v_pages,
                                     8, 2, interleaved)
    qkv = bf16_bits_to_f32(ab.qkv).astype(np.float64)
    bias = bf16_bits_to_f32(ab.bias).astype(np.float64).reshape(12, 64)
    n_pages = ab.k_pages.shape[0]
    assert n_pages <= 256                       # addresses exact in bf16
    addr = np.zeros((n_pages, 2, 16, 64), np.float32)
    addr[:, :, :, 0] = np.arange(n_pages)[:, None, None]
    addr[:, :, :, 1] = np.arange(16)[None, None, :]
    view = type("View", (), dict(k=W.to_bf16_bits(addr), v=W.to_bf16_bits(addr),
                                 page_indices=ab.page_indices, page_size=16, num_kv_heads=2,
                                 head_dim=64, kv_indptr=ab.page_indptr, kv_len=ab.kv_len))
    written = np.zeros(kc.shape[:3], bool)
    for b, (n, L) in enumerate(zip(qlens, kvl)):
        where, _ = _gather_kv(view, b)          # [L, Hkv, D]: (page, slot) of each position
        for t in range(n):
            row, p = int(ab.qo_indptr[b]) + t, L - n + t
            page, slot = int(where[p, 0, 0]), int(where[p, 0, 1])
            for g in range(2):
                kref = rope.rotate(qkv[row, 8 + g] + bias[8 + g], tab[p, :32], tab[p, 32:],
                                   interleaved)
                np.testing.assert_array_equal(kc[page, g, slot], kref)
                np.testing.assert_array_equal(vc[page, g, slot], qkv[row, 10 + g] + bias[10 + g])
            for h in range(8):
                np.testing.assert_array_equal(
                    q[row, h], rope.rotate(qkv[row, h] + bias[h], tab[p, :32], tab[p, 32:],
                                           interleaved))
            written[page, :, slot] = True
    old_k = bf16_bits_to_f32(ab.k_pages).astype(np.float64)
    old_v = bf16_bits_to_f32(ab.v_pages).astype(np.float64)
    np.testing.assert_array_equal(kc[~written], old_k[~written])
    np.testing.assert_array_equal(vc[~written], old_v[~written])
    assert written.sum() == 2 * sum(qlens)


def test_no_bias_and_sampled_rows():
    ab = W.make_append_batch(23, qlens=[4, 6], kv_lens=[10, 6], hq=4, hkv=1, bias=False)
    tab = rope.rope_table(16, 64, 10000.0, 1.0, 4096, 32.0, 1.0)
    q, kc, vc = rope.qkv_rope_append(ab.qkv, None, tab, ab.qo_indptr, ab.kv_len, ab.page_indptr,
                                     ab.page_indices, ab.k_pages, ab.v_pages, 4, 1, False)
    qs, _, _ = rope.qkv_rope_append(ab.qkv, None, tab, ab.qo_indptr, ab.kv_len, ab.page_indptr,
                                    ab.page_indices, ab.k_pages, ab.v_pages, 4, 1, False,
                                    rows=[1, 7])
    np.testing.assert_array_equal(qs[[1, 7]], q[[1, 7]])
    assert np.all(qs[[0, 2, 3, 4, 5, 6, 8, 9]] == 0)
    # the value heads without bias are the projection's own values
    v = bf16_bits_to_f32(ab.qkv).astype(np.float64)[:, 5]
    page = ab.page_indices[ab.page_indptr[1]]
    np.testing.assert_array_equal(vc[page, 0, :6], v[4:10])


def test_golden_pair_ramp():
    """The pair-index ramp: rounded correction pairs, the same keep / ramp /
    interpolate classes as the rotation-count ramp, and a hand-derived blend
    of one ramped pair under each ramp."""
    g = json.load(open(GOLDEN))["pair_ramp"]
    for c in g["cases"]:
        D, base, s, L = c["head_dim"], c["base"], c["factor"], c["original_max_pos"]
        args = (D, base, s, L, c["beta_fast"], c["beta_slow"])
        assert math.floor(rope.correction_pair(c["beta_fast"], D, base, L)) == c["low"]
        assert math.ceil(rope.correction_pair(c["beta_slow"], D, base, L)) == c["high"]
        fp = rope.yarn_frequencies(*args, ramp="pairs")
        ft = rope.yarn_frequencies(*args, ramp="turns")
        theta = base ** (-2.0 * np.arange(D // 2) / D)
        k0, k1 = c["kept"]
        i0, i1 = c["interpolated"]
        r0, r1 = c["ramped"]
        for f in (fp, ft):
            np.testing.assert_allclose(f[k0:k1 + 1], theta[k0:k1 + 1], rtol=1e-15, atol=0)
            np.testing.assert_allclose(f[i0:i1 + 1], theta[i0:i1 + 1] / s, rtol=1e-15, atol=0)
            mid = slice(r0, r1 + 1)
            assert np.all(f[mid] > theta[mid] / s) and np.all(f[mid] < theta[mid])
        d = c["pair"]
        assert abs(theta[d] - c["theta"]) <= 1e-15
        assert abs(fp[d] - c["pairs_frequency"]) <= 1e-15
        assert abs(ft[d] - c["turns_frequency"]) <= 1e-15
        # linear in the pair index: equal steps of the kept fraction
        keep = (fp - theta / s) / (theta - theta / s)
        steps = np.diff(keep[c["low"]:c["high"] + 1])
        np.testing.assert_allclose(steps, -1.0 / (c["high"] - c["low"]), rtol=1e-12)


def test_pair_ramp_degenerate_range_is_a_step():
    """When the rounded correction pairs leave no room for a ramp (high <=
    low) the blend is a step: pairs up to low keep, the rest divide by s.
    With beta_fast = 1e6 turns, d(beta) is negative, so low clamps to pair 0
    and high (also negative) falls below it."""
    D, base, s, L = 64, 10000.0, 4.0, 4096
    assert rope.correction_pair(1e6, D, base, L) < -25
    f = rope.yarn_frequencies(D, base, s, L, 1e6, 1e6 - 1e-3, ramp="pairs")
    theta = base ** (-2.0 * np.arange(D // 2) / D)
    assert f[0] == theta[0]
    np.testing.assert_allclose(f[1:], theta[1:] / s, rtol=1e-15)
