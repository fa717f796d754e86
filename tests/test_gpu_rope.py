"""Parity of the projection-side step (sink_attn_rope_table and
sink_attn_qkv_rope_append) against the fp64 oracle in oracle/rope.py.

Bars, from the arithmetic:
  * table: fp32 stores of fp64 values no larger than the temperature T, so
    |gpu - oracle| <= 2^-23 T (one fp32 rounding, with margin);
  * appended q / k / v: one bf16 rounding (relative 2^-9) after an fp32 bias
    add and rotation whose own error is ~1e-7 of the inputs, so
    |gpu - oracle| <= 2^-8 |oracle| + 1e-5;
  * every cache slot that is not a new token's slot stays bitwise unchanged.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import rope  # noqa: E402
import workloads as W  # noqa: E402
from workloads import bf16_bits_to_f32  # noqa: E402

YARN = dict(rope_theta=150000.0, factor=32.0, original_max_pos=4096, beta_fast=32.0,
            beta_slow=1.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_attn_amd  # noqa: F401  (fails loudly if not built)
    yield


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def _ref_table(max_pos, cfg, attn_factor=0.0, ramp="turns"):
    return rope.rope_table(max_pos, 64, cfg["rope_theta"], cfg["factor"], cfg["original_max_pos"],
                           cfg["beta_fast"], cfg["beta_slow"], attn_factor, ramp)


def _gpu_table(max_pos, cfg, attn_factor=0.0, ramp="turns"):
    from gqa_attention_sinks_attn_amd import (YARN_RAMP_PAIRS, YARN_RAMP_TURNS,
                                              sink_attn_rope_table)
    t = torch.full((max_pos, 64), float("nan"), dtype=torch.float32, device="cuda")
    sink_attn_rope_table(t, max_pos, 64, cfg["rope_theta"], cfg["factor"],
                         cfg["original_max_pos"], cfg["beta_fast"], cfg["beta_slow"], attn_factor,
                         YARN_RAMP_PAIRS if ramp == "pairs" else YARN_RAMP_TURNS)
    torch.cuda.synchronize()
    return t


@pytest.mark.parametrize("cfg,attn_factor,ramp", [
    (YARN, 0.0, "turns"),
    (YARN, 1.0, "turns"),
    (YARN, 0.0, "pairs"),
    (dict(rope_theta=10000.0, factor=1.0, original_max_pos=0, beta_fast=0.0, beta_slow=0.0), 0.0,
     "turns"),
    (dict(rope_theta=10000.0, factor=8.0, original_max_pos=2048, beta_fast=16.0, beta_slow=2.0), 0.0,
     "turns"),
    (dict(rope_theta=10000.0, factor=8.0, original_max_pos=2048, beta_fast=16.0, beta_slow=2.0), 0.0,
     "pairs"),
])
def test_rope_table_matches_oracle(cfg, attn_factor, ramp):
    max_pos = 131072
    t = _gpu_table(max_pos, cfg, attn_factor, ramp).cpu().numpy().astype(np.float64)
    temp = attn_factor if attn_factor > 0 else rope.yarn_temperature(cfg["factor"])
    first = _ref_table(2048, cfg, attn_factor, ramp)
    err = np.abs(t[:2048] - first).max()
    print(f"[rope table {cfg['factor']} {ramp}] first 2048 positions max err {err:.3e}", flush=True)
    assert err <= 2.0 ** -23 * temp
    # large positions, where the angle reaches 1e5 rad
    f = rope.yarn_frequencies(64, cfg["rope_theta"], cfg["factor"], cfg["original_max_pos"],
                              cfg["beta_fast"], cfg["beta_slow"], ramp)
    rng = np.random.default_rng(5)
    for p in list(rng.integers(2048, max_pos, size=200)) + [max_pos - 1]:
        ref = np.concatenate([temp * np.cos(p * f), temp * np.sin(p * f)])
        assert np.abs(t[p] - ref).max() <= 2.0 ** -23 * temp, p


def _run_append(ab, table_t, max_pos, interleaved, bias=True):
    from gqa_attention_sinks_attn_amd import sink_attn_qkv_rope_append
    T = ab.total_q
    q_out = torch.full((max(T, 1), ab.num_qo_heads, 64), -1, dtype=torch.int16, device="cuda")
    kp = _bf16_dev(ab.k_pages)
    vp = _bf16_dev(ab.v_pages)
    sink_attn_qkv_rope_append(_bf16_dev(ab.qkv), _bf16_dev(ab.bias) if bias else None, table_t,
                              max_pos, _i32(ab.qo_indptr), _i32(ab.kv_len),
                              _i32(ab.page_indptr), _i32(ab.page_indices), ab.batch,
                              ab.num_qo_heads, ab.num_kv_heads, 64, 16, T, int(interleaved),
                              q_out, kp, vp)
    torch.cuda.synchronize()
    u16 = lambda x: x.cpu().numpy().view(np.uint16)  # noqa: E731
    return u16(q_out)[:T], u16(kp), u16(vp)


def _close(name, got_bits, ref):
    got = bf16_bits_to_f32(got_bits).astype(np.float64)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5
    print(f"[{name}] max err {err.max() if err.size else 0:.3e}", flush=True)
    assert np.all(err <= bound), f"{name}: worst excess {(err - bound).max()}"


@pytest.mark.parametrize("interleaved", [0, 1])
@pytest.mark.parametrize("hq,hkv,bias", [(64, 8, True), (16, 16, True), (8, 1, False)])
def test_append_matches_oracle(hq, hkv, bias, interleaved):
    rng = np.random.default_rng(40 + hq + hkv + interleaved)
    B = 12
    qlens = rng.integers(0, 40, size=B)
    qlens[:3] = [1, 0, 17]                       # a decode token, an empty request, a page straddle
    kvl = qlens + rng.integers(0, 3000, size=B)
    kvl[0] = 1                                   # the very first token of a cache
    ab = W.make_append_batch(rng, qlens=qlens, kv_lens=kvl, hq=hq, hkv=hkv, bias=bias)
    max_pos = int(kvl.max())
    tab_t = _gpu_table(max_pos, YARN)
    q, kp, vp = _run_append(ab, tab_t, max_pos, interleaved, bias)
    tab = _ref_table(max_pos, YARN)
    rq, rk, rv = rope.qkv_rope_append(ab.qkv, ab.bias if bias else None, tab, ab.qo_indptr,
                                      ab.kv_len, ab.page_indptr, ab.page_indices, ab.k_pages,
                                      ab.v_pages, hq, hkv, bool(interleaved))
    tag = f"append hq={hq} hkv={hkv} bias={bias} inter={interleaved}"
    _close(tag + " q", q, rq)
    new = np.zeros(ab.k_pages.shape[:3], bool)
    for b in range(B):
        for t in range(int(qlens[b])):
            p = int(kvl[b]) - int(qlens[b]) + t
            new[int(ab.page_indices[ab.page_indptr[b] + p // 16]), :, p % 16] = True
    _close(tag + " k", kp[new], rk[new])
    _close(tag + " v", vp[new], rv[new])
    assert np.array_equal(kp[~new], ab.k_pages[~new]), "a key slot outside the new tokens changed"
    assert np.array_equal(vp[~new], ab.v_pages[~new]), "a value slot outside the new tokens changed"


def test_append_large_positions_and_prefill_shape():
    """A long-context decode step and a prefill chunk deep into the cache."""
    rng = np.random.default_rng(61)
    qlens = [1, 1, 300, 64]
    kvl = [131072, 70001, 100000, 64]
    ab = W.make_append_batch(rng, qlens=qlens, kv_lens=kvl, hq=16, hkv=2, spare_pages=1)
    max_pos = 131072
    tab_t = _gpu_table(max_pos, YARN)
    q, kp, vp = _run_append(ab, tab_t, max_pos, 0)
    pos = [(b, t, kvl[b] - qlens[b] + t) for b in range(4) for t in range(qlens[b])]
    rows = [int(ab.qo_indptr[b]) + t for b, t, _ in pos]
    need = sorted({p for _, _, p in pos})
    tab = np.zeros((max_pos, 64))               # only the rows in use are filled
    f = rope.yarn_frequencies(64, YARN["rope_theta"], YARN["factor"], YARN["original_max_pos"],
                              YARN["beta_fast"], YARN["beta_slow"])
    m = rope.yarn_temperature(YARN["factor"])
    for p in need:
        tab[p] = np.concatenate([m * np.cos(p * f), m * np.sin(p * f)])
    rq, rk, rv = rope.qkv_rope_append(ab.qkv, ab.bias, tab, ab.qo_indptr, ab.kv_len,
                                      ab.page_indptr, ab.page_indices, ab.k_pages, ab.v_pages,
                                      16, 2, False, rows=rows)
    _close("large positions q", q[rows], rq[rows])
    for b, t, p in pos:
        page = int(ab.page_indices[ab.page_indptr[b] + p // 16])
        _close(f"large positions k p={p}", kp[page, :, p % 16], rk[page, :, p % 16])
        _close(f"large positions v p={p}", vp[page, :, p % 16], rv[page, :, p % 16])


def _new_slots(ab, reqs, kvl):
    new = np.zeros(ab.k_pages.shape[:3], bool)
    for b in reqs:
        n = int(ab.qo_indptr[b + 1] - ab.qo_indptr[b])
        for t in range(n):
            p = int(kvl[b]) - n + t
            new[int(ab.page_indices[ab.page_indptr[b] + p // 16]), :, p % 16] = True
    return new


@pytest.mark.parametrize("case", ["past_table", "past_pages"])
def test_tokens_outside_the_table_or_pages_are_skipped(case):
    """Positions past max_pos, or past the request's reserved pages, are a
    caller error: the kernel writes nothing for those tokens and everything
    for the others."""
    qlens, kvl = [3, 4, 2], np.array([10, 70, 30])
    ab = W.make_append_batch(62, qlens=qlens, kv_lens=kvl, hq=8, hkv=2)
    if case == "past_table":
        max_pos, bad = 40, 1                    # request 1 sits at 66..69
    else:
        max_pos, bad = 4096, 2
        ab.kv_len = ab.kv_len.copy()
        ab.kv_len[2] = 70                       # positions 68, 69: page 4 of a 2-page request
    good = [b for b in range(3) if b != bad]
    q, kp, vp = _run_append(ab, _gpu_table(max_pos, YARN), max_pos, 0)
    rows_bad = list(range(int(ab.qo_indptr[bad]), int(ab.qo_indptr[bad + 1])))
    rows_good = [r for r in range(ab.total_q) if r not in rows_bad]
    assert np.all(q[rows_bad].view(np.int16) == -1), "skipped rows must stay unwritten"
    tab = _ref_table(80, YARN)
    rq, rk, rv = rope.qkv_rope_append(ab.qkv, ab.bias, tab, ab.qo_indptr, kvl, ab.page_indptr,
                                      ab.page_indices, ab.k_pages, ab.v_pages, 8, 2, False,
                                      rows=rows_good)
    _close(f"skip {case}: q", q[rows_good], rq[rows_good])
    new = _new_slots(ab, good, kvl)
    _close(f"skip {case}: k", kp[new], rk[new])
    _close(f"skip {case}: v", vp[new], rv[new])
    assert np.array_equal(kp[~new], ab.k_pages[~new])
    assert np.array_equal(vp[~new], ab.v_pages[~new])


def test_append_many_and_empty_requests():
    """Thousands of requests, nearly all empty: the rows of one workgroup lie
    dozens of requests apart, so the request lookup takes its sampled first
    level (batch > 64) and slides its window of 64 entries."""
    rng = np.random.default_rng(63)
    B = 5000
    qlens = np.where(rng.random(B) < 0.97, 0, rng.integers(1, 4, size=B))
    qlens[:2] = [0, 1]
    qlens[-1] = 2
    kvl = qlens + np.where(qlens > 0, rng.integers(0, 40, size=B), rng.integers(0, 3, size=B))
    ab = W.make_append_batch(rng, qlens=qlens, kv_lens=kvl, hq=8, hkv=2, spare_pages=2)
    max_pos = int(kvl.max())
    q, kp, vp = _run_append(ab, _gpu_table(max_pos, YARN), max_pos, 0)
    rq, rk, rv = rope.qkv_rope_append(ab.qkv, ab.bias, _ref_table(max_pos, YARN), ab.qo_indptr,
                                      ab.kv_len, ab.page_indptr, ab.page_indices, ab.k_pages,
                                      ab.v_pages, 8, 2, False)
    _close("many requests q", q, rq)
    new = _new_slots(ab, range(B), kvl)
    _close("many requests k", kp[new], rk[new])
    _close("many requests v", vp[new], rv[new])
    assert np.array_equal(kp[~new], ab.k_pages[~new])
    assert np.array_equal(vp[~new], ab.v_pages[~new])
