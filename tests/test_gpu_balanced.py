"""GPU parity of the load-balanced decode (sink_attn_decode_balanced and its
two passes) against the fp64 oracle, to the same bar as the other GPU
parity tests (max-abs 1e-2, rel-L2 5e-3, LSE 5e-3; bf16 outputs get their
own rounding on top).

The cases aim at what the page partition adds: ranges that start or end
inside a request, steps whose two pages belong to different requests,
requests without pages, ranges holding many requests, a request spread over
hundreds of ranges, page-table rows with more pages than the request's keys,
and a workspace that holds stale or NaN data from an earlier call.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from tests.test_gpu_parity import check  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_attn_amd  # noqa: F401  (fails loudly if not built)
    yield


def bal_device(b, num_ranges=0, out_dtype=None):
    from gqa_attention_sinks_attn_amd import device
    db = device.to_device(b, out_dtype=out_dtype, plan="balanced", num_ranges=num_ranges)
    db.workspace.fill_(0xFF)        # NaN in every fp32 slot: nothing may read unwritten slots
    return db


def bal_run(b, num_ranges=0, out_dtype=None):
    from gqa_attention_sinks_attn_amd import device
    db = bal_device(b, num_ranges, out_dtype)
    device.run(db)
    torch.cuda.synchronize()
    bf16 = db.out.dtype == torch.bfloat16
    return (db.out.float().cpu().numpy().astype(np.float64),
            db.lse.cpu().numpy().astype(np.float64), bf16)


def _case(name, b, num_ranges=0, out_dtype=None):
    print(f"[balanced] {name} batch={len(b.kv_len)} ranges={num_ranges}", flush=True)
    out, lse, bf16 = bal_run(b, num_ranges, out_dtype)
    ref, rl = oracle.attend(b)
    check(name, out, ref, lse, rl, bf16_out=bf16)


def test_balanced_c2_paged_decode_full():
    _case("balanced c2", W.config(2))


def test_balanced_c3_split_decode_full():
    _case("balanced c3", W.config(3))


def test_balanced_c5_decode_sampled():
    from tests.test_gpu_parity import _sample_rows
    part = W.config(5).decode
    out, lse, bf16 = bal_run(part)
    rows, heads = _sample_rows(part, 3000, 53)
    ex = np.array([0, 17, 42, 5, 31, 63], np.int32)
    rows = np.concatenate([rows, np.repeat(rows[:8], ex.size)])
    heads = np.concatenate([heads, np.tile(ex, 8)])
    ref, rl = oracle.attend_rows(part, rows, heads)
    check("balanced c5 decode", out[rows, heads], ref, lse[rows, heads], rl, bf16_out=bf16)


MIX = [0, 1, 15, 16, 17, 33, 100, 0, 250, 31, 32, 48, 0, 2, 400, 1]


@pytest.mark.parametrize("num_ranges", [0, 4, 8, 12, 28, 64, 400])
def test_balanced_range_counts(num_ranges):
    """Odd and even range widths, ranges smaller and larger than requests."""
    b = W.make_batch(300 + num_ranges, kind="decode", qlens=[1] * len(MIX), kv_lens=MIX, hq=16,
                     hkv=2, paged=True, sinks="normal", sink_std=2.0, causal=False)
    _case(f"balanced mix R={num_ranges}", b, num_ranges)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (16, 4), (64, 8), (32, 2)])
@pytest.mark.parametrize("num_ranges", [0, 8])
def test_balanced_group_sizes(hq, hkv, num_ranges):
    b = W.make_batch(17 + hq + hkv, kind="decode", qlens=[1] * 6, kv_lens=[1, 40, 257, 1000, 3, 64],
                     hq=hq, hkv=hkv, paged=True, sinks="normal")
    _case(f"balanced G={hq // hkv} R={num_ranges}", b, num_ranges)


@pytest.mark.parametrize("sink", [None, -1e4, 0.0, 10.0, "normal"])
def test_balanced_sink_values(sink):
    b = W.make_batch(23, kind="decode", qlens=[1] * 4, kv_lens=[5, 64, 300, 1], hq=64, hkv=8,
                     paged=True, sinks=sink, sink_std=2.0)
    _case(f"balanced sink={sink}", b, 8)


def test_balanced_infinite_sink():
    s = np.zeros(8, np.float32)
    s[3] = np.inf
    b = W.make_batch(25, kind="decode", qlens=[1, 1, 1], kv_lens=[50, 700, 0], hq=8, hkv=2,
                     paged=True, sinks=s, causal=False)
    for R in (0, 4, 12):
        out, lse, bf16 = bal_run(b, R)
        ref, rl = oracle.attend(b)
        assert np.all(out[:, 3] == 0) and np.all(lse[:, 3] == np.inf), R
        keep = [h for h in range(8) if h != 3]
        check(f"balanced +inf sink others R={R}", out[:, keep], ref[:, keep], lse[:, keep],
              rl[:, keep], bf16_out=bf16)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_balanced_output_dtypes(out_dtype):
    b = W.make_batch(27, kind="decode", qlens=[1] * 5, kv_lens=[40, 90, 1, 700, 16], hq=16, hkv=2,
                     paged=True, sinks="normal", out_dtype=out_dtype)
    for R in (0, 4):
        _case(f"balanced out={out_dtype} R={R}", b, R)


def _with_extra_pages(b, extra, seed):
    """Give every request `extra` more page-table entries than its keys need,
    pointing at fresh pages full of NaN: the definition never reads those
    keys, so they must not reach the output."""
    rng = np.random.default_rng(seed)
    B = len(b.kv_len)
    n_old = b.k.shape[0]
    n_new = B * extra
    nan = np.full((n_new,) + b.k.shape[1:], 0x7FC0, dtype=b.k.dtype)
    k = np.concatenate([b.k, nan])
    v = np.concatenate([b.v, nan])
    new_ids = n_old + rng.permutation(n_new)
    rows, indptr = [], [0]
    for r in range(B):
        row = list(b.page_indices[b.kv_indptr[r]:b.kv_indptr[r + 1]])
        row += list(new_ids[r * extra:(r + 1) * extra])
        rows += row
        indptr.append(len(rows))
    b.k, b.v = k, v
    b.page_indices = np.array(rows, np.int32)
    b.kv_indptr = np.array(indptr, np.int32)
    return b


def test_balanced_extra_pages_and_nan_tails():
    b = W.make_batch(29, kind="decode", qlens=[1] * 5, kv_lens=[5, 17, 40, 0, 33], hq=16, hkv=2,
                     paged=True, sinks="normal", causal=False)
    for r, L in enumerate(b.kv_len):
        n = b.kv_indptr[r + 1] - b.kv_indptr[r]
        used = int(L) % 16
        if n and used:
            last = b.page_indices[b.kv_indptr[r + 1] - 1]
            b.k[last, :, used:, :] = 0x7FC0
            b.v[last, :, used:, :] = 0x7FC0
    b = _with_extra_pages(b, 3, 29)
    for R in (0, 4, 8, 12):
        _case(f"balanced extra pages R={R}", b, R)


def test_balanced_many_and_empty_requests():
    """Thousands of short requests (a range holds dozens of them; the request
    lookup walks a two-level search), empty requests at both ends."""
    rng = np.random.default_rng(7)
    L = rng.integers(0, 40, size=4500)
    L[:7] = 0
    L[-3:] = 0
    L[100:110] = 16
    b = W.make_batch(95, kind="decode", qlens=[1] * L.size, kv_lens=L, hq=8, hkv=2, paged=True,
                     sinks="normal", causal=False)
    for R in (0, 8, 100):
        _case(f"balanced many requests R={R}", b, R)


@pytest.mark.parametrize("lens", [[1], [16] * 64, [17, 4096, 1, 2000], [131072, 3],
                                  [0] * 5 + [300] + [0] * 5])
def test_balanced_length_mixes(lens):
    b = W.make_batch(97 + len(lens), kind="decode", qlens=[1] * len(lens), kv_lens=lens, hq=64,
                     hkv=8, paged=True, sinks="normal", causal=False)
    _case(f"balanced length mix {lens[:6]}", b)


@pytest.mark.parametrize("case", ["very_negative_no_sink", "very_positive_zero_sink", "growing_keys"])
def test_balanced_extreme_score_ranges(case):
    b = W.make_batch(83, kind="decode", qlens=[1, 1, 1], kv_lens=[300, 77, 64], hq=16, hkv=2,
                     paged=True, sinks=None if case == "very_negative_no_sink" else 0.0)
    qf = W.bf16_bits_to_f32(b.q)
    kf = W.bf16_bits_to_f32(b.k)
    if case == "very_negative_no_sink":
        qf = np.full_like(qf, 4.0)
        kf = np.full_like(kf, -4.0) + np.round(kf * 4) / 64
    elif case == "very_positive_zero_sink":
        qf = np.full_like(qf, 4.0)
        kf = np.full_like(kf, 4.0) + np.round(kf * 4) / 64
    else:
        kf = kf * (1.0 + np.arange(16, dtype=np.float32)[None, None, :, None] / 4.0)
    b.q = W.to_bf16_bits(qf)
    b.k = W.to_bf16_bits(kf)
    for R in (0, 8):
        _case(f"balanced {case} R={R}", b, R)


def test_balanced_two_passes_match_one_call_and_reuse_workspace():
    """partial + finish == the one-call entry point, bit for bit; a second,
    smaller batch on the same workspace sees none of the first's partials;
    repeated calls are deterministic."""
    from gqa_attention_sinks_attn_amd import (F32, device, sink_attn_decode_balanced_finish,
                                              sink_attn_decode_balanced_partial)
    big = W.make_batch(61, kind="decode", qlens=[1] * 6, kv_lens=[3000, 17, 900, 1, 2500, 64],
                       hq=16, hkv=2, paged=True, sinks="normal")
    db = bal_device(big, 8)
    device.run(db)
    one = db.out.clone(), db.lse.clone()
    db.out.zero_()
    db.lse.zero_()
    sink_attn_decode_balanced_partial(db.q, db.k, db.v, db.kv_indptr, db.page_indices, db.kv_len,
                                      db.sinks, db.batch, db.num_qo_heads, db.num_kv_heads,
                                      db.head_dim, db.page_size, db.max_kv_len, 8, db.sm_scale,
                                      db.out, F32, db.lse, db.workspace, db.workspace_bytes)
    sink_attn_decode_balanced_finish(db.kv_indptr, db.sinks, db.batch, db.num_qo_heads,
                                     db.num_kv_heads, db.head_dim, db.max_kv_len, 8, db.out, F32,
                                     db.lse, db.workspace, db.workspace_bytes)
    torch.cuda.synchronize()
    assert torch.equal(one[0], db.out) and torch.equal(one[1], db.lse)
    device.run(db)
    torch.cuda.synchronize()
    assert torch.equal(one[0], db.out) and torch.equal(one[1], db.lse)
    ref, rl = oracle.attend(big)
    check("balanced two passes", db.out.cpu().numpy(), ref, db.lse.cpu().numpy(), rl,
          bf16_out=False)

    small = W.make_batch(62, kind="decode", qlens=[1] * 3, kv_lens=[40, 700, 5], hq=16, hkv=2,
                         paged=True, sinks="normal")
    ds = device.to_device(small, plan="balanced", num_ranges=8)
    assert ds.workspace_bytes <= db.workspace_bytes
    ds.workspace, ds.workspace_bytes = db.workspace, db.workspace_bytes   # stale partials inside
    device.run(ds)
    torch.cuda.synchronize()
    ref, rl = oracle.attend(small)
    check("balanced reused workspace", ds.out.cpu().numpy(), ref, ds.lse.cpu().numpy(), rl,
          bf16_out=False)


def test_balanced_agrees_with_chunked():
    """Both decode plans on the same batch: two roundings of the same sums."""
    from gqa_attention_sinks_attn_amd import device
    b = W.make_batch(63, kind="decode", qlens=[1] * 16, kv_lens=list(range(1, 4000, 250)), hq=64,
                     hkv=8, paged=True, sinks="normal")
    dc = device.to_device(b)
    device.run(dc)
    out_b, lse_b, _ = bal_run(b)
    torch.cuda.synchronize()
    assert np.abs(dc.out.cpu().numpy() - out_b).max() <= 1e-2
    assert np.abs(dc.lse.cpu().numpy() - lse_b).max() <= 5e-3
