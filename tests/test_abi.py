"""C-ABI tests that need no GPU: the library loads, exports every entry point
that include/sink_attn.h declares, and rejects bad arguments on the host
before anything is enqueued (so no device is touched).  Fake, aligned
addresses stand in for device pointers: validation never dereferences."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sink_attn.h")

import gqa_attention_sinks_attn_amd as sa  # noqa: E402

OK, NULL, SHAPE, UNSUP, MISAL, WS, HIP = range(7)
A = 0x10000    # a 16-byte aligned fake address
A2 = 0x20000
A3 = 0x30000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(sink_attn_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) >= {"sink_attn_prefill", "sink_attn_decode", "sink_attn_merge",
                          "sink_attn_decode_workspace_size", "sink_attn_status_string",
                          "sink_attn_last_error"}
    lib = ctypes.CDLL(sa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(sa.SYMBOLS) == set(names)


def test_status_strings():
    for s in range(7):
        assert sa.sink_attn_status_string(s)
    assert sa.sink_attn_status_string(99) == "unknown status"
    assert "gfx950" in sa.sink_attn_version()


def prefill_args(**over):
    args = dict(q=A, qo_indptr=A, k=A, v=A, kv_indptr=A, page_indices=None, kv_len=None,
                sinks=A, batch=2, num_qo_heads=64, num_kv_heads=8, head_dim=64, page_size=16,
                total_q=10, max_qlen=6, max_kv_len=6, sm_scale=0.125, causal=1, out=A2,
                out_dtype=0, lse=A3, stream=0)
    args.update(over)
    return args


def call_prefill(**over):
    a = prefill_args(**over)
    return sa.lib().sink_attn_prefill(
        a["q"], a["qo_indptr"], a["k"], a["v"], a["kv_indptr"], a["page_indices"], a["kv_len"],
        a["sinks"], a["batch"], a["num_qo_heads"], a["num_kv_heads"], a["head_dim"],
        a["page_size"], a["total_q"], a["max_qlen"], a["max_kv_len"], a["sm_scale"],
        a["causal"], a["out"], a["out_dtype"], a["lse"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), NULL), (dict(out=None), NULL), (dict(kv_indptr=None), NULL),
    (dict(page_indices=A, kv_len=None), NULL),
    (dict(batch=0), SHAPE), (dict(total_q=-1), SHAPE), (dict(max_qlen=11), SHAPE),
    (dict(num_kv_heads=7), SHAPE), (dict(num_qo_heads=0), SHAPE), (dict(sm_scale=0.0), SHAPE),
    (dict(sm_scale=float("inf")), SHAPE), (dict(max_kv_len=0), SHAPE),
    (dict(head_dim=128), UNSUP), (dict(page_indices=A, kv_len=A, page_size=32), UNSUP),
    (dict(num_qo_heads=256, num_kv_heads=8), UNSUP), (dict(num_qo_heads=24, num_kv_heads=8), UNSUP),
    (dict(out_dtype=7), UNSUP),
    (dict(q=A + 2), MISAL), (dict(k=A + 8), MISAL), (dict(out=A2 + 4), MISAL),
    (dict(qo_indptr=A + 1), MISAL), (dict(lse=A3 + 2), MISAL),
])
def test_prefill_rejects(over, code):
    assert call_prefill(**over) == code
    assert sa.sink_attn_last_error() != ""


def test_prefill_empty_batch_is_a_noop():
    # nothing to compute -> OK without touching the device
    assert call_prefill(total_q=0, max_qlen=0) == OK
    assert sa.sink_attn_last_error() == ""


def call_decode(**over):
    a = dict(q=A, k=A, v=A, page_indptr=A, page_indices=A, kv_len=A, sinks=A, batch=4,
             num_qo_heads=64, num_kv_heads=8, head_dim=64, page_size=16, max_kv_len=131072,
             num_splits=32, sm_scale=0.125, out=A2, out_dtype=0, lse=None, workspace=A3,
             workspace_bytes=0, stream=0)
    a.update(over)
    return sa.lib().sink_attn_decode(
        a["q"], a["k"], a["v"], a["page_indptr"], a["page_indices"], a["kv_len"], a["sinks"],
        a["batch"], a["num_qo_heads"], a["num_kv_heads"], a["head_dim"], a["page_size"],
        a["max_kv_len"], a["num_splits"], a["sm_scale"], a["out"], a["out_dtype"], a["lse"],
        a["workspace"], a["workspace_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), NULL), (dict(page_indices=None), NULL), (dict(kv_len=None), NULL),
    (dict(batch=-1), SHAPE), (dict(num_splits=-2), SHAPE), (dict(num_kv_heads=3), SHAPE),
    (dict(head_dim=96), UNSUP), (dict(page_size=8), UNSUP),
    (dict(num_qo_heads=256, num_kv_heads=8), UNSUP),
    (dict(v=A + 2), MISAL), (dict(kv_len=A + 2), MISAL),
    (dict(workspace=None, workspace_bytes=10 ** 9), WS), (dict(workspace_bytes=100), WS),
])
def test_decode_rejects(over, code):
    assert call_decode(**over) == code
    assert sa.sink_attn_last_error() != ""


def call_partial(**over):
    a = dict(q=A, k=A, v=A, page_indptr=A, page_indices=A, kv_len=A, sinks=None, batch=4,
             num_qo_heads=64, num_kv_heads=8, head_dim=64, page_size=16, max_kv_len=4096,
             num_splits=0, sm_scale=0.125, o=A2, l=A3, stream=0)
    a.update(over)
    return sa.lib().sink_attn_decode_partial(
        a["q"], a["k"], a["v"], a["page_indptr"], a["page_indices"], a["kv_len"], a["sinks"],
        a["batch"], a["num_qo_heads"], a["num_kv_heads"], a["head_dim"], a["page_size"],
        a["max_kv_len"], a["num_splits"], a["sm_scale"], a["o"], a["l"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(o=None), NULL), (dict(l=None), NULL), (dict(k=None), NULL), (dict(batch=0), SHAPE),
    (dict(head_dim=32), UNSUP), (dict(o=A2 + 4), MISAL), (dict(l=A3 + 2), MISAL),
])
def test_decode_partial_rejects(over, code):
    assert call_partial(**over) == code


def test_decode_rejects_misaligned_workspace():
    need = sa.sink_attn_decode_workspace_size(4, 64, 8, 64, 131072, 32)
    assert call_decode(workspace=A3 + 8, workspace_bytes=need) == MISAL


def test_workspace_and_plan():
    # 32 explicit splits: o [4,64,32,64] fp32 + lse [4,64,32] fp32 (256-B padded)
    need = sa.sink_attn_decode_workspace_size(4, 64, 8, 64, 131072, 32)
    assert need == 4 * 64 * 32 * 64 * 4 + ((4 * 64 * 32 * 4 + 255) // 256) * 256
    assert sa.sink_attn_decode_num_splits(4, 64, 8, 131072, 32) == 32
    # one split needs no workspace
    assert sa.sink_attn_decode_workspace_size(64, 64, 8, 64, 16, 0) == 0
    assert sa.sink_attn_decode_num_splits(64, 64, 8, 16, 0) == 1
    # never more splits than pages
    assert sa.sink_attn_decode_num_splits(1, 8, 8, 40, 32) == 3
    # the automatic plan stays within bounds
    for B, L in [(1, 1), (64, 4096), (4, 131072), (256, 16384), (1, 10 ** 6)]:
        s = sa.sink_attn_decode_num_splits(B, 64, 8, L, 0)
        assert 1 <= s <= 256
        pages = (L + 15) // 16
        assert s <= max(1, pages)


def call_merge(**over):
    a = dict(o=A, l=A2, rows=4, heads=64, splits=8, d=64, out=A3, dt=0, lse=None, stream=0)
    a.update(over)
    return sa.lib().sink_attn_merge(a["o"], a["l"], a["rows"], a["heads"], a["splits"], a["d"],
                                    a["out"], a["dt"], a["lse"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(o=None), NULL), (dict(out=None), NULL), (dict(splits=0), SHAPE),
    (dict(heads=0), SHAPE), (dict(rows=-1), SHAPE), (dict(d=32), UNSUP), (dict(dt=3), UNSUP),
    (dict(o=A + 4), MISAL), (dict(l=A2 + 1), MISAL),
])
def test_merge_rejects(over, code):
    assert call_merge(**over) == code


def test_merge_zero_rows_is_a_noop():
    assert call_merge(rows=0) == OK


def test_python_binding_raises_with_detail():
    with pytest.raises(sa.SinkAttnError) as e:
        sa.sink_attn_merge(None, A2, 4, 64, 8, 64, A3, 0, None, stream=0)
    assert e.value.status == NULL and "required" in e.value.detail


# ------------------------------------------------------- load-balanced decode

def call_balanced(fn="sink_attn_decode_balanced", **over):
    a = dict(q=A, k=A, v=A, page_indptr=A, page_indices=A, kv_len=A, sinks=A, batch=64,
             num_qo_heads=64, num_kv_heads=8, head_dim=64, page_size=16, max_kv_len=4096,
             num_ranges=0, sm_scale=0.125, out=A2, out_dtype=1, lse=None, workspace=A3,
             workspace_bytes=None, stream=0)
    a.update(over)
    if a["workspace_bytes"] is None:
        a["workspace_bytes"] = sa.sink_attn_decode_balanced_workspace_size(
            a["batch"], a["num_qo_heads"], a["num_kv_heads"], 64, a["max_kv_len"], a["num_ranges"])
    f = getattr(sa.lib(), fn)
    if fn == "sink_attn_decode_balanced_finish":
        return f(a["page_indptr"], a["sinks"], a["batch"], a["num_qo_heads"], a["num_kv_heads"],
                 a["head_dim"], a["max_kv_len"], a["num_ranges"], a["out"], a["out_dtype"],
                 a["lse"], a["workspace"], a["workspace_bytes"], a["stream"])
    return f(a["q"], a["k"], a["v"], a["page_indptr"], a["page_indices"], a["kv_len"], a["sinks"],
             a["batch"], a["num_qo_heads"], a["num_kv_heads"], a["head_dim"], a["page_size"],
             a["max_kv_len"], a["num_ranges"], a["sm_scale"], a["out"], a["out_dtype"], a["lse"],
             a["workspace"], a["workspace_bytes"], a["stream"])


@pytest.mark.parametrize("fn", ["sink_attn_decode_balanced", "sink_attn_decode_balanced_partial"])
@pytest.mark.parametrize("over,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(page_indices=None), NULL),
    (dict(out=None), NULL), (dict(batch=0), SHAPE), (dict(num_ranges=-4), SHAPE),
    (dict(num_kv_heads=3), SHAPE), (dict(max_kv_len=-1), SHAPE), (dict(sm_scale=-1.0), SHAPE),
    (dict(head_dim=128), UNSUP), (dict(page_size=32), UNSUP), (dict(out_dtype=5), UNSUP),
    (dict(num_qo_heads=256, num_kv_heads=8), UNSUP),
    (dict(q=A + 4), MISAL), (dict(out=A2 + 8), MISAL), (dict(page_indptr=A + 2), MISAL),
    (dict(workspace=None), WS), (dict(workspace_bytes=1024), WS), (dict(workspace=A3 + 8), MISAL),
])
def test_balanced_rejects(fn, over, code):
    assert call_balanced(fn, **over) == code
    assert sa.sink_attn_last_error() != ""


@pytest.mark.parametrize("over,code", [
    (dict(page_indptr=None), NULL), (dict(out=None), NULL), (dict(batch=-1), SHAPE),
    (dict(num_ranges=-1), SHAPE), (dict(head_dim=32), UNSUP), (dict(out_dtype=9), UNSUP),
    (dict(workspace=None), WS), (dict(workspace_bytes=64), WS), (dict(lse=A + 2), MISAL),
])
def test_balanced_finish_rejects(over, code):
    # the finish pass needs neither q nor the cache
    assert call_balanced("sink_attn_decode_balanced_finish", q=None, k=None, v=None,
                         **over) == code


def test_balanced_plan_and_workspace():
    # automatic plan: one workgroup (four ranges) per CU over all KV heads
    assert sa.sink_attn_decode_num_ranges(64, 8, 4096, 0) == 128
    assert sa.sink_attn_decode_num_ranges(4, 8, 131072, 0) == 128
    assert sa.sink_attn_decode_num_ranges(4, 1, 131072, 0) == 1024
    for hkv in (1, 2, 3, 4, 5, 8, 16, 64):
        r = sa.sink_attn_decode_num_ranges(256, hkv, 16384, 0)
        assert r % 4 == 0 and r >= 4 and hkv * r // 4 <= 256
    # short batches: ranges of at least 8 pages
    assert sa.sink_attn_decode_num_ranges(1, 8, 100, 0) == 4
    assert sa.sink_attn_decode_num_ranges(2, 8, 16 * 64, 0) == 16
    # explicit counts round up to a multiple of 4
    assert sa.sink_attn_decode_num_ranges(64, 8, 4096, 5) == 8
    assert sa.sink_attn_decode_num_ranges(64, 8, 4096, 400) == 400
    # workspace: partials for n_ranges + batch - 1 slots, lse at the next 256-byte boundary
    for B, R in [(64, 0), (64, 12), (1, 0), (4500, 100)]:
        n = sa.sink_attn_decode_num_ranges(B, 2, 4096, R)
        rows = (n + B - 1) * 16
        assert sa.sink_attn_decode_balanced_workspace_size(B, 16, 2, 64, 4096, R) == \
            rows * 64 * 4 + ((rows * 4 + 255) // 256) * 256


def test_decode_automatic_plan_uses_the_balanced_workspace():
    # more than 16 pages per request: the balanced plan and its workspace
    assert sa.sink_attn_decode_workspace_size(64, 64, 8, 64, 4096, 0) == \
        sa.sink_attn_decode_balanced_workspace_size(64, 64, 8, 64, 4096, 0)
    need = sa.sink_attn_decode_workspace_size(64, 64, 8, 64, 4096, 0)
    assert call_decode(batch=64, max_kv_len=4096, num_splits=0, workspace=None,
                       workspace_bytes=0) == WS
    assert call_decode(batch=64, max_kv_len=4096, num_splits=0, workspace_bytes=need - 1) == WS
    # up to 16 pages: one chunk, no workspace
    assert sa.sink_attn_decode_workspace_size(64, 64, 8, 64, 256, 0) == 0


def _simulate_partition(indptr, n_ranges, min_pages):
    """Host model of the page partition of the balanced decode: the ranges,
    the segments each range's wave closes (request, first page, sink?, slot
    or direct), and the slots the finish pass reads per request."""
    B = len(indptr) - 1
    nnz = indptr[-1]
    Rw = max(min_pages, -(-nnz // n_ranges))
    owner = np.repeat(np.arange(B), np.diff(indptr))
    segs = []
    for u in range(n_ranges):
        p0, p1 = u * Rw, min(nnz, u * Rw + Rw)
        pg = p0
        while pg < p1:
            b = owner[pg]
            end = min(p1, indptr[b + 1])
            whole = indptr[b] // Rw == (indptr[b + 1] - 1) // Rw
            segs.append((u, b, pg, end, pg == indptr[b], None if whole else u + b))
            pg = end
    reads = {}
    for b in range(B):
        if indptr[b + 1] > indptr[b]:
            u0, u1 = indptr[b] // Rw, (indptr[b + 1] - 1) // Rw
            if u0 != u1:
                reads[b] = [u + b for u in range(u0, u1 + 1)]
    return Rw, segs, reads


@pytest.mark.parametrize("seed", range(6))
def test_balanced_partition_covers_every_page_once(seed):
    """Every page is streamed by exactly one wave; each request gets the sink
    exactly once (in the segment holding its first page); partial slots are
    unique and within the workspace; the finish pass reads exactly the slots
    the first pass wrote for the request."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 300))
    pages = rng.integers(0, 40, size=B)
    pages[rng.random(B) < 0.2] = 0
    indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int64)
    for R in (4, 8, 12, 100):
        n = sa.sink_attn_decode_num_ranges(B, 2, 40 * 16, R)
        Rw, segs, reads = _simulate_partition(indptr, n, 1)
        assert Rw * n >= indptr[-1]
        seen = np.zeros(int(indptr[-1]), np.int64)
        sinks = np.zeros(B, np.int64)
        slots = {}
        for u, b, s0, s1, has_sink, slot in segs:
            seen[s0:s1] += 1
            sinks[b] += has_sink
            if slot is not None:
                assert slot not in slots and 0 <= slot < n + B - 1
                slots[slot] = b
        assert np.all(seen == 1)
        assert np.array_equal(sinks, (pages > 0).astype(np.int64))
        for b, rs in reads.items():
            assert all(slots.get(s) == b for s in rs)
        assert sorted(slots) == sorted(s for rs in reads.values() for s in rs)


# ------------------------------------------------------------- verification

def call_verify(**over):
    # 8 requests: the automatic plan splits, so a missing workspace is an
    # error and no argument set below reaches a launch
    a = dict(q=A, qo=A, k=A, v=A, page_indptr=A, page_indices=A, kv_len=A, sinks=A, batch=8,
             num_qo_heads=64, num_kv_heads=8, head_dim=64, page_size=16, total_q=256, max_qlen=4,
             max_kv_len=4096, num_splits=0, sm_scale=0.125, out=A2, out_dtype=1, lse=None,
             workspace=A3, workspace_bytes=None, stream=0)
    a.update(over)
    if a["workspace_bytes"] is None:
        a["workspace_bytes"] = sa.sink_attn_verify_workspace_size(
            a["batch"], a["num_qo_heads"], a["num_kv_heads"], 64, a["total_q"], a["max_qlen"],
            a["max_kv_len"], a["num_splits"])
    return sa.lib().sink_attn_verify(
        a["q"], a["qo"], a["k"], a["v"], a["page_indptr"], a["page_indices"], a["kv_len"],
        a["sinks"], a["batch"], a["num_qo_heads"], a["num_kv_heads"], a["head_dim"],
        a["page_size"], a["total_q"], a["max_qlen"], a["max_kv_len"], a["num_splits"],
        a["sm_scale"], a["out"], a["out_dtype"], a["lse"], a["workspace"], a["workspace_bytes"],
        a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(qo=None), NULL), (dict(q=None), NULL), (dict(out=None), NULL), (dict(kv_len=None), NULL),
    (dict(batch=0), SHAPE), (dict(max_qlen=300), SHAPE), (dict(total_q=-1), SHAPE),
    (dict(max_qlen=65), UNSUP),                      # more drafted tokens than a mask word
    (dict(num_qo_heads=64, num_kv_heads=4, max_qlen=200), UNSUP),
    (dict(head_dim=128), UNSUP), (dict(page_size=32), UNSUP), (dict(out_dtype=4), UNSUP),
    (dict(out=A2 + 4), MISAL), (dict(qo=A + 2), MISAL), (dict(workspace=A3 + 8), MISAL),
    (dict(workspace=None), WS), (dict(workspace_bytes=16), WS),
])
def test_verify_rejects(over, code):
    assert call_verify(**over) == code
    assert sa.sink_attn_last_error() != ""


def test_verify_plan_and_workspace():
    nsp = sa.sink_attn_verify_num_splits
    # 64 requests x 8 KV heads fill the GPU: one chunk, no workspace
    assert nsp(64, 64, 8, 4, 4096, 0) == 1
    assert sa.sink_attn_verify_workspace_size(64, 64, 8, 64, 256, 4, 4096, 0) == 0
    # 8 requests: 64 (request, KV head) pairs x 1 column group -> 8 chunks
    assert nsp(8, 64, 8, 4, 4096, 0) == 8
    # 8-token drafts at G = 8: 64 pairs = 2 groups of 32 -> 4 chunks
    assert nsp(8, 64, 8, 8, 4096, 0) == 4
    # past 64 pairs per KV head the tile kernel runs: 128-row tiles, chunks
    # of >= 8 tiles (512 keys) towards 1,024 (request, KV head, chunk) items
    assert nsp(64, 64, 8, 16, 4096, 0) == 2          # 512 (request, KV head) pairs
    assert nsp(128, 64, 8, 16, 4096, 0) == 1         # 1,024 pairs: one chunk
    assert sa.sink_attn_verify_workspace_size(128, 64, 8, 64, 2048, 16, 4096, 0) == 0
    assert nsp(64, 64, 8, 32, 4096, 0) == 2          # 512 pairs, whatever the 2 row tiles
    assert nsp(8, 64, 8, 16, 4096, 0) == 8           # 64 pairs, 64 tiles
    assert nsp(2, 64, 8, 32, 4096, 0) == 8           # 16 pairs (2 row tiles)
    assert nsp(2, 64, 4, 32, 4096, 0) == 8           # G = 16: 4 row tiles, 8 pairs
    assert nsp(8, 64, 8, 16, 300, 0) == 1            # 5 tiles: too short to split
    assert nsp(2, 64, 8, 16, 131072, 0) == 64        # 16 pairs -> 64 chunks of 32 tiles
    # at most 64 chunks: an explicit request is capped there
    assert nsp(1, 64, 8, 16, 131072, 1000) == 64
    S = nsp(2, 64, 8, 32, 4096, 0)
    rows = 64 * 64 * S
    assert sa.sink_attn_verify_workspace_size(2, 64, 8, 64, 64, 32, 4096, 0) == \
        rows * 64 * 4 + ((rows * 4 + 255) // 256) * 256
    # nothing to compute (no rows, no requests) plans one chunk
    assert nsp(8, 64, 8, 0, 4096, 0) == 1 and nsp(0, 64, 8, 4, 4096, 0) == 1
    # chunks keep >= 16 pages; short caches are not split
    assert nsp(1, 64, 8, 2, 1024, 0) == 4 and nsp(1, 64, 8, 2, 256, 0) == 1
    # an explicit count is taken, clamped to the page count
    assert nsp(64, 64, 8, 4, 4096, 3) == 3 and nsp(2, 64, 8, 4, 40, 9) == 3
    S = nsp(8, 64, 8, 4, 4096, 0)
    need = sa.sink_attn_verify_workspace_size(8, 64, 8, 64, 32, 4, 4096, 0)
    rows = 32 * 64 * S
    assert need == rows * 64 * 4 + ((rows * 4 + 255) // 256) * 256
    assert sa.sink_attn_verify_workspace_size(8, 64, 8, 64, 32, 4, 4096, 1) == 0
    # nothing to compute: OK without a workspace
    assert call_verify(total_q=0, max_qlen=0, workspace=None, workspace_bytes=0) == OK
    # up to 64 drafted tokens, whatever the group size
    assert call_verify(num_qo_heads=32, num_kv_heads=8, max_qlen=65) == UNSUP
    assert call_verify(num_qo_heads=16, num_kv_heads=16, max_qlen=65) == UNSUP


def call_verify_tree(mask=A, **over):
    a = dict(q=A, qo=A, k=A, v=A, page_indptr=A, page_indices=A, kv_len=A, sinks=A, batch=64,
             num_qo_heads=64, num_kv_heads=8, head_dim=64, page_size=16, total_q=256, max_qlen=4,
             max_kv_len=4096, num_splits=1, sm_scale=0.125, out=A2, out_dtype=1, lse=None,
             workspace=None, workspace_bytes=0, stream=0)
    a.update(over)
    return sa.lib().sink_attn_verify_tree(
        a["q"], a["qo"], mask, a["k"], a["v"], a["page_indptr"], a["page_indices"], a["kv_len"],
        a["sinks"], a["batch"], a["num_qo_heads"], a["num_kv_heads"], a["head_dim"],
        a["page_size"], a["total_q"], a["max_qlen"], a["max_kv_len"], a["num_splits"],
        a["sm_scale"], a["out"], a["out_dtype"], a["lse"], a["workspace"], a["workspace_bytes"],
        a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(mask=None), NULL), (dict(mask=A + 4), MISAL), (dict(max_qlen=65, total_q=300), UNSUP),
    (dict(qo=None), NULL), (dict(batch=0), SHAPE), (dict(head_dim=128), UNSUP),
    (dict(num_splits=0, batch=8), WS),               # the automatic plan splits 8 requests
])
def test_verify_tree_rejects(over, code):
    assert call_verify_tree(**over) == code
    assert sa.sink_attn_last_error() != ""


def test_verify_tree_empty_call_is_ok():
    assert call_verify_tree(total_q=0, max_qlen=0) == OK


def call_rope_table(**over):
    a = dict(table=A, max_pos=4096, head_dim=64, theta=150000.0, factor=32.0, orig=4096,
             beta_fast=32.0, beta_slow=1.0, attn_factor=0.0, ramp=0, stream=0)
    a.update(over)
    return sa.lib().sink_attn_rope_table(a["table"], a["max_pos"], a["head_dim"], a["theta"],
                                         a["factor"], a["orig"], a["beta_fast"], a["beta_slow"],
                                         a["attn_factor"], a["ramp"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(table=None), NULL), (dict(max_pos=0), SHAPE), (dict(head_dim=128), UNSUP),
    (dict(theta=1.0), SHAPE), (dict(factor=0.0), SHAPE), (dict(attn_factor=-1.0), SHAPE),
    (dict(orig=0), SHAPE), (dict(beta_fast=1.0), SHAPE), (dict(beta_slow=0.0), SHAPE),
    (dict(theta=float("inf")), SHAPE), (dict(table=A + 4), MISAL), (dict(ramp=2), UNSUP),
    (dict(ramp=-1), UNSUP),
])
def test_rope_table_rejects(over, code):
    assert call_rope_table(**over) == code
    assert sa.sink_attn_last_error() != ""


def call_append(**over):
    a = dict(qkv=A, bias=A, table=A, max_pos=4096, qo=A, kv_len=A, page_indptr=A,
             page_indices=A, batch=4, hq=64, hkv=8, head_dim=64, page_size=16, total_q=0,
             interleaved=0, q_out=A2, k=A3, v=A3, stream=0)
    a.update(over)
    return sa.lib().sink_attn_qkv_rope_append(
        a["qkv"], a["bias"], a["table"], a["max_pos"], a["qo"], a["kv_len"], a["page_indptr"],
        a["page_indices"], a["batch"], a["hq"], a["hkv"], a["head_dim"], a["page_size"],
        a["total_q"], a["interleaved"], a["q_out"], a["k"], a["v"], a["stream"])


# total_q = 0 everywhere: a valid set of arguments returns before any launch
@pytest.mark.parametrize("over,code", [
    (dict(), OK), (dict(bias=None), OK),
    (dict(qkv=None), NULL), (dict(table=None), NULL), (dict(page_indices=None), NULL),
    (dict(q_out=None), NULL), (dict(k=None), NULL),
    (dict(batch=0), SHAPE), (dict(total_q=-1), SHAPE), (dict(max_pos=0), SHAPE),
    (dict(head_dim=128), UNSUP), (dict(page_size=32), UNSUP), (dict(interleaved=2), UNSUP),
    (dict(qkv=A + 8), MISAL), (dict(bias=A + 2), MISAL), (dict(q_out=A2 + 4), MISAL),
    (dict(qo=A + 2), MISAL),
])
def test_qkv_rope_append_validation(over, code):
    assert call_append(**over) == code


def test_decode_noalloc_rejects_sizes_beyond_its_array():
    """The static scratch array holds 16 MiB: larger workspaces are refused on
    the host, before any device access (fake pointers stay untouched)."""
    lib = sa.lib()
    B, Hq, Hkv = 1200, 64, 8
    need = lib.sink_attn_decode_workspace_size(B, Hq, Hkv, 64, 4096, 0)
    assert need > 16 << 20
    rc = lib.sink_attn_decode_noalloc(A, A, A, A, A, A, A, B, Hq, Hkv, 64, 16, 4096, 0, 0.125, A2,
                                      1, None, None)
    assert rc == WS
    assert "static scratch" in sa.sink_attn_last_error()
    # the usual argument checks still come first for invalid sizes
    assert lib.sink_attn_decode_noalloc(None, A, A, A, A, A, A, 4, Hq, Hkv, 64, 16, 4096, 0, 0.125,
                                        A2, 1, None, None) == NULL


def call_step(**over):
    a = dict(qkv=A, bias=A, table=A, max_pos=4096, interleaved=0, k=A3, v=A3, page_indptr=A,
             page_indices=A, kv_len=A, sinks=A, batch=4, hq=64, hkv=8, head_dim=64,
             page_size=16, max_kv_len=4096, sm_scale=0.125, out=A2, out_dtype=1, lse=A3,
             ws=A, ws_bytes=1 << 30, stream=0)
    a.update(over)
    return sa.lib().sink_attn_decode_step(
        a["qkv"], a["bias"], a["table"], a["max_pos"], a["interleaved"], a["k"], a["v"],
        a["page_indptr"], a["page_indices"], a["kv_len"], a["sinks"], a["batch"], a["hq"],
        a["hkv"], a["head_dim"], a["page_size"], a["max_kv_len"], a["sm_scale"], a["out"],
        a["out_dtype"], a["lse"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(qkv=None), NULL), (dict(table=None), NULL), (dict(k=None), NULL),
    (dict(page_indices=None), NULL), (dict(out=None), NULL),
    (dict(max_pos=0), SHAPE), (dict(batch=0), SHAPE), (dict(sm_scale=0.0), SHAPE),
    (dict(interleaved=2), UNSUP), (dict(head_dim=128), UNSUP), (dict(page_size=32), UNSUP),
    (dict(hq=24, hkv=8), UNSUP), (dict(hq=12, hkv=8), SHAPE), (dict(out_dtype=7), UNSUP),
    (dict(bias=A + 2), MISAL), (dict(table=A + 4), MISAL), (dict(qkv=A + 8), MISAL),
    (dict(k=A3 + 2), MISAL), (dict(out=A2 + 4), MISAL),
    (dict(ws=None), WS), (dict(ws_bytes=16), WS),
])
def test_decode_step_validation(over, code):
    assert call_step(**over) == code, sa.sink_attn_last_error()


def test_decode_step_workspace_holds_the_queries():
    """The step's workspace is the balanced decode's plus the rotated
    queries (bf16 [batch, Hq, 64]); one byte less is refused."""
    lib = sa.lib()
    for B, Hq, Hkv, L in [(64, 64, 8, 4096), (3, 16, 1, 20), (256, 128, 8, 16384)]:
        bal = lib.sink_attn_decode_balanced_workspace_size(B, Hq, Hkv, 64, L, 0)
        step = lib.sink_attn_decode_step_workspace_size(B, Hq, Hkv, 64, L)
        assert step >= bal + B * Hq * 64 * 2
        assert step - bal < B * Hq * 64 * 2 + 256
        assert call_step(batch=B, hq=Hq, hkv=Hkv, max_kv_len=L, ws_bytes=step - 1) == WS


def call_prefill_step(**over):
    a = dict(qkv=A, bias=A, table=A, max_pos=4096, interleaved=0, qo=A, k=A3, v=A3,
             page_indptr=A, page_indices=A, kv_len=A, sinks=A, batch=4, hq=64, hkv=8,
             head_dim=64, page_size=16, total_q=40, max_qlen=10, max_kv_len=4096,
             sm_scale=0.125, causal=1, out=A2, out_dtype=1, lse=A3, stream=0)
    a.update(over)
    return sa.lib().sink_attn_prefill_step(
        a["qkv"], a["bias"], a["table"], a["max_pos"], a["interleaved"], a["qo"], a["k"], a["v"],
        a["page_indptr"], a["page_indices"], a["kv_len"], a["sinks"], a["batch"], a["hq"],
        a["hkv"], a["head_dim"], a["page_size"], a["total_q"], a["max_qlen"], a["max_kv_len"],
        a["sm_scale"], a["causal"], a["out"], a["out_dtype"], a["lse"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(qkv=None), NULL), (dict(table=None), NULL), (dict(page_indices=None), NULL),
    (dict(kv_len=None), NULL), (dict(k=None), NULL), (dict(out=None), NULL),
    (dict(qo=None), NULL),
    (dict(max_pos=0), SHAPE), (dict(batch=0), SHAPE), (dict(max_qlen=50), SHAPE),
    (dict(sm_scale=-1.0), SHAPE), (dict(hq=12, hkv=8), SHAPE),
    (dict(interleaved=3), UNSUP), (dict(head_dim=32), UNSUP), (dict(page_size=8), UNSUP),
    (dict(hq=24, hkv=8), UNSUP), (dict(out_dtype=5), UNSUP),
    (dict(bias=A + 2), MISAL), (dict(table=A + 4), MISAL), (dict(qkv=A + 8), MISAL),
    (dict(k=A3 + 2), MISAL), (dict(out=A2 + 8), MISAL), (dict(lse=A3 + 2), MISAL),
])
def test_prefill_step_validation(over, code):
    assert call_prefill_step(**over) == code, sa.sink_attn_last_error()


def test_prefill_step_with_no_rows_launches_nothing():
    assert call_prefill_step(total_q=0, max_qlen=0) == OK


def test_a_plain_c_caller_builds_and_runs(tmp_path):
    """The header is C99 and the library links from C: tests/c_abi_consumer.c,
    compiled with gcc (no C++ runtime of its own) against libsink_attn.so,
    makes the device-free calls (planning queries, host validation) and
    checks their results."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(sa.LIB_PATH)
    exe = str(tmp_path / "c_abi_consumer")
    build = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                            "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "c_abi_consumer.c"), "-o", exe,
                            "-L", libdir, "-lsink_attn", f"-Wl,-rpath,{libdir}"],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "c consumer ok" in run.stdout
