"""The fused decode step (sink_attn_decode_step): each request's new token
gets its bias, rotary encoding and cache append inside the decode's first
pass.  It must equal, bit for bit (output, LSE and the whole cache), the
append (sink_attn_qkv_rope_append) followed by the balanced decode
(sink_attn_decode_balanced, automatic plan) on the same inputs; and, as
that pair, match the rope oracle (queries and cache) and the attention
oracle (output) at the parity bar.
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


MAX_POS = 20000


@pytest.fixture(scope="module")
def table():
    from gqa_attention_sinks_attn_amd import sink_attn_rope_table
    t = torch.empty((MAX_POS, 64), dtype=torch.float32, device="cuda")
    sink_attn_rope_table(t, MAX_POS, 64, 150000.0, 32.0, 4096, 32.0, 1.0, 0.0)
    torch.cuda.synchronize()
    return t


def _dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_both(ab, table, sinks, interleaved, out_dtype=torch.float32, bias=True, max_pos=MAX_POS,
             name=""):
    """The fused step and the append + balanced decode pair on two copies of
    the same inputs; returns both results (out, lse, k cache, v cache) and
    the pair's queries."""
    import gqa_attention_sinks_attn_amd as sa
    B, Hq, Hkv = len(ab.kv_len), ab.num_qo_heads, ab.num_kv_heads
    max_L = int(np.max(ab.kv_len)) if B else 0
    qkv = _dev_bf16(ab.qkv)
    bias_t = _dev_bf16(ab.bias) if (bias and ab.bias is not None) else None
    indptr, indices, kv_len = _dev_i32(ab.page_indptr), _dev_i32(ab.page_indices), _dev_i32(ab.kv_len)
    sinks_t = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    res = {}
    for mode in ("pair", "step"):
        ws_bytes = (sa.sink_attn_decode_balanced_workspace_size(B, Hq, Hkv, 64, max_L, 0)
                    if mode == "pair" else
                    sa.sink_attn_decode_step_workspace_size(B, Hq, Hkv, 64, max_L))
        k, v = _dev_bf16(ab.k_pages), _dev_bf16(ab.v_pages)
        out = torch.full((B, Hq, 64), float("nan"), dtype=out_dtype, device="cuda")
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        # workspace full of NaN bit patterns: nothing may depend on its contents
        ws = torch.full((max(ws_bytes, 256),), 0xFF, dtype=torch.uint8, device="cuda")
        q = None
        if mode == "pair":
            q = torch.zeros((B, Hq, 64), dtype=torch.bfloat16, device="cuda")
            qo = torch.arange(B + 1, dtype=torch.int32, device="cuda")
            sa.sink_attn_qkv_rope_append(qkv, bias_t, table, max_pos, qo, kv_len, indptr, indices,
                                         B, Hq, Hkv, 64, 16, B, interleaved, q, k, v)
            sa.sink_attn_decode_balanced(q, k, v, indptr, indices, kv_len, sinks_t, B, Hq, Hkv,
                                         64, 16, max_L, 0, 0.125, out, out_dtype, lse, ws,
                                         ws_bytes)
        else:
            sa.sink_attn_decode_step(qkv, bias_t, table, max_pos, interleaved, k, v, indptr,
                                     indices, kv_len, sinks_t, B, Hq, Hkv, 64, 16, max_L, 0.125,
                                     out, out_dtype, lse, ws, ws_bytes)
        torch.cuda.synchronize()
        res[mode] = dict(out=out, lse=lse, k=_bits(k), v=_bits(v),
                         q=None if q is None else _bits(q))
    print(f"[decode step {name}] B={B} Hq={Hq} Hkv={Hkv} max_L={max_L}", flush=True)
    return res


def assert_bitwise(res, rows=None):
    a, b = res["pair"], res["step"]
    oa, ob = a["out"], b["out"]
    la, lb = a["lse"], b["lse"]
    if rows is not None:
        oa, ob, la, lb = oa[rows], ob[rows], la[rows], lb[rows]
    ia = oa.view(torch.int16 if oa.dtype == torch.bfloat16 else torch.int32)
    ib = ob.view(torch.int16 if ob.dtype == torch.bfloat16 else torch.int32)
    assert torch.equal(ia, ib), f"outputs differ at {int((ia != ib).sum())} values"
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), "lse differs"
    assert np.array_equal(a["k"], b["k"]), "k cache differs"
    assert np.array_equal(a["v"], b["v"]), "v cache differs"


def oracle_check(name, ab, res, sinks, table_np, interleaved, bias=True):
    """The pair's queries and the (shared) cache against the rope oracle, the
    output against the attention oracle on them."""
    from oracle import rope
    B, Hq, Hkv = len(ab.kv_len), ab.num_qo_heads, ab.num_kv_heads
    pair = res["pair"]
    rq, rk, rv = rope.qkv_rope_append(ab.qkv, ab.bias if bias else None, table_np,
                                      np.arange(B + 1), ab.kv_len, ab.page_indptr,
                                      ab.page_indices, ab.k_pages, ab.v_pages, Hq, Hkv,
                                      bool(interleaved))
    got_q = W.bf16_bits_to_f32(pair["q"]).astype(np.float64)
    live = np.asarray(ab.kv_len) > 0
    assert np.all(np.abs(got_q[live] - rq[live]) <= 2.0 ** -8 * np.abs(rq[live]) + 1e-5), "q"
    got_k = W.bf16_bits_to_f32(res["step"]["k"]).astype(np.float64)
    got_v = W.bf16_bits_to_f32(res["step"]["v"]).astype(np.float64)
    assert np.all(np.abs(got_k - rk) <= 2.0 ** -8 * np.abs(rk) + 1e-5), "k cache"
    assert np.all(np.abs(got_v - rv) <= 2.0 ** -8 * np.abs(rv) + 1e-5), "v cache"
    b = W.Batch(kind="decode", q=pair["q"], qo_indptr=np.arange(B + 1, dtype=np.int32),
                k=res["step"]["k"], v=res["step"]["v"], kv_indptr=ab.page_indptr,
                page_indices=ab.page_indices, kv_len=np.asarray(ab.kv_len, np.int32),
                sinks=None if sinks is None else np.asarray(sinks, np.float32),
                num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=64, page_size=16, sm_scale=0.125,
                causal=True)
    ref, rl = oracle.attend(b)
    step = res["step"]
    bf16 = step["out"].dtype == torch.bfloat16
    check(name, step["out"].float().cpu().numpy(), ref,
          step["lse"].cpu().numpy().astype(np.float64), rl, bf16_out=bf16)


@pytest.fixture(scope="module")
def table_np():
    from oracle import rope
    return rope.rope_table(MAX_POS, 64, 150000.0, 32.0, 4096, 32.0, 1.0)


LENGTHS = [1, 2, 15, 16, 17, 31, 32, 33, 100, 257, 1000, 4096, 3, 48, 49, 700]


@pytest.mark.parametrize("interleaved", [0, 1])
def test_decode_step_equals_append_then_decode(table, table_np, interleaved):
    rng = np.random.default_rng(500 + interleaved)
    ab = W.make_append_batch(rng, qlens=[1] * len(LENGTHS), kv_lens=LENGTHS, hq=64, hkv=8,
                             spare_pages=3)
    sinks = rng.standard_normal(64).astype(np.float32)
    res = run_both(ab, table, sinks, interleaved, name=f"interleaved={interleaved}")
    assert_bitwise(res)
    oracle_check(f"decode step interleaved={interleaved}", ab, res, sinks, table_np, interleaved)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (16, 4), (64, 8), (64, 4), (128, 8)])
def test_decode_step_group_sizes(table, hq, hkv):
    rng = np.random.default_rng(510 + hq + hkv)
    L = rng.integers(1, 3000, size=12)
    ab = W.make_append_batch(rng, qlens=[1] * 12, kv_lens=L, hq=hq, hkv=hkv, spare_pages=2)
    sinks = (2.0 * rng.standard_normal(hq)).astype(np.float32)
    res = run_both(ab, table, sinks, 0, name=f"G={hq // hkv}")
    assert_bitwise(res)


def test_decode_step_no_bias_no_sinks_bf16_output(table, table_np):
    rng = np.random.default_rng(520)
    L = rng.integers(1, 2000, size=10)
    ab = W.make_append_batch(rng, qlens=[1] * 10, kv_lens=L, hq=16, hkv=2, bias=False)
    res = run_both(ab, table, None, 1, out_dtype=torch.bfloat16, bias=False, name="no bias")
    assert_bitwise(res)
    oracle_check("decode step no bias bf16", ab, res, None, table_np, 1, bias=False)


def test_decode_step_many_short_requests(table, table_np):
    """Hundreds of short requests: many request boundaries per page range,
    one-page requests, steps that straddle two requests, and empty ones."""
    rng = np.random.default_rng(530)
    L = rng.integers(0, 40, size=600)
    L[::7] = 1
    L[3::11] = 16
    L[5::13] = 17
    L[1::17] = 0     # requests without pages
    ab = W.make_append_batch(rng, qlens=[0 if x == 0 else 1 for x in L], kv_lens=L, hq=64, hkv=8,
                             spare_pages=1)
    # make_append_batch counts new tokens per request; the decode step has
    # one row per request, an empty request's row unused
    ab = _one_row_per_request(ab, rng)
    s = rng.standard_normal(64).astype(np.float32)
    s[3] = np.inf
    s[9] = -np.inf
    res = run_both(ab, table, s, 0, name="many short")
    assert_bitwise(res)
    live = np.flatnonzero(np.asarray(ab.kv_len) > 0)
    keep = [h for h in range(64) if h != 3]
    out = res["step"]["out"].float().cpu().numpy()
    lse = res["step"]["lse"].cpu().numpy().astype(np.float64)
    assert np.all(out[:, 3] == 0) and np.all(lse[:, 3] == np.inf)
    empty = np.flatnonzero(np.asarray(ab.kv_len) == 0)
    assert np.all(out[empty] == 0)
    # the attention oracle on the live requests
    from oracle import rope
    B = len(ab.kv_len)
    pair = res["pair"]
    b = W.Batch(kind="decode", q=pair["q"], qo_indptr=np.arange(B + 1, dtype=np.int32),
                k=res["step"]["k"], v=res["step"]["v"], kv_indptr=ab.page_indptr,
                page_indices=ab.page_indices, kv_len=np.asarray(ab.kv_len, np.int32), sinks=s,
                num_qo_heads=64, num_kv_heads=8, head_dim=64, page_size=16, sm_scale=0.125,
                causal=True)
    ref, rl = oracle.attend(b)
    check("decode step many short", out[live][:, keep], ref[live][:, keep], lse[live][:, keep],
          rl[live][:, keep], bf16_out=False)
    # rope oracle: the live requests' rows only (an empty request has no
    # position for its token)
    qo_live = np.zeros(B + 1, np.int64)
    qo_live[1:] = np.cumsum(np.asarray(ab.kv_len) > 0)
    rq, rk, rv = rope.qkv_rope_append(ab.qkv[live], ab.bias, table_np, qo_live, ab.kv_len,
                                      ab.page_indptr, ab.page_indices, ab.k_pages, ab.v_pages,
                                      64, 8, False)
    got_q = W.bf16_bits_to_f32(pair["q"][live]).astype(np.float64)
    assert np.all(np.abs(got_q - rq) <= 2.0 ** -8 * np.abs(rq) + 1e-5), "q"
    got_k = W.bf16_bits_to_f32(res["step"]["k"]).astype(np.float64)
    assert np.all(np.abs(got_k - rk) <= 2.0 ** -8 * np.abs(rk) + 1e-5), "k cache"


def _one_row_per_request(ab, rng):
    """The decode step reads qkv row b for request b: give every request a
    row (empty requests an unused random one)."""
    B = len(ab.kv_len)
    H = ab.num_qo_heads + 2 * ab.num_kv_heads
    qkv = W.to_bf16_bits(rng.standard_normal((B, H, 64), dtype=np.float32))
    return W.AppendBatch(qkv=qkv, bias=ab.bias, qo_indptr=np.arange(B + 1, dtype=np.int32),
                         kv_len=ab.kv_len, page_indptr=ab.page_indptr,
                         page_indices=ab.page_indices, k_pages=ab.k_pages, v_pages=ab.v_pages,
                         num_qo_heads=ab.num_qo_heads, num_kv_heads=ab.num_kv_heads,
                         head_dim=ab.head_dim, page_size=ab.page_size, name=ab.name)


def test_decode_step_positions_past_the_table(table):
    """A request whose new position has no table row: nothing of it is
    written to the cache (as the append skips it); the other requests are
    unaffected and equal the pair bit for bit."""
    rng = np.random.default_rng(540)
    L = np.array([5, 300, 1200, 40, 999], np.int64)
    ab = W.make_append_batch(rng, qlens=[1] * 5, kv_lens=L, hq=16, hkv=4, spare_pages=2)
    max_pos = 1000        # requests 2 (1200 keys) has position 1199 >= max_pos
    res = run_both(ab, table, rng.standard_normal(16).astype(np.float32), 0, max_pos=max_pos,
                   name="past the table")
    ok = [0, 1, 3, 4]
    assert_bitwise(res, rows=ok)   # caches: request 2's slot unwritten in both
    p = 1199
    page = ab.page_indices[ab.page_indptr[2] + p // 16]
    assert np.array_equal(res["step"]["k"][page, :, p % 16], ab.k_pages[page, :, p % 16])
    assert np.array_equal(res["step"]["v"][page, :, p % 16], ab.v_pages[page, :, p % 16])


def test_decode_step_graph_replays_over_a_growing_cache(table):
    """The fused step captured once and replayed over steps whose caches grow
    by one token, each replay equal bit for bit to the eager pair on the same
    inputs."""
    import gqa_attention_sinks_attn_amd as sa
    B, Hq, Hkv, max_L = 24, 64, 8, 2000
    H = Hq + 2 * Hkv
    rng = np.random.default_rng(550)
    L0 = rng.integers(1, max_L - 8, size=B)
    ab = W.make_append_batch(rng, qlens=[1] * B, kv_lens=L0 + 8, hq=Hq, hkv=Hkv, spare_pages=0)
    qkv = torch.zeros((B, H, 64), dtype=torch.bfloat16, device="cuda")
    bias = _dev_bf16(ab.bias)
    k, v = _dev_bf16(ab.k_pages), _dev_bf16(ab.v_pages)
    indptr, indices = _dev_i32(ab.page_indptr), _dev_i32(ab.page_indices)
    kv_len = torch.zeros(B, dtype=torch.int32, device="cuda")
    sinks = torch.from_numpy(rng.standard_normal(Hq).astype(np.float32)).cuda()
    out = torch.empty((B, Hq, 64), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws_bytes = sa.sink_attn_decode_step_workspace_size(B, Hq, Hkv, 64, max_L)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    ws2_bytes = sa.sink_attn_decode_balanced_workspace_size(B, Hq, Hkv, 64, max_L, 0)

    def call():
        sa.sink_attn_decode_step(qkv, bias, table, MAX_POS, 0, k, v, indptr, indices, kv_len,
                                 sinks, B, Hq, Hkv, 64, 16, max_L, 0.125, out, sa.F32, lse, ws,
                                 ws_bytes)

    def load(t):
        qkv.view(torch.int16).copy_(torch.from_numpy(W.to_bf16_bits(
            rng.standard_normal((B, H, 64), dtype=np.float32)).view(np.int16)).cuda())
        kv_len.copy_(torch.from_numpy((L0 + t).astype(np.int32)).cuda())

    load(0)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    torch.cuda.synchronize()
    for t in range(1, 6):
        load(t)
        # the eager pair on copies of this step's inputs
        k2, v2 = k.clone(), v.clone()
        q2 = torch.zeros((B, Hq, 64), dtype=torch.bfloat16, device="cuda")
        out2 = torch.empty_like(out)
        lse2 = torch.empty_like(lse)
        ws2 = torch.zeros(ws2_bytes, dtype=torch.uint8, device="cuda")
        qo = torch.arange(B + 1, dtype=torch.int32, device="cuda")
        sa.sink_attn_qkv_rope_append(qkv, bias, table, MAX_POS, qo, kv_len, indptr, indices, B,
                                     Hq, Hkv, 64, 16, B, 0, q2, k2, v2)
        sa.sink_attn_decode_balanced(q2, k2, v2, indptr, indices, kv_len, sinks, B, Hq, Hkv, 64,
                                     16, max_L, 0, 0.125, out2, sa.F32, lse2, ws2, ws2_bytes)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[decode step graph] replay {t}", flush=True)
        assert torch.equal(out.view(torch.int32), out2.view(torch.int32)), f"replay {t}: out"
        assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)), f"replay {t}: lse"
        assert torch.equal(k.view(torch.int16), k2.view(torch.int16)), f"replay {t}: k cache"
        assert torch.equal(v.view(torch.int16), v2.view(torch.int16)), f"replay {t}: v cache"
