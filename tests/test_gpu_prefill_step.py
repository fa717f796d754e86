"""The fused prefill step (sink_attn_prefill_step): the new tokens' keys and
values appended by a key/value-only append, their queries biased and
rotated inside the attention kernel as it loads them.  It must equal, bit
for bit (output, LSE and the whole cache), the append
(sink_attn_qkv_rope_append) followed by sink_attn_prefill on the same
inputs; and, as that pair, match the rope oracle (queries and cache) and
the attention oracle (output) at the parity bar.
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


@pytest.fixture(scope="module")
def table_np():
    from oracle import rope
    return rope.rope_table(MAX_POS, 64, 150000.0, 32.0, 4096, 32.0, 1.0)


def _dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_both(ab, table, sinks, interleaved, causal=True, out_dtype=torch.float32, bias=True,
             max_pos=MAX_POS, name=""):
    import gqa_attention_sinks_attn_amd as sa
    B, Hq, Hkv = len(ab.kv_len), ab.num_qo_heads, ab.num_kv_heads
    qlens = np.diff(ab.qo_indptr)
    T = int(ab.qo_indptr[-1])
    max_qlen = int(qlens.max()) if B else 0
    max_L = int(np.max(ab.kv_len)) if B else 0
    qkv = _dev_bf16(ab.qkv)
    bias_t = _dev_bf16(ab.bias) if (bias and ab.bias is not None) else None
    qo, kv_len = _dev_i32(ab.qo_indptr), _dev_i32(ab.kv_len)
    indptr, indices = _dev_i32(ab.page_indptr), _dev_i32(ab.page_indices)
    sinks_t = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    res = {}
    for mode in ("pair", "step"):
        k, v = _dev_bf16(ab.k_pages), _dev_bf16(ab.v_pages)
        out = torch.full((T, Hq, 64), float("nan"), dtype=out_dtype, device="cuda")
        lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda")
        q = None
        if mode == "pair":
            q = torch.zeros((T, Hq, 64), dtype=torch.bfloat16, device="cuda")
            sa.sink_attn_qkv_rope_append(qkv, bias_t, table, max_pos, qo, kv_len, indptr, indices,
                                         B, Hq, Hkv, 64, 16, T, interleaved, q, k, v)
            sa.sink_attn_prefill(q, qo, k, v, indptr, indices, kv_len, sinks_t, B, Hq, Hkv, 64, 16,
                                 T, max_qlen, max_L, 0.125, causal, out, out_dtype, lse)
        else:
            sa.sink_attn_prefill_step(qkv, bias_t, table, max_pos, interleaved, qo, k, v, indptr,
                                      indices, kv_len, sinks_t, B, Hq, Hkv, 64, 16, T, max_qlen,
                                      max_L, 0.125, causal, out, out_dtype, lse)
        torch.cuda.synchronize()
        res[mode] = dict(out=out, lse=lse, k=_bits(k), v=_bits(v),
                         q=None if q is None else _bits(q))
    print(f"[prefill step {name}] B={B} T={T} Hq={Hq} Hkv={Hkv} max_L={max_L}", flush=True)
    return res


def assert_bitwise(res, rows=None):
    a, b = res["pair"], res["step"]
    oa, ob, la, lb = a["out"], b["out"], a["lse"], b["lse"]
    if rows is not None:
        oa, ob, la, lb = oa[rows], ob[rows], la[rows], lb[rows]
    dt = torch.int16 if oa.dtype == torch.bfloat16 else torch.int32
    same = oa.view(dt) == ob.view(dt)
    assert bool(same.all()), f"outputs differ at {int((~same).sum())} values"
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), "lse differs"
    assert np.array_equal(a["k"], b["k"]), "k cache differs"
    assert np.array_equal(a["v"], b["v"]), "v cache differs"


def oracle_check(name, ab, res, sinks, table_np, interleaved, causal=True, bias=True):
    from oracle import rope
    B, Hq, Hkv = len(ab.kv_len), ab.num_qo_heads, ab.num_kv_heads
    pair = res["pair"]
    rq, rk, rv = rope.qkv_rope_append(ab.qkv, ab.bias if bias else None, table_np, ab.qo_indptr,
                                      ab.kv_len, ab.page_indptr, ab.page_indices, ab.k_pages,
                                      ab.v_pages, Hq, Hkv, bool(interleaved))
    got_q = W.bf16_bits_to_f32(pair["q"]).astype(np.float64)
    assert np.all(np.abs(got_q - rq) <= 2.0 ** -8 * np.abs(rq) + 1e-5), "q"
    got_k = W.bf16_bits_to_f32(res["step"]["k"]).astype(np.float64)
    got_v = W.bf16_bits_to_f32(res["step"]["v"]).astype(np.float64)
    assert np.all(np.abs(got_k - rk) <= 2.0 ** -8 * np.abs(rk) + 1e-5), "k cache"
    assert np.all(np.abs(got_v - rv) <= 2.0 ** -8 * np.abs(rv) + 1e-5), "v cache"
    b = W.Batch(kind="prefill", q=pair["q"], qo_indptr=np.asarray(ab.qo_indptr, np.int32),
                k=res["step"]["k"], v=res["step"]["v"], kv_indptr=ab.page_indptr,
                page_indices=ab.page_indices, kv_len=np.asarray(ab.kv_len, np.int32),
                sinks=None if sinks is None else np.asarray(sinks, np.float32),
                num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=64, page_size=16, sm_scale=0.125,
                causal=causal)
    ref, rl = oracle.attend(b)
    step = res["step"]
    check(name, step["out"].float().cpu().numpy(), ref,
          step["lse"].cpu().numpy().astype(np.float64), rl,
          bf16_out=step["out"].dtype == torch.bfloat16)


QLENS = [1, 7, 40, 256, 300, 33]
PREFIX = [0, 5, 100, 1000, 300, 4000]


@pytest.mark.parametrize("interleaved", [0, 1])
def test_prefill_step_equals_append_then_prefill(table, table_np, interleaved):
    rng = np.random.default_rng(600 + interleaved)
    ab = W.make_append_batch(rng, qlens=QLENS, kv_lens=np.add(QLENS, PREFIX), hq=64, hkv=8,
                             spare_pages=3)
    sinks = rng.standard_normal(64).astype(np.float32)
    res = run_both(ab, table, sinks, interleaved, name=f"interleaved={interleaved}")
    assert_bitwise(res)
    oracle_check(f"prefill step interleaved={interleaved}", ab, res, sinks, table_np, interleaved)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (16, 4), (64, 8), (64, 4), (128, 8)])
def test_prefill_step_group_sizes(table, hq, hkv):
    rng = np.random.default_rng(610 + hq + hkv)
    ql = rng.integers(1, 200, size=5)
    L = ql + rng.integers(0, 1500, size=5)
    ab = W.make_append_batch(rng, qlens=ql, kv_lens=L, hq=hq, hkv=hkv, spare_pages=2)
    sinks = (2.0 * rng.standard_normal(hq)).astype(np.float32)
    res = run_both(ab, table, sinks, 0, name=f"G={hq // hkv}")
    assert_bitwise(res)


def test_prefill_step_no_bias_no_sinks_bf16_noncausal(table, table_np):
    rng = np.random.default_rng(620)
    ab = W.make_append_batch(rng, qlens=[17, 64, 3], kv_lens=[50, 64, 900], hq=16, hkv=2,
                             bias=False)
    res = run_both(ab, table, None, 1, causal=False, out_dtype=torch.bfloat16, bias=False,
                   name="no bias, non-causal")
    assert_bitwise(res)
    oracle_check("prefill step no bias bf16 non-causal", ab, res, None, table_np, 1,
                 causal=False, bias=False)


def test_prefill_step_positions_past_the_table(table):
    """Tokens whose position has no table row are not appended (as the
    append skips them); every other row equals the pair bit for bit."""
    rng = np.random.default_rng(630)
    ab = W.make_append_batch(rng, qlens=[5, 20, 8], kv_lens=[30, 1010, 500], hq=16, hkv=4,
                             spare_pages=1)
    max_pos = 1000   # request 1's last 10 tokens (positions 1000..1009) are past the table
    res = run_both(ab, table, rng.standard_normal(16).astype(np.float32), 0, max_pos=max_pos,
                   name="past the table")
    qo = ab.qo_indptr
    ok = list(range(qo[0], qo[1])) + list(range(qo[2], qo[3]))
    assert_bitwise(res, rows=ok)
    for p in range(1000, 1010):
        page = ab.page_indices[ab.page_indptr[1] + p // 16]
        assert np.array_equal(res["step"]["k"][page, :, p % 16], ab.k_pages[page, :, p % 16])


def test_prefill_step_verification_shape(table):
    """A verification batch: 64 requests x 4 drafted tokens on long caches."""
    rng = np.random.default_rng(640)
    L = rng.integers(4, 4097, size=64)
    ab = W.make_append_batch(rng, qlens=[4] * 64, kv_lens=L, hq=64, hkv=8, spare_pages=0)
    res = run_both(ab, table, rng.standard_normal(64).astype(np.float32), 0, name="verify 4")
    assert_bitwise(res)
