"""HIP-graph capture of the decode, prefill, tree-verification and append
entry points, and of a whole decode step (append, then attend).

The library reads no device data on the host, allocates nothing and issues
no memset, so a call can be captured once, at fixed host scalars (batch,
head counts, max_kv_len / max_qlen), and replayed over new contents of the
same buffers: new lengths, page tables, queries and caches.  The load-
balanced decode derives its page ranges from page_indptr on the device, so
a replay over a different total page count re-plans itself.

Each replay is checked against the oracle, with eager work and host
synchronisation between replays.
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


def _bf16_into(dst: torch.Tensor, a: np.ndarray):
    src = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    dst.view(-1)[: src.numel()].copy_(src.reshape(-1).to(dst.device))


def _i32_into(dst: torch.Tensor, a: np.ndarray):
    src = torch.from_numpy(np.ascontiguousarray(a, np.int32))
    dst[: src.numel()].copy_(src.to(dst.device))


@pytest.mark.parametrize("num_splits", [0, 4])
def test_decode_graph_replays_over_new_batches(num_splits):
    from gqa_attention_sinks_attn_amd import (F32, sink_attn_decode,
                                              sink_attn_decode_workspace_size)
    B, Hq, Hkv, max_L = 24, 64, 8, 2000
    max_pages = B * ((max_L + 15) // 16)
    dev = "cuda"
    q = torch.zeros((B, Hq, 64), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((max_pages, Hkv, 16, 64), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    indptr = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    indices = torch.zeros(max_pages, dtype=torch.int32, device=dev)
    kv_len = torch.ones(B, dtype=torch.int32, device=dev)
    sinks = torch.zeros(Hq, dtype=torch.float32, device=dev)
    out = torch.empty((B, Hq, 64), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws_bytes = sink_attn_decode_workspace_size(B, Hq, Hkv, 64, max_L, num_splits)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def load(b):
        _bf16_into(q, b.q)
        _bf16_into(k, b.k)
        _bf16_into(v, b.v)
        _i32_into(indptr, b.kv_indptr)
        _i32_into(indices, b.page_indices)
        _i32_into(kv_len, b.kv_len)
        sinks.copy_(torch.from_numpy(np.asarray(b.sinks, np.float32)).to(dev))

    def call():
        sink_attn_decode(q, k, v, indptr, indices, kv_len, sinks, B, Hq, Hkv, 64, 16, max_L,
                         num_splits, 0.125, out, F32, lse, ws, ws_bytes)

    rng = np.random.default_rng(11)
    batches = []
    for t in range(4):
        L = rng.integers(1, max_L + 1, size=B)
        if t == 2:
            L[:] = rng.integers(1, 40, size=B)     # far fewer pages than at capture
        if t == 3:
            L[:] = max_L                           # the maximum
        batches.append(W.make_batch(200 + t, kind="decode", qlens=[1] * B, kv_lens=L, hq=Hq,
                                    hkv=Hkv, paged=True, sinks="normal"))
    load(batches[0])
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call()                                     # warm up on the capture stream
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    torch.cuda.synchronize()
    for t, b in enumerate(batches + batches[:1]):
        load(b)
        out.fill_(float("nan"))                   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref, rl = oracle.attend(b)
        print(f"[graph decode] S={num_splits} replay {t}: {int(np.sum(b.kv_len))} keys", flush=True)
        check(f"graph decode S={num_splits} replay {t}", out.cpu().numpy(), ref,
              lse.cpu().numpy().astype(np.float64), rl, bf16_out=False)


def test_prefill_graph_replays_over_new_batches():
    from gqa_attention_sinks_attn_amd import F32, sink_attn_prefill
    B, Hq, Hkv, max_qlen, max_L = 4, 16, 2, 100, 600
    max_pages = B * ((max_L + 15) // 16)
    total_q_max = B * max_qlen
    dev = "cuda"
    q = torch.zeros((total_q_max, Hq, 64), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((max_pages, Hkv, 16, 64), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    qo = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    indptr = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    indices = torch.zeros(max_pages, dtype=torch.int32, device=dev)
    kv_len = torch.ones(B, dtype=torch.int32, device=dev)
    sinks = torch.zeros(Hq, dtype=torch.float32, device=dev)
    out = torch.zeros((total_q_max, Hq, 64), dtype=torch.float32, device=dev)
    lse = torch.zeros((total_q_max, Hq), dtype=torch.float32, device=dev)

    def load(b):
        _bf16_into(q, b.q)
        _bf16_into(k, b.k)
        _bf16_into(v, b.v)
        _i32_into(qo, b.qo_indptr)
        _i32_into(indptr, b.kv_indptr)
        _i32_into(indices, b.page_indices)
        _i32_into(kv_len, b.kv_len)
        sinks.copy_(torch.from_numpy(np.asarray(b.sinks, np.float32)).to(dev))

    def call():
        sink_attn_prefill(q, qo, k, v, indptr, indices, kv_len, sinks, B, Hq, Hkv, 64, 16,
                          total_q_max, max_qlen, max_L, 0.125, True, out, F32, lse)

    rng = np.random.default_rng(12)
    batches = []
    for t in range(3):
        ql = rng.integers(1, max_qlen + 1, size=B)
        L = np.minimum(max_L, ql + rng.integers(0, 300, size=B))
        batches.append(W.make_batch(300 + t, kind="prefill", qlens=ql, kv_lens=L, hq=Hq, hkv=Hkv,
                                    paged=True, sinks="normal"))
    load(batches[0])
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    torch.cuda.synchronize()
    for t, b in enumerate(batches + batches[:1]):
        load(b)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        n = int(b.qo_indptr[-1])
        ref, rl = oracle.attend(b)
        print(f"[graph prefill] replay {t}: {n} query rows", flush=True)
        check(f"graph prefill replay {t}", out[:n].cpu().numpy(), ref,
              lse[:n].cpu().numpy().astype(np.float64), rl, bf16_out=False)


def test_decode_step_graph_append_then_attend():
    """One decode step as a graph: bias + YaRN rotary + paged append of each
    request's new token, then the balanced decode over the grown cache.
    Captured once at fixed maxima; replayed over steps whose caches grow by
    one token, with new projections and a new batch of lengths."""
    from gqa_attention_sinks_attn_amd import (F32, sink_attn_decode,
                                              sink_attn_decode_workspace_size,
                                              sink_attn_qkv_rope_append, sink_attn_rope_table)
    from oracle import rope
    B, Hq, Hkv, max_L, max_pos = 16, 64, 8, 1500, 4096
    H = Hq + 2 * Hkv
    dev = "cuda"
    max_pages = B * ((max_L + 15) // 16)
    qkv = torch.zeros((B, H, 64), dtype=torch.bfloat16, device=dev)
    bias = torch.zeros((H * 64,), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((B, Hq, 64), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((max_pages, Hkv, 16, 64), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    qo = torch.arange(B + 1, dtype=torch.int32, device=dev)
    indptr = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    indices = torch.zeros(max_pages, dtype=torch.int32, device=dev)
    kv_len = torch.ones(B, dtype=torch.int32, device=dev)
    sinks = torch.zeros(Hq, dtype=torch.float32, device=dev)
    out = torch.empty((B, Hq, 64), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    table = torch.empty((max_pos, 64), dtype=torch.float32, device=dev)
    sink_attn_rope_table(table, max_pos, 64, 150000.0, 32.0, 4096, 32.0, 1.0, 0.0)
    ws_bytes = sink_attn_decode_workspace_size(B, Hq, Hkv, 64, max_L, 0)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def call():
        sink_attn_qkv_rope_append(qkv, bias, table, max_pos, qo, kv_len, indptr, indices, B, Hq,
                                  Hkv, 64, 16, B, 0, q, k, v)
        sink_attn_decode(q, k, v, indptr, indices, kv_len, sinks, B, Hq, Hkv, 64, 16, max_L, 0,
                         0.125, out, F32, lse, ws, ws_bytes)

    rng = np.random.default_rng(31)
    L0 = rng.integers(1, max_L - 8, size=B)
    L0[0] = 1
    tab = rope.rope_table(max_pos, 64, 150000.0, 32.0, 4096, 32.0, 1.0)
    # one page pool for all steps; each step's cache = the previous one + 1 token
    ab = W.make_append_batch(rng, qlens=[1] * B, kv_lens=L0 + 8, hq=Hq, hkv=Hkv, spare_pages=0)
    _bf16_into(k, ab.k_pages)
    _bf16_into(v, ab.v_pages)
    _i32_into(indptr, ab.page_indptr)
    _i32_into(indices, ab.page_indices)
    _bf16_into(bias, ab.bias)
    sinks.copy_(torch.from_numpy(rng.standard_normal(Hq).astype(np.float32)).to(dev))

    def load_step(t):
        _bf16_into(qkv, W.to_bf16_bits(rng.standard_normal((B, H, 64), dtype=np.float32)))
        _i32_into(kv_len, L0 + t)

    load_step(0)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    torch.cuda.synchronize()
    for t in range(1, 8):
        load_step(t)
        before_k = k.view(torch.int16).cpu().numpy().view(np.uint16)
        before_v = v.view(torch.int16).cpu().numpy().view(np.uint16)
        qkv_bits = qkv.view(torch.int16).cpu().numpy().view(np.uint16)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # the append, against the rope oracle on this step's inputs
        rq, rk, rv = rope.qkv_rope_append(qkv_bits, ab.bias, tab, np.arange(B + 1), L0 + t,
                                          ab.page_indptr, ab.page_indices, before_k, before_v,
                                          Hq, Hkv, False)
        kb = k.view(torch.int16).cpu().numpy().view(np.uint16)
        vb = v.view(torch.int16).cpu().numpy().view(np.uint16)
        qb = q.view(torch.int16).cpu().numpy().view(np.uint16)
        got_q = W.bf16_bits_to_f32(qb).astype(np.float64)
        assert np.all(np.abs(got_q - rq) <= 2.0 ** -8 * np.abs(rq) + 1e-5), f"step {t}: q"
        got_k = W.bf16_bits_to_f32(kb).astype(np.float64)
        assert np.all(np.abs(got_k - rk) <= 2.0 ** -8 * np.abs(rk) + 1e-5), f"step {t}: k cache"
        # the attention, against the sink-attention oracle on the cache as appended
        b = W.Batch(kind="decode", q=qb, qo_indptr=np.arange(B + 1, dtype=np.int32), k=kb, v=vb,
                    kv_indptr=ab.page_indptr, page_indices=ab.page_indices,
                    kv_len=(L0 + t).astype(np.int32),
                    sinks=sinks.cpu().numpy(), num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=64,
                    page_size=16, sm_scale=0.125, causal=True)
        ref, rl = oracle.attend(b)
        print(f"[graph step] replay {t}: {int(np.sum(L0 + t))} keys", flush=True)
        check(f"graph decode step {t}", out.cpu().numpy(), ref,
              lse.cpu().numpy().astype(np.float64), rl, bf16_out=False)


def test_verify_tree_graph_replays_over_new_drafts():
    """Tree verification captured once (fixed maxima and split plan) and
    replayed over new lengths, draft trees, queries and caches."""
    from gqa_attention_sinks_attn_amd import (F32, sink_attn_verify_tree,
                                              sink_attn_verify_workspace_size)
    B, Hq, Hkv, max_qlen, max_L = 8, 64, 8, 12, 900
    max_pages = B * ((max_L + 15) // 16)
    dev = "cuda"
    q = torch.zeros((B * max_qlen, Hq, 64), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((max_pages, Hkv, 16, 64), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    qo = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    mask = torch.zeros(B * max_qlen, dtype=torch.int64, device=dev)
    indptr = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    indices = torch.zeros(max_pages, dtype=torch.int32, device=dev)
    kv_len = torch.ones(B, dtype=torch.int32, device=dev)
    sinks = torch.zeros(Hq, dtype=torch.float32, device=dev)
    out = torch.zeros((B * max_qlen, Hq, 64), dtype=torch.float32, device=dev)
    lse = torch.zeros((B * max_qlen, Hq), dtype=torch.float32, device=dev)
    S = 3
    ws_bytes = sink_attn_verify_workspace_size(B, Hq, Hkv, 64, B * max_qlen, max_qlen, max_L, S)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def call():
        sink_attn_verify_tree(q, qo, mask, k, v, indptr, indices, kv_len, sinks, B, Hq, Hkv, 64,
                              16, B * max_qlen, max_qlen, max_L, S, 0.125, out, F32, lse, ws,
                              ws_bytes)

    rng = np.random.default_rng(41)
    batches = []
    for t in range(3):
        ql = rng.integers(1, max_qlen + 1, size=B)
        L = np.minimum(max_L, ql + rng.integers(0, 800, size=B))
        b = W.make_batch(500 + t, kind="prefill", qlens=ql, kv_lens=L, hq=Hq, hkv=Hkv, paged=True,
                         sinks="normal")
        b.draft_mask = np.concatenate([W.tree_mask(W.draft_tree(rng, int(n))) for n in ql])
        batches.append(b)

    def load(b):
        _bf16_into(q, b.q)
        _bf16_into(k, b.k)
        _bf16_into(v, b.v)
        _i32_into(qo, b.qo_indptr)
        _i32_into(indptr, b.kv_indptr)
        _i32_into(indices, b.page_indices)
        _i32_into(kv_len, b.kv_len)
        mask[: len(b.draft_mask)].copy_(
            torch.from_numpy(b.draft_mask.astype(np.uint64).view(np.int64)).to(dev))
        sinks.copy_(torch.from_numpy(np.asarray(b.sinks, np.float32)).to(dev))

    load(batches[0])
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    torch.cuda.synchronize()
    for t, b in enumerate(batches + batches[:1]):
        load(b)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        n = int(b.qo_indptr[-1])
        ref, rl = oracle.attend(b)
        print(f"[graph verify tree] replay {t}: {n} drafted tokens", flush=True)
        check(f"graph verify tree replay {t}", out[:n].cpu().numpy(), ref,
              lse[:n].cpu().numpy().astype(np.float64), rl, bf16_out=False)
