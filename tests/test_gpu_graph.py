"""HIP-graph capture of the decode and prefill entry points.

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
