"""Parity at the exact batches `bench.py --extra` times, in the launch
configuration it times them: the verification batches (automatic plan,
which puts the 16- and 32-token drafts on the tile kernel) against the attention
oracle in full, and the bias + rotary + append steps against the rope
oracle (in full for the decode step, on sampled tokens for the 32,768-token
prefill step).  Bars as in test_gpu_parity.py and test_gpu_rope.py.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from oracle import rope  # noqa: E402
import workloads as W  # noqa: E402
from tests.test_gpu_parity import check  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_attn_amd  # noqa: F401  (fails loudly if not built)
    yield


@pytest.mark.parametrize("name", W.VERIFY_WORKLOADS)
def test_verify_bench_batches(name):
    from gqa_attention_sinks_attn_amd import device
    b = W.verify_workload(name)
    db = device.to_device(b, plan="verify")
    device.run(db)
    torch.cuda.synchronize()
    out = db.out.float().cpu().numpy().astype(np.float64)
    lse = db.lse.cpu().numpy().astype(np.float64)
    ref, rl = oracle.attend(b)
    check(name, out, ref, lse, rl, bf16_out=False)


@pytest.mark.parametrize("name", W.APPEND_WORKLOADS)
def test_append_bench_batches(name):
    from gqa_attention_sinks_attn_amd import sink_attn_qkv_rope_append, sink_attn_rope_table
    ab = W.append_workload(name)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa: E731
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731
    table = torch.empty((131072, 64), dtype=torch.float32, device="cuda")
    sink_attn_rope_table(table, 131072, 64, 150000.0, 32.0, 4096, 32.0, 1.0, 0.0)
    kp, vp = dev(ab.k_pages), dev(ab.v_pages)
    q_out = torch.empty((ab.total_q, 64, 64), dtype=torch.int16, device="cuda")
    sink_attn_qkv_rope_append(dev(ab.qkv), dev(ab.bias), table, 131072, i32(ab.qo_indptr),
                              i32(ab.kv_len), i32(ab.page_indptr), i32(ab.page_indices),
                              ab.batch, 64, 8, 64, 16, ab.total_q, 0, q_out, kp, vp)
    torch.cuda.synchronize()
    q = q_out.cpu().numpy().view(np.uint16)
    kb = kp.cpu().numpy().view(np.uint16)
    vb = vp.cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(3)
    if ab.total_q > 256:   # first and last token of every request, and random ones
        rows = sorted(set(ab.qo_indptr[:-1].tolist()) | set((ab.qo_indptr[1:] - 1).tolist())
                      | set(rng.integers(0, ab.total_q, size=48).tolist()))
    else:
        rows = list(range(ab.total_q))
    need = set()
    slots = []
    for r in rows:
        b = int(np.searchsorted(ab.qo_indptr, r, side="right") - 1)
        p = int(ab.kv_len[b]) - int(ab.qo_indptr[b + 1] - ab.qo_indptr[b]) + (r - int(ab.qo_indptr[b]))
        need.add(p)
        slots.append((int(ab.page_indices[ab.page_indptr[b] + p // 16]), p % 16))
    f = rope.yarn_frequencies(64, 150000.0, 32.0, 4096, 32.0, 1.0)
    m = rope.yarn_temperature(32.0)
    tab = np.zeros((int(ab.kv_len.max()), 64))
    for p in need:
        tab[p] = np.concatenate([m * np.cos(p * f), m * np.sin(p * f)])
    rq, rk, rv = rope.qkv_rope_append(ab.qkv, ab.bias, tab, ab.qo_indptr, ab.kv_len,
                                      ab.page_indptr, ab.page_indices, ab.k_pages, ab.v_pages,
                                      64, 8, False, rows=rows)

    def close(tag, got_bits, ref):
        got = W.bf16_bits_to_f32(got_bits).astype(np.float64)
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * np.abs(ref) + 1e-5
        print(f"[{name} {tag}] {len(rows)} tokens, max err {err.max():.3e}", flush=True)
        assert np.all(err <= bound), f"{name} {tag}: worst excess {(err - bound).max()}"

    close("q", q[rows], rq[rows])
    pg = np.array([s[0] for s in slots])
    sl = np.array([s[1] for s in slots])
    close("k", kb[pg, :, sl], rk[pg, :, sl])
    close("v", vb[pg, :, sl], rv[pg, :, sl])
