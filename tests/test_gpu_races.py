"""Repeatability under perturbed timing: a race check for the kernels' LDS
pipelines and cross-wave hand-offs.

Every kernel family is run again and again on the same inputs while other
work competes for the GPU from a second stream (a 256 MiB device copy that
loads HBM, an fp32 matrix product that occupies compute units, or nothing),
so that its waves start, stall and finish in a different order each time.
The kernels' arithmetic does not depend on timing, so every run must give
the first run's output and LSE bit for bit; a missing barrier or wait (a
tile read before it has landed, a buffer overwritten while still read, a
partial read before it is written) shows up as a difference between runs.
The first run is also checked against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from tests.test_gpu_parity import check  # noqa: E402

RUNS = 12


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_attn_amd  # noqa: F401  (fails loudly if not built)
    yield


@pytest.fixture(scope="module")
def noise():
    """Work for a second stream (default priority, like every stream here)."""
    s = torch.cuda.Stream()
    x = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    a = torch.randn(3072, 3072, dtype=torch.float32, device="cuda")
    b = torch.randn(3072, 3072, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def launch(i):
        kind = i % 3
        if kind == 2:
            return
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            if kind == 0:
                y.copy_(x)
            else:
                torch.mm(a, b)
    yield launch
    torch.cuda.synchronize()
    del x, y, a, b


def repeat(name, run, noise):
    """run() enqueues the call and returns (out, lse) tensors; every run must
    equal the first bit for bit."""
    first = None
    for i in range(RUNS):
        noise(i)
        out, lse = run()
        torch.cuda.synchronize()
        o = out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32).clone()
        l_ = lse.view(torch.int32).clone()
        if first is None:
            first = (o, l_, out.float().cpu().numpy().astype(np.float64),
                     lse.cpu().numpy().astype(np.float64))
            continue
        diff = int((o != first[0]).sum())
        assert diff == 0, f"{name}: run {i} differs from run 0 at {diff} output values"
        assert torch.equal(l_, first[1]), f"{name}: run {i} lse differs from run 0"
    print(f"[race {name}] {RUNS} runs bit-identical", flush=True)
    return first[2], first[3]


def device_call(b, plan="chunked", num_ranges=0):
    from gqa_attention_sinks_attn_amd import device
    db = device.to_device(b, plan=plan, num_ranges=num_ranges)

    def run():
        if db.workspace is not None:
            db.workspace.fill_(0xFF)     # NaN partials before every run
        db.out.fill_(float("nan"))
        db.lse.fill_(float("nan"))
        device.run(db)
        return db.out, db.lse
    return run


CASES = {
    "prefill contiguous causal": lambda: W.make_batch(
        801, kind="prefill", qlens=[700, 333, 1], kv_lens=[700, 333, 1], hq=16, hkv=2,
        sinks="normal"),
    "prefill paged chunked prefix": lambda: W.make_batch(
        802, kind="prefill", qlens=[300, 77, 512], kv_lens=[1800, 77, 2600], hq=64, hkv=8,
        paged=True, sinks="normal"),
    "prefill group 16 non-causal": lambda: W.make_batch(
        803, kind="prefill", qlens=[90, 200], kv_lens=[500, 260], hq=32, hkv=2, paged=True,
        causal=False, sinks="normal"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_runs_are_bit_identical(case, noise):
    b = CASES[case]()
    out, lse = repeat(case, device_call(b), noise)
    ref, rl = oracle.attend(b)
    check(f"race {case}", out, ref, lse, rl, bf16_out=False)


@pytest.mark.parametrize("plan,n", [("chunked", 1), ("chunked", 7), ("balanced", 0),
                                    ("balanced", 40)])
def test_decode_runs_are_bit_identical(plan, n, noise):
    rng = np.random.default_rng(810)
    L = rng.integers(1, 3000, size=40)
    b = W.make_batch(rng, kind="decode", qlens=[1] * 40, kv_lens=L, hq=64, hkv=8, paged=True,
                     sinks="normal", num_splits=n if plan == "chunked" else 0)
    out, lse = repeat(f"decode {plan} {n}", device_call(b, plan, n if plan == "balanced" else 0),
                      noise)
    ref, rl = oracle.attend(b)
    check(f"race decode {plan} {n}", out, ref, lse, rl, bf16_out=False)


@pytest.mark.parametrize("qlen,tree,splits", [(4, False, 0), (4, True, 3), (16, False, 0),
                                              (32, True, 0), (40, True, 2)])
def test_verify_runs_are_bit_identical(qlen, tree, splits, noise):
    rng = np.random.default_rng(820 + qlen)
    L = rng.integers(qlen, 3000, size=24, endpoint=True)
    b = W.make_batch(rng, kind="prefill", qlens=[qlen] * 24, kv_lens=L, hq=64, hkv=8,
                     paged=True, sinks="normal", num_splits=splits)
    if tree:
        b.draft_mask = np.concatenate([W.tree_mask(W.draft_tree(rng, qlen)) for _ in range(24)])
    out, lse = repeat(f"verify qlen={qlen} tree={tree} S={splits}", device_call(b, "verify"),
                      noise)
    ref, rl = oracle.attend(b)
    check(f"race verify qlen={qlen} tree={tree}", out, ref, lse, rl, bf16_out=False)


def _dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_fused_steps_are_bit_identical(kind, noise):
    """The fused steps write the cache and read it back (in the decode step,
    inside one wave; in the prefill step, in the next kernel): repeated on
    the same inputs, output, LSE and cache are the first run's."""
    import gqa_attention_sinks_attn_amd as sa
    rng = np.random.default_rng(830)
    if kind == "decode":
        qlens = [1] * 48
        kvl = rng.integers(1, 2500, size=48)
    else:
        qlens = [200, 37, 511]
        kvl = np.add(qlens, [0, 900, 1500])
    ab = W.make_append_batch(rng, qlens=qlens, kv_lens=kvl, hq=64, hkv=8, spare_pages=2)
    B, T = len(kvl), int(np.sum(qlens))
    max_L, max_q = int(np.max(kvl)), int(np.max(qlens))
    table = torch.empty((4096, 64), dtype=torch.float32, device="cuda")
    sa.sink_attn_rope_table(table, 4096, 64, 150000.0, 32.0, 4096, 32.0, 1.0, 0.0)
    qkv, bias = _dev_bf16(ab.qkv), _dev_bf16(ab.bias)
    qo, kv_len = _dev_i32(ab.qo_indptr), _dev_i32(ab.kv_len)
    indptr, indices = _dev_i32(ab.page_indptr), _dev_i32(ab.page_indices)
    sinks = torch.from_numpy(rng.standard_normal(64).astype(np.float32)).cuda()
    k0, v0 = _dev_bf16(ab.k_pages), _dev_bf16(ab.v_pages)
    k, v = k0.clone(), v0.clone()
    out = torch.empty((T, 64, 64), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, 64), dtype=torch.float32, device="cuda")
    ws_bytes = sa.sink_attn_decode_step_workspace_size(B, 64, 8, 64, max_L) if kind == "decode" else 0
    ws = torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device="cuda")
    caches = []

    def run():
        k.copy_(k0)
        v.copy_(v0)
        ws.fill_(0xFF)
        out.fill_(float("nan"))
        if kind == "decode":
            sa.sink_attn_decode_step(qkv, bias, table, 4096, 0, k, v, indptr, indices, kv_len,
                                     sinks, B, 64, 8, 64, 16, max_L, 0.125, out, sa.F32, lse, ws,
                                     ws_bytes)
        else:
            sa.sink_attn_prefill_step(qkv, bias, table, 4096, 0, qo, k, v, indptr, indices,
                                      kv_len, sinks, B, 64, 8, 64, 16, T, max_q, max_L, 0.125, 1,
                                      out, sa.F32, lse)
        caches.append((k.view(torch.int16).clone(), v.view(torch.int16).clone()))
        return out, lse
    repeat(f"{kind} step", run, noise)
    for i, (kc, vc) in enumerate(caches[1:], 1):
        assert torch.equal(kc, caches[0][0]) and torch.equal(vc, caches[0][1]), \
            f"{kind} step: cache of run {i} differs from run 0"
