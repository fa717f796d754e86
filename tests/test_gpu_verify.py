"""Multi-token verification shapes (speculative / multi-token-prediction
verify): every request appends qlen = 2..8 drafted tokens to its paged cache
and attends causally within them and to its whole prefix -- the same
operation as a chunked prefill at a small qlen (bottom-right alignment:
drafted token t sits at kv_len - qlen + t).  Through both sink_attn_prefill
and the dedicated sink_attn_verify (split-KV plans S = 0 (automatic), 1, 3,
64), against the oracle, at the parity bar of the other GPU tests.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from tests.test_gpu_parity import check  # noqa: E402


def run(b, entry, num_splits=0):
    from gqa_attention_sinks_attn_amd import device
    b.num_splits = num_splits
    db = device.to_device(b, plan="verify" if entry == "verify" else "chunked")
    if db.workspace is not None:
        db.workspace.fill_(0xFF)      # NaN partials: nothing may read unwritten slots
    device.run(db)
    torch.cuda.synchronize()
    return (db.out.float().cpu().numpy().astype(np.float64),
            db.lse.cpu().numpy().astype(np.float64), db.out.dtype == torch.bfloat16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_attn_amd  # noqa: F401  (fails loudly if not built)
    yield


@pytest.mark.parametrize("entry", ["prefill", "verify"])
@pytest.mark.parametrize("qlen", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("hq,hkv", [(64, 8), (32, 8), (16, 16)])
def test_verify_shapes(qlen, hq, hkv, entry):
    if entry == "verify" and qlen * hq // hkv > 64:
        pytest.skip("more than 64 (token, head) rows per KV head: sink_attn_prefill's shape")
    rng = np.random.default_rng(400 + qlen + hq)
    B = 24
    L = rng.integers(qlen, 3000, size=B, endpoint=True)
    L[0] = qlen                    # the whole request is drafted tokens
    L[1] = qlen + 15               # a page boundary inside the draft
    b = W.make_batch(rng, kind="prefill", qlens=[qlen] * B, kv_lens=L, hq=hq, hkv=hkv,
                     paged=True, sinks="normal")
    out, lse, bf16 = run(b, entry)
    ref, rl = oracle.attend(b)
    check(f"{entry} qlen={qlen} G={hq // hkv}", out, ref, lse, rl, bf16_out=bf16)


@pytest.mark.parametrize("entry,splits", [("prefill", 0), ("verify", 0), ("verify", 1),
                                          ("verify", 3), ("verify", 64)])
def test_verify_mixed_draft_lengths_bf16(entry, splits):
    rng = np.random.default_rng(470)
    B = 40
    ql = rng.integers(1, 8, size=B, endpoint=True)
    L = ql + rng.integers(0, 5000, size=B)
    b = W.make_batch(rng, kind="prefill", qlens=ql, kv_lens=L, hq=64, hkv=8, paged=True,
                     sinks="normal", out_dtype="bf16")
    out, lse, bf16 = run(b, entry, splits)
    ref, rl = oracle.attend(b)
    check(f"{entry} S={splits} mixed qlen bf16", out, ref, lse, rl, bf16_out=bf16)


def test_verify_empty_requests_and_sinks():
    """Requests without rows between others, +inf / none sinks, one-key caches."""
    s = np.random.default_rng(3).standard_normal(16).astype(np.float32)
    s[5] = np.inf
    b = W.make_batch(481, kind="prefill", qlens=[3, 0, 1, 0, 4, 2], kv_lens=[3, 50, 1, 9, 700, 16],
                     hq=16, hkv=4, paged=True, sinks=s)
    for entry in ("prefill", "verify"):
        out, lse, bf16 = run(b, entry, 2)
        ref, rl = oracle.attend(b)
        assert np.all(out[:, 5] == 0) and np.all(lse[:, 5] == np.inf)
        keep = [h for h in range(16) if h != 5]
        check(f"{entry} empty requests", out[:, keep], ref[:, keep], lse[:, keep], rl[:, keep],
              bf16_out=bf16)
