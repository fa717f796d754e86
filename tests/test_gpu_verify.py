"""Multi-token verification shapes (speculative / multi-token-prediction
verify): every request appends qlen = 2..8 drafted tokens to its paged cache
and attends causally within them and to its whole prefix -- the same
operation as a chunked prefill at a small qlen (bottom-right alignment:
drafted token t sits at kv_len - qlen + t).  Through sink_attn_prefill, against
the oracle, at the parity bar of the other GPU tests.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from tests.test_gpu_parity import check, gpu_run  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_attn_amd  # noqa: F401  (fails loudly if not built)
    yield


@pytest.mark.parametrize("qlen", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("hq,hkv", [(64, 8), (32, 8), (16, 16)])
def test_verify_shapes(qlen, hq, hkv):
    rng = np.random.default_rng(400 + qlen + hq)
    B = 24
    L = rng.integers(qlen, 3000, size=B, endpoint=True)
    L[0] = qlen                    # the whole request is drafted tokens
    L[1] = qlen + 15               # a page boundary inside the draft
    b = W.make_batch(rng, kind="prefill", qlens=[qlen] * B, kv_lens=L, hq=hq, hkv=hkv,
                     paged=True, sinks="normal")
    out, lse = gpu_run(b)
    ref, rl = oracle.attend(b)
    check(f"verify qlen={qlen} G={hq // hkv}", out, ref, lse, rl)


def test_verify_mixed_draft_lengths_bf16():
    rng = np.random.default_rng(470)
    B = 40
    ql = rng.integers(1, 8, size=B, endpoint=True)
    L = ql + rng.integers(0, 5000, size=B)
    b = W.make_batch(rng, kind="prefill", qlens=ql, kv_lens=L, hq=64, hkv=8, paged=True,
                     sinks="normal", out_dtype="bf16")
    out, lse = gpu_run(b)
    ref, rl = oracle.attend(b)
    check("verify mixed qlen bf16", out, ref, lse, rl)
