"""sink_attn_decode_noalloc: the decode with its workspace taken from the
library's static device scratch array instead of a caller's buffer, called
through the C ABI.

Checked against sink_attn_decode with a caller workspace (bitwise: the same
kernels run on the same inputs) and against the oracle at the parity bar, on
two calls in a row whose second batch is smaller than the first (the array
keeps the first call's contents), on an explicit split count, and on a batch
short enough to need no workspace.  Sizes beyond the array are rejected on
the host (tests/test_abi.py).  This module is collected last, so that its
use of the array also follows every other test's launches.
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


def _both(b, num_splits):
    """Batch b through sink_attn_decode (caller workspace), then through
    sink_attn_decode_noalloc into fresh NaN-filled outputs."""
    import gqa_attention_sinks_attn_amd as sa
    from gqa_attention_sinks_attn_amd import device
    b.num_splits = num_splits
    db = device.to_device(b, plan="chunked")
    device.run(db)
    out = torch.full_like(db.out, float("nan"))
    lse = torch.full_like(db.lse, float("nan"))
    sa.sink_attn_decode_noalloc(db.q, db.k, db.v, db.kv_indptr, db.page_indices, db.kv_len,
                                db.sinks, db.batch, db.num_qo_heads, db.num_kv_heads,
                                db.head_dim, db.page_size, db.max_kv_len, num_splits,
                                db.sm_scale, out, out.dtype, lse)
    torch.cuda.synchronize()
    return db, out, lse


@pytest.mark.parametrize("num_splits", [0, 8])
def test_noalloc_matches_workspace_decode_twice(num_splits):
    big = W.config(2)     # 64 requests, L ~ U[1, 4096]: the balanced plan's workspace
    rng = np.random.default_rng(7)
    L = rng.integers(1, 1500, size=9)
    small = W.make_batch(1207, kind="decode", qlens=[1] * L.size, kv_lens=L, hq=64, hkv=8,
                         paged=True, sinks="normal")
    for name, b in (("first, 64 requests", big), ("second, 9 requests", small)):
        db, out, lse = _both(b, num_splits)
        assert torch.equal(out, db.out), name
        assert torch.equal(lse, db.lse), name
        ref, rl = oracle.attend(b)
        check(f"noalloc S={num_splits} {name}", out.float().cpu().numpy(), ref,
              lse.cpu().numpy().astype(np.float64), rl, bf16_out=out.dtype == torch.bfloat16)


def test_noalloc_short_batch_needs_no_workspace():
    b = W.make_batch(1209, kind="decode", qlens=[1] * 5, kv_lens=[1, 7, 16, 200, 256], hq=16,
                     hkv=2, paged=True, sinks="normal")
    db, out, lse = _both(b, 0)
    assert torch.equal(out, db.out) and torch.equal(lse, db.lse)
