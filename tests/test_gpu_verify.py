"""Multi-token verification shapes (speculative / multi-token-prediction
verify): every request appends qlen = 2..8 drafted tokens to its paged cache
and attends causally within them and to its whole prefix -- the same
operation as a chunked prefill at a small qlen (bottom-right alignment:
drafted token t sits at kv_len - qlen + t).  Through both sink_attn_prefill
and the dedicated sink_attn_verify (split-KV plans S = 0 (automatic), 1, 3,
64), against the oracle, at the parity bar of the other GPU tests.  Drafts
of up to 64 (token, head) pairs per KV head run the column-group kernel
(verify.hip); wider ones run the tile kernel (verify_tile.hip): the qlen 16,
33, 40 and 64 cases below, and the dedicated tile tests.

Tree drafts go through sink_attn_verify_tree: random trees in breadth-first
order, one uint64 visibility word per drafted token, against the oracle's
draft-mask reading (prefix always visible, drafted key i visible when bit i
is set).
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
@pytest.mark.parametrize("qlen", [2, 3, 4, 6, 8, 16, 33])
@pytest.mark.parametrize("hq,hkv", [(64, 8), (32, 8), (16, 16)])
def test_verify_shapes(qlen, hq, hkv, entry):
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


def _tree_batch(seed, qlens, kv_lens, hq, hkv, sinks="normal", junk_bits=True, out_dtype="f32"):
    rng = np.random.default_rng(seed)
    b = W.make_batch(rng, kind="prefill", qlens=qlens, kv_lens=kv_lens, hq=hq, hkv=hkv,
                     paged=True, sinks=sinks, out_dtype=out_dtype)
    words = []
    for n in qlens:
        m = W.tree_mask(W.draft_tree(rng, int(n))) if n else np.zeros(0, np.uint64)
        if junk_bits and n < 64:      # bits at or above qlen must be ignored
            noise = rng.integers(0, 1 << 63, size=len(m), dtype=np.int64).astype(np.uint64)
            m = m | (noise & np.uint64(((1 << 64) - 1) ^ ((1 << int(n)) - 1)))
        words.append(m)
    b.draft_mask = np.concatenate(words).astype(np.uint64)
    return b


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("qlen", [1, 4, 8, 16, 40, 64])
@pytest.mark.parametrize("hq,hkv", [(64, 8), (32, 8), (16, 16)])
def test_verify_tree_shapes(qlen, hq, hkv, splits):
    rng = np.random.default_rng(700 + qlen + hq)
    B = 12
    L = rng.integers(qlen, 2500, size=B, endpoint=True)
    L[0] = qlen                        # no prefix: the whole cache is the draft
    L[1] = qlen + 7                    # drafted keys straddle a page boundary
    b = _tree_batch(int(rng.integers(1 << 30)), [qlen] * B, L, hq, hkv)
    out, lse, bf16 = run(b, "verify", splits)
    ref, rl = oracle.attend(b)
    check(f"tree qlen={qlen} G={hq // hkv} S={splits}", out, ref, lse, rl, bf16_out=bf16)


def test_verify_tree_linear_draft_matches_causal_verify():
    """A chain mask selects the causal key set: same arithmetic, same bits."""
    rng = np.random.default_rng(760)
    ql = rng.integers(1, 20, size=16)
    L = ql + rng.integers(0, 3000, size=16)
    b = W.make_batch(rng, kind="prefill", qlens=ql, kv_lens=L, hq=64, hkv=8, paged=True,
                     sinks="normal")
    causal_out, causal_lse, _ = run(b, "verify", 2)
    b.draft_mask = np.concatenate([W.chain_mask(int(n)) for n in ql])
    tree_out, tree_lse, _ = run(b, "verify", 2)
    np.testing.assert_array_equal(tree_out, causal_out)
    np.testing.assert_array_equal(tree_lse, causal_lse)


def test_verify_tree_mixed_sizes_empty_rows_and_sinks():
    """Mixed draft sizes with requests of no rows, a row that sees no key at
    all (no prefix, empty mask word), +inf and no-sink heads, bf16 output."""
    rng = np.random.default_rng(771)
    ql = [5, 0, 1, 23, 0, 64, 2, 9]
    L = [5, 30, 1, 900, 4, 2100, 2, 40]
    s = rng.standard_normal(16).astype(np.float32)
    s[3] = np.inf
    s[7] = -np.inf
    b = _tree_batch(772, ql, L, 16, 4, sinks=s, out_dtype="bf16")
    b.draft_mask[0] = np.uint64(0)     # request 0, token 0: no prefix and no visible draft
    for splits in (0, 1, 4):
        out, lse, bf16 = run(b, "verify", splits)
        ref, rl = oracle.attend(b)
        assert np.all(out[0] == 0)
        assert np.all(out[:, 3] == 0) and np.all(lse[:, 3] == np.inf)
        keep = [h for h in range(16) if h != 3]
        check(f"tree mixed S={splits}", out[:, keep], ref[:, keep], lse[:, keep], rl[:, keep],
              bf16_out=bf16)


@pytest.mark.parametrize("tree", [False, True])
def test_verify_long_context_split_plan(tree):
    """Two requests at the maximum context of the long-decode workload
    (131,072 keys): the automatic plan splits each request into many chunks
    (sink in chunk 0 only) and merges them; drafted keys sit at the very end
    of the cache."""
    rng = np.random.default_rng(790 + int(tree))
    ql = [4, 2]
    b = W.make_batch(rng, kind="prefill", qlens=ql, kv_lens=[131072, 131072 - 5], hq=64, hkv=8,
                     paged=True, sinks="normal")
    if tree:
        b.draft_mask = np.concatenate([W.tree_mask(W.draft_tree(rng, n)) for n in ql])
    from gqa_attention_sinks_attn_amd import sink_attn_verify_num_splits
    S = sink_attn_verify_num_splits(2, 64, 8, 4, 131072, 0)
    assert S > 1
    out, lse, bf16 = run(b, "verify", 0)
    ref, rl = oracle.attend(b)
    check(f"long context tree={tree} S={S}", out, ref, lse, rl, bf16_out=bf16)


@pytest.mark.parametrize("tree", [False, True])
def test_verify_tiles_long_context_split_plan(tree):
    """Wide drafts on the tile kernel (16 and 24 tokens x G = 8: 128 and 192
    (token, head) pairs per KV head, one and two 128-row tiles) on two long
    caches: the automatic plan splits each request into chunks (sink in
    chunk 0 only), the shorter request into fewer, and the finish pass
    merges them; drafted keys sit at the very end of each cache."""
    rng = np.random.default_rng(830 + int(tree))
    ql = [16, 24]
    b = W.make_batch(rng, kind="prefill", qlens=ql, kv_lens=[65536, 20003], hq=64, hkv=8,
                     paged=True, sinks="normal")
    if tree:
        b.draft_mask = np.concatenate([W.tree_mask(W.draft_tree(rng, n)) for n in ql])
    from gqa_attention_sinks_attn_amd import sink_attn_verify_num_splits
    S = sink_attn_verify_num_splits(2, 64, 8, 24, 65536, 0)
    assert S > 1
    out, lse, bf16 = run(b, "verify", 0)
    ref, rl = oracle.attend(b)
    check(f"tiles long context tree={tree} S={S}", out, ref, lse, rl, bf16_out=bf16)


@pytest.mark.parametrize("qlens,tree", [([4, 3, 4], False),            # column kernel
                                         ([16, 24, 9], False),          # tile kernel
                                         ([16, 24, 9], True)])
@pytest.mark.parametrize("splits", [0, 2])
def test_verify_nan_tails_do_not_leak(qlens, tree, splits):
    """NaN bit patterns in the unused slots of each request's last page
    (never read by the definition) must not reach the output: the tile
    kernel's rows past the last key read a key of the request instead, and
    their probabilities are 0; the column kernel masks them."""
    rng = np.random.default_rng(910 + 3 * splits + int(tree) + qlens[0])
    L = [40, 57, 1013]                     # every last page part-used
    b = W.make_batch(rng, kind="prefill", qlens=qlens, kv_lens=L, hq=64, hkv=8, paged=True,
                     sinks="normal")
    if tree:
        b.draft_mask = np.concatenate([W.tree_mask(W.draft_tree(rng, n)) for n in qlens])
    for r, n in enumerate(b.kv_len):
        used = int(n) % 16
        if used:
            last = b.page_indices[b.kv_indptr[r + 1] - 1]
            b.k[last, :, used:, :] = 0x7FC0  # NaN
            b.v[last, :, used:, :] = 0x7FC0
    out, lse, bf16 = run(b, "verify", splits)
    ref, rl = oracle.attend(b)
    check(f"NaN tails qlens={qlens} tree={tree} S={splits}", out, ref, lse, rl, bf16_out=bf16)


@pytest.mark.parametrize("tree", [False, True])
@pytest.mark.parametrize("splits", [1, 2])
def test_verify_tiles_long_chunks(tree, splits):
    """Chunks of more than 64 tiles on the tile kernel (one or two chunks
    per request over caches of up to 20,003 keys): each wave reads its page
    ids 64 tiles at a time, so a chunk's 65th and 129th tiles take a fresh
    batch of ids, and a second chunk starts far from key 0."""
    rng = np.random.default_rng(890 + 2 * splits + int(tree))
    ql = [16, 24, 9]
    b = W.make_batch(rng, kind="prefill", qlens=ql, kv_lens=[9000, 20003, 4100], hq=64, hkv=8,
                     paged=True, sinks="normal")
    if tree:
        b.draft_mask = np.concatenate([W.tree_mask(W.draft_tree(rng, n)) for n in ql])
    out, lse, bf16 = run(b, "verify", splits)
    ref, rl = oracle.attend(b)
    check(f"tiles long chunks tree={tree} S={splits}", out, ref, lse, rl, bf16_out=bf16)


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_verify_tiles_group16_and_extreme_sinks(splits):
    """The tile kernel at G = 16 (64 query / 4 KV heads, 8 tokens = 128 rows)
    with sinks of -1e4 and +10 and a request whose cache is only its draft."""
    rng = np.random.default_rng(850 + splits)
    s = rng.standard_normal(64).astype(np.float32)
    s[[0, 17, 42]] = -1e4
    s[[5, 31, 63]] = 10.0
    ql = [8, 8, 5, 8]
    b = W.make_batch(rng, kind="prefill", qlens=ql, kv_lens=[8, 3000, 777, 1500], hq=64, hkv=4,
                     paged=True, sinks=s, out_dtype="bf16")
    out, lse, bf16 = run(b, "verify", splits)
    ref, rl = oracle.attend(b)
    check(f"tiles G=16 S={splits}", out, ref, lse, rl, bf16_out=bf16)


@pytest.mark.parametrize("tree", [False, True])
@pytest.mark.parametrize("hq,hkv,qlens", [(32, 16, [64, 40, 33]),       # G = 2: 1 row tile
                                          (64, 4, [64, 17, 9]),         # G = 16: up to 8 row tiles
                                          (64, 8, [64, 1, 30, 16])])    # G = 8: 4 row tiles, a 1-token row
@pytest.mark.parametrize("splits", [0, 3])
def test_verify_tiles_row_tiles_and_group_sizes(hq, hkv, qlens, tree, splits):
    """The tile kernel at group sizes 2, 8 and 16 with drafts up to the
    64-token maximum (several 128-row tiles per (request, KV head), the last
    one partly padding), mixed draft lengths in one batch, causal and tree
    masks, one or three chunks."""
    rng = np.random.default_rng(870 + hq + hkv + int(tree) + splits)
    L = [int(n) + int(rng.integers(0, 1500)) for n in qlens]
    if tree:
        b = _tree_batch(int(rng.integers(1 << 30)), qlens, L, hq, hkv)
    else:
        b = W.make_batch(rng, kind="prefill", qlens=qlens, kv_lens=L, hq=hq, hkv=hkv, paged=True,
                         sinks="normal")
    out, lse, bf16 = run(b, "verify", splits)
    ref, rl = oracle.attend(b)
    check(f"tiles G={hq // hkv} tree={tree} S={splits}", out, ref, lse, rl, bf16_out=bf16)


@pytest.mark.parametrize("B,tree,splits", [(256, True, 0), (257, False, 0), (300, True, 3),
                                             (64, False, 2), (200, True, 5)])
def test_verify_tiles_job_orders(B, tree, splits):
    """Both job orders of the tile kernel: longest first (up to 256 requests;
    workgroup i computes the i-th longest (request, KV head, chunk, row tile)
    from the request lengths) and index order (more requests), at the
    boundary and across it, with ragged drafts (some empty), ragged caches
    and several chunks: every row of every request is written once."""
    rng = np.random.default_rng(900 + B + splits)
    ql = rng.integers(0, 25, size=B)
    ql[0] = 17
    L = ql + rng.integers(0, 700, size=B)
    L[1] = ql[1]                  # a cache that is only its draft
    L[2] = ql[2] + 2048           # whole chunks and a long last one
    if tree:
        b = _tree_batch(int(rng.integers(1 << 30)), list(ql), list(L), 64, 8)
    else:
        b = W.make_batch(rng, kind="prefill", qlens=ql, kv_lens=L, hq=64, hkv=8, paged=True,
                         sinks="normal")
    out, lse, bf16 = run(b, "verify", splits)
    ref, rl = oracle.attend(b)
    check(f"tiles job order B={B} tree={tree} S={splits}", out, ref, lse, rl, bf16_out=bf16)


@pytest.mark.parametrize("qlen,tree", [(4, False), (4, True), (40, True), (33, False)])
def test_verify_without_lse_bf16(qlen, tree):
    """lse = NULL and bf16 output, on the column-group kernel (4 tokens) and
    on the tile kernel the plan picks for wide drafts (33, 40)."""
    from gqa_attention_sinks_attn_amd import device
    rng = np.random.default_rng(810 + qlen + int(tree))
    B = 10
    L = rng.integers(qlen, 2000, size=B, endpoint=True)
    b = W.make_batch(rng, kind="prefill", qlens=[qlen] * B, kv_lens=L, hq=64, hkv=8, paged=True,
                     sinks="normal", out_dtype="bf16")
    if tree:
        b.draft_mask = np.concatenate([W.tree_mask(W.draft_tree(rng, qlen)) for _ in range(B)])
    db = device.to_device(b, with_lse=False, plan="verify")
    assert db.lse is None
    device.run(db)
    torch.cuda.synchronize()
    out = db.out.float().cpu().numpy().astype(np.float64)
    ref, _ = oracle.attend(b)
    check(f"no lse qlen={qlen} tree={tree}", out, ref, bf16_out=True)
