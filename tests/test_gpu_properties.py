"""Property tests of the HIP path (hypothesis, small random shapes), through
the C ABI like every other GPU test.

Each test draws a small batch -- request count, lengths, group size, page
permutation, sinks, layout and plan -- and checks a property that must hold
for every such batch:
- prefill, decode (split-KV and balanced plans) and tree verification match
  the fp64 oracle at the parity bar of the other GPU tests;
- the result does not depend on where the pages sit in the pool: permuting
  the physical pages (and leaving unreferenced NaN pages in it) gives
  bit-for-bit the same output and LSE;
- the split plans agree with one another (the split-KV reading of "GPT-OSS
  on Day 0", "Kernels for GPT-OSS" / "Sink Attention": chunks along the
  KV length merged by log-sum-exp, the sink in the first chunk only);
- prefill row t of a request is the decode of that row's query over the
  first P + t + 1 keys of the same pages (bottom-right causal alignment).

Examples are derandomized (fixed per test), so every run checks the same
batches; each prints its case before its GPU step.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from tests.test_gpu_parity import check  # noqa: E402

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                    suppress_health_check=list(HealthCheck))

# (Hq, Hkv): every group size the kernels are built for, one and several KV heads
GROUPS = [(1, 1), (2, 1), (4, 1), (8, 1), (16, 1), (4, 2), (16, 2), (32, 2), (64, 8), (16, 4)]
SINKS = st.sampled_from(["none", "normal", "wide", "neg", "pos"])


def sinks_arg(kind):
    return {"none": (None, 1.0), "normal": ("normal", 1.0), "wide": ("normal", 2.0),
            "neg": (-1e4, 1.0), "pos": (10.0, 1.0)}[kind]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_attn_amd  # noqa: F401  (fails loudly if not built)
    yield


def say(msg):
    print(msg, flush=True)


def gpu(b, plan="chunked", num_ranges=0, out_dtype=None):
    from gqa_attention_sinks_attn_amd import device
    db = device.to_device(b, plan=plan, num_ranges=num_ranges, out_dtype=out_dtype)
    if db.workspace is not None:
        db.workspace.fill_(0xFF)      # NaN partials: nothing may read an unwritten slot
    device.run(db)
    torch.cuda.synchronize()
    return (db.out.float().cpu().numpy().astype(np.float64),
            db.lse.cpu().numpy().astype(np.float64), db.out.dtype == torch.bfloat16)


def repool(b, rng, extra_pages):
    """The same batch with its pages moved to other slots of a larger pool;
    the unreferenced slots hold NaN bit patterns."""
    P = b.k.shape[0]
    sigma = rng.permutation(P + extra_pages).astype(np.int32)[:P]   # old page p -> sigma[p]
    nan = np.uint16(0x7FC0)
    k2 = np.full((P + extra_pages,) + b.k.shape[1:], nan, np.uint16)
    v2 = np.full_like(k2, nan)
    k2[sigma] = b.k
    v2[sigma] = b.v
    return W.Batch(kind=b.kind, q=b.q, qo_indptr=b.qo_indptr, k=k2, v=v2, kv_indptr=b.kv_indptr,
                   page_indices=sigma[b.page_indices], kv_len=b.kv_len, sinks=b.sinks,
                   num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                   head_dim=b.head_dim, page_size=b.page_size, sm_scale=b.sm_scale,
                   causal=b.causal, out_dtype=b.out_dtype, num_splits=b.num_splits,
                   draft_mask=b.draft_mask)


# ------------------------------------------------------------------ prefill

@st.composite
def prefill_cases(draw):
    hq, hkv = draw(st.sampled_from(GROUPS))
    B = draw(st.integers(1, 4))
    qlens = draw(st.lists(st.integers(0, 90), min_size=B, max_size=B))
    prefix = draw(st.lists(st.integers(0, 170), min_size=B, max_size=B))
    qlens[0] = max(qlens[0], 1)     # the ABI wants non-empty q and out buffers
    return dict(hq=hq, hkv=hkv, qlens=qlens, kv_lens=[p + q for p, q in zip(prefix, qlens)],
                paged=draw(st.booleans()), causal=draw(st.booleans()), sinks=draw(SINKS),
                seed=draw(st.integers(0, 2**31 - 1)))


def prefill_batch(c):
    s, std = sinks_arg(c["sinks"])
    return W.make_batch(c["seed"], kind="prefill", qlens=c["qlens"], kv_lens=c["kv_lens"],
                        hq=c["hq"], hkv=c["hkv"], paged=c["paged"], causal=c["causal"],
                        sinks=s, sink_std=std)


@SETTINGS
@given(c=prefill_cases())
def test_prefill_random_batches_match_the_oracle(c):
    say(f"[case] prefill {c}")
    b = prefill_batch(c)
    out, lse, bf16 = gpu(b)
    ref, rl = oracle.attend(b)
    check(f"property prefill G={c['hq'] // c['hkv']}", out, ref, lse, rl, bf16_out=bf16)


# ------------------------------------------------------------------- decode

DECODE_PLANS = [("chunked", 0), ("chunked", 1), ("chunked", 2), ("chunked", 5),
                ("balanced", 0), ("balanced", 4), ("balanced", 12)]


@st.composite
def decode_cases(draw):
    hq, hkv = draw(st.sampled_from(GROUPS))
    B = draw(st.integers(1, 16))
    kv_lens = draw(st.lists(st.integers(0, 420), min_size=B, max_size=B))
    kv_lens[0] = max(kv_lens[0], 1)               # a page table is never empty
    return dict(hq=hq, hkv=hkv, kv_lens=kv_lens,
                plan=draw(st.sampled_from(DECODE_PLANS)), sinks=draw(SINKS),
                out=draw(st.sampled_from(["f32", "bf16"])), seed=draw(st.integers(0, 2**31 - 1)))


def decode_batch(c, num_splits=0):
    s, std = sinks_arg(c["sinks"])
    # non-causal: the definition then allows empty requests (kv_len 0); a
    # single query at position kv_len - 1 sees every key either way
    return W.make_batch(c["seed"], kind="decode", qlens=[1] * len(c["kv_lens"]),
                        kv_lens=c["kv_lens"], hq=c["hq"], hkv=c["hkv"], paged=True,
                        causal=False, sinks=s, sink_std=std, num_splits=num_splits,
                        out_dtype=c.get("out", "f32"))


@SETTINGS
@given(c=decode_cases())
def test_decode_random_batches_match_the_oracle(c):
    say(f"[case] decode {c}")
    plan, n = c["plan"]
    b = decode_batch(c, num_splits=n if plan == "chunked" else 0)
    out, lse, bf16 = gpu(b, plan=plan, num_ranges=n if plan == "balanced" else 0)
    ref, rl = oracle.attend(b)
    check(f"property decode {plan} {n}", out, ref, lse, rl, bf16_out=bf16)


@SETTINGS
@given(c=decode_cases(), extra=st.integers(0, 9), pseed=st.integers(0, 2**31 - 1))
def test_decode_does_not_depend_on_where_pages_sit(c, extra, pseed):
    say(f"[case] decode page placement {c} extra={extra} pseed={pseed}")
    plan, n = c["plan"]
    b = decode_batch(c, num_splits=n if plan == "chunked" else 0)
    b2 = repool(b, np.random.default_rng(pseed), extra)
    kw = dict(plan=plan, num_ranges=n if plan == "balanced" else 0)
    out1, lse1, _ = gpu(b, **kw)
    out2, lse2, _ = gpu(b2, **kw)
    assert np.array_equal(out1, out2), "output moved with the pages"
    assert np.array_equal(lse1, lse2, equal_nan=True), "lse moved with the pages"


@SETTINGS
@given(c=decode_cases())
def test_split_plans_agree(c):
    """Unsplit, split-KV with S = 3 and 7, and the balanced plan with 4 and
    20 ranges: each at the bar against the oracle, and within twice the bar
    of the unsplit call."""
    say(f"[case] split plans {c}")
    c = dict(c, out="f32")
    ref, rl = None, None
    base = None
    for plan, n in [("chunked", 1), ("chunked", 3), ("chunked", 7), ("balanced", 4),
                    ("balanced", 20)]:
        b = decode_batch(c, num_splits=n if plan == "chunked" else 0)
        if ref is None:
            ref, rl = oracle.attend(b)
        out, lse, _ = gpu(b, plan=plan, num_ranges=n if plan == "balanced" else 0)
        check(f"property plans {plan} {n}", out, ref, lse, rl, bf16_out=False)
        if base is None:
            base = (out, lse)
        else:
            assert float(np.abs(out - base[0]).max()) <= 2e-2
            fin = np.isfinite(base[1])
            assert np.array_equal(np.isfinite(lse), fin)
            if fin.any():
                assert float(np.abs(lse[fin] - base[1][fin]).max()) <= 1e-2


# ------------------------------------------------- prefill row == decode row

@st.composite
def row_cases(draw):
    hq, hkv = draw(st.sampled_from(GROUPS))
    B = draw(st.integers(1, 3))
    qlens = draw(st.lists(st.integers(1, 40), min_size=B, max_size=B))
    prefix = draw(st.lists(st.integers(0, 200), min_size=B, max_size=B))
    return dict(hq=hq, hkv=hkv, qlens=qlens, kv_lens=[p + q for p, q in zip(prefix, qlens)],
                paged=True, causal=True, sinks=draw(SINKS), seed=draw(st.integers(0, 2**31 - 1)))


@SETTINGS
@given(c=row_cases(), plan=st.sampled_from(DECODE_PLANS))
def test_prefill_row_is_the_decode_of_its_query(c, plan):
    """Every row of a causal paged prefill, as a decode request of its own:
    its query, the first P + t + 1 keys, the request's own page list (the
    rest of its last page holds the request's later keys, not poison)."""
    say(f"[case] prefill rows as decodes {c} plan={plan}")
    pb = prefill_batch(c)
    qlens = np.diff(pb.qo_indptr)
    rows_L, rows_pages = [], []
    for r in range(pb.batch):
        L = int(pb.kv_len[r])
        pages = pb.page_indices[pb.kv_indptr[r]:pb.kv_indptr[r + 1]]
        for t in range(int(qlens[r])):
            n = L - int(qlens[r]) + t + 1
            rows_L.append(n)
            rows_pages.append(pages[: (n + 15) // 16])
    indptr = np.zeros(len(rows_L) + 1, np.int32)
    indptr[1:] = np.cumsum([len(p) for p in rows_pages])
    name, n = plan
    db = W.Batch(kind="decode", q=pb.q, qo_indptr=np.arange(len(rows_L) + 1, dtype=np.int32),
                 k=pb.k, v=pb.v, kv_indptr=indptr,
                 page_indices=np.concatenate(rows_pages).astype(np.int32),
                 kv_len=np.asarray(rows_L, np.int32), sinks=pb.sinks,
                 num_qo_heads=pb.num_qo_heads, num_kv_heads=pb.num_kv_heads,
                 head_dim=pb.head_dim, page_size=16, sm_scale=pb.sm_scale, causal=True,
                 num_splits=n if name == "chunked" else 0)
    out_p, lse_p, _ = gpu(pb)
    out_d, lse_d, _ = gpu(db, plan=name, num_ranges=n if name == "balanced" else 0)
    ref, rl = oracle.attend(pb)
    check("property prefill rows", out_p, ref, lse_p, rl, bf16_out=False)
    check("property rows as decodes", out_d, ref, lse_d, rl, bf16_out=False)
    assert float(np.abs(out_p - out_d).max()) <= 2e-2
    assert np.array_equal(np.isfinite(lse_p), np.isfinite(lse_d))


@SETTINGS
@given(c=row_cases(), extra=st.integers(0, 9), pseed=st.integers(0, 2**31 - 1))
def test_prefill_does_not_depend_on_where_pages_sit(c, extra, pseed):
    say(f"[case] prefill page placement {c} extra={extra} pseed={pseed}")
    b = prefill_batch(c)
    b2 = repool(b, np.random.default_rng(pseed), extra)
    out1, lse1, _ = gpu(b)
    out2, lse2, _ = gpu(b2)
    assert np.array_equal(out1, out2)
    assert np.array_equal(lse1, lse2, equal_nan=True)


# ------------------------------------------------------- tree verification

VERIFY_GROUPS = [(8, 1), (16, 1), (4, 2), (64, 8), (16, 16), (2, 1), (32, 2)]


@st.composite
def tree_cases(draw):
    hq, hkv = draw(st.sampled_from(VERIFY_GROUPS))
    B = draw(st.integers(1, 6))
    qlens = draw(st.lists(st.integers(0, 64), min_size=B, max_size=B))
    prefix = draw(st.lists(st.integers(0, 300), min_size=B, max_size=B))
    qlens[0] = max(qlens[0], 1)     # the ABI wants non-empty q and out buffers
    return dict(hq=hq, hkv=hkv, qlens=qlens, kv_lens=[p + q for p, q in zip(prefix, qlens)],
                splits=draw(st.sampled_from([0, 1, 3])), tree=draw(st.booleans()),
                sinks=draw(SINKS), seed=draw(st.integers(0, 2**31 - 1)))


@SETTINGS
@given(c=tree_cases())
def test_verify_random_drafts_match_the_oracle(c):
    say(f"[case] verify {c}")
    s, std = sinks_arg(c["sinks"])
    rng = np.random.default_rng(c["seed"])
    b = W.make_batch(rng, kind="prefill", qlens=c["qlens"], kv_lens=c["kv_lens"], hq=c["hq"],
                     hkv=c["hkv"], paged=True, sinks=s, sink_std=std, num_splits=c["splits"])
    if c["tree"]:
        b.draft_mask = np.concatenate(
            [W.tree_mask(W.draft_tree(rng, n)) if n else np.zeros(0, np.uint64)
             for n in c["qlens"]]).astype(np.uint64)
    out, lse, bf16 = gpu(b, plan="verify")
    ref, rl = oracle.attend(b)
    check(f"property verify tree={c['tree']}", out, ref, lse, rl, bf16_out=bf16)


# ------------------------------------------------------------ the fused steps

STEP_MAX_POS = 4096


@pytest.fixture(scope="module")
def rope_table():
    from gqa_attention_sinks_attn_amd import sink_attn_rope_table
    t = torch.empty((STEP_MAX_POS, 64), dtype=torch.float32, device="cuda")
    sink_attn_rope_table(t, STEP_MAX_POS, 64, 150000.0, 32.0, 4096, 32.0, 1.0, 0.0)
    torch.cuda.synchronize()
    return t


def sink_values(kind, hq, rng):
    s, std = sinks_arg(kind)
    if s is None:
        return None
    if isinstance(s, str):
        return (std * rng.standard_normal(hq)).astype(np.float32)
    return np.full(hq, s, np.float32)


@st.composite
def step_cases(draw, decode):
    hq, hkv = draw(st.sampled_from(GROUPS))
    B = draw(st.integers(1, 12 if decode else 4))
    if decode:
        qlens = [1] * B
        kv_lens = draw(st.lists(st.integers(1, 600), min_size=B, max_size=B))
    else:
        qlens = draw(st.lists(st.integers(1, 80), min_size=B, max_size=B))
        prefix = draw(st.lists(st.integers(0, 200), min_size=B, max_size=B))
        kv_lens = [p + q for p, q in zip(prefix, qlens)]
    return dict(hq=hq, hkv=hkv, qlens=qlens, kv_lens=kv_lens,
                interleaved=draw(st.sampled_from([0, 1])), bias=draw(st.booleans()),
                spare=draw(st.integers(0, 4)), sinks=draw(SINKS),
                out=draw(st.sampled_from(["f32", "bf16"])),
                causal=True if decode else draw(st.booleans()),
                seed=draw(st.integers(0, 2**31 - 1)))


def step_inputs(c):
    rng = np.random.default_rng(c["seed"])
    ab = W.make_append_batch(rng, qlens=c["qlens"], kv_lens=c["kv_lens"], hq=c["hq"],
                             hkv=c["hkv"], bias=c["bias"], spare_pages=c["spare"])
    od = torch.float32 if c["out"] == "f32" else torch.bfloat16
    return ab, sink_values(c["sinks"], c["hq"], rng), od


@SETTINGS
@given(c=step_cases(decode=True))
def test_decode_step_is_the_append_then_the_decode(rope_table, c):
    """sink_attn_decode_step against sink_attn_qkv_rope_append followed by
    sink_attn_decode_balanced: output, LSE and the whole cache bit for bit."""
    from tests import test_gpu_decode_step as DS
    say(f"[case] decode step {c}")
    ab, sinks, od = step_inputs(c)
    res = DS.run_both(ab, rope_table, sinks, c["interleaved"], out_dtype=od, bias=c["bias"],
                      max_pos=STEP_MAX_POS, name="property")
    DS.assert_bitwise(res)


@SETTINGS
@given(c=step_cases(decode=False))
def test_prefill_step_is_the_append_then_the_prefill(rope_table, c):
    """sink_attn_prefill_step against sink_attn_qkv_rope_append followed by
    sink_attn_prefill: output, LSE and the whole cache bit for bit."""
    from tests import test_gpu_prefill_step as PS
    say(f"[case] prefill step {c}")
    ab, sinks, od = step_inputs(c)
    res = PS.run_both(ab, rope_table, sinks, c["interleaved"], causal=c["causal"], out_dtype=od,
                      bias=c["bias"], max_pos=STEP_MAX_POS, name="property")
    PS.assert_bitwise(res)
