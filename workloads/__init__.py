"""Seeded synthetic inputs for sink attention.

This module only draws and lays out inputs: lengths, page tables, Q/K/V and
per-head sinks.  It holds none of the attention arithmetic, so the oracle and
the GPU library can both consume what it produces.

Recipe (every workload):
  * generator: numpy ``default_rng(seed)`` (PCG64);
  * draw order: (1) lengths, (2) page permutation, (3) Q, (4) K, (5) V,
    (6) sinks;
  * Q, K and V are drawn fp32 ~ N(0, 1), then rounded once to bf16
    (round-to-nearest-even) on the host; both sides read those bits.  Large
    pools are drawn in chunks of 2^22 values, chunk i from child i of a
    seed sequence whose seed the workload's generator draws (deterministic
    for any thread count);
  * a paged cache holds exactly sum(ceil(L_b / page_size)) pages whose ids
    are a random permutation of the pool, handed out in request order, so
    the pages of different requests interleave in memory;
  * the unused slots of a request's last page hold finite poison
    (K = 8.0, V = 100.0): a kernel that reads past the end of a request
    lets those keys dominate its softmax, so the error is large.

Layouts (the library's documented format):
  q       bf16 bits uint16 [total_q, Hq, D]; qo_indptr int32 [B+1]
  contiguous k/v  uint16 [total_kv, Hkv, D]; kv_indptr = token offsets
  paged k/v       uint16 [num_pages, Hkv, page_size, D];
                  kv_indptr = offsets into page_indices (int32)
  kv_len  int32 [B];  sinks fp32 [Hq] or None (no sink)
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Batch", "Mixed", "to_bf16_bits", "bf16_bits_to_f32", "make_batch",
    "config", "CONFIG_NAMES", "K_POISON", "V_POISON", "draft_tree", "tree_mask",
    "chain_mask", "AppendBatch", "make_append_batch", "verify_workload", "append_workload",
    "VERIFY_WORKLOADS", "APPEND_WORKLOADS",
]

K_POISON = 8.0
V_POISON = 100.0
PAGE_SIZE = 16
HEAD_DIM = 64


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the fp32 values they denote (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Batch:
    """One call's worth of inputs (prefill or decode)."""
    kind: str                       # "prefill" or "decode"
    q: np.ndarray                   # uint16 [total_q, Hq, D]
    qo_indptr: np.ndarray           # int32 [B+1]
    k: np.ndarray                   # uint16, contiguous or paged (see module doc)
    v: np.ndarray
    kv_indptr: np.ndarray           # int32 [B+1]
    page_indices: Optional[np.ndarray]  # int32 [nnz] or None (contiguous)
    kv_len: np.ndarray              # int32 [B]
    sinks: Optional[np.ndarray]     # float32 [Hq] or None
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    sm_scale: float
    causal: bool
    out_dtype: str = "f32"          # "f32" or "bf16"
    num_splits: int = 0             # decode: 0 = library's automatic plan
    name: str = ""
    draft_mask: Optional[np.ndarray] = None  # uint64 [total_q]: drafted-token visibility

    @property
    def batch(self) -> int:
        return int(self.kv_len.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def qlens(self) -> np.ndarray:
        return np.diff(self.qo_indptr)

    @property
    def max_qlen(self) -> int:
        return int(self.qlens.max()) if self.batch else 0

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_len.max()) if self.batch else 0

    @property
    def paged(self) -> bool:
        return self.page_indices is not None


@dataclasses.dataclass
class Mixed:
    """A chunked-prefill call and a decode call over one shared page pool."""
    prefill: Batch
    decode: Batch
    name: str = ""


def _draw_qkv_pool(rng, shape_q, shape_kv):
    q = to_bf16_bits(rng.standard_normal(shape_q, dtype=np.float32))
    k = _normal_bf16(rng, shape_kv)
    v = _normal_bf16(rng, shape_kv)
    return q, k, v


def _normal_bf16(rng, shape, chunk_elems: int = 1 << 22) -> np.ndarray:
    """N(0,1) fp32 draws rounded to bf16.  The parent generator draws one
    128-bit seed; chunk i of 2^22 elements is drawn by child i of that seed
    sequence, so the values do not depend on how many threads fill them."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    ss = np.random.SeedSequence(int(rng.integers(0, 2**63)))
    n_chunks = (n + chunk_elems - 1) // chunk_elems
    children = ss.spawn(max(n_chunks, 1))

    def fill(i):
        s = i * chunk_elems
        e = min(n, s + chunk_elems)
        g = np.random.default_rng(children[i])
        out[s:e] = to_bf16_bits(g.standard_normal(e - s, dtype=np.float32))

    if n_chunks <= 1:
        if n:
            fill(0)
    else:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def _poison_tails(k, v, page_indices, kv_indptr, kv_len, page_size):
    """Fill the unused slots of each request's last page with poison."""
    kp, vp = to_bf16_bits(np.float32(K_POISON)), to_bf16_bits(np.float32(V_POISON))
    for b in range(kv_len.shape[0]):
        L = int(kv_len[b])
        used = L % page_size
        n_pages = int(kv_indptr[b + 1] - kv_indptr[b])
        if n_pages == 0:
            continue
        if used == 0 and L > 0:
            continue
        last = int(page_indices[kv_indptr[b + 1] - 1])
        k[last, :, used:, :] = kp
        v[last, :, used:, :] = vp


def _draw_sinks(rng, hq: int, sinks, std: float = 1.0) -> Optional[np.ndarray]:
    if sinks is None or sinks is False:
        return None
    if isinstance(sinks, str) and sinks == "normal":
        return (std * rng.standard_normal(hq)).astype(np.float32)
    arr = np.asarray(sinks, dtype=np.float32)
    if arr.ndim == 0:
        return np.full(hq, float(arr), dtype=np.float32)
    assert arr.shape == (hq,)
    return arr.copy()


def make_batch(seed, *, kind: str, qlens: Sequence[int], kv_lens: Sequence[int],
               hq: int, hkv: int, d: int = HEAD_DIM, paged: bool = False,
               page_size: int = PAGE_SIZE, sinks="normal", sink_std: float = 1.0,
               causal: bool = True, out_dtype: str = "f32", num_splits: int = 0,
               sm_scale: Optional[float] = None, permute_pages: bool = True,
               name: str = "") -> Batch:
    """Draw one batch.  `seed` is an int or a numpy Generator that has already
    drawn the lengths (step 1); `qlens`/`kv_lens` are given and the remaining
    draws follow the recipe order."""
    rng = seed if isinstance(seed, np.random.Generator) else np.random.default_rng(seed)
    qlens = np.asarray(qlens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    B = qlens.shape[0]
    assert kv_lens.shape == (B,)
    if causal:
        assert np.all(qlens <= kv_lens), "a causal query must have its own key"
    qo_indptr = np.zeros(B + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qlens)
    total_q = int(qo_indptr[-1])
    if paged:
        pages_per = (kv_lens + page_size - 1) // page_size
        kv_indptr = np.zeros(B + 1, dtype=np.int32)
        kv_indptr[1:] = np.cumsum(pages_per)
        n_pages = int(kv_indptr[-1])
        page_indices = (rng.permutation(n_pages) if permute_pages
                        else np.arange(n_pages)).astype(np.int32)
        q, k, v = _draw_qkv_pool(rng, (total_q, hq, d), (max(n_pages, 1), hkv, page_size, d))
        _poison_tails(k, v, page_indices, kv_indptr, kv_lens, page_size)
    else:
        kv_indptr = np.zeros(B + 1, dtype=np.int32)
        kv_indptr[1:] = np.cumsum(kv_lens)
        page_indices = None
        q, k, v = _draw_qkv_pool(rng, (total_q, hq, d), (max(int(kv_indptr[-1]), 1), hkv, d))
    s = _draw_sinks(rng, hq, sinks, sink_std)
    return Batch(kind=kind, q=q, qo_indptr=qo_indptr, k=k, v=v, kv_indptr=kv_indptr,
                 page_indices=page_indices, kv_len=kv_lens.astype(np.int32), sinks=s,
                 num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=page_size,
                 sm_scale=(1.0 / math.sqrt(d)) if sm_scale is None else float(sm_scale),
                 causal=causal, out_dtype=out_dtype, num_splits=num_splits, name=name)


CONFIG_NAMES = {
    1: "c1 tiny causal prefill: B=1 x 128, 4q/1kv, d=64, fp32 out",
    2: "c2 paged decode: B=64, L~U[1,4096], 64q/8kv, d=64, page 16",
    3: "c3 split-KV decode: B=4, L=131072, 64q/8kv, d=64, page 16, 32 splits",
    4: "c4 causal prefill: B=8 x 4096, 64q/8kv, d=64, contiguous KV",
    5: "c5 mixed: 16 chunked prefills (n~U[256,2048], prefix~U[0,8192]) + "
       "256 decodes (L~U[1,16384]), 64q/8kv, d=64, page 16",
}


def config(n: int, seed: Optional[int] = None):
    """The five workloads with their seeded recipes (seed = 1000 + n)."""
    seed = 1000 + n if seed is None else seed
    if n == 1:
        return make_batch(seed, kind="prefill", qlens=[128], kv_lens=[128], hq=4, hkv=1,
                          causal=True, out_dtype="f32", name=CONFIG_NAMES[1])
    if n == 2:
        rng = np.random.default_rng(seed)
        L = rng.integers(1, 4096, size=64, endpoint=True)
        return make_batch(rng, kind="decode", qlens=[1] * 64, kv_lens=L, hq=64, hkv=8,
                          paged=True, causal=True, name=CONFIG_NAMES[2])
    if n == 3:
        return make_batch(seed, kind="decode", qlens=[1] * 4, kv_lens=[131072] * 4, hq=64,
                          hkv=8, paged=True, sink_std=2.0, num_splits=32, name=CONFIG_NAMES[3])
    if n == 4:
        return make_batch(seed, kind="prefill", qlens=[4096] * 8, kv_lens=[4096] * 8, hq=64,
                          hkv=8, paged=False, causal=True, name=CONFIG_NAMES[4])
    if n == 5:
        return mixed(seed)
    raise ValueError(f"no workload {n}")


def c5_sinks(rng, hq: int = 64) -> np.ndarray:
    """N(0,1) sinks with the extremes of workload 5 planted on fixed heads."""
    s = rng.standard_normal(hq).astype(np.float32)
    for h in (0, 17, 42):
        if h < hq:
            s[h] = -1e4
    for h in (5, 31, 63):
        if h < hq:
            s[h] = 10.0
    return s


def mixed(seed: int = 1005, n_prefill: int = 16, n_decode: int = 256, hq: int = 64,
          hkv: int = 8, scale: float = 1.0) -> Mixed:
    """Workload 5: chunked prefills on cached prefixes plus decodes, one page
    pool.  `scale` < 1 shrinks every length (for fast parity cases)."""
    rng = np.random.default_rng(seed)
    n_new = rng.integers(256, 2048, size=n_prefill, endpoint=True)
    prefix = rng.integers(0, 8192, size=n_prefill, endpoint=True)
    dec_L = rng.integers(1, 16384, size=n_decode, endpoint=True)
    if scale != 1.0:
        n_new = np.maximum(1, (n_new * scale).astype(np.int64))
        prefix = (prefix * scale).astype(np.int64)
        dec_L = np.maximum(1, (dec_L * scale).astype(np.int64))
    pf_kv = prefix + n_new
    all_L = np.concatenate([pf_kv, dec_L])
    ps = PAGE_SIZE
    pages_per = (all_L + ps - 1) // ps
    indptr_all = np.zeros(all_L.shape[0] + 1, dtype=np.int64)
    indptr_all[1:] = np.cumsum(pages_per)
    n_pages = int(indptr_all[-1])
    perm = rng.permutation(n_pages).astype(np.int32)
    d = HEAD_DIM
    total_q_pf = int(n_new.sum())
    q_pf = to_bf16_bits(rng.standard_normal((total_q_pf, hq, d), dtype=np.float32))
    q_dec = to_bf16_bits(rng.standard_normal((n_decode, hq, d), dtype=np.float32))
    k = _normal_bf16(rng, (n_pages, hkv, ps, d))
    v = _normal_bf16(rng, (n_pages, hkv, ps, d))
    _poison_tails(k, v, perm, indptr_all, all_L, ps)
    sinks = c5_sinks(rng, hq)

    pf_pages = int(indptr_all[n_prefill])
    pf_indptr = indptr_all[: n_prefill + 1].astype(np.int32)
    dec_indptr = (indptr_all[n_prefill:] - pf_pages).astype(np.int32)
    qo_pf = np.zeros(n_prefill + 1, dtype=np.int32)
    qo_pf[1:] = np.cumsum(n_new)
    scale_attn = 1.0 / math.sqrt(d)
    pre = Batch(kind="prefill", q=q_pf, qo_indptr=qo_pf, k=k, v=v, kv_indptr=pf_indptr,
                page_indices=perm[:pf_pages].copy(), kv_len=pf_kv.astype(np.int32), sinks=sinks,
                num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                sm_scale=scale_attn, causal=True, name="c5 chunked prefill part")
    dec = Batch(kind="decode", q=q_dec, qo_indptr=np.arange(n_decode + 1, dtype=np.int32),
                k=k, v=v, kv_indptr=dec_indptr, page_indices=perm[pf_pages:].copy(),
                kv_len=dec_L.astype(np.int32), sinks=sinks, num_qo_heads=hq, num_kv_heads=hkv,
                head_dim=d, page_size=ps, sm_scale=scale_attn, causal=True,
                name="c5 decode part")
    return Mixed(prefill=pre, decode=dec, name=CONFIG_NAMES[5])


# --- drafted-token trees (inputs for verification with a draft mask) ---------

def draft_tree(rng, n: int, max_children: int = 4) -> np.ndarray:
    """A random draft tree over n tokens in breadth-first order: parents[i] is
    the index of token i's parent among the drafted tokens, or -1 when token
    i hangs directly off the cached prefix.  Token 0 is always a root; each
    later token picks a parent among the earlier ones that still have fewer
    than max_children children (or becomes another root)."""
    parents = np.full(n, -1, dtype=np.int64)
    children = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        open_ = [-1] + [j for j in range(i) if children[j] < max_children]
        p = int(open_[int(rng.integers(0, len(open_)))])
        parents[i] = p
        if p >= 0:
            children[p] += 1
    return parents


def tree_mask(parents: Sequence[int]) -> np.ndarray:
    """Visibility bits of a draft tree: bit j of word i is set when drafted
    token j is token i itself or one of its ancestors.  uint64 [n], n <= 64."""
    n = len(parents)
    assert n <= 64
    out = np.zeros(n, dtype=np.uint64)
    for i in range(n):
        w = 0
        j = i
        while j >= 0:
            w |= 1 << j
            j = int(parents[j])
        out[i] = np.uint64(w)
    return out


def chain_mask(n: int) -> np.ndarray:
    """The linear draft (each token sees itself and every earlier one)."""
    return np.array([(1 << (i + 1)) - 1 for i in range(n)], dtype=np.uint64)


# --- new tokens for the projection-side step (bias, rotary, paged append) ---

@dataclasses.dataclass
class AppendBatch:
    """One step's new tokens before attention: the fused QKV projection output
    of every new token, the projection bias, and a paged cache whose pages for
    the new positions are already reserved (kv_len counts the new tokens)."""
    qkv: np.ndarray                 # uint16 [T, Hq + 2 Hkv, D]
    bias: Optional[np.ndarray]      # uint16 [(Hq + 2 Hkv) D] or None
    qo_indptr: np.ndarray           # int32 [B+1]
    kv_len: np.ndarray              # int32 [B], after the append
    page_indptr: np.ndarray         # int32 [B+1]
    page_indices: np.ndarray        # int32 [nnz]
    k_pages: np.ndarray             # uint16 [num_pages, Hkv, page_size, D] (old contents)
    v_pages: np.ndarray
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    name: str = ""

    @property
    def batch(self) -> int:
        return int(self.kv_len.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])


def make_append_batch(seed, *, qlens: Sequence[int], kv_lens: Sequence[int], hq: int, hkv: int,
                      d: int = HEAD_DIM, page_size: int = PAGE_SIZE, bias: bool = True,
                      bias_std: float = 0.5, spare_pages: int = 3, name: str = "") -> AppendBatch:
    """Draw order: page permutation, qkv (N(0,1)), bias (N(0, bias_std)), old
    cache contents (N(0,1)).  The pool holds the requests' pages plus
    spare_pages unused ones, so writes outside the reserved slots show."""
    rng = seed if isinstance(seed, np.random.Generator) else np.random.default_rng(seed)
    qlens = np.asarray(qlens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    assert np.all(qlens <= kv_lens)
    B = qlens.shape[0]
    qo = np.zeros(B + 1, np.int32)
    qo[1:] = np.cumsum(qlens)
    pages_per = (kv_lens + page_size - 1) // page_size
    indptr = np.zeros(B + 1, np.int32)
    indptr[1:] = np.cumsum(pages_per)
    n_pages = int(indptr[-1]) + spare_pages
    perm = rng.permutation(n_pages).astype(np.int32)
    indices = perm[: int(indptr[-1])]
    T = int(qo[-1])
    H = hq + 2 * hkv
    qkv = to_bf16_bits(rng.standard_normal((T, H, d), dtype=np.float32))
    bb = (to_bf16_bits(bias_std * rng.standard_normal(H * d, dtype=np.float32))
          if bias else None)
    kp = to_bf16_bits(rng.standard_normal((max(n_pages, 1), hkv, page_size, d), dtype=np.float32))
    vp = to_bf16_bits(rng.standard_normal((max(n_pages, 1), hkv, page_size, d), dtype=np.float32))
    return AppendBatch(qkv=qkv, bias=bb, qo_indptr=qo, kv_len=kv_lens.astype(np.int32),
                       page_indptr=indptr, page_indices=np.ascontiguousarray(indices),
                       k_pages=kp, v_pages=vp, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d,
                       page_size=page_size, name=name)


# --- the verification and append batches the benchmark times ----------------

VERIFY_WORKLOADS = ("verify_4tok", "verify_16tok", "verify_tree_16tok", "verify_tree_32tok")
APPEND_WORKLOADS = ("append_prefill_8x4096", "append_decode_64")


def verify_workload(name: str) -> Batch:
    """64 requests, 64q/8kv, 16-token pages, KV lengths U[qlen, 4096]:
    4 drafted tokens (seed 1090), 16 (seed 1091; linear, or random draft
    trees drawn after the batch) or 32-token draft trees (seed 1094)."""
    qlen, seed, tree = {"verify_4tok": (4, 1090, False), "verify_16tok": (16, 1091, False),
                        "verify_tree_16tok": (16, 1091, True),
                        "verify_tree_32tok": (32, 1094, True)}[name]
    rng = np.random.default_rng(seed)
    L = rng.integers(qlen, 4096, size=64, endpoint=True)
    kind = "draft trees" if tree else "drafted tokens"
    b = make_batch(rng, kind="prefill", qlens=[qlen] * 64, kv_lens=L, hq=64, hkv=8, paged=True,
                   sinks="normal",
                   name=f"verify: B=64 x {qlen} {kind}, L~U[{qlen},4096], 64q/8kv, page 16")
    if tree:
        b.draft_mask = np.concatenate([tree_mask(draft_tree(rng, qlen)) for _ in range(64)])
    return b


def append_workload(name: str) -> AppendBatch:
    """The bias + rotary + append step of 64q/8kv: a prefill step of 8 x 4096
    new tokens, or a decode step of 64 requests x 1 token with KV lengths
    U[1, 4096] (seed 1092); the projections and caches from seed 1093."""
    if name == "append_prefill_8x4096":
        qlens, kvl = [4096] * 8, [4096] * 8
    elif name == "append_decode_64":
        qlens, kvl = [1] * 64, list(np.random.default_rng(1092).integers(1, 4097, size=64))
    else:
        raise ValueError(name)
    return make_append_batch(1093, qlens=qlens, kv_lens=kvl, hq=64, hkv=8, spare_pages=0,
                             name=f"{sum(qlens)} new tokens, 64q/8kv, d=64, page 16, YaRN table")
