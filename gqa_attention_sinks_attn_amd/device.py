"""Device marshalling for callers that hold numpy batches (tests, benchmark).

Copies a batch's arrays to the GPU once, derives the host scalars the C ABI
asks for (max_qlen, max_kv_len, total_q) from the host copies, so no call
needs a device->host read, allocates outputs and the decode workspace, and
calls the binding.  Nothing here computes any part of the attention.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import (BF16, F32, sink_attn_decode, sink_attn_decode_balanced,
               sink_attn_decode_balanced_workspace_size, sink_attn_decode_num_splits,
               sink_attn_decode_workspace_size, sink_attn_prefill, sink_attn_verify,
               sink_attn_verify_tree, sink_attn_verify_workspace_size)


@dataclasses.dataclass
class DeviceBatch:
    kind: str
    q: torch.Tensor
    qo_indptr: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    kv_indptr: torch.Tensor
    page_indices: Optional[torch.Tensor]
    kv_len: Optional[torch.Tensor]
    sinks: Optional[torch.Tensor]
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    total_q: int
    max_qlen: int
    max_kv_len: int
    sm_scale: float
    causal: bool
    out_dtype: torch.dtype
    num_splits: int
    out: torch.Tensor = None
    lse: torch.Tensor = None
    workspace: Optional[torch.Tensor] = None
    workspace_bytes: int = 0
    plan: str = "chunked"          # decode: "chunked" (split-KV) or "balanced";
                                   # a paged prefill batch: "verify" calls sink_attn_verify
    num_ranges: int = 0            # balanced plan: ranges per KV head, 0 = automatic
    draft_mask: Optional[torch.Tensor] = None   # verify: int64 view of the uint64 mask words


def _bf16(a: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def _i32(a, device):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)


def to_device(b, device="cuda", with_lse: bool = True, out_dtype=None, plan: str = "chunked",
              num_ranges: int = 0) -> DeviceBatch:
    """b: a workloads.Batch (or any object with the same attributes).
    plan / num_ranges select the decode entry point: "chunked" calls
    sink_attn_decode with the batch's num_splits, "balanced" calls
    sink_attn_decode_balanced with num_ranges.  For a paged prefill batch,
    plan "verify" calls sink_attn_verify (with the batch's num_splits)
    instead of sink_attn_prefill, or sink_attn_verify_tree when the batch
    carries a draft_mask."""
    if plan not in ("chunked", "balanced", "verify"):
        raise ValueError(plan)
    od = out_dtype if out_dtype is not None else (
        torch.float32 if getattr(b, "out_dtype", "bf16") == "f32" else torch.bfloat16)
    total_q = int(b.qo_indptr[-1])
    qlens = np.diff(np.asarray(b.qo_indptr))
    max_qlen = int(qlens.max()) if qlens.size else 0
    kv_len_np = (np.asarray(b.kv_len) if b.kv_len is not None
                 else np.diff(np.asarray(b.kv_indptr)))
    max_kv_len = int(kv_len_np.max()) if kv_len_np.size else 0
    db = DeviceBatch(
        kind=b.kind, q=_bf16(b.q, device), qo_indptr=_i32(b.qo_indptr, device),
        k=_bf16(b.k, device), v=_bf16(b.v, device), kv_indptr=_i32(b.kv_indptr, device),
        page_indices=_i32(b.page_indices, device), kv_len=_i32(b.kv_len, device),
        sinks=None if b.sinks is None else torch.from_numpy(
            np.ascontiguousarray(b.sinks, np.float32)).to(device),
        batch=int(len(b.qo_indptr) - 1), num_qo_heads=int(b.num_qo_heads),
        num_kv_heads=int(b.num_kv_heads), head_dim=int(b.head_dim), page_size=int(b.page_size),
        total_q=total_q, max_qlen=max_qlen, max_kv_len=max_kv_len, sm_scale=float(b.sm_scale),
        causal=bool(b.causal), out_dtype=od, num_splits=int(getattr(b, "num_splits", 0)),
        plan=plan, num_ranges=int(num_ranges))
    db.out = torch.empty((total_q, db.num_qo_heads, db.head_dim), dtype=od, device=device)
    db.lse = (torch.empty((total_q, db.num_qo_heads), dtype=torch.float32, device=device)
              if with_lse else None)
    if db.kind == "prefill" and plan == "verify":
        dm = getattr(b, "draft_mask", None)
        if dm is not None:
            db.draft_mask = torch.from_numpy(
                np.ascontiguousarray(dm, np.uint64).view(np.int64)).to(device)
        db.workspace_bytes = sink_attn_verify_workspace_size(
            db.batch, db.num_qo_heads, db.num_kv_heads, db.head_dim, db.total_q, db.max_qlen,
            db.max_kv_len, db.num_splits)
        db.workspace = (torch.zeros(db.workspace_bytes, dtype=torch.uint8, device=device)
                        if db.workspace_bytes else None)
    if db.kind == "decode" and plan == "balanced":
        db.workspace_bytes = sink_attn_decode_balanced_workspace_size(
            db.batch, db.num_qo_heads, db.num_kv_heads, db.head_dim, db.max_kv_len, db.num_ranges)
    elif db.kind == "decode":
        db.workspace_bytes = sink_attn_decode_workspace_size(
            db.batch, db.num_qo_heads, db.num_kv_heads, db.head_dim, db.max_kv_len, db.num_splits)
    if db.kind == "decode":
        db.workspace = (torch.zeros(db.workspace_bytes, dtype=torch.uint8, device=device)
                        if db.workspace_bytes else None)
    return db


def splits_of(db: DeviceBatch) -> int:
    return sink_attn_decode_num_splits(db.batch, db.num_qo_heads, db.num_kv_heads, db.max_kv_len,
                                       db.num_splits)


def run(db: DeviceBatch, stream=None) -> None:
    """Enqueue the batch's call (prefill or decode) on the current stream."""
    code = F32 if db.out_dtype == torch.float32 else BF16
    if db.kind == "prefill" and db.plan == "verify" and db.draft_mask is not None:
        sink_attn_verify_tree(db.q, db.qo_indptr, db.draft_mask, db.k, db.v, db.kv_indptr,
                              db.page_indices, db.kv_len, db.sinks, db.batch, db.num_qo_heads,
                              db.num_kv_heads, db.head_dim, db.page_size, db.total_q,
                              db.max_qlen, db.max_kv_len, db.num_splits, db.sm_scale, db.out,
                              code, db.lse, db.workspace, db.workspace_bytes, stream)
    elif db.kind == "prefill" and db.plan == "verify":
        sink_attn_verify(db.q, db.qo_indptr, db.k, db.v, db.kv_indptr, db.page_indices, db.kv_len,
                         db.sinks, db.batch, db.num_qo_heads, db.num_kv_heads, db.head_dim,
                         db.page_size, db.total_q, db.max_qlen, db.max_kv_len, db.num_splits,
                         db.sm_scale, db.out, code, db.lse, db.workspace, db.workspace_bytes,
                         stream)
    elif db.kind == "prefill":
        sink_attn_prefill(db.q, db.qo_indptr, db.k, db.v, db.kv_indptr, db.page_indices,
                          db.kv_len, db.sinks, db.batch, db.num_qo_heads, db.num_kv_heads,
                          db.head_dim, db.page_size, db.total_q, db.max_qlen, db.max_kv_len,
                          db.sm_scale, db.causal, db.out, code, db.lse, stream)
    elif db.kind == "decode" and db.plan == "balanced":
        sink_attn_decode_balanced(
            db.q, db.k, db.v, db.kv_indptr, db.page_indices, db.kv_len, db.sinks, db.batch,
            db.num_qo_heads, db.num_kv_heads, db.head_dim, db.page_size, db.max_kv_len,
            db.num_ranges, db.sm_scale, db.out, code, db.lse, db.workspace, db.workspace_bytes,
            stream)
    elif db.kind == "decode":
        sink_attn_decode(db.q, db.k, db.v, db.kv_indptr, db.page_indices, db.kv_len, db.sinks,
                         db.batch, db.num_qo_heads, db.num_kv_heads, db.head_dim, db.page_size,
                         db.max_kv_len, db.num_splits, db.sm_scale, db.out, code, db.lse,
                         db.workspace, db.workspace_bytes, stream)
    else:
        raise ValueError(db.kind)
