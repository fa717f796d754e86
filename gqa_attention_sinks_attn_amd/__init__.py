"""Python binding of the gfx950 sink-attention library (libsink_attn.so).

Argument marshalling only: every function here has the name of the C entry
point it calls (include/sink_attn.h), takes torch tensors that already live
on the GPU plus the same host scalars, passes their device pointers and the
current HIP stream, and raises SinkAttnError on a non-OK status.  No step
of the attention runs in Python or in torch; the library must be built
(``python -m gqa_attention_sinks_attn_amd.build``): the first call loads it
and raises ImportError when it is missing.

GQA attention with a per-head sink logit (GPT-OSS on Day 0, Perplexity:
"Attention: GQA with attention sinks"; "Sink attention" under "Kernels for
GPT-OSS").
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SinkAttnError", "LIB_PATH", "lib", "BF16", "F32",
    "sink_attn_prefill", "sink_attn_decode", "sink_attn_decode_partial", "sink_attn_merge",
    "sink_attn_decode_workspace_size", "sink_attn_decode_num_splits",
    "sink_attn_decode_balanced", "sink_attn_decode_balanced_partial",
    "sink_attn_decode_balanced_finish", "sink_attn_decode_balanced_workspace_size",
    "sink_attn_decode_num_ranges", "sink_attn_verify", "sink_attn_verify_workspace_size",
    "sink_attn_verify_tree", "sink_attn_verify_num_splits", "sink_attn_rope_table",
    "sink_attn_qkv_rope_append", "sink_attn_decode_noalloc", "sink_attn_decode_step",
    "sink_attn_decode_step_workspace_size", "sink_attn_prefill_step",
    "sink_attn_status_string", "sink_attn_last_error", "sink_attn_version",
    "SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsink_attn.so")
BF16 = 0
F32 = 1
SYMBOLS = (
    "sink_attn_prefill", "sink_attn_decode", "sink_attn_decode_partial", "sink_attn_merge",
    "sink_attn_decode_workspace_size", "sink_attn_decode_num_splits",
    "sink_attn_decode_balanced", "sink_attn_decode_balanced_partial",
    "sink_attn_decode_balanced_finish", "sink_attn_decode_balanced_workspace_size",
    "sink_attn_decode_num_ranges", "sink_attn_verify", "sink_attn_verify_workspace_size",
    "sink_attn_verify_tree", "sink_attn_verify_num_splits", "sink_attn_rope_table",
    "sink_attn_qkv_rope_append", "sink_attn_decode_noalloc", "sink_attn_decode_step",
    "sink_attn_decode_step_workspace_size", "sink_attn_prefill_step",
    "sink_attn_status_string", "sink_attn_last_error", "sink_attn_version",
)


class SinkAttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"sink_attn status {status}: {detail}")


_P = ctypes.c_void_p
_I = ctypes.c_int32
_lib = None


def lib():
    """The loaded ctypes library (loaded on first use).  Raises ImportError if
    the library was never built: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m gqa_attention_sinks_attn_amd.build); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    L.sink_attn_prefill.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                    _I, ctypes.c_float, _I, _P, ctypes.c_int, _P, _P]
    L.sink_attn_prefill.restype = ctypes.c_int
    L.sink_attn_decode.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                   ctypes.c_float, _P, ctypes.c_int, _P, _P, ctypes.c_size_t, _P]
    L.sink_attn_decode.restype = ctypes.c_int
    L.sink_attn_decode_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                           _I, ctypes.c_float, _P, ctypes.c_int, _P, _P]
    L.sink_attn_decode_noalloc.restype = ctypes.c_int
    L.sink_attn_decode_partial.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                           _I, ctypes.c_float, _P, _P, _P]
    L.sink_attn_decode_partial.restype = ctypes.c_int
    L.sink_attn_merge.argtypes = [_P, _P, _I, _I, _I, _I, _P, ctypes.c_int, _P, _P]
    L.sink_attn_merge.restype = ctypes.c_int
    L.sink_attn_decode_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I]
    L.sink_attn_decode_workspace_size.restype = ctypes.c_size_t
    L.sink_attn_decode_num_splits.argtypes = [_I, _I, _I, _I, _I]
    L.sink_attn_decode_num_splits.restype = _I
    for name in ("sink_attn_decode_balanced", "sink_attn_decode_balanced_partial"):
        f = getattr(L, name)
        f.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P,
                      ctypes.c_int, _P, _P, ctypes.c_size_t, _P]
        f.restype = ctypes.c_int
    L.sink_attn_decode_balanced_finish.argtypes = [_P, _P, _I, _I, _I, _I, _I, _I, _P,
                                                   ctypes.c_int, _P, _P, ctypes.c_size_t, _P]
    L.sink_attn_decode_balanced_finish.restype = ctypes.c_int
    L.sink_attn_decode_balanced_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I]
    L.sink_attn_decode_balanced_workspace_size.restype = ctypes.c_size_t
    L.sink_attn_decode_num_ranges.argtypes = [_I, _I, _I, _I]
    L.sink_attn_decode_num_ranges.restype = _I
    L.sink_attn_verify.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                   _I, _I, ctypes.c_float, _P, ctypes.c_int, _P, _P,
                                   ctypes.c_size_t, _P]
    L.sink_attn_verify.restype = ctypes.c_int
    L.sink_attn_verify_tree.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                        _I, _I, _I, _I, ctypes.c_float, _P, ctypes.c_int, _P, _P,
                                        ctypes.c_size_t, _P]
    L.sink_attn_verify_tree.restype = ctypes.c_int
    L.sink_attn_verify_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I]
    L.sink_attn_verify_workspace_size.restype = ctypes.c_size_t
    L.sink_attn_verify_num_splits.argtypes = [_I, _I, _I, _I, _I, _I]
    L.sink_attn_verify_num_splits.restype = _I
    _D = ctypes.c_double
    L.sink_attn_rope_table.argtypes = [_P, _I, _I, _D, _D, _I, _D, _D, _D, ctypes.c_int, _P]
    L.sink_attn_rope_table.restype = ctypes.c_int
    L.sink_attn_qkv_rope_append.argtypes = [_P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                            _I, _I, _P, _P, _P, _P]
    L.sink_attn_qkv_rope_append.restype = ctypes.c_int
    L.sink_attn_decode_step.argtypes = [_P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I, _I,
                                        _I, _I, _I, ctypes.c_float, _P, ctypes.c_int, _P, _P,
                                        ctypes.c_size_t, _P]
    L.sink_attn_decode_step.restype = ctypes.c_int
    L.sink_attn_prefill_step.argtypes = [_P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _I,
                                         _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P,
                                         ctypes.c_int, _P, _P]
    L.sink_attn_prefill_step.restype = ctypes.c_int
    L.sink_attn_decode_step_workspace_size.argtypes = [_I, _I, _I, _I, _I]
    L.sink_attn_decode_step_workspace_size.restype = ctypes.c_size_t
    L.sink_attn_status_string.argtypes = [ctypes.c_int]
    L.sink_attn_status_string.restype = ctypes.c_char_p
    L.sink_attn_last_error.argtypes = []
    L.sink_attn_last_error.restype = ctypes.c_char_p
    L.sink_attn_version.argtypes = []
    L.sink_attn_version.restype = ctypes.c_char_p
    _lib = L
    return _lib


def _ptr(t):
    """Device (or host) address of a tensor, None for None; ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(out_dtype) -> int:
    if isinstance(out_dtype, int):
        return out_dtype
    import torch
    if out_dtype == torch.bfloat16:
        return BF16
    if out_dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported output dtype {out_dtype}")


def _check(rc: int):
    if rc != 0:
        raise SinkAttnError(rc, lib().sink_attn_last_error().decode())


def sink_attn_status_string(status: int) -> str:
    return lib().sink_attn_status_string(int(status)).decode()


def sink_attn_last_error() -> str:
    return lib().sink_attn_last_error().decode()


def sink_attn_version() -> str:
    return lib().sink_attn_version().decode()


def sink_attn_prefill(q, qo_indptr, k, v, kv_indptr, page_indices, kv_len, sinks,
                      batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                      total_q, max_qlen, max_kv_len, sm_scale, causal,
                      out, out_dtype, lse, stream=None) -> None:
    _check(lib().sink_attn_prefill(
        _ptr(q), _ptr(qo_indptr), _ptr(k), _ptr(v), _ptr(kv_indptr), _ptr(page_indices),
        _ptr(kv_len), _ptr(sinks), int(batch), int(num_qo_heads), int(num_kv_heads),
        int(head_dim), int(page_size), int(total_q), int(max_qlen), int(max_kv_len),
        float(sm_scale), int(bool(causal)), _ptr(out), _dtype_code(out_dtype), _ptr(lse),
        _stream(stream)))


def sink_attn_decode_num_splits(batch, num_qo_heads, num_kv_heads, max_kv_len, num_splits) -> int:
    return int(lib().sink_attn_decode_num_splits(int(batch), int(num_qo_heads), int(num_kv_heads),
                                                int(max_kv_len), int(num_splits)))


def sink_attn_decode_workspace_size(batch, num_qo_heads, num_kv_heads, head_dim, max_kv_len,
                                    num_splits) -> int:
    return int(lib().sink_attn_decode_workspace_size(int(batch), int(num_qo_heads),
                                                    int(num_kv_heads), int(head_dim),
                                                    int(max_kv_len), int(num_splits)))


def sink_attn_decode(q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks,
                     batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                     max_kv_len, num_splits, sm_scale, out, out_dtype, lse,
                     workspace, workspace_bytes, stream=None) -> None:
    _check(lib().sink_attn_decode(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_indptr), _ptr(page_indices),
        _ptr(kv_len), _ptr(sinks), int(batch), int(num_qo_heads), int(num_kv_heads),
        int(head_dim), int(page_size), int(max_kv_len), int(num_splits), float(sm_scale),
        _ptr(out), _dtype_code(out_dtype), _ptr(lse), _ptr(workspace), int(workspace_bytes),
        _stream(stream)))


def sink_attn_decode_noalloc(q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks,
                             batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                             max_kv_len, num_splits, sm_scale, out, out_dtype, lse,
                             stream=None) -> None:
    _check(lib().sink_attn_decode_noalloc(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_indptr), _ptr(page_indices),
        _ptr(kv_len), _ptr(sinks), int(batch), int(num_qo_heads), int(num_kv_heads),
        int(head_dim), int(page_size), int(max_kv_len), int(num_splits), float(sm_scale),
        _ptr(out), _dtype_code(out_dtype), _ptr(lse), _stream(stream)))


def sink_attn_decode_partial(q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks,
                             batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                             max_kv_len, num_splits, sm_scale, o_parts, lse_parts,
                             stream=None) -> None:
    _check(lib().sink_attn_decode_partial(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_indptr), _ptr(page_indices),
        _ptr(kv_len), _ptr(sinks), int(batch), int(num_qo_heads), int(num_kv_heads),
        int(head_dim), int(page_size), int(max_kv_len), int(num_splits), float(sm_scale),
        _ptr(o_parts), _ptr(lse_parts), _stream(stream)))


def sink_attn_merge(o_parts, lse_parts, num_rows, num_heads, num_splits, head_dim,
                    out, out_dtype, lse_out, stream=None) -> None:
    _check(lib().sink_attn_merge(
        _ptr(o_parts), _ptr(lse_parts), int(num_rows), int(num_heads), int(num_splits),
        int(head_dim), _ptr(out), _dtype_code(out_dtype), _ptr(lse_out), _stream(stream)))


def sink_attn_decode_num_ranges(batch, num_kv_heads, max_kv_len, num_ranges) -> int:
    return int(lib().sink_attn_decode_num_ranges(int(batch), int(num_kv_heads), int(max_kv_len),
                                                int(num_ranges)))


def sink_attn_decode_balanced_workspace_size(batch, num_qo_heads, num_kv_heads, head_dim,
                                             max_kv_len, num_ranges) -> int:
    return int(lib().sink_attn_decode_balanced_workspace_size(
        int(batch), int(num_qo_heads), int(num_kv_heads), int(head_dim), int(max_kv_len),
        int(num_ranges)))


def _balanced(fn, q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks, batch,
              num_qo_heads, num_kv_heads, head_dim, page_size, max_kv_len, num_ranges, sm_scale,
              out, out_dtype, lse, workspace, workspace_bytes, stream):
    _check(fn(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_indptr), _ptr(page_indices),
        _ptr(kv_len), _ptr(sinks), int(batch), int(num_qo_heads), int(num_kv_heads),
        int(head_dim), int(page_size), int(max_kv_len), int(num_ranges), float(sm_scale),
        _ptr(out), _dtype_code(out_dtype), _ptr(lse), _ptr(workspace), int(workspace_bytes),
        _stream(stream)))


def sink_attn_decode_balanced(q, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks,
                              batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                              max_kv_len, num_ranges, sm_scale, out, out_dtype, lse,
                              workspace, workspace_bytes, stream=None) -> None:
    _balanced(lib().sink_attn_decode_balanced, q, k_pages, v_pages, page_indptr, page_indices,
              kv_len, sinks, batch, num_qo_heads, num_kv_heads, head_dim, page_size, max_kv_len,
              num_ranges, sm_scale, out, out_dtype, lse, workspace, workspace_bytes, stream)


def sink_attn_decode_balanced_partial(q, k_pages, v_pages, page_indptr, page_indices, kv_len,
                                      sinks, batch, num_qo_heads, num_kv_heads, head_dim,
                                      page_size, max_kv_len, num_ranges, sm_scale, out,
                                      out_dtype, lse, workspace, workspace_bytes,
                                      stream=None) -> None:
    _balanced(lib().sink_attn_decode_balanced_partial, q, k_pages, v_pages, page_indptr,
              page_indices, kv_len, sinks, batch, num_qo_heads, num_kv_heads, head_dim,
              page_size, max_kv_len, num_ranges, sm_scale, out, out_dtype, lse, workspace,
              workspace_bytes, stream)


def sink_attn_decode_balanced_finish(page_indptr, sinks, batch, num_qo_heads, num_kv_heads,
                                     head_dim, max_kv_len, num_ranges, out, out_dtype, lse,
                                     workspace, workspace_bytes, stream=None) -> None:
    _check(lib().sink_attn_decode_balanced_finish(
        _ptr(page_indptr), _ptr(sinks), int(batch), int(num_qo_heads), int(num_kv_heads),
        int(head_dim), int(max_kv_len), int(num_ranges), _ptr(out), _dtype_code(out_dtype),
        _ptr(lse), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def sink_attn_verify_workspace_size(batch, num_qo_heads, num_kv_heads, head_dim, total_q,
                                    max_qlen, max_kv_len, num_splits) -> int:
    return int(lib().sink_attn_verify_workspace_size(
        int(batch), int(num_qo_heads), int(num_kv_heads), int(head_dim), int(total_q),
        int(max_qlen), int(max_kv_len), int(num_splits)))


def sink_attn_verify_num_splits(batch, num_qo_heads, num_kv_heads, max_qlen, max_kv_len,
                                num_splits) -> int:
    return int(lib().sink_attn_verify_num_splits(
        int(batch), int(num_qo_heads), int(num_kv_heads), int(max_qlen), int(max_kv_len),
        int(num_splits)))


def sink_attn_verify(q, qo_indptr, k_pages, v_pages, page_indptr, page_indices, kv_len, sinks,
                     batch, num_qo_heads, num_kv_heads, head_dim, page_size, total_q, max_qlen,
                     max_kv_len, num_splits, sm_scale, out, out_dtype, lse, workspace,
                     workspace_bytes, stream=None) -> None:
    _check(lib().sink_attn_verify(
        _ptr(q), _ptr(qo_indptr), _ptr(k_pages), _ptr(v_pages), _ptr(page_indptr),
        _ptr(page_indices), _ptr(kv_len), _ptr(sinks), int(batch), int(num_qo_heads),
        int(num_kv_heads), int(head_dim), int(page_size), int(total_q), int(max_qlen),
        int(max_kv_len), int(num_splits), float(sm_scale), _ptr(out), _dtype_code(out_dtype),
        _ptr(lse), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def sink_attn_verify_tree(q, qo_indptr, draft_mask, k_pages, v_pages, page_indptr, page_indices,
                          kv_len, sinks, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                          total_q, max_qlen, max_kv_len, num_splits, sm_scale, out, out_dtype,
                          lse, workspace, workspace_bytes, stream=None) -> None:
    _check(lib().sink_attn_verify_tree(
        _ptr(q), _ptr(qo_indptr), _ptr(draft_mask), _ptr(k_pages), _ptr(v_pages),
        _ptr(page_indptr), _ptr(page_indices), _ptr(kv_len), _ptr(sinks), int(batch),
        int(num_qo_heads), int(num_kv_heads), int(head_dim), int(page_size), int(total_q),
        int(max_qlen), int(max_kv_len), int(num_splits), float(sm_scale), _ptr(out),
        _dtype_code(out_dtype), _ptr(lse), _ptr(workspace), int(workspace_bytes),
        _stream(stream)))


YARN_RAMP_TURNS = 0
YARN_RAMP_PAIRS = 1


def sink_attn_rope_table(table, max_pos, head_dim, rope_theta, factor, original_max_pos,
                         beta_fast, beta_slow, attn_factor=0.0, yarn_ramp=YARN_RAMP_TURNS,
                         stream=None) -> None:
    _check(lib().sink_attn_rope_table(
        _ptr(table), int(max_pos), int(head_dim), float(rope_theta), float(factor),
        int(original_max_pos), float(beta_fast), float(beta_slow), float(attn_factor),
        int(yarn_ramp), _stream(stream)))


def sink_attn_prefill_step(qkv, bias, rope_table, max_pos, interleaved, qo_indptr, k_pages,
                           v_pages, page_indptr, page_indices, kv_len, sinks, batch,
                           num_qo_heads, num_kv_heads, head_dim, page_size, total_q, max_qlen,
                           max_kv_len, sm_scale, causal, out, out_dtype, lse,
                           stream=None) -> None:
    _check(lib().sink_attn_prefill_step(
        _ptr(qkv), _ptr(bias), _ptr(rope_table), int(max_pos), int(interleaved),
        _ptr(qo_indptr), _ptr(k_pages), _ptr(v_pages), _ptr(page_indptr), _ptr(page_indices),
        _ptr(kv_len), _ptr(sinks), int(batch), int(num_qo_heads), int(num_kv_heads),
        int(head_dim), int(page_size), int(total_q), int(max_qlen), int(max_kv_len),
        float(sm_scale), int(bool(causal)), _ptr(out), _dtype_code(out_dtype), _ptr(lse),
        _stream(stream)))


def sink_attn_decode_step_workspace_size(batch, num_qo_heads, num_kv_heads, head_dim,
                                         max_kv_len) -> int:
    return int(lib().sink_attn_decode_step_workspace_size(
        int(batch), int(num_qo_heads), int(num_kv_heads), int(head_dim), int(max_kv_len)))


def sink_attn_decode_step(qkv, bias, rope_table, max_pos, interleaved, k_pages, v_pages,
                          page_indptr, page_indices, kv_len, sinks, batch, num_qo_heads,
                          num_kv_heads, head_dim, page_size, max_kv_len, sm_scale, out, out_dtype,
                          lse, workspace, workspace_bytes, stream=None) -> None:
    _check(lib().sink_attn_decode_step(
        _ptr(qkv), _ptr(bias), _ptr(rope_table), int(max_pos), int(interleaved), _ptr(k_pages),
        _ptr(v_pages), _ptr(page_indptr), _ptr(page_indices), _ptr(kv_len), _ptr(sinks),
        int(batch), int(num_qo_heads), int(num_kv_heads), int(head_dim), int(page_size),
        int(max_kv_len), float(sm_scale), _ptr(out), _dtype_code(out_dtype), _ptr(lse),
        _ptr(workspace), int(workspace_bytes), _stream(stream)))


def sink_attn_qkv_rope_append(qkv, bias, rope_table, max_pos, qo_indptr, kv_len, page_indptr,
                              page_indices, batch, num_qo_heads, num_kv_heads, head_dim,
                              page_size, total_q, interleaved, q_out, k_pages, v_pages,
                              stream=None) -> None:
    _check(lib().sink_attn_qkv_rope_append(
        _ptr(qkv), _ptr(bias), _ptr(rope_table), int(max_pos), _ptr(qo_indptr), _ptr(kv_len),
        _ptr(page_indptr), _ptr(page_indices), int(batch), int(num_qo_heads),
        int(num_kv_heads), int(head_dim), int(page_size), int(total_q), int(interleaved),
        _ptr(q_out), _ptr(k_pages), _ptr(v_pages), _stream(stream)))
