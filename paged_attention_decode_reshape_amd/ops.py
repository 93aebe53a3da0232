"""ctypes binding of libpagedattn.so: tensor checks and argument marshalling.

Names match the C entry points without their ``pa_`` prefix.  Each call
enqueues on the current torch stream of the tensors' device and returns
without synchronising.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Tuple

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpagedattn.so")

LAYOUT_SHUFFLED_KV = 0
LAYOUT_MLA_LATENT = 1
LAYOUT_STANDARD_KV = 2
# Bytes of the completion-counter region at the start of every workspace
# (PA_WORKSPACE_COUNTER_BYTES in the C header).
WORKSPACE_COUNTER_BYTES = 1 << 20
# Bytes of the per-device array paged_decode_attn_write_noalloc works in
# (PA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 32 << 20
_BF16, _F32 = 0, 1

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "workspace too small",
           4: "HIP error"}


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} (status {status})")
        self.status = status


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

_SIGS = {
    "pa_status_string": ([_i32], ctypes.c_char_p),
    "pa_reshape_and_cache": ([_i32, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _vp], _i32),
    "pa_decode_partition_tokens": ([_i32, _i32, _i32, _i32], _i32),
    "pa_decode_uses_balanced_split": ([_i32, _i32, _i32, _i32], _i32),
    "pa_decode_workspace_size": ([_i32, _i32, _i32, _i32, _i32, _i32], _sz),
    "pa_paged_decode_attn": ([_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                              _i32, _i32, _i64, _f32, _i32, _vp, _sz, _vp], _i32),
    "pa_paged_decode_attn_write": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                    _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32, _i32, _vp,
                                    _sz, _vp], _i32),
    "pa_paged_decode_attn_write_noalloc": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                            _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32,
                                            _i32, _vp], _i32),
    "pa_paged_decode_attn_layout": ([_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                     _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32, _i32,
                                     _vp, _sz, _vp], _i32),
    "pa_mla_workspace_size": ([_i32, _i32, _i32, _i32, _i32], _sz),
    "pa_mla_decode_attn": ([_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                            _i32, _i64, _f32, _i32, _vp, _sz, _vp], _i32),
    "pa_mla_decode_attn_write": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                  _i32, _i32, _i32, _i64, _f32, _i32, _vp, _sz, _vp], _i32),
    "pa_mla_decode_attn_mfma": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                 _i32, _i32, _i32, _i64, _f32, _i32, _vp, _sz, _vp], _i32),
    "pa_merge_attn_states": ([_vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _vp],
                             _i32),
    "pa_gather_cache_chunk": ([_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i64,
                               _i32, _i32, _vp], _i32),
    "pa_extend_chunk_tokens": ([_i32, _i32, _i32], _i32),
    "pa_extend_workspace_size": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32], _sz),
    "pa_chunked_extend_attn": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                                _i32, _i32, _i32, _i32, _i32, _i64, _f32, _i32, _vp, _sz, _vp],
                               _i32),
    "pa_stream_read": ([_vp, _sz, _vp, _i32, _i32, _vp], _i32),
    "pa_gather_read": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _vp, _i32, _vp],
                       _i32),
    "pa_reshape_and_cache_fp8": ([_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _f32,
                                  _f32, _vp], _i32),
    "pa_paged_decode_attn_fp8": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                  _i32, _i32, _i32, _i32, _i32, _i64, _f32, _f32, _f32, _i32,
                                  _vp, _sz, _vp], _i32),
    "pa_gather_cache_chunk_fp8": ([_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                   _i64, _i32, _i32, _f32, _f32, _vp], _i32),
    "pa_reshape_and_cache_mla_fp8": ([_vp, _vp, _vp, _i64, _i32, _i32, _i64, _f32, _vp], _i32),
    "pa_mla_decode_attn_fp8": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                _i32, _i32, _i32, _i64, _f32, _f32, _i32, _vp, _sz, _vp], _i32),
    "pa_mla_decode_attn_fp8_mfma": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                     _i32, _i32, _i32, _i32, _i64, _f32, _f32, _i32, _vp, _sz,
                                     _vp], _i32),
    "pa_mixed_batch_plan": ([_i32, _vp, _vp, _vp, _vp], _i32),
    "pa_mixed_batch_workspace_size": ([_i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32], _sz),
    "pa_mixed_batch_attn": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32, _i32, _vp, _sz,
                             _vp], _i32),
}

# Entries that only compute on the host (sizes, plans, strings); every other
# entry enqueues work on a stream.
_HOST_ONLY = {"pa_status_string", "pa_decode_partition_tokens", "pa_decode_uses_balanced_split",
              "pa_decode_workspace_size", "pa_mla_workspace_size", "pa_extend_workspace_size",
              "pa_extend_chunk_tokens", "pa_mixed_batch_plan", "pa_mixed_batch_workspace_size"}

_lib = None
_tls = threading.local()  # .capture: the prepare() record in progress, if any


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run "
                               "`python -m paged_attention_decode_reshape_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
    return _lib


class _Capture:
    """Stands in for the library while prepare() runs a wrapper: host-only
    entries run, the one enqueuing entry is recorded instead of called."""

    def __init__(self, lib):
        self.lib = lib
        self.calls = []
        self.keep = []  # objects the recorded pointers point into

    def __getattr__(self, name):
        if name in _HOST_ONLY:
            return getattr(self.lib, name)
        f = getattr(self.lib, name)

        def record(*args):
            self.calls.append((name, f, args))
            return 0
        return record


def library():
    """The loaded libpagedattn.so; raises if it has not been built."""
    lib = _load()
    cap = getattr(_tls, "capture", None)
    return cap if cap is not None else lib


def _keep(obj):
    """Keep obj alive for as long as a prepared call that points into it."""
    cap = getattr(_tls, "capture", None)
    if cap is not None:
        cap.keep.append(obj)
    return obj


class PreparedCall:
    """One library call whose arguments were checked and marshalled once by
    prepare(); calling it enqueues the same work again, on the same tensors
    and the stream that was current when it was prepared, and returns what
    the wrapper returned (e.g. the (out, lse) it writes)."""

    def __init__(self, name, fn, args, keep, result):
        self.name = name
        self._fn = fn
        self._args = tuple(None if a is None else t(a) for t, a in zip(fn.argtypes, args))
        self._keep = keep
        self.result = result

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise PagedAttnError(self.name[3:] if self.name.startswith("pa_") else self.name, st)
        return self.result


def prepare(wrapper, *args, **kwargs) -> PreparedCall:
    """Run a wrapper of this module (e.g. paged_decode_attn_write) once for
    its checks, sizing and marshalling, without enqueuing anything; returns a
    PreparedCall that enqueues that call each time it is called.  Tensors the
    caller passes must stay alive and keep their storage while the prepared
    call is used; outputs and workspaces the wrapper allocates are kept by
    the PreparedCall."""
    cap = _Capture(_load())
    _tls.capture = cap
    try:
        result = wrapper(*args, **kwargs)
    finally:
        _tls.capture = None
    if len(cap.calls) != 1:
        raise ValueError(f"prepare() needs a wrapper that makes exactly one enqueuing call, "
                         f"got {len(cap.calls)}")
    name, fn, cargs = cap.calls[0]
    return PreparedCall(name, fn, cargs, cap.keep + [result], result)


def _check(fn: str, status: int):
    if status != 0:
        raise PagedAttnError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _gpu(name: str, t: torch.Tensor, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (no CPU path exists)")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


# Shape checks.  The C ABI receives bare pointers, so every tensor's shape is
# checked against the sizes passed with it before anything is launched.

def _shape(name: str, t: Optional[torch.Tensor], shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")


def _shuffled_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, D: int, x: int):
    """Shuffled caches for head_dim D with x elements per 16 bytes:
    k_cache [NB, Hkv, D/x, B, x], v_cache [NB, Hkv, B/x, D, x]; returns
    (NB, Hkv, B)."""
    NB, Hkv, _, B, _ = k_cache.shape
    if D % x or B % x:
        raise ValueError(f"head_dim {D} and block size {B} must be multiples of {x}")
    _shape("k_cache", k_cache, (NB, Hkv, D // x, B, x))
    _shape("v_cache", v_cache, (NB, Hkv, B // x, D, x))
    return NB, Hkv, B


def _batch(S: int, block_table: torch.Tensor, context_lens: torch.Tensor):
    if block_table.shape[0] < S:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for {S} sequences")
    if block_table.shape[1] < 1:
        raise ValueError("block_table needs at least one column")
    if context_lens.numel() != S:
        raise ValueError(f"context_lens has {context_lens.numel()} entries for {S} sequences")


def _new_tokens(S: int, Hkv: int, D: int, new_key, new_value, slot_mapping):
    _shape("new_key", new_key, (S, Hkv, D))
    _shape("new_value", new_value, (S, Hkv, D))
    if slot_mapping is not None and slot_mapping.numel() != S:
        raise ValueError("slot_mapping must hold one slot per sequence")


def _overlap(a: torch.Tensor, b: torch.Tensor) -> bool:
    """a and b share a byte of device memory."""
    if a.device != b.device:
        return False
    a0, b0 = a.data_ptr(), b.data_ptr()
    an, bn = a.numel() * a.element_size(), b.numel() * b.element_size()
    return an > 0 and bn > 0 and a0 < b0 + bn and b0 < a0 + an


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    """A caller-supplied workspace, or a fresh zero-filled one.  Every
    workspace starts with a fixed region of completion counters
    (``WORKSPACE_COUNTER_BYTES``) that must be zero before its first use;
    every call leaves the region zero and keeps its other data after it, so
    one workspace, zero-filled once and at least as large as each call's size
    query, can be reused across calls of any shape and any entry point on
    one stream."""
    if nbytes == 0:
        return None
    if workspace is None:
        return _keep(torch.zeros(nbytes, dtype=torch.uint8, device=device))
    _gpu("workspace", workspace)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace


# ---------------------------------------------------------------------------

def reshape_and_cache(key: torch.Tensor, value: Optional[torch.Tensor], k_cache: torch.Tensor,
                      v_cache: Optional[torch.Tensor], slot_mapping: torch.Tensor,
                      layout: int = LAYOUT_SHUFFLED_KV) -> None:
    """Write new tokens into the paged cache.

    Shuffled: key/value [T, Hkv, D] bf16, k_cache [NB, Hkv, D/8, B, 8],
    v_cache [NB, Hkv, B/8, D, 8].  Standard (kept for comparison): k_cache,
    v_cache [NB, B, Hkv, D].  MLA latent: key [T, Dl], value None,
    k_cache [NB, B, Dl], v_cache None.  slot_mapping [T] int64.
    """
    lib = library()
    _gpu("slot_mapping", slot_mapping, torch.int64, 1)
    if layout == LAYOUT_SHUFFLED_KV:
        _gpu("key", key, torch.bfloat16, 3)
        _gpu("value", value, torch.bfloat16, 3)
        _gpu("k_cache", k_cache, torch.bfloat16, 5)
        _gpu("v_cache", v_cache, torch.bfloat16, 5)
        T, Hkv, D = key.shape
        NB, B = k_cache.shape[0], k_cache.shape[3]
        if (value.shape != key.shape or tuple(k_cache.shape) != (NB, Hkv, D // 8, B, 8)
                or tuple(v_cache.shape) != (NB, Hkv, B // 8, D, 8)):
            raise ValueError("cache shapes do not match key/value")
        vptr, vcptr = value.data_ptr(), v_cache.data_ptr()
    elif layout == LAYOUT_STANDARD_KV:
        _gpu("key", key, torch.bfloat16, 3)
        _gpu("value", value, torch.bfloat16, 3)
        _gpu("k_cache", k_cache, torch.bfloat16, 4)
        _gpu("v_cache", v_cache, torch.bfloat16, 4)
        T, Hkv, D = key.shape
        NB, B = k_cache.shape[0], k_cache.shape[1]
        if (value.shape != key.shape or tuple(k_cache.shape) != (NB, B, Hkv, D)
                or tuple(v_cache.shape) != (NB, B, Hkv, D)):
            raise ValueError("cache shapes do not match key/value")
        vptr, vcptr = value.data_ptr(), v_cache.data_ptr()
    elif layout == LAYOUT_MLA_LATENT:
        _gpu("key", key, torch.bfloat16, 2)
        _gpu("k_cache", k_cache, torch.bfloat16, 3)
        T, D = key.shape
        Hkv = 1
        NB, B = k_cache.shape[0], k_cache.shape[1]
        if k_cache.shape[2] != D or value is not None or v_cache is not None:
            raise ValueError("latent cache must be [NB, B, Dl]; value and v_cache must be None")
        vptr = vcptr = None
    else:
        raise ValueError(f"unknown layout {layout}")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must have one entry per token")
    st = lib.pa_reshape_and_cache(layout, key.data_ptr(), vptr, k_cache.data_ptr(), vcptr,
                                  slot_mapping.data_ptr(), T, Hkv, D, B, NB, _stream(key))
    _check("reshape_and_cache", st)


def decode_partition_tokens(num_seqs: int, num_kv_heads: int, max_context_len: int,
                            partition_tokens: int = 0) -> int:
    return int(library().pa_decode_partition_tokens(num_seqs, num_kv_heads, max_context_len,
                                                    partition_tokens))


def decode_uses_balanced_split(num_seqs: int, num_kv_heads: int, max_context_len: int,
                               partition_tokens: int = 0) -> bool:
    return bool(library().pa_decode_uses_balanced_split(num_seqs, num_kv_heads, max_context_len,
                                                        partition_tokens))


def decode_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          max_context_len: int, partition_tokens: int = 0) -> int:
    return int(library().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                  max_context_len, partition_tokens))


def paged_decode_attn(query: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                      max_context_len: int, partition_tokens: int = 0,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """GQA paged decode: query [S, Hq, D] bf16 -> (out [S, Hq, D] bf16, lse [S, Hq] f32)."""
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("k_cache", k_cache, torch.bfloat16, 5)
    _gpu("v_cache", v_cache, torch.bfloat16, 5)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    S, Hq, D = query.shape
    NB, Hkv, B = _shuffled_kv(k_cache, v_cache, D, 8)
    _batch(S, block_table, context_lens)
    if out is None:
        out = torch.empty_like(query)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (S, Hq, D))
    if lse is None and return_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=query.device)
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (S, Hq))
    nbytes = decode_workspace_size(S, Hq, Hkv, D, max_context_len, partition_tokens)
    ws = _workspace(nbytes, query.device, workspace)
    st = lib.pa_paged_decode_attn(out.data_ptr(), _ptr(lse), query.data_ptr(), k_cache.data_ptr(),
                                  v_cache.data_ptr(), block_table.data_ptr(), block_table.shape[1],
                                  context_lens.data_ptr(), int(max_context_len), S, Hq, Hkv, D, B,
                                  NB, float(scale), int(partition_tokens), _ptr(ws), nbytes,
                                  _stream(query))
    _check("paged_decode_attn", st)
    return out, lse


def paged_decode_attn_write(query: torch.Tensor, new_key: torch.Tensor, new_value: torch.Tensor,
                            slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, block_table: torch.Tensor,
                            context_lens: torch.Tensor, scale: float, max_context_len: int,
                            partition_tokens: int = 0, out: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                            workspace: Optional[torch.Tensor] = None
                            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One decode step in one launch: each sequence's new token (new_key,
    new_value [S, Hkv, D] bf16 at slot_mapping [S] int64) is written into the
    shuffled caches, then GQA paged decode runs over them."""
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("new_key", new_key, torch.bfloat16, 3)
    _gpu("new_value", new_value, torch.bfloat16, 3)
    _gpu("slot_mapping", slot_mapping, torch.int64, 1)
    _gpu("k_cache", k_cache, torch.bfloat16, 5)
    _gpu("v_cache", v_cache, torch.bfloat16, 5)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    S, Hq, D = query.shape
    NB, Hkv, B = _shuffled_kv(k_cache, v_cache, D, 8)
    _batch(S, block_table, context_lens)
    _new_tokens(S, Hkv, D, new_key, new_value, slot_mapping)
    if out is None:
        out = torch.empty_like(query)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (S, Hq, D))
    if lse is None and return_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=query.device)
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (S, Hq))
    nbytes = decode_workspace_size(S, Hq, Hkv, D, max_context_len, partition_tokens)
    ws = _workspace(nbytes, query.device, workspace)
    st = lib.pa_paged_decode_attn_write(out.data_ptr(), _ptr(lse), query.data_ptr(),
                                        new_key.data_ptr(), new_value.data_ptr(),
                                        slot_mapping.data_ptr(), k_cache.data_ptr(),
                                        v_cache.data_ptr(), block_table.data_ptr(),
                                        block_table.shape[1], context_lens.data_ptr(),
                                        int(max_context_len), S, Hq, Hkv, D, B, NB, float(scale),
                                        int(partition_tokens), _ptr(ws), nbytes, _stream(query))
    _check("paged_decode_attn_write", st)
    return out, lse


def paged_decode_attn_write_noalloc(query: torch.Tensor, new_key: torch.Tensor,
                                    new_value: torch.Tensor, slot_mapping: torch.Tensor,
                                    k_cache: torch.Tensor, v_cache: torch.Tensor,
                                    block_table: torch.Tensor, context_lens: torch.Tensor,
                                    scale: float, max_context_len: int, partition_tokens: int = 0,
                                    out: Optional[torch.Tensor] = None,
                                    lse: Optional[torch.Tensor] = None
                                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """paged_decode_attn_write with the workspace in the library's own
    per-device array (NOALLOC_SCRATCH_BYTES), for callers that cannot allocate
    device memory.  Pass `out` (and `lse`) to allocate nothing here either;
    calls that overlap in time on one device race."""
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("new_key", new_key, torch.bfloat16, 3)
    _gpu("new_value", new_value, torch.bfloat16, 3)
    _gpu("slot_mapping", slot_mapping, torch.int64, 1)
    _gpu("k_cache", k_cache, torch.bfloat16, 5)
    _gpu("v_cache", v_cache, torch.bfloat16, 5)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    S, Hq, D = query.shape
    NB, Hkv, B = _shuffled_kv(k_cache, v_cache, D, 8)
    _batch(S, block_table, context_lens)
    _new_tokens(S, Hkv, D, new_key, new_value, slot_mapping)
    if out is None:
        out = torch.empty_like(query)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (S, Hq, D))
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (S, Hq))
    st = lib.pa_paged_decode_attn_write_noalloc(
        out.data_ptr(), _ptr(lse), query.data_ptr(), new_key.data_ptr(), new_value.data_ptr(),
        slot_mapping.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
        block_table.shape[1], context_lens.data_ptr(), int(max_context_len), S, Hq, Hkv, D, B, NB,
        float(scale), int(partition_tokens), _stream(query))
    _check("paged_decode_attn_write_noalloc", st)
    return out, lse


def paged_decode_attn_layout(layout: int, query: torch.Tensor, k_cache: torch.Tensor,
                             v_cache: torch.Tensor, block_table: torch.Tensor,
                             context_lens: torch.Tensor, scale: float, max_context_len: int,
                             partition_tokens: int = 0, new_key: Optional[torch.Tensor] = None,
                             new_value: Optional[torch.Tensor] = None,
                             slot_mapping: Optional[torch.Tensor] = None,
                             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                             return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                             ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """GQA paged decode over caches in `layout` (LAYOUT_SHUFFLED_KV or
    LAYOUT_STANDARD_KV [NB, B, Hkv, D]), with the fused write of each
    sequence's new token when new_key / new_value / slot_mapping are given."""
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    S, Hq, D = query.shape
    if layout == LAYOUT_STANDARD_KV:
        _gpu("k_cache", k_cache, torch.bfloat16, 4)
        _gpu("v_cache", v_cache, torch.bfloat16, 4)
        NB, B, Hkv, _ = k_cache.shape
        if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[3] != D:
            raise ValueError("standard caches must both be [NB, B, Hkv, head_dim]")
    elif layout == LAYOUT_SHUFFLED_KV:
        _gpu("k_cache", k_cache, torch.bfloat16, 5)
        _gpu("v_cache", v_cache, torch.bfloat16, 5)
        NB, Hkv, B = _shuffled_kv(k_cache, v_cache, D, 8)
    else:
        raise ValueError(f"unsupported layout {layout}")
    _batch(S, block_table, context_lens)
    given = [t is not None for t in (new_key, new_value, slot_mapping)]
    if any(given) and not all(given):
        raise ValueError("new_key, new_value and slot_mapping go together")
    if all(given):
        _gpu("new_key", new_key, torch.bfloat16, 3)
        _gpu("new_value", new_value, torch.bfloat16, 3)
        _gpu("slot_mapping", slot_mapping, torch.int64, 1)
        _new_tokens(S, Hkv, D, new_key, new_value, slot_mapping)
    if out is None:
        out = torch.empty_like(query)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (S, Hq, D))
    if lse is None and return_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=query.device)
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (S, Hq))
    nbytes = decode_workspace_size(S, Hq, Hkv, D, max_context_len, partition_tokens)
    ws = _workspace(nbytes, query.device, workspace)
    st = lib.pa_paged_decode_attn_layout(int(layout), out.data_ptr(), _ptr(lse), query.data_ptr(),
                                         _ptr(new_key), _ptr(new_value), _ptr(slot_mapping),
                                         k_cache.data_ptr(), v_cache.data_ptr(),
                                         block_table.data_ptr(), block_table.shape[1],
                                         context_lens.data_ptr(), int(max_context_len), S, Hq,
                                         Hkv, D, B, NB, float(scale), int(partition_tokens),
                                         _ptr(ws), nbytes, _stream(query))
    _check("paged_decode_attn_layout", st)
    return out, lse


def mla_workspace_size(num_seqs: int, num_q_heads: int, v_dim: int, max_context_len: int,
                       partition_tokens: int = 0) -> int:
    return int(library().pa_mla_workspace_size(num_seqs, num_q_heads, v_dim, max_context_len,
                                               partition_tokens))


def mla_decode_attn(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                    context_lens: torch.Tensor, scale: float, max_context_len: int,
                    v_dim: int = 512, partition_tokens: int = 0,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Absorbed MLA decode: query [S, Hq, Dl] -> (out [S, Hq, v_dim], lse [S, Hq])."""
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("kv_cache", kv_cache, torch.bfloat16, 3)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    S, Hq, Dl = query.shape
    NB, B, Dl2 = kv_cache.shape
    if Dl2 != Dl:
        raise ValueError("kv_cache latent width differs from the query's")
    _batch(S, block_table, context_lens)
    if out is None:
        out = torch.empty((S, Hq, v_dim), dtype=torch.bfloat16, device=query.device)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (S, Hq, v_dim))
    if lse is None and return_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=query.device)
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (S, Hq))
    nbytes = mla_workspace_size(S, Hq, v_dim, max_context_len, partition_tokens)
    ws = _workspace(nbytes, query.device, workspace)
    st = lib.pa_mla_decode_attn(out.data_ptr(), _ptr(lse), query.data_ptr(), kv_cache.data_ptr(),
                                block_table.data_ptr(), block_table.shape[1],
                                context_lens.data_ptr(), int(max_context_len), S, Hq, Dl, v_dim, B,
                                NB, float(scale), int(partition_tokens), _ptr(ws), nbytes,
                                _stream(query))
    _check("mla_decode_attn", st)
    return out, lse


def mla_decode_attn_write(query: torch.Tensor, new_latent: torch.Tensor,
                          slot_mapping: torch.Tensor, kv_cache: torch.Tensor,
                          block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                          max_context_len: int, v_dim: int = 512, partition_tokens: int = 0,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One MLA decode step in one launch: each sequence's new latent
    (new_latent [S, Dl] bf16 at slot_mapping [S] int64) is written into the
    latent cache, then absorbed MLA decode runs over it."""
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("new_latent", new_latent, torch.bfloat16, 2)
    _gpu("slot_mapping", slot_mapping, torch.int64, 1)
    _gpu("kv_cache", kv_cache, torch.bfloat16, 3)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    S, Hq, Dl = query.shape
    NB, B, Dl2 = kv_cache.shape
    if Dl2 != Dl or tuple(new_latent.shape) != (S, Dl):
        raise ValueError("new_latent must be [num_seqs, latent_dim] of the cache's width")
    if slot_mapping.numel() != S:
        raise ValueError("slot_mapping must hold one slot per sequence")
    _batch(S, block_table, context_lens)
    if out is None:
        out = torch.empty((S, Hq, v_dim), dtype=torch.bfloat16, device=query.device)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (S, Hq, v_dim))
    if lse is None and return_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=query.device)
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (S, Hq))
    nbytes = mla_workspace_size(S, Hq, v_dim, max_context_len, partition_tokens)
    ws = _workspace(nbytes, query.device, workspace)
    st = lib.pa_mla_decode_attn_write(out.data_ptr(), _ptr(lse), query.data_ptr(),
                                      new_latent.data_ptr(), slot_mapping.data_ptr(),
                                      kv_cache.data_ptr(), block_table.data_ptr(),
                                      block_table.shape[1], context_lens.data_ptr(),
                                      int(max_context_len), S, Hq, Dl, v_dim, B, NB, float(scale),
                                      int(partition_tokens), _ptr(ws), nbytes, _stream(query))
    _check("mla_decode_attn_write", st)
    return out, lse


def mla_decode_attn_mfma(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                         context_lens: torch.Tensor, scale: float, max_context_len: int,
                         v_dim: int = 512, partition_tokens: int = 0,
                         new_latent: Optional[torch.Tensor] = None,
                         slot_mapping: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                         ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Absorbed MLA decode on the matrix cores (same result as mla_decode_attn
    to rounding), with the fused latent write when new_latent and
    slot_mapping are given."""
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("kv_cache", kv_cache, torch.bfloat16, 3)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    S, Hq, Dl = query.shape
    NB, B, Dl2 = kv_cache.shape
    if Dl2 != Dl:
        raise ValueError("kv_cache latent width differs from the query's")
    if (new_latent is None) != (slot_mapping is None):
        raise ValueError("new_latent and slot_mapping go together")
    if new_latent is not None:
        _gpu("new_latent", new_latent, torch.bfloat16, 2)
        _gpu("slot_mapping", slot_mapping, torch.int64, 1)
        if tuple(new_latent.shape) != (S, Dl) or slot_mapping.numel() != S:
            raise ValueError("new_latent [num_seqs, latent_dim] and one slot per sequence")
    _batch(S, block_table, context_lens)
    if out is None:
        out = torch.empty((S, Hq, v_dim), dtype=torch.bfloat16, device=query.device)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (S, Hq, v_dim))
    if lse is None and return_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=query.device)
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (S, Hq))
    nbytes = mla_workspace_size(S, Hq, v_dim, max_context_len, partition_tokens)
    ws = _workspace(nbytes, query.device, workspace)
    st = lib.pa_mla_decode_attn_mfma(out.data_ptr(), _ptr(lse), query.data_ptr(),
                                     _ptr(new_latent), _ptr(slot_mapping), kv_cache.data_ptr(),
                                     block_table.data_ptr(), block_table.shape[1],
                                     context_lens.data_ptr(), int(max_context_len), S, Hq, Dl,
                                     v_dim, B, NB, float(scale), int(partition_tokens), _ptr(ws),
                                     nbytes, _stream(query))
    _check("mla_decode_attn_mfma", st)
    return out, lse


def merge_attn_states(prefix_out: torch.Tensor, prefix_lse: torch.Tensor,
                      suffix_out: torch.Tensor, suffix_lse: torch.Tensor,
                      out: Optional[torch.Tensor] = None, out_lse: Optional[torch.Tensor] = None,
                      out_dtype: Optional[torch.dtype] = None, return_lse: bool = True
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """LSE merge of two partial results [T, H, D] (bf16 or f32) with lse [T, H] f32."""
    lib = library()
    dt = prefix_out.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise ValueError("outputs must be bf16 or f32")
    _gpu("prefix_out", prefix_out, dt, 3)
    _gpu("suffix_out", suffix_out, dt, 3)
    _gpu("prefix_lse", prefix_lse, torch.float32, 2)
    _gpu("suffix_lse", suffix_lse, torch.float32, 2)
    T, H, D = prefix_out.shape
    if suffix_out.shape != prefix_out.shape or prefix_lse.shape != (T, H) or \
            suffix_lse.shape != (T, H):
        raise ValueError("shape mismatch")
    odt = out_dtype or (out.dtype if out is not None else dt)
    if out is None:
        out = torch.empty((T, H, D), dtype=odt, device=prefix_out.device)
    _gpu("out", out, odt, 3)
    _shape("out", out, (T, H, D))
    if out_lse is None and return_lse:
        out_lse = torch.empty((T, H), dtype=torch.float32, device=prefix_out.device)
    if out_lse is not None:
        _gpu("out_lse", out_lse, torch.float32, 2)
        _shape("out_lse", out_lse, (T, H))
        for name, t in (("prefix_lse", prefix_lse), ("suffix_lse", suffix_lse),
                        ("prefix_out", prefix_out), ("suffix_out", suffix_out), ("out", out)):
            if _overlap(out_lse, t):
                raise ValueError(f"out_lse must not overlap {name}")
    for name, t in (("prefix_out", prefix_out), ("suffix_out", suffix_out)):
        same = out.data_ptr() == t.data_ptr() and out.dtype == t.dtype
        if not same and _overlap(out, t):
            raise ValueError(f"out may be {name} itself but must not partly overlap it")
    for name, t in (("prefix_lse", prefix_lse), ("suffix_lse", suffix_lse)):
        if _overlap(out, t):
            raise ValueError(f"out must not overlap {name}")
    code = {torch.bfloat16: _BF16, torch.float32: _F32}
    st = lib.pa_merge_attn_states(out.data_ptr(), _ptr(out_lse), code[odt], prefix_out.data_ptr(),
                                  prefix_lse.data_ptr(), suffix_out.data_ptr(),
                                  suffix_lse.data_ptr(), code[dt], T, H, D, _stream(prefix_out))
    _check("merge_attn_states", st)
    return out, out_lse


def gather_cache_chunk(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                       context_lens: torch.Tensor, iteration: int, chunk_tokens: int,
                       k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None
                       ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Copy every request's context tokens [iteration * chunk_tokens, +chunk_tokens)
    out of the shuffled caches into standard [rows, kv_heads, head_dim] tensors
    (requests one after another; rows <= num_seqs * chunk_tokens)."""
    lib = library()
    _gpu("k_cache", k_cache, torch.bfloat16, 5)
    _gpu("v_cache", v_cache, torch.bfloat16, 5)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    NB, Hkv, C, B, x = k_cache.shape
    D = C * x
    _shuffled_kv(k_cache, v_cache, D, 8)
    S = context_lens.shape[0]
    _batch(S, block_table, context_lens)
    rows = S * chunk_tokens
    if k_out is None:
        k_out = torch.empty((rows, Hkv, D), dtype=torch.bfloat16, device=k_cache.device)
    if v_out is None:
        v_out = torch.empty((rows, Hkv, D), dtype=torch.bfloat16, device=k_cache.device)
    _gpu("k_out", k_out, torch.bfloat16, 3)
    _gpu("v_out", v_out, torch.bfloat16, 3)
    if k_out.shape[0] < rows or v_out.shape[0] < rows:
        raise ValueError("output tensors need num_seqs * chunk_tokens rows")
    if tuple(k_out.shape[1:]) != (Hkv, D) or tuple(v_out.shape[1:]) != (Hkv, D):
        raise ValueError(f"k_out / v_out must be [rows, {Hkv}, {D}]")
    st = lib.pa_gather_cache_chunk(k_out.data_ptr(), v_out.data_ptr(), k_cache.data_ptr(),
                                   v_cache.data_ptr(), block_table.data_ptr(),
                                   block_table.shape[1], context_lens.data_ptr(), S, Hkv, D, B, NB,
                                   int(iteration), int(chunk_tokens), _stream(k_cache))
    _check("gather_cache_chunk", st)
    return k_out, v_out


def extend_chunk_tokens(num_seqs: int, block_size: int, chunk_budget_tokens: int) -> int:
    return int(library().pa_extend_chunk_tokens(num_seqs, block_size, chunk_budget_tokens))


def extend_workspace_size(num_seqs: int, total_new_tokens: int, num_q_heads: int,
                          num_kv_heads: int, head_dim: int, block_size: int,
                          chunk_budget_tokens: int) -> int:
    return int(library().pa_extend_workspace_size(num_seqs, total_new_tokens, num_q_heads,
                                                  num_kv_heads, head_dim, block_size,
                                                  chunk_budget_tokens))


def chunked_extend_attn(query: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        query_start_loc: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, block_table: torch.Tensor,
                        context_lens: torch.Tensor, scale: float, query_start_loc_host,
                        context_lens_host, chunk_budget_tokens: int = 32768,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked extend: query [Tn, Hq, D], k_new/v_new [Tn, Hkv, D] -> (out, lse).

    ``query_start_loc_host`` and ``context_lens_host`` are host copies (lists
    or CPU int32 tensors/arrays) of the device tensors, used to plan chunks.
    """
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("k_new", k_new, torch.bfloat16, 3)
    _gpu("v_new", v_new, torch.bfloat16, 3)
    _gpu("query_start_loc", query_start_loc, torch.int32, 1)
    _gpu("k_cache", k_cache, torch.bfloat16, 5)
    _gpu("v_cache", v_cache, torch.bfloat16, 5)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    Tn, Hq, D = query.shape
    NB, Hkv, B = _shuffled_kv(k_cache, v_cache, D, 8)
    S = context_lens.shape[0]
    _batch(S, block_table, context_lens)
    _shape("k_new", k_new, (Tn, Hkv, D))
    _shape("v_new", v_new, (Tn, Hkv, D))
    if query_start_loc.numel() != S + 1:
        raise ValueError("query_start_loc needs num_seqs + 1 entries")
    qsl_h = _keep(torch.as_tensor(query_start_loc_host, dtype=torch.int32).contiguous())
    cl_h = _keep(torch.as_tensor(context_lens_host, dtype=torch.int32).contiguous())
    if qsl_h.device.type != "cpu" or cl_h.device.type != "cpu":
        raise ValueError("host copies must be on the CPU")
    if qsl_h.numel() != S + 1 or cl_h.numel() != S:
        raise ValueError("host copies have the wrong length")
    if int(qsl_h[-1]) != Tn:
        raise ValueError(f"query_start_loc_host ends at {int(qsl_h[-1])}, query has {Tn} rows")
    if out is None:
        out = torch.empty_like(query)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (Tn, Hq, D))
    if lse is None and return_lse:
        lse = torch.empty((Tn, Hq), dtype=torch.float32, device=query.device)
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (Tn, Hq))
    nbytes = extend_workspace_size(S, Tn, Hq, Hkv, D, B, chunk_budget_tokens)
    ws = _workspace(nbytes, query.device, workspace)
    st = lib.pa_chunked_extend_attn(out.data_ptr(), _ptr(lse), query.data_ptr(), k_new.data_ptr(),
                                    v_new.data_ptr(), query_start_loc.data_ptr(),
                                    qsl_h.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                    block_table.data_ptr(), block_table.shape[1],
                                    context_lens.data_ptr(), cl_h.data_ptr(), S, Hq, Hkv, D, B, NB,
                                    float(scale), int(chunk_budget_tokens), _ptr(ws), nbytes,
                                    _stream(query))
    _check("chunked_extend_attn", st)
    return out, lse


def stream_read(src: torch.Tensor, workgroups: int, sink: Optional[torch.Tensor] = None,
                verify: bool = True) -> torch.Tensor:
    """Read every byte of `src` once with the library's plain streaming-read
    kernel (a bandwidth yardstick, not part of attention); with `verify` the
    per-workgroup xor words are stored in the returned sink (otherwise a word
    is stored only if it is all ones, for timing)."""
    lib = library()
    _gpu("src", src)
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(workgroups, dtype=torch.int32, device=src.device)
    _gpu("sink", sink, torch.int32, 1)
    if sink.numel() < workgroups:
        raise ValueError("sink needs one word per workgroup")
    _check("stream_read", lib.pa_stream_read(src.data_ptr(), nbytes, sink.data_ptr(),
                                             int(workgroups), int(bool(verify)), _stream(src)))
    return sink


def gather_read(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                context_lens: torch.Tensor, sink: Optional[torch.Tensor] = None,
                verify: bool = True) -> torch.Tensor:
    """Read the K and V blocks that a decode over the preshuffled cache reads
    (every kv head's unit of each block holding a sequence's context),
    through the block table, with no arithmetic: the library's gather-read
    kernel (a bandwidth yardstick, not part of attention).  Caches
    [num_blocks, kv_heads, ...] of either preshuffled shape; with `verify`
    the per-workgroup xor words are stored in the returned sink."""
    lib = library()
    _gpu("k_cache", k_cache)
    _gpu("v_cache", v_cache)
    if k_cache.shape[:2] != v_cache.shape[:2] or k_cache.numel() != v_cache.numel():
        raise ValueError("k_cache and v_cache must hold the same units")
    if k_cache.dim() != 5 or not k_cache.is_contiguous() or not v_cache.is_contiguous():
        raise ValueError("caches must be contiguous [num_blocks, kv_heads, a, b, x] tensors")
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    NB, Hkv = int(k_cache.shape[0]), int(k_cache.shape[1])
    B = int(k_cache.shape[3])
    unit = (k_cache.numel() // (NB * Hkv)) * k_cache.element_size()
    S, maxb = int(context_lens.shape[0]), int(block_table.shape[1])
    if block_table.shape[0] < S:
        raise ValueError("block_table needs a row per sequence")
    words = S * Hkv * ((maxb + 3) // 4)
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=k_cache.device)
    _gpu("sink", sink, torch.int32, 1)
    if sink.numel() < words:
        raise ValueError("sink needs one word per workgroup")
    _check("gather_read", lib.pa_gather_read(k_cache.data_ptr(), v_cache.data_ptr(),
                                             block_table.data_ptr(), context_lens.data_ptr(), S,
                                             Hkv, maxb, B, NB, int(unit), sink.data_ptr(),
                                             int(bool(verify)), _stream(k_cache)))
    return sink


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def mixed_batch_plan(query_start_loc_host, context_lens_host) -> Tuple[np.ndarray, np.ndarray]:
    """Host routing of a mixed batch: (order, counts) with order the request
    indices in [decode : extend : prefill] order and counts the three sizes."""
    qsl = _host_i32(query_start_loc_host)
    ctx = _host_i32(context_lens_host)
    R = ctx.shape[0]
    if qsl.shape[0] != R + 1:
        raise ValueError("query_start_loc needs num_reqs + 1 entries")
    order = np.zeros(R, dtype=np.int32)
    counts = np.zeros(3, dtype=np.int32)
    _check("mixed_batch_plan", library().pa_mixed_batch_plan(
        R, qsl.ctypes.data, ctx.ctypes.data, order.ctypes.data, counts.ctypes.data))
    return order, counts


def mixed_batch_attn(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                     slot_mapping: torch.Tensor, query_start_loc: torch.Tensor,
                     context_lens: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     block_table: torch.Tensor, scale: float, query_start_loc_host,
                     context_lens_host, chunk_budget_tokens: int = 32768,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                     ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention of a mixed batch in [decode : extend : prefill] order: the
    new tokens' cache write, then the decode, extend and prefill paths."""
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("key", key, torch.bfloat16, 3)
    _gpu("value", value, torch.bfloat16, 3)
    _gpu("slot_mapping", slot_mapping, torch.int64, 1)
    _gpu("query_start_loc", query_start_loc, torch.int32, 1)
    _gpu("context_lens", context_lens, torch.int32, 1)
    _gpu("k_cache", k_cache, torch.bfloat16, 5)
    _gpu("v_cache", v_cache, torch.bfloat16, 5)
    _gpu("block_table", block_table, torch.int32, 2)
    qsl_h = _keep(_host_i32(query_start_loc_host))
    ctx_h = _keep(_host_i32(context_lens_host))
    R = ctx_h.shape[0]
    T, Hq, D = query.shape
    NB, Hkv, B = _shuffled_kv(k_cache, v_cache, D, 8)
    if qsl_h.shape[0] != R + 1 or int(qsl_h[-1]) != T or block_table.shape[0] != R:
        raise ValueError("batch arrays disagree")
    _batch(R, block_table, context_lens)
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc needs num_reqs + 1 entries")
    _shape("key", key, (T, Hkv, D))
    _shape("value", value, (T, Hkv, D))
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must hold one slot per new token")
    if out is None:
        out = torch.empty_like(query)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (T, Hq, D))
    if lse is None and return_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=query.device)
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (T, Hq))
    nbytes = int(lib.pa_mixed_batch_workspace_size(R, qsl_h.ctypes.data, ctx_h.ctypes.data, Hq,
                                                   Hkv, D, B, int(chunk_budget_tokens)))
    ws = _workspace(nbytes, query.device, workspace)
    st = lib.pa_mixed_batch_attn(out.data_ptr(), _ptr(lse), query.data_ptr(), key.data_ptr(),
                                 value.data_ptr(), slot_mapping.data_ptr(),
                                 query_start_loc.data_ptr(), qsl_h.ctypes.data,
                                 context_lens.data_ptr(), ctx_h.ctypes.data, k_cache.data_ptr(),
                                 v_cache.data_ptr(), block_table.data_ptr(), block_table.shape[1],
                                 R, Hq, Hkv, D, B, NB, float(scale), int(chunk_budget_tokens),
                                 _ptr(ws), nbytes, _stream(query))
    _check("mixed_batch_attn", st)
    return out, lse


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV cache: uint8 codes, x = 16 shuffled layout, per-tensor scales

def reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float,
                          v_scale: float) -> None:
    """Quantise key/value [T, Hkv, D] bf16 into k_cache [NB, Hkv, D/16, B, 16] and
    v_cache [NB, Hkv, B/16, D, 16] (uint8 E4M3 codes)."""
    lib = library()
    _gpu("key", key, torch.bfloat16, 3)
    _gpu("value", value, torch.bfloat16, 3)
    _gpu("k_cache", k_cache, torch.uint8, 5)
    _gpu("v_cache", v_cache, torch.uint8, 5)
    _gpu("slot_mapping", slot_mapping, torch.int64, 1)
    T, Hkv, D = key.shape
    NB, B = k_cache.shape[0], k_cache.shape[3]
    if (value.shape != key.shape or tuple(k_cache.shape) != (NB, Hkv, D // 16, B, 16)
            or tuple(v_cache.shape) != (NB, Hkv, B // 16, D, 16) or slot_mapping.numel() != T):
        raise ValueError("fp8 cache shapes do not match key/value")
    _check("reshape_and_cache_fp8", lib.pa_reshape_and_cache_fp8(
        key.data_ptr(), value.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        slot_mapping.data_ptr(), T, Hkv, D, B, NB, float(k_scale), float(v_scale), _stream(key)))


def paged_decode_attn_fp8(query: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                          max_context_len: int, k_scale: float, v_scale: float,
                          partition_tokens: int = 0, new_key: Optional[torch.Tensor] = None,
                          new_value: Optional[torch.Tensor] = None,
                          slot_mapping: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """GQA paged decode over FP8 caches (K = code * k_scale, V = code * v_scale),
    with the fused quantised write when new_key / new_value / slot_mapping are given."""
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("k_cache", k_cache, torch.uint8, 5)
    _gpu("v_cache", v_cache, torch.uint8, 5)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    S, Hq, D = query.shape
    NB, Hkv, B = _shuffled_kv(k_cache, v_cache, D, 16)
    _batch(S, block_table, context_lens)
    given = [t is not None for t in (new_key, new_value, slot_mapping)]
    if any(given) and not all(given):
        raise ValueError("new_key, new_value and slot_mapping go together")
    if all(given):
        _gpu("new_key", new_key, torch.bfloat16, 3)
        _gpu("new_value", new_value, torch.bfloat16, 3)
        _gpu("slot_mapping", slot_mapping, torch.int64, 1)
        _new_tokens(S, Hkv, D, new_key, new_value, slot_mapping)
    if out is None:
        out = torch.empty_like(query)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (S, Hq, D))
    if lse is None and return_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=query.device)
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (S, Hq))
    nbytes = decode_workspace_size(S, Hq, Hkv, D, max_context_len, partition_tokens)
    ws = _workspace(nbytes, query.device, workspace)
    st = lib.pa_paged_decode_attn_fp8(out.data_ptr(), _ptr(lse), query.data_ptr(), _ptr(new_key),
                                      _ptr(new_value), _ptr(slot_mapping), k_cache.data_ptr(),
                                      v_cache.data_ptr(), block_table.data_ptr(),
                                      block_table.shape[1], context_lens.data_ptr(),
                                      int(max_context_len), S, Hq, Hkv, D, B, NB, float(scale),
                                      float(k_scale), float(v_scale), int(partition_tokens),
                                      _ptr(ws), nbytes, _stream(query))
    _check("paged_decode_attn_fp8", st)
    return out, lse


def gather_cache_chunk_fp8(k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_table: torch.Tensor, context_lens: torch.Tensor, iteration: int,
                           chunk_tokens: int, k_scale: float, v_scale: float,
                           k_out: Optional[torch.Tensor] = None,
                           v_out: Optional[torch.Tensor] = None
                           ) -> Tuple[torch.Tensor, torch.Tensor]:
    """gather_cache_chunk over FP8 caches: dequantised bf16 [rows, Hkv, D] outputs."""
    lib = library()
    _gpu("k_cache", k_cache, torch.uint8, 5)
    _gpu("v_cache", v_cache, torch.uint8, 5)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    NB, Hkv, C, B, x = k_cache.shape
    D = C * x
    _shuffled_kv(k_cache, v_cache, D, 16)
    S = context_lens.shape[0]
    _batch(S, block_table, context_lens)
    rows = S * chunk_tokens
    if k_out is None:
        k_out = torch.empty((rows, Hkv, D), dtype=torch.bfloat16, device=k_cache.device)
    if v_out is None:
        v_out = torch.empty((rows, Hkv, D), dtype=torch.bfloat16, device=k_cache.device)
    _gpu("k_out", k_out, torch.bfloat16, 3)
    _gpu("v_out", v_out, torch.bfloat16, 3)
    if k_out.shape[0] < rows or v_out.shape[0] < rows:
        raise ValueError("output tensors need num_seqs * chunk_tokens rows")
    if tuple(k_out.shape[1:]) != (Hkv, D) or tuple(v_out.shape[1:]) != (Hkv, D):
        raise ValueError(f"k_out / v_out must be [rows, {Hkv}, {D}]")
    st = lib.pa_gather_cache_chunk_fp8(k_out.data_ptr(), v_out.data_ptr(), k_cache.data_ptr(),
                                       v_cache.data_ptr(), block_table.data_ptr(),
                                       block_table.shape[1], context_lens.data_ptr(), S, Hkv, D,
                                       B, NB, int(iteration), int(chunk_tokens), float(k_scale),
                                       float(v_scale), _stream(k_cache))
    _check("gather_cache_chunk_fp8", st)
    return k_out, v_out


def reshape_and_cache_mla_fp8(latent: torch.Tensor, kv_cache: torch.Tensor,
                              slot_mapping: torch.Tensor, kv_scale: float) -> None:
    """Quantise latent [T, Dl] bf16 into kv_cache [NB, B, Dl] (uint8 E4M3 codes)."""
    lib = library()
    _gpu("latent", latent, torch.bfloat16, 2)
    _gpu("kv_cache", kv_cache, torch.uint8, 3)
    _gpu("slot_mapping", slot_mapping, torch.int64, 1)
    T, Dl = latent.shape
    NB, B, Dl2 = kv_cache.shape
    if Dl2 != Dl or slot_mapping.numel() != T:
        raise ValueError("latent cache shape does not match the latent rows")
    _check("reshape_and_cache_mla_fp8", lib.pa_reshape_and_cache_mla_fp8(
        latent.data_ptr(), kv_cache.data_ptr(), slot_mapping.data_ptr(), T, Dl, B, NB,
        float(kv_scale), _stream(latent)))


def mla_decode_attn_fp8(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                        context_lens: torch.Tensor, scale: float, max_context_len: int,
                        kv_scale: float, v_dim: int = 512, partition_tokens: int = 0,
                        new_latent: Optional[torch.Tensor] = None,
                        slot_mapping: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        return_lse: bool = True, workspace: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Absorbed MLA decode over an FP8 latent cache (rows = code * kv_scale), with
    the fused quantised write when new_latent and slot_mapping are given."""
    return _mla_fp8("pa_mla_decode_attn_fp8", query, kv_cache, block_table, context_lens, scale,
                    max_context_len, kv_scale, v_dim, partition_tokens, new_latent, slot_mapping,
                    out, lse, return_lse, workspace)


def mla_decode_attn_fp8_mfma(query: torch.Tensor, kv_cache: torch.Tensor,
                             block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                             max_context_len: int, kv_scale: float, v_dim: int = 512,
                             partition_tokens: int = 0, new_latent: Optional[torch.Tensor] = None,
                             slot_mapping: Optional[torch.Tensor] = None,
                             out: Optional[torch.Tensor] = None,
                             lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                             workspace: Optional[torch.Tensor] = None
                             ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """mla_decode_attn_fp8 on the matrix cores (codes widened to bf16 on chip)."""
    return _mla_fp8("pa_mla_decode_attn_fp8_mfma", query, kv_cache, block_table, context_lens,
                    scale, max_context_len, kv_scale, v_dim, partition_tokens, new_latent,
                    slot_mapping, out, lse, return_lse, workspace)


def _mla_fp8(fn, query, kv_cache, block_table, context_lens, scale, max_context_len, kv_scale,
             v_dim, partition_tokens, new_latent, slot_mapping, out, lse, return_lse, workspace):
    lib = library()
    _gpu("query", query, torch.bfloat16, 3)
    _gpu("kv_cache", kv_cache, torch.uint8, 3)
    _gpu("block_table", block_table, torch.int32, 2)
    _gpu("context_lens", context_lens, torch.int32, 1)
    S, Hq, Dl = query.shape
    NB, B, Dl2 = kv_cache.shape
    if Dl2 != Dl:
        raise ValueError("kv_cache latent width differs from the query's")
    if (new_latent is None) != (slot_mapping is None):
        raise ValueError("new_latent and slot_mapping go together")
    if new_latent is not None:
        _gpu("new_latent", new_latent, torch.bfloat16, 2)
        _gpu("slot_mapping", slot_mapping, torch.int64, 1)
        if tuple(new_latent.shape) != (S, Dl) or slot_mapping.numel() != S:
            raise ValueError("new_latent [num_seqs, latent_dim] and one slot per sequence")
    _batch(S, block_table, context_lens)
    if out is None:
        out = torch.empty((S, Hq, v_dim), dtype=torch.bfloat16, device=query.device)
    _gpu("out", out, torch.bfloat16, 3)
    _shape("out", out, (S, Hq, v_dim))
    if lse is None and return_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=query.device)
    if lse is not None:
        _gpu("lse", lse, torch.float32, 2)
        _shape("lse", lse, (S, Hq))
    nbytes = mla_workspace_size(S, Hq, v_dim, max_context_len, partition_tokens)
    ws = _workspace(nbytes, query.device, workspace)
    st = getattr(lib, fn)(out.data_ptr(), _ptr(lse), query.data_ptr(), _ptr(new_latent),
                          _ptr(slot_mapping), kv_cache.data_ptr(), block_table.data_ptr(),
                          block_table.shape[1], context_lens.data_ptr(), int(max_context_len), S,
                          Hq, Dl, v_dim, B, NB, float(scale), float(kv_scale),
                          int(partition_tokens), _ptr(ws), nbytes, _stream(query))
    _check(fn[3:], st)
    return out, lse
