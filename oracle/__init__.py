"""fp64 CPU oracle for paged attention over a shuffled block-table KV cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never imports, links or calls it, and it imports nothing from the GPU
library: the two share only the seeded input generators.

The arithmetic lives in ``oracle.c`` (plain C, double precision); this file
builds it with gcc, loads it with ctypes and adapts numpy arrays.  The FP8
(E4M3) cache -- codes, quantisation, its write, the gather with
dequantisation and decode over it -- is plain numpy in ``oracle/fp8.py``.  The
extend "recipe" (new-token attention, then a loop of gather -> attention ->
merge over context chunks, then a final merge; "ROCm attention backends"
blog, extend-path pseudocode) is composed here from the C primitives.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_c_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_c_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_c_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_c_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_c_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_f64 = ctypes.c_double


def build(src: str = SRC, out: str = LIB, openmp: bool = True) -> str:
    """Compile the oracle with gcc (-O2; no fast-math, so IEEE double holds)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", src, "-o", out + ".tmp", "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    return a


def _i32a(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _i64a(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int64)


class Oracle:
    """ctypes handle on one build of oracle.c."""

    def __init__(self, lib_path: str = LIB):
        if not os.path.exists(lib_path):
            build(out=lib_path)
        lib = ctypes.CDLL(lib_path)
        self.lib = lib
        lib.oracle_cache_write_shuffled.argtypes = [_c_u16p, _c_u16p, _c_i64p, _i64, _i32, _i32,
                                                    _i32, _i32, _i64, _c_u16p, _c_u16p]
        lib.oracle_cache_write_latent.argtypes = [_c_u16p, _c_i64p, _i64, _i32, _i32, _i64,
                                                  _c_u16p]
        lib.oracle_gather_shuffled.argtypes = [_c_u16p, _c_u16p, _c_i32p, _i32, _i32, _c_i32p,
                                               _c_i32p, _c_i64p, _i32, _i32, _i32, _i32,
                                               _c_u16p, _c_u16p]
        lib.oracle_paged_attn_gqa.argtypes = [_c_u16p, _c_u16p, _c_u16p, _c_i32p, _i32, _c_i32p,
                                              _c_i32p, _i32, _i32, _i32, _i32, _i32, _i32, _f64,
                                              _c_vp, _c_f64p, _c_f64p]
        lib.oracle_paged_attn_mla.argtypes = [_c_u16p, _c_u16p, _c_i32p, _i32, _c_i32p, _c_i32p,
                                              _i32, _i32, _i32, _i32, _i32, _f64, _c_vp,
                                              _c_f64p, _c_f64p]
        lib.oracle_merge.argtypes = [_i32, _c_f64p, _c_f64p, _i64, _i32, _c_f64p, _c_f64p]
        lib.oracle_dense_attn.argtypes = [_c_u16p, _c_u16p, _c_u16p, _c_i64p, _c_i64p, _i32,
                                          _i32, _i32, _i32, _f64, _i32, _c_f64p, _c_f64p]
        lib.oracle_extend.argtypes = [_c_u16p, _c_u16p, _c_u16p, _c_i32p, _c_u16p, _c_u16p,
                                      _c_i32p, _i32, _c_i32p, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _f64, _c_vp, _c_f64p, _c_f64p]
        lib.oracle_max_threads.restype = _i32
        lib.oracle_set_threads.argtypes = [_i32]
        lib.oracle_set_threads.restype = None
        for f in ("oracle_cache_write_shuffled", "oracle_cache_write_latent",
                  "oracle_gather_shuffled", "oracle_paged_attn_gqa", "oracle_paged_attn_mla",
                  "oracle_merge", "oracle_dense_attn", "oracle_extend"):
            getattr(lib, f).restype = None

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def set_threads(self, n: int) -> None:
        """Threads of the C oracle's parallel loops from now on."""
        self.lib.oracle_set_threads(int(n))

    # ---- caches ----------------------------------------------------------
    @staticmethod
    def empty_shuffled_cache(num_blocks: int, Hkv: int, D: int, B: int, x: int = 8,
                             fill: int = 0x7FC0):
        """Two uint16 pools, every element set to ``fill`` (bf16 NaN by default)."""
        k = np.full((num_blocks, Hkv, D // x, B, x), fill, dtype=np.uint16)
        v = np.full((num_blocks, Hkv, B // x, D, x), fill, dtype=np.uint16)
        return k, v

    def cache_write_shuffled(self, key, value, slot_mapping, k_cache, v_cache, B: int, x: int = 8):
        key, value = _u16(key), _u16(value)
        T, Hkv, D = key.shape
        nb = k_cache.shape[0]
        self.lib.oracle_cache_write_shuffled(key, value, _i64a(slot_mapping), T, Hkv, D, B, x, nb,
                                             k_cache, v_cache)

    # The standard layout [num_blocks, block_size, kv_heads, head_dim] is the
    # one the shuffled layout replaces ("ROCm attention backends" blog,
    # ROCM_AITER_FA section, hardware-optimised KV cache layout: the decode
    # gain is stated against the standard KV cache layout); token o of block
    # p keeps its [kv_heads, head_dim] rows as they are.
    @staticmethod
    def empty_standard_cache(num_blocks: int, B: int, Hkv: int, D: int, fill: int = 0x7FC0):
        k = np.full((num_blocks, B, Hkv, D), fill, dtype=np.uint16)
        return k, k.copy()

    @staticmethod
    def cache_write_standard(key, value, slot_mapping, k_cache, v_cache):
        """Token i goes to block slot // B, offset slot % B; slots outside the
        pool are skipped (the same rule as the shuffled write)."""
        key, value = _u16(key), _u16(value)
        nb, B = k_cache.shape[0], k_cache.shape[1]
        for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
            if 0 <= slot < nb * B:
                k_cache[slot // B, slot % B] = key[i]
                v_cache[slot // B, slot % B] = value[i]

    @staticmethod
    def standard_to_shuffled(k_std, v_std, x: int = 8):
        """The shuffle of the pages' cache shapes applied to a standard cache:
        k_cache[p][g][d div x][o][d mod x] = K[p][o][g][d] and
        v_cache[p][g][o div x][d][o mod x] = V[p][o][g][d]."""
        nb, B, Hkv, D = k_std.shape
        k = np.empty((nb, Hkv, D // x, B, x), dtype=np.uint16)
        v = np.empty((nb, Hkv, B // x, D, x), dtype=np.uint16)
        for o in range(B):
            for d in range(D):
                k[:, :, d // x, o, d % x] = k_std[:, o, :, d]
                v[:, :, o // x, d, o % x] = v_std[:, o, :, d]
        return k, v

    def paged_decode_gqa_standard(self, q, k_std, v_std, block_table, context_lens,
                                  scale: float, row_mask=None):
        """Decode over a standard-layout cache: the same tokens, so the same
        attention as over their shuffled copy."""
        k, v = self.standard_to_shuffled(k_std, v_std)
        return self.paged_decode_gqa(q, k, v, block_table, context_lens, k_std.shape[1], scale,
                                     row_mask=row_mask)

    def cache_write_latent(self, latent, slot_mapping, kv_cache, B: int):
        latent = _u16(latent)
        T, Dl = latent.shape
        self.lib.oracle_cache_write_latent(latent, _i64a(slot_mapping), T, Dl, B,
                                           kv_cache.shape[0], kv_cache)

    def gather_shuffled(self, k_cache, v_cache, block_table, tok_begin, tok_end, B: int, x: int = 8):
        """Unshuffle token ranges into the standard layout; returns (K, V, cu)."""
        bt = _i32a(block_table)
        tb, te = _i32a(tok_begin), _i32a(tok_end)
        S = bt.shape[0]
        n = np.maximum(te.astype(np.int64) - tb, 0)
        cu = np.zeros(S + 1, dtype=np.int64)
        cu[1:] = np.cumsum(n)
        Hkv = k_cache.shape[1]
        D = k_cache.shape[2] * k_cache.shape[4]
        ko = np.zeros((int(cu[-1]), Hkv, D), dtype=np.uint16)
        vo = np.zeros_like(ko)
        self.lib.oracle_gather_shuffled(k_cache, v_cache, bt, bt.shape[1], S, tb, te,
                                        np.ascontiguousarray(cu[:-1]), Hkv, D, B, x, ko, vo)
        return ko, vo, cu

    # ---- attention -------------------------------------------------------
    def paged_attn_gqa(self, q, k_cache, v_cache, block_table, tok_begin, tok_end, B: int,
                       scale: float, x: int = 8, row_mask: Optional[np.ndarray] = None):
        q = _u16(q)
        S, Hq, D = q.shape
        Hkv = k_cache.shape[1]
        bt = _i32a(block_table)
        out = np.zeros((S, Hq, D), dtype=np.float64)
        lse = np.zeros((S, Hq), dtype=np.float64)
        mask = None
        if row_mask is not None:
            mask = np.ascontiguousarray(row_mask, dtype=np.uint8)
        self.lib.oracle_paged_attn_gqa(q, k_cache, v_cache, bt, bt.shape[1], _i32a(tok_begin),
                                       _i32a(tok_end), S, Hq, Hkv, D, B, x, float(scale),
                                       None if mask is None else mask.ctypes.data, out, lse)
        return out, lse

    def paged_decode_gqa(self, q, k_cache, v_cache, block_table, context_lens, B: int,
                         scale: float, x: int = 8, row_mask=None):
        cl = _i32a(context_lens)
        return self.paged_attn_gqa(q, k_cache, v_cache, block_table, np.zeros_like(cl), cl, B,
                                   scale, x, row_mask)

    def paged_attn_mla(self, q, kv_cache, block_table, tok_begin, tok_end, B: int, Dv: int,
                       scale: float, row_mask: Optional[np.ndarray] = None):
        q = _u16(q)
        S, Hq, Dl = q.shape
        bt = _i32a(block_table)
        out = np.zeros((S, Hq, Dv), dtype=np.float64)
        lse = np.zeros((S, Hq), dtype=np.float64)
        mask = None
        if row_mask is not None:
            mask = np.ascontiguousarray(row_mask, dtype=np.uint8)
        self.lib.oracle_paged_attn_mla(q, kv_cache, bt, bt.shape[1], _i32a(tok_begin),
                                       _i32a(tok_end), S, Hq, Dl, Dv, B, float(scale),
                                       None if mask is None else mask.ctypes.data, out, lse)
        return out, lse

    def paged_decode_mla(self, q, kv_cache, block_table, context_lens, B: int, Dv: int,
                         scale: float, row_mask=None):
        cl = _i32a(context_lens)
        return self.paged_attn_mla(q, kv_cache, block_table, np.zeros_like(cl), cl, B, Dv, scale,
                                   row_mask)

    def merge(self, outs, lses):
        """n-way log-sum-exp merge; outs [n, ..., D], lses [n, ...]."""
        outs = np.ascontiguousarray(outs, dtype=np.float64)
        lses = np.ascontiguousarray(lses, dtype=np.float64)
        n = outs.shape[0]
        D = outs.shape[-1]
        rows = lses.shape[1:]
        R = int(np.prod(rows)) if rows else 1
        out = np.zeros(rows + (D,), dtype=np.float64)
        lse = np.zeros(rows, dtype=np.float64)
        self.lib.oracle_merge(n, outs.reshape(n, R, D), lses.reshape(n, R), R, D,
                              out.reshape(R, D), lse.reshape(R))
        return out, lse

    def dense_attn(self, q, k, v, cu_q, cu_k, scale: float, causal: bool):
        q, k, v = _u16(q), _u16(k), _u16(v)
        Tq, Hq, D = q.shape
        Hkv = k.shape[1]
        cu_q, cu_k = _i64a(cu_q), _i64a(cu_k)
        out = np.zeros((Tq, Hq, D), dtype=np.float64)
        lse = np.zeros((Tq, Hq), dtype=np.float64)
        self.lib.oracle_dense_attn(q, k, v, cu_q, cu_k, len(cu_q) - 1, Hq, Hkv, D, float(scale),
                                   1 if causal else 0, out, lse)
        return out, lse

    def extend(self, q, k_new, v_new, query_start_loc, k_cache, v_cache, block_table, ctx_lens,
               B: int, scale: float, x: int = 8, row_mask: Optional[np.ndarray] = None):
        """Extend attention by its definition (no chunking).  row_mask [Tn, Hq]
        selects the (new token, head) rows to compute; the rest stay zero."""
        q, k_new, v_new = _u16(q), _u16(k_new), _u16(v_new)
        Tn, Hq, D = q.shape
        Hkv = k_new.shape[1]
        bt = _i32a(block_table)
        cl = _i32a(ctx_lens)
        out = np.zeros((Tn, Hq, D), dtype=np.float64)
        lse = np.zeros((Tn, Hq), dtype=np.float64)
        mask = None
        if row_mask is not None:
            mask = np.ascontiguousarray(row_mask, dtype=np.uint8)
            assert mask.shape == (Tn, Hq)
        self.lib.oracle_extend(q, k_new, v_new, _i32a(query_start_loc), k_cache, v_cache, bt,
                               bt.shape[1], cl, len(cl), Hq, Hkv, D, B, x, float(scale),
                               None if mask is None else mask.ctypes.data, out, lse)
        return out, lse

    def extend_chunked(self, q, k_new, v_new, query_start_loc, k_cache, v_cache, block_table,
                       ctx_lens, B: int, scale: float, chunk_tokens: int, x: int = 8):
        """Extend attention by the pages' three-stage recipe.

        Stage 1: causal attention of the new tokens over themselves.
        Stage 2: for each context chunk, gather it to the standard layout,
        attend to it without a mask, and merge into the running context
        result.  Stage 3: merge the context result with the stage-1 result.
        ``chunk_tokens`` is the per-request chunk length of one iteration.
        """
        qsl = _i64a(query_start_loc)
        cl = _i32a(ctx_lens)
        S = len(cl)
        new_out, new_lse = self.dense_attn(q, k_new, v_new, qsl, qsl, scale, causal=True)
        Tn, Hq, D = new_out.shape
        ctx_out = np.zeros_like(new_out)
        ctx_lse = np.full((Tn, Hq), -np.inf)
        iters = int(-(-int(cl.max()) // chunk_tokens)) if S and cl.max() > 0 else 0
        for it in range(iters):
            tb = np.minimum(cl, it * chunk_tokens).astype(np.int32)
            te = np.minimum(cl, (it + 1) * chunk_tokens).astype(np.int32)
            kc, vc, cu = self.gather_shuffled(k_cache, v_cache, block_table, tb, te, B, x)
            c_out, c_lse = self.dense_attn(q, kc, vc, qsl, cu, scale, causal=False)
            ctx_out, ctx_lse = self.merge(np.stack([ctx_out, c_out]), np.stack([ctx_lse, c_lse]))
        return self.merge(np.stack([ctx_out, new_out]), np.stack([ctx_lse, new_lse]))


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from this directory's oracle.c (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle(LIB)
    return _default
