"""FP8 (OCP E4M3, "fn": finite only) KV cache for the oracle.

TEST INFRASTRUCTURE, like the rest of ``oracle/``.  The pages' MLA extend
path gathers the context "and maybe dequantises" it ("vLLM ROCm attention
backends" blog, AITER MLA section, extend-path pseudocode), i.e. the KV cache
may hold FP8 codes with a scale.  The pages fix no format; this file reads
it as the OCP 8-bit E4M3 format (sign, 4 exponent bits with bias 7, 3
mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448) with
one float32 scale per tensor (K and V each):

    value(code) = decode(code) * scale
    code(x)     = encode(float32(x) * float32(1 / scale)),

where ``1 / scale`` is rounded to float32 once, the product is a float32
multiply, and encode rounds to the nearest E4M3 value, ties to the even code,
saturating at +-448 (a float32 above 448 becomes 448).  Everything here is
plain numpy written from that definition; nothing is shared with the GPU
library.

In the shuffled layout an FP8 x-vector is still 16 bytes, so x = 16:
    k_cache [num_blocks, kv_heads, head_dim / 16, block_size, 16]
    v_cache [num_blocks, kv_heads, block_size / 16, head_dim, 16]
("vLLM ROCm attention backends" blog, ROCM_AITER_FA section, the cache
shapes with x the number of elements in 16 bytes).
"""
from __future__ import annotations

import numpy as np

X = 16  # FP8 elements per 16-byte vector


def decode_table() -> np.ndarray:
    """float64 value of every code 0..255 (NaN for the two NaN codes)."""
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            t[c] = np.nan
            continue
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7) if e else m * 2.0 ** -9
        t[c] = -v if s else v
    return t


_TABLE = decode_table()
_POS = _TABLE[:0x7F]  # codes 0x00 .. 0x7E: the non-negative finite values, increasing


def encode(y) -> np.ndarray:
    """Nearest E4M3 code to each float32 in y (ties to the even code,
    saturating at 448), found by comparing against every finite value."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64)).reshape(-1)
    sign = (np.signbit(y).reshape(-1)).astype(np.uint8) << 7
    # index of the largest finite value <= a, and the next one up
    lo = np.searchsorted(_POS, a, side="right") - 1
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a >= 448.0, np.uint8(0x7E), code)
    return (code | sign).reshape(y.shape)


def quantize_bf16(bits, scale: float) -> np.ndarray:
    """Codes of bf16 values (uint16 bit patterns) under `scale`."""
    x = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    return encode((x * inv).astype(np.float32))


def dequant_f64(codes, scale: float) -> np.ndarray:
    """Exact values code * scale (float64 holds the product of the two float32s)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)] * float(np.float32(scale))


def bf16_rne(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def empty_cache(num_blocks: int, Hkv: int, D: int, B: int, fill: int = 0x7F):
    """FP8 shuffled pools, every byte `fill` (NaN by default)."""
    k = np.full((num_blocks, Hkv, D // X, B, X), fill, dtype=np.uint8)
    v = np.full((num_blocks, Hkv, B // X, D, X), fill, dtype=np.uint8)
    return k, v


def cache_write(key_bits, value_bits, slot_mapping, k_cache, v_cache, k_scale, v_scale):
    """Token i (slot s = block * B + o, skipped unless 0 <= s < blocks * B):
    k_cache[p][g][d div 16][o][d mod 16] = code(K[i][g][d]) and
    v_cache[p][g][o div 16][d][o mod 16] = code(V[i][g][d])."""
    nb, Hkv, _, B, _ = k_cache.shape
    kq = quantize_bf16(key_bits, k_scale)
    vq = quantize_bf16(value_bits, v_scale)
    D = kq.shape[2]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if not 0 <= slot < nb * B:
            continue
        p, o = int(slot) // B, int(slot) % B
        # dim d = 16 c + j of token o: K at [p][g][c][o][j], V at [p][g][o div 16][d][o mod 16]
        k_cache[p, :, :, o, :] = kq[i].reshape(Hkv, D // X, X)
        v_cache[p, :, o // X, :, o % X] = vq[i]


def gather_codes(k_cache, v_cache, block_table, seq, tokens):
    """Codes [len(tokens), Hkv, D] of sequence `seq`'s tokens through the table."""
    nb, Hkv, C, B, _ = k_cache.shape
    D = C * X
    K = np.empty((len(tokens), Hkv, D), dtype=np.uint8)
    V = np.empty_like(K)
    for j, t in enumerate(tokens):
        p, o = int(block_table[seq][t // B]), t % B
        K[j] = k_cache[p, :, :, o, :].reshape(Hkv, D)
        V[j] = v_cache[p, :, o // X, :, o % X]
    return K, V


def gather_dequant(k_cache, v_cache, block_table, context_lens, iteration, chunk, k_scale,
                   v_scale):
    """One chunk iteration of the gather with dequantisation: tokens
    [iteration * chunk, min((iteration + 1) * chunk, ctx)) of every sequence,
    requests one after another, as bf16 bit patterns of float32(code value)
    * float32(scale) rounded to nearest even."""
    ks, vs = [], []
    for s, n in enumerate(np.asarray(context_lens)):
        t0, t1 = iteration * chunk, min((iteration + 1) * chunk, int(n))
        if t1 <= t0:
            continue
        K, V = gather_codes(k_cache, v_cache, block_table, s, range(t0, t1))
        kf = _TABLE[K].astype(np.float32) * np.float32(k_scale)
        vf = _TABLE[V].astype(np.float32) * np.float32(v_scale)
        ks.append(bf16_rne(kf))
        vs.append(bf16_rne(vf))
    if not ks:
        return np.zeros((0,), np.uint16), np.zeros((0,), np.uint16)
    return np.concatenate(ks), np.concatenate(vs)


def paged_decode_gqa(q_bits, k_cache, v_cache, block_table, context_lens, scale, k_scale,
                     v_scale, seqs=None):
    """Exact softmax attention in float64 of each sequence's query over its
    dequantised tokens (K = code * k_scale, V = code * v_scale), query head h
    on kv head h div (Hq / Hkv); returns (out [S, Hq, D], lse [S, Hq])."""
    q = (np.asarray(q_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    q = q.astype(np.float64)
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D))
    lse = np.full((S, Hq), -np.inf)
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        K, V = gather_codes(k_cache, v_cache, block_table, s, range(n))
        Kf = dequant_f64(K, k_scale)
        Vf = dequant_f64(V, v_scale)
        for h in range(Hq):
            g = h // G
            z = float(np.float32(scale)) * (Kf[:, g, :] @ q[s, h])
            m = z.max()
            w = np.exp(z - m)
            lsum = w.sum()
            out[s, h] = (w @ Vf[:, g, :]) / lsum
            lse[s, h] = m + np.log(lsum)
    return out, lse


# ---- MLA latent cache in FP8 -------------------------------------------------
# The latent row of a token (576 values: keys are the whole row, values its
# first 512) is one tensor with one scale; the cache is [num_blocks,
# block_size, 576] codes, rows as they are (no shuffle, as for bf16).

def cache_write_latent(latent_bits, slot_mapping, kv_cache, scale):
    """Token i's row of codes goes to kv_cache[slot // B][slot % B]; slots
    outside the pool are skipped."""
    nb, B, _ = kv_cache.shape
    codes = quantize_bf16(latent_bits, scale)
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if 0 <= slot < nb * B:
            kv_cache[int(slot) // B, int(slot) % B] = codes[i]


def paged_decode_mla(q_bits, kv_cache, block_table, context_lens, Dv, scale, kv_scale,
                     seqs=None):
    """Exact attention in float64 of each head's query over the dequantised
    latent rows (K = row, V = row[:Dv]); returns (out [S, Hq, Dv], lse [S, Hq])."""
    q = (np.asarray(q_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    q = q.astype(np.float64)
    S, Hq, Dl = q.shape
    B = kv_cache.shape[1]
    out = np.zeros((S, Hq, Dv))
    lse = np.full((S, Hq), -np.inf)
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        t = np.arange(n)
        rows = kv_cache[np.asarray(block_table[s])[t // B], t % B]  # [n, Dl] codes
        K = dequant_f64(rows, kv_scale)
        z = float(np.float32(scale)) * (K @ q[s].T)  # [n, Hq]
        m = z.max(axis=0)
        w = np.exp(z - m)
        lsum = w.sum(axis=0)
        out[s] = (w.T @ K[:, :Dv]) / lsum[:, None]
        lse[s] = m + np.log(lsum)
    return out, lse
