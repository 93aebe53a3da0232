"""NumPy brute-force attention on the logical (token-major) inputs.

Independent of the oracle: it never touches a block table or the shuffled
layout, and its arithmetic is numpy matmul + scipy's logsumexp in float64.
Used only to pin the oracle on small inputs.
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a).view(np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dense_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """q [Dq], K [n, Dq], V [n, Dv] float64 -> (out [Dv], lse)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -np.inf
    z = scale * (K @ q)
    lse = logsumexp(z)
    w = np.exp(z - lse)
    return w @ V, lse


def gqa_decode(q, key, value, seq_start, lens, scale):
    """q [S, Hq, D]; key/value [T, Hkv, D] logical rows (float64)."""
    S, Hq, D = q.shape
    Hkv = key.shape[1]
    grp = Hq // Hkv
    out = np.zeros((S, Hq, D))
    lse = np.zeros((S, Hq))
    for s in range(S):
        rows = slice(int(seq_start[s]), int(seq_start[s]) + int(lens[s]))
        for h in range(Hq):
            g = h // grp
            out[s, h], lse[s, h] = dense_attention(q[s, h], key[rows, g], value[rows, g], scale)
    return out, lse


def mla_decode(q, latent, seq_start, lens, Dv, scale):
    """Absorbed MLA as multi-query attention: K = latent, V = latent[:, :Dv]."""
    S, Hq, Dl = q.shape
    out = np.zeros((S, Hq, Dv))
    lse = np.zeros((S, Hq))
    for s in range(S):
        rows = slice(int(seq_start[s]), int(seq_start[s]) + int(lens[s]))
        L = latent[rows]
        for h in range(Hq):
            out[s, h], lse[s, h] = dense_attention(q[s, h], L, L[:, :Dv], scale)
    return out, lse


def extend(q, key, value, seq_start, ctx_lens, new_lens, scale):
    """Causal attention over the concatenation [context; new] of each request,
    with the mask aligned to the bottom-right: new token i sits at position
    ctx + i and sees positions 0 .. ctx + i."""
    Tn, Hq, D = q.shape
    Hkv = key.shape[1]
    grp = Hq // Hkv
    out = np.zeros((Tn, Hq, D))
    lse = np.zeros((Tn, Hq))
    qi = 0
    for s in range(len(ctx_lens)):
        base = int(seq_start[s])
        c = int(ctx_lens[s])
        for i in range(int(new_lens[s])):
            rows = slice(base, base + c + i + 1)
            for h in range(Hq):
                g = h // grp
                out[qi, h], lse[qi, h] = dense_attention(q[qi, h], key[rows, g], value[rows, g],
                                                         scale)
            qi += 1
    return out, lse
