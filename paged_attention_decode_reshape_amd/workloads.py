"""Seeded synthetic inputs for paged attention over a block-table KV cache.

This module draws context lengths, physical block assignments, slot numbers
and bf16 tensors.  It performs none of the attention arithmetic and none of
the cache-layout arithmetic: it produces token-major (standard layout) K/V,
queries and latents plus the block tables that say where each token lives.
Both the HIP path and the CPU oracle build their own shuffled caches from
these inputs.

Workload shapes follow the serving cases on the pages ("ROCm attention
backends" blog, MHA and MLA benchmark sections: Qwen3-235B with TP8 and
DeepSeek-R1 with TP8), reduced to one GPU's share of heads.

Draw order for every case (one ``torch.Generator('cpu')`` seeded per case):
context lengths (integer-uniform, bounds inclusive), then the physical block
permutation, then Q, then K (or the latents), then V, then outlier positions.
Values are float32 N(0, 1) rounded to bf16 (round-to-nearest-even, torch's
``.to(torch.bfloat16)``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# bf16 quiet NaN, used to poison cache memory that no sequence owns.
BF16_NAN_BITS = 0x7FC0
X_BF16 = 8  # elements per 16-byte vector in the shuffled layout (16 B / 2 B)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a CPU bf16 tensor as a uint16 numpy array."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_from_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


@dataclass
class Paging:
    """Logical-to-physical block assignment for S sequences."""
    block_size: int
    num_blocks: int
    lens: np.ndarray            # int32 [S] tokens owned by each sequence
    block_table: np.ndarray     # int32 [S, max_blocks_per_seq]
    seq_start: np.ndarray       # int64 [S+1] offsets of each sequence's tokens
    slot_mapping: np.ndarray    # int64 [sum(lens)] slot of every token, seq-major
    pad_block: int              # physical id used for table entries past a sequence's end

    @property
    def S(self) -> int:
        return int(self.lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def total_tokens(self) -> int:
        return int(self.seq_start[-1])


def make_paging(gen: torch.Generator, lens, block_size: int, *, pool_factor: float = 1.25,
                num_blocks: Optional[int] = None, max_blocks_per_seq: Optional[int] = None) -> Paging:
    """Random block tables over a pool of ``ceil(pool_factor * used)`` physical blocks.

    Physical ids are a seeded permutation of the pool, handed out in
    (sequence, logical block) order.  Table entries past a sequence's last
    block point at a block no sequence owns (``pad_block``), so a kernel that
    wrongly reads them sees poisoned memory instead of faulting.
    """
    lens = np.asarray(lens, dtype=np.int32)
    B = int(block_size)
    nblk = [(int(n) + B - 1) // B for n in lens]
    used = sum(nblk)
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * used))
    if num_blocks <= used:
        num_blocks = used + 1  # keep one block for padding entries
    perm = torch.randperm(num_blocks, generator=gen).numpy().astype(np.int32)
    maxb = max(nblk) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    assert maxb >= max(nblk)
    pad = int(perm[used])
    table = np.full((len(lens), maxb), pad, dtype=np.int32)
    k = 0
    for s, nb in enumerate(nblk):
        table[s, :nb] = perm[k:k + nb]
        k += nb
    seq_start = np.zeros(len(lens) + 1, dtype=np.int64)
    seq_start[1:] = np.cumsum(lens.astype(np.int64))
    slots = np.empty(int(seq_start[-1]), dtype=np.int64)
    for s, n in enumerate(lens):
        pos = np.arange(int(n), dtype=np.int64)
        slots[seq_start[s]:seq_start[s + 1]] = table[s, pos // B].astype(np.int64) * B + pos % B
    return Paging(B, int(num_blocks), lens, table, seq_start, slots, pad)


def _randn_bf16(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def _uniform_lens(gen: torch.Generator, S: int, lo: int, hi: int) -> np.ndarray:
    return torch.randint(lo, hi + 1, (S,), generator=gen).numpy().astype(np.int32)


@dataclass
class GQADecodeCase:
    """One decode step of GQA attention: one query token per sequence.

    ``context_lens`` counts every cached token including the one the step
    has just written (the cache write runs before attention).
    """
    name: str
    Hq: int
    Hkv: int
    D: int
    paging: Paging
    query: torch.Tensor          # bf16 [S, Hq, D]
    key: torch.Tensor            # bf16 [T, Hkv, D] token-major, seq-major
    value: torch.Tensor          # bf16 [T, Hkv, D]
    scale: float                 # float32-representable
    partition_tokens: int = 0    # 0: library chooses; -1: no split

    @property
    def S(self):
        return self.paging.S

    @property
    def B(self):
        return self.paging.block_size

    @property
    def context_lens(self):
        return self.paging.lens

    def new_token_rows(self) -> np.ndarray:
        """Row index (into key/value) of each sequence's newest token."""
        return (self.paging.seq_start[1:] - 1).astype(np.int64)


def gqa_decode_case(name: str, seed: int, lens, *, Hq: int, Hkv: int, D: int, block_size: int,
                    num_blocks: Optional[int] = None, partition_tokens: int = 0,
                    k_outlier_frac: float = 0.0, k_outlier_mult: float = 3.0,
                    lens_range: Optional[tuple] = None, S: Optional[int] = None) -> GQADecodeCase:
    gen = torch.Generator("cpu").manual_seed(seed)
    if lens_range is not None:
        lens = _uniform_lens(gen, S, *lens_range)
    paging = make_paging(gen, lens, block_size, num_blocks=num_blocks)
    T = paging.total_tokens
    q = _randn_bf16(gen, (paging.S, Hq, D))
    k32 = torch.randn(T, Hkv, D, generator=gen, dtype=torch.float32)
    v = _randn_bf16(gen, (T, Hkv, D))
    if k_outlier_frac > 0:
        # exactly floor(frac * n) token positions per sequence, without replacement;
        # the whole token (all kv heads, all dims) is scaled in f32 before rounding
        for s in range(paging.S):
            n = int(paging.lens[s])
            cnt = int(math.floor(k_outlier_frac * n))
            if cnt == 0:
                continue
            pos = torch.randperm(n, generator=gen)[:cnt]
            rows = pos + int(paging.seq_start[s])
            k32[rows] *= k_outlier_mult
    k = k32.to(torch.bfloat16)
    del k32
    scale = float(np.float32(1.0 / math.sqrt(D)))
    return GQADecodeCase(name, Hq, Hkv, D, paging, q, k, v, scale, partition_tokens)


@dataclass
class MLADecodeCase:
    """Absorbed MLA decode: every query head reads the same 576-wide latent row."""
    name: str
    Hq: int
    Dl: int
    Dv: int
    paging: Paging
    query: torch.Tensor          # bf16 [S, Hq, Dl]
    latent: torch.Tensor         # bf16 [T, Dl] token-major, seq-major
    scale: float
    partition_tokens: int = 0

    @property
    def S(self):
        return self.paging.S

    @property
    def B(self):
        return self.paging.block_size

    @property
    def context_lens(self):
        return self.paging.lens

    def new_token_rows(self) -> np.ndarray:
        return (self.paging.seq_start[1:] - 1).astype(np.int64)


def mla_decode_cases(name: str, seed: int, *, S: int, lens_range, Hq: int, Dl: int, Dv: int,
                     block_sizes=(1, 64), scale: float, lens=None) -> dict:
    """Same logical latents and queries laid out at several block sizes."""
    gen = torch.Generator("cpu").manual_seed(seed)
    if lens is None:
        lens = _uniform_lens(gen, S, *lens_range)
    lens = np.asarray(lens, dtype=np.int32)
    T = int(lens.astype(np.int64).sum())
    q = _randn_bf16(gen, (len(lens), Hq, Dl))
    lat = _randn_bf16(gen, (T, Dl))
    out = {}
    for B in block_sizes:
        paging = make_paging(gen, lens, B)
        out[B] = MLADecodeCase(f"{name}_bs{B}", Hq, Dl, Dv, paging, q, lat, float(np.float32(scale)))
    return out


@dataclass
class ExtendCase:
    """Chunked extend: each request has cached context plus new query tokens.

    ``paging`` covers cached + new tokens (the new tokens' K/V are written to
    the cache before attention runs); ``ctx_lens`` counts only the cached
    tokens before the new ones.
    """
    name: str
    Hq: int
    Hkv: int
    D: int
    paging: Paging
    ctx_lens: np.ndarray         # int32 [S]
    new_lens: np.ndarray         # int32 [S]
    query_start_loc: np.ndarray  # int32 [S+1]
    query: torch.Tensor          # bf16 [Tn, Hq, D]
    key: torch.Tensor            # bf16 [T, Hkv, D] all tokens (cached then new), seq-major
    value: torch.Tensor
    scale: float
    chunk_budget_tokens: int = 32768

    @property
    def S(self):
        return int(self.ctx_lens.shape[0])

    @property
    def B(self):
        return self.paging.block_size

    def new_rows(self) -> np.ndarray:
        """Rows of key/value holding the new tokens, in query order."""
        rows = []
        for s in range(self.S):
            st = int(self.paging.seq_start[s]) + int(self.ctx_lens[s])
            rows.append(np.arange(st, st + int(self.new_lens[s]), dtype=np.int64))
        return np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)


def extend_case(name: str, seed: int, *, ctx_lens=None, ctx_range=None, S=None, new_tokens,
                Hq: int, Hkv: int, D: int, block_size: int, chunk_budget_tokens: int = 32768) -> ExtendCase:
    gen = torch.Generator("cpu").manual_seed(seed)
    if ctx_lens is None:
        ctx_lens = _uniform_lens(gen, S, *ctx_range)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    if np.isscalar(new_tokens):
        new_lens = np.full(len(ctx_lens), int(new_tokens), dtype=np.int32)
    else:
        new_lens = np.asarray(new_tokens, dtype=np.int32)
    total = ctx_lens + new_lens
    paging = make_paging(gen, total, block_size)
    qsl = np.zeros(len(ctx_lens) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(new_lens)
    q = _randn_bf16(gen, (int(qsl[-1]), Hq, D))
    T = paging.total_tokens
    k = _randn_bf16(gen, (T, Hkv, D))
    v = _randn_bf16(gen, (T, Hkv, D))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    return ExtendCase(name, Hq, Hkv, D, paging, ctx_lens, new_lens, qsl, q, k, v, scale,
                      chunk_budget_tokens)


# ---------------------------------------------------------------------------
# The five named workloads.  Sizes are those of the serving cases: one GPU's
# share (TP8) of Qwen3-235B GQA decode and DeepSeek-R1 MLA decode, plus a
# long-context split-KV case and a chunked-extend case.
# ---------------------------------------------------------------------------

def tiny_gqa(partition_tokens: int = 0) -> GQADecodeCase:
    """4 sequences, lengths {37,100,256,511}, 4 q heads on 1 kv head, D=128,
    B=16, over exactly 64 physical blocks; seed 1001."""
    return gqa_decode_case("tiny_gqa", 1001, [37, 100, 256, 511], Hq=4, Hkv=1, D=128,
                           block_size=16, num_blocks=64, partition_tokens=partition_tokens)


def qwen3_decode(S: int = 64, lens_range=(1000, 2000)) -> GQADecodeCase:
    """Qwen3-235B per-GPU decode share: 64 requests, GQA 8:1, D=128, B=16,
    lengths U[1000,2000]; seed 1002."""
    return gqa_decode_case("qwen3_decode_64req", 1002, None, S=S, lens_range=lens_range,
                           Hq=8, Hkv=1, D=128, block_size=16)


def long_context_decode(S: int = 8, lens_range=(32768, 131072)) -> GQADecodeCase:
    """8 requests, 64 q heads on 4 kv heads, D=128, B=16, lengths
    U[32768,131072], 2048-token partitions, K x3 on 1% of tokens; seed 1003."""
    return gqa_decode_case("long_context_decode", 1003, None, S=S, lens_range=lens_range,
                           Hq=64, Hkv=4, D=128, block_size=16, partition_tokens=2048,
                           k_outlier_frac=0.01, k_outlier_mult=3.0)


def deepseek_mla_decode(S: int = 64, lens_range=(1024, 4096), block_sizes=(1, 64)) -> dict:
    """DeepSeek-R1 per-GPU absorbed MLA decode: 64 requests, 16 heads over one
    576-wide latent (512 + 64 rope), V = first 512 dims, scale 1/sqrt(192),
    lengths U[1024,4096], block sizes 1 and 64; seed 1004."""
    return mla_decode_cases("deepseek_mla_decode", 1004, S=S, lens_range=lens_range, Hq=16,
                            Dl=576, Dv=512, block_sizes=block_sizes, scale=1.0 / math.sqrt(192.0))


def chunked_extend(S: int = 16, ctx_range=(8192, 40960), new_tokens: int = 256,
                   chunk_budget_tokens: int = 32768) -> ExtendCase:
    """16 requests x 256 new tokens over cached U[8192,40960], 64 q heads on
    4 kv heads, D=128, B=16, 32768-token chunk budget; seed 1005."""
    return extend_case("chunked_extend", 1005, S=S, ctx_range=ctx_range, new_tokens=new_tokens,
                       Hq=64, Hkv=4, D=128, block_size=16, chunk_budget_tokens=chunk_budget_tokens)
