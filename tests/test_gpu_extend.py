"""GPU parity: context gather (bit-exact) and chunked extend attention
(tolerance) vs the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
import oracle_pins
from gpu_util import assert_attn_close, device, empty_gpu_cache, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


class GpuExtend:
    """An extend case on the GPU: all tokens (cached and new) written to the
    shuffled cache with the library's cache write, new K/V also kept apart."""

    def __init__(self, case: W.ExtendCase):
        dev = device()
        self.case = case
        pg = case.paging
        self.kc, self.vc = empty_gpu_cache(pg.num_blocks, case.Hkv, case.D, case.B, dev)
        pa.reshape_and_cache(case.key.to(dev), case.value.to(dev), self.kc, self.vc,
                             torch.from_numpy(pg.slot_mapping).to(dev))
        rows = torch.from_numpy(case.new_rows())
        self.k_new = case.key[rows].to(dev).contiguous()
        self.v_new = case.value[rows].to(dev).contiguous()
        self.q = case.query.to(dev)
        self.qsl = torch.from_numpy(case.query_start_loc).to(dev)
        self.bt = torch.from_numpy(pg.block_table).to(dev)
        self.cl = torch.from_numpy(case.ctx_lens).to(dev)

    def run(self, budget=None, **kw):
        c = self.case
        return pa.chunked_extend_attn(self.q, self.k_new, self.v_new, self.qsl, self.kc, self.vc,
                                      self.bt, self.cl, c.scale, c.query_start_loc, c.ctx_lens,
                                      chunk_budget_tokens=budget or c.chunk_budget_tokens, **kw)


def oracle_extend(orc, case):
    kc, vc, kn, vn = oracle_pins.extend_oracle_inputs(orc, case)
    return orc.extend(W.bf16_bits(case.query), kn, vn, case.query_start_loc, kc, vc,
                      case.paging.block_table, case.ctx_lens, case.B, case.scale)


@pytest.mark.parametrize("chunk", [16, 48, 4096])
def test_gather_bitexact(orc, chunk):
    case = W.extend_case("gather", 601, ctx_lens=[300, 0, 45, 129], new_tokens=[3, 5, 1, 2],
                         Hq=4, Hkv=2, D=128, block_size=16)
    g = GpuExtend(case)
    kc, vc = oracle_pins.oracle_cache(orc, case)
    iters = -(-int(case.ctx_lens.max()) // chunk)
    for it in range(iters):
        ko, vo = pa.gather_cache_chunk(g.kc, g.vc, g.bt, g.cl, it, chunk)
        torch.cuda.synchronize()
        tb = np.minimum(case.ctx_lens, it * chunk).astype(np.int32)
        te = np.minimum(case.ctx_lens, (it + 1) * chunk).astype(np.int32)
        rk, rv, cu = orc.gather_shuffled(kc, vc, case.paging.block_table, tb, te, case.B)
        n = int(cu[-1])
        assert np.array_equal(_bits(ko[:n]), rk), f"K chunk {chunk} iteration {it}"
        assert np.array_equal(_bits(vo[:n]), rv), f"V chunk {chunk} iteration {it}"


@pytest.mark.parametrize("budget", [64, 512, 32768])
def test_extend_small(orc, budget):
    """Contexts {300, 0, 45, 700} with {37, 5, 16, 130} new tokens; a small
    budget forces many chunk iterations."""
    case = W.extend_case("ext_small", 602, ctx_lens=[300, 0, 45, 700], new_tokens=[37, 5, 16, 130],
                         Hq=8, Hkv=2, D=128, block_size=16, chunk_budget_tokens=budget)
    say(f"extend small budget={budget}")
    g = GpuExtend(case)
    out, lse = g.run()
    ref_out, ref_lse = oracle_extend(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what=f"extend budget {budget}")


def test_extend_no_context(orc):
    """Requests without cached context: causal attention over the new tokens only."""
    case = W.extend_case("ext_noctx", 603, ctx_lens=[0, 0], new_tokens=[1, 200], Hq=4, Hkv=4,
                         D=128, block_size=32)
    g = GpuExtend(case)
    out, lse = g.run()
    ref_out, ref_lse = oracle_extend(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what="extend without context")


@pytest.mark.parametrize("block_size,budget", [(32, 256), (16, 1024), (32, 32768)])
def test_extend_pieces_group3(orc, block_size, budget):
    """12 q heads on 4 kv heads (group 3: 85 tokens x 3 heads per 256-row
    workgroup, one row unused), contexts that are not multiples of the tile
    or of 8, up to 4 context pieces per request merged by LSE, and a request
    whose new tokens span three workgroups."""
    case = W.extend_case("ext_g3", 606, ctx_lens=[5000, 17, 64, 1000, 0],
                         new_tokens=[40, 3, 200, 1, 9], Hq=12, Hkv=4, D=128,
                         block_size=block_size, chunk_budget_tokens=budget)
    say(f"extend group 3, block {block_size}, budget {budget}")
    g = GpuExtend(case)
    out, lse = g.run()
    ref_out, ref_lse = oracle_extend(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what=f"extend g3 B={block_size} budget {budget}")


def test_extend_budget_invariance():
    case = W.extend_case("ext_inv", 604, ctx_lens=[1000, 3000], new_tokens=[64, 200], Hq=16,
                         Hkv=2, D=128, block_size=16)
    g = GpuExtend(case)
    o1, l1 = g.run(budget=256)
    o2, l2 = g.run(budget=32768)
    torch.cuda.synchronize()
    d = (o1.float() - o2.float()).abs().max().item()
    say(f"  budget 256 vs 32768: {d:.3e}")
    assert d <= 1e-2 and (l1 - l2).abs().max().item() <= 1e-3


def extend_workload_rows(case, seed=91):
    """A stratified row sample of an extend workload: in every request, the
    first and last new tokens and the rows on each side of every 128-row
    query-block boundary, each with one q head drawn from every kv head's
    group, and four random (row, head) pairs.  Every row of a request attends to all of its context pieces, so
    every (request, kv head, piece) is covered."""
    rng = np.random.default_rng(seed)
    grp = case.Hq // case.Hkv
    mask = np.zeros((int(case.query_start_loc[-1]), case.Hq), dtype=np.uint8)
    for r in range(case.S):
        n = int(case.new_lens[r])
        picks = {0, n - 1}
        for b in range(128, n, 128):
            picks.update((b - 1, b))
        for i in sorted(p for p in picks if 0 <= p < n):
            row = int(case.query_start_loc[r]) + i
            for g in range(case.Hkv):
                mask[row, g * grp + int(rng.integers(grp))] = 1
        for _ in range(4):  # and a few rows anywhere
            if n > 0:
                mask[int(case.query_start_loc[r]) + int(rng.integers(n)), int(rng.integers(case.Hq))] = 1
    return mask


def test_extend_chunked_workload_sampled(orc):
    """16 requests x 256 new tokens over cached U[8192, 40960], 64 q heads on
    4 kv heads, 32768-token budget, in the benchmark's launch configuration:
    a stratified row sample vs the oracle's extend definition."""
    case = W.chunked_extend()
    say(f"extend workload, contexts {case.ctx_lens.tolist()}")
    g = GpuExtend(case)
    out, lse = g.run()
    torch.cuda.synchronize()
    mask = extend_workload_rows(case)
    rows = np.nonzero(mask)
    say(f"  {len(rows[0])} sampled (token, head) rows")
    kc, vc, kn, vn = oracle_pins.extend_oracle_inputs(orc, case)
    ref_out, ref_lse = orc.extend(W.bf16_bits(case.query), kn, vn, case.query_start_loc, kc, vc,
                                  case.paging.block_table, case.ctx_lens, case.B, case.scale,
                                  row_mask=mask)
    assert_attn_close(out, lse, ref_out, ref_lse, rows=rows, what="extend workload sampled")


def test_extend_rejects_bad_args():
    case = W.extend_case("ext_bad", 605, ctx_lens=[10], new_tokens=[4], Hq=2, Hkv=2, D=128,
                         block_size=16)
    g = GpuExtend(case)
    with pytest.raises(pa.PagedAttnError) as e:
        pa.chunked_extend_attn(g.q, g.k_new, g.v_new, g.qsl, g.kc, g.vc, g.bt, g.cl, float("nan"),
                               case.query_start_loc, case.ctx_lens)
    assert e.value.status == 1
