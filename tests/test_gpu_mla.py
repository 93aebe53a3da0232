"""GPU parity: absorbed MLA paged decode (576-wide latent, V = first 512 dims)
vs the fp64 oracle, through the C ABI.
"""
import math

import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
from gpu_util import assert_attn_close, device, say

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(192.0)


class GpuMLA:
    """An MLA case on the GPU; the latent cache is filled by the library's cache write."""

    def __init__(self, case: W.MLADecodeCase):
        dev = device()
        self.case = case
        pg = case.paging
        self.kv = torch.full((pg.num_blocks, case.B, case.Dl), float("nan"), dtype=torch.bfloat16,
                             device=dev)
        pa.reshape_and_cache(case.latent.to(dev), None, self.kv, None,
                             torch.from_numpy(pg.slot_mapping).to(dev),
                             layout=pa.LAYOUT_MLA_LATENT)
        self.q = case.query.to(dev)
        self.bt = torch.from_numpy(pg.block_table).to(dev)
        self.cl = torch.from_numpy(pg.lens).to(dev)
        self.max_ctx = int(pg.lens.max()) if pg.S else 0

    def decode(self, partition_tokens=0, **kw):
        return pa.mla_decode_attn(self.q, self.kv, self.bt, self.cl, self.case.scale, self.max_ctx,
                                  v_dim=self.case.Dv, partition_tokens=partition_tokens, **kw)


def oracle_mla(orc, case, row_mask=None):
    kv = np.full((case.paging.num_blocks, case.B, case.Dl), 0x7FC0, dtype=np.uint16)
    orc.cache_write_latent(W.bf16_bits(case.latent), case.paging.slot_mapping, kv, case.B)
    return orc.paged_decode_mla(W.bf16_bits(case.query), kv, case.paging.block_table,
                                case.context_lens, case.B, case.Dv, case.scale, row_mask=row_mask)


MLA_LENS = [1, 31, 32, 33, 0, 100, 257, 700]


@pytest.mark.parametrize("Hq", [16, 3])
@pytest.mark.parametrize("partition", [-1, 64, 0, -2])
def test_mla_small(orc, Hq, partition):
    cases = W.mla_decode_cases("mla_small", 410 + Hq, S=len(MLA_LENS), lens_range=None,
                               lens=MLA_LENS, Hq=Hq, Dl=576, Dv=512, block_sizes=(1, 64, 5),
                               scale=SCALE)
    ref = None
    for B, case in cases.items():
        say(f"mla Hq={Hq} B={B} P={partition}")
        g = GpuMLA(case)
        out, lse = g.decode(partition_tokens=partition)
        if ref is None:
            ref = oracle_mla(orc, case)
        assert_attn_close(out, lse, ref[0], ref[1], what=f"mla Hq={Hq} B={B} P={partition}")
        s0 = MLA_LENS.index(0)
        assert torch.all(out[s0] == 0) and torch.all(torch.isneginf(lse[s0]))


def test_mla_block_size_invariance():
    """The same logical latents at block sizes 1 and 64 give identical bits."""
    cases = W.mla_decode_cases("mla_inv", 420, S=6, lens_range=(200, 900), Hq=16, Dl=576,
                               Dv=512, block_sizes=(1, 64), scale=SCALE)
    o1, l1 = GpuMLA(cases[1]).decode(partition_tokens=256)
    o2, l2 = GpuMLA(cases[64]).decode(partition_tokens=256)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_mla_split_invariance():
    cases = W.mla_decode_cases("mla_split", 421, S=4, lens_range=(1500, 3000), Hq=16, Dl=576,
                               Dv=512, block_sizes=(64,), scale=SCALE)
    g = GpuMLA(cases[64])
    o1, l1 = g.decode(partition_tokens=-1)
    o2, l2 = g.decode(partition_tokens=128)
    torch.cuda.synchronize()
    d = (o1.float() - o2.float()).abs().max().item()
    say(f"  mla split vs unsplit: {d:.3e}")
    assert d <= 1e-2 and (l1 - l2).abs().max().item() <= 1e-4


def test_mla_balanced_matches_partitioned():
    cases = W.mla_decode_cases("mla_bal", 423, S=12, lens_range=(100, 4000), Hq=16, Dl=576,
                               Dv=512, block_sizes=(64,), scale=SCALE)
    g = GpuMLA(cases[64])
    o1, l1 = g.decode(partition_tokens=-2)
    o2, l2 = g.decode(partition_tokens=256)
    torch.cuda.synchronize()
    d = (o1.float() - o2.float()).abs().max().item()
    say(f"  mla balanced vs 256-token partitions: {d:.3e}")
    assert d <= 1e-2 and (l1 - l2).abs().max().item() <= 1e-4


def test_mla_balanced_more_sequences_than_workgroups(orc):
    """1500 short sequences: more sequences than the balanced grid has
    workgroups, so each is one piece and workgroups take several."""
    rng = np.random.default_rng(424)
    lens = rng.integers(0, 80, size=1500)
    cases = W.mla_decode_cases("mla_many", 424, S=len(lens), lens_range=None, lens=lens.tolist(),
                               Hq=4, Dl=576, Dv=512, block_sizes=(16,), scale=SCALE)
    case = cases[16]
    say("mla balanced 1500 sequences")
    out, lse = GpuMLA(case).decode(partition_tokens=-2)
    ref_out, ref_lse = oracle_mla(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what="mla balanced, sequences > workgroups")


@pytest.mark.parametrize("B", [1, 64])
def test_mla_deepseek_sampled(orc, B):
    """64 requests, 16 heads, lengths U[1024,4096] at block sizes 1 and 64, in the
    launch configuration the benchmark uses: 4 heads of every request vs the oracle."""
    cases = W.deepseek_mla_decode(block_sizes=(B,))
    case = cases[B]
    say(f"mla deepseek B={B}")
    g = GpuMLA(case)
    out, lse = g.decode()
    rng = np.random.default_rng(77)
    mask = np.zeros((case.S, case.Hq), dtype=np.uint8)
    for s in range(case.S):
        mask[s, rng.choice(case.Hq, size=4, replace=False)] = 1
    ref_out, ref_lse = oracle_mla(orc, case, row_mask=mask)
    assert_attn_close(out, lse, ref_out, ref_lse, rows=np.nonzero(mask), what=f"deepseek bs{B}")


def test_mla_rejects_unsupported():
    cases = W.mla_decode_cases("mla_bad", 422, S=2, lens_range=None, lens=[5, 9], Hq=4, Dl=576,
                               Dv=512, block_sizes=(16,), scale=SCALE)
    g = GpuMLA(cases[16])
    with pytest.raises(pa.PagedAttnError) as e:
        pa.mla_decode_attn(g.q, g.kv, g.bt, g.cl, SCALE, g.max_ctx, v_dim=448)
    assert e.value.status == 2
    with pytest.raises(pa.PagedAttnError) as e:
        pa.mla_decode_attn(g.q, g.kv, g.bt, g.cl, float("inf"), g.max_ctx)
    assert e.value.status == 1


@pytest.mark.parametrize("partition", [-1, 64, 0, -2])
def test_mla_fused_cache_write(orc, partition):
    """An MLA decode step in one launch equals the latent cache write
    followed by decode (output, LSE and cache bits), and matches the oracle,
    at block sizes 1, 64 and 5."""
    lens = [1, 31, 32, 33, 100, 257, 700]
    cases = W.mla_decode_cases("mla_fw", 420, S=len(lens), lens_range=None, lens=lens, Hq=16,
                               Dl=576, Dv=512, block_sizes=(1, 64, 5), scale=SCALE)
    dev = device()
    for B, case in cases.items():
        say(f"mla fused cache write B={B} P={partition}")
        g = GpuMLA(case)
        rows = case.new_token_rows()
        nl = case.latent[torch.from_numpy(rows)].to(dev).contiguous()
        slots = torch.from_numpy(case.paging.slot_mapping[rows]).to(dev).contiguous()
        gen = torch.Generator("cpu").manual_seed(79)
        junk = torch.randn(tuple(nl.shape), generator=gen).to(torch.bfloat16).to(dev)
        pa.reshape_and_cache(junk, None, g.kv, None, slots, layout=pa.LAYOUT_MLA_LATENT)
        kv2 = g.kv.clone()
        o1, l1 = pa.mla_decode_attn_write(g.q, nl, slots, g.kv, g.bt, g.cl, case.scale, g.max_ctx,
                                          v_dim=case.Dv, partition_tokens=partition)
        pa.reshape_and_cache(nl, None, kv2, None, slots, layout=pa.LAYOUT_MLA_LATENT)
        o2, l2 = pa.mla_decode_attn(g.q, kv2, g.bt, g.cl, case.scale, g.max_ctx, v_dim=case.Dv,
                                    partition_tokens=partition)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
        assert torch.equal(g.kv.view(torch.int16), kv2.view(torch.int16))
        ref_out, ref_lse = oracle_mla(orc, case)
        assert_attn_close(o1, l1, ref_out, ref_lse, what=f"mla fused B={B} P={partition}")
