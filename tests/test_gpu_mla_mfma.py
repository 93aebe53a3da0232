"""GPU parity: absorbed MLA decode on the matrix cores (pa_mla_decode_attn_mfma)
vs the fp64 oracle, through the C ABI; the same cases as the VALU engine's
tests, plus agreement between the two engines.
"""
import math

import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
from gpu_util import assert_attn_close, device, say
from test_gpu_mla import MLA_LENS, GpuMLA, oracle_mla

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(192.0)


def mfma(g, partition_tokens=0, **kw):
    return pa.mla_decode_attn_mfma(g.q, g.kv, g.bt, g.cl, g.case.scale, g.max_ctx,
                                   v_dim=g.case.Dv, partition_tokens=partition_tokens, **kw)


@pytest.mark.parametrize("Hq", [16, 3])
@pytest.mark.parametrize("partition", [-1, 64, 0, -2])
def test_mla_mfma_small(orc, Hq, partition):
    cases = W.mla_decode_cases("mla_small", 410 + Hq, S=len(MLA_LENS), lens_range=None,
                               lens=MLA_LENS, Hq=Hq, Dl=576, Dv=512, block_sizes=(1, 64, 5),
                               scale=SCALE)
    ref = None
    for B, case in cases.items():
        say(f"mla mfma Hq={Hq} B={B} P={partition}")
        g = GpuMLA(case)
        out, lse = mfma(g, partition)
        if ref is None:
            ref = oracle_mla(orc, case)
        assert_attn_close(out, lse, ref[0], ref[1], what=f"mla mfma Hq={Hq} B={B} P={partition}")
        s0 = MLA_LENS.index(0)
        assert torch.all(out[s0] == 0) and torch.all(torch.isneginf(lse[s0]))


def test_mla_mfma_block_size_invariance():
    """The same logical latents at block sizes 1 and 64 give identical bits."""
    cases = W.mla_decode_cases("mla_inv", 420, S=6, lens_range=(200, 900), Hq=16, Dl=576,
                               Dv=512, block_sizes=(1, 64), scale=SCALE)
    o1, l1 = mfma(GpuMLA(cases[1]), 256)
    o2, l2 = mfma(GpuMLA(cases[64]), 256)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_mla_mfma_agrees_with_valu(orc):
    """Both engines on the same cache: each within tolerance of the oracle,
    and of each other."""
    cases = W.mla_decode_cases("mla_eng", 425, S=10, lens_range=(1, 3000), Hq=16, Dl=576,
                               Dv=512, block_sizes=(64,), scale=SCALE)
    case = cases[64]
    g = GpuMLA(case)
    o1, l1 = g.decode()
    o2, l2 = mfma(g)
    ref_out, ref_lse = oracle_mla(orc, case)
    assert_attn_close(o2, l2, ref_out, ref_lse, what="mla mfma vs oracle")
    d = (o1.float() - o2.float()).abs().max().item()
    say(f"  mla mfma vs valu: {d:.3e}")
    assert d <= 1e-2 and (l1 - l2).abs().max().item() <= 1e-3


def test_mla_mfma_balanced_more_sequences_than_workgroups(orc):
    rng = np.random.default_rng(424)
    lens = rng.integers(0, 80, size=1500)
    cases = W.mla_decode_cases("mla_many", 424, S=len(lens), lens_range=None, lens=lens.tolist(),
                               Hq=4, Dl=576, Dv=512, block_sizes=(16,), scale=SCALE)
    case = cases[16]
    say("mla mfma balanced 1500 sequences")
    out, lse = mfma(GpuMLA(case), -2)
    ref_out, ref_lse = oracle_mla(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what="mla mfma balanced, sequences > workgroups")


def test_mla_mfma_out_of_range_blocks(orc):
    """A block-table entry outside [0, num_blocks) contributes no tokens, as
    in the VALU engine."""
    cases = W.mla_decode_cases("mla_oob", 426, S=3, lens_range=None, lens=[40, 100, 70], Hq=16,
                               Dl=576, Dv=512, block_sizes=(16,), scale=SCALE)
    case = cases[16]
    g = GpuMLA(case)
    bt = g.bt.clone()
    bt[1, 2] = case.paging.num_blocks + 5  # tokens 32..47 of sequence 1
    bt[2, 0] = -3                          # tokens 0..15 of sequence 2
    o1, l1 = pa.mla_decode_attn(g.q, g.kv, bt, g.cl, SCALE, g.max_ctx)
    o2, l2 = pa.mla_decode_attn_mfma(g.q, g.kv, bt, g.cl, SCALE, g.max_ctx)
    torch.cuda.synchronize()
    assert torch.isfinite(o2.float()).all()
    d = (o1.float() - o2.float()).abs().max().item()
    assert d <= 1e-2 and (l1 - l2).abs().max().item() <= 1e-3


@pytest.mark.parametrize("B", [1, 64])
def test_mla_mfma_deepseek_sampled(orc, B):
    """64 requests, 16 heads, lengths U[1024,4096] at block sizes 1 and 64 in the
    benchmark's launch configuration: 8 heads of every request vs the oracle."""
    cases = W.deepseek_mla_decode(block_sizes=(B,))
    case = cases[B]
    say(f"mla mfma deepseek B={B}")
    g = GpuMLA(case)
    out, lse = mfma(g)
    rng = np.random.default_rng(78)
    mask = np.zeros((case.S, case.Hq), dtype=np.uint8)
    for s in range(case.S):
        mask[s, rng.choice(case.Hq, size=8, replace=False)] = 1
    ref_out, ref_lse = oracle_mla(orc, case, row_mask=mask)
    assert_attn_close(out, lse, ref_out, ref_lse, rows=np.nonzero(mask), what=f"mfma deepseek bs{B}")


@pytest.mark.parametrize("partition", [-1, 64, 0, -2])
def test_mla_mfma_fused_cache_write(orc, partition):
    """The fused step equals the latent write followed by the decode (output,
    LSE and cache bits) and matches the oracle, at block sizes 1, 64 and 5."""
    lens = [1, 31, 32, 33, 100, 257, 700]
    cases = W.mla_decode_cases("mla_fw", 420, S=len(lens), lens_range=None, lens=lens, Hq=16,
                               Dl=576, Dv=512, block_sizes=(1, 64, 5), scale=SCALE)
    dev = device()
    for B, case in cases.items():
        say(f"mla mfma fused cache write B={B} P={partition}")
        g = GpuMLA(case)
        rows = case.new_token_rows()
        nl = case.latent[torch.from_numpy(rows)].to(dev).contiguous()
        slots = torch.from_numpy(case.paging.slot_mapping[rows]).to(dev).contiguous()
        gen = torch.Generator("cpu").manual_seed(79)
        junk = torch.randn(tuple(nl.shape), generator=gen).to(torch.bfloat16).to(dev)
        pa.reshape_and_cache(junk, None, g.kv, None, slots, layout=pa.LAYOUT_MLA_LATENT)
        kv2 = g.kv.clone()
        o1, l1 = mfma(g, partition, new_latent=nl, slot_mapping=slots)
        pa.reshape_and_cache(nl, None, kv2, None, slots, layout=pa.LAYOUT_MLA_LATENT)
        o2, l2 = pa.mla_decode_attn_mfma(g.q, kv2, g.bt, g.cl, case.scale, g.max_ctx,
                                         v_dim=case.Dv, partition_tokens=partition)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
        assert torch.equal(g.kv.view(torch.int16), kv2.view(torch.int16))
        ref_out, ref_lse = oracle_mla(orc, case)
        assert_attn_close(o1, l1, ref_out, ref_lse, what=f"mla mfma fused B={B} P={partition}")
