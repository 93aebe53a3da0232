"""GPU parity of absorbed MLA decode over an FP8 (E4M3) latent cache against
the oracle (oracle/fp8.py): the quantising latent write bit for bit, decode
on the vector ALUs (pa_mla_decode_attn_fp8) and on the matrix cores
(pa_mla_decode_attn_fp8_mfma) to the usual tolerance at block sizes 1, 64
and 5 and every split, the fused write + decode equal to the write followed
by decode.  Calls go through the C ABI."""
import math

import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
from oracle import fp8 as OF
from gpu_util import assert_attn_close, device, say

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(192.0)
KVS = 0.0123  # not a power of two: the products round
ENGINES = {"valu": pa.mla_decode_attn_fp8, "mfma": pa.mla_decode_attn_fp8_mfma}
LENS = [1, 31, 32, 33, 0, 100, 257, 700]


def halved(cases):
    """The cases with every latent halved (exact in bf16).  A one-token
    sequence's output is a single dequantised row rounded to bf16; at
    |x| >= 4 that rounding alone can reach 1/64, above the 1e-2 absolute
    bar, so the short-sequence cases keep their rows below 4."""
    for c in cases.values():
        c.latent = (c.latent.float() * 0.5).to(torch.bfloat16)
    return cases


class GpuMLAFp8:
    def __init__(self, case, kv_scale=KVS):
        dev = device()
        pg = case.paging
        self.case, self.kvs = case, kv_scale
        self.kv = torch.full((pg.num_blocks, case.B, case.Dl), 0x7F, dtype=torch.uint8, device=dev)
        self.slots = torch.from_numpy(pg.slot_mapping).to(dev)
        pa.reshape_and_cache_mla_fp8(case.latent.to(dev), self.kv, self.slots, kv_scale)
        self.q = case.query.to(dev)
        self.bt = torch.from_numpy(pg.block_table).to(dev)
        self.cl = torch.from_numpy(pg.lens).to(dev)
        self.max_ctx = int(pg.lens.max()) if pg.S else 0

    def oracle_cache(self, slots=None):
        pg = self.case.paging
        kv = np.full((pg.num_blocks, self.case.B, self.case.Dl), 0x7F, dtype=np.uint8)
        OF.cache_write_latent(W.bf16_bits(self.case.latent),
                              pg.slot_mapping if slots is None else slots, kv, self.kvs)
        return kv

    def decode(self, partition, engine="valu", **kw):
        return ENGINES[engine](self.q, self.kv, self.bt, self.cl, self.case.scale, self.max_ctx,
                               self.kvs, v_dim=self.case.Dv, partition_tokens=partition, **kw)

    def oracle(self, kv=None, seqs=None):
        c = self.case
        return OF.paged_decode_mla(W.bf16_bits(c.query), self.oracle_cache() if kv is None else kv,
                                   c.paging.block_table, c.context_lens, c.Dv, c.scale, self.kvs,
                                   seqs=seqs)


def test_mla_fp8_cache_write_bitexact():
    """Every byte of the pool, including slots skipped (negative, past the
    pool) and never written (still the 0x7F fill)."""
    cases = W.mla_decode_cases("mla8w", 430, S=5, lens_range=None, lens=[3, 40, 64, 65, 200],
                               Hq=4, Dl=576, Dv=512, block_sizes=(16,), scale=SCALE)
    case = cases[16]
    dev = device()
    g = GpuMLAFp8(case)
    slots = case.paging.slot_mapping.copy()
    slots[::7] = -1
    slots[1] = case.paging.num_blocks * case.B  # one past the pool
    kv = torch.full_like(g.kv, 0x7F)
    say("mla fp8 cache write")
    pa.reshape_and_cache_mla_fp8(case.latent.to(dev), kv, torch.from_numpy(slots).to(dev), KVS)
    torch.cuda.synchronize()
    assert np.array_equal(kv.cpu().numpy(), g.oracle_cache(slots))
    assert np.array_equal(g.kv.cpu().numpy(), g.oracle_cache())


@pytest.mark.parametrize("engine", ["valu", "mfma"])
@pytest.mark.parametrize("Hq", [16, 3])
@pytest.mark.parametrize("partition", [-1, 64, 0, -2])
def test_mla_fp8_small(Hq, partition, engine):
    cases = halved(W.mla_decode_cases("mla8", 431 + Hq, S=len(LENS), lens_range=None, lens=LENS,
                                      Hq=Hq, Dl=576, Dv=512, block_sizes=(1, 64, 5), scale=SCALE))
    ref = None
    for B, case in cases.items():
        say(f"mla fp8 {engine} Hq={Hq} B={B} P={partition}")
        g = GpuMLAFp8(case)
        out, lse = g.decode(partition, engine)
        if ref is None:
            ref = g.oracle()
        assert_attn_close(out, lse, ref[0], ref[1],
                          what=f"mla fp8 {engine} Hq={Hq} B={B} P={partition}")
        s0 = LENS.index(0)
        assert torch.all(out[s0] == 0) and torch.all(torch.isneginf(lse[s0]))


@pytest.mark.parametrize("engine", ["valu", "mfma"])
@pytest.mark.parametrize("partition", [-1, 64, -2])
def test_mla_fp8_fused_cache_write(partition, engine):
    """One launch (quantised write of each sequence's new latent, then
    decode) equals the write followed by decode, bits of output, LSE and
    cache, and matches the oracle."""
    lens = [1, 31, 32, 33, 100, 257, 700]
    cases = halved(W.mla_decode_cases("mla8fw", 432, S=len(lens), lens_range=None, lens=lens,
                                      Hq=16, Dl=576, Dv=512, block_sizes=(1, 64, 5), scale=SCALE))
    dev = device()
    for B, case in cases.items():
        say(f"mla fp8 {engine} fused cache write B={B} P={partition}")
        g = GpuMLAFp8(case)
        rows = case.new_token_rows()
        nl = case.latent[torch.from_numpy(rows)].to(dev).contiguous()
        slots = torch.from_numpy(case.paging.slot_mapping[rows]).to(dev).contiguous()
        gen = torch.Generator("cpu").manual_seed(81)
        junk = torch.randn(tuple(nl.shape), generator=gen).to(torch.bfloat16).to(dev)
        pa.reshape_and_cache_mla_fp8(junk, g.kv, slots, KVS)
        kv2 = g.kv.clone()
        o1, l1 = g.decode(partition, engine, new_latent=nl, slot_mapping=slots)
        pa.reshape_and_cache_mla_fp8(nl, kv2, slots, KVS)
        o2, l2 = ENGINES[engine](g.q, kv2, g.bt, g.cl, case.scale, g.max_ctx, KVS,
                                 v_dim=case.Dv, partition_tokens=partition)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
        assert torch.equal(g.kv, kv2)
        ref_out, ref_lse = g.oracle()
        assert_attn_close(o1, l1, ref_out, ref_lse,
                          what=f"mla fp8 {engine} fused B={B} P={partition}")


@pytest.mark.parametrize("engine", ["valu", "mfma"])
@pytest.mark.parametrize("B", [1, 64])
def test_mla_fp8_deepseek_sampled(B, engine):
    """64 requests, 16 heads, lengths U[1024,4096], in the benchmark's launch
    configuration (scale amax / 448): 8 whole requests vs the oracle."""
    case = W.deepseek_mla_decode(block_sizes=(B,))[B]
    kvs = float(np.float32(case.latent.float().abs().max().item() / 448.0))
    say(f"mla fp8 {engine} deepseek B={B} kv_scale={kvs:.4g}")
    g = GpuMLAFp8(case, kv_scale=kvs)
    out, lse = g.decode(0, engine)
    seqs = np.random.default_rng(83).choice(case.S, size=8, replace=False)
    ref_out, ref_lse = g.oracle(kv=g.kv.cpu().numpy(), seqs=seqs)
    mask = np.zeros((case.S, case.Hq), dtype=bool)
    mask[seqs] = True
    assert_attn_close(out, lse, ref_out, ref_lse, rows=np.nonzero(mask),
                      what=f"mla fp8 {engine} deepseek bs{B}")


def test_mla_fp8_mfma_balanced_more_sequences_than_workgroups():
    """The balanced split when the sequences outnumber the resident
    workgroups (one whole sequence per piece, in turn), matrix-core engine."""
    lens = np.random.default_rng(434).integers(0, 80, size=1500)
    case = halved(W.mla_decode_cases("mla8many", 434, S=len(lens), lens_range=None,
                                     lens=lens.tolist(), Hq=4, Dl=576, Dv=512, block_sizes=(16,),
                                     scale=SCALE))[16]
    say("mla fp8 mfma balanced 1500 sequences")
    g = GpuMLAFp8(case)
    out, lse = g.decode(-2, "mfma")
    ref_out, ref_lse = g.oracle()
    assert_attn_close(out, lse, ref_out, ref_lse, what="mla fp8 mfma balanced, many sequences")


def test_mla_fp8_mfma_out_of_range_blocks():
    """Block ids outside the pool read as zero rows (weight exp(-max) on a
    zero value) in both engines: the two agree to rounding."""
    case = halved(W.mla_decode_cases("mla8oor", 435, S=3, lens_range=None, lens=[40, 70, 33],
                                     Hq=16, Dl=576, Dv=512, block_sizes=(16,), scale=SCALE))[16]
    g = GpuMLAFp8(case)
    bt = g.bt.clone()
    bt[0, 1] = case.paging.num_blocks + 5
    bt[1, 0] = -3
    say("mla fp8 out-of-range block ids, both engines")
    o1, l1 = pa.mla_decode_attn_fp8(g.q, g.kv, bt, g.cl, SCALE, g.max_ctx, KVS)
    o2, l2 = pa.mla_decode_attn_fp8_mfma(g.q, g.kv, bt, g.cl, SCALE, g.max_ctx, KVS)
    torch.cuda.synchronize()
    assert torch.isfinite(o2.float()).all() and torch.isfinite(l2).all()
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


def test_mla_fp8_rejects_bad_arguments():
    case = W.mla_decode_cases("mla8bad", 433, S=2, lens_range=None, lens=[5, 9], Hq=4, Dl=576,
                              Dv=512, block_sizes=(16,), scale=SCALE)[16]
    g = GpuMLAFp8(case)
    with pytest.raises(pa.PagedAttnError) as e:
        pa.mla_decode_attn_fp8(g.q, g.kv, g.bt, g.cl, SCALE, g.max_ctx, 0.0)
    assert e.value.status == 1
    with pytest.raises(pa.PagedAttnError) as e:
        pa.mla_decode_attn_fp8(g.q, g.kv, g.bt, g.cl, SCALE, g.max_ctx, KVS, v_dim=448)
    assert e.value.status == 2
    with pytest.raises(pa.PagedAttnError) as e:
        pa.mla_decode_attn_fp8_mfma(g.q, g.kv, g.bt, g.cl, SCALE, g.max_ctx, float("nan"))
    assert e.value.status == 1
