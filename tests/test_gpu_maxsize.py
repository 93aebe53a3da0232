"""GPU parity at the largest supported context, 2^20 tokens (the library's
bound), with a ragged neighbour: GQA decode in four split modes, MLA decode
(both engines, balanced and unsplit),
and chunked extend over a 2^20-token context.  Every output is checked
against the oracle.  Inputs are about 1 GB of KV per case."""
import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
import oracle_pins
from gpu_util import GpuGQA, assert_attn_close, device, oracle_gqa, say

pytestmark = pytest.mark.gpu

MAX_CTX = 1 << 20


@pytest.fixture(scope="module")
def gqa_max():
    case = W.gqa_decode_case("max_gqa", 701, [MAX_CTX, MAX_CTX - 5, 3], Hq=8, Hkv=1, D=128,
                             block_size=16)
    return case, GpuGQA(case)


@pytest.fixture(scope="module")
def gqa_max_ref(orc, gqa_max):
    return oracle_gqa(orc, gqa_max[0])


@pytest.mark.parametrize("partition", [-1, 0, -2, 4096])
def test_decode_max_context(gqa_max, gqa_max_ref, partition):
    case, g = gqa_max
    say(f"decode at 2^20 tokens, partition {partition}")
    out, lse = g.decode(partition)
    torch.cuda.synchronize()
    assert_attn_close(out, lse, gqa_max_ref[0], gqa_max_ref[1], what=f"max ctx P={partition}")


@pytest.fixture(scope="module")
def mla_max(orc):
    case = W.mla_decode_cases("max_mla", 702, S=2, lens_range=None, lens=[MAX_CTX, 77], Hq=16,
                              Dl=576, Dv=512, block_sizes=(64,), scale=1.0 / 192 ** 0.5)[64]
    dev = device()
    pg = case.paging
    kv = torch.full((pg.num_blocks, case.B, case.Dl), float("nan"), dtype=torch.bfloat16,
                    device=dev)
    pa.reshape_and_cache(case.latent.to(dev), None, kv, None,
                         torch.from_numpy(pg.slot_mapping).to(dev), layout=pa.LAYOUT_MLA_LATENT)
    g = (torch.from_numpy(pg.block_table).to(dev), torch.from_numpy(pg.lens).to(dev),
         case.query.to(dev), kv)
    okv = np.full((pg.num_blocks, case.B, case.Dl), 0x7FC0, dtype=np.uint16)
    orc.cache_write_latent(W.bf16_bits(case.latent), pg.slot_mapping, okv, case.B)
    ref = orc.paged_decode_mla(W.bf16_bits(case.query), okv, pg.block_table, case.context_lens,
                               case.B, case.Dv, case.scale)
    return case, g, ref


@pytest.mark.parametrize("engine", ["valu", "mfma"])
@pytest.mark.parametrize("partition", [0, -1])
def test_mla_max_context(mla_max, engine, partition):
    case, (bt, cl, q, kv), (ref_out, ref_lse) = mla_max
    say(f"mla decode at 2^20 tokens, {engine} engine, partition {partition}")
    fn = pa.mla_decode_attn_mfma if engine == "mfma" else pa.mla_decode_attn
    out, lse = fn(q, kv, bt, cl, case.scale, MAX_CTX, v_dim=512, partition_tokens=partition)
    torch.cuda.synchronize()
    assert_attn_close(out, lse, ref_out, ref_lse, what=f"mla max ctx {engine} P={partition}")


def test_extend_max_context(orc):
    case = W.extend_case("max_ext", 703, ctx_lens=[MAX_CTX, 300], new_tokens=[37, 5], Hq=2,
                         Hkv=1, D=128, block_size=16)
    say("extend over a 2^20-token context")
    dev = device()
    pg = case.paging
    kc = torch.full((pg.num_blocks, 1, 16, 16, 8), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full((pg.num_blocks, 1, 2, 128, 8), float("nan"), dtype=torch.bfloat16, device=dev)
    pa.reshape_and_cache(case.key.to(dev), case.value.to(dev), kc, vc,
                         torch.from_numpy(pg.slot_mapping).to(dev))
    rows = torch.from_numpy(case.new_rows())
    out, lse = pa.chunked_extend_attn(case.query.to(dev), case.key[rows].to(dev).contiguous(),
                                      case.value[rows].to(dev).contiguous(),
                                      torch.from_numpy(case.query_start_loc).to(dev), kc, vc,
                                      torch.from_numpy(pg.block_table).to(dev),
                                      torch.from_numpy(case.ctx_lens).to(dev), case.scale,
                                      case.query_start_loc, case.ctx_lens)
    torch.cuda.synchronize()
    okc, ovc, kn, vn = oracle_pins.extend_oracle_inputs(orc, case)
    ref_out, ref_lse = orc.extend(W.bf16_bits(case.query), kn, vn, case.query_start_loc, okc, ovc,
                                  pg.block_table, case.ctx_lens, case.B, case.scale)
    assert_attn_close(out, lse, ref_out, ref_lse, what="extend max ctx")


@pytest.mark.parametrize("engine", ["valu", "mfma"])
def test_mla_fp8_max_context(engine):
    """MLA decode over an FP8 latent cache at 2^20 tokens (row offsets past
    2^29 bytes) against the FP8 oracle, on either engine."""
    from oracle import fp8 as OF
    case = W.mla_decode_cases("max_mla8", 703, S=2, lens_range=None, lens=[MAX_CTX, 77], Hq=16,
                              Dl=576, Dv=512, block_sizes=(64,), scale=1.0 / 192 ** 0.5)[64]
    say(f"mla fp8 decode at 2^20 tokens, {engine} engine")
    dev = device()
    pg = case.paging
    kvs = float(np.float32(case.latent.float().abs().max().item() / 448.0))
    kv = torch.full((pg.num_blocks, case.B, case.Dl), 0x7F, dtype=torch.uint8, device=dev)
    pa.reshape_and_cache_mla_fp8(case.latent.to(dev), kv, torch.from_numpy(pg.slot_mapping).to(dev),
                                 kvs)
    q = case.query.to(dev)
    bt = torch.from_numpy(pg.block_table).to(dev)
    cl = torch.from_numpy(pg.lens).to(dev)
    fn = pa.mla_decode_attn_fp8_mfma if engine == "mfma" else pa.mla_decode_attn_fp8
    out, lse = fn(q, kv, bt, cl, case.scale, MAX_CTX, kvs, v_dim=512)
    torch.cuda.synchronize()
    okv = np.full((pg.num_blocks, case.B, case.Dl), 0x7F, dtype=np.uint8)
    OF.cache_write_latent(W.bf16_bits(case.latent), pg.slot_mapping, okv, kvs)
    assert np.array_equal(kv.cpu().numpy(), okv)
    ref_out, ref_lse = OF.paged_decode_mla(W.bf16_bits(case.query), okv, pg.block_table,
                                           case.context_lens, case.Dv, case.scale, kvs)
    assert_attn_close(out, lse, ref_out, ref_lse, what=f"mla fp8 max ctx {engine}")
