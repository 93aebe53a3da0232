"""GPU: the standard cache layout [num_blocks, block_size, kv_heads, head_dim]
(the layout the shuffled one replaces, kept to measure the difference).

The standard-layout write is bit-exact against the oracle's; decode over a
standard cache is bit-identical to decode over the shuffled cache of the same
tokens (the kernel transposes V into the same registers), and within the
tolerance of the oracle.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
from gpu_util import GpuGQA, assert_attn_close, device, say

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 0, 300, 511]


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _t(x):
    return x.view(torch.int16)


def std_caches(case, dev, slots=None):
    pg = case.paging
    shape = (pg.num_blocks, case.B, case.Hkv, case.D)
    ks = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    vs = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev)
    if slots is None:
        slots = torch.from_numpy(pg.slot_mapping).to(dev)
    pa.reshape_and_cache(case.key.to(dev), case.value.to(dev), ks, vs, slots,
                         layout=pa.LAYOUT_STANDARD_KV)
    return ks, vs


def oracle_std(orc, case, slots=None):
    pg = case.paging
    ks, vs = orc.empty_standard_cache(pg.num_blocks, case.B, case.Hkv, case.D, fill=0x7FC0)
    orc.cache_write_standard(W.bf16_bits(case.key), W.bf16_bits(case.value),
                             pg.slot_mapping if slots is None else slots, ks, vs)
    return ks, vs


@pytest.mark.parametrize("mk", [
    lambda: W.tiny_gqa(),
    lambda: W.gqa_decode_case("d64b32", 211, [1, 31, 32, 33, 200], Hq=8, Hkv=4, D=64,
                              block_size=32),
    lambda: W.gqa_decode_case("h3", 212, [5, 17, 64, 65], Hq=6, Hkv=3, D=128, block_size=16),
], ids=["tiny", "d64b32_hkv4", "hkv3"])
def test_standard_cache_write_bitexact(orc, mk):
    case = mk()
    say(f"standard cache write {case.name}")
    dev = device()
    slots = case.paging.slot_mapping.copy()
    slots[::7] = -1                              # skipped
    slots[3] = case.paging.num_blocks * case.B   # outside the pool: skipped
    ks, vs = std_caches(case, dev, torch.from_numpy(slots).to(dev))
    oks, ovs = oracle_std(orc, case, slots)
    assert np.array_equal(_bits(ks), oks) and np.array_equal(_bits(vs), ovs)


CASES = [
    (lambda: W.tiny_gqa(), -1),
    (lambda: W.tiny_gqa(), 128),
    (lambda: W.gqa_decode_case("std_e1", 213, EDGE_LENS, Hq=8, Hkv=2, D=128, block_size=16), 64),
    (lambda: W.gqa_decode_case("std_e2", 214, EDGE_LENS, Hq=8, Hkv=2, D=128, block_size=16), -2),
    (lambda: W.gqa_decode_case("std_e3", 215, EDGE_LENS, Hq=16, Hkv=1, D=64, block_size=32), 0),
    (lambda: W.gqa_decode_case("std_e4", 216, EDGE_LENS, Hq=12, Hkv=4, D=128, block_size=32), 256),
    (lambda: W.gqa_decode_case("std_e5", 217, EDGE_LENS, Hq=5, Hkv=5, D=64, block_size=16), -1),
    (lambda: W.qwen3_decode(S=16), 256),
    (lambda: W.qwen3_decode(S=16), -2),
]
IDS = ["tiny_unsplit", "tiny_p128", "e128b16_p64", "e128b16_bal", "e64b32_g16_auto",
       "e128b32_hkv4_p256", "e64b16_mha_unsplit", "qwen16_p256", "qwen16_bal"]


@pytest.mark.parametrize("mk,partition", CASES, ids=IDS)
def test_decode_standard_equals_shuffled(orc, mk, partition):
    case = mk()
    say(f"standard-layout decode {case.name} partition {partition}")
    dev = device()
    g = GpuGQA(case)
    ks, vs = std_caches(case, dev)
    o_sh, l_sh = g.decode(partition)
    o_st, l_st = pa.paged_decode_attn_layout(pa.LAYOUT_STANDARD_KV, g.q, ks, vs, g.bt, g.cl,
                                             case.scale, g.max_ctx, partition_tokens=partition)
    o_sh2, l_sh2 = pa.paged_decode_attn_layout(pa.LAYOUT_SHUFFLED_KV, g.q, g.kc, g.vc, g.bt, g.cl,
                                               case.scale, g.max_ctx, partition_tokens=partition)
    torch.cuda.synchronize()
    assert torch.equal(_t(o_st), _t(o_sh)), "standard layout output differs from shuffled"
    assert torch.equal(l_st, l_sh), "standard layout lse differs from shuffled"
    assert torch.equal(_t(o_sh2), _t(o_sh)) and torch.equal(l_sh2, l_sh)
    oks, ovs = oracle_std(orc, case)
    ref_out, ref_lse = orc.paged_decode_gqa_standard(W.bf16_bits(case.query), oks, ovs,
                                                     case.paging.block_table, case.context_lens,
                                                     case.scale)
    assert_attn_close(o_st, l_st, ref_out, ref_lse, what=f"standard {case.name}")


@pytest.mark.parametrize("mk,partition", [
    (lambda: W.tiny_gqa(), 128),
    (lambda: W.gqa_decode_case("stdfw", 218, [1, 16, 17, 64, 65, 300, 0], Hq=8, Hkv=2, D=128,
                               block_size=16), 64),
    (lambda: W.qwen3_decode(S=16), -2),
], ids=["tiny_p128", "edges_p64", "qwen16_balanced"])
def test_decode_standard_fused_write(orc, mk, partition):
    """The fused write + decode over a standard cache equals the standard
    write followed by decode (bits), and leaves the caches equal to the
    oracle's standard cache."""
    case = mk()
    say(f"standard-layout fused write {case.name} partition {partition}")
    dev = device()
    g = GpuGQA(case)
    ks, vs = std_caches(case, dev)
    rows = torch.from_numpy(case.new_token_rows())
    nk = case.key[rows].to(dev).contiguous()
    nv = case.value[rows].to(dev).contiguous()
    slots = g.slots[rows.to(dev)].contiguous()
    gen = torch.Generator("cpu").manual_seed(78)
    junk = torch.randn((2,) + tuple(nk.shape), generator=gen).to(torch.bfloat16).to(dev)
    pa.reshape_and_cache(junk[0].contiguous(), junk[1].contiguous(), ks, vs, slots,
                         layout=pa.LAYOUT_STANDARD_KV)
    ks2, vs2 = ks.clone(), vs.clone()
    o1, l1 = pa.paged_decode_attn_layout(pa.LAYOUT_STANDARD_KV, g.q, ks, vs, g.bt, g.cl,
                                         case.scale, g.max_ctx, partition_tokens=partition,
                                         new_key=nk, new_value=nv, slot_mapping=slots)
    pa.reshape_and_cache(nk, nv, ks2, vs2, slots, layout=pa.LAYOUT_STANDARD_KV)
    o2, l2 = pa.paged_decode_attn_layout(pa.LAYOUT_STANDARD_KV, g.q, ks2, vs2, g.bt, g.cl,
                                         case.scale, g.max_ctx, partition_tokens=partition)
    o3, l3 = g.decode(partition)
    torch.cuda.synchronize()
    assert torch.equal(_t(o1), _t(o2)) and torch.equal(l1, l2), "fused differs from separate"
    assert torch.equal(_t(ks), _t(ks2)) and torch.equal(_t(vs), _t(vs2)), "caches differ"
    assert torch.equal(_t(o1), _t(o3)) and torch.equal(l1, l3), "differs from shuffled decode"
    oks, ovs = oracle_std(orc, case)
    assert np.array_equal(_bits(ks), oks) and np.array_equal(_bits(vs), ovs)
