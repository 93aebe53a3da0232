"""GPU parity: cache write (bit-exact) and GQA paged decode (tolerance) vs the oracle.

Every call goes through the C ABI (libpagedattn.so) via the Python binding.
"""
import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
import oracle_pins
from gpu_util import GpuGQA, assert_attn_close, device, oracle_gqa, say, to_f64

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# cache write
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mk", [
    lambda: W.tiny_gqa(),
    lambda: W.gqa_decode_case("d64b32", 201, [1, 31, 32, 33, 200], Hq=8, Hkv=4, D=64,
                              block_size=32),
    lambda: W.gqa_decode_case("h3", 202, [5, 17, 64, 65], Hq=6, Hkv=3, D=128, block_size=16),
    lambda: W.qwen3_decode(),
], ids=["tiny", "d64b32_hkv4", "hkv3", "qwen3_64req_93k_tokens"])
def test_cache_write_bitexact(orc, mk):
    case = mk()
    say(f"cache write {case.name}")
    g = GpuGQA(case)
    kc, vc = oracle_pins.oracle_cache(orc, case)
    assert np.array_equal(_bits(g.kc), kc.reshape(-1).reshape(kc.shape))
    assert np.array_equal(_bits(g.vc), vc)


@pytest.mark.parametrize("reps", [1, 128], ids=["small", "bulk"])
@pytest.mark.parametrize("D,B,Hkv", [(128, 16, 1), (64, 32, 3), (128, 32, 2)])
def test_cache_write_mixed_slot_runs(orc, D, B, Hkv, reps):
    """Bulk write whose slot mapping mixes every case of an 8-slot V group:
    runs that start mid-group and mid-block, aligned runs of exactly 8, runs
    crossing a 32-token chunk boundary, scattered single slots, skipped (-1)
    and out-of-range slots, and a token count that is not a multiple of 32;
    into NaN-filled pools, bit for bit against the oracle's write.  The
    pattern is repeated over fresh blocks ``reps`` times: once stays below
    12288 token-heads (one thread per source vector), 128 times goes above
    (32-token chunks staged in LDS)."""
    rng = np.random.default_rng(D + B + Hkv)
    nb = 48 * reps
    perm = rng.permutation(nb)
    slots = []
    for rep in range(reps):
        def run(block, start, n):
            slots.extend(int(perm[48 * rep + block]) * B + start + j for j in range(n))
        run(0, 3, B - 3)          # mid-block start, to the block's end
        run(1, 0, 8)              # exactly one aligned group
        run(2, 0, B)              # a whole block, then the next block of the same run
        run(3, 0, B)
        slots.extend(int(perm[48 * rep + 5]) * B + int(o)
                     for o in rng.choice(B, size=5, replace=False))
        slots.extend([-1, nb * B + 3, -1])
        run(6, 5, 2)              # a short run inside one group
        run(7, 0, 13)             # an aligned run ending mid-group
        run(8, 8, 8)              # the second group of a block
        run(9, 1, 30 if B == 32 else 15)
    slots.extend(int(perm[10]) * B + j for j in range(5))  # a ragged tail on an unused block
    assert (len(slots) * Hkv >= 12288) == (reps > 1)
    T = len(slots)
    assert T % 32 != 0
    assert len(set(s for s in slots if 0 <= s < nb * B)) == sum(1 for s in slots if 0 <= s < nb * B)
    dev = device()
    key = torch.randn(T, Hkv, D, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    value = torch.randn(T, Hkv, D, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16)
    kc = torch.full((nb, Hkv, D // 8, B, 8), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full((nb, Hkv, B // 8, D, 8), float("nan"), dtype=torch.bfloat16, device=dev)
    sm = np.array(slots, dtype=np.int64)
    pa.reshape_and_cache(key.to(dev), value.to(dev), kc, vc, torch.from_numpy(sm).to(dev))
    torch.cuda.synchronize()
    okc, ovc = orc.empty_shuffled_cache(nb, Hkv, D, B)
    orc.cache_write_shuffled(W.bf16_bits(key), W.bf16_bits(value), sm, okc, ovc, B)
    assert np.array_equal(_bits(kc), okc) and np.array_equal(_bits(vc), ovc)


def test_cache_write_skips_bad_slots(orc):
    dev = device()
    case = W.gqa_decode_case("skip", 203, [20], Hq=2, Hkv=2, D=128, block_size=16)
    g = GpuGQA(case)
    before_k, before_v = g.kc.clone(), g.vc.clone()
    nb = case.paging.num_blocks
    key = torch.randn(4, 2, 128, device=dev).to(torch.bfloat16)
    slots = torch.tensor([-1, nb * 16, nb * 16 + 100, -7], dtype=torch.int64, device=dev)
    pa.reshape_and_cache(key, key.clone(), g.kc, g.vc, slots)
    torch.cuda.synchronize()
    assert torch.equal(_t(g.kc), _t(before_k)) and torch.equal(_t(g.vc), _t(before_v))


def _t(x):
    return x.view(torch.int16)


def test_cache_write_decode_step_overwrite(orc):
    """A decode step rewrites each sequence's newest token; bytes stay identical."""
    case = W.tiny_gqa()
    g = GpuGQA(case)
    dev = device()
    rows = torch.from_numpy(case.new_token_rows())
    pa.reshape_and_cache(case.key[rows].to(dev), case.value[rows].to(dev), g.kc, g.vc,
                         g.slots[rows.to(dev)])
    kc, vc = oracle_pins.oracle_cache(orc, case)
    assert np.array_equal(_bits(g.kc), kc) and np.array_equal(_bits(g.vc), vc)


def _fused_vs_separate(case, partition, skip=None):
    """Overwrite every sequence's newest token in the caches with other
    values, then run (a) the fused write + decode and (b) the cache write
    followed by decode on a copy: outputs, LSEs and caches must agree bit for
    bit.  `skip`: sequences whose slot is -1 in both (nothing written)."""
    dev = device()
    g = GpuGQA(case)
    rows = torch.from_numpy(case.new_token_rows())
    nk = case.key[rows].to(dev).contiguous()
    nv = case.value[rows].to(dev).contiguous()
    real_slots = g.slots[rows.to(dev)].contiguous()
    gen = torch.Generator("cpu").manual_seed(77)
    junk = torch.randn((2,) + tuple(nk.shape), generator=gen).to(torch.bfloat16).to(dev)
    pa.reshape_and_cache(junk[0].contiguous(), junk[1].contiguous(), g.kc, g.vc, real_slots)
    slots = real_slots.clone()
    if skip is not None:
        slots[skip] = -1
    kc2, vc2 = g.kc.clone(), g.vc.clone()
    o1, l1 = pa.paged_decode_attn_write(g.q, nk, nv, slots, g.kc, g.vc, g.bt, g.cl, case.scale,
                                        g.max_ctx, partition_tokens=partition)
    pa.reshape_and_cache(nk, nv, kc2, vc2, slots)
    o2, l2 = pa.paged_decode_attn(g.q, kc2, vc2, g.bt, g.cl, case.scale, g.max_ctx,
                                  partition_tokens=partition)
    torch.cuda.synchronize()
    assert torch.equal(_t(o1), _t(o2)) and torch.equal(l1, l2), "output differs"
    assert torch.equal(_t(g.kc), _t(kc2)) and torch.equal(_t(g.vc), _t(vc2)), "cache differs"
    return g, o1, l1


@pytest.mark.parametrize("mk,partition", [
    (lambda: W.tiny_gqa(), -1),
    (lambda: W.tiny_gqa(), 128),
    (lambda: W.gqa_decode_case("fw", 205, [1, 16, 17, 64, 65, 300], Hq=8, Hkv=2, D=128,
                               block_size=16), 64),
    (lambda: W.gqa_decode_case("fw32", 206, [1, 31, 32, 33, 200], Hq=8, Hkv=4, D=64,
                               block_size=32), 0),
    (lambda: W.qwen3_decode(S=16), -2),
    (lambda: W.qwen3_decode(S=16), 256),
], ids=["tiny_unsplit", "tiny_p128", "edges_p64", "d64b32_auto", "qwen16_balanced",
        "qwen16_p256"])
def test_decode_fused_cache_write(orc, mk, partition):
    """A decode step in one launch equals the cache write followed by decode
    (bits), leaves the caches equal to the oracle's, and matches the oracle's
    attention."""
    case = mk()
    say(f"fused cache write + decode {case.name} partition {partition}")
    g, out, lse = _fused_vs_separate(case, partition)
    kc, vc = oracle_pins.oracle_cache(orc, case)
    assert np.array_equal(_bits(g.kc), kc) and np.array_equal(_bits(g.vc), vc)
    ref_out, ref_lse = oracle_gqa(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what=f"fused {case.name}")


@pytest.mark.parametrize("partition", [-1, 64, -2])
def test_decode_fused_cache_write_skipped_slot(partition):
    """A negative slot writes nothing, exactly like the separate cache write."""
    case = W.gqa_decode_case("fwskip", 207, [40, 3, 129], Hq=4, Hkv=1, D=128, block_size=16)
    _fused_vs_separate(case, partition, skip=1)


def test_latent_cache_write_bitexact(orc):
    cases = W.mla_decode_cases("lat", 204, S=3, lens_range=None, lens=[1, 70, 129], Hq=2, Dl=576,
                               Dv=512, block_sizes=(1, 64, 5), scale=0.1)
    dev = device()
    for B, case in cases.items():
        kv = torch.full((case.paging.num_blocks, B, 576), float("nan"), dtype=torch.bfloat16,
                        device=dev)
        pa.reshape_and_cache(case.latent.to(dev), None, kv, None,
                             torch.from_numpy(case.paging.slot_mapping).to(dev),
                             layout=pa.LAYOUT_MLA_LATENT)
        ref = np.full((case.paging.num_blocks, B, 576), 0x7FC0, dtype=np.uint16)
        orc.cache_write_latent(W.bf16_bits(case.latent), case.paging.slot_mapping, ref, B)
        assert np.array_equal(_bits(kv), ref), f"block size {B}"


# ---------------------------------------------------------------------------
# GQA decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("partition", [-1, 128, 0, 64])
def test_decode_tiny(orc, partition):
    case = W.tiny_gqa(partition_tokens=partition)
    say(f"decode tiny partition={partition}")
    g = GpuGQA(case)
    out, lse = g.decode()
    ref_out, ref_lse = oracle_gqa(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what=f"tiny P={partition}")


def test_decode_split_matches_unsplit():
    """128-token partitions + LSE merge equal the unsplit result."""
    case = W.tiny_gqa()
    g = GpuGQA(case)
    o1, l1 = g.decode(partition_tokens=-1)
    o2, l2 = g.decode(partition_tokens=128)
    torch.cuda.synchronize()
    d = (o1.float() - o2.float()).abs().max().item()
    dl = (l1 - l2).abs().max().item()
    say(f"  split vs unsplit: out {d:.3e} lse {dl:.3e}")
    assert d <= 1e-2 and dl <= 1e-4


EDGE_LENS = [1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 0, 300, 511]


@pytest.mark.parametrize("D,B,Hq,Hkv", [
    (128, 16, 4, 1), (128, 32, 8, 1), (64, 16, 2, 2), (64, 32, 16, 1),
    (128, 16, 3, 1), (128, 16, 12, 2), (128, 32, 64, 4), (128, 16, 5, 5),
])
@pytest.mark.parametrize("partition", [-1, 64, 256, 0, -2])
def test_decode_edges(orc, D, B, Hq, Hkv, partition):
    case = W.gqa_decode_case(f"edge_{D}_{B}_{Hq}_{Hkv}", 300 + D + B + Hq, EDGE_LENS, Hq=Hq,
                             Hkv=Hkv, D=D, block_size=B, partition_tokens=partition)
    say(f"decode edges D={D} B={B} Hq={Hq} Hkv={Hkv} P={partition}")
    g = GpuGQA(case)
    out, lse = g.decode()
    ref_out, ref_lse = oracle_gqa(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what=case.name)
    # the empty sequence: zero output, -inf lse
    s0 = EDGE_LENS.index(0)
    assert torch.all(out[s0] == 0) and torch.all(torch.isneginf(lse[s0]))


def test_decode_balanced_many_sequences(orc):
    """200 sequences (several 64-sequence scan windows of the balanced split),
    lengths U[0, 700] with a run of empty ones: every output vs the oracle."""
    rng = np.random.default_rng(77)
    lens = rng.integers(0, 701, size=200)
    lens[50:60] = 0
    case = W.gqa_decode_case("many", 305, lens.tolist(), Hq=8, Hkv=2, D=128, block_size=16)
    say("decode balanced 200 sequences")
    g = GpuGQA(case)
    out, lse = g.decode(partition_tokens=-2)
    ref_out, ref_lse = oracle_gqa(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what="balanced many sequences")


def test_decode_balanced_more_units_than_waves(orc):
    """1100 sequences x 4 kv heads: more (sequence, kv head) units than the
    grid has workgroups, so every unit is one piece and workgroups take several."""
    rng = np.random.default_rng(78)
    lens = rng.integers(0, 120, size=1100)
    case = W.gqa_decode_case("units", 306, lens.tolist(), Hq=8, Hkv=4, D=64, block_size=32)
    say("decode balanced 1100 sequences x 4 kv heads")
    g = GpuGQA(case)
    out, lse = g.decode(partition_tokens=-2)
    ref_out, ref_lse = oracle_gqa(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what="balanced, units > workgroups")


def test_decode_balanced_matches_partitioned():
    case = W.qwen3_decode(S=16)
    g = GpuGQA(case)
    o1, l1 = g.decode(partition_tokens=-2)
    o2, l2 = g.decode(partition_tokens=256)
    torch.cuda.synchronize()
    d = (o1.float() - o2.float()).abs().max().item()
    say(f"  balanced vs 256-token partitions: {d:.3e}")
    assert d <= 1e-2 and (l1 - l2).abs().max().item() <= 1e-4


def test_decode_block_permutation_bitexact():
    """Relabelling physical blocks changes no output bit."""
    case = W.tiny_gqa()
    g = GpuGQA(case)
    o1, l1 = g.decode(partition_tokens=128)
    dev = device()
    nb = case.paging.num_blocks
    perm = torch.from_numpy(np.random.default_rng(8).permutation(nb)).to(dev)
    kc2 = torch.empty_like(g.kc)
    vc2 = torch.empty_like(g.vc)
    kc2[perm] = g.kc
    vc2[perm] = g.vc
    bt2 = perm[g.bt.long()].to(torch.int32).contiguous()
    o2, l2 = pa.paged_decode_attn(g.q, kc2, vc2, bt2, g.cl, case.scale, g.max_ctx,
                                  partition_tokens=128)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_decode_deterministic():
    case = W.qwen3_decode(S=8)
    g = GpuGQA(case)
    o1, l1 = g.decode()
    o2, l2 = g.decode()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("partition", [0, 128, 64])
def test_decode_repeated_launches_identical(partition):
    """Which workgroup merges a split unit's partials depends on timing (the
    last to finish); the partitions combine in index order whoever merges,
    so 20 launches of the 64-request decode must agree bit for bit (8, 16
    and 32 partitions per request)."""
    case = W.qwen3_decode()
    g = GpuGQA(case)
    o1, l1 = g.decode(partition_tokens=partition)
    for _ in range(20):
        o2, l2 = g.decode(partition_tokens=partition)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_decode_qwen3_full(orc):
    """64 requests, GQA 8:1, lengths U[1000,2000]: every output vs the oracle."""
    case = W.qwen3_decode()
    say("decode qwen3 64-request full")
    g = GpuGQA(case)
    out, lse = g.decode()
    ref_out, ref_lse = oracle_gqa(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what="qwen3 full")


def test_decode_long_context_sampled(orc):
    """8 requests up to 131072 tokens, 2048-token partitions, K outliers:
    sampled (seq, head) rows (every kv head of every sequence) vs the oracle,
    plus partition-size invariance."""
    case = W.long_context_decode()
    say(f"decode long context, lens {case.context_lens.tolist()}")
    g = GpuGQA(case)
    out, lse = g.decode()
    rng = np.random.default_rng(31)
    mask = np.zeros((case.S, case.Hq), dtype=np.uint8)
    grp = case.Hq // case.Hkv
    for s in range(case.S):
        # one q head of every kv head's group, plus one more anywhere
        for kv in range(case.Hkv):
            mask[s, kv * grp + int(rng.integers(grp))] = 1
        mask[s, int(rng.integers(case.Hq))] = 1
    ref_out, ref_lse = oracle_gqa(orc, case, row_mask=mask)
    rows = np.nonzero(mask)
    assert_attn_close(out, lse, ref_out, ref_lse, rows=rows, what="long context sampled")
    for P in (8192, -2):
        o2, l2 = g.decode(partition_tokens=P)
        torch.cuda.synchronize()
        d = (out.float() - o2.float()).abs().max().item()
        say(f"  P=2048 vs P={P}: {d:.3e}")
        assert d <= 1e-2 and (lse - l2).abs().max().item() <= 1e-3


def test_decode_rejects_bad_args():
    case = W.tiny_gqa()
    g = GpuGQA(case)
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_decode_attn(g.q, g.kc, g.vc, g.bt, g.cl, float("nan"), g.max_ctx)
    assert e.value.status == 1
    with pytest.raises(ValueError):
        pa.paged_decode_attn(g.q, g.kc, g.vc, g.bt, g.cl, 0.1, g.max_ctx, partition_tokens=128,
                             workspace=torch.empty(16, dtype=torch.uint8, device=device()))
    with pytest.raises(ValueError):
        pa.paged_decode_attn(g.q.cpu(), g.kc, g.vc, g.bt, g.cl, 0.1, g.max_ctx)
