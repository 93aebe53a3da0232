"""GPU parity of the FP8 (E4M3) KV cache against the oracle (oracle/fp8.py):
the quantising cache write and the gather with dequantisation bit for bit,
decode over the FP8 caches to the usual tolerance, the fused write + decode
equal to the write followed by decode.  Calls go through the C ABI."""
import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
from oracle import fp8 as OF
from gpu_util import assert_attn_close, device, say

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 0, 300, 511]
KS, VS = 0.05, 0.07  # non-power-of-two scales: the products round


def _u8(t):
    return t.detach().cpu().numpy()


class GpuFp8:
    def __init__(self, case, k_scale=KS, v_scale=VS, slots=None):
        dev = device()
        pg = case.paging
        self.case, self.ks, self.vs = case, k_scale, v_scale
        self.kc = torch.full((pg.num_blocks, case.Hkv, case.D // 16, case.B, 16), 0x7F,
                             dtype=torch.uint8, device=dev)
        self.vc = torch.full((pg.num_blocks, case.Hkv, case.B // 16, case.D, 16), 0x7F,
                             dtype=torch.uint8, device=dev)
        self.slots_np = pg.slot_mapping if slots is None else slots
        self.slots = torch.from_numpy(self.slots_np).to(dev)
        pa.reshape_and_cache_fp8(case.key.to(dev), case.value.to(dev), self.kc, self.vc,
                                 self.slots, k_scale, v_scale)
        self.q = case.query.to(dev)
        self.bt = torch.from_numpy(pg.block_table).to(dev)
        self.cl = torch.from_numpy(pg.lens).to(dev)
        self.max_ctx = int(pg.lens.max()) if pg.S else 0

    def oracle_cache(self):
        pg = self.case.paging
        kc, vc = OF.empty_cache(pg.num_blocks, self.case.Hkv, self.case.D, self.case.B)
        OF.cache_write(W.bf16_bits(self.case.key), W.bf16_bits(self.case.value), self.slots_np,
                       kc, vc, self.ks, self.vs)
        return kc, vc

    def decode(self, partition, **kw):
        return pa.paged_decode_attn_fp8(self.q, self.kc, self.vc, self.bt, self.cl,
                                        self.case.scale, self.max_ctx, self.ks, self.vs,
                                        partition_tokens=partition, **kw)


@pytest.mark.parametrize("mk", [
    lambda: W.gqa_decode_case("f8w1", 601, [37, 100, 256, 511], Hq=4, Hkv=1, D=128, block_size=16),
    lambda: W.gqa_decode_case("f8w2", 602, [1, 31, 32, 33, 200], Hq=8, Hkv=4, D=64, block_size=32),
    lambda: W.gqa_decode_case("f8w3", 603, [5, 17, 64, 65], Hq=6, Hkv=3, D=128, block_size=16),
], ids=["d128b16", "d64b32_hkv4", "hkv3"])
def test_fp8_cache_write_bitexact(mk):
    case = mk()
    say(f"fp8 cache write {case.name}")
    slots = case.paging.slot_mapping.copy()
    slots[::5] = -1
    slots[2] = case.paging.num_blocks * case.B + 7
    g = GpuFp8(case, slots=slots)
    kc, vc = g.oracle_cache()
    assert np.array_equal(_u8(g.kc), kc) and np.array_equal(_u8(g.vc), vc)


def test_fp8_encoder_every_code_and_tie():
    """Scale 1: keys on every E4M3 value, every midpoint between neighbours
    (ties), the bf16 values either side of each midpoint, and out-of-range
    magnitudes; the GPU codes equal the oracle's."""
    dev = device()
    t = OF.decode_table()
    vals = []
    for c in range(0x7E):
        vals += [t[c], (t[c] + t[c + 1]) / 2]  # every value and every midpoint: all bf16
    vals += [448.0, 460.0, 464.0, 500.0, 1e4, 3e38, 2.0 ** -11, 2.0 ** -10, 0.0]
    mids = OF.bf16_rne(np.array(vals, dtype=np.float32))
    near = np.concatenate([mids + 1, mids[mids > 0] - 1]).astype(np.uint16)  # bf16 neighbours
    pos = np.concatenate([mids, near])
    bits = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    n = bits.size
    D = 128
    T = (n + D - 1) // D
    kb = np.zeros(T * D, dtype=np.uint16)
    kb[:n] = bits
    kb = kb.reshape(T, 1, D)
    key = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(dev)
    B = 16
    nb = (T + B - 1) // B
    kc = torch.full((nb, 1, D // 16, B, 16), 0x7F, dtype=torch.uint8, device=dev)
    vc = torch.full((nb, 1, B // 16, D, 16), 0x7F, dtype=torch.uint8, device=dev)
    slots = torch.arange(T, dtype=torch.int64, device=dev)
    pa.reshape_and_cache_fp8(key, key.clone(), kc, vc, slots, 1.0, 1.0)
    okc, ovc = OF.empty_cache(nb, 1, D, B)
    OF.cache_write(kb, kb, np.arange(T), okc, ovc, 1.0, 1.0)
    assert np.array_equal(_u8(kc), okc) and np.array_equal(_u8(vc), ovc)


CASES = [
    (lambda: W.gqa_decode_case("f8d_tiny", 611, [37, 100, 256, 511], Hq=4, Hkv=1, D=128,
                               block_size=16), -1),
    (lambda: W.gqa_decode_case("f8d_e1", 612, EDGE_LENS, Hq=8, Hkv=2, D=128, block_size=16), 64),
    (lambda: W.gqa_decode_case("f8d_e2", 613, EDGE_LENS, Hq=8, Hkv=2, D=128, block_size=16), -2),
    (lambda: W.gqa_decode_case("f8d_e3", 614, EDGE_LENS, Hq=16, Hkv=1, D=64, block_size=32), 0),
    (lambda: W.gqa_decode_case("f8d_e4", 615, EDGE_LENS, Hq=12, Hkv=4, D=128, block_size=32), 256),
    (lambda: W.gqa_decode_case("f8d_e5", 616, EDGE_LENS, Hq=5, Hkv=5, D=64, block_size=16), -1),
    (lambda: W.qwen3_decode(S=16), 256),
    (lambda: W.qwen3_decode(S=16), -2),
]
IDS = ["tiny_unsplit", "e128b16_p64", "e128b16_bal", "e64b32_g16_auto", "e128b32_hkv4_p256",
       "e64b16_mha", "qwen16_p256", "qwen16_bal"]


@pytest.mark.parametrize("mk,partition", CASES, ids=IDS)
def test_fp8_decode_vs_oracle(mk, partition):
    case = mk()
    say(f"fp8 decode {case.name} partition {partition}")
    g = GpuFp8(case)
    out, lse = g.decode(partition)
    torch.cuda.synchronize()
    kc, vc = g.oracle_cache()
    ref_out, ref_lse = OF.paged_decode_gqa(W.bf16_bits(case.query), kc, vc,
                                           case.paging.block_table, case.context_lens,
                                           case.scale, KS, VS)
    assert_attn_close(out, lse, ref_out, ref_lse, what=f"fp8 {case.name}")
    if 0 in list(case.context_lens):
        s0 = list(case.context_lens).index(0)
        assert torch.all(out[s0] == 0) and torch.all(torch.isneginf(lse[s0]))


def test_fp8_decode_qwen3_full_sampled():
    """The full 64-request workload, every request checked (the oracle's
    numpy decode is fast enough here)."""
    case = W.qwen3_decode()
    say("fp8 decode qwen3 64 requests")
    pg = case.paging
    amax = float(case.key.abs().max()), float(case.value.abs().max())
    ks, vs = amax[0] / 448.0, amax[1] / 448.0
    g = GpuFp8(case, ks, vs)
    out, lse = g.decode(256)
    torch.cuda.synchronize()
    kc, vc = g.oracle_cache()
    assert np.array_equal(_u8(g.kc), kc) and np.array_equal(_u8(g.vc), vc)
    seqs = list(range(0, 64, 3))
    ref_out, ref_lse = OF.paged_decode_gqa(W.bf16_bits(case.query), kc, vc, pg.block_table,
                                           case.context_lens, case.scale, ks, vs, seqs=seqs)
    assert_attn_close(out[seqs], lse[seqs], ref_out[seqs], ref_lse[seqs], what="fp8 qwen3")


@pytest.mark.parametrize("partition", [128, -2])
def test_fp8_fused_write(partition):
    case = W.gqa_decode_case("f8fw", 621, [1, 16, 17, 64, 65, 300, 0], Hq=8, Hkv=2, D=128,
                             block_size=16)
    say(f"fp8 fused write partition {partition}")
    dev = device()
    g = GpuFp8(case)
    rows = torch.from_numpy(case.new_token_rows())
    nk = case.key[rows].to(dev).contiguous()
    nv = case.value[rows].to(dev).contiguous()
    slots = g.slots[rows.to(dev)].contiguous()
    gen = torch.Generator("cpu").manual_seed(79)
    junk = torch.randn((2,) + tuple(nk.shape), generator=gen).to(torch.bfloat16).to(dev)
    pa.reshape_and_cache_fp8(junk[0].contiguous(), junk[1].contiguous(), g.kc, g.vc, slots, KS, VS)
    kc2, vc2 = g.kc.clone(), g.vc.clone()
    o1, l1 = g.decode(partition, new_key=nk, new_value=nv, slot_mapping=slots)
    pa.reshape_and_cache_fp8(nk, nv, kc2, vc2, slots, KS, VS)
    o2, l2 = pa.paged_decode_attn_fp8(g.q, kc2, vc2, g.bt, g.cl, case.scale, g.max_ctx, KS, VS,
                                      partition_tokens=partition)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert torch.equal(g.kc, kc2) and torch.equal(g.vc, vc2)
    kc, vc = g.oracle_cache()
    assert np.array_equal(_u8(g.kc), kc) and np.array_equal(_u8(g.vc), vc)


@pytest.mark.parametrize("chunk", [64, 256])
def test_fp8_gather_dequant_bitexact(chunk):
    case = W.gqa_decode_case("f8g", 631, [1, 100, 257, 0, 700], Hq=8, Hkv=2, D=128,
                             block_size=16)
    say(f"fp8 gather chunk {chunk}")
    g = GpuFp8(case)
    kc, vc = g.oracle_cache()
    its = (int(case.context_lens.max()) + chunk - 1) // chunk
    for it in range(its):
        ko, vo = pa.gather_cache_chunk_fp8(g.kc, g.vc, g.bt, g.cl, it, chunk, KS, VS)
        torch.cuda.synchronize()
        rk, rv = OF.gather_dequant(kc, vc, case.paging.block_table, case.context_lens, it, chunk,
                                   KS, VS)
        n = rk.shape[0]
        bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(bits(ko[:n]), rk) and np.array_equal(bits(vo[:n]), rv), it
