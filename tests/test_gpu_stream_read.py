"""The read yardsticks: the streaming read reads every byte once (the xor of
its per-workgroup words equals the xor of all 32-bit words of the buffer);
the gather read reads exactly the K and V units of the blocks a decode
reads (each workgroup's word equals the xor of its blocks' units)."""
import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,workgroups", [(16, 1), (4096, 3), (1 << 20, 256),
                                               ((1 << 20) + 48, 7), (12345 * 16, 4096)])
def test_stream_read_covers_every_word(nbytes, workgroups):
    rng = np.random.default_rng(nbytes + workgroups)
    host = rng.integers(-2**31, 2**31 - 1, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).cuda()
    sink = pa.stream_read(src, workgroups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy()[:workgroups].view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert got == want



def _gather_want(kc, vc, bt, lens, B):
    """Per-workgroup xor words of the gather read, from the host copies."""
    NB, Hkv = kc.shape[:2]
    S, maxb = lens.shape[0], bt.shape[1]
    ku = kc.reshape(NB, Hkv, -1).view(np.uint32)
    vu = vc.reshape(NB, Hkv, -1).view(np.uint32)
    units = S * Hkv
    want = np.zeros(units * ((maxb + 3) // 4), dtype=np.uint32)
    for b4 in range((maxb + 3) // 4):
        for s in range(S):
            ctx = min(max(int(lens[s]), 0), maxb * B)
            for g in range(Hkv):
                w = np.uint32(0)
                for b in range(4 * b4, min(4 * b4 + 4, maxb)):
                    blk = int(bt[s, b])
                    if b * B < ctx and 0 <= blk < NB:
                        w ^= np.bitwise_xor.reduce(ku[blk, g]) ^ np.bitwise_xor.reduce(vu[blk, g])
                want[b4 * units + s * Hkv + g] = w
    return want


@pytest.mark.parametrize("D,B,Hkv,lens", [
    (128, 16, 1, [37, 100, 256, 511, 0]),
    (128, 32, 2, [1, 64, 65, 300]),
    (64, 16, 4, [17, 48, 2000]),
])
def test_gather_read_reads_the_decode_blocks(D, B, Hkv, lens):
    rng = np.random.default_rng(D + B + Hkv)
    lens = np.array(lens, dtype=np.int32)
    S = lens.shape[0]
    maxb = int(np.ceil(max(lens.max(), 1) / B)) + 1
    NB = S * maxb + 3
    kc = rng.integers(0, 2**16, size=(NB, Hkv, D // 8, B, 8), dtype=np.int64).astype(np.uint16)
    vc = rng.integers(0, 2**16, size=(NB, Hkv, B // 8, D, 8), dtype=np.int64).astype(np.uint16)
    bt = rng.permutation(NB)[:S * maxb].reshape(S, maxb).astype(np.int32)
    bt[0, -1] = -1          # entries past the context and invalid ids are not read
    bt[-1, 0] = NB + 5
    dev = torch.device("cuda")
    as_t = lambda a: torch.from_numpy(a.view(np.int16)).to(dev)
    sink = pa.gather_read(as_t(kc), as_t(vc), torch.from_numpy(bt).to(dev),
                          torch.from_numpy(lens).to(dev))
    torch.cuda.synchronize()
    want = _gather_want(kc, vc, bt, lens, B)
    assert np.array_equal(sink.cpu().numpy()[:want.size].view(np.uint32), want)
