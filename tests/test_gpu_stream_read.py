"""The streaming-read yardstick kernel reads every byte once: the xor of its
per-workgroup words equals the xor of all 32-bit words of the buffer."""
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

