"""GPU: pa_paged_decode_attn_write_noalloc, whose workspace is the library's
own per-device array, against pa_paged_decode_attn_write with a caller
workspace.  Two calls in a row, the second smaller, each on fresh caches:
outputs, LSEs and the written caches must be bit-identical.  A call that
needs more than the array holds is refused before anything is enqueued.
Calls go through the C ABI.
"""
import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
from gpu_util import GpuGQA, assert_attn_close, device, oracle_gqa, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _fused_inputs(g):
    case = g.case
    dev = device()
    rows = torch.from_numpy(case.new_token_rows())
    nk = case.key[rows].to(dev).contiguous()
    nv = case.value[rows].to(dev).contiguous()
    slots = g.slots[rows.to(dev)].contiguous()
    return nk, nv, slots


def _noalloc_vs_workspace(case, partition, orc=None):
    say(f"noalloc vs workspace entry: {case.name} S={case.S} partition {partition}")
    dev = device()
    g = GpuGQA(case)
    nk, nv, slots = _fused_inputs(g)
    kc2, vc2 = g.kc.clone(), g.vc.clone()
    out = torch.empty_like(g.q)
    lse = torch.empty((case.S, case.Hq), dtype=torch.float32, device=dev)
    pa.paged_decode_attn_write_noalloc(g.q, nk, nv, slots, g.kc, g.vc, g.bt, g.cl, case.scale,
                                       g.max_ctx, partition_tokens=partition, out=out, lse=lse)
    o2, l2 = pa.paged_decode_attn_write(g.q, nk, nv, slots, kc2, vc2, g.bt, g.cl, case.scale,
                                        g.max_ctx, partition_tokens=partition)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(o2)), f"{case.name}: output differs"
    assert torch.equal(lse, l2), f"{case.name}: lse differs"
    assert torch.equal(_bits(g.kc), _bits(kc2)) and torch.equal(_bits(g.vc), _bits(vc2))
    if orc is not None:
        mask = np.zeros((case.S, case.Hq), dtype=np.uint8)
        mask[::5, ::3] = 1
        ref_out, ref_lse = oracle_gqa(orc, case, row_mask=mask)
        assert_attn_close(out, lse, ref_out, ref_lse, rows=np.nonzero(mask),
                          what=f"noalloc {case.name}")


def test_noalloc_two_calls_second_smaller(orc):
    # 1: the 64-request Qwen3 decode share with the balanced split
    _noalloc_vs_workspace(W.qwen3_decode(S=64), -2, orc)
    # 2: a smaller batch with fixed 64-token partitions (other counters, partials)
    small = W.gqa_decode_case("noalloc_small", 241, [1, 17, 300, 64, 1000, 65], Hq=8, Hkv=2,
                              D=128, block_size=16)
    _noalloc_vs_workspace(small, 64, orc)


def test_noalloc_refuses_a_call_beyond_the_array():
    """16 heads x 64 sequences x 64 partitions of 128-dim fp32 partials need
    more than the array: PA_ERR_WORKSPACE_TOO_SMALL, outputs untouched; the
    next call that fits still matches the workspace entry."""
    case = W.gqa_decode_case("noalloc_big", 242, None, S=64, lens_range=(1, 40), Hq=16, Hkv=2,
                             D=128, block_size=16)
    g = GpuGQA(case)
    nk, nv, slots = _fused_inputs(g)
    max_ctx, partition = 4096, 64
    need = pa.decode_workspace_size(case.S, case.Hq, case.Hkv, case.D, max_ctx, partition)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(g.q, 7.0)
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_decode_attn_write_noalloc(g.q, nk, nv, slots, g.kc, g.vc, g.bt, g.cl, case.scale,
                                           max_ctx, partition_tokens=partition, out=out)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    _noalloc_vs_workspace(case, -1)
