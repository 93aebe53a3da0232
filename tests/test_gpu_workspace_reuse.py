"""GPU: one workspace, zero-filled once, reused by a sequence of calls of
different shapes and entry points (GQA decode with fixed partitions and with
the balanced split, chunked extend, MLA decode on both engines, the mixed
batch).  Every call must give the same bits as the same call on a fresh
workspace, and leave the counter region at the start of the workspace zero.
Calls go through the C ABI.
"""
import math

import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
from gpu_util import GpuGQA, assert_attn_close, device, oracle_gqa, say
from test_gpu_extend import GpuExtend
from test_gpu_mla import GpuMLA
from test_gpu_router import run_routed

pytestmark = pytest.mark.gpu


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def test_workspace_reused_across_shapes_and_entry_points(orc):
    dev = device()
    ws = torch.zeros(96 << 20, dtype=torch.uint8, device=dev)
    counters = ws[:pa.WORKSPACE_COUNTER_BYTES]

    small = GpuGQA(W.gqa_decode_case("ws_s4", 231, [100, 700, 33, 1500], Hq=8, Hkv=2, D=128,
                                     block_size=16))
    big_case = W.gqa_decode_case("ws_s200", 232, None, Hq=16, Hkv=4, D=128, block_size=16,
                                 lens_range=(1, 600), S=200)
    big = GpuGQA(big_case)
    ext = GpuExtend(W.extend_case("ws_ext", 233, ctx_lens=[300, 0, 45, 700],
                                  new_tokens=[37, 5, 16, 130], Hq=8, Hkv=2, D=128,
                                  block_size=16, chunk_budget_tokens=128))
    mla = GpuMLA(W.mla_decode_cases("ws_mla", 234, S=6, lens_range=(1, 2000), Hq=16, Dl=576,
                                    Dv=512, block_sizes=(64,), scale=1.0 / math.sqrt(192.0))[64])
    routed = W.extend_case("ws_mixed", 235, ctx_lens=[40, 0, 300, 17, 0, 90],
                           new_tokens=[1, 9, 1, 30, 1, 1], Hq=8, Hkv=2, D=128, block_size=16,
                           chunk_budget_tokens=64)

    def gqa(g, partition):
        return lambda w: g.decode(partition, workspace=w)

    def mla_valu(w):
        return mla.decode(partition_tokens=64, workspace=w)

    def mla_mfma(w):
        return pa.mla_decode_attn_mfma(mla.q, mla.kv, mla.bt, mla.cl, mla.case.scale,
                                       mla.max_ctx, partition_tokens=-2, workspace=w)

    def routed_call(w):
        out, lse = run_routed(routed, workspace=w)[:2]
        return out, lse

    steps = [
        ("decode S=4 partition 64", gqa(small, 64)),
        ("decode S=200 balanced", gqa(big, -2)),
        ("extend", lambda w: ext.run(workspace=w)),
        ("decode S=4 balanced", gqa(small, -2)),
        ("MLA VALU partition 64", mla_valu),
        ("decode S=200 partition 128", gqa(big, 128)),
        ("MLA matrix cores balanced", mla_mfma),
        ("mixed batch", routed_call),
        ("decode S=200 auto", gqa(big, 0)),
        ("decode S=4 partition 64 again", gqa(small, 64)),
    ]
    for name, call in steps:
        say(f"workspace reuse: {name}")
        o1, l1 = call(ws)
        o2, l2 = call(None)  # a fresh zero-filled workspace
        torch.cuda.synchronize()
        assert _same(o1, o2) and _same(l1, l2), f"{name}: reused workspace changes the result"
        assert int(torch.count_nonzero(counters)) == 0, f"{name}: counter region left nonzero"

    # and the reused-workspace results are right, not merely repeatable
    out, lse = big.decode(-2, workspace=ws)
    mask = np.zeros((big_case.S, big_case.Hq), dtype=np.uint8)
    mask[::7] = 1
    ref_out, ref_lse = oracle_gqa(orc, big_case, row_mask=mask)
    assert_attn_close(out, lse, ref_out, ref_lse, rows=np.nonzero(mask),
                      what="decode S=200 balanced on a reused workspace")
