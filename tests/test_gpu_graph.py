"""HIP graphs: every step captured once and replayed several times, with
eager work and synchronisation between replays, gives the eager result bit
for bit each time.  The library allocates nothing and clears what it needs
with its own kernels (no memset nodes), so a whole step can be captured.
Outputs and workspaces are allocated before capture."""
import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
from gpu_util import GpuGQA, device, say

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def check_graph(step, outs, restore=None):
    """step(): launches into preallocated outs; restore(): resets inputs a
    step modifies (caches) before each run."""
    if restore:
        restore()
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream
        if restore:
            restore()
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    if restore:
        restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o in outs:  # eager work between replays
            o.zero_()
        if restore:
            restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert _same(o, r), f"replay {i} differs"


@pytest.mark.parametrize("partition", [256, -2])
def test_graph_fused_decode_step(partition):
    case = W.qwen3_decode(S=32)
    say(f"graph: fused GQA decode step P={partition}")
    g = GpuGQA(case)
    dev = device()
    rows = torch.from_numpy(case.new_token_rows()).to(dev)
    nk = case.key[rows.cpu()].to(dev).contiguous()
    nv = case.value[rows.cpu()].to(dev).contiguous()
    slots = g.slots[rows].contiguous()
    out = torch.empty_like(g.q)
    lse = torch.empty((case.S, case.Hq), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(1, pa.decode_workspace_size(case.S, case.Hq, case.Hkv, case.D,
                                                     g.max_ctx, partition)),
                     dtype=torch.uint8, device=dev)

    def step():
        pa.paged_decode_attn_write(g.q, nk, nv, slots, g.kc, g.vc, g.bt, g.cl, case.scale,
                                   g.max_ctx, partition_tokens=partition, out=out, lse=lse,
                                   workspace=ws)
    check_graph(step, [out, lse])


def test_graph_fp8_decode_step():
    case = W.qwen3_decode(S=16)
    say("graph: fused FP8 decode step")
    dev = device()
    pg = case.paging
    kc = torch.zeros((pg.num_blocks, 1, 8, 16, 16), dtype=torch.uint8, device=dev)
    vc = torch.zeros((pg.num_blocks, 1, 1, 128, 16), dtype=torch.uint8, device=dev)
    slots_all = torch.from_numpy(pg.slot_mapping).to(dev)
    pa.reshape_and_cache_fp8(case.key.to(dev), case.value.to(dev), kc, vc, slots_all, 0.02, 0.03)
    rows = torch.from_numpy(case.new_token_rows())
    nk = case.key[rows].to(dev).contiguous()
    nv = case.value[rows].to(dev).contiguous()
    slots = slots_all[rows.to(dev)].contiguous()
    q = case.query.to(dev)
    bt = torch.from_numpy(pg.block_table).to(dev)
    cl = torch.from_numpy(pg.lens).to(dev)
    mc = int(pg.lens.max())
    out = torch.empty_like(q)
    lse = torch.empty((case.S, case.Hq), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(1, pa.decode_workspace_size(case.S, case.Hq, 1, 128, mc, 0)),
                     dtype=torch.uint8, device=dev)

    def step():
        pa.paged_decode_attn_fp8(q, kc, vc, bt, cl, case.scale, mc, 0.02, 0.03, new_key=nk,
                                 new_value=nv, slot_mapping=slots, out=out, lse=lse, workspace=ws)
    check_graph(step, [out, lse])


def test_graph_mla_step():
    case = W.deepseek_mla_decode(S=16, block_sizes=(64,))[64]
    say("graph: fused MLA decode step")
    dev = device()
    pg = case.paging
    kv = torch.zeros((pg.num_blocks, 64, 576), dtype=torch.bfloat16, device=dev)
    slots_all = torch.from_numpy(pg.slot_mapping).to(dev)
    pa.reshape_and_cache(case.latent.to(dev), None, kv, None, slots_all,
                         layout=pa.LAYOUT_MLA_LATENT)
    starts = np.concatenate([[0], np.cumsum(pg.lens)[:-1]])
    rows = torch.from_numpy((starts + pg.lens - 1).astype(np.int64))
    nl = case.latent[rows].to(dev).contiguous()
    slots = slots_all[rows.to(dev)].contiguous()
    q = case.query.to(dev)
    bt = torch.from_numpy(pg.block_table).to(dev)
    cl = torch.from_numpy(pg.lens).to(dev)
    mc = int(pg.lens.max())
    out = torch.empty((case.S, case.Hq, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((case.S, case.Hq), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(1, pa.mla_workspace_size(case.S, case.Hq, 512, mc, 0)),
                     dtype=torch.uint8, device=dev)

    def step():
        pa.mla_decode_attn_write(q, nl, slots, kv, bt, cl, case.scale, mc, out=out, lse=lse,
                                 workspace=ws)
    check_graph(step, [out, lse])


@pytest.mark.parametrize("engine", ["valu", "mfma"])
def test_graph_mla_fp8_step(engine):
    """The fused MLA decode step over an FP8 latent cache (the quantised
    write of the new latents included), captured and replayed, on either
    engine."""
    case = W.deepseek_mla_decode(S=16, block_sizes=(64,))[64]
    say(f"graph: fused MLA decode step, FP8 cache, {engine} engine")
    fn = pa.mla_decode_attn_fp8_mfma if engine == "mfma" else pa.mla_decode_attn_fp8
    dev = device()
    pg = case.paging
    kvs = float(np.float32(case.latent.float().abs().max().item() / 448.0))
    kv = torch.zeros((pg.num_blocks, 64, 576), dtype=torch.uint8, device=dev)
    slots_all = torch.from_numpy(pg.slot_mapping).to(dev)
    pa.reshape_and_cache_mla_fp8(case.latent.to(dev), kv, slots_all, kvs)
    rows = torch.from_numpy(case.new_token_rows())
    nl = case.latent[rows].to(dev).contiguous()
    slots = slots_all[rows.to(dev)].contiguous()
    q = case.query.to(dev)
    bt = torch.from_numpy(pg.block_table).to(dev)
    cl = torch.from_numpy(pg.lens).to(dev)
    mc = int(pg.lens.max())
    out = torch.empty((case.S, case.Hq, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((case.S, case.Hq), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(1, pa.mla_workspace_size(case.S, case.Hq, 512, mc, 0)),
                     dtype=torch.uint8, device=dev)

    kv_exp = kv.clone()  # the cache after the step's write (the same every replay)
    pa.reshape_and_cache_mla_fp8(nl, kv_exp, slots, kvs)

    def step():
        fn(q, kv, bt, cl, case.scale, mc, kvs, new_latent=nl, slot_mapping=slots, out=out,
           lse=lse, workspace=ws)
    check_graph(step, [out, lse])
    assert torch.equal(kv, kv_exp)


def test_graph_extend_and_routed_batch():
    case = W.extend_case("graph_ext", 801, ctx_lens=[300, 0, 1000, 64], new_tokens=[37, 100, 1, 2],
                         Hq=8, Hkv=2, D=128, block_size=16, chunk_budget_tokens=512)
    say("graph: chunked extend, then the routed mixed batch")
    dev = device()
    pg = case.paging
    kc = torch.zeros((pg.num_blocks, 2, 16, 16, 8), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((pg.num_blocks, 2, 2, 128, 8), dtype=torch.bfloat16, device=dev)
    pa.reshape_and_cache(case.key.to(dev), case.value.to(dev), kc, vc,
                         torch.from_numpy(pg.slot_mapping).to(dev))
    rows = torch.from_numpy(case.new_rows())
    kn = case.key[rows].to(dev).contiguous()
    vn = case.value[rows].to(dev).contiguous()
    q = case.query.to(dev)
    qsl = torch.from_numpy(case.query_start_loc).to(dev)
    bt = torch.from_numpy(pg.block_table).to(dev)
    cl = torch.from_numpy(case.ctx_lens).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], case.Hq), dtype=torch.float32, device=dev)
    nb = pa.extend_workspace_size(case.S, q.shape[0], case.Hq, case.Hkv, case.D, case.B, 512)
    ws = torch.zeros(max(1, nb), dtype=torch.uint8, device=dev)

    def step():
        pa.chunked_extend_attn(q, kn, vn, qsl, kc, vc, bt, cl, case.scale, case.query_start_loc,
                               case.ctx_lens, chunk_budget_tokens=512, out=out, lse=lse,
                               workspace=ws)
    check_graph(step, [out, lse])

    # the same requests through the router, reordered
    order, _ = pa.mixed_batch_plan(case.query_start_loc, case.ctx_lens)
    qs = case.query_start_loc
    starts = np.cumsum(np.concatenate([[0], case.new_lens]))
    q_rows = np.concatenate([np.arange(qs[r], qs[r + 1]) for r in order])
    n_rows = np.concatenate([case.new_rows()[starts[r]:starts[r + 1]] for r in order])
    new_qsl = np.concatenate([[0], np.cumsum(case.new_lens[order])]).astype(np.int32)
    ctx = case.ctx_lens[order].astype(np.int32)
    q2 = case.query[torch.from_numpy(q_rows)].to(dev).contiguous()
    k2 = case.key[torch.from_numpy(n_rows)].to(dev).contiguous()
    v2 = case.value[torch.from_numpy(n_rows)].to(dev).contiguous()
    s2 = torch.from_numpy(pg.slot_mapping[n_rows]).to(dev)
    bt2 = torch.from_numpy(np.ascontiguousarray(pg.block_table[order])).to(dev)
    qsl2 = torch.from_numpy(new_qsl).to(dev)
    ctx2 = torch.from_numpy(ctx).to(dev)
    out2 = torch.empty_like(q2)
    lse2 = torch.empty((q2.shape[0], case.Hq), dtype=torch.float32, device=dev)
    nb2 = int(pa.library().pa_mixed_batch_workspace_size(len(ctx), new_qsl.ctypes.data,
                                                         ctx.ctypes.data, case.Hq, case.Hkv,
                                                         case.D, case.B, 512))
    ws2 = torch.zeros(max(1, nb2), dtype=torch.uint8, device=dev)

    def routed():
        pa.mixed_batch_attn(q2, k2, v2, s2, qsl2, ctx2, kc, vc, bt2, case.scale, new_qsl, ctx,
                            chunk_budget_tokens=512, out=out2, lse=lse2, workspace=ws2)
    check_graph(routed, [out2, lse2])
