"""GPU: three-path routing of a mixed batch (decode, extend and prefill
requests in one call) against the oracle's extend definition, which covers
all three (a decode request is one new token over its cached context, a
prefill request new tokens over nothing cached).  Calls go through the C ABI.
"""
import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W
import oracle_pins
from gpu_util import assert_attn_close, device, empty_gpu_cache, say

pytestmark = pytest.mark.gpu


def run_routed(case, workspace=None):
    """Write the cached tokens, reorder the batch with the plan, run the
    routed call; returns (out, lse) in the case's own request order."""
    dev = device()
    pg = case.paging
    R = case.S
    new_rows = case.new_rows()
    is_new = np.zeros(pg.total_tokens, dtype=bool)
    is_new[new_rows] = True
    kc, vc = empty_gpu_cache(pg.num_blocks, case.Hkv, case.D, case.B, dev)
    cached = np.nonzero(~is_new)[0]
    if cached.size:
        pa.reshape_and_cache(case.key[cached].to(dev), case.value[cached].to(dev), kc, vc,
                             torch.from_numpy(pg.slot_mapping[cached]).to(dev))
    qsl = case.query_start_loc
    order, counts = pa.mixed_batch_plan(qsl, case.ctx_lens)
    q_rows, n_rows, new_qsl = [], [], [0]
    starts = np.cumsum(np.concatenate([[0], case.new_lens]))
    for r in order:
        q_rows.append(np.arange(qsl[r], qsl[r + 1]))
        n_rows.append(new_rows[starts[r]:starts[r + 1]])
        new_qsl.append(new_qsl[-1] + int(case.new_lens[r]))
    q_rows = np.concatenate(q_rows)
    n_rows = np.concatenate(n_rows)
    new_qsl = np.asarray(new_qsl, dtype=np.int32)
    ctx = case.ctx_lens[order].astype(np.int32)
    q = case.query[torch.from_numpy(q_rows)].to(dev).contiguous()
    k = case.key[torch.from_numpy(n_rows)].to(dev).contiguous()
    v = case.value[torch.from_numpy(n_rows)].to(dev).contiguous()
    slots = torch.from_numpy(pg.slot_mapping[n_rows]).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(pg.block_table[order])).to(dev)
    out, lse = pa.mixed_batch_attn(q, k, v, slots, torch.from_numpy(new_qsl).to(dev),
                                   torch.from_numpy(ctx).to(dev), kc, vc, bt, case.scale,
                                   new_qsl, ctx, chunk_budget_tokens=case.chunk_budget_tokens,
                                   workspace=workspace)
    torch.cuda.synchronize()
    # back to the case's order
    inv = torch.empty(len(q_rows), dtype=torch.long)
    inv[torch.from_numpy(q_rows)] = torch.arange(len(q_rows))
    return out.cpu()[inv], lse.cpu()[inv], order, counts, kc, vc


def oracle_extend(orc, case):
    kc, vc, kn, vn = oracle_pins.extend_oracle_inputs(orc, case)
    return orc.extend(W.bf16_bits(case.query), kn, vn, case.query_start_loc, kc, vc,
                      case.paging.block_table, case.ctx_lens, case.B, case.scale)


MIXES = {
    # interleaved decode / extend / prefill, a one-token prompt (decode over itself)
    "mixed": dict(ctx_lens=[37, 300, 500, 0, 64, 0, 1000, 0, 129, 2],
                  new_tokens=[1, 37, 1, 100, 2, 7, 1, 1, 129, 300], Hq=8, Hkv=2, block_size=16),
    "mixed_b32_no_extend": dict(ctx_lens=[0, 700, 0, 31, 33], new_tokens=[64, 1, 3, 1, 1],
                                Hq=16, Hkv=1, block_size=32),
    "decode_only": dict(ctx_lens=[5, 16, 17, 400], new_tokens=[1, 1, 1, 1], Hq=4, Hkv=1,
                        block_size=16),
    "extend_only_budget": dict(ctx_lens=[900, 2500], new_tokens=[40, 130], Hq=4, Hkv=1,
                               block_size=16, chunk_budget_tokens=512),
}


@pytest.mark.parametrize("name", list(MIXES))
def test_routed_batch_vs_oracle(orc, name):
    kw = dict(MIXES[name])
    case = W.extend_case(f"route_{name}", 400 + len(name), D=128, **kw)
    say(f"routed batch {name}: ctx {list(case.ctx_lens)} new {list(case.new_lens)}")
    out, lse, order, counts, kc, vc = run_routed(case)
    n = case.new_lens
    assert counts[0] == np.sum(n == 1)
    assert counts[2] == np.sum((n > 1) & (case.ctx_lens == 0))
    ref_out, ref_lse = oracle_extend(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what=f"routed {name}")
    # the routed call wrote every new token: the caches equal the oracle's
    okc, ovc = oracle_pins.oracle_cache(orc, case)
    bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits(kc), okc) and np.array_equal(bits(vc), ovc)


def test_routed_serving_mix(orc):
    """A serving-shaped step: 60 decode requests (contexts U[1000,2000]), 3
    extend requests (256 new tokens over 4000 cached), 1 prefill of 512."""
    rng = np.random.default_rng(9)
    ctx = list(rng.integers(1000, 2001, size=60)) + [4000, 4100, 3900, 0]
    new = [1] * 60 + [256, 256, 256, 512]
    perm = rng.permutation(len(ctx))
    case = W.extend_case("route_serving", 431, ctx_lens=[ctx[i] for i in perm],
                         new_tokens=[new[i] for i in perm], Hq=8, Hkv=1, D=128, block_size=16)
    say("routed serving mix: 60 decode + 3 extend + 1 prefill")
    out, lse, order, counts, _, _ = run_routed(case)
    assert list(counts) == [60, 3, 1]
    ref_out, ref_lse = oracle_extend(orc, case)
    assert_attn_close(out, lse, ref_out, ref_lse, what="routed serving mix")
