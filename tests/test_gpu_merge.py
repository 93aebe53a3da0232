"""GPU parity: pairwise LSE merge (merge_attn_states) vs the oracle's merge."""
import numpy as np
import pytest
import torch

import paged_attention_decode_reshape_amd as pa
from gpu_util import device, say

pytestmark = pytest.mark.gpu


def _case(T, H, D, seed, dt):
    g = torch.Generator().manual_seed(seed)
    po = torch.randn(T, H, D, generator=g)
    so = torch.randn(T, H, D, generator=g)
    pl = torch.randn(T, H, generator=g) * 5
    sl = torch.randn(T, H, generator=g) * 5
    # empty parts: one side, the other side, both
    pl[0, :] = -float("inf")
    sl[1, :] = -float("inf")
    pl[2, 0] = sl[2, 0] = -float("inf")
    sl[3, :] = pl[3, :]  # equal weights
    # an empty part holding garbage must not leak into the result
    po[0] = float("nan")
    return po.to(dt), pl, so.to(dt), sl


@pytest.mark.parametrize("in_dt,out_dt", [(torch.bfloat16, torch.bfloat16),
                                          (torch.float32, torch.float32),
                                          (torch.float32, torch.bfloat16),
                                          (torch.bfloat16, torch.float32)])
@pytest.mark.parametrize("T,H,D", [(37, 8, 128), (5, 3, 64), (4, 64, 128), (9, 2, 512)])
def test_merge_vs_oracle(orc, in_dt, out_dt, T, H, D):
    dev = device()
    po, pl, so, sl = _case(T, H, D, T * H + D, in_dt)
    out, lse = pa.merge_attn_states(po.to(dev), pl.to(dev), so.to(dev), sl.to(dev),
                                    out_dtype=out_dt)
    torch.cuda.synchronize()
    po64 = np.nan_to_num(po.double().numpy(), nan=0.0)  # the empty part's garbage has weight 0
    ref_o, ref_l = orc.merge(np.stack([po64, so.double().numpy()]),
                             np.stack([pl.double().numpy(), sl.double().numpy()]))
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    tol = 1e-2 if out_dt == torch.bfloat16 else 1e-5
    err = np.abs(o - ref_o).max()
    both = np.isneginf(l) & np.isneginf(ref_l)
    lerr = np.abs(np.where(both, 0.0, l) - np.where(both, 0.0, ref_l)).max()
    say(f"  merge {in_dt}->{out_dt} {T}x{H}x{D}: out {err:.3e} lse {lerr:.3e}")
    assert err <= tol * max(1.0, np.abs(ref_o).max()) and lerr <= 1e-5
    assert torch.all(out[2, 0].float() == 0) and torch.isneginf(lse[2, 0])


def test_merge_in_place():
    dev = device()
    po, pl, so, sl = _case(16, 4, 128, 5, torch.float32)
    ref, ref_l = pa.merge_attn_states(po.to(dev), pl.to(dev), so.to(dev), sl.to(dev))
    p = po.to(dev)
    pa.merge_attn_states(p, pl.to(dev), so.to(dev), sl.to(dev), out=p)
    torch.cuda.synchronize()
    assert torch.equal(p, ref)
