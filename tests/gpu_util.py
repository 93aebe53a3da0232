"""Helpers for the GPU parity tests: upload seeded cases, build the GPU
caches with the library's own cache write, and compare against the oracle
under the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import workloads as W

# bf16 outputs vs the fp64 oracle: max abs <= 1e-2, max rel <= 2e-2 with the
# relative error's denominator floored at 1e-2; LSE max abs <= 1e-3.
ATOL = 1e-2
RTOL = 2e-2
REL_FLOOR = 1e-2
LSE_ATOL = 1e-3


def device() -> torch.device:
    assert torch.cuda.is_available(), "GPU tests need an MI355X; none is visible"
    return torch.device("cuda:0")


def say(msg: str):
    print(msg, flush=True)


def empty_gpu_cache(num_blocks, Hkv, D, B, dev, fill=float("nan")):
    kc = torch.full((num_blocks, Hkv, D // 8, B, 8), fill, dtype=torch.bfloat16, device=dev)
    vc = torch.full((num_blocks, Hkv, B // 8, D, 8), fill, dtype=torch.bfloat16, device=dev)
    return kc, vc


class GpuGQA:
    """A GQA decode case on the GPU, caches filled by pa.reshape_and_cache."""

    def __init__(self, case: W.GQADecodeCase, dev=None):
        dev = dev or device()
        self.case = case
        pg = case.paging
        self.kc, self.vc = empty_gpu_cache(pg.num_blocks, case.Hkv, case.D, case.B, dev)
        self.slots = torch.from_numpy(pg.slot_mapping).to(dev)
        key = case.key.to(dev)
        value = case.value.to(dev)
        pa.reshape_and_cache(key, value, self.kc, self.vc, self.slots)
        del key, value
        self.q = case.query.to(dev)
        self.bt = torch.from_numpy(pg.block_table).to(dev)
        self.cl = torch.from_numpy(pg.lens).to(dev)
        self.max_ctx = int(pg.lens.max()) if pg.S else 0

    def decode(self, partition_tokens=None, **kw):
        pt = self.case.partition_tokens if partition_tokens is None else partition_tokens
        return pa.paged_decode_attn(self.q, self.kc, self.vc, self.bt, self.cl, self.case.scale,
                                    self.max_ctx, partition_tokens=pt, **kw)


def oracle_gqa(orc, case: W.GQADecodeCase, row_mask=None):
    import oracle_pins
    kc, vc = oracle_pins.oracle_cache(orc, case)
    return orc.paged_decode_gqa(W.bf16_bits(case.query), kc, vc, case.paging.block_table,
                                case.context_lens, case.B, case.scale, row_mask=row_mask)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def attn_errors(out, lse, ref_out, ref_lse, rows=None):
    """(max abs, max floored rel, max lse abs) over the selected rows."""
    o = to_f64(out)
    r = np.asarray(ref_out)
    if rows is not None:
        o, r = o[rows], r[rows]
    err = np.abs(o - r)
    rel = err / np.maximum(np.abs(r), REL_FLOOR)
    e_lse = 0.0
    if lse is not None:
        l = to_f64(lse)
        rl = np.asarray(ref_lse)
        if rows is not None:
            l, rl = l[rows], rl[rows]
        both = np.isneginf(l) & np.isneginf(rl)
        # mask the rows where both are -inf before subtracting
        d = np.abs(np.where(both, 0.0, l) - np.where(both, 0.0, rl))
        e_lse = float(np.max(d)) if l.size else 0.0
    if err.size == 0:
        return 0.0, 0.0, e_lse
    return float(np.nanmax(err)) if not np.isnan(err).any() else float("nan"), \
        float(np.max(rel)) if not np.isnan(rel).any() else float("nan"), e_lse


def assert_attn_close(out, lse, ref_out, ref_lse, rows=None, what=""):
    e_abs, e_rel, e_lse = attn_errors(out, lse, ref_out, ref_lse, rows)
    say(f"  {what}: max abs {e_abs:.3e}  max rel {e_rel:.3e}  lse abs {e_lse:.3e}")
    assert e_abs <= ATOL, f"{what}: max abs {e_abs}"
    assert e_rel <= RTOL, f"{what}: max rel {e_rel}"
    assert e_lse <= LSE_ATOL, f"{what}: lse abs {e_lse}"
