"""The C ABI on the CPU: every declared symbol is exported, and argument
checks return their status before anything is enqueued (no GPU needed; only
argument combinations that fail validation are passed, so no kernel is
ever launched from these tests)."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_attention_decode_reshape_amd as pa
from paged_attention_decode_reshape_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
FAKE = 0x10000  # aligned non-null address; never dereferenced by a failing call


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def test_header_declares_the_five_operations():
    names = declared_functions()
    for op in ("reshape_and_cache", "paged_decode_attn", "mla_decode_attn",
               "chunked_extend_attn", "merge_attn_states"):
        assert f"pa_{op}" in names
        assert hasattr(pa, op)


def test_library_exports_every_declared_symbol():
    lib = pa.library()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) <= set(ops._SIGS)


def test_status_strings():
    lib = pa.library()
    assert lib.pa_status_string(0) == b"ok"
    assert lib.pa_status_string(3) == b"workspace too small"


def _decode(lib, **kw):
    a = dict(out=FAKE, lse=None, query=FAKE, k=FAKE, v=FAKE, bt=FAKE, maxb=8, cl=FAKE, maxctx=100,
             S=4, Hq=8, Hkv=1, D=128, B=16, NB=64, scale=0.1, P=0, ws=None, wsb=0)
    a.update(kw)
    return lib.pa_paged_decode_attn(a["out"], a["lse"], a["query"], a["k"], a["v"], a["bt"],
                                    a["maxb"], a["cl"], a["maxctx"], a["S"], a["Hq"], a["Hkv"],
                                    a["D"], a["B"], a["NB"], a["scale"], a["P"], a["ws"], a["wsb"],
                                    None)


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), INVALID),
    (dict(k=FAKE + 8), INVALID),                      # cache not 16-byte aligned
    (dict(Hq=6, Hkv=4), INVALID),                     # group not integral
    (dict(scale=float("inf")), INVALID),
    (dict(D=96), UNSUPPORTED),
    (dict(B=8), UNSUPPORTED),
    (dict(Hq=32, Hkv=1), UNSUPPORTED),                # group 32 > 16
    (dict(maxctx=(1 << 20) + 1, P=-1), UNSUPPORTED),
    (dict(P=-3), INVALID),
    (dict(P=-2), WS_SMALL),                           # the balanced split needs a workspace
    (dict(maxctx=1000, P=128), WS_SMALL),             # 8 partitions need a workspace
    (dict(maxctx=1000, P=128, ws=FAKE, wsb=100), WS_SMALL),
])
def test_decode_validation(kw, status):
    assert _decode(pa.library(), **kw) == status


def test_decode_workspace_sizes():
    assert pa.decode_partition_tokens(4, 1, 511, 128) == 128
    assert pa.decode_partition_tokens(4, 1, 511, 100) == 128   # rounded up to 64
    assert pa.decode_partition_tokens(4, 1, 511, -1) == 512
    assert pa.decode_partition_tokens(64, 1, 2000, 0) == 256
    assert pa.decode_partition_tokens(8, 4, 131072, 8192) == 4096
    assert pa.decode_partition_tokens(1, 1, 100000, -1) == 4096
    assert pa.decode_workspace_size(4, 4, 1, 128, 511, -1) == 0
    # balanced split: the fixed counter region + one partial per workgroup
    # (at most four workgroups per compute unit; 256 CUs where no device is visible)
    cus = 256
    try:
        import torch
        if torch.cuda.is_available():
            cus = torch.cuda.get_device_properties(0).multi_processor_count
    except Exception:
        pass
    a256 = lambda n: (n + 255) // 256 * 256
    nw = 4 * cus
    region = pa.WORKSPACE_COUNTER_BYTES
    assert region == 1 << 20
    assert pa.decode_workspace_size(64, 8, 1, 128, 2000, -2) == \
        region + a256(nw * 8 * 128 * 4) + a256(nw * 8 * 4)
    # auto: 64 x 8 partitions of 256 tokens fit in one wave of workgroups;
    # 32 x 32 partitions of 4096 tokens do not
    assert not pa.decode_uses_balanced_split(64, 1, 2000, 0)
    assert pa.decode_uses_balanced_split(8, 4, 131072, 0)
    assert pa.decode_uses_balanced_split(8, 4, 131072, -2)
    assert not pa.decode_uses_balanced_split(8, 4, 131072, 2048)
    parts = 4  # 511 tokens in 128-token partitions
    a256 = lambda n: (n + 255) // 256 * 256
    want = region + a256(4 * 4 * parts * 128 * 4) + a256(4 * 4 * parts * 4)
    assert pa.decode_workspace_size(4, 4, 1, 128, 511, 128) == want
    # the counter region holds one counter per (sequence, kv head) of a split call
    cap = region // 4
    # auto with more pairs than counters: fixed partitions, unsplit up to 4096 tokens
    assert not pa.decode_uses_balanced_split(cap // 8 + 1, 8, 4096, 0)
    assert pa.decode_workspace_size(cap // 8 + 1, 64, 8, 128, 4096, 0) == 0
    assert pa.decode_uses_balanced_split(cap // 8, 8, 4096, 0)
    # the extend workspace also starts with the (untouched) counter region
    assert pa.extend_workspace_size(1, 8, 8, 2, 128, 16, 4096) > region


def test_split_beyond_counter_capacity_is_unsupported():
    """A split decode call with more (sequence, kv head) pairs than the
    counter region holds returns PA_ERR_UNSUPPORTED before any launch."""
    lib = pa.library()
    S = pa.WORKSPACE_COUNTER_BYTES // 4 // 8 + 1     # 8 kv heads
    big = 1 << 40
    for P in (-2, 256):
        assert _decode(lib, S=S, Hq=8, Hkv=8, maxctx=4096, P=P, ws=FAKE, wsb=big) == UNSUPPORTED


def test_fused_decode_validation():
    f = pa.library().pa_paged_decode_attn_write
    args = lambda nk, nv, sl: (FAKE, None, FAKE, nk, nv, sl, FAKE, FAKE, FAKE, 8, FAKE, 100, 4, 8, 1,
                               128, 16, 64, 0.1, -1, None, 0, None)
    assert f(*args(None, FAKE, FAKE)) == INVALID          # no new key
    assert f(*args(FAKE, FAKE, None)) == INVALID          # no slot mapping
    assert f(*args(FAKE + 8, FAKE, FAKE)) == INVALID      # new key not 16-byte aligned
    assert f(*args(FAKE, FAKE, FAKE + 4)) == INVALID      # slots not 8-byte aligned
    bad = list(args(FAKE, FAKE, FAKE))
    bad[15] = 96                                          # head_dim
    assert f(*bad) == UNSUPPORTED


def test_fused_mla_validation():
    f = pa.library().pa_mla_decode_attn_write
    args = lambda nl, sl: (FAKE, None, FAKE, nl, sl, FAKE, FAKE, 8, FAKE, 100, 4, 16, 576, 512, 64,
                           64, 0.1, -1, None, 0, None)
    assert f(*args(None, FAKE)) == INVALID                # no new latent
    assert f(*args(FAKE, None)) == INVALID                # no slot mapping
    assert f(*args(FAKE + 8, FAKE)) == INVALID            # latent not 16-byte aligned
    bad = list(args(FAKE, FAKE))
    bad[12] = 512                                         # latent_dim
    assert f(*bad) == UNSUPPORTED


def test_cache_write_validation():
    lib = pa.library()
    f = lib.pa_reshape_and_cache
    assert f(0, FAKE, None, FAKE, FAKE, FAKE, 4, 1, 128, 16, 8, None) == INVALID   # value NULL
    assert f(0, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1, 96, 16, 8, None) == UNSUPPORTED
    assert f(0, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1, 128, 24, 8, None) == UNSUPPORTED
    assert f(1, FAKE, FAKE, FAKE, None, FAKE, 4, 1, 576, 1, 8, None) == INVALID    # MLA + value
    assert f(1, FAKE, None, FAKE, None, FAKE, 4, 2, 576, 1, 8, None) == INVALID    # MLA Hkv != 1
    assert f(7, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1, 128, 16, 8, None) == INVALID   # bad layout
    assert f(0, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 1, 128, 16, 8, None) == INVALID
    assert f(0, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 128, 16, 8, None) == OK        # no-op


def test_merge_validation():
    f = pa.library().pa_merge_attn_states
    assert f(FAKE, None, 0, FAKE, FAKE, FAKE, FAKE, 0, 4, 2, 12, None) == UNSUPPORTED
    assert f(FAKE, None, 5, FAKE, FAKE, FAKE, FAKE, 0, 4, 2, 128, None) == INVALID
    assert f(None, None, 0, FAKE, FAKE, FAKE, FAKE, 0, 4, 2, 128, None) == INVALID
    assert f(FAKE, None, 0, FAKE, FAKE, FAKE, FAKE, 0, 0, 2, 128, None) == OK     # no rows


def test_merge_rejects_overlapping_outputs():
    """out_lse may not overlap an input LSE (a row's LSE is read by threads of
    several workgroups); out may be an input itself, with the same dtype, but
    may not partly overlap one.  All of these fail before any launch."""
    f = pa.library().pa_merge_attn_states
    T, H, D = 4, 2, 192                  # 24 vectors of 8 per row: a row spans workgroups
    rows, F32 = T * H, 1
    vo = rows * D * 4                    # bytes of one f32 output
    po, so, out = FAKE, FAKE + vo, FAKE + 2 * vo
    pl, sl = FAKE + 3 * vo, FAKE + 3 * vo + 256
    assert f(out, pl, F32, po, pl, so, sl, F32, T, H, D, None) == INVALID        # out_lse = prefix
    assert f(out, sl, F32, po, pl, so, sl, F32, T, H, D, None) == INVALID        # out_lse = suffix
    assert f(out, sl + 16, F32, po, pl, so, sl, F32, T, H, D, None) == INVALID   # partly
    assert f(out, po + 64, F32, po, pl, so, sl, F32, T, H, D, None) == INVALID   # in an input
    assert f(out, out, F32, po, pl, so, sl, F32, T, H, D, None) == INVALID       # in out
    assert f(po + 32, None, F32, po, pl, so, sl, F32, T, H, D, None) == INVALID  # out partly on po
    assert f(po, None, 0, po, pl, so, sl, F32, T, H, D, None) == INVALID         # bf16 out on f32 po
    assert f(pl - 64, None, F32, po, pl, so, sl, F32, T, H, D, None) == INVALID  # out on the LSEs


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pa.paged_decode_attn(q, q, q, q, q, 0.1, 1)


@pytest.mark.parametrize("args", [
    (FAKE, 100, FAKE, 8),        # bytes not a multiple of 16
    (FAKE + 4, 64, FAKE, 8),     # source not 16-byte aligned
    (FAKE, 64, FAKE, 0),         # no workgroups
    (FAKE, 64, FAKE, 65537),     # too many workgroups
    (None, 64, FAKE, 8),
    (FAKE, 64, None, 8),
])
def test_stream_read_validation(args):
    assert pa.library().pa_stream_read(*args, 1, None) == INVALID


# (k, v, block_table, context_lens, S, Hkv, max_blocks, block_size, num_blocks, unit_bytes, sink)
_GR = (FAKE, FAKE, FAKE, FAKE, 4, 1, 8, 16, 64, 4096, FAKE)


@pytest.mark.parametrize("i,value", [
    (0, None), (1, None), (2, None), (3, None), (10, None),
    (0, FAKE + 8),      # cache not 16-byte aligned
    (4, -1),            # negative sequence count
    (5, 0),             # no kv heads
    (6, 0),             # no block-table columns
    (7, 0),             # block size 0
    (8, 0),             # no blocks
    (9, 512),           # unit below one 16-byte vector per lane
    (9, 3000),          # unit not whole 1 KiB
    (9, 1 << 17),       # unit above 64 KiB
])
def test_gather_read_validation(i, value):
    args = list(_GR)
    args[i] = value
    assert pa.library().pa_gather_read(*args, 1, None) == INVALID


def _decode_layout(lib, layout=0, nk=None, nv=None, sm=None, **kw):
    a = dict(out=FAKE, lse=None, query=FAKE, k=FAKE, v=FAKE, bt=FAKE, maxb=8, cl=FAKE, maxctx=100,
             S=4, Hq=8, Hkv=1, D=128, B=16, NB=64, scale=0.1, P=-1, ws=None, wsb=0)
    a.update(kw)
    return lib.pa_paged_decode_attn_layout(layout, a["out"], a["lse"], a["query"], nk, nv, sm,
                                           a["k"], a["v"], a["bt"], a["maxb"], a["cl"],
                                           a["maxctx"], a["S"], a["Hq"], a["Hkv"], a["D"], a["B"],
                                           a["NB"], a["scale"], a["P"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(layout=1), INVALID),                            # latent layout is not GQA
    (dict(layout=3), INVALID),
    (dict(nk=FAKE), INVALID),                             # write triple incomplete
    (dict(nk=FAKE, nv=FAKE), INVALID),
    (dict(nk=FAKE + 4, nv=FAKE, sm=FAKE), INVALID),       # misaligned new key
    (dict(layout=2, D=96), UNSUPPORTED),
    (dict(layout=2, B=8), UNSUPPORTED),
    (dict(layout=2, out=None), INVALID),
    (dict(layout=2, P=-2), WS_SMALL),
])
def test_decode_layout_validation(kw, status):
    assert _decode_layout(pa.library(), **kw) == status


def test_standard_cache_write_validation():
    lib = pa.library()
    # value missing, misaligned cache, head_dim not a multiple of 8
    assert lib.pa_reshape_and_cache(2, FAKE, None, FAKE, FAKE, FAKE, 4, 1, 128, 16, 8, None) == INVALID
    assert lib.pa_reshape_and_cache(2, FAKE, FAKE, FAKE + 8, FAKE + 8, FAKE, 4, 1, 128, 16, 8,
                                    None) == INVALID
    assert lib.pa_reshape_and_cache(2, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1, 100, 16, 8,
                                    None) == UNSUPPORTED
    assert lib.pa_reshape_and_cache(2, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 128, 16, 8, None) == OK


def _classify(n, c):
    return 0 if n <= 1 else (2 if c == 0 else 1)


@pytest.mark.parametrize("seed", range(5))
def test_mixed_batch_plan(seed):
    """The plan is the stable [decode : extend : prefill] order of a plain
    classification (one new token: decode; nothing cached: prefill)."""
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 40))
    n = rng.choice([1, 1, 1, 2, 5, 300], size=R)
    c = rng.choice([0, 0, 1, 17, 4000], size=R)
    qsl = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    order, counts = pa.mixed_batch_plan(qsl, c)
    kinds = [_classify(int(n[r]), int(c[r])) for r in range(R)]
    want = sorted(range(R), key=lambda r: (kinds[r], r))
    assert list(order) == want
    assert list(counts) == [kinds.count(0), kinds.count(1), kinds.count(2)]


def test_mixed_batch_plan_rejects():
    with pytest.raises(pa.PagedAttnError):
        pa.mixed_batch_plan([0, 1, 1], [3, 4])          # a request without new tokens
    with pytest.raises(pa.PagedAttnError):
        pa.mixed_batch_plan([1, 2], [3])                # offsets not starting at 0
    with pytest.raises(pa.PagedAttnError):
        pa.mixed_batch_plan([0, 1], [-1])               # negative context


def test_mixed_batch_attn_validation():
    """Unordered batches and short workspaces are refused before any launch."""
    lib = pa.library()
    i32 = lambda a: np.ascontiguousarray(np.asarray(a, dtype=np.int32))

    def call(qsl, ctx, ws=FAKE, wsb=1 << 30):
        qsl, ctx = i32(qsl), i32(ctx)
        R = ctx.shape[0]
        return lib.pa_mixed_batch_attn(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, qsl.ctypes.data,
                                       FAKE, ctx.ctypes.data, FAKE, FAKE, FAKE, 8, R, 8, 1, 128,
                                       16, 64, 0.1, 32768, ws, wsb, None)

    assert call([0, 5, 6], [10, 3]) == INVALID            # extend before decode
    assert call([0, 4, 5], [0, 3]) == INVALID             # prefill before decode
    assert call([0, 4, 10], [0, 3]) == INVALID            # prefill before extend
    assert call([0, 1, 5], [3, 3], ws=FAKE + 8) == INVALID  # misaligned workspace
    assert call([0, 1, 5], [3, 3], wsb=16) == WS_SMALL
    assert call([0, 1, 1], [3, 3]) == INVALID             # request without a token


def test_fp8_entry_validation():
    """FP8 entries refuse bad scales, shapes and partial write triples before any launch."""
    lib = pa.library()
    nan = float("nan")
    # cache write: bad scale, misaligned, unsupported head_dim / block size
    w = lambda **k: lib.pa_reshape_and_cache_fp8(
        k.get("key", FAKE), FAKE, k.get("kc", FAKE), FAKE, FAKE, 4, 1, k.get("D", 128),
        k.get("B", 16), 8, k.get("ks", 0.1), k.get("vs", 0.1), None)
    assert w(ks=0.0) == INVALID and w(vs=-1.0) == INVALID and w(ks=nan) == INVALID
    assert w(ks=1e-45) == INVALID                      # 1 / scale overflows
    assert w(kc=FAKE + 4) == INVALID
    assert w(D=96) == UNSUPPORTED and w(B=8) == UNSUPPORTED
    # decode: partial triple, bad scales, unsupported shapes
    d = lambda nk=None, nv=None, sm=None, ks=0.1, vs=0.1, D=128, B=16, P=-1: \
        lib.pa_paged_decode_attn_fp8(FAKE, None, FAKE, nk, nv, sm, FAKE, FAKE, FAKE, 8, FAKE, 100,
                                     4, 8, 1, D, B, 64, 0.1, ks, vs, P, None, 0, None)
    assert d(nk=FAKE) == INVALID and d(ks=0.0) == INVALID and d(vs=float("inf")) == INVALID
    assert d(D=96) == UNSUPPORTED and d(B=8) == UNSUPPORTED
    assert d(P=-2) == WS_SMALL
    # gather: block size must be a multiple of 16
    g = lambda B=16, ks=0.1: lib.pa_gather_cache_chunk_fp8(
        FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 4, 1, 128, B, 64, 0, 64, ks, 0.1, None)
    assert g(B=8) == UNSUPPORTED and g(ks=nan) == INVALID


def test_mla_fp8_entry_validation():
    """FP8 latent write and MLA FP8 decode refuse bad scales, half-given
    write pairs and unsupported widths before any launch."""
    lib = pa.library()
    w = lambda Dl=576, ks=0.01, lat=FAKE: lib.pa_reshape_and_cache_mla_fp8(
        lat, FAKE, FAKE, 4, Dl, 16, 8, ks, None)
    assert w(ks=0.0) == INVALID and w(ks=float("nan")) == INVALID and w(ks=1e-45) == INVALID
    assert w(lat=None) == INVALID and w(lat=FAKE + 8) == INVALID
    assert w(Dl=520) == UNSUPPORTED
    assert lib.pa_reshape_and_cache_mla_fp8(FAKE, FAKE, FAKE, 0, 576, 16, 8, 0.01, None) == OK
    d = lambda nl=None, sm=None, ks=0.01, Dv=512, P=-1: lib.pa_mla_decode_attn_fp8(
        FAKE, None, FAKE, nl, sm, FAKE, FAKE, 8, FAKE, 100, 4, 16, 576, Dv, 16, 64, 0.07, ks, P,
        None, 0, None)
    assert d(nl=FAKE) == INVALID and d(sm=FAKE) == INVALID
    assert d(ks=-1.0) == INVALID and d(ks=float("inf")) == INVALID
    assert d(Dv=448) == UNSUPPORTED
    assert d(P=-2) == WS_SMALL
    m = lambda nl=None, sm=None, ks=0.01, Dv=512, P=-1: lib.pa_mla_decode_attn_fp8_mfma(
        FAKE, None, FAKE, nl, sm, FAKE, FAKE, 8, FAKE, 100, 4, 16, 576, Dv, 16, 64, 0.07, ks, P,
        None, 0, None)
    assert m(nl=FAKE) == INVALID and m(sm=FAKE) == INVALID
    assert m(ks=0.0) == INVALID and m(ks=float("nan")) == INVALID
    assert m(Dv=448) == UNSUPPORTED
    assert m(P=-2) == WS_SMALL


def test_noalloc_decode_validation():
    """The no-allocation decode entry checks everything, the size of its
    array included, before it touches the device."""
    f = pa.library().pa_paged_decode_attn_write_noalloc
    args = lambda nk, S, Hq, maxctx, P: (FAKE, None, FAKE, nk, FAKE, FAKE, FAKE, FAKE, FAKE, 256,
                                         FAKE, maxctx, S, Hq, 2, 128, 16, 4096, 0.1, P, None)
    assert f(*args(None, 4, 8, 100, -1)) == INVALID               # no new key
    assert f(*args(FAKE + 8, 4, 8, 100, -1)) == INVALID           # new key misaligned
    assert f(*args(FAKE, 4, 7, 100, -1)) == INVALID               # 7 q heads on 2 kv heads
    assert f(*args(FAKE, 4, 8, 100, -3)) == INVALID
    # 64 x 16 heads x 64 partitions of fp32 partials: more than the array holds
    assert pa.decode_workspace_size(64, 16, 2, 128, 4096, 64) > pa.NOALLOC_SCRATCH_BYTES
    assert f(*args(FAKE, 64, 16, 4096, 64)) == WS_SMALL
    assert pa.NOALLOC_SCRATCH_BYTES == 32 << 20
