"""The Python binding checks every tensor's shape against the sizes it passes
to the C ABI, and raises ValueError before anything is launched.

Runs on the CPU: the device check is lifted and the library is replaced by a
recorder, so a correctly shaped call reaches exactly one recorded launch and
every mismatched call raises with none.
"""
import pytest
import torch

from paged_attention_decode_reshape_amd import ops

bf16, f32, i32, i64, u8 = torch.bfloat16, torch.float32, torch.int32, torch.int64, torch.uint8


class Recorder:
    """Stands in for the loaded library: size queries return 0, entry points
    record their name and return success."""

    def __init__(self):
        self.launches = []

    def __getattr__(self, name):
        def fn(*args):
            if not (name.endswith("_size") or name.endswith("_tokens")
                    or name.startswith("pa_decode_uses")):
                self.launches.append(name)
            return 0
        return fn


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()

    def gpu_no_device(name, t, dtype=None, ndim=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(name)
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} dtype")
        if ndim is not None and t.dim() != ndim:
            raise ValueError(f"{name} ndim")
        if not t.is_contiguous():
            raise ValueError(f"{name} contiguous")
        return t

    monkeypatch.setattr(ops, "library", lambda: r)
    monkeypatch.setattr(ops, "_gpu", gpu_no_device)
    monkeypatch.setattr(ops, "_stream", lambda t: 0)
    return r


S, Hq, Hkv, D, B, NB, MAXB = 3, 8, 2, 128, 16, 10, 4


def z(*shape, dtype=bf16):
    return torch.zeros(shape, dtype=dtype)


def decode_args(**over):
    a = dict(query=z(S, Hq, D), k_cache=z(NB, Hkv, D // 8, B, 8), v_cache=z(NB, Hkv, B // 8, D, 8),
             block_table=z(S, MAXB, dtype=i32), context_lens=z(S, dtype=i32), scale=0.1,
             max_context_len=64)
    a.update(over)
    return a


DECODE_BAD = {
    "k_cache head_dim": dict(k_cache=z(NB, Hkv, 64 // 8, B, 8)),
    "k_cache x": dict(k_cache=z(NB, Hkv, D // 16, B, 16)),
    "v_cache kv heads": dict(v_cache=z(NB, Hkv + 1, B // 8, D, 8)),
    "v_cache block size": dict(v_cache=z(NB, Hkv, 32 // 8, D, 8)),
    "v_cache head_dim": dict(v_cache=z(NB, Hkv, B // 8, 64, 8)),
    "block_table rows": dict(block_table=z(S - 1, MAXB, dtype=i32)),
    "context_lens length": dict(context_lens=z(S + 1, dtype=i32)),
    "out shape": dict(out=z(S, Hq, 64)),
    "lse shape": dict(lse=z(S, Hq + 1, dtype=f32)),
}


def test_decode_good_call_launches(rec):
    ops.paged_decode_attn(**decode_args())
    assert rec.launches == ["pa_paged_decode_attn"]


@pytest.mark.parametrize("what", list(DECODE_BAD))
def test_decode_mismatch_raises_before_launch(rec, what):
    with pytest.raises(ValueError):
        ops.paged_decode_attn(**decode_args(**DECODE_BAD[what]))
    assert rec.launches == []


def write_args(**over):
    a = decode_args()
    a.update(new_key=z(S, Hkv, D), new_value=z(S, Hkv, D), slot_mapping=z(S, dtype=i64))
    a.update(over)
    return a


WRITE_BAD = dict(DECODE_BAD)
WRITE_BAD.update({
    "new_key kv heads": dict(new_key=z(S, Hkv + 1, D)),
    "new_value rows": dict(new_value=z(S + 1, Hkv, D)),
    "slot_mapping length": dict(slot_mapping=z(S - 1, dtype=i64)),
})


@pytest.mark.parametrize("what", [None] + list(WRITE_BAD))
def test_decode_write_and_layout(rec, what):
    over = {} if what is None else WRITE_BAD[what]
    a = write_args(**over)
    w = dict(a)
    q = w.pop("query")
    nk, nv, sm = w.pop("new_key"), w.pop("new_value"), w.pop("slot_mapping")
    kc, vc = w.pop("k_cache"), w.pop("v_cache")
    calls = [
        lambda: ops.paged_decode_attn_write(q, nk, nv, sm, kc, vc, **w),
        lambda: ops.paged_decode_attn_layout(ops.LAYOUT_SHUFFLED_KV, q, kc, vc, new_key=nk,
                                             new_value=nv, slot_mapping=sm, **w),
    ]
    for call in calls:
        if what is None:
            call()
        else:
            with pytest.raises(ValueError):
                call()
    assert len(rec.launches) == (2 if what is None else 0)


def test_standard_layout_mismatch(rec):
    a = decode_args(k_cache=z(NB, B, Hkv, D), v_cache=z(NB, B, Hkv, D))
    ops.paged_decode_attn_layout(ops.LAYOUT_STANDARD_KV, **a)
    assert len(rec.launches) == 1
    for bad in (dict(v_cache=z(NB, B, Hkv, 64)), dict(block_table=z(1, MAXB, dtype=i32)),
                dict(out=z(S, Hq + 1, D))):
        b = dict(a)
        b.update(bad)
        with pytest.raises(ValueError):
            ops.paged_decode_attn_layout(ops.LAYOUT_STANDARD_KV, **b)
    assert len(rec.launches) == 1


def fp8_args(**over):
    a = decode_args(k_cache=z(NB, Hkv, D // 16, B, 16, dtype=u8),
                    v_cache=z(NB, Hkv, B // 16, D, 16, dtype=u8), k_scale=0.5, v_scale=0.5)
    a.update(over)
    return a


@pytest.mark.parametrize("bad", [
    None,
    dict(k_cache=z(NB, Hkv, D // 8, B, 8, dtype=u8)),        # bf16 geometry
    dict(v_cache=z(NB, Hkv, 2, D, 16, dtype=u8)),             # block size 32
    dict(context_lens=z(S - 1, dtype=i32)),
    dict(lse=z(S, Hq, 1, dtype=f32)),
    dict(new_key=z(S, Hkv, 64), new_value=z(S, Hkv, D), slot_mapping=z(S, dtype=i64)),
], ids=["good", "k_x8", "v_block", "lens", "lse_ndim", "new_key"])
def test_fp8_decode(rec, bad):
    if bad is None:
        ops.paged_decode_attn_fp8(**fp8_args())
        assert rec.launches == ["pa_paged_decode_attn_fp8"]
    else:
        with pytest.raises(ValueError):
            ops.paged_decode_attn_fp8(**fp8_args(**bad))
        assert rec.launches == []


def mla_args(**over):
    a = dict(query=z(S, 16, 576), kv_cache=z(NB, 64, 576), block_table=z(S, MAXB, dtype=i32),
             context_lens=z(S, dtype=i32), scale=0.1, max_context_len=100)
    a.update(over)
    return a


MLA_BAD = {
    "latent width": dict(kv_cache=z(NB, 64, 512)),
    "block_table rows": dict(block_table=z(S - 1, MAXB, dtype=i32)),
    "context_lens": dict(context_lens=z(S + 2, dtype=i32)),
    "out v_dim": dict(out=z(S, 16, 576)),
    "lse heads": dict(lse=z(S, 8, dtype=f32)),
}


@pytest.mark.parametrize("fn", ["mla_decode_attn", "mla_decode_attn_mfma"])
@pytest.mark.parametrize("what", [None] + list(MLA_BAD))
def test_mla(rec, fn, what):
    a = mla_args(**({} if what is None else MLA_BAD[what]))
    if what is None:
        getattr(ops, fn)(**a)
        assert rec.launches == ["pa_" + fn]
    else:
        with pytest.raises(ValueError):
            getattr(ops, fn)(**a)
        assert rec.launches == []


@pytest.mark.parametrize("bad", [None, dict(new_latent=z(S, 512)),
                                 dict(slot_mapping=z(S + 1, dtype=i64)),
                                 dict(block_table=z(1, MAXB, dtype=i32))],
                         ids=["good", "latent", "slots", "table"])
def test_mla_write(rec, bad):
    a = mla_args(new_latent=z(S, 576), slot_mapping=z(S, dtype=i64))
    if bad:
        a.update(bad)
        with pytest.raises(ValueError):
            ops.mla_decode_attn_write(**a)
        assert rec.launches == []
    else:
        ops.mla_decode_attn_write(**a)
        assert rec.launches == ["pa_mla_decode_attn_write"]


@pytest.mark.parametrize("fn", ["mla_decode_attn_fp8", "mla_decode_attn_fp8_mfma"])
def test_mla_fp8(rec, fn):
    a = mla_args(kv_cache=z(NB, 64, 576, dtype=u8), kv_scale=0.5)
    getattr(ops, fn)(**a)
    assert rec.launches == ["pa_" + fn]
    a["block_table"] = z(S - 1, MAXB, dtype=i32)
    with pytest.raises(ValueError):
        getattr(ops, fn)(**a)
    assert len(rec.launches) == 1


def extend_args(**over):
    Tn = 10
    a = dict(query=z(Tn, Hq, D), k_new=z(Tn, Hkv, D), v_new=z(Tn, Hkv, D),
             query_start_loc=z(S + 1, dtype=i32), k_cache=z(NB, Hkv, D // 8, B, 8),
             v_cache=z(NB, Hkv, B // 8, D, 8), block_table=z(S, MAXB, dtype=i32),
             context_lens=z(S, dtype=i32), scale=0.1, query_start_loc_host=[0, 3, 3, 10],
             context_lens_host=[5, 0, 17])
    a.update(over)
    return a


EXTEND_BAD = {
    "k_new rows": dict(k_new=z(9, Hkv, D)),
    "v_new heads": dict(v_new=z(10, Hkv + 1, D)),
    "v_cache": dict(v_cache=z(NB, Hkv, B // 8, 64, 8)),
    "qsl device length": dict(query_start_loc=z(S, dtype=i32)),
    "qsl host end": dict(query_start_loc_host=[0, 3, 3, 11]),
    "block_table rows": dict(block_table=z(S - 1, MAXB, dtype=i32)),
    "out rows": dict(out=z(11, Hq, D)),
    "lse": dict(lse=z(10, Hq - 1, dtype=f32)),
}


@pytest.mark.parametrize("what", [None] + list(EXTEND_BAD))
def test_extend(rec, what):
    a = extend_args(**({} if what is None else EXTEND_BAD[what]))
    if what is None:
        ops.chunked_extend_attn(**a)
        assert rec.launches == ["pa_chunked_extend_attn"]
    else:
        with pytest.raises(ValueError):
            ops.chunked_extend_attn(**a)
        assert rec.launches == []


@pytest.mark.parametrize("fp8", [False, True])
def test_gather(rec, fp8):
    if fp8:
        kc, vc = z(NB, Hkv, D // 16, B, 16, dtype=u8), z(NB, Hkv, B // 16, D, 16, dtype=u8)
        fn = lambda **k: ops.gather_cache_chunk_fp8(k_scale=1.0, v_scale=1.0, **k)
        bad_v = z(NB, Hkv, B // 16, 64, 16, dtype=u8)
    else:
        kc, vc = z(NB, Hkv, D // 8, B, 8), z(NB, Hkv, B // 8, D, 8)
        fn = ops.gather_cache_chunk
        bad_v = z(NB, Hkv, B // 8, 64, 8)
    base = dict(k_cache=kc, v_cache=vc, block_table=z(S, MAXB, dtype=i32),
                context_lens=z(S, dtype=i32), iteration=0, chunk_tokens=16)
    fn(**base)
    assert len(rec.launches) == 1
    for bad in (dict(v_cache=bad_v), dict(block_table=z(S - 1, MAXB, dtype=i32)),
                dict(k_out=z(S * 16, Hkv, 64)), dict(v_out=z(S * 16, Hkv + 1, D))):
        b = dict(base)
        b.update(bad)
        with pytest.raises(ValueError):
            fn(**b)
    assert len(rec.launches) == 1


def mixed_args(**over):
    T = 6
    a = dict(query=z(T, Hq, D), key=z(T, Hkv, D), value=z(T, Hkv, D), slot_mapping=z(T, dtype=i64),
             query_start_loc=z(S + 1, dtype=i32), context_lens=z(S, dtype=i32),
             k_cache=z(NB, Hkv, D // 8, B, 8), v_cache=z(NB, Hkv, B // 8, D, 8),
             block_table=z(S, MAXB, dtype=i32), scale=0.1, query_start_loc_host=[0, 1, 2, 6],
             context_lens_host=[4, 9, 0])
    a.update(over)
    return a


MIXED_BAD = {
    "key rows": dict(key=z(5, Hkv, D)),
    "value head_dim": dict(value=z(6, Hkv, 64)),
    "slots": dict(slot_mapping=z(5, dtype=i64)),
    "qsl device": dict(query_start_loc=z(S + 2, dtype=i32)),
    "context_lens": dict(context_lens=z(S - 1, dtype=i32)),
    "k_cache": dict(k_cache=z(NB, Hkv + 1, D // 8, B, 8)),
    "out": dict(out=z(6, Hq, 64)),
}


@pytest.mark.parametrize("what", [None] + list(MIXED_BAD))
def test_mixed(rec, what):
    a = mixed_args(**({} if what is None else MIXED_BAD[what]))
    if what is None:
        ops.mixed_batch_attn(**a)
        assert rec.launches == ["pa_mixed_batch_attn"]
    else:
        with pytest.raises(ValueError):
            ops.mixed_batch_attn(**a)
        assert rec.launches == []


def test_merge_shapes_and_aliasing(rec):
    T, H, Dm = 4, 2, 192
    po, so = z(T, H, Dm, dtype=f32), z(T, H, Dm, dtype=f32)
    pl, sl = z(T, H, dtype=f32), z(T, H, dtype=f32)
    ops.merge_attn_states(po, pl, so, sl)
    ops.merge_attn_states(po, pl, so, sl, out=po)   # in place: out is prefix_out itself
    assert len(rec.launches) == 2
    big = z(2 * T * H, dtype=f32)
    bad = [
        dict(out=z(T, H, 128, dtype=f32)),
        dict(out_lse=z(T, H + 1, dtype=f32)),
        dict(out_lse=pl),                             # the natural in-place LSE accumulation
        dict(out_lse=sl),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            ops.merge_attn_states(po, pl, so, sl, **kw)
    # partial overlap of out_lse with suffix_lse
    pl2, sl2 = big[:T * H].view(T, H), big[T * H // 2:T * H // 2 + T * H].view(T, H)
    with pytest.raises(ValueError):
        ops.merge_attn_states(po, z(T, H, dtype=f32), so, sl2, out_lse=pl2)
    # bf16 out over the f32 prefix's first half: same address, another dtype
    over = po.view(-1).view(bf16)[:T * H * Dm].view(T, H, Dm)
    assert over.is_contiguous() and over.data_ptr() == po.data_ptr()
    with pytest.raises(ValueError, match="overlap"):
        ops.merge_attn_states(po, pl, so, sl, out=over, out_dtype=bf16)
    assert len(rec.launches) == 2


def test_prepare_records_one_call_and_checks_first(monkeypatch):
    """prepare() runs the wrapper's checks and marshalling against the real
    library without enqueuing: exactly one entry is recorded, host-only
    queries run, a shape mismatch raises at prepare time."""
    monkeypatch.setattr(ops, "_gpu", lambda name, t, dtype=None, ndim=None: t)
    monkeypatch.setattr(ops, "_stream", lambda t: 0)
    a = decode_args(partition_tokens=64, max_context_len=200)
    call = ops.prepare(ops.paged_decode_attn, **a)
    assert isinstance(call, ops.PreparedCall) and call.name == "pa_paged_decode_attn"
    out, lse = call.result
    assert tuple(out.shape) == (S, Hq, D) and tuple(lse.shape) == (S, Hq)
    # the split call's workspace (counter region + partials) is held by the call
    nbytes = ops.decode_workspace_size(S, Hq, Hkv, D, 200, 64)
    assert nbytes > ops.WORKSPACE_COUNTER_BYTES
    assert any(isinstance(k, torch.Tensor) and k.numel() == nbytes for k in call._keep)
    with pytest.raises(ValueError):
        ops.prepare(ops.paged_decode_attn, **decode_args(block_table=z(1, MAXB, dtype=i32)))
    with pytest.raises(ValueError, match="exactly one"):
        ops.prepare(lambda: None)
    assert getattr(ops._tls, "capture", None) is None
