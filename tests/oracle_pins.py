"""Pins of the oracle to things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` handle and raises
AssertionError if the oracle disagrees with what the pages' definitions
and the mathematics fix:

  * the cache layout shapes of the "ROCm attention backends" blog
    (ROCM_AITER_FA section, item 4), rebuilt with numpy reshape/transpose;
  * NumPy brute-force dense attention on the logical token order (no block
    table, no shuffled layout);
  * closed forms (one token, zero query, identical keys);
  * invariants: split + log-sum-exp merge equals the unsplit result
    (extend-path pseudocode: each chunk yields an output and an LSE, merged
    stably), block-table permutation, GQA == MHA with repeated K/V, MLA
    block-size independence, chunk-budget independence of extend.

The functions are parameterised by the oracle build so that the mutation
tests can run them against deliberately broken copies of ``oracle.c``.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import np_ref
from paged_attention_decode_reshape_amd import workloads as W

TIGHT = 1e-12  # fp64 vs fp64, different summation orders


def _close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    diff = np.where(both_inf, 0.0, np.abs(a - b))
    bad = ~(diff <= tol * np.maximum(1.0, np.abs(b)))
    assert not bad.any(), f"{what}: max diff {np.nanmax(np.where(both_inf, 0, np.abs(a - b)))}"


def oracle_cache(orc, case):
    kc, vc = orc.empty_shuffled_cache(case.paging.num_blocks, case.Hkv, case.D, case.B)
    orc.cache_write_shuffled(W.bf16_bits(case.key), W.bf16_bits(case.value),
                             case.paging.slot_mapping, kc, vc, case.B)
    return kc, vc


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# layout: cache write, gather
# ---------------------------------------------------------------------------

def _distinct_tokens(T, H, D, seed):
    """bf16 bit patterns, all distinct and all finite: every (token, head, dim)
    is identifiable after the scatter."""
    rng = np.random.default_rng(seed)
    n = T * H * D
    # positive normal bf16 values: exponent field 1..254, any mantissa
    pool = np.arange(0x0080, 0x7F80, dtype=np.uint16)
    assert n <= pool.size
    return rng.choice(pool, size=n, replace=False).reshape(T, H, D)


def pin_shuffle_layout(orc):
    """The scatter puts (token, head, dim) where the pages' shapes say."""
    for (Hkv, D, B, nb, T) in [(2, 64, 16, 7, 70), (1, 128, 32, 5, 100), (3, 128, 16, 4, 40)]:
        x = 8
        rng = np.random.default_rng(Hkv * 1000 + D + B)
        slots = rng.choice(nb * B, size=T, replace=False).astype(np.int64)
        key = _distinct_tokens(T, Hkv, D, 1)
        val = _distinct_tokens(T, Hkv, D, 2)
        kc, vc = orc.empty_shuffled_cache(nb, Hkv, D, B, x, fill=0x7FC0)
        orc.cache_write_shuffled(key, val, slots, kc, vc, B, x)
        # standard pool [nb, B, Hkv, D] then the shapes of the pages
        kstd = np.full((nb * B, Hkv, D), 0x7FC0, dtype=np.uint16)
        vstd = np.full((nb * B, Hkv, D), 0x7FC0, dtype=np.uint16)
        kstd[slots] = key
        vstd[slots] = val
        kstd = kstd.reshape(nb, B, Hkv, D)
        vstd = vstd.reshape(nb, B, Hkv, D)
        # k_cache [nb, Hkv, D//x, B, x]: dim split into (D//x, x), token between
        k_exp = kstd.reshape(nb, B, Hkv, D // x, x).transpose(0, 2, 3, 1, 4)
        # v_cache [nb, Hkv, B//x, D, x]: token split into (B//x, x), dim between
        v_exp = vstd.reshape(nb, B // x, x, Hkv, D).transpose(0, 3, 1, 4, 2)
        assert np.array_equal(kc, k_exp), "k_cache placement"
        assert np.array_equal(vc, v_exp), "v_cache placement"


def pin_shuffle_golden(orc, golden):
    """Offsets hand-derived from the shapes (tests/golden/shuffle_offsets.json)."""
    g = golden
    Hkv, D, B, x, nb = g["Hkv"], g["D"], g["B"], g["x"], g["num_blocks"]
    for e in g["entries"]:
        key = np.zeros((1, Hkv, D), dtype=np.uint16)
        val = np.zeros((1, Hkv, D), dtype=np.uint16)
        key[0, e["head"], e["dim"]] = 0x3F80  # 1.0
        val[0, e["head"], e["dim"]] = 0x4000  # 2.0
        kc, vc = orc.empty_shuffled_cache(nb, Hkv, D, B, x, fill=0)
        orc.cache_write_shuffled(key, val, np.array([e["slot"]], dtype=np.int64), kc, vc, B, x)
        assert kc.reshape(-1)[e["k_flat"]] == 0x3F80, ("k", e)
        assert vc.reshape(-1)[e["v_flat"]] == 0x4000, ("v", e)


def pin_cache_write_skips(orc):
    """Negative and out-of-pool slots leave the cache untouched."""
    Hkv, D, B, nb = 2, 64, 16, 3
    key = _distinct_tokens(4, Hkv, D, 3)
    val = _distinct_tokens(4, Hkv, D, 4)
    kc, vc = orc.empty_shuffled_cache(nb, Hkv, D, B)
    k0, v0 = kc.copy(), vc.copy()
    orc.cache_write_shuffled(key, val, np.array([-1, nb * B, nb * B + 5, -100], np.int64),
                             kc, vc, B)
    assert np.array_equal(kc, k0) and np.array_equal(vc, v0)


def pin_gather_roundtrip(orc):
    """Scatter then gather of every token gives back the logical rows, bit for bit."""
    case = W.tiny_gqa()
    kc, vc = oracle_cache(orc, case)
    lens = case.context_lens
    ko, vo, cu = orc.gather_shuffled(kc, vc, case.paging.block_table, np.zeros_like(lens), lens,
                                     case.B)
    assert np.array_equal(ko, W.bf16_bits(case.key))
    assert np.array_equal(vo, W.bf16_bits(case.value))
    # a middle range of each sequence
    tb = (lens // 3).astype(np.int32)
    te = (lens - lens // 5).astype(np.int32)
    ko, vo, cu = orc.gather_shuffled(kc, vc, case.paging.block_table, tb, te, case.B)
    kk = W.bf16_bits(case.key)
    for s in range(case.S):
        st = int(case.paging.seq_start[s])
        assert np.array_equal(ko[cu[s]:cu[s + 1]], kk[st + tb[s]:st + te[s]])


def pin_standard_layout(orc):
    """The standard-layout write puts (token, head, dim) at [slot // B][slot % B]
    [head][dim], element by element, leaves every other element alone and
    skips the slots the shuffled write skips; shuffling the standard cache
    gives exactly what the shuffled write produces from the same tokens."""
    for (Hkv, D, B, nb, T) in [(2, 64, 16, 7, 70), (1, 128, 32, 5, 100), (3, 128, 16, 4, 40)]:
        rng = np.random.default_rng(Hkv * 77 + D + B)
        slots = rng.choice(nb * B, size=T, replace=False).astype(np.int64)
        slots[::9] = -1
        slots[5] = nb * B + 3
        key = _distinct_tokens(T, Hkv, D, 5)
        val = _distinct_tokens(T, Hkv, D, 6)
        ks, vs = orc.empty_standard_cache(nb, B, Hkv, D, fill=0x7FC0)
        orc.cache_write_standard(key, val, slots, ks, vs)
        written = np.zeros((nb, B), dtype=bool)
        for i in range(T):
            sl = int(slots[i])
            if sl < 0 or sl >= nb * B:
                continue
            written[sl // B, sl % B] = True
            for g in range(Hkv):
                for d in range(0, D, 7):
                    assert ks[sl // B, sl % B, g, d] == key[i, g, d]
                    assert vs[sl // B, sl % B, g, d] == val[i, g, d]
        assert np.all(ks[~written] == 0x7FC0) and np.all(vs[~written] == 0x7FC0)
        assert written.sum() == np.sum((slots >= 0) & (slots < nb * B))
        kc, vc = orc.empty_shuffled_cache(nb, Hkv, D, B, fill=0x7FC0)
        orc.cache_write_shuffled(key, val, slots, kc, vc, B)
        k2, v2 = orc.standard_to_shuffled(ks, vs)
        assert np.array_equal(k2, kc) and np.array_equal(v2, vc)


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV cache
# ---------------------------------------------------------------------------

def pin_fp8_codes(orc):
    """E4M3 values from its definition: hand-listed codes, symmetry,
    monotonicity; encode inverts decode on every finite code, sends every
    midpoint between neighbours to the even code and anything just off a
    midpoint to the nearer one, and saturates at 448."""
    from oracle import fp8
    t = fp8.decode_table()
    hand = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2 ** -6,
            0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x48: 4.0, 0x77: 240.0,
            0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in hand.items():
        assert t[c] == v, (hex(c), t[c], v)
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.signbit(t[0x80]) and t[0x80] == 0
    assert np.all(np.diff(t[:0x7F]) > 0)
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F])
    finite = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    assert np.array_equal(fp8.encode(t[finite].astype(np.float32)), finite)
    for c in range(0, 0x7E):
        lo, hi = np.float32(t[c]), np.float32(t[c + 1])
        mid = np.float32((t[c] + t[c + 1]) / 2)  # exact in float32
        even = c if c % 2 == 0 else c + 1
        assert fp8.encode(mid) == even, hex(c)
        assert fp8.encode(np.nextafter(mid, hi)) == c + 1
        assert fp8.encode(np.nextafter(mid, lo)) == c
        assert fp8.encode(-mid) == (even | 0x80)
    for big in (448.0, 449.0, 464.0, 480.0, 1e30):
        assert fp8.encode(np.float32(big)) == 0x7E and fp8.encode(np.float32(-big)) == 0xFE


def pin_fp8_quantize_and_bf16(orc):
    """Quantisation error within half a code step times the scale (inside the
    range), exact for values on the grid; bf16 rounding of known values."""
    from oracle import fp8
    rng = np.random.default_rng(81)
    x = rng.standard_normal(20000).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncated to bf16
    xb = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for scale in (2.0 ** -5, 0.0137, 0.5):
        codes = fp8.quantize_bf16(bits, scale)
        got = fp8.dequant_f64(codes, scale)
        y = np.abs(xb) / scale
        # code spacing at |y|: 2^(floor(log2 y) - 3) above 2^-6, 2^-9 below
        e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
        step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))
        inside = y < 440
        assert np.all(np.abs(got - xb)[inside] <= 0.5 * step[inside] * scale * (1 + 1e-6) + 1e-12)
        assert np.all(np.abs(got[~inside]) == 448 * float(np.float32(scale)))
    grid = fp8.decode_table()[[0x01, 0x08, 0x38, 0x3F, 0x77]] * 2.0 ** -5
    gb = fp8.bf16_rne(grid.astype(np.float32))
    assert np.array_equal(fp8.quantize_bf16(gb, 2.0 ** -5), np.array([0x01, 0x08, 0x38, 0x3F, 0x77]))
    vals = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -9, 1 + 2.0 ** -7 + 2.0 ** -8, -2.5],
                    dtype=np.float32)
    assert list(fp8.bf16_rne(vals)) == [0x3F80, 0x3F80, 0x3F81, 0x3F82, 0xC020]


def pin_fp8_cache_layout(orc):
    """FP8 codes land at [p][g][d div 16][o][d mod 16] and [p][g][o div 16][d][o mod 16],
    nothing else changes, bad slots are skipped."""
    from oracle import fp8
    for (Hkv, D, B, nb, T) in [(2, 64, 16, 5, 40), (1, 128, 32, 3, 60)]:
        rng = np.random.default_rng(D + B)
        slots = rng.choice(nb * B, size=T, replace=False).astype(np.int64)
        slots[::6] = -1
        key = rng.standard_normal((T, Hkv, D)).astype(np.float32)
        val = rng.standard_normal((T, Hkv, D)).astype(np.float32)
        kb = (key.view(np.uint32) >> 16).astype(np.uint16)
        vb = (val.view(np.uint32) >> 16).astype(np.uint16)
        kc, vc = fp8.empty_cache(nb, Hkv, D, B)
        fp8.cache_write(kb, vb, slots, kc, vc, 0.05, 0.07)
        kq, vq = fp8.quantize_bf16(kb, 0.05), fp8.quantize_bf16(vb, 0.07)
        seen_k = np.zeros(kc.shape, dtype=bool)
        seen_v = np.zeros(vc.shape, dtype=bool)
        for i in range(T):
            if slots[i] < 0:
                continue
            p, o = int(slots[i]) // B, int(slots[i]) % B
            for g in range(Hkv):
                for d in range(D):
                    assert kc[p, g, d // 16, o, d % 16] == kq[i, g, d]
                    assert vc[p, g, o // 16, d, o % 16] == vq[i, g, d]
                    seen_k[p, g, d // 16, o, d % 16] = True
                    seen_v[p, g, o // 16, d, o % 16] = True
        assert np.all(kc[~seen_k] == 0x7F) and np.all(vc[~seen_v] == 0x7F)


def pin_fp8_decode_matches_bf16(orc):
    """With power-of-two scales every dequantised value is a bf16, so FP8
    decode equals the C oracle's bf16 decode over caches holding those values."""
    from oracle import fp8
    case = W.gqa_decode_case("fp8pin", 82, [1, 17, 100, 300], Hq=8, Hkv=2, D=64, block_size=16)
    pg = case.paging
    ks, vs = 2.0 ** -5, 2.0 ** -4
    kc8, vc8 = fp8.empty_cache(pg.num_blocks, case.Hkv, case.D, case.B)
    fp8.cache_write(W.bf16_bits(case.key), W.bf16_bits(case.value), pg.slot_mapping, kc8, vc8,
                    ks, vs)
    out8, lse8 = fp8.paged_decode_gqa(W.bf16_bits(case.query), kc8, vc8, pg.block_table,
                                      case.context_lens, case.scale, ks, vs)
    kdq = fp8.bf16_rne(fp8.dequant_f64(fp8.quantize_bf16(W.bf16_bits(case.key), ks), ks)
                       .astype(np.float32))
    vdq = fp8.bf16_rne(fp8.dequant_f64(fp8.quantize_bf16(W.bf16_bits(case.value), vs), vs)
                       .astype(np.float32))
    assert np.array_equal(fp8.dequant_f64(fp8.quantize_bf16(W.bf16_bits(case.key), ks), ks),
                          (kdq.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    kc, vc = orc.empty_shuffled_cache(pg.num_blocks, case.Hkv, case.D, case.B)
    orc.cache_write_shuffled(kdq, vdq, pg.slot_mapping, kc, vc, case.B)
    out, lse = orc.paged_decode_gqa(W.bf16_bits(case.query), kc, vc, pg.block_table,
                                    case.context_lens, case.B, case.scale)
    _close(out8, out, what="fp8 out")
    _close(lse8, lse, what="fp8 lse")


def pin_fp8_mla_matches_bf16(orc):
    """FP8 latent cache: codes land at [slot // B][slot % B] (bad slots skipped),
    and with a power-of-two scale the FP8 MLA decode equals the C oracle's
    bf16 MLA decode over the dequantised latents."""
    from oracle import fp8
    case = W.mla_decode_cases("fp8mla", 83, S=3, lens_range=None, lens=[1, 70, 300], Hq=4,
                              Dl=576, Dv=512, block_sizes=(16,), scale=1 / 192 ** 0.5)[16]
    pg = case.paging
    s8 = 2.0 ** -5
    kv8 = np.full((pg.num_blocks, case.B, 576), 0x7F, dtype=np.uint8)
    slots = pg.slot_mapping.copy()
    lat = W.bf16_bits(case.latent)
    fp8.cache_write_latent(lat, slots, kv8, s8)
    codes = fp8.quantize_bf16(lat, s8)
    for i in range(0, len(slots), 7):
        assert np.array_equal(kv8[slots[i] // case.B, slots[i] % case.B], codes[i])
    k0 = kv8.copy()
    fp8.cache_write_latent(lat[:2], np.array([-1, pg.num_blocks * case.B]), kv8, s8)
    assert np.array_equal(kv8, k0)
    out8, lse8 = fp8.paged_decode_mla(W.bf16_bits(case.query), kv8, pg.block_table,
                                      case.context_lens, 512, case.scale, s8)
    deq = fp8.bf16_rne(fp8.dequant_f64(codes, s8).astype(np.float32))
    kv = np.full((pg.num_blocks, case.B, 576), 0x7FC0, dtype=np.uint16)
    orc.cache_write_latent(deq, slots, kv, case.B)
    out, lse = orc.paged_decode_mla(W.bf16_bits(case.query), kv, pg.block_table,
                                    case.context_lens, case.B, 512, case.scale)
    _close(out8, out, what="fp8 mla out")
    _close(lse8, lse, what="fp8 mla lse")


def _e4m3_value(code: int) -> float:
    """E4M3 value from its bit fields (sign, 4 exponent bits, bias 7, 3
    mantissa bits; exponent field 0 is subnormal), written out separately
    from the oracle's table."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0:
        return sign * math.ldexp(m / 8.0, -6)
    return sign * math.ldexp(1.0 + m / 8.0, e - 7)


def _bf16_bits_torch(f32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns by torch's own round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def pin_fp8_gather_dequant(orc):
    """The chunk gather with dequantisation (the MLA extend path's gather
    "and maybe dequant", "ROCm attention backends" blog, AITER MLA extend
    pseudocode): iteration `it` of chunk length c yields, request after
    request, tokens [it c, min((it + 1) c, n)) as bf16(float32(value(code))
    * float32(scale)), K under k_scale and V under v_scale.  Expected rows
    come from the logical token codes (scattered by hand into the pages'
    shapes), a bit-field decode and torch's bf16 rounding."""
    from oracle import fp8
    X = 16
    rng = np.random.default_rng(77)
    Hkv, D, B = 2, 32, 16
    lens = [0, 5, 37, 70, 16]  # an empty request, a partial block, whole blocks
    k_scale = np.float32(0.0371)   # distinct, not powers of two
    v_scale = np.float32(1.7)
    nblk = [(n + B - 1) // B for n in lens]
    nb = sum(nblk) + 3
    perm = rng.permutation(nb)
    maxb = max(nblk)
    table = np.zeros((len(lens), maxb), dtype=np.int32)
    k_cache = np.full((nb, Hkv, D // X, B, X), 0x7F, dtype=np.uint8)
    v_cache = np.full((nb, Hkv, B // X, D, X), 0x7F, dtype=np.uint8)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    kcodes, vcodes = [], []  # logical [n, Hkv, D] codes per request
    nxt = 0
    for s, n in enumerate(lens):
        for j in range(nblk[s]):
            table[s, j] = perm[nxt]
            nxt += 1
        kq = rng.choice(finite, size=(n, Hkv, D))
        vq = rng.choice(finite, size=(n, Hkv, D))
        for t in range(n):
            p, o = int(table[s, t // B]), t % B
            for g in range(Hkv):
                for d in range(D):
                    k_cache[p, g, d // X, o, d % X] = kq[t, g, d]
                    v_cache[p, g, o // X, d, o % X] = vq[t, g, d]
        kcodes.append(kq)
        vcodes.append(vq)
    # the constructed double-rounding case: code 0x3A is 1.25 and
    # 1.25 * v_scale2 = 1 + 2^-8 + 2^-25 exactly; float32 rounds that to the
    # tie 1 + 2^-8, which goes to the even bf16 0x3F80, while rounding the
    # exact product straight to bf16 would give 0x3F81
    v_scale2 = np.float32(13474202 * 2.0 ** -24)
    assert 1.25 * float(v_scale2) == 1 + 2 ** -8 + 2 ** -25
    vcodes[3][0, 0, 0] = 0x3A
    p0 = int(table[3, 0])
    v_cache[p0, 0, 0, 0, 0] = 0x3A
    dec = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
    for chunk in (16, 32):
        for vs in (v_scale, v_scale2):
            for it in range(-(-max(lens) // chunk) + 1):  # one iteration past every end
                ek, ev = [], []
                for s, n in enumerate(lens):
                    t0, t1 = it * chunk, min((it + 1) * chunk, n)
                    if t1 > t0:
                        ek.append(_bf16_bits_torch(
                            dec[kcodes[s][t0:t1]].astype(np.float32) * k_scale))
                        ev.append(_bf16_bits_torch(
                            dec[vcodes[s][t0:t1]].astype(np.float32) * vs))
                gk, gv = fp8.gather_dequant(k_cache, v_cache, table, np.array(lens), it, chunk,
                                            float(k_scale), float(vs))
                if not ek:
                    assert gk.size == 0 and gv.size == 0, (chunk, it)
                    continue
                assert np.array_equal(gk, np.concatenate(ek)), ("fp8 gather K", chunk, it)
                assert np.array_equal(gv, np.concatenate(ev)), ("fp8 gather V", chunk, it)
    gk, gv = fp8.gather_dequant(k_cache, v_cache, table, np.array(lens), 0, 16,
                                float(k_scale), float(v_scale2))
    row = sum(min(16, n) for n in lens[:3])  # request 3's first token
    assert gv[row, 0, 0] == 0x3F80, hex(gv[row, 0, 0])


def pin_latent_write(orc):
    B, nb, Dl, T = 4, 9, 576, 20
    rng = np.random.default_rng(5)
    slots = rng.choice(nb * B, size=T, replace=False).astype(np.int64)
    lat = rng.integers(0x0080, 0x7F80, size=(T, Dl), dtype=np.uint16)
    kv = np.full((nb, B, Dl), 0x7FC0, dtype=np.uint16)
    orc.cache_write_latent(lat, slots, kv, B)
    exp = np.full((nb * B, Dl), 0x7FC0, dtype=np.uint16)
    exp[slots] = lat
    assert np.array_equal(kv.reshape(nb * B, Dl), exp)


# ---------------------------------------------------------------------------
# GQA decode
# ---------------------------------------------------------------------------

def _np_decode(case):
    return np_ref.gqa_decode(_f64(case.query), _f64(case.key), _f64(case.value),
                             case.paging.seq_start, case.context_lens, case.scale)


def _small_cases():
    yield W.tiny_gqa()
    yield W.gqa_decode_case("d64_b32_gqa2", 11, [1, 31, 32, 33, 200], Hq=4, Hkv=2, D=64,
                            block_size=32)
    yield W.gqa_decode_case("mha", 12, [15, 16, 17], Hq=3, Hkv=3, D=128, block_size=16)
    yield W.gqa_decode_case("gqa16", 13, [5, 140], Hq=32, Hkv=2, D=128, block_size=16)


def pin_decode_vs_numpy(orc):
    for case in _small_cases():
        kc, vc = oracle_cache(orc, case)
        out, lse = orc.paged_decode_gqa(W.bf16_bits(case.query), kc, vc, case.paging.block_table,
                                        case.context_lens, case.B, case.scale)
        rout, rlse = _np_decode(case)
        _close(out, rout, 1e-12, f"{case.name} out")
        _close(lse, rlse, 1e-12, f"{case.name} lse")


def pin_decode_closed_forms(orc):
    D, B, Hkv, Hq = 64, 16, 1, 2
    gen = torch.Generator().manual_seed(7)
    # one token: out = V_0 exactly, lse = z_0
    case = W.gqa_decode_case("one", 21, [1, 1], Hq=Hq, Hkv=Hkv, D=D, block_size=B)
    kc, vc = oracle_cache(orc, case)
    out, lse = orc.paged_decode_gqa(W.bf16_bits(case.query), kc, vc, case.paging.block_table,
                                    case.context_lens, B, case.scale)
    q, k, v = _f64(case.query), _f64(case.key), _f64(case.value)
    for s in range(2):
        for h in range(Hq):
            assert np.array_equal(out[s, h], v[s, 0]), "n=1 output"
            z0 = case.scale * float(np.dot(q[s, h], k[s, 0]))
            assert abs(lse[s, h] - z0) <= 1e-12 * max(1, abs(z0)), "n=1 lse"
    # zero query: uniform weights, out = mean V, lse = ln n
    case = W.gqa_decode_case("zq", 22, [7, 50], Hq=Hq, Hkv=Hkv, D=D, block_size=B)
    case.query.zero_()
    kc, vc = oracle_cache(orc, case)
    out, lse = orc.paged_decode_gqa(W.bf16_bits(case.query), kc, vc, case.paging.block_table,
                                    case.context_lens, B, case.scale)
    v = _f64(case.value)
    for s, n in enumerate(case.context_lens):
        st = int(case.paging.seq_start[s])
        _close(out[s, 0], v[st:st + n, 0].mean(0), 1e-12, "q=0 mean")
        _close(lse[s], np.full(Hq, math.log(n)), 1e-12, "q=0 lse")
    # identical keys: uniform weights again, lse = z + ln n
    case = W.gqa_decode_case("samek", 23, [9, 33], Hq=Hq, Hkv=Hkv, D=D, block_size=B)
    case.key[:] = case.key[0]
    kc, vc = oracle_cache(orc, case)
    out, lse = orc.paged_decode_gqa(W.bf16_bits(case.query), kc, vc, case.paging.block_table,
                                    case.context_lens, B, case.scale)
    q, k, v = _f64(case.query), _f64(case.key), _f64(case.value)
    for s, n in enumerate(case.context_lens):
        st = int(case.paging.seq_start[s])
        for h in range(Hq):
            z = case.scale * float(np.dot(q[s, h], k[0, 0]))
            _close(out[s, h], v[st:st + n, 0].mean(0), 1e-12, "same-k mean")
            _close(lse[s, h], z + math.log(n), 1e-12, "same-k lse")


def pin_gqa_equals_mha(orc):
    """GQA with group g equals MHA over K/V repeated g times per head."""
    case = W.gqa_decode_case("g", 31, [20, 77], Hq=6, Hkv=2, D=64, block_size=16)
    kc, vc = oracle_cache(orc, case)
    out, lse = orc.paged_decode_gqa(W.bf16_bits(case.query), kc, vc, case.paging.block_table,
                                    case.context_lens, 16, case.scale)
    mha = W.GQADecodeCase("m", 6, 6, 64, case.paging, case.query,
                          case.key.repeat_interleave(3, dim=1).contiguous(),
                          case.value.repeat_interleave(3, dim=1).contiguous(), case.scale)
    kc2, vc2 = oracle_cache(orc, mha)
    out2, lse2 = orc.paged_decode_gqa(W.bf16_bits(mha.query), kc2, vc2, mha.paging.block_table,
                                      mha.context_lens, 16, mha.scale)
    _close(out, out2, 1e-13, "gqa vs mha out")
    _close(lse, lse2, 1e-13, "gqa vs mha lse")


def pin_split_invariance(orc):
    """Partial attention over any split, LSE-merged, equals the unsplit result."""
    case = W.tiny_gqa()
    kc, vc = oracle_cache(orc, case)
    qb = W.bf16_bits(case.query)
    bt = case.paging.block_table
    lens = case.context_lens
    full_out, full_lse = orc.paged_decode_gqa(qb, kc, vc, bt, lens, case.B, case.scale)
    rng = np.random.default_rng(9)
    splits = [[128 * i for i in range(1, 5)]]  # 128-token partitions
    splits += [sorted(rng.choice(np.arange(1, 511), size=k, replace=False).tolist())
               for k in (1, 3, 7)]
    for cuts in splits:
        edges = [0] + cuts + [10 ** 9]
        outs, lses = [], []
        for a, b in zip(edges[:-1], edges[1:]):
            tb = np.minimum(lens, a).astype(np.int32)
            te = np.minimum(lens, b).astype(np.int32)
            o, l = orc.paged_attn_gqa(qb, kc, vc, bt, tb, te, case.B, case.scale)
            outs.append(o)
            lses.append(l)
        m_out, m_lse = orc.merge(np.stack(outs), np.stack(lses))
        _close(m_out, full_out, 1e-12, f"split {cuts} out")
        _close(m_lse, full_lse, 1e-12, f"split {cuts} lse")


def pin_merge_properties(orc):
    rng = np.random.default_rng(3)
    R, D = 5, 16
    o = rng.standard_normal((3, R, D))
    l = rng.standard_normal((3, R)) * 4
    # an empty (-inf) part is the identity
    e_out, e_lse = orc.merge(np.stack([o[0], np.zeros((R, D))]),
                             np.stack([l[0], np.full(R, -np.inf)]))
    _close(e_out, o[0], 0, "merge identity out")
    _close(e_lse, l[0], 0, "merge identity lse")
    # all parts empty: zero output, -inf lse, no NaN
    z_out, z_lse = orc.merge(np.zeros((2, R, D)), np.full((2, R), -np.inf))
    assert np.all(z_out == 0) and np.all(np.isneginf(z_lse))
    # commutative and associative
    a_out, a_lse = orc.merge(o[[0, 1, 2]], l[[0, 1, 2]])
    b_out, b_lse = orc.merge(o[[2, 0, 1]], l[[2, 0, 1]])
    _close(a_out, b_out, 1e-13, "commute")
    _close(a_lse, b_lse, 1e-13, "commute lse")
    p_out, p_lse = orc.merge(o[[0, 1]], l[[0, 1]])
    c_out, c_lse = orc.merge(np.stack([p_out, o[2]]), np.stack([p_lse, l[2]]))
    _close(c_out, a_out, 1e-13, "assoc")
    _close(c_lse, a_lse, 1e-13, "assoc lse")
    # closed form: lse = log(sum exp), weights exp(l_i - lse)
    L = np.log(np.exp(l).sum(0))
    _close(a_lse, L, 1e-13, "merge lse closed form")
    _close(a_out, (np.exp(l - L)[..., None] * o).sum(0), 1e-13, "merge out closed form")


def pin_block_permutation(orc):
    """Relabelling physical blocks (and the table) leaves results unchanged."""
    case = W.tiny_gqa()
    kc, vc = oracle_cache(orc, case)
    qb = W.bf16_bits(case.query)
    out, lse = orc.paged_decode_gqa(qb, kc, vc, case.paging.block_table, case.context_lens,
                                    case.B, case.scale)
    rng = np.random.default_rng(4)
    nb = case.paging.num_blocks
    perm = rng.permutation(nb)  # new id of old block b is perm[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = perm[case.paging.block_table].astype(np.int32)
    out2, lse2 = orc.paged_decode_gqa(qb, kc2, vc2, bt2, case.context_lens, case.B, case.scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# ---------------------------------------------------------------------------
# MLA
# ---------------------------------------------------------------------------

def _mla_cache(orc, case):
    kv = np.full((case.paging.num_blocks, case.B, case.Dl), 0x7FC0, dtype=np.uint16)
    orc.cache_write_latent(W.bf16_bits(case.latent), case.paging.slot_mapping, kv, case.B)
    return kv


def pin_mla_vs_numpy(orc):
    cases = W.mla_decode_cases("mla_small", 41, S=3, lens_range=None, lens=[1, 70, 129], Hq=4,
                               Dl=576, Dv=512, block_sizes=(1, 64, 16), scale=1 / math.sqrt(192))
    ref = None
    for B, case in cases.items():
        kv = _mla_cache(orc, case)
        out, lse = orc.paged_decode_mla(W.bf16_bits(case.query), kv, case.paging.block_table,
                                        case.context_lens, B, case.Dv, case.scale)
        if ref is None:
            ref = np_ref.mla_decode(_f64(case.query), _f64(case.latent), case.paging.seq_start,
                                    case.context_lens, case.Dv, case.scale)
        _close(out, ref[0], 1e-12, f"mla bs{B} out")
        _close(lse, ref[1], 1e-12, f"mla bs{B} lse")


# ---------------------------------------------------------------------------
# Extend
# ---------------------------------------------------------------------------

def extend_oracle_inputs(orc, case):
    kc, vc = oracle_cache(orc, case)
    rows = case.new_rows()
    kn = W.bf16_bits(case.key)[rows]
    vn = W.bf16_bits(case.value)[rows]
    return kc, vc, kn, vn


def pin_extend_vs_numpy(orc):
    case = W.extend_case("ext_small", 51, ctx_lens=[300, 0, 45], new_tokens=[37, 5, 16], Hq=4,
                         Hkv=2, D=64, block_size=16)
    kc, vc, kn, vn = extend_oracle_inputs(orc, case)
    qb = W.bf16_bits(case.query)
    out, lse = orc.extend(qb, kn, vn, case.query_start_loc, kc, vc, case.paging.block_table,
                          case.ctx_lens, case.B, case.scale)
    rout, rlse = np_ref.extend(_f64(case.query), _f64(case.key), _f64(case.value),
                               case.paging.seq_start, case.ctx_lens, case.new_lens, case.scale)
    _close(out, rout, 1e-12, "extend out")
    _close(lse, rlse, 1e-12, "extend lse")
    # a row selection computes exactly the selected rows and leaves the rest zero
    mask = np.zeros(lse.shape, dtype=np.uint8)
    mask[::3, 1] = 1
    mask[-1, :] = 1
    mo, ml = orc.extend(qb, kn, vn, case.query_start_loc, kc, vc, case.paging.block_table,
                        case.ctx_lens, case.B, case.scale, row_mask=mask)
    sel = mask.astype(bool)
    _close(mo[sel], rout[sel], 1e-12, "masked extend out")
    _close(ml[sel], rlse[sel], 1e-12, "masked extend lse")
    assert not mo[~sel].any() and not ml[~sel].any()
    # the chunked recipe equals the definition for any chunk length
    for chunk in (16, 64, 160, 4096):
        cout, clse = orc.extend_chunked(qb, kn, vn, case.query_start_loc, kc, vc,
                                        case.paging.block_table, case.ctx_lens, case.B,
                                        case.scale, chunk)
        _close(cout, out, 1e-12, f"extend chunk {chunk} out")
        _close(clse, lse, 1e-12, f"extend chunk {chunk} lse")


ALL_PINS = [
    pin_shuffle_layout,
    pin_cache_write_skips,
    pin_gather_roundtrip,
    pin_standard_layout,
    pin_fp8_codes,
    pin_fp8_quantize_and_bf16,
    pin_fp8_cache_layout,
    pin_fp8_decode_matches_bf16,
    pin_fp8_mla_matches_bf16,
    pin_fp8_gather_dequant,
    pin_latent_write,
    pin_decode_vs_numpy,
    pin_decode_closed_forms,
    pin_gqa_equals_mha,
    pin_split_invariance,
    pin_merge_properties,
    pin_block_permutation,
    pin_mla_vs_numpy,
    pin_extend_vs_numpy,
]
