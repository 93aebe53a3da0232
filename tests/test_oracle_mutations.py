"""Plant plausible mistakes in a copy of the oracle and check that a pin fails.

Each mutation is a (snippet, replacement) text edit: a dropped term, a wrong
index, a transposed operand, an off-by-one.  An edited copy of oracle.c is
compiled to a temporary library on the CPU, an edited copy of fp8.py is
loaded in place of ``oracle.fp8``, and every pin in oracle_pins runs against it;
the mutation must make at least one of them fail.  This shows the pins are
strong enough to catch that class of error in the oracle.  Each mutant runs
in a child process, since a planted index error may also crash it (which
counts as caught too, but is reported separately).
"""
import json
import os
import subprocess
import sys

import pytest

import oracle
import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MUTATIONS = {
    "k_layout_dim_split_swapped": (
        "((((p * Hkv + g) * (D / x) + d / x) * B + o) * x) + d % x",
        "((((p * Hkv + g) * (D / x) + d % x) * B + o) * x) + d / x"),
    "v_layout_token_dim_transposed": (
        "((((p * Hkv + g) * (B / x) + o / x) * D + d) * x) + o % x",
        "((((p * Hkv + g) * (B / x) + o % x) * D + d) * x) + o / x"),
    "bf16_wrong_shift": ("((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    "scale_dropped": ("z[t] = scale * acc;\n            }\n            softmax_apply(z, n, V, D,",
                      "z[t] = acc;\n            }\n            softmax_apply(z, n, V, D,"),
    "lse_max_term_dropped": ("*lse = m + log(l);", "*lse = log(l);"),
    "normalisation_dropped": ("out[d] /= l;", "out[d] /= 1.0;"),
    "gqa_head_map_modulo": ("int g = h / group;\n            int64_t b",
                            "int g = h % Hkv;\n            int64_t b"),
    "block_index_uses_offset": (
        "int64_t p = block_table[(int64_t)s * max_blocks + pos / B], o = pos % B;\n                double acc = 0.0;\n                for (int d = 0; d < D; d++) {",
        "int64_t p = block_table[(int64_t)s * max_blocks + pos % B], o = pos % B;\n                double acc = 0.0;\n                for (int d = 0; d < D; d++) {"),
    "merge_weight_unnormalised": ("double w = exp(li - L);", "double w = exp(li - m);"),
    "extend_misses_self": ("int64_t n = c + i + 1;", "int64_t n = c + i;"),
    "mla_value_offset": ("V[t * Dv + c] = bf(row[c]);", "V[t * Dv + c] = bf(row[c + 64]);"),
    "gather_row_offset": ("int64_t row = out_start[s] + (t - tok_begin[s]);",
                          "int64_t row = out_start[s] + t;"),
    "latent_write_transposed": ("kv_cache[(p * B + o) * Dl + c]", "kv_cache[(o * B + p) * Dl + c]"),
    "cache_write_skip_check_dropped": ("if (slot < 0 || slot >= num_blocks * B)\n            continue;\n        int64_t p = slot / B, o = slot % B;\n        for (int g",
                                       "if (slot < 0)\n            continue;\n        if (slot >= num_blocks * B) slot = num_blocks * B - 1;\n        int64_t p = slot / B, o = slot % B;\n        for (int g"),
}


# mistakes in the FP8 oracle (oracle/fp8.py)
FP8_MUTATIONS = {
    "gather_scales_swapped": ("kf = _TABLE[K].astype(np.float32) * np.float32(k_scale)",
                              "kf = _TABLE[K].astype(np.float32) * np.float32(v_scale)"),
    "gather_range_one_too_long": ("t0, t1 = iteration * chunk, min((iteration + 1) * chunk, int(n))",
                                  "t0, t1 = iteration * chunk, min((iteration + 1) * chunk + 1, int(n))"),
    "gather_range_starts_late": ("t0, t1 = iteration * chunk, min((iteration + 1) * chunk, int(n))",
                                 "t0, t1 = iteration * chunk + 1, min((iteration + 1) * chunk, int(n))"),
    "gather_v_token_dim_transposed": ("V[j] = v_cache[p, :, o // X, :, o % X]",
                                      "V[j] = v_cache[p, :, o % X, :, o // X]"),
    "gather_product_rounded_from_f64": (
        "vs.append(bf16_rne(vf))",
        "vs.append(_bf16_direct(_TABLE[V] * float(np.float32(v_scale))))"),
}
_BF16_DIRECT = '''

def _bf16_direct(x):
    """float64 -> bf16 by rounding the float64 itself to nearest even."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    for i, v in np.ndenumerate(x):
        m, e = np.frexp(v)
        q = np.round(m * 256.0)  # numpy rounds halves to even
        out[i] = (np.float32(np.ldexp(q, e - 8)).view(np.uint32) >> 16).astype(np.uint16)
    return out
'''


def _run_all_pins(orc):
    """Names of the pins that fail against ``orc``."""
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    with open(os.path.join(GOLDEN, "shuffle_offsets.json")) as f:
        try:
            P.pin_shuffle_golden(orc, json.load(f))
        except AssertionError:
            failed.append("pin_shuffle_golden")
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    with open(oracle.SRC) as f:
        src = f.read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation site for {name} no longer in oracle.c"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = str(tmp_path / "liboracle_mut.so")
    oracle.build(str(mutated), lib, openmp=False)
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle, test_oracle_mutations as T\n"
            "failed = T._run_all_pins(oracle.Oracle(%r))\n"
            "print('FAILED_PINS', failed)\n"
            "sys.exit(3 if failed else 0)\n") % (os.path.dirname(here), here, lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutation {name} passed every pin: {r.stdout[-500:]}"
    if r.returncode == 3:
        assert "FAILED_PINS" in r.stdout


@pytest.mark.parametrize("name", sorted(FP8_MUTATIONS))
def test_fp8_mutation_is_caught(name, tmp_path):
    src_path = os.path.join(os.path.dirname(oracle.SRC), "fp8.py")
    with open(src_path) as f:
        src = f.read()
    old, new = FP8_MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation site for {name} no longer in fp8.py"
    mutated = tmp_path / "fp8_mut.py"
    mutated.write_text(src.replace(old, new, 1) + _BF16_DIRECT)
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import importlib.util, oracle\n"
            "spec = importlib.util.spec_from_file_location('oracle.fp8', %r)\n"
            "mod = importlib.util.module_from_spec(spec); spec.loader.exec_module(mod)\n"
            "sys.modules['oracle.fp8'] = mod; oracle.fp8 = mod\n"
            "import test_oracle_mutations as T\n"
            "failed = T._run_all_pins(oracle.get())\n"
            "print('FAILED_PINS', failed)\n"
            "sys.exit(3 if failed else 0)\n") % (os.path.dirname(here), here, str(mutated))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutation {name} passed every pin: {r.stdout[-500:]}"
    if r.returncode == 3:
        assert "FAILED_PINS" in r.stdout
