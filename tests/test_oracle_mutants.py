"""Plausible mistakes planted in a copy of the oracle must each fail a pin.

Every mutant below is a one-spot textual change to oracle/pa_oracle.c,
compiled into a temporary library and checked by running oracle_pins.py
against it in a child process (a mutant may read out of bounds, so it never
runs inside the test process).  A mutant that passes every pin would mean
the pins cannot see that mistake.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pa_oracle.c")

MUTANTS = {
    "block_index_mod": ("int32_t logical_block = i / block_size;",
                        "int32_t logical_block = i % block_size;"),
    "offset_div": ("int32_t logical_block = i / block_size;\n        int32_t offset = i % block_size;",
                   "int32_t logical_block = i / block_size;\n        int32_t offset = i / block_size;"),
    "fp8_gather_offset_div": ("int32_t offset = i % block_size;\n        if (physical < 0",
                              "int32_t offset = i / block_size;\n        if (physical < 0"),
    "fp8_gather_block_mod": ("max_blocks_per_seq + i / block_size];", "max_blocks_per_seq + i % block_size];"),
    "drop_last_token": ("for (int32_t i = 0; i < L; ++i) {\n        int32_t logical_block",
                        "for (int32_t i = 0; i < L - 1; ++i) {\n        int32_t logical_block"),
    "drop_first_token": ("for (int32_t i = 0; i < L; ++i) {\n        double w",
                         "for (int32_t i = 1; i < L; ++i) {\n        double w"),
    "no_scale": ("logits[i] = dot * scale;", "logits[i] = dot;"),
    "exp_sign": ("logits[i] = exp(logits[i] - m);", "logits[i] = exp(m - logits[i]);"),
    "no_max_shift": ("logits[i] = exp(logits[i] - m);", "logits[i] = exp(logits[i]);"),
    "no_normalise": ("double w = logits[i] / Z;", "double w = logits[i];"),
    "layout_head_offset_swapped": ("return (size_t)(((block * block_size + offset) * num_heads + head) * head_dim + d);",
                                   "return (size_t)(((block * num_heads + head) * block_size + offset) * head_dim + d);"),
    "value_from_key_cache": ("v_out[(int64_t)i * head_dim + d] = oracle_half_to_double(v_cache[src]);",
                             "v_out[(int64_t)i * head_dim + d] = oracle_half_to_double(k_cache[src]);"),
    "q_row_of_head0": ("const uint16_t *qrow = q + ((int64_t)s * num_heads + h) * head_dim;",
                       "const uint16_t *qrow = q + ((int64_t)s * num_heads) * head_dim;"),
    "dot_skips_last_dim": ("for (int32_t d = 0; d < head_dim; ++d)\n            dot += q[d]",
                           "for (int32_t d = 0; d < head_dim - 1; ++d)\n            dot += q[d]"),
    "half_bias": ("v = ldexp((double)(1024 + frac), expo - 25);",
                  "v = ldexp((double)(1024 + frac), expo - 24);"),
    "half_subnormal": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    "half_no_implicit_bit": ("v = ldexp((double)(1024 + frac), expo - 25);",
                             "v = ldexp((double)frac, expo - 25);"),
    "half_nan_as_inf": ("v = frac ? NAN : INFINITY;", "v = INFINITY;"),
    "reshape_block_mod": ("int64_t block = slot / block_size;", "int64_t block = slot % block_size;"),
    "reshape_no_upper_check": ("if (slot < 0 || slot >= num_slots)\n            continue;\n        int64_t block",
                               "if (slot < 0)\n            continue;\n        int64_t block"),
    "fp8_reshape_no_upper_check": ("if (slot < 0 || slot >= num_slots)\n            continue;\n        /*",
                                   "if (slot < 0)\n            continue;\n        /*"),
    "reshape_value_gets_key": ("v_cache[dst] = value[src];", "v_cache[dst] = key[src];"),
    "copy_direction": ("k_cache[dst * block_elems + e] = k_cache[src * block_elems + e];",
                       "k_cache[src * block_elems + e] = k_cache[dst * block_elems + e];"),
    "copy_skips_v": ("            v_cache[dst * block_elems + e] = v_cache[src * block_elems + e];\n", ""),
    "swap_no_range_check": ("        if (a < 0 || a >= src_blocks || b < 0 || b >= dst_blocks)\n            return OR_ERR_RANGE;\n", ""),
    "swap_uses_dst_index_for_src": ("dst[b * block_elems + e] = src[a * block_elems + e];",
                                    "dst[b * block_elems + e] = src[b * block_elems + e];"),
    "e4m3_bias": ("v = ldexp((double)(8 + mant), expo - 10);", "v = ldexp((double)(8 + mant), expo - 9);"),
    "e4m3_subnormal": ("v = ldexp((double)mant, -9);", "v = ldexp((double)mant, -10);"),
    "e4m3_no_nan": ("    if (expo == 15 && mant == 7)\n        return NAN;\n", ""),
    "e4m3_ties_away": ("if (dc < db || (dc == db && (c & 1) == 0))", "if (dc < db || dc == db)"),
    "e4m3_ties_down": ("if (dc < db || (dc == db && (c & 1) == 0))", "if (dc < db)"),
    "e4m3_overflow_to_nan": ("        return (uint8_t)(sign | 0x7E);", "        return (uint8_t)(sign | 0x7F);"),
    "fp8_k_scale_dropped": ("oracle_e4m3_to_double(k_cache[src]) * (double)k_scale;",
                            "oracle_e4m3_to_double(k_cache[src]);"),
    "fp8_v_from_k": ("oracle_e4m3_to_double(v_cache[src]) * (double)v_scale;",
                     "oracle_e4m3_to_double(k_cache[src]) * (double)v_scale;"),
    "fp8_reshape_value_k_scale": ("oracle_quantize_e4m3(value + t * row, v_cache + slot * row, row, v_scale);",
                                  "oracle_quantize_e4m3(value + t * row, v_cache + slot * row, row, k_scale);"),
    "fp8_quantize_scale_not_inverted": ("float y = xf * inv;", "float y = xf * scale;"),
    "prefill_excludes_self": ("int32_t visible = L - n + i + 1;", "int32_t visible = L - n + i;"),
    "prefill_positions_from_zero": ("int32_t visible = L - n + i + 1;", "int32_t visible = i + 1;"),
    "prefill_sees_everything": ("int32_t visible = L - n + i + 1;", "int32_t visible = L;"),
    "prefill_rows_reversed": ("int32_t row = query_start[s] + i;",
                              "int32_t row = query_start[s + 1] - 1 - i;"),
    "prefill_fp8_scales_swapped": ("max_blocks_per_seq, k_scale, v_scale)",
                                   "max_blocks_per_seq, v_scale, k_scale)"),
    "prefill_fp8_v_scale_as_k": ("k_cache, v_cache, k_scale, v_scale, block_tables,",
                                 "k_cache, v_cache, k_scale, k_scale, block_tables,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    lib = obuild.build(str(src), str(tmp_path / f"lib{name}.so"), quiet=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), "--lib", lib,
                        "--fail-fast"],
                       capture_output=True, text=True, timeout=300,
                       env={**os.environ, "OMP_NUM_THREADS": "2"})
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"


def test_unmutated_copy_passes(tmp_path):
    """Control: the same harness accepts the oracle as committed."""
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    lib = obuild.build(SRC, str(tmp_path / "libcontrol.so"), quiet=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), "--lib", lib],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
