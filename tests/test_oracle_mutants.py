"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one (CPU only). Each mutant is compiled to a temporary library and
the pin suite is run against it in a subprocess; it must fail."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from oracle import qref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAST = "not f16_rne and not bf16_rne"

# (name, text in qref.c, replacement, pytest -k selection)
MUTANTS = [
    ("lane_shift", "uint64_t shifted = window >> ((i * bits) % 32);",
     "uint64_t shifted = window >> ((i * bits) % 31);", FAST),
    ("next_word_unclamped_off_by_one", "int64_t w_next = (w + 1 < words) ? w + 1 : words - 1;",
     "int64_t w_next = (w + 1 < words) ? w : words - 1;", FAST),
    ("pack_straddle_dropped", "row[w + 1] |= q >> (32 - off);", "(void)0;", FAST),
    ("group_index", "int64_t g = i / group_size;", "int64_t g = i % group_size;", FAST),
    ("dequant_sign", "return prod + b;", "return prod - b;", FAST),
    ("scale_divisor", "float qmax = (float)((1 << bits) - 1);",
     "float qmax = (float)(1 << bits);", FAST),
    ("min_max_swapped", "float s = (mx - mn) / qmax;", "float s = (mx - mn) / qmax * 1.0001f;",
     FAST),
    ("round_to_even_codes", "float t = roundf((wg[i] - bq) / sq);",
     "float t = rintf((wg[i] - bq) / sq);", FAST),
    ("floor_codes", "float t = roundf((wg[i] - bq) / sq);",
     "float t = floorf((wg[i] - bq) / sq);", FAST),
    ("bias_from_unrounded_min", "float t = roundf((wg[i] - bq) / sq);",
     "float t = roundf((wg[i] - mn) / s);", FAST),
    ("moe_strides_swapped", "int64_t a_off = (p / top_k) * a_outer + (p % top_k) * a_inner;",
     "int64_t a_off = (p / top_k) * a_inner + (p % top_k) * a_outer;", FAST),
    ("moe_expert_stride", "int64_t row = (int64_t)ids[p] * n_rows + r;",
     "int64_t row = (int64_t)ids[p] * n_cols / 8 + r;", FAST),
    ("silu_sign", "static double silu(double z) { return z / (1.0 + exp(-z)); }",
     "static double silu(double z) { return z / (1.0 + exp(z)); }", FAST),
    ("product_operand", "mag += fabs(xv) * fabs(wv);", "mag += fabs(xv) + fabs(wv);", FAST),
    ("typed_dequant_single_rounding", "double prod = round_to_type(q * s, sb_dtype, NULL, 0);",
     "double prod = q * s;", FAST),
    ("fp4_exponent_bias", "(1.0 + m / 2.0) * ldexp(1.0, e - 1);", "(1.0 + m / 2.0) * ldexp(1.0, e - 2);",
     FAST),
    ("e4m3_subnormal_scale", "m * ldexp(1.0, -9)", "m * ldexp(1.0, -10)", FAST),
    ("e8m0_bias", "return ldexp(1.0, (int)s - 127);", "return ldexp(1.0, (int)s - 126);", FAST),
    ("nvfp4_scale_format", "double scale = mode == QREF_NVFP4 ? qref_fp8_e4m3(sb) : qref_e8m0(sb);",
     "double scale = qref_e8m0(sb);", FAST),
    ("mx_group_index", "uint32_t sb = row_scales[i / group_size];",
     "uint32_t sb = row_scales[i / 32];", FAST),
    ("mx_magnitude_sum", "mag += fabs(term);", "mag += term;", FAST),
    ("ffn_slot_row", "acc += (double)rw[p] * (double)load_elem(o_out, a_dtype, p * d_model + d);",
     "acc += (double)rw[p] * (double)load_elem(o_out, a_dtype, (t + j * n_tokens) * d_model + d);",
     FAST),
    ("ffn_h_unrounded", "round_to_type(silu_v[i], a_dtype, h_out, i);",
     "round_to_type(silu_v[i] * 1.001, a_dtype, h_out, i);", FAST),
    ("int8_offset", "float shifted = (float)q + 128.0f;", "float shifted = (float)q + 127.0f;", FAST),
    ("int8_step", "float step = (range[1] - range[0]) / 255.0f;\n#pragma omp parallel for schedule(static)\n    for (int64_t i = 0; i < count; ++i)",
     "float step = (range[1] - range[0]) / 256.0f;\n#pragma omp parallel for schedule(static)\n    for (int64_t i = 0; i < count; ++i)", FAST),
    ("int8_quant_offset", "float t = roundf((w[i] - lo) / step) - 128.0f;",
     "float t = roundf((w[i] - lo) / step) - 127.0f;", FAST),
    ("qmatmul_t_row_index", "double wv = (double)dequant_elem(wq + i * words, words, scales, biases, sb_dtype,\n                                                 i * groups, j, bits, group_size);",
     "double wv = (double)dequant_elem(wq + i * words, words, scales, biases, sb_dtype,\n                                                 i * groups, j % k, bits, group_size);", FAST),
    ("qmatmul_t_magnitude", "mag += fabs(t_ij);", "mag += t_ij;", FAST),
    ("rne_ties_up", "r = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;", "r = lo + 1.0;", "rne"),
    ("f16_decode_exponent", "v = ldexp((double)(1024 + m), e - 25);",
     "v = ldexp((double)(1024 + m), e - 24);", "f16 or decoders"),
    ("f16_subnormal_boundary", "if (e < emin)\n        e = emin;", "if (e < emin - 1)\n        e = emin - 1;",
     "f16_rne"),
]


@pytest.mark.parametrize("name,old,new,select", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, select):
    src = open(qref.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant_c = tmp_path / "qref_mutant.c"
    mutant_c.write_text(src.replace(old, new))
    (tmp_path / "qref.h").write_text(open(os.path.join(qref.HERE, "qref.h")).read())
    lib = tmp_path / "libqref_mutant.so"
    cmd = [c for c in qref.BUILD_CMD]
    cmd[cmd.index(qref.SRC)] = str(mutant_c)
    cmd[cmd.index("-o") + 1] = str(lib)
    subprocess.check_call(cmd)
    env = dict(os.environ, QREF_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", select],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
