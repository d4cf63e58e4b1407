"""The pins catch plausible mistakes: each mutant below plants one mistake in a copy
of the oracle's C source (on the CPU), and the pin suite must fail on it."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bitlinear_oracle.c")

# (name, text in the source, replacement, occurrence index or None for all)
MUTANTS = [
    ("round_half_away", "rintf(", "roundf(", None),
    ("no_weight_clip", "if (v > 1.0f) v = 1.0f;", "", None),
    ("int8_no_eps_clamp", "float s = 127.0f / a;", "float s = 127.0f / (amax + 1e-7f);", None),
    ("int8_divide_not_multiply", "load_elem(X, x_dtype, m * K + k) * s", "load_elem(X, x_dtype, m * K + k) / (1.0f / s)", None),
    ("int4_scale_over_8", "float s = a / 7.0f;", "float s = a / 8.0f;", None),
    ("dequant_swapped", "bits == 8 ? gamma / s : s * gamma", "bits == 8 ? s * gamma : gamma / s", None),
    ("gamma_ties_away", "round_up = half && (sticky || (mant & 1u));", "round_up = half;", None),
    ("gamma_truncated", "mant += (uint64_t)round_up;", "", None),
    ("relu2_unrectified", "y = r * r;", "y = y * y;", None),
    ("bias_before_rescale", "if (bias) y = y + bias[n];", "if (bias) y = y + bias[n] * f;", None),
    ("pack_msb_first", "(uint8_t)((c + 1) << (2 * (k % 4)))", "(uint8_t)((c + 1) << (2 * (3 - k % 4)))", None),
    ("nibble_high_first", "(uint8_t)((q & 0xF) << (4 * (k % 2)))", "(uint8_t)((q & 0xF) << (4 * (1 - k % 2)))", None),
    ("field_offset", "return field - 1;", "return field - 2 + (field == 0);", None),
    ("bf16_truncate", "u += 0x7FFFu + lsb;", "(void)lsb;", None),
    ("rmsnorm_mean_not_sum", "ss / (double)K + (double)eps", "ss + (double)eps", None),
    ("rmsnorm_no_sqrt", "1.0 / sqrt(ss / (double)K + (double)eps)", "1.0 / (ss / (double)K + (double)eps)", None),
    ("sumsq_truncated", "if (half && (sticky || (mant & 1u))) mant += 1;", "", None),
    ("sumsq_ties_away", "if (half && (sticky || (mant & 1u))) mant += 1;", "if (half) mant += 1;", None),
    ("sumsq_subnormal_hidden_bit", "(h & 0x7Fu) | (e ? 0x80u : 0u)", "(h & 0x7Fu) | 0x80u", None),
    ("sumsq_exponent_not_doubled", "sq_add(acc, m * m, 2 * ee - 2);", "sq_add(acc, m * m, ee - 1);", None),
    ("sumsq_carry_dropped", "const uint64_t t = (uint64_t)acc[i] + add + carry;\n        acc[i] = (uint32_t)t;\n        carry = t >> 32;",
     "const uint64_t t = (uint64_t)acc[i] + add + carry;\n        acc[i] = (uint32_t)t;\n        carry = 0;", None),
    ("layernorm_mean_not_subtracted", "narrow_bf16((float)((v - mu) * r))", "narrow_bf16((float)(v * r))", None),
    ("layernorm_var_over_k", "d / ((double)K * (double)K)", "d / (double)K", None),
    ("layernorm_negatives_added", "ln_add((h & 0x8000u) ? neg : pos, m, ee - 1);", "ln_add(pos, m, ee - 1);", None),
    ("layernorm_mean_square_not_variance", "ln_sub(ks2, s1sq, d);", "memcpy(d, ks2, sizeof d);", None),
    ("layernorm_mean_sign_lost", "*s1_out = negative ? -a1 : a1;", "*s1_out = a1;", None),
    ("layernorm_mul_carry_dropped", "r[i + j] = (uint32_t)t;\n            carry = t >> 32;", "r[i + j] = (uint32_t)t;\n            carry = 0;", None),
    ("layernorm_sums_truncated", "if (half && (sticky || (mant & 1u))) mant += 1;\n    return ldexp((double)mant, low + unit);", "return ldexp((double)mant, low + unit);", None),
    ("layernorm_eps_outside_sqrt", "1.0 / sqrt(var + (double)eps)", "1.0 / (sqrt(var) + (double)eps)", None),
    ("layernorm_subnormal_hidden_bit", "const uint64_t m = (h & 0x7Fu) | (e ? 0x80u : 0u);\n        const int ee", "const uint64_t m = (h & 0x7Fu) | 0x80u;\n        const int ee", None),
    ("rmsnorm_residual_dropped", "v = widen_bf16(narrow_bf16(v + widen_bf16(delta[m * K + k])));", "(void)delta;", None),
    ("hadamard_butterfly_swapped", "blk[i] = u + v;\n                    blk[i + h] = u - v;", "blk[i] = u - v;\n                    blk[i + h] = u + v;", None),
    ("hadamard_stage_skipped", "for (int64_t h = 1; h < b; h *= 2)", "for (int64_t h = 2; h < b; h *= 2)", None),
    ("hadamard_block_uncapped", "while (b < 8192 && K % (2 * b) == 0) b *= 2;", "while (K % (2 * b) == 0) b *= 2;", None),
    ("hadamard_gamma_not_over_b", "*gamma_out = ldexpf(g, -t);", "*gamma_out = g;", None),
    ("hadamard_normalized_by_half", "blk[i + h] = u - v;", "blk[i + h] = 0.5f * (u - v);", None),
    ("bwd_int4_no_gamma", "(double)((float)weight_code(packed, K, n, k) * g)", "(double)weight_code(packed, K, n, k)", None),
    ("bwd_weight_mask_inclusive", "fabsf(load_elem(W, w_dtype, n * K + k)) > 1.5f", "fabsf(load_elem(W, w_dtype, n * K + k)) >= 1.5f", None),
    ("bwd_act_mask_dropped", "if (v < -8.0f || v > 7.0f) acc = 0.0;", "(void)v;", None),
    ("bwd_int8_scale_inverted", "const float f = gamma / act_scale[gran == 0 ? m : 0];", "const float f = act_scale[gran == 0 ? m : 0] / gamma;", None),
    ("bwd_int4_dw_codes_not_dequantized", "(double)((float)q * s)", "(double)q", None),
    ("per_tensor_uses_row_max", "float amax = tensor_max;", "float amax = 0.0f; if (gran == 1) { for (int64_t k = 0; k < K; ++k) { float t = fabsf(load_elem(X, x_dtype, m * K + k)); if (t > amax) amax = t; } }", None),
]


def _build_mutant(src_text: str, out_dir: str, name: str) -> str:
    c_path = os.path.join(out_dir, name + ".c")
    so_path = os.path.join(out_dir, name + ".so")
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-w",
                    "-o", so_path, c_path, "-lm"], check=True)
    return so_path


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, occ):
    src = open(SRC).read()
    assert old in src, "mutation site vanished: " + old
    mutated = src.replace(old, new)
    assert mutated != src
    with tempfile.TemporaryDirectory() as d:
        so = _build_mutant(mutated, d, name)
        env = dict(os.environ, ORACLE_LIB=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pin suite did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
