"""Each plausible mistake planted in a copy of the C oracle (on the CPU, in a temp
directory) must make at least one pin fail; otherwise the pins would not pin."""
import os
import tempfile

import pytest

import oracle
from tests.oracle_pins import PINS

# (name, original text, replacement) -- every original must occur in the source exactly once
MUTANTS = [
    ("scale_divides_by_16", "(hi - lo) / 15.0f", "(hi - lo) / 16.0f"),
    ("range_excludes_zero", "float lo = 0.0f, hi = 0.0f;", "float lo = w[0], hi = w[0];"),
    ("zp_sign_flipped", "rintf(-lo / s)", "rintf(lo / s)"),
    ("codes_subtract_zp", "(int)rintf(w[i] / s) + zp;", "(int)rintf(w[i] / s) - zp;"),
    ("codes_use_fp32_scale", "(int)rintf(w[i] / s) + zp;", "(int)rintf(w[i] / s32) + zp;"),
    ("codes_truncate", "(int)rintf(w[i] / s) + zp;", "(int)(w[i] / s) + zp;"),
    ("codes_round_half_away", "(int)rintf(w[i] / s) + zp;", "(int)roundf(w[i] / s) + zp;"),
    ("scale_stored_transposed", "scale16[g * N + n] = sh;", "scale16[n * G + g] = sh;"),
    ("nibbles_swapped", "(uint8_t)(first | (second << 4))", "(uint8_t)(second | (first << 4))"),
    ("act_divides_by_128", "float s = amax / 127.0f;", "float s = amax / 128.0f;"),
    ("act_clamps_to_128", "if (r < -127.0f)\n                    r = -127.0f;",
     "if (r < -128.0f)\n                    r = -128.0f;"),
    ("act_rounds_half_away", "float r = rintf(row[k] / s);", "float r = roundf(row[k] / s);"),
    ("isum_adds_zp",
     "isums[(g * M + m) * N + n] = acc;", "isums[(g * M + m) * N + n] = acc + 2 * z * 0 + (m == 0 ? z : 0);"),
    ("gemm_scale_index_transposed",
     "double term = (double)a_scale[m] * (double)orc_f16_to_f32(scale16[g * N + n]) * (double)isum;\n"
     "                total += term;",
     "double term = (double)a_scale[m] * (double)orc_f16_to_f32(scale16[n * G + g]) * (double)isum;\n"
     "                total += term;"),
    ("gemm_drops_act_scale",
     "double term = (double)a_scale[m] * (double)orc_f16_to_f32(scale16[g * N + n]) * (double)isum;\n"
     "                total += term;",
     "double term = (double)orc_f16_to_f32(scale16[g * N + n]) * (double)isum;\n"
     "                total += term;"),
    ("gemm_group_off_by_one", "for (int64_t k = g * group; k < (g + 1) * group; ++k)\n"
     "                    isum += (int32_t)qa[m * K + k] * ((int32_t)q[n * K + k] - z);\n"
     "                double term",
     "for (int64_t k = g * group; k < (g + 1) * group; ++k)\n"
     "                    isum += (int32_t)qa[m * K + k] * ((int32_t)q[n * K + (k + 1) % K] - z);\n"
     "                double term"),
    ("f16_truncates", "double frac = rint((m - 1.0) * 1024.0);", "double frac = floor((m - 1.0) * 1024.0);"),
    ("f16_no_subnormals", "double n = rint(ldexp(a, 24));", "double n = 0.0;"),
    ("topk_ties_to_higher_id", "if (best < 0 || z[e] > z[best])", "if (best < 0 || z[e] >= z[best])"),
    ("softmax_without_exp", "denom += exp((double)z[ids[t * k + j]] - zmax);",
     "denom += ((double)z[ids[t * k + j]] - zmax) + 1.0;"),
    ("bucket_offsets_inclusive", "offsets[ids[p] + 1] += 1;", "offsets[ids[p]] += 1;"),
    ("silu_uses_plus", "h[p * I + i] = g / (1.0 + exp(-g)) * u;", "h[p * I + i] = g / (1.0 + exp(g)) * u;"),
    ("combine_drops_shared", "acc += (double)y_shared[t * H + c];", "acc += 0.0;"),
    ("sym_divides_by_8", "orc_f32_to_f16(amax / 7.0f)", "orc_f32_to_f16(amax / 8.0f)"),
    ("sym_scale_transposed", "scale16[n + g * N] = sh;", "scale16[n * G + g] = sh;"),
    ("sym_code_offset_7", "(uint8_t)((int)r + 8)", "(uint8_t)((int)r + 7)"),
    ("sym_uses_signed_max", "if (fabsf(w[i]) > amax)\n                    amax = fabsf(w[i]);",
     "if (w[i] > amax)\n                    amax = w[i];"),
    ("percentile_no_interpolation", "r += (h - (double)i) * ((double)t[i + 1] - (double)t[i]);",
     "r += 0.0 * ((double)t[i + 1] - (double)t[i]);"),
    ("percentile_index_over_n", "double h = (double)(n - 1) * pct / 100.0;", "double h = (double)n * pct / 100.0;"),
    ("clip_upper_only", "out[n * K + k] = w < lo ? lo : (w > hi ? hi : w);", "out[n * K + k] = w > hi ? hi : w;"),
    ("smooth_alpha_swapped", "pow((double)ax[k], alpha) / pow((double)aw[k], 1.0 - alpha)",
     "pow((double)ax[k], 1.0 - alpha) / pow((double)aw[k], alpha)"),
    ("smooth_zero_guard_either", "if (ax[k] > 0.0f && aw[k] > 0.0f)", "if (ax[k] > 0.0f || aw[k] > 0.0f)"),
    ("smooth_inv_from_unrounded", "inv_s[k] = (float)(1.0 / (double)s[k]);", "inv_s[k] = (float)(1.0 / f);"),
    ("smooth_weights_divide", "out[n * K + k] = W[n * K + k] * s[k];", "out[n * K + k] = W[n * K + k] / s[k];"),
    ("smooth_act_divides", "y[m * K + k] = x[m * ldx + k] * inv_s[k];", "y[m * K + k] = x[m * ldx + k] / inv_s[k];"),
    ("absmax_signed", "float a = fabsf(A[r * K + k]);", "float a = A[r * K + k];"),
    ("absmax_transposed", "float a = fabsf(A[r * K + k]);", "float a = fabsf(A[k * rows + r]);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.build(source=path, out=os.path.join(d, f"lib_{name}.so"))
        orc = oracle.Oracle(lib)
        failed = []
        for pin_name, pin in PINS.items():
            try:
                pin(orc)
            except AssertionError:
                failed.append(pin_name)
            except (ValueError, IndexError, FloatingPointError):
                failed.append(pin_name)
        assert failed, f"planted mistake {name} was not caught by any pin"
