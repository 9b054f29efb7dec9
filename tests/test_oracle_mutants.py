"""Planted mistakes in a copy of the CPU oracle must fail its pins (no GPU).

Each mutant is the oracle's C source with one plausible slip (a transposed
operand, a wrong index or stride, a dropped term, a wrong sign, an off-by-one
k loop, a wrong rounding rule), built with gcc into a temporary library.  The
pins of tests/test_oracle.py are re-run against it and at least one must
fail; the unmodified source must pass the same pins.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build

from oracle import IN_BF16
from test_oracle import (ACT_PROBE, _brute_force, _encode_bf16_probe_values,
                         _encode_probe_values, bf16_bits, bf16_values, scipy_activation,
                         test_epilogue_bias_and_activation_brute_force)

MUTANTS = {
    "transposed_A_row_major": ("A[i * j->lda + k]", "A[k * j->lda + i]"),
    "transposed_B_col_major": ("B[k + n * j->ldb]", "B[n + k * j->ldb]"),
    "dropped_beta_term": ("out[n] = j->alpha * s + j->beta * cin;",
                          "out[n] = j->alpha * s;"),
    "wrong_sign_beta": ("out[n] = j->alpha * s + j->beta * cin;",
                        "out[n] = j->alpha * s - j->beta * cin;"),
    "short_k_loop": ("for (int64_t k = 0; k < K; ++k) {\n                double p",
                     "for (int64_t k = 0; k < K - 1; ++k) {\n                double p"),
    "c_row_stride": ("i * j->ldc + n", "i * j->N + n"),
    "b_batch_stride": ("j->B + b * j->stride_b", "j->B + b * j->stride_a"),
    "scale_without_abs": ("t += fabs(p);", "t += p;"),
    "subnormal_exponent": ("mag = ldexp((double)f, -24);", "mag = ldexp((double)f, -25);"),
    "ties_away_from_zero": ("double r = nearbyint(n);", "double r = floor(n + 0.5);"),
    "bf16_exponent_bias": ("mag = ldexp((double)(128 + f), e - 134);",
                           "mag = ldexp((double)(128 + f), e - 133);"),
    "bf16_fraction_width": ("int f = h & 127;", "int f = h & 255;"),
    "bf16_ties_away_from_zero": ("double q = nearbyint(t);", "double q = floor(t + 0.5);"),
    "bf16_no_carry_on_rounding": ("        qi = 128;\n        E += 1;\n", "        qi = 128;\n"),
    "bf16_A_decoded_as_binary16": (
        "A[i + k * j->lda];\n    return j->in_type == ORACLE_IN_BF16 ? oracle_decbf16(h) : oracle_dec16(h);",
        "A[i + k * j->lda];\n    return oracle_dec16(h);"),
    "bf16_C_decoded_as_binary16": ("return oracle_decbf16(((const uint16_t *)j->C)[off]);",
                                   "return oracle_dec16(((const uint16_t *)j->C)[off]);"),
    "bias_scaled_by_alpha": ("out[n] += (double)j->bias[n];",
                             "out[n] += j->alpha * (double)j->bias[n];"),
    "scale_without_bias": ("sc[n] += fabs((double)j->bias[n]);", "sc[n] += 0.0;"),
    "activation_dropped": ("out[n] = oracle_activate(j->act, out[n]);", "(void)0;"),
    "gelu_tanh_approximation": ("return 0.5 * x * erfc(-x / sqrt(2.0));",
                                "return 0.5 * x * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)));"),
    "silu_wrong_sign": ("return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));"),
    "relu_leaky": ("return x > 0.0 ? x : 0.0;", "return x > 0.0 ? x : 0.01 * x;"),
}

SHAPES = [(1, 1, 1), (2, 3, 4), (3, 5, 7), (4, 1, 6)]


def _pins_pass(lib) -> bool:
    try:
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        got = oracle.dec16(bits, lib=lib)
        want = bits.view(np.float16).astype(np.float64)
        ok = ~np.isnan(want)
        assert np.array_equal(got[ok], want[ok])
        v = _encode_probe_values()
        with np.errstate(over="ignore"):
            assert np.array_equal(oracle.enc16(v, lib=lib),
                                  v.astype(np.float16).view(np.uint16))
        _brute_force(lib, SHAPES, full_combos=True)
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        got = oracle.decbf16(bits, lib=lib)
        want = bf16_values(bits)
        ok = ~np.isnan(want)
        assert np.array_equal(got[ok], want[ok])
        v = _encode_bf16_probe_values()
        assert np.array_equal(oracle.encbf16(v, lib=lib), bf16_bits(v.astype(np.float32)))
        _brute_force(lib, SHAPES, full_combos=True, in_type=IN_BF16)
        for act in range(4):
            assert np.allclose(oracle.activate(act, ACT_PROBE, lib=lib),
                               scipy_activation(act, ACT_PROBE), rtol=1e-13, atol=1e-300)
        test_epilogue_bias_and_activation_brute_force(lib)
    except (AssertionError, ValueError, OverflowError):
        return False   # a pin failed (or met a NaN/inf where a number was due)
    return True


def _build_variant(tmp_path, name, src):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
                    "-shared", "-fPIC", "-pthread", str(c), "-o", str(so), "-lm"],
                   check=True)
    return oracle.load_library(str(so))


def test_unmodified_oracle_passes(tmp_path):
    src = open(oracle_build.SRC).read()
    assert _pins_pass(_build_variant(tmp_path, "clean", src))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle_build.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    lib = _build_variant(tmp_path, name, src.replace(old, new))
    assert not _pins_pass(lib), f"pins did not catch {name}"


# ------------------------------------------------------------ attention oracle

ATTN_MUTANTS = {
    "softmax_sum_without_max": ("        s += exp(x[j] - m);\n", "        s += exp(x[j]);\n"),
    "online_sum_not_rescaled": ("s = (m == -INFINITY ? 0.0 : s * exp(m - m2)) + acc;",
                                "s = s + acc;"),
    "causal_off_by_one": ("nvis = i + Sk - j->Sq + 1;", "nvis = i + Sk - j->Sq;"),
    "causal_top_left_aligned": ("nvis = i + Sk - j->Sq + 1;", "nvis = i + 1;"),
    "scale_dropped": ("s[k] = j->scale * dot;", "s[k] = dot;"),
    "v_transposed": ("Vb[k * j->v_ld + c]", "Vb[c * j->v_ld + k]"),
    "k_head_stride_of_q": ("j->K + b * j->k_sb + h * j->k_sh", "j->K + b * j->k_sb + h * j->q_sh"),
    "error_scale_without_abs": ("aacc += p[k] * fabs(v);", "aacc += p[k] * v;"),
    "masked_row_divides_zero_by_zero": ("    if (m == -INFINITY) {\n        for (int64_t j = 0; j < n; ++j)\n            y[j] = 0.0;\n        return;\n    }\n",
                                        ""),
}


def _attn_pins_pass(lib, monkeypatch) -> bool:
    import test_oracle_attention as T
    monkeypatch.setattr(oracle, "_lib", lib)
    try:
        for n in (1, 7, 333):
            T.test_softmax_row_matches_scipy(n)
        T.test_softmax_row_masked_elements_and_rows()
        for b in (1, 3, 64):
            T.test_online_recurrence_equals_two_pass(b)
        T.test_softmax_matrix_on_binary16_and_fp32_storage()
        for args in [(1, 1, 5, 9, 8, 8), (2, 3, 33, 47, 64, 64), (2, 1, 17, 65, 16, 24)]:
            T.test_attention_matches_torch_sdpa(*args)
        T.test_attention_matches_torch_sdpa(1, 2, 16, 16, 16, 16)
        T.test_causal_mask_aligns_the_last_query_with_the_last_key()
        T.test_fully_masked_rows_and_no_keys_give_zeros()
        T.test_uniform_scores_give_the_mean_of_the_visible_values()
        T.test_one_dominant_score_closed_form()
        T.test_common_key_component_and_key_permutation_leave_o_unchanged()
        T.test_strides_describe_the_tensors()
        for args in [(3, 5, 4, 2, False), (5, 3, 4, 3, True)]:
            T.test_attention_pure_python_brute_force(*args)
        T.test_error_scales()
    except (AssertionError, ValueError, OverflowError, RuntimeError):
        return False
    finally:
        monkeypatch.undo()
    return True


def _build_attention_variant(tmp_path, name, attn_src):
    c = tmp_path / f"{name}_attention.c"
    so = tmp_path / f"{name}.so"
    c.write_text(attn_src)
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
                    "-shared", "-fPIC", "-pthread", oracle_build.SRC, str(c), "-o", str(so), "-lm"],
                   check=True)
    return oracle.load_library(str(so))


def test_unmodified_attention_oracle_passes(tmp_path, monkeypatch):
    src = open(oracle_build.SRC_ATTENTION).read()
    assert _attn_pins_pass(_build_attention_variant(tmp_path, "clean", src), monkeypatch)


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attention_mutant_is_caught(tmp_path, monkeypatch, name):
    old, new = ATTN_MUTANTS[name]
    src = open(oracle_build.SRC_ATTENTION).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    lib = _build_attention_variant(tmp_path, name, src.replace(old, new))
    assert not _attn_pins_pass(lib, monkeypatch), f"pins did not catch {name}"


# ------------------------------------------------------------ residual + LayerNorm oracle

LN_MUTANTS = {
    "unbiased_variance": ("const double var = n > 0 ? sq / (double)n : 0.0;",
                          "const double var = n > 1 ? sq / (double)(n - 1) : 0.0;"),
    "eps_outside_sqrt": ("const double s = sqrt(var + eps);", "const double s = sqrt(var) + eps;"),
    "gamma_beta_swapped": ("y[j] = (z[j] - mu) / s * (double)gamma[j] + (double)beta_ln[j];",
                           "y[j] = (z[j] - mu) / s * (double)beta_ln[j] + (double)gamma[j];"),
    "mean_of_magnitudes": ("        sum += z[j];\n", "        sum += fabs(z[j]);\n"),
    "residual_dropped": ("A, B, C, alpha, beta, bias, 0, rows,", "A, B, C, alpha, 0.0, bias, 0, rows,"),
    "bias_dropped": ("alpha, beta, bias, 0, rows,", "alpha, beta, NULL, 0, rows,"),
    "bound_without_deviation_term": ("(2.0 * Di + fabs(zr[j] - st[0]) * Di / s) / s", "(2.0 * Di) / s"),
    "shift_not_subtracted": ("sq += (z[j] - mu) * (z[j] - mu);", "sq += z[j] * z[j];"),
}


def _ln_pins_pass(lib, monkeypatch) -> bool:
    import test_oracle_layernorm as T
    monkeypatch.setattr(oracle, "_lib", lib)
    try:
        for args in [(5, 64, 32, 0.0), (17, 333, 70, 1.0), (3, 1, 9, 0.5)]:
            T.test_layernorm_matches_torch_on_the_gemm_oracle(*args)
        T.test_constant_row_gives_beta_ln()
        T.test_two_point_row_closed_form()
        T.test_row_constant_residual_and_positive_alpha_change_nothing()
        for args in [(3, 7, 5), (4, 16, 9)]:
            T.test_layer_pure_python_brute_force(*args)
        T.test_bound_term_definition()
    except (AssertionError, ValueError, OverflowError, RuntimeError):
        return False
    finally:
        monkeypatch.undo()
    return True


def _build_layernorm_variant(tmp_path, name, ln_src):
    c = tmp_path / f"{name}_layernorm.c"
    so = tmp_path / f"{name}.so"
    c.write_text(ln_src)
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
                    "-shared", "-fPIC", "-pthread", oracle_build.SRC, str(c), "-o", str(so), "-lm"],
                   check=True)
    return oracle.load_library(str(so))


def test_unmodified_layernorm_oracle_passes(tmp_path, monkeypatch):
    src = open(oracle_build.SRC_LAYERNORM).read()
    assert _ln_pins_pass(_build_layernorm_variant(tmp_path, "clean", src), monkeypatch)


@pytest.mark.parametrize("name", sorted(LN_MUTANTS))
def test_layernorm_mutant_is_caught(tmp_path, monkeypatch, name):
    old, new = LN_MUTANTS[name]
    src = open(oracle_build.SRC_LAYERNORM).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    lib = _build_layernorm_variant(tmp_path, name, src.replace(old, new))
    assert not _ln_pins_pass(lib, monkeypatch), f"pins did not catch {name}"


# ------------------------------------------------------------ convolution oracle

CONV_MUTANTS = {
    "padding_not_subtracted": ("const int64_t ih = p * j->sh - j->ph + r * j->dh;",
                               "const int64_t ih = p * j->sh + r * j->dh;"),
    "dilation_ignored": ("const int64_t iw = q * j->sw - j->pw + ss * j->dw;",
                         "const int64_t iw = q * j->sw - j->pw + ss;"),
    "stride_ignored": ("const int64_t ih = p * j->sh - j->ph + r * j->dh;",
                       "const int64_t ih = p - j->ph + r * j->dh;"),
    "filter_flipped": ("const uint16_t *wp = j->w + ((k * j->R + r) * j->S + ss) * j->C;",
                       "const uint16_t *wp = j->w + ((k * j->R + (j->R - 1 - r)) * j->S + (j->S - 1 - ss)) * j->C;"),
    "output_size_without_dilation": ("const int64_t span = dil * (k - 1) + 1;",
                                     "const int64_t span = k;"),
    "border_taps_kept": ("                if (ih < 0 || ih >= j->H)\n                    continue;\n", ""),
    "scale_without_abs": ("a += fabs(prod);", "a += prod;"),
    "beta_term_dropped": ("double v = j->alpha * s + j->beta * yo;", "double v = j->alpha * s;"),
}


def _conv_pins_pass(lib, monkeypatch) -> bool:
    import test_oracle_conv as T
    monkeypatch.setattr(oracle, "_lib", lib)
    try:
        for args in [(1, 5, 5, 3, 2, 3, 3, (1, 1), (0, 0), (1, 1)),
                     (2, 9, 7, 8, 5, 3, 3, (2, 1), (1, 1), (1, 1)),
                     (1, 12, 10, 16, 4, 3, 2, (1, 2), (2, 0), (2, 3))]:
            T.test_conv_matches_torch(*args)
        T.test_one_by_one_filter_is_the_gemm()
        T.test_identity_filter_returns_the_input()
        T.test_all_ones_count_the_taps_inside_the_image()
        T.test_output_size()
        T.test_epilogue_composition()
        T.test_conv_pure_python_brute_force((1, 5, 4, 2, 2, 3, 2, (2, 1), (1, 1), (1, 2)))
        T.test_scale_equals_value_for_nonnegative_inputs()
    except (AssertionError, ValueError, OverflowError, RuntimeError, IndexError):
        return False
    finally:
        monkeypatch.undo()
    return True


def _build_conv_variant(tmp_path, name, conv_src):
    c = tmp_path / f"{name}_conv.c"
    so = tmp_path / f"{name}.so"
    c.write_text(conv_src)
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
                    "-shared", "-fPIC", "-pthread", oracle_build.SRC, str(c), "-o", str(so), "-lm"],
                   check=True)
    return oracle.load_library(str(so))


def test_unmodified_conv_oracle_passes(tmp_path, monkeypatch):
    src = open(oracle_build.SRC_CONV).read()
    assert _conv_pins_pass(_build_conv_variant(tmp_path, "clean", src), monkeypatch)


@pytest.mark.parametrize("name", sorted(CONV_MUTANTS))
def test_conv_mutant_is_caught(tmp_path, monkeypatch, name):
    old, new = CONV_MUTANTS[name]
    src = open(oracle_build.SRC_CONV).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    lib = _build_conv_variant(tmp_path, name, src.replace(old, new))
    assert not _conv_pins_pass(lib, monkeypatch), f"pins did not catch {name}"
