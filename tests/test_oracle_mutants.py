"""Planted mistakes: each plausible slip in the oracle must make its pin tests fail.

Each case copies oracle/ob_oracle.c to a temporary folder, applies one textual change (a dropped
term, a wrong sign or index, a transposed operand, a wrong constant), builds it with the oracle's own
flags and runs tests/test_oracle.py against that copy in a subprocess.  The real oracle is never
modified.  CPU only.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ob_oracle.c")

MUTANTS = {
    "sign_of_zero": ("return x >= 0.0f ? 1 : 0;", "return x > 0.0f ? 1 : 0;"),
    "bit_order": ("words[i / 32] |= (uint32_t)1u << (i % 32);",
                  "words[i / 32] |= (uint32_t)1u << (31 - i % 32);"),
    "dense_drops_eps": ("(mh / (sqrt(vh) + (double)eps))", "(mh / (sqrt(vh)))"),
    "scale_count": ("return (float)sqrt(s / (double)(end - begin));",
                    "return (float)sqrt(s / (double)(end - begin + 1));"),
    "scale_no_sqrt": ("return (float)sqrt(s / (double)(end - begin));",
                      "return (float)(s / (double)(end - begin));"),
    "error_sign": ("float delta = (float)((double)x[i] - (double)gh);",
                   "float delta = (float)((double)gh - (double)x[i]);", 2),
    "momentum_uses_x": ("m[i] = (float)(b1 * (double)m[i] + (1.0 - b1) * (double)gh);",
                        "m[i] = (float)(b1 * (double)m[i] + (1.0 - b1) * (double)x[i]);"),
    "momentum_coeffs_swapped": ("m[i] = (float)(b1 * (double)m[i] + (1.0 - b1) * (double)gh);",
                                "m[i] = (float)((1.0 - b1) * (double)m[i] + b1 * (double)gh);"),
    "update_sign": ("p[i] = (float)((double)p[i] -\n                               (double)lr",
                    "p[i] = (float)((double)p[i] +\n                               (double)lr"),
    "update_drops_eps": ("(sqrt((double)v[i]) + (double)eps)));\n            if (signs",
                         "(sqrt((double)v[i]))));\n            if (signs"),
    "update_no_sqrt": ("((double)m[i] / (sqrt((double)v[i]) + (double)eps)",
                       "((double)m[i] / ((double)v[i] + (double)eps)", 2),
    "ema_coeffs_swapped": ("e_new = (float)(eb * (double)err[i] + (1.0 - eb) * (double)delta);",
                           "e_new = (float)((1.0 - eb) * (double)err[i] + eb * (double)delta);"),
    "ema_unscaled_sign": ("float delta = (float)((double)x[i] - (double)gh);",
                          "float delta = (float)((double)x[i] - (b ? 1.0 : -1.0));", 2),
    "clip_lower_bound": ("gi = -c;", "gi = c;", 2),
    "gh_wrong_chunk": ("float gh = b ? scales[c] : -scales[c];",
                       "float gh = b ? scales[0] : -scales[0];", 2),
    "nonfinite_nan_only": ("!isfinite(stored)", "isnan(stored)", 2),
    "nonfinite_counts_unrounded": ("!isfinite(stored)", "!isfinite(err[i])", 2),
    "format_ties_away": ("nearbyint(a / q)", "round(a / q)"),
    "format_truncates": ("nearbyint(a / q)", "trunc(a / q)"),
    "overflow_saturates": ("if (r > maxf) r = INFINITY;", "if (r > maxf) r = maxf;"),
    "f16_emin": ("round_to_format(e, 11, -14, F16_MAXF)", "round_to_format(e, 11, -15, F16_MAXF)"),
    "f16_precision": ("round_to_format(e, 11, -14, F16_MAXF)", "round_to_format(e, 10, -14, F16_MAXF)"),
    "bf16_precision": ("round_to_format(e, 8, -126, BF16_MAXF)", "round_to_format(e, 9, -126, BF16_MAXF)"),
    "f16_decode_bias": ("v = ldexp((double)(mant + 1024), ex - 25);", "v = ldexp((double)(mant + 1024), ex - 24);"),
    "f16_subnormal_decode": ("v = ldexp((double)mant, -24);", "v = ldexp((double)mant, -25);"),
    "error_not_widened": ("for (int64_t i = 0; i < n; ++i) err[i] = load_err(err_store, err_fmt, i);",
                          "for (int64_t i = 0; i < n; ++i) err[i] = 0.0f;", 2),
    "error_stored_unrounded_bf16": ("uint16_t b = bf16_bits_of(round_to_format(e, 8, -126, BF16_MAXF));",
                                    "uint16_t b = bf16_bits_of((double)(float)((double)e));"),
    "int8_zero_for_plus": ("signs[i] = (int8_t)(b ? 1 : -1);", "signs[i] = (int8_t)(b ? 0 : -1);", 2),
    "dense_v_not_squared": ("(1.0 - b2) * (gi * gi)", "(1.0 - b2) * gi"),
    "dense_v_uses_beta1": ("v[i] = (float)(b2 * (double)v[i]", "v[i] = (float)(b1 * (double)v[i]"),
    "dense_bias_corr_power": ("bc2 = 1.0 - pow(b2, (double)step);", "bc2 = 1.0 - pow(b1, (double)step);"),
    "dense_old_m_in_update": ("double mh = (double)m[i] / bc1;", "double mh = (double)m[i] / bc1 / b1;"),
    "server_bit_polarity": ("a += word_bit(worker_words + (int64_t)w * nw, i) ? s : -s;",
                            "a += word_bit(worker_words + (int64_t)w * nw, i) ? -s : s;", 2),
    "server_row_stride": ("a += word_bit(worker_words + (int64_t)w * nw, i) ? s : -s;",
                          "a += word_bit(worker_words + (int64_t)w * K, i) ? s : -s;", 2),
    "server_scale_row_stride": ("double s = (double)worker_scales[(int64_t)w * K + c];",
                                "double s = (double)worker_scales[(int64_t)c * W + w];", 2),
    "server_divisor": ("float avg = (float)(a / (double)W);", "float avg = (float)(a / (double)(W + 1));"),
    "server_error_uses_avg": ("server_err[i] = (float)((double)x[i] - (double)gh);",
                              "server_err[i] = (float)((double)x[i] - (double)gh + (double)server_err[i]);"),
    "lamb_ratio_inverted": ("(float)(sqrt(sw) / sqrt(su))", "(float)(sqrt(su) / sqrt(sw))"),
    "lamb_ratio_squared": ("(float)(sqrt(sw) / sqrt(su))", "(float)(sw / su)"),
    "lamb_degenerate_zero": ("(sw == 0.0 || su == 0.0) ? 1.0f :", "(sw == 0.0 || su == 0.0) ? 0.0f :"),
    "lamb_u_drops_eps": ("(sqrt((double)v[i] / bc2) + (double)eps)", "(sqrt((double)v[i] / bc2))", 2),
    "lamb_update_without_ratio": ("(double)lr * ((double)r * u)", "(double)lr * u"),
    "lamb_dense_no_bias_correction": ("lamb_update(K, off, m, v, p, ratios, lr, eps, bc1, bc2);",
                                      "lamb_update(K, off, m, v, p, ratios, lr, eps, 1.0, 1.0);"),
    "lamb_weight_norm_of_m": ("sw += (double)p[i] * (double)p[i];", "sw += (double)m[i] * (double)m[i];"),
    "lamb_compress_also_adam": ("nonfinite, lr, beta1, eps, clip, ef_mode, ef_beta, 0, 0, 0, 0, 0);",
                                "nonfinite, lr, beta1, eps, clip, ef_mode, ef_beta, 1, 0, 0, 0, 0);"),
    "lamb_dense_also_adam": ("bias_correction, step, 0);", "bias_correction, step, 1);"),
    "diag_norm_not_squared": ("            s += e * e;", "            s += fabs(e);"),
    "diag_counts_minus": ("plus += word_bit(words, i);", "plus += 1 - word_bit(words, i);"),
    "sr_counter_shift": ("uint64_t blk = (uint64_t)i >> 2;", "uint64_t blk = (uint64_t)i >> 4;"),
    "sr_decision_inverted": ("(double)r * q < (a - lo) * 65536.0", "(double)r * q > (a - lo) * 65536.0"),
    "sr_overflow_saturates": ("    if (v > maxf) v = INFINITY;\n    return copysign(v, x);",
                              "    if (v > maxf) v = maxf;\n    return copysign(v, x);"),
    "sr_falls_back_to_nearest": ("float stored = stochastic ? store_err_sr(", "float stored = 0 ? store_err_sr(", 2),
    "sr_ignores_index0": ("sr_bits(sr_seed, sr_step, sr_index0 + i))", "sr_bits(sr_seed, sr_step, i))", 2),
    "philox_no_key_bump": ("            k0 += W0;\n            k1 += W1;", "            k0 += 0;\n            k1 += W1;"),
    "philox_lanes_swapped": ("uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;",
                             "uint32_t n0 = hi0 ^ c1 ^ k0, n1 = lo0, n2 = hi1 ^ c3 ^ k1, n3 = lo1;"),
    "sr_wrong_word": ("return out[i & 3] >> 16;", "return out[(i >> 1) & 3] >> 16;"),
    "sr_low_half": ("return out[i & 3] >> 16;", "return out[i & 3] & 0xFFFFu;"),
    "sr_step_dropped": ("(uint32_t)step, (uint32_t)(step >> 32)};", "0, 0};"),
    "sr_seed_high_dropped": ("uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)}, out[4];",
                             "uint32_t key[2] = {(uint32_t)seed, 0}, out[4];"),
    # R19: the worker's split step
    "worker_update_polarity": ("float ghat = word_bit(words, i) ? scales[c] : -scales[c];",
                               "float ghat = word_bit(words, i) ? -scales[c] : scales[c];"),
    "worker_update_momentum_coeff": ("(1.0 - b1) * (double)ghat);", "(double)ghat);"),
    "worker_update_skips_p": ("            p[i] = (float)((double)p[i] - (double)lr * ((double)m[i] / (sqrt((double)v[i]) + (double)eps)));\n        }\n    }\n    return OR_OK;",
                              "        }\n    }\n    return OR_OK;"),
    "worker_compress_global_error": ("err[i] = ef_mode == 1 ? (float)(eb * (double)err[i] + (1.0 - eb) * (double)delta) : delta;",
                                     "err[i] = ef_mode == 1 ? (float)(eb * (double)err[i] + (1.0 - eb) * (double)delta) : x[i];"),
    "lamb_worker_polarity": ("float gl = word_bit(words, i) ? scales[c] : -scales[c];",
                             "float gl = word_bit(words, i) ? -scales[c] : scales[c];"),
    "lamb_worker_momentum_coeff": ("(1.0 - b1) * (double)gl);", "(double)gl);"),
    "unpack_polarity": ("out[i] = word_bit(words, i) ? scales[c] : -scales[c];",
                        "out[i] = word_bit(words, i) ? -scales[c] : scales[c];"),
}


def _run_mutant(name, workdir):
    """Build the oracle with the planted mistake and run the pin suite against it; returns the
    pytest subprocess's exit code and the end of its output."""
    old, new, *count = MUTANTS[name]
    count = count[0] if count else 1
    src = open(SRC).read()
    if src.count(old) != count:
        return None, f"mutation anchor for {name} does not match {count} time(s)"
    csrc = os.path.join(workdir, f"{name}.c")
    lib = os.path.join(workdir, f"lib_{name}.so")
    with open(csrc, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", lib, csrc, "-lm"], check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    env = dict(os.environ, OB_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def mutant_runs():
    """Every mutant's run, started on first use and run several at a time (each is an independent
    subprocess); a test waits only for its own mutant."""
    with tempfile.TemporaryDirectory(prefix="ob_mutants_") as d, \
            cf.ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as pool:
        futs = {name: pool.submit(_run_mutant, name, d) for name in sorted(MUTANTS)}
        yield futs
        for f in futs.values():
            f.cancel()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, mutant_runs):
    rc, out = mutant_runs[name].result()
    assert rc is not None, out
    assert rc != 0, f"planted mistake '{name}' passed every pin:\n{out}"
