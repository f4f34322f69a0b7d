"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source, builds it
with gcc into a temporary library, and runs the oracle pin tests against it
in a subprocess; the pins must fail.  The committed oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ngram_oracle.c")

MUTATIONS = {
    "no_gamma": ("uint64_t z = x + ORACLE_GAMMA;", "uint64_t z = x;"),
    "wrong_shift": ("(z ^ (z >> 27))", "(z ^ (z >> 28))"),
    "wrong_multiplier": ("0x94D049BB133111EBull", "0x94D049BB133111EDull"),
    "bigram_trigram_swapped": ("k < 8 ? bigram : trigram", "k < 8 ? trigram : bigram"),
    "field_width_20": ("uint64_t bigram = (c1 << 21) | c0;", "uint64_t bigram = (c1 << 20) | c0;"),
    "trigram_drops_c2": ("uint64_t trigram = (c2 << 42) | (c1 << 21) | c0;",
                         "uint64_t trigram = (c1 << 21) | c0;"),
    "context_off_by_one": ("ctx[3 * i + 2] = ext[p];", "ctx[3 * i + 2] = ext[p + 1];"),
    "history_swapped": ("ext[0] = history ? history[2 * s] : ORACLE_PAD;",
                        "ext[0] = history ? history[2 * s + 1] : ORACLE_PAD;"),
    "seed_index": ("uint64_t h = oracle_splitmix64(key ^ seeds[k]);",
                   "uint64_t h = oracle_splitmix64(key ^ seeds[k & 7]);"),
    "mod_low_word": ("(int32_t)(h % (uint64_t)R)", "(int32_t)((uint32_t)h % (uint64_t)R)"),
    "sum_reversed": ("acc = acc + oracle_bf16_to_f32(T[r * d + j]);",
                     "acc = oracle_bf16_to_f32(T[(int64_t)rows[i * ORACLE_K + 15 - k] * d + j]) + acc;"),
    "sum_skips_last_row": ("acc = acc + oracle_bf16_to_f32(T[r * d + j]);",
                           "if (k < 15) acc = acc + oracle_bf16_to_f32(T[r * d + j]);"),
    "int8_unfused": ("acc = fmaf((float)Q[r * d + j], scale[r], acc);",
                     "acc = (float)Q[r * d + j] * scale[r] + acc;"),
    "int8_wrong_scale_row": ("acc = fmaf((float)Q[r * d + j], scale[r], acc);",
                             "acc = fmaf((float)Q[r * d + j], scale[k], acc);"),
    "gate_unfused": ("float h = fmaf(W_g[j], eN[i * d + j], base);",
                     "float h = W_g[j] * eN[i * d + j] + base;"),
    "gate_drops_residual": ("float y = residual ? oracle_bf16_to_f32(residual[i * d + j]) + h : h;",
                            "float y = h;"),
    "gate_wrong_e1_row": ("e1[(int64_t)e1_rows[i] * d + j]", "e1[(int64_t)i * d + j]"),
    "round_half_up": ("return (uint16_t)((u + 0x7FFFu + lsb) >> 16);",
                      "return (uint16_t)((u + 0x8000u) >> 16);"),
    "round_truncate": ("return (uint16_t)((u + 0x7FFFu + lsb) >> 16);",
                       "return (uint16_t)(u >> 16);"),
    "grad_table_token_index": ("const int64_t i = t / ORACLE_K;", "const int64_t i = t % ORACLE_K;"),
    "grad_table_no_weight": ("acc[j] = fmaf(W_g[j], oracle_bf16_to_f32(g[i * d + j]), acc[j]);",
                             "acc[j] = acc[j] + oracle_bf16_to_f32(g[i * d + j]);"),
    "grad_table_unfused": ("acc[j] = fmaf(W_g[j], oracle_bf16_to_f32(g[i * d + j]), acc[j]);",
                           "acc[j] = W_g[j] * oracle_bf16_to_f32(g[i * d + j]) + acc[j];"),
    "grad_e1_keeps_invalid": ("if (tokens[i] != query[q] || rows[i * ORACLE_K] < 0)",
                              "if (tokens[i] != query[q])"),
    "grad_gate_float_accumulator": ("acc = acc + (double)oracle_bf16_to_f32(g[i * d + j]) * (double)eN[i * d + j];",
                                    "acc = (float)(acc + (double)oracle_bf16_to_f32(g[i * d + j]) * (double)eN[i * d + j]);"),
    "grad_gate_skips_first_token": ("for (int64_t i = 0; i < n; ++i) {\n            if (rows[i * ORACLE_K] < 0)",
                                    "for (int64_t i = 1; i < n; ++i) {\n            if (rows[i * ORACLE_K] < 0)"),
    "grad_gate_wrong_operand": ("* (double)eN[i * d + j];", "* (double)eN[i * d + (j + 1) % d];"),
    "mxfp4_nibbles_swapped": ("int code = (j % 2 == 0) ? (byte & 15) : (byte >> 4);",
                              "int code = (j % 2 == 0) ? (byte >> 4) : (byte & 15);"),
    "mxfp4_scale_group_16": ("int E = row[d / 2 + j / 32];", "int E = row[d / 2 + j / 16];"),
    "mxfp4_scale_bias_128": ("return ldexpf(oracle_e2m1(code), E - 127);", "return ldexpf(oracle_e2m1(code), E - 128);"),
    "e2m1_exponent_bias_0": ("ldexpf(1.0f + 0.5f * (float)m, e - 1);", "ldexpf(1.0f + 0.5f * (float)m, e);"),
    "mxfp4_nan_scale_ignored": ("    if (E == 255)\n        return NAN;\n", ""),
    "grad_gate_keeps_invalid": ("if (rows[i * ORACLE_K] < 0)\n                continue;\n            acc = acc +",
                                "acc = acc +"),
    "norm_drops_eps": ("sqrt(S / (double)d + (double)eps)", "sqrt(S / (double)d)"),
    "norm_mean_over_d_minus_1": ("sqrt(S / (double)d + (double)eps)", "sqrt(S / (double)(d - 1) + (double)eps)"),
    "norm_no_gamma": ("nv[j] = (double)x[j] * r * (double)gamma[j];", "nv[j] = (double)x[j] * r;"),
    "norm_sum_in_float": ("S = S + (double)x[j] * (double)x[j];", "S = (float)(S + (double)x[j] * (double)x[j]);"),
    "norm_skips_last_square": ("for (int32_t j = 0; j < d; ++j)\n            S = S +",
                               "for (int32_t j = 0; j + 1 < d; ++j)\n            S = S +"),
    "gate_sign_flipped": ("const double alpha = 1.0 / (1.0 + exp(-logit));",
                          "const double alpha = 1.0 / (1.0 + exp(logit));"),
    "gate_uv_swapped": ("Z = Z + ((double)u[j] * (double)oracle_bf16_to_f32(e1_token[j]) + (double)v[j] * nv[j]);",
                        "Z = Z + ((double)v[j] * (double)oracle_bf16_to_f32(e1_token[j]) + (double)u[j] * nv[j]);"),
    "gate_z_in_float": ("Z = Z + ((double)u[j] * (double)oracle_bf16_to_f32(e1_token[j]) + (double)v[j] * nv[j]);",
                        "Z = (float)(Z + ((double)u[j] * (double)oracle_bf16_to_f32(e1_token[j]) + (double)v[j] * nv[j]));"),
    "gate_no_bias": ("const double logit = Z + (double)b;", "const double logit = Z;"),
    "gate_alpha_not_applied": ("alpha * (double)W_g[j] * nv[j]", "(double)W_g[j] * nv[j]"),
    "gate_uses_raw_sum": ("alpha * (double)W_g[j] * nv[j]", "alpha * (double)W_g[j] * (double)x[j]"),
    "norm_gate_wrong_e1_row": ("const uint16_t* e1_token = e1 + (int64_t)e1_rows[i] * d;",
                               "const uint16_t* e1_token = e1 + (int64_t)(e1_rows[i] + 1) * d;"),
    "norm_gate_drops_residual": ("const uint16_t* res_token = residual ? residual + i * d : NULL;",
                                 "const uint16_t* res_token = NULL;"),
    "norm_gate_rounds_through_fp32": ("out[i * d + j] = oracle_bf16_rne_f64(y);",
                                      "out[i * d + j] = oracle_bf16_rne((float)y);"),
    "bf16f64_ties_away": ("(a > mid || (a == mid && odd))", "(a >= mid)"),
    "bf16f64_truncates": ("const double r = (a > mid || (a == mid && odd)) ? hi : lo;", "const double r = lo;"),
    "bf16f64_spacing_off_by_one": ("int qe = e - 8;", "int qe = e - 9;"),
    "project_no_bf16_round": ("xb[j] = (double)oracle_bf16_to_f32(oracle_bf16_rne(x[i * d_in + j]));",
                              "xb[j] = (double)x[i * d_in + j];"),
    "project_transposed": ("oracle_bf16_to_f32(P[(int64_t)o * d_in + j])", "oracle_bf16_to_f32(P[(int64_t)j * d_out + o])"),
    "project_skips_last_term": ("for (int32_t j = 0; j < d_in; ++j) {\n                const double t",
                                "for (int32_t j = 0; j + 1 < d_in; ++j) {\n                const double t"),
    "project_float_accumulator": ("acc = acc + t;", "acc = (float)(acc + t);"),
    "project_abs_signed": ("a = a + fabs(t);", "a = a + t;"),
    "project_wrong_x_row": ("oracle_bf16_rne(x[i * d_in + j])", "oracle_bf16_rne(x[((i + 1) % n) * d_in + j])"),
}


ALL_PINS = ["tests/test_oracle_hash.py", "tests/test_oracle_sum_gate.py", "tests/test_oracle_grad.py",
            "tests/test_oracle_mxfp4.py", "tests/test_oracle_norm_gate.py", "tests/test_oracle_project.py"]


def pins_for(name):
    """The pin file of the function a mutation hits (so each run imports only
    what it needs); the whole set for anything else."""
    for prefix, f in (("grad_", "test_oracle_grad.py"), ("mxfp4_", "test_oracle_mxfp4.py"),
                      ("project_", "test_oracle_project.py"),
                      ("e2m1_", "test_oracle_mxfp4.py"), ("norm_", "test_oracle_norm_gate.py"),
                      ("bf16f64_", "test_oracle_norm_gate.py"), ("gate_z_", "test_oracle_norm_gate.py"),
                      ("gate_sign", "test_oracle_norm_gate.py"), ("gate_uv", "test_oracle_norm_gate.py"),
                      ("gate_no_bias", "test_oracle_norm_gate.py"), ("gate_alpha", "test_oracle_norm_gate.py"),
                      ("gate_uses_raw", "test_oracle_norm_gate.py"), ("sum_", "test_oracle_sum_gate.py"),
                      ("int8_", "test_oracle_sum_gate.py"), ("gate_", "test_oracle_sum_gate.py"),
                      ("round_", "test_oracle_sum_gate.py")):
        if name.startswith(prefix):
            return ["tests/" + f]
    if name in ("no_gamma", "wrong_shift", "wrong_multiplier", "bigram_trigram_swapped", "field_width_20",
                "trigram_drops_c2", "context_off_by_one", "history_swapped", "seed_index", "mod_low_word"):
        return ["tests/test_oracle_hash.py"]
    return ALL_PINS


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src.replace(before, after))
    mlib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", str(mlib), str(msrc), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(mlib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + pins_for(name),
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutation {name}:\n{r.stdout[-2000:]}"
