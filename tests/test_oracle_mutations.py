"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the
pins in test_oracle_pins.py catch every one of them.

Each mutation is a one-line edit of bitnet_oracle.c of the kind a reader might make
by accident: a wrong rounding mode, constant, index, sign, dropped term, reversed bit
order or transposed operand.  The mutated file is compiled to a temporary library and
the whole pin module is run against it in a subprocess; the run must fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bitnet_oracle.c")

MUTATIONS = {
    "act_round_half_away": ("float r = nearbyintf(p);", "float r = roundf(p);"),
    "act_scale_constant": ("float a = 127.0f / amax;", "float a = 128.0f / amax;"),
    "act_no_eps": ("if (amax < 1e-5f) amax = 1e-5f;", ""),
    "act_skip_last_element": ("float v = fabsf(bf16_to_f32(x[m * K + k]));",
                              "float v = (k + 1 < K) ? fabsf(bf16_to_f32(x[m * K + k])) : 0.0f;"),
    "act_truncate": ("float r = nearbyintf(p);", "float r = truncf(p);"),
    "weight_mean_wrong_count": ("float s = (float)(sum / (double)K);",
                                "float s = (float)(sum / (double)(K + 1));"),
    "weight_no_abs": ("sum += fabs((double)W[n * K + k]);", "sum += ((double)W[n * K + k]);"),
    "weight_no_clamp": ("if (r > 1.0f) r = 1.0f;", ""),
    "weight_eps_too_big": ("if (s < 1e-5f) s = 1e-5f;", "if (s < 1e-3f) s = 1e-3f;"),
    "pack_reversed_bits": ("byte |= code << (2 * i);", "byte |= code << (2 * (3 - i));"),
    "decode_wrong_field": ("unsigned code = (packed[n * KB + k / 4] >> (2 * (k % 4))) & 3u;\n    return",
                           "unsigned code = (packed[n * KB + k / 4] >> (2 * ((k + 1) % 4))) & 3u;\n    return"),
    "accumulate_transposed_k": ("sum += (int64_t)xq[m * K + k] * weight_at(packed, KB, n, k);\n            if (sum > INT32_MAX",
                                "sum += (int64_t)xq[m * K + k] * weight_at(packed, KB, n, K - 1 - k);\n            if (sum > INT32_MAX"),
    "rescale_multiplies_by_a": ("double r = (double)acc * (double)s / (double)a;",
                                "double r = (double)acc * (double)s * (double)a;"),
    "rescale_drops_weight_scale": ("double r = (double)acc * (double)s / (double)a;",
                                   "double r = (double)acc / (double)a;"),
    "bf16_floor": ("double r = nearbyint(x / quantum) * quantum;",
                   "double r = floor(x / quantum) * quantum;"),
    "bf16_double_rounding": ("double r = nearbyint(x / quantum) * quantum;",
                             "double r = nearbyint((double)(float)x / quantum) * quantum;"),
    "per_tensor_scale_constant": ("const float a_t = 127.0f / amax_t;",
                                  "const float a_t = 128.0f / amax_t;"),
    "per_tensor_uses_first_row": ("for (int64_t i = 0; i < M * K; ++i) {\n        float v = fabsf",
                                  "for (int64_t i = 0; i < K; ++i) {\n        float v = fabsf"),
    "repack_sign_table_minus_one": ("return w == 1 ? 3u : (w == -1 ? 1u : 0u);",
                                    "return w == 1 ? 3u : (w == -1 ? 2u : 0u);"),
    "repack_field_order": ("byte |= table_code(to, w) << (2 * i);",
                           "byte |= table_code(to, w) << (2 * (3 - i));"),
    "a16_drops_weight_scale": ("ref[m * N + n] = s * (double)w_scale[n];",
                               "ref[m * N + n] = s;"),
    "a16_weight_index": ("const double t = (double)bf16_to_f32(x[m * K + k]) * weight_at(packed, KB, n, k);",
                         "const double t = (double)bf16_to_f32(x[m * K + k]) * weight_at(packed, KB, n, K - 1 - k);"),
    "swiglu_sign_of_exp": ("h[t] = g[t] / (1.0 + exp(-g[t])) * u[t];",
                           "h[t] = g[t] / (1.0 + exp(g[t])) * u[t];"),
    "swiglu_sigmoid_only": ("h[t] = g[t] / (1.0 + exp(-g[t])) * u[t];",
                            "h[t] = 1.0 / (1.0 + exp(-g[t])) * u[t];"),
    "b3_round_down": ("out[n * RB + j] = (uint8_t)((256 * v + 242) / 243);",
                      "out[n * RB + j] = (uint8_t)((256 * v) / 243);"),
    "b3_pack_code_table": ("v = 3 * v + (w + 1);", "v = 3 * v + (w + 2) % 3;"),
    "b3_unpack_scale": ("const int v = (b3[n * RB + j] * 243) / 256;",
                        "const int v = (b3[n * RB + j] * 242) / 256;"),
    "b3_accumulate_digit_order": ("for (int t = (int)(k % 5); t < 4; ++t) p *= 3;",
                                  "for (int t = 0; t < (int)(k % 5); ++t) p *= 3;"),
    "b3_row_padding": ("return (K + B3_CHUNK - 1) / B3_CHUNK * 64;", "return (K + 4) / 5;"),
    "swiglu_swapped_operands": ("h[t] = g[t] / (1.0 + exp(-g[t])) * u[t];",
                                "h[t] = u[t] / (1.0 + exp(-u[t])) * g[t];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/absent"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                           "-shared", "-o", str(lib), str(mutated), "-lm"])
    env = dict(os.environ, BITNET_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"pins did not catch mutation {name}:\n{res.stdout[-2000:]}"
