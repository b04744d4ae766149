"""The pins must catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake in a copy of the oracle's C source, builds it
into a temporary library, and runs the pin suite against it in a fresh
process: the suite must fail.  The product code is never involved.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sprms_oracle.c")

MUTATIONS = {
    "drop_deepstack": ("if (deepstack) x += load(deepstack", "if (0) x += load(deepstack"),
    "drop_last_partial": ("for (int64_t q = 0; q < tp; ++q)\n        x += p->partial_scale",
                          "for (int64_t q = 0; q < tp - 1; ++q)\n        x += p->partial_scale"),
    "partial_scale_ignored": ("x += p->partial_scale * load(", "x += load("),
    "eps_outside_sqrt": ("1.0 / sqrt(ss / (double)H + (double)eps)",
                         "1.0 / (sqrt(ss / (double)H) + (double)eps)"),
    "mean_over_h_minus_1": ("sqrt(ss / (double)H + ", "sqrt(ss / (double)(H - 1) + "),
    "bias_subtracted": ("if (bias) y[h] += load(bias", "if (bias) y[h] -= load(bias"),
    "residual_chunk_ignored": ("(p->residual_rows == tp * S && tp > 1) ? r * S : 0",
                               "(p->residual_rows == tp * S && tp > 1) ? 0 : 0"),
    "deepstack_chunk_off_by_one": ("p->deepstack_rows == tp * S && tp > 1) ? r * S : 0",
                                   "p->deepstack_rows == tp * S && tp > 1) ? r * S + 1 : 0"),
    "qmax_240": ("(float)(amax / 448.0)", "(float)(amax / 240.0)"),
    "e4m3_no_tie_to_even": ("for (int c = 0; c <= 0x7E; ++c) {\n    double err = fabs(orc_e4m3_to_double((uint8_t)c) - a);\n    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {",
                            "for (int c = 0; c <= 0x7E; ++c) {\n    double err = fabs(orc_e4m3_to_double((uint8_t)c) - a);\n    if (err < best_err) {"),
    "bf16_ties_away": ("r = rint(a / spacing) * spacing;", "r = floor(a / spacing + 0.5) * spacing;"),
    "pad_rows_off_by_one": ("if (s >= v) {", "if (s > v) {"),
    "residual_not_added": ("z[h] = x + load(residual, p->act_dtype, (roff + s) * H + h);",
                           "z[h] = x;"),
    "weight_ignored": ("y[h] = z[h] * rstd * load(weight, p->act_dtype, h);",
                       "y[h] = z[h] * rstd;"),
    "static_scale_multiplied": ("y[h] / (double)static_scale)", "y[h] * (double)static_scale)"),
    "mx_emax_e2m1_off_by_one": ("const int emax = p->out_dtype == ORC_E4M3 ? 8 : 2;",
                                "const int emax = p->out_dtype == ORC_E4M3 ? 8 : 3;"),
    "mx_exponent_not_floor": ("e = k - 1 - emax;", "e = k - emax;"),
    "mx_no_clamp_low": ("if (e < -127) e = -127;", "if (e < -150) e = -150;"),
    "e2m1_no_tie_to_even": ("if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {\n      best = c;\n      best_err = err;\n    }\n  }\n  return (uint8_t)(best | (signbit(x) ? 0x8 : 0x0));",
                            "if (err <= best_err) {\n      best = c;\n      best_err = err;\n    }\n  }\n  return (uint8_t)(best | (signbit(x) ? 0x8 : 0x0));"),
    "fc2_contiguous_segments": ("ids[j * otp + k] = j + k * odp;", "ids[j * otp + k] = j * otp + k;"),
    "fc2_senders_reversed": ("const char* from = (const char*)src[g * odp + i]",
                             "const char* from = (const char*)src[g * odp + (odp - 1 - i)]"),
    "dsacp_chunk_of_sender": ("memcpy((char*)out[q] + (size_t)p * chunk, send + (size_t)q * chunk, chunk);",
                              "memcpy((char*)out[q] + (size_t)p * chunk, send + (size_t)p * chunk, chunk);"),
    "dsacp_head_major_view": ("((size_t)s * (size_t)tp + (size_t)q) * (size_t)piece",
                              "((size_t)q * (size_t)S + (size_t)s) * (size_t)piece"),
    "mm_slot_of_destination": ("store(dst[r], out_dtype, ((int64_t)rank * S + s) * N + n, acc);",
                               "store(dst[r], out_dtype, ((int64_t)r * S + s) * N + n, acc);"),
    "mm_round_robin_tokens": ("const int64_t r = m / S;     /* destination rank of this token */\n"
                              "    const int64_t s = m - r * S; /* its row in that rank's shard */\n"
                              "    for (int64_t n = 0; n < N; ++n) {",
                              "const int64_t r = m % tp;\n    const int64_t s = m / tp;\n"
                              "    for (int64_t n = 0; n < N; ++n) {"),
    "fp8_round_robin_tokens": ("const int64_t r = m / S;     /* destination rank of this token */\n"
                               "    const int64_t s = m - r * S; /* its row in that rank's shard */\n"
                               "    const double sx",
                               "const int64_t r = m % tp;\n    const int64_t s = m / tp;\n"
                               "    const double sx"),
    "mm_weight_transposed": ("orc_bf16_to_double(w[n * K + k])", "orc_bf16_to_double(w[k * N + n])"),
    "fp8_x_scale_dropped": ("store(dst[r], out_dtype, ((int64_t)rank * S + s) * N + n, acc * sx * sw);",
                            "store(dst[r], out_dtype, ((int64_t)rank * S + s) * N + n, acc * sw);"),
    "fp8_w_scale_by_token": ("const double sw = (double)w_scale[w_scale_rows == 1 ? 0 : n];",
                             "const double sw = (double)w_scale[w_scale_rows == 1 ? 0 : m % N];"),
    "gather_rows_reversed": ("(const char*)shards[q] + (size_t)(s * row_bytes),",
                             "(const char*)shards[q] + (size_t)((S - 1 - s) * row_bytes),"),
    "row_max_skips_nan": ("if (isnan(y[h]) || fabs(y[h]) > amax) amax = fabs(y[h]);",
                          "if (fabs(y[h]) > amax) amax = fabs(y[h]);"),
    "nan_scale_gives_zero_codes": ("scale == 0.0f ? 0.0 : y[h] / (double)scale",
                                   "scale > 0.0f ? y[h] / (double)scale : 0.0"),
    "block_max_skips_nan": ("if (isnan(y[h]) || fabs(y[h]) > bmax) bmax = fabs(y[h]);",
                            "if (fabs(y[h]) > bmax) bmax = fabs(y[h]);"),
    "nan_saturates_to_448": ("if (isnan(x)) return 0x7F;", "if (isnan(x)) return 0x7E;"),
    "gather_scale_from_wrong_rank": ("(const char*)scales[q] + (size_t)(s * scale_row_bytes)",
                                     "(const char*)scales[0] + (size_t)(s * scale_row_bytes)"),
}


# mistakes in the entry point with the library's argument list, which
# tests/test_oracle_abi.py pins to the (unchanged) row-list function
ABI_MUTATIONS = {
    "abi_in_place_wrong_block": ("(a->residual_rows == tp * S && tp > 1) ? (int64_t)a->tp_rank * S : 0",
                                 "(a->residual_rows == tp * S && tp > 1) ? 0 : 0"),
    "abi_valid_rows_flag_ignored": ("const int64_t n = (a->flags & 1) ? v : S;", "const int64_t n = S;"),
    "abi_stride_ignored": ("if (partials && stride != S * H) {", "if (0) {"),
    "abi_static_scale_not_read": ("static_scale = ((const float*)out_scale)[0];", "static_scale = 1.0f;"),
    "abi_in_place_overlap_allowed": ("if (o == 0 && k == 4 && in_place) continue;",
                                     "if (o == 0 && in_place) continue;"),
    "abi_static_scale_not_an_input": ("quant_mode == ORC_QUANT_STATIC_TENSOR ? 4 : 0};", "0};"),
    "abi_span_unbounded": ("span_bytes > ORC_MAX_SPAN)", "span_bytes < 0)"),
    "abi_zero_partial_scale_kept": ("a->partial_scale == 0.0f ? 1.0 :", "a->partial_scale == 0.0f ? 0.0 :"),
}


def _caught(name, old, new, pins, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "oracle"), "-o", str(lib), str(mutated), "-lm"],
                   check=True)
    env = dict(os.environ, SPRMS_ORACLE_LIB=str(lib))
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", pins)],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert proc.returncode != 0, f"pins did not catch mutation {name}:\n{proc.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(ABI_MUTATIONS))
def test_abi_pins_catch_planted_mistake(name, tmp_path):
    _caught(name, *ABI_MUTATIONS[name], "test_oracle_abi.py", tmp_path)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    _caught(name, *MUTATIONS[name], "test_oracle_pins.py", tmp_path)
