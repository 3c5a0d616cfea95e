"""Planted mistakes in copies of the CPU oracle must each fail at least one pin.

Each mutant is the oracle's C source with one plausible mistake (a wrong bit or
byte order, a dropped term, a flipped sign, a wrong or transposed index, a
missing scale), compiled to a temporary library and checked in a subprocess
(so a mutant that misbehaves cannot take the test process down).  This shows
that the pins are strong enough to notice such mistakes in the oracle.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTANTS = {
    "unpack_msb_first": ("q |= stream_bit(col, i * bits + j) << j;",
                         "q |= stream_bit(col, i * bits + j) << (bits - 1 - j);"),
    "pack_msb_first_bytes": ("col[p >> 3] |= (uint8_t)(1u << (p & 7));",
                             "col[p >> 3] |= (uint8_t)(0x80u >> (p & 7));"),
    "stream_bit_wrong_byte": ("return (col[p >> 3] >> (p & 7)) & 1u;",
                              "return (col[p >> 3] >> (p % 6)) & 1u;"),
    "codes_transposed": ("unsigned q = codes[i * N + n] & mask;",
                         "unsigned q = codes[n * K + i] & mask;"),
    "zero_point_off_by_one": ("return z ? z[n * ngroups + g] : (double)(1u << (bits - 1));",
                              "return z ? z[n * ngroups + g] : (double)((1u << (bits - 1)) - 1u);"),
    "per_group_z_ignored": ("return z ? z[n * ngroups + g] : (double)(1u << (bits - 1));",
                            "return (double)(1u << (bits - 1));"),
    "dequant_sign_flipped": ("w[i] = (q - zero_point(z, n, g, ngroups, bits)) * s[n * ngroups + g];",
                             "w[i] = (zero_point(z, n, g, ngroups, bits) - q) * s[n * ngroups + g];"),
    "group_index_modulo": ("            int64_t g = i / G;\n            double q = (double)column_code(col, i, bits);\n"
                           "            w[i] =",
                           "            int64_t g = i % ngroups;\n            double q = (double)column_code(col, i, bits);\n"
                           "            w[i] ="),
    "scale_transposed": ("w[i] = (q - zero_point(z, n, g, ngroups, bits)) * s[n * ngroups + g];",
                         "w[i] = (q - zero_point(z, n, g, ngroups, bits)) * s[(g * N + n) % (N * ngroups)];"),
    "scale_dropped": ("w[i] = (q - zero_point(z, n, g, ngroups, bits)) * s[n * ngroups + g];",
                      "w[i] = (q - zero_point(z, n, g, ngroups, bits));"),
    "matmul_drops_last_term": ("            for (int64_t i = 0; i < K; ++i)\n                acc += X[m * K + i] * w[i];",
                               "            for (int64_t i = 0; i + 1 < K; ++i)\n                acc += X[m * K + i] * w[i];"),
    "matmul_x_transposed": ("                acc += X[m * K + i] * w[i];",
                            "                acc += X[i * M + m] * w[i];"),
    "w4a8_zero_sign": ("a += (int64_t)Xq[m * K + i] * (q[i] - zg);",
                       "a += (int64_t)Xq[m * K + i] * (q[i] + zg);"),
    "w4a8_first_group_scale": ("y += s[n * ngroups + g] * (double)a;",
                               "y += s[n * ngroups] * (double)a;"),
    "w4a8_token_scale_dropped": ("Y[m * N + n] = sx[m] * y;", "Y[m * N + n] = y;"),
    "w4a8_group_short": ("for (int64_t i = g * G; i < (g + 1) * G; ++i)",
                         "for (int64_t i = g * G; i + 1 < (g + 1) * G; ++i)"),
    "quantize_range_without_zero": ("            double lo = 0.0, hi = 0.0;\n",
                                    "            double lo = W[g * G * N + n], hi = W[g * G * N + n];\n"),
    "quantize_round_half_up": ("const double q = fmin(fmax(rint(W[i * N + n] / sg) + zg, 0.0), qmax);",
                               "const double q = fmin(fmax(floor(W[i * N + n] / sg + 0.5) + zg, 0.0), qmax);"),
    "quantize_zero_point_sign": ("const double zg = fmin(fmax(rint(-lo / sg), 0.0), qmax);",
                                 "const double zg = fmin(fmax(rint(lo / sg), 0.0), qmax);"),
    "quantize_levels_off_by_one": ("const double qmax = (double)((1 << bits) - 1);",
                                   "const double qmax = (double)(1 << bits);"),
    "quantize_scale_truncated": ("const double r = rint(x / quantum) * quantum;",
                                 "const double r = floor(x / quantum) * quantum;"),
    "quantize_scale_not_fp16": ("double sg = round_to_fp16((hi - lo) / qmax);",
                                "double sg = (hi - lo) / qmax;"),
    "e2m1_bias_off_by_one": ("return sign * (e == 0 ? ldexp((double)m, -1) : ldexp(1.0 + (double)m / 2.0, (int)e - 1));",
                             "return sign * (e == 0 ? ldexp((double)m, -1) : ldexp(1.0 + (double)m / 2.0, (int)e));"),
    "e4m3_no_subnormals": ("return sign * (e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7));",
                           "return sign * (e == 0 ? ldexp(1.0 + (double)m / 8.0, -7) : ldexp(1.0 + (double)m / 8.0, (int)e - 7));"),
    "e4m3_mantissa_halved": ("return sign * (e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7));",
                             "return sign * (e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 16.0, (int)e - 7));"),
    "fp6_formats_swapped": ("const int mb = fmt == 2 ? 2 : 3, bias = fmt == 2 ? 3 : 1;",
                            "const int mb = fmt == 2 ? 3 : 2, bias = fmt == 2 ? 1 : 3;"),
    "fp6_no_subnormals": ("return sign * (e == 0 ? ldexp(frac, 1 - bias) : ldexp(1.0 + frac, (int)e - bias));",
                          "return sign * (e == 0 ? ldexp(1.0 + frac, -bias) : ldexp(1.0 + frac, (int)e - bias));"),
    "fp6_sign_bit_wrong": ("const double sign = (q & 0x20u) ? -1.0 : 1.0;",
                           "const double sign = (q & 0x10u) ? -1.0 : 1.0;"),
    "fp357_bias_off_by_one": ("const int eb = fmt - 3, mbits = fmt - 3, k = 1 + eb + mbits, bias = (1 << (eb - 1)) - 1;",
                              "const int eb = fmt - 3, mbits = fmt - 3, k = 1 + eb + mbits, bias = (1 << (eb - 1));"),
    "fp357_sign_bit_wrong": ("const double sign = ((q >> (k - 1)) & 1u) ? -1.0 : 1.0;",
                             "const double sign = ((q >> (k - 2)) & 1u) ? -1.0 : 1.0;"),
    "fp_product_scale_dropped": ("w[i] = float_code_value(column_code(col, i, bits), fmt) * s[n * ngroups + i / G];",
                                 "w[i] = float_code_value(column_code(col, i, bits), fmt);"),
    "sampled_drops_scale": ("            double w = (q - zero_point(z, n, g, ngroups, bits)) * s[n * ngroups + g];",
                            "            double w = (q - zero_point(z, n, g, ngroups, bits));"),
}

RUNNER = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
orc = oracle.Oracle({lib!r})
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(orc)
    except Exception as e:
        failed.append(pin.__name__)
print("FAILED_PINS", ",".join(failed))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found in the oracle source"
    mutated = src.replace(old, new, 1)
    c_path = tmp_path / "mutant.c"
    c_path.write_text(mutated)
    lib = str(tmp_path / "libmutant.so")
    oracle.build(str(c_path), lib, strict=False)
    code = RUNNER.format(root=ROOT, tests=HERE, lib=lib)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    line = [l for l in proc.stdout.splitlines() if l.startswith("FAILED_PINS")]
    if proc.returncode != 0 and not line:
        return  # the mutant crashed the pin run outright: caught
    failed = line[0].split(" ", 1)[1] if line and " " in line[0] else ""
    assert failed.strip(), f"mutant {name} passed every pin"
