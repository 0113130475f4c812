"""The oracle's pins are not vacuous: each plausible mistake, planted in a
copy of the oracle's C source and compiled on the CPU, fails at least one pin.

Every mutation is an in-bounds change (no planted mistake can read or write
outside its arrays), so a mutant can fail but cannot crash the test process.
"""

import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = open(oracle.SRC).read()

# (name, text in mnb_oracle.c, replacement)
MUTANTS = [
    ("pack_nibble_order_swapped",
     "if (k % 2 == 0)\n                packed[byte] |= v;",
     "if (k % 2 == 1)\n                packed[byte] |= v;"),
    ("unpack_nibble_order_swapped",
     "q[n * K + k] = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
     "q[n * K + k] = (k % 2 == 1) ? (byte & 0x0F) : (byte >> 4);"),
    ("zero_point_nibble_order_swapped",
     "zp[n * nb + b] = (b % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
     "zp[n * nb + b] = (b % 2 == 1) ? (byte & 0x0F) : (byte >> 4);"),
    ("zero_point_pack_swapped",
     "if (b % 2 == 0)\n                packed[n * row + b / 2] |= v;",
     "if (b % 2 == 1)\n                packed[n * row + b / 2] |= v;"),
    ("default_zero_point_7", "zp ? zp[n * nb + b] : 8;", "zp ? zp[n * nb + b] : 7;"),
    ("zero_point_dropped", "(double)((int)q[n * K + k] - zero)",
     "(double)((int)q[n * K + k])"),
    ("block_index_halved", "int64_t b = k / bs;", "int64_t b = k / bs / 2;"),
    ("sign_flipped_sum", "acc += p;", "acc -= p;"),
    ("bias_dropped", "acc += (double)bias[n];", "acc += 0.0;"),
    ("scale_index_transposed", "load_value(act_dtype, scales, n * nb + b)",
     "load_value(act_dtype, scales, b * N + n)"),
    ("tolerance_sum_without_abs", "mag += fabs(p);", "mag += p;"),
    ("bf16_ties_away", "double r = nearbyint(ldexp(ax, -quantum));",
     "double r = round(ldexp(ax, -quantum));"),
    ("bf16_truncates", "double r = nearbyint(ldexp(ax, -quantum));",
     "double r = floor(ldexp(ax, -quantum));"),
    ("bf16_one_bit_short", "int quantum = e - 8;", "int quantum = e - 7;"),
    ("pad_nibbles_not_cleared", "memset(packed, 0, (size_t)(N * col_bytes));",
     "memset(packed, 0x80, (size_t)(N * col_bytes));"),
    ("dequant_int_zero_point_dropped",
     "(int8_t)((int)q[n * K + k] - (zp ? zp[n * nb + k / bs] : 8))",
     "(int8_t)((int)q[n * K + k] - (zp ? 8 : 8))"),
    ("f32_rounding_toward_zero", "out[i] = (float)x[i]; /* one RTNE rounding */",
     "out[i] = nextafterf((float)x[i], 0.0f); /* one RTNE rounding */"),
    ("dequant_scale_from_wrong_block", "double s = load_value(scale_dtype, scales, n * nb + b);",
     "double s = load_value(scale_dtype, scales, n * nb + (b == 0 ? 0 : b - 1));"),
    ("qdq_nibble_order_swapped", "return (i % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
     "return (i % 2 == 1) ? (byte & 0x0F) : (byte >> 4);"),
    ("qdq_projection_read_as_tied", "return axis == 0 ? k * N + n : n * K + k;",
     "return axis == 0 ? n * K + k : n * K + k;"),
    ("qdq_projection_scales_read_as_tied", "return axis == 0 ? b * N + n : n * nb + b;",
     "return axis == 0 ? n * nb + b : n * nb + b;"),
    ("qdq_dequant_default_zero_point_8", "int zero = zp_q ? qdq_nibble(zp_q, si) : 0;",
     "int zero = zp_q ? qdq_nibble(zp_q, si) : 8;"),
    ("qdq_import_default_zero_point_8", "zp[n * nb + b] = zp_q ? qdq_nibble(zp_q, si) : 0;",
     "zp[n * nb + b] = zp_q ? qdq_nibble(zp_q, si) : 8;"),
    ("silu_sigmoid_sign_flipped", "double sig = 1.0 / (1.0 + exp(-g));",
     "double sig = 1.0 / (1.0 + exp(g));"),
    ("silu_gate_factor_dropped", "h[i] = g * sig * up[i];", "h[i] = sig * up[i];"),
    ("argmax_last_of_ties", "if (isnan(v) || v > bv) {", "if (isnan(v) || v >= bv) {"),
    ("argmax_nan_ignored", "if (isnan(v) || v > bv) {", "if (v > bv) {"),
    ("rmsnorm_sum_not_mean", "double rms = sqrt(ss / (double)K + eps);", "double rms = sqrt(ss + eps);"),
    ("rmsnorm_eps_dropped", "double rms = sqrt(ss / (double)K + eps);", "double rms = sqrt(ss / (double)K);"),
    ("rmsnorm_no_root", "double rms = sqrt(ss / (double)K + eps);", "double rms = ss / (double)K + eps;"),
    ("rmsnorm_gamma_dropped", "/ rms * load_value(dtype, gamma, k);", "/ rms * 1.0;"),
    ("rmsnorm_gamma_reversed", "/ rms * load_value(dtype, gamma, k);", "/ rms * load_value(dtype, gamma, K - 1 - k);"),
    ("matmul_f64a_zero_point_dropped",
     "double w = (double)((int)q[n * K + k] - zero) * load_value(scale_dtype, scales, n * nb + b);",
     "double w = (double)((int)q[n * K + k]) * load_value(scale_dtype, scales, n * nb + b);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    assert SRC.count(old) >= 1, f"mutation site for {name} not found in source"
    src = tmp_path / f"{name}.c"
    src.write_text(SRC.replace(old, new))
    lib = oracle.build(str(src), str(tmp_path / f"lib{name}.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} survived every pin"


def test_unmutated_copy_passes(tmp_path):
    src = tmp_path / "copy.c"
    src.write_text(SRC)
    orc = oracle.Oracle(oracle.build(str(src), str(tmp_path / "libcopy.so")))
    for pin in ALL_PINS:
        pin(orc)
