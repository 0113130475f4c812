"""The decode GEMV forms the exact integers q - zp in packed f16 pairs
(one AND-OR of the nibble into the mantissa of 1024, then one packed f16
add, or FMA with 1/16 for nibbles four bits up).  These identities hold for
every (q, zp) in 0..15 and are checked here on the IEEE binary16 encodings,
each f16 operation rounded once, as the hardware does."""

import numpy as np


def f16(bits: int) -> float:
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def round_f16(x: float) -> float:
    return float(np.float16(x))


def test_mantissa_encodings_are_the_biased_integers():
    for q in range(16):
        assert f16(0x6400 | q) == 1024 + q
        assert f16(0x6400 | (q << 4)) == 1024 + 16 * q


def test_zero_point_constants():
    for zp in range(16):
        assert f16(0xE400 | zp) == -(1024 + zp)
        assert f16(0xD400 | (zp << 4)) == -(64 + zp)


def test_packed_add_and_fma_give_q_minus_zp_exactly():
    for q in range(16):
        for zp in range(16):
            add = round_f16(f16(0x6400 | q) + f16(0xE400 | zp))
            fma = round_f16(f16(0x6400 | (q << 4)) * 0.0625 + f16(0xD400 | (zp << 4)))
            assert add == q - zp and fma == q - zp, (q, zp)
