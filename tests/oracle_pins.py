"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with a fact that the pages or plain mathematics fix:

* hand-worked examples (``golden/hand_examples.json``) derived from the
  low-nibble-first, per-block storage described on the page "Qwen3 CPU
  Inference Critical Path" ("Export contract" and "Exact kernel inventory");
* exact rational arithmetic (``fractions.Fraction``) on tiny inputs, a method
  that shares nothing with the oracle's binary64 loops;
* exactness special cases (power-of-two scales, small-integer activations),
  closed forms, scaling invariants and the identity-matrix case;
* torch's float32->bfloat16 cast (a library routine) where the exact value is
  representable in float32, and brute-force nearest-neighbour search
  otherwise.

``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py``
runs them on deliberately broken copies of the oracle source to show that each
plausible mistake is caught by at least one pin.
"""

from __future__ import annotations

import json
import os
import struct
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def _bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns with torch's RTNE cast (library)."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_value(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0])


def _fr_value(x) -> Fraction:
    """Exact value of a float32 number or a bf16 bit pattern (uint16)."""
    if isinstance(x, (np.uint16,)):
        return _bf16_value(int(x))
    return Fraction(float(x))


def _exact_matmul(a, q, zp, scales, bs, bias=None):
    """Exact rational y and S from the definition, by brute force."""
    M, K = a.shape
    N = q.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                b = k // bs
                z = 8 if zp is None else int(zp[n, b])
                w = (int(q[n, k]) - z) * _fr_value(scales[n, b])
                p = _fr_value(a[m, k]) * w
                acc += p
                mag += abs(p)
            if bias is not None:
                acc += Fraction(float(bias[n]))
                mag += abs(Fraction(float(bias[n])))
            y[m][n] = acc
            S[m][n] = mag
    return y, S


# --------------------------------------------------------------------------
# hand-worked examples
# --------------------------------------------------------------------------

def pin_hand_nibble_order(orc):
    for key in ("nibble_order", "two_blocks_partial_tail"):
        g = _golden()[key]
        q = np.array(g["q"], np.uint8)
        packed = orc.pack_weights(q, g["block_size"])
        assert packed.tolist() == g["packed"], (key, packed.tolist())
        back = orc.unpack_weights(np.array(g["packed"], np.uint8), g["K"],
                                  g["N"], g["block_size"])
        assert np.array_equal(back, q), key


def pin_hand_zero_point_order(orc):
    g = _golden()["zero_point_order"]
    zp = np.array(g["zp"], np.uint8)
    packed = orc.pack_zero_points(zp)
    assert packed.tolist() == g["packed"], packed.tolist()
    back = orc.unpack_zero_points(np.array(g["packed"], np.uint8), g["N"],
                                  g["n_blocks"])
    assert np.array_equal(back, zp)


def pin_hand_worked_matmul(orc):
    g = _golden()["worked_matmul"]
    bs = g["block_size"]
    a = _f32(g["a"])
    q = np.array(g["q"], np.uint8)
    zp = np.array(g["zp"], np.uint8)
    sc = _f32(g["scales"])
    w = orc.dequant(q, zp, sc, bs)
    assert w.tolist() == g["w"], w.tolist()
    y, S = orc.matmul(a, q, zp, sc, bs)
    assert y.tolist() == g["y"] and S.tolist() == g["S"], (y, S)
    y, S = orc.matmul(a, q, zp, sc, bs, bias=_f32(g["bias"]))
    assert y.tolist() == g["y_bias"] and S.tolist() == g["S_bias"], (y, S)
    # the same numbers are exact in bfloat16 (activations and scales)
    y, S = orc.matmul(_bf16_bits(a), q, zp, _bf16_bits(sc), bs)
    assert y.tolist() == g["y"] and S.tolist() == g["S"], (y, S)


def pin_hand_rounding_ties(orc):
    g = _golden()["rounding_ties"]
    for c in g["bf16_cases"]:
        # q - zp chosen via zp=8 and q = 8 + (q-zp); one block of 16
        q = np.full((1, 16), 8 + c["q_minus_zp"], np.uint8)
        w = orc.dequant(q, None, _f32([[c["scale"]]]), 16)
        bits = orc.round_to_bf16(w)
        assert int(bits[0, 0]) == c["bf16_bits"], (c, hex(int(bits[0, 0])))
    for c in g["f32_cases"]:
        s = np.array([[c["scale_bits"]]], np.uint32).view(np.float32)
        q = np.full((1, 16), 8 + c["q_minus_zp"], np.uint8)
        w = orc.dequant(q, None, s, 16)
        f = orc.round_to_f32(w).view(np.uint32)
        assert int(f[0, 0]) == c["f32_bits"], (c, hex(int(f[0, 0])))


# --------------------------------------------------------------------------
# packing invariants
# --------------------------------------------------------------------------

def pin_pack_roundtrip_and_stream_view(orc):
    """unpack(pack(q)) == q; and each column's bytes, read as a stream of
    nibbles low-first, are that column's K values followed by zero pads."""
    rng = np.random.default_rng(1)
    for bs in (16, 32, 64, 128, 256):
        for K in sorted({1, 2, 3, bs - 1, bs, bs + 1, 2 * bs + 3, 3 * bs}):
            for N in (1, 2, 3, 5):
                q = rng.integers(0, 16, (N, K), dtype=np.uint8)
                p = orc.pack_weights(q, bs)
                nb = -(-K // bs)
                assert p.size == N * nb * bs // 2
                assert np.array_equal(orc.unpack_weights(p, K, N, bs), q)
                cols = p.reshape(N, nb * bs // 2)
                stream = np.stack([cols & 0x0F, cols >> 4], -1).reshape(N, -1)
                assert np.array_equal(stream[:, :K], q), (bs, K, N)
                assert not stream[:, K:].any(), "pad nibbles must be 0"


def pin_zero_point_roundtrip(orc):
    rng = np.random.default_rng(2)
    for nb in (1, 2, 3, 4, 7, 76):
        for N in (1, 2, 5):
            zp = rng.integers(0, 16, (N, nb), dtype=np.uint8)
            p = orc.pack_zero_points(zp)
            assert p.size == N * ((nb + 1) // 2)
            assert np.array_equal(orc.unpack_zero_points(p, N, nb), zp)
            rows = p.reshape(N, -1)
            stream = np.stack([rows & 0x0F, rows >> 4], -1).reshape(N, -1)
            assert np.array_equal(stream[:, :nb], zp)
            assert not stream[:, nb:].any()


# --------------------------------------------------------------------------
# dequantization
# --------------------------------------------------------------------------

def pin_dequant_exhaustive(orc):
    """All 16x16 (q, zp) pairs, several scales: w equals the exact rational
    (q - zp) * s; the f32 / bf16 roundings agree with torch's cast where the
    exact value is a float32, and with a nearest-neighbour search otherwise."""
    rng = np.random.default_rng(3)
    scales = [2.0 ** -7, 0.005, 0.0125, 0.02, 3.0, 2.0 ** -130]
    scales += list(rng.uniform(0.002, 0.02, 4))
    qv, zv = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    q = qv.reshape(16, 16).astype(np.uint8)          # row n = q value
    zp_col = zv.reshape(16, 16).astype(np.uint8)     # vary zp per column n
    for s in scales:
        s32 = np.float32(s)
        # N = 256 columns (q, zp), K = 16 (one block), constant q per column
        qq = np.repeat(q.reshape(256, 1), 16, 1)
        zz = zp_col.reshape(256, 1)
        sc = np.full((256, 1), s32, np.float32)
        w = orc.dequant(qq, zz, sc, 16)
        for n in range(256):
            exact = (int(qq[n, 0]) - int(zz[n, 0])) * Fraction(float(s32))
            assert Fraction(w[n, 0]) == exact, (n, s)
        f = orc.round_to_f32(w)
        b = orc.round_to_bf16(w)
        for n in range(256):
            exact = Fraction(w[n, 0])
            if Fraction(float(np.float32(float(exact)))) == exact:
                assert f[n, 0] == np.float32(float(exact))
                assert b[n, 0] == _bf16_bits(np.array([f[n, 0]]))[0]
            else:
                assert Fraction(float(f[n, 0])) == _nearest_f32(exact)
                assert _bf16_value(b[n, 0]) == _nearest_bf16(exact)


def pin_dequant_multiblock(orc):
    """Several blocks per column, partial last block, with and without zero
    points, binary32 and bfloat16 scales: every w equals the exact rational
    (q - zp[block]) * s[block], and the integer form equals q - zp[block]."""
    rng = np.random.default_rng(11)
    for K, N, bs, zp_on, bf in [(70, 3, 16, True, False), (100, 4, 32, False, False),
                                (300, 2, 128, True, True), (17, 5, 16, True, True)]:
        nb = -(-K // bs)
        q = rng.integers(0, 16, (N, K), dtype=np.uint8)
        zp = rng.integers(0, 16, (N, nb), dtype=np.uint8) if zp_on else None
        sc = rng.uniform(0.002, 0.02, (N, nb)).astype(np.float32)
        if bf:
            sc = _bf16_bits(sc)
        w = orc.dequant(q, zp, sc, bs)
        wi = orc.dequant_int(q, zp, bs)
        for n in range(N):
            for k in range(K):
                z = 8 if zp is None else int(zp[n, k // bs])
                assert int(wi[n, k]) == int(q[n, k]) - z, (n, k)
                exact = (int(q[n, k]) - z) * _fr_value(sc[n, k // bs])
                assert Fraction(w[n, k]) == exact, (K, bs, n, k)


def _nearest_by_search(x: Fraction, neighbours, even_of):
    best = None
    for c in neighbours:
        d = abs(Fraction(c) - x)
        if best is None or d < best[0] or (d == best[0] and even_of(c)):
            best = (d, c)
    return Fraction(best[1])


def _nearest_f32(x: Fraction) -> Fraction:
    f = np.float32(float(x))
    cands = {float(f), float(np.nextafter(f, np.float32(np.inf))),
             float(np.nextafter(f, np.float32(-np.inf)))}
    even = lambda c: int(np.array([c], np.float32).view(np.uint32)[0]) % 2 == 0  # noqa: E731
    return _nearest_by_search(x, cands, even)


def _nearest_bf16(x: Fraction) -> Fraction:
    base = int(np.array([float(x)], np.float32).view(np.uint32)[0]) >> 16
    cands = {}
    for h in (base - 1, base, base + 1, base + 2):
        h &= 0xFFFF
        if (h & 0x7F80) == 0x7F80:      # inf / NaN patterns are no candidates
            continue
        cands[float(_bf16_value(h))] = h
    even = lambda c: cands[c] % 2 == 0  # noqa: E731
    return _nearest_by_search(x, list(cands), even)


def pin_round_bf16_bruteforce(orc):
    """Random binary64 values (including bf16 subnormals and exact ties) are
    rounded to the neighbour a brute-force search picks."""
    rng = np.random.default_rng(4)
    xs = list(rng.standard_normal(400) * np.exp2(rng.integers(-20, 20, 400)))
    xs += [float(_bf16_value(h) + _bf16_value(h + 1)) / 2
           for h in range(0x3F80, 0x3F90)]               # exact ties
    xs += [3.5 * 2.0 ** -133, 5.5 * 2.0 ** -133, 2.0 ** -140, -1e-41]
    x = np.array(xs, np.float64)
    got = orc.round_to_bf16(x)
    for xi, g in zip(xs, got):
        assert _bf16_value(g) == _nearest_bf16(Fraction(xi)), (xi, hex(g))


def pin_default_zero_point(orc):
    """No zero-point tensor behaves as zp = 8 everywhere; q = 8 then gives
    w = 0 exactly."""
    rng = np.random.default_rng(5)
    K, N, bs = 70, 6, 32
    nb = -(-K // bs)
    q = rng.integers(0, 16, (N, K), dtype=np.uint8)
    sc = rng.uniform(0.005, 0.02, (N, nb)).astype(np.float32)
    a = rng.standard_normal((3, K)).astype(np.float32)
    y0, S0 = orc.matmul(a, q, None, sc, bs)
    y8, S8 = orc.matmul(a, q, np.full((N, nb), 8, np.uint8), sc, bs)
    assert np.array_equal(y0, y8) and np.array_equal(S0, S8)
    w = orc.dequant(np.full((N, K), 8, np.uint8), None, sc, bs)
    assert not w.any()


# --------------------------------------------------------------------------
# matmul
# --------------------------------------------------------------------------

def pin_bruteforce_fractions(orc):
    """Tiny random problems against exact rational arithmetic: the binary64
    result is within (K+1) * 2^-53 * S of the exact value, and S is exact to
    the same bound."""
    rng = np.random.default_rng(6)
    for (M, K, N, bs, zp_on, bias_on, bf) in [
            (1, 5, 3, 16, False, False, False), (2, 17, 4, 16, True, True, False),
            (3, 33, 2, 32, True, False, True), (1, 40, 3, 16, False, True, True),
            (2, 64, 2, 64, True, True, False)]:
        nb = -(-K // bs)
        q = rng.integers(0, 16, (N, K), dtype=np.uint8)
        zp = rng.integers(0, 16, (N, nb), dtype=np.uint8) if zp_on else None
        sc = rng.uniform(0.005, 0.02, (N, nb)).astype(np.float32)
        a = rng.standard_normal((M, K)).astype(np.float32)
        bias = (0.02 * rng.standard_normal(N)).astype(np.float32) if bias_on else None
        if bf:
            a, sc = _bf16_bits(a), _bf16_bits(sc)
        y, S = orc.matmul(a, q, zp, sc, bs, bias=bias)
        ye, Se = _exact_matmul(a, q, zp, sc, bs, bias)
        for m in range(M):
            for n in range(N):
                tol = (K + 1) * Fraction(2) ** -53 * Se[m][n]
                assert abs(Fraction(y[m, n]) - ye[m][n]) <= tol, (m, n)
                assert abs(Fraction(S[m, n]) - Se[m][n]) <= tol, (m, n)


def pin_exact_small_integers(orc):
    """Power-of-two scales and small-integer activations make every partial
    sum an exact binary64 number, so y must equal the integer result exactly
    (computed here with Python integers)."""
    rng = np.random.default_rng(7)
    for K, N, bs, e in [(100, 7, 16, 5), (257, 5, 128, 9), (64, 3, 64, 0)]:
        nb = -(-K // bs)
        q = rng.integers(0, 16, (N, K), dtype=np.uint8)
        zp = rng.integers(0, 16, (N, nb), dtype=np.uint8)
        ex = rng.integers(0, 4, (N, nb))
        sc = (2.0 ** -(e + ex)).astype(np.float32)
        a = rng.integers(-8, 9, (2, K)).astype(np.float32)
        y, _ = orc.matmul(a, q, zp, sc, bs)
        for m in range(2):
            for n in range(N):
                tot = Fraction(0)
                for k in range(K):
                    b = k // bs
                    tot += int(a[m, k]) * (int(q[n, k]) - int(zp[n, b])) * \
                        Fraction(1, 2 ** int(e + ex[n, b]))
                assert Fraction(y[m, n]) == tot, (K, m, n)


def pin_closed_form_constant(orc):
    """Constant a, q, zp, s: y = K * a * (q - zp) * s (a closed form)."""
    for K, bs, qv, zv, s, av in [(96, 32, 13, 3, 0.25, 1.5), (33, 16, 2, 11, 0.125, -2.0),
                                 (1000, 128, 15, 0, 2.0 ** -6, 0.75)]:
        nb = -(-K // bs)
        q = np.full((2, K), qv, np.uint8)
        zp = np.full((2, nb), zv, np.uint8)
        sc = np.full((2, nb), s, np.float32)
        a = np.full((1, K), av, np.float32)
        y, S = orc.matmul(a, q, zp, sc, bs)
        expect = K * av * (qv - zv) * s
        assert y[0, 0] == expect and y[0, 1] == expect, (y, expect)
        assert S[0, 0] == abs(expect)


def pin_scaling_invariance(orc):
    """Scaling every activation, or every scale, by 2^j scales y by 2^j
    exactly (binary64, no overflow)."""
    rng = np.random.default_rng(8)
    K, N, bs = 90, 5, 32
    nb = -(-K // bs)
    q = rng.integers(0, 16, (N, K), dtype=np.uint8)
    zp = rng.integers(0, 16, (N, nb), dtype=np.uint8)
    sc = rng.uniform(0.005, 0.02, (N, nb)).astype(np.float32)
    a = rng.standard_normal((2, K)).astype(np.float32)
    y, _ = orc.matmul(a, q, zp, sc, bs)
    for j in (-3, 5):
        ya, _ = orc.matmul((a * np.float32(2.0 ** j)).astype(np.float32), q, zp, sc, bs)
        ys, _ = orc.matmul(a, q, zp, (sc * np.float32(2.0 ** j)).astype(np.float32), bs)
        assert np.array_equal(ya, y * 2.0 ** j) and np.array_equal(ys, y * 2.0 ** j)


def pin_identity_activation(orc):
    """A = I_K returns the dequantized weights: y[k][n] = w[n][k], and a
    one-hot row picks one weight; both exact."""
    rng = np.random.default_rng(9)
    K, N, bs = 48, 6, 16
    nb = -(-K // bs)
    q = rng.integers(0, 16, (N, K), dtype=np.uint8)
    zp = rng.integers(0, 16, (N, nb), dtype=np.uint8)
    sc = rng.uniform(0.005, 0.02, (N, nb)).astype(np.float32)
    y, _ = orc.matmul(np.eye(K, dtype=np.float32), q, zp, sc, bs)
    for k in range(K):
        for n in range(N):
            w = (int(q[n, k]) - int(zp[n, k // bs])) * Fraction(float(sc[n, k // bs]))
            assert Fraction(y[k, n]) == w, (k, n)


def pin_fused_columns_independent(orc):
    """Concatenating two weight matrices along N gives the concatenation of
    the separate results, and permuting columns permutes y (the operation is
    column-separable)."""
    rng = np.random.default_rng(10)
    K, bs = 80, 16
    nb = -(-K // bs)
    a = rng.standard_normal((2, K)).astype(np.float32)
    parts = []
    for N in (3, 5):
        parts.append((rng.integers(0, 16, (N, K), dtype=np.uint8),
                      rng.integers(0, 16, (N, nb), dtype=np.uint8),
                      rng.uniform(0.005, 0.02, (N, nb)).astype(np.float32)))
    ys = [orc.matmul(a, *p, bs)[0] for p in parts]
    cat = [np.concatenate(x, 0) for x in zip(*parts)]
    yc, _ = orc.matmul(a, *cat, bs)
    assert np.array_equal(yc, np.concatenate(ys, 1))
    perm = rng.permutation(8)
    yp, _ = orc.matmul(a, cat[0][perm], cat[1][perm], cat[2][perm], bs)
    assert np.array_equal(yp, yc[:, perm])


def pin_contract_rules(orc):
    ok = [bs for bs in range(0, 600) if orc.contract_ok(64, 8, 4, bs)]
    assert ok == [16, 32, 64, 128, 256], ok
    assert not orc.contract_ok(64, 8, 8, 32)
    assert not orc.contract_ok(0, 8, 4, 32)
    assert not orc.contract_ok(64, 0, 4, 32)


# ---------------------------------------------------------------------------
# the QDQ encoding, the gated MLP product and greedy ArgMax
# ---------------------------------------------------------------------------

QDQ_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qdq_examples.json")


def _qdq_golden():
    with open(QDQ_GOLDEN) as f:
        return json.load(f)


def pin_qdq_hand_unpack(orc):
    g = _qdq_golden()["unpack"]
    got = orc.qdq_unpack(np.array(g["packed"], np.uint8), len(g["values"]))
    assert got.tolist() == g["values"]


def pin_qdq_hand_projection(orc):
    g = _qdq_golden()["projection_axis0"]
    K, N, bs = g["K"], g["N"], g["block_size"]
    w_q = np.array(g["w_q"], np.uint8)
    zp_q = np.array(g["zp_q"], np.uint8)
    sc = _f32(g["scales_q_bN"])
    # the fixture's packed bytes really are the row-major flattening
    assert orc.qdq_unpack(w_q, K * N).tolist() == sum(g["w_logical_KN"], [])
    b, s, z = orc.qdq_import(w_q, zp_q, sc, K, N, bs, axis=0)
    assert b.tolist() == g["b_packed"]
    assert s.tolist() == g["scales_Nb"]
    assert z.tolist() == g["zp_packed"]
    assert orc.qdq_dequant(w_q, zp_q, sc, K, N, bs, axis=0).tolist() == g["dequant_KN"]


def pin_qdq_hand_projection_two_blocks(orc):
    g = _qdq_golden()["projection_axis0_two_blocks"]
    K, N, bs = g["K"], g["N"], g["block_size"]
    w_q = np.array(g["w_q"], np.uint8)
    zp_q = np.array(g["zp_q"], np.uint8)
    sc = _f32(g["scales_q_bN"])
    b, s, z = orc.qdq_import(w_q, zp_q, sc, K, N, bs, axis=0)
    assert b.tolist() == g["b_packed"]
    assert s.tolist() == g["scales_Nb"]
    assert z.tolist() == g["zp_packed"]
    w = orc.qdq_dequant(w_q, zp_q, sc, K, N, bs, axis=0)
    assert all(w[k].tolist() == g["dequant_rows"]["k_below_16"] for k in range(16))
    assert all(w[k].tolist() == g["dequant_rows"]["k_from_16"] for k in range(16, K))


def pin_qdq_hand_tied(orc):
    g = _qdq_golden()["tied_axis1"]
    K, N, bs = g["K"], g["N"], g["block_size"]
    w_q = np.array(g["w_q"], np.uint8)
    sc = _f32(g["scales_q_Nb"])
    assert orc.qdq_unpack(w_q, K * N).tolist() == sum(g["w_logical_NK"], [])
    b, s, z = orc.qdq_import(w_q, None, sc, K, N, bs, axis=1)
    assert b.tolist() == g["b_packed"]
    assert s.tolist() == g["scales_q_Nb"]
    assert z.tolist() == g["zp_packed"]
    assert orc.qdq_dequant(w_q, None, sc, K, N, bs, axis=1).tolist() == g["dequant_KN"]


def pin_qdq_roundtrip_both_axes(orc):
    """DequantizeLinear evaluated on the QDQ tensors equals the MatMulNBits
    dequantization of the normalized tensors (two independent index
    formulations), for odd sizes, partial blocks, with and without zero
    points, float32 and bfloat16 scales."""
    rng = np.random.default_rng(21)
    for K, N, bs, axis, has_zp, dt in [(37, 5, 16, 0, True, "f32"), (64, 7, 32, 0, False, "bf16"),
                                       (100, 3, 64, 1, True, "f32"), (33, 9, 16, 1, False, "bf16"),
                                       (256, 4, 128, 0, True, "bf16"), (17, 1, 256, 1, True, "f32")]:
        nb = -(-K // bs)
        w_q = rng.integers(0, 256, (K * N + 1) // 2, dtype=np.uint8)
        zp_q = rng.integers(0, 256, (nb * N + 1) // 2, dtype=np.uint8) if has_zp else None
        sc = rng.uniform(0.005, 0.05, nb * N).astype(np.float32)
        if dt == "bf16":
            sc = _bf16_bits(sc)
        ref = orc.qdq_dequant(w_q, zp_q, sc, K, N, bs, axis)
        b, s, z = orc.qdq_import(w_q, zp_q, sc, K, N, bs, axis)
        q = orc.unpack_weights(b, K, N, bs)
        zp = orc.unpack_zero_points(z, N, nb)
        w = orc.dequant(q, zp, s, bs)                      # [N][K]
        assert np.array_equal(w.T, ref), (K, N, bs, axis, has_zp, dt)
        if not has_zp:
            assert not zp.any()


def pin_qdq_tied_is_native_storage(orc):
    """axis 1 with whole blocks and an even block count: the QDQ bytes already
    are the MatMulNBits storage (the tied weight needs no copy)."""
    rng = np.random.default_rng(22)
    for K, N, bs in [(64, 5, 32), (256, 3, 128), (1024, 2, 32)]:
        nb = K // bs
        assert nb % 2 == 0
        w_q = rng.integers(0, 256, K * N // 2, dtype=np.uint8)
        zp_q = rng.integers(0, 256, nb * N // 2, dtype=np.uint8)
        sc = rng.uniform(0.005, 0.05, nb * N).astype(np.float32)
        b, s, z = orc.qdq_import(w_q, zp_q, sc, K, N, bs, axis=1)
        assert np.array_equal(b, w_q) and np.array_equal(z, zp_q)
        assert np.array_equal(s.ravel(), sc)


def pin_silu_mul_closed_forms(orc):
    g = _qdq_golden()["silu_mul"]
    h = orc.silu_mul(np.array(g["gate"]), np.array(g["up"]))
    assert np.allclose(h, g["h"], rtol=1e-15, atol=0)
    x = np.linspace(-30, 30, 61)
    one = np.ones_like(x)
    # silu(x) - silu(-x) = x, silu is x for large x, linear in the up value
    assert np.allclose(orc.silu_mul(x, one) - orc.silu_mul(-x, one), x, rtol=1e-14, atol=1e-14)
    assert orc.silu_mul(np.array([60.0]), np.array([1.0]))[0] == 60.0
    assert np.array_equal(orc.silu_mul(x, 3 * one), 3 * orc.silu_mul(x, one))


def pin_argmax_hand(orc):
    g = _qdq_golden()["argmax"]
    rows = np.array([[float(v) for v in r] for r in g["rows"]], np.float32)
    assert orc.argmax(rows).tolist() == g["index"]
    # the same decisions on bfloat16 bit patterns of these exact values
    assert orc.argmax(_bf16_bits(rows)).tolist() == g["index"]


def pin_argmax_bruteforce(orc):
    rng = np.random.default_rng(23)
    x = rng.integers(-3, 4, (50, 37)).astype(np.float32)     # many ties
    want = [int(min(i for i in range(37) if r[i] == r.max())) for r in x]
    assert orc.argmax(x).tolist() == want




def pin_rmsnorm_exact(orc):
    """Rows whose mean square is a perfect square (eps = 0): the normalized
    input is rational and known by hand; eps enters under the root."""
    x = np.array([[3, 4, 0, 0], [1, 1, 1, 1], [-2, 0, 0, 0], [0, 0, 0, 8]], np.float32)
    g = np.array([1, 2, 3, 4], np.float32)
    a = orc.rmsnorm(x, g, 0.0)
    # rms: sqrt(25 / 4) = 5 / 2; 1; sqrt(4 / 4) = 1; sqrt(64 / 4) = 4
    want = np.array([[1.2, 3.2, 0, 0], [1, 2, 3, 4], [-2, 0, 0, 0], [0, 0, 0, 8]])
    assert np.allclose(a, want, rtol=1e-15, atol=0)
    # eps = 1 on a unit row: rms = sqrt(1 + 1)
    a1 = orc.rmsnorm(np.ones((1, 4), np.float32), np.ones(4, np.float32), 1.0)
    assert np.allclose(a1, 1 / np.sqrt(2.0), rtol=1e-15)
    # a zero row with eps > 0 is zero (no division by zero)
    assert np.array_equal(orc.rmsnorm(np.zeros((1, 8), np.float32), np.ones(8, np.float32), 1e-6),
                          np.zeros((1, 8)))
    # bfloat16 bit patterns of the same exact values give the same result
    assert np.allclose(orc.rmsnorm(_bf16_bits(x), _bf16_bits(g), 0.0), want, rtol=1e-15, atol=0)


def pin_rmsnorm_invariants(orc):
    rng = np.random.default_rng(31)
    x = rng.standard_normal((3, 40)).astype(np.float32)
    g = rng.standard_normal(40).astype(np.float32)
    a = orc.rmsnorm(x, g, 0.0)
    # scale invariance without eps; K = 1 gives sign(x) * gamma
    assert np.allclose(orc.rmsnorm(x * np.float32(4.0), g, 0.0), a, rtol=1e-15, atol=0)
    # (x * 3 rounds each input once in float32: relative 2^-24)
    assert np.allclose(orc.rmsnorm(x * np.float32(3.0), g, 0.0), a, rtol=2.0 ** -22, atol=0)
    assert np.array_equal(orc.rmsnorm(np.array([[-5.0]], np.float32), np.array([7.0], np.float32), 0.0),
                          np.array([[-7.0]]))
    # with gamma = 1 every row has mean square 1
    a1 = orc.rmsnorm(x, np.ones(40, np.float32), 0.0)
    assert np.allclose((a1 * a1).mean(axis=1), 1.0, rtol=1e-14)


def pin_matmul_f64a_bruteforce(orc):
    """Binary64 activations against the quantized weight: exact rational
    evaluation on a tiny shape (the activations chosen dyadic, so every
    product is exact), and agreement with the float32 matmul when the
    activations are float32 values."""
    from fractions import Fraction
    rng = np.random.default_rng(5)
    K, N, bs = 24, 5, 16
    q = rng.integers(0, 16, (N, K), dtype=np.uint8)
    zp = rng.integers(0, 16, (N, 2), dtype=np.uint8)
    sc = rng.uniform(0.005, 0.02, (N, 2)).astype(np.float32)
    a = (rng.integers(-40, 41, (2, K)) / 8.0).astype(np.float64)
    bias = rng.standard_normal(N).astype(np.float32)
    y, S = orc.matmul_f64a(a, q, zp, sc, bs, bias)
    for m in range(2):
        for n in range(N):
            acc = sum(Fraction(float(a[m, k])) * (int(q[n, k]) - int(zp[n, k // bs])) * Fraction(float(sc[n, k // bs]))
                      for k in range(K)) + Fraction(float(bias[n]))
            assert abs(float(acc) - y[m, n]) <= 1e-15 * S[m, n] + 1e-300
    y32, S32 = orc.matmul(a.astype(np.float32), q, zp, sc, bs, bias=bias)
    assert np.array_equal(y, y32) and np.array_equal(S, S32)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
