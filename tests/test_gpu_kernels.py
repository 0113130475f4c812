"""GPU parity of every kernel against the CPU oracle, through the C ABI.

Bit-exact: packed bytes, dequantized weights (f32, bf16, the integer tile),
exact-arithmetic cases, identity / one-hot, fusion and permutation, pad
contents, default zero point, run-to-run determinism.  Within tolerance: GEMV
and GEMM sweeps over ragged K, N and M, every block size, with and without
zero points and bias, float32 and bfloat16.
"""

import itertools

import numpy as np
import pytest
import torch

import weight_only_int4_matmulnbits_amd as mnb
from parity import act_np, assert_close, log, oracle_ref, out_f64
from workloads.generate import random_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(K, N, M, bs, dt, zp, bias, seed):
    inp = random_inputs(K, N, M, bs, dt, zp, bias, seed=seed)
    return inp, inp.to(DEV)


def _packed(g, bs):
    return mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs)


# ---------------------------------------------------------------------------
# pack and dequant: bit-exact
# ---------------------------------------------------------------------------

PACK_K = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 127, 128, 129, 255, 256, 257, 1000]


@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_pack_bytes_match_oracle(orc, bs):
    for K, N, zp in itertools.product(PACK_K, [1, 2, 3, 65], [False, True]):
        log(f"pack bs={bs} K={K} N={N} zp={zp}")
        inp, g = _inputs(K, N, 1, bs, "f32", zp, False, seed=K * 7 + N)
        b, zpp = mnb.pack(g.q, g.zp, bs)
        ref = orc.pack_weights(inp.q.numpy(), bs)
        assert np.array_equal(b.cpu().numpy(), ref), (bs, K, N)
        if zp:
            assert np.array_equal(zpp.cpu().numpy(), orc.pack_zero_points(inp.zp.numpy()))


def test_pack_ignores_high_bits(orc):
    inp, g = _inputs(100, 7, 1, 32, "f32", True, False, seed=3)
    b0, z0 = mnb.pack(g.q, g.zp, 32)
    b1, z1 = mnb.pack(g.q | 0xF0, g.zp | 0x30, 32)
    assert torch.equal(b0, b1) and torch.equal(z0, z1)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [16, 32, 128])
def test_dequant_bit_exact(orc, dt, bs):
    for K, N, zp in [(1, 1, False), (33, 5, True), (257, 9, True), (1000, 17, False),
                     (bs * 3, 4, True)]:
        log(f"dequant {dt} bs={bs} K={K} N={N} zp={zp}")
        inp, g = _inputs(K, N, 1, bs, dt, zp, False, seed=K + N)
        pw = _packed(g, bs)
        adt = torch.float32 if dt == "f32" else torch.bfloat16
        kw = dict(K=K, N=N, block_size=bs, act_dtype=adt)
        w_exact = orc.dequant(inp.q.numpy(), None if inp.zp is None else inp.zp.numpy(),
                              act_np(inp.scales), bs)
        w32 = mnb.dequant(pw.b_packed, pw.scales, pw.zp_packed, out_kind=mnb.DEQUANT_F32, **kw)
        assert np.array_equal(w32.cpu().numpy().view(np.uint32),
                              orc.round_to_f32(w_exact).view(np.uint32))
        w16 = mnb.dequant(pw.b_packed, pw.scales, pw.zp_packed, out_kind=mnb.DEQUANT_BF16, **kw)
        assert np.array_equal(act_np(w16), orc.round_to_bf16(w_exact))
        wi = mnb.dequant(pw.b_packed, pw.scales, pw.zp_packed, out_kind=mnb.DEQUANT_INT8, **kw)
        assert np.array_equal(wi.cpu().numpy(),
                              orc.dequant_int(inp.q.numpy(),
                                              None if inp.zp is None else inp.zp.numpy(), bs))


def test_dequant_rounding_ties(orc):
    """Scales chosen so that (q - zp) * s falls exactly between two bfloat16
    values (ties to even) or two float32 values."""
    N, K, bs = 4, 16, 16
    q = torch.full((N, K), 8, dtype=torch.uint8)
    q[:, :4] = torch.tensor([9, 11, 7, 9], dtype=torch.uint8)
    s = torch.tensor([[1.00390625], [1.00390625], [1.01171875],
                      [np.frombuffer(np.uint32(0x3F800001).tobytes(), np.float32)[0]]],
                     dtype=torch.float32)
    g_q, g_s = q.to(DEV), s.to(DEV)
    pw = mnb.PackedWeight.from_logical(g_q, g_s, block_size=bs)
    w_exact = orc.dequant(q.numpy(), None, s.numpy(), bs)
    w16 = mnb.dequant(pw.b_packed, pw.scales, None, K=K, N=N, block_size=bs,
                      out_kind=mnb.DEQUANT_BF16)
    assert np.array_equal(act_np(w16), orc.round_to_bf16(w_exact))
    w32 = mnb.dequant(pw.b_packed, pw.scales, None, K=K, N=N, block_size=bs)
    assert np.array_equal(w32.cpu().numpy(), orc.round_to_f32(w_exact))


# ---------------------------------------------------------------------------
# GEMV / GEMM: within tolerance
# ---------------------------------------------------------------------------

GEMV_K = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 127, 128, 129, 255, 256, 257,
          1000, 1024, 1536, 2048, 2560, 3072, 4096, 5120, 6144, 8192 + 96, 9728, 12288]
GEMV_N = [1, 2, 3, 63, 64, 65, 127, 129]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_gemv_parity_sweep(orc, dt, bs):
    rng = np.random.default_rng(bs)
    worst = 0.0
    for K in GEMV_K:
        Ns = GEMV_N if K <= 1024 else [1, 65, 129]
        for N in Ns:
            zp, bias = bool(rng.integers(2)), bool(rng.integers(2))
            log(f"gemv {dt} bs={bs} K={K} N={N} zp={zp} bias={bias}")
            inp, g = _inputs(K, N, 1, bs, dt, zp, bias, seed=K * 131 + N)
            y = _packed(g, bs).matmul(g.a)
            y_ref, S = oracle_ref(orc, inp)
            worst = max(worst, assert_close(out_f64(y), y_ref, S, dt, f"K={K} N={N}"))
    log(f"gemv {dt} bs={bs}: worst err/tol {worst:.3g}")


GEMM_CASES = [  # (M, K, N)
    (1, 64, 64), (2, 33, 5), (3, 257, 129), (17, 1000, 63), (64, 128, 128),
    (65, 129, 130), (128, 256, 256), (130, 512, 200), (257, 320, 300),
    (512, 1024, 257), (33, 2560, 96), (40, 9728, 64), (7, 16, 1), (300, 1, 9),
    (96, 544, 200),   # K % 64 == 32: float32 products keep 32-value K steps
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_gemm_parity_sweep(orc, dt, bs):
    rng = np.random.default_rng(100 + bs)
    worst = 0.0
    for M, K, N in GEMM_CASES:
        zp, bias = bool(rng.integers(2)), bool(rng.integers(2))
        log(f"gemm {dt} bs={bs} M={M} K={K} N={N} zp={zp} bias={bias}")
        inp, g = _inputs(K, N, M, bs, dt, zp, bias, seed=M * 7 + K * 131 + N)
        pw = _packed(g, bs)
        y = mnb.gemm(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=N,
                     block_size=bs)
        y_ref, S = oracle_ref(orc, inp)
        worst = max(worst, assert_close(out_f64(y), y_ref, S, dt, f"M={M} K={K} N={N}"))
    log(f"gemm {dt} bs={bs}: worst err/tol {worst:.3g}")


@pytest.mark.parametrize("K,bs", [(5120, 16), (5120 + 16, 16), (14560, 32),
                                  (14560 + 32, 32), (12288, 128), (16384 + 100, 256)])
def test_gemv_long_k_and_beyond_register_limit(orc, K, bs):
    """Split-K across wavefronts up to mnb_gemv_max_k; K above it is served
    at M = 1 by the tiled kernel."""
    N = 40
    d = mnb.make_desc(K, N, bs)
    log(f"long K={K} bs={bs} max_k={mnb.gemv_max_k(d)}")
    inp, g = _inputs(K, N, 1, bs, "f32", True, True, seed=5)
    y = _packed(g, bs).matmul(g.a)
    y_ref, S = oracle_ref(orc, inp)
    assert_close(out_f64(y), y_ref, S, "f32", f"K={K} bs={bs}")


# ---------------------------------------------------------------------------
# bit-exact special cases and invariants
# ---------------------------------------------------------------------------

def _exact_case(K, N, M, bs, dt, seed):
    """Power-of-two scales and small-integer activations: every partial sum is
    exact in float32, so any summation order gives the exact result."""
    rng = np.random.default_rng(seed)
    nb = -(-K // bs)
    q = torch.from_numpy(rng.integers(0, 16, (N, K), dtype=np.uint8))
    zp = torch.from_numpy(rng.integers(0, 16, (N, nb), dtype=np.uint8))
    sc = torch.from_numpy((2.0 ** -rng.integers(5, 9, (N, nb))).astype(np.float32))
    a = torch.from_numpy(rng.integers(-8, 9, (M, K)).astype(np.float32))
    bias = torch.from_numpy((rng.integers(-64, 65, N) / 8.0).astype(np.float32))
    if dt == "bf16":
        sc, a = sc.to(torch.bfloat16), a.to(torch.bfloat16)
    return q, zp, sc, a, bias


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M", [1, 5, 130])
def test_exact_arithmetic_bit_exact(orc, dt, M):
    for K, N, bs in [(1024, 70, 32), (2560, 33, 128), (333, 17, 16)]:
        log(f"exact {dt} M={M} K={K} N={N} bs={bs}")
        q, zp, sc, a, bias = _exact_case(K, N, M, bs, dt, seed=K + M)
        pw = mnb.PackedWeight.from_logical(q.to(DEV), sc.to(DEV), zp.to(DEV), bias.to(DEV),
                                           block_size=bs)
        y = pw.matmul(a.to(DEV))
        y_ref, _ = orc.matmul(act_np(a), q.numpy(), zp.numpy(), act_np(sc), bs,
                              bias=bias.numpy())
        if dt == "f32":
            assert np.array_equal(y.cpu().numpy(), orc.round_to_f32(y_ref)), (K, N, M)
        else:
            assert np.array_equal(act_np(y), orc.round_to_bf16(y_ref)), (K, N, M)


def test_identity_and_one_hot_return_dequantized_weights(orc):
    K, N, bs = 96, 40, 32
    inp, g = _inputs(K, N, 1, bs, "f32", True, False, seed=11)
    pw = _packed(g, bs)
    w = orc.round_to_f32(orc.dequant(inp.q.numpy(), inp.zp.numpy(), inp.scales.numpy(), bs))
    y = mnb.gemm(torch.eye(K, device=DEV), pw.b_packed, pw.scales, pw.zp_packed, K=K, N=N,
                 block_size=bs)
    assert np.array_equal(y.cpu().numpy(), w.T)
    for k in (0, 1, 31, 32, 95):
        a = torch.zeros(1, K, device=DEV)
        a[0, k] = 1.0
        yv = pw.matmul(a)
        assert np.array_equal(yv.cpu().numpy()[0], w[:, k]), k


@pytest.mark.parametrize("bs,zp", [(16, True), (32, True), (32, False), (128, True)])
def test_f32_gemm_large_tiles_matches_oracle(orc, bs, zp):
    """Float32 products with at least two 128 x 128 output tiles per CU take
    the 128 x 128 tile kernel (short ones take 64 x 64 tiles): every output
    of a ragged shape against the oracle, and identity rows return the
    float32 dequantized weights bit for bit."""
    M, K, N = 130, 320, 256 * 128 + 37
    log(f"f32 large tiles M={M} K={K} N={N} bs={bs} zp={zp}")
    inp, g = _inputs(K, N, M, bs, "f32", zp, not zp, seed=bs * 7 + zp)
    pw = _packed(g, bs)
    y = pw.matmul(g.a)
    y_ref, S = oracle_ref(orc, inp)
    assert_close(out_f64(y), y_ref, S, "f32", f"large tiles bs={bs} zp={zp}")
    Ki = 256
    inp, g = _inputs(Ki, N, 1, bs, "f32", zp, False, seed=bs + 3)
    pw = _packed(g, bs)
    w = orc.round_to_f32(orc.dequant(inp.q.numpy(), None if inp.zp is None else inp.zp.numpy(),
                                     inp.scales.numpy(), bs))
    y = pw.matmul(torch.eye(Ki, device=DEV))
    assert np.array_equal(y.cpu().numpy(), w.T)


@pytest.mark.parametrize("M", [1, 64])
def test_fused_launch_bit_identical_to_separate(M):
    """gate||up in one launch == the two launches; any column permutation of
    the packed matrix permutes y exactly."""
    for K, bs, dt in [(1024, 32, "f32"), (2560, 128, "f32"), (2560, 128, "bf16")]:
        log(f"fusion M={M} K={K} bs={bs} {dt}")
        _, g1 = _inputs(K, 300, M, bs, dt, True, False, seed=1)
        _, g2 = _inputs(K, 200, M, bs, dt, True, False, seed=2)
        p1, p2 = _packed(g1, bs), _packed(g2, bs)
        a = g1.a
        y1, y2 = p1.matmul(a), p2.matmul(a)
        q = torch.cat([g1.q, g2.q])
        fused = mnb.PackedWeight.from_logical(q, torch.cat([g1.scales, g2.scales]),
                                              torch.cat([g1.zp, g2.zp]), block_size=bs)
        yf = fused.matmul(a)
        assert torch.equal(yf, torch.cat([y1, y2], 1))
        perm = torch.randperm(500, generator=torch.Generator().manual_seed(0)).to(DEV)
        pp = mnb.PackedWeight.from_logical(q[perm], torch.cat([g1.scales, g2.scales])[perm],
                                           torch.cat([g1.zp, g2.zp])[perm], block_size=bs)
        assert torch.equal(pp.matmul(a), yf[:, perm])


@pytest.mark.parametrize("K,bs,dt,zp,bias,N", [(2560, 128, "f32", True, True, 131072 + 37),
                                                (2560, 128, "bf16", False, False, 131072 + 37),
                                                (4096, 64, "f32", True, False, 40000),
                                                (12288, 128, "f32", True, True, 3001)])
def test_wide_gemv_bit_identical_to_narrow_launches(K, bs, dt, zp, bias, N):
    """A one-row launch over so many columns that its teams each walk many
    column groups (an LM head) holds the activations in registers; narrow
    launches read them from LDS chunk by chunk.  Both add the same values in
    the same order, so every column has the same bits.  K = 12288: split-K
    teams of two wavefronts on a grid past the resident workgroups."""
    log(f"wide vs narrow gemv K={K} bs={bs} {dt} N={N}")
    inp, g = _inputs(K, N, 1, bs, dt, zp, bias, seed=K + N)
    y = _packed(g, bs).matmul(g.a)
    for lo, hi in [(0, 1000), (N - 517, N), (N // 2, N // 2 + 64)]:
        part = mnb.PackedWeight.from_logical(g.q[lo:hi], g.scales[lo:hi], g.zp[lo:hi] if zp else None,
                                             g.bias[lo:hi] if bias else None, block_size=bs)
        assert torch.equal(part.matmul(g.a), y[:, lo:hi]), (lo, hi)


@pytest.mark.parametrize("M", [1, 20])
def test_pad_nibbles_do_not_matter(M):
    K, N, bs = 100, 33, 64          # partial last block (36 of 64 values)
    _, g = _inputs(K, N, M, bs, "f32", True, True, seed=4)
    pw = _packed(g, bs)
    y0 = pw.matmul(g.a)
    nb = 2
    b = pw.b_packed.view(N, nb * bs // 2).clone()
    b[:, K // 2:] = 0xFF                        # every pad nibble set to 15
    zp = pw.zp_packed.clone()                   # nb = 2: no zero-point pad nibble
    y1 = mnb.PackedWeight(K, N, bs, torch.float32, b.view(-1).contiguous(), pw.scales, zp,
                          pw.bias).matmul(g.a)
    assert torch.equal(y0, y1)
    # odd number of blocks: the pad nibble of the zero-point row
    K3 = 150
    _, g3 = _inputs(K3, N, M, bs, "f32", True, False, seed=5)
    p3 = _packed(g3, bs)
    z3 = p3.zp_packed.view(N, 2).clone()
    z3[:, 1] |= 0xF0
    y3a = p3.matmul(g3.a)
    y3b = mnb.PackedWeight(K3, N, bs, torch.float32, p3.b_packed, p3.scales,
                           z3.view(-1).contiguous()).matmul(g3.a)
    assert torch.equal(y3a, y3b)


@pytest.mark.parametrize("M", [1, 48])
def test_default_zero_point_equals_explicit_eight(M):
    K, N, bs = 700, 90, 32
    _, g = _inputs(K, N, M, bs, "f32", False, True, seed=6)
    y0 = _packed(g, bs).matmul(g.a)
    z8 = torch.full((N, -(-K // bs)), 8, dtype=torch.uint8, device=DEV)
    y8 = mnb.PackedWeight.from_logical(g.q, g.scales, z8, g.bias, block_size=bs).matmul(g.a)
    assert torch.equal(y0, y8)


@pytest.mark.parametrize("M", [1, 96])
def test_deterministic(M):
    K, N, bs = 2048, 1024, 32
    _, g = _inputs(K, N, M, bs, "f32", True, True, seed=8)
    pw = _packed(g, bs)
    y0 = pw.matmul(g.a).clone()
    for _ in range(3):
        assert torch.equal(pw.matmul(g.a), y0)


def test_scaling_by_powers_of_two_is_exact():
    K, N, bs = 512, 64, 32
    _, g = _inputs(K, N, 1, bs, "f32", True, False, seed=9)
    y = _packed(g, bs).matmul(g.a)
    y2 = _packed(g, bs).matmul(g.a * 4.0)
    assert torch.equal(y2, y * 4.0)
    ys = mnb.PackedWeight.from_logical(g.q, g.scales * 0.5, g.zp, block_size=bs).matmul(g.a)
    assert torch.equal(ys, y * 0.5)


def test_unaligned_view_is_rejected():
    K, N, bs = 64, 8, 32
    _, g = _inputs(K, N, 1, bs, "f32", False, False, seed=1)
    pw = _packed(g, bs)
    big = torch.zeros(K + 1, device=DEV)
    with pytest.raises(mnb.MnbError) as e:
        mnb.gemv(big[1:].view(1, K), pw.b_packed, pw.scales, K=K, N=N, block_size=bs)
    assert e.value.status == -3


@pytest.mark.parametrize("K,N,bs,zp", [(256, 300, 128, True), (160, 70, 32, False),
                                       (48, 33, 16, True), (80, 17, 16, False)])
def test_bf16_gemm_identity_returns_bf16_dequant(orc, K, N, bs, zp):
    """With bfloat16 activations the prefill kernel multiplies the bf16
    rounding of the exact weight: A = I_K must return exactly the bf16
    dequantization (itself checked bit-exactly against the oracle)."""
    inp, g = _inputs(K, N, 1, bs, "bf16", zp, False, seed=K + N)
    pw = _packed(g, bs)
    w16 = mnb.dequant(pw.b_packed, pw.scales, pw.zp_packed, K=K, N=N, block_size=bs,
                      act_dtype=torch.bfloat16, out_kind=mnb.DEQUANT_BF16)
    w_exact = orc.dequant(inp.q.numpy(), None if inp.zp is None else inp.zp.numpy(),
                          act_np(inp.scales), bs)
    assert np.array_equal(act_np(w16), orc.round_to_bf16(w_exact))
    eye = torch.eye(K, device=DEV, dtype=torch.bfloat16)
    y = mnb.gemm(eye, pw.b_packed, pw.scales, pw.zp_packed, K=K, N=N, block_size=bs)
    assert np.array_equal(act_np(y), act_np(w16).T)


@pytest.mark.parametrize("M,K,N,bs,zp,bias", [(1000, 192, 24676, 64, True, True),
                                              (2048, 128, 12288, 128, False, False),
                                              (1030, 320, 24600, 32, True, False)])
def test_bf16_gemm_large_grid_sampled(orc, M, K, N, bs, zp, bias):
    """bfloat16, more than 128 rows, K a multiple of 64 and of the block size:
    the 256 x 256 x 64 wide kernel over many rounds of tiles (no K split);
    ragged M and N, an odd number of K steps; sampled rows x columns against
    the oracle."""
    log(f"large bf16 gemm M={M} K={K} N={N} bs={bs} zp={zp} bias={bias}")
    inp, g = _inputs(K, N, M, bs, "bf16", zp, bias, seed=M + K + N)
    pw = _packed(g, bs)
    y = mnb.gemm(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=N, block_size=bs)
    rng = np.random.default_rng(M)
    rows = sorted({0, M - 1, 255, 256, *rng.choice(M, 12, replace=False).tolist()})
    cols = sorted({0, N - 1, 255, 256, N - 257, *rng.choice(N, 40, replace=False).tolist()})
    y_ref, S = oracle_ref(orc, inp, rows, cols)
    ys = y[torch.as_tensor(rows, device=DEV)][:, torch.as_tensor(cols, device=DEV)]
    assert_close(out_f64(ys), y_ref, S, "bf16", f"M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,bs,zp,bias", [(64, 2560, 151936, 128, True, True),
                                              (17, 1024, 98305, 32, False, True),
                                              (300, 1056, 49200, 32, True, False)])
def test_bf16_gemm_128_tiles_wide_n_sampled(orc, M, K, N, bs, zp, bias):
    """bfloat16 products the wide kernel does not take -- 17..128 rows (a
    64-token prefill through the 151,936-column LM head), or K not a multiple
    of 64 (K = 1056) -- run on the 128 x 128 tile kernel however many tiles
    the grid has.  Random weights, zero points and bias; all rows of the
    short products, sampled rows otherwise, x sampled columns including the
    ragged last tile, against the oracle."""
    log(f"bf16 128-tile gemm M={M} K={K} N={N} bs={bs} zp={zp} bias={bias}")
    inp, g = _inputs(K, N, M, bs, "bf16", zp, bias, seed=M * 5 + K + N)
    pw = _packed(g, bs)
    y = mnb.gemm(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=N, block_size=bs)
    rng = np.random.default_rng(M + 1)
    rows = list(range(M)) if M <= 64 else sorted({0, M - 1, 127, 128, *rng.choice(M, 10, replace=False).tolist()})
    last = (N - 1) // 128 * 128
    cols = sorted({0, 127, 128, last - 1, *range(last, N), *rng.choice(N, 48, replace=False).tolist()})
    y_ref, S = oracle_ref(orc, inp, rows, cols)
    ys = y[torch.as_tensor(rows, device=DEV)][:, torch.as_tensor(cols, device=DEV)]
    assert_close(out_f64(ys), y_ref, S, "bf16", f"M={M} K={K} N={N}")


@pytest.mark.parametrize("zp,bias", [(True, True), (False, False)])
def test_bf16_gemm_tail_split_matches_oracle(orc, zp, bias):
    """Whole rounds of 256x256 tiles run unsplit; when the last round would
    leave more than half of the CUs idle, its tiles are split along K and
    their partials reduced separately.  M = 512, N = 38400: 300 tiles, the
    last 44 (columns 32768..38399 on a 256-CU device) in the split tail.
    Sampled columns on both sides of the boundary, all rows; run twice,
    bit-identical."""
    M, K, N, bs = 512, 1024, 38400, 128
    inp, g = _inputs(K, N, M, bs, "bf16", zp, bias, seed=31)
    pw = _packed(g, bs)
    y = mnb.gemm(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=N, block_size=bs)
    y2 = mnb.gemm(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=N, block_size=bs)
    assert torch.equal(y, y2)
    rng = np.random.default_rng(5)
    cols = np.unique(np.concatenate([rng.integers(0, 32768, 48), rng.integers(32768, N, 80),
                                     [0, 32767, 32768, N - 1]]))
    y_ref, S = oracle_ref(orc, inp, cols=cols)
    assert_close(out_f64(y[:, torch.as_tensor(cols, device=DEV)]), y_ref, S, "bf16", "tail split")


SPLIT_CASES = [
    ("bf16", 512, 4096, 384, 128, True, True),    # 4 tiles of 256x256: 16 K splits
    ("bf16", 300, 1536, 520, 32, False, False),   # ragged M and N: 6 splits
    ("f32", 256, 2048, 256, 32, True, True),      # 16 tiles of 64x64: 4 splits
    ("f32", 200, 1024, 136, 16, True, False),     # block 16, ragged: 4 splits
]


@pytest.mark.parametrize("dt,M,K,N,bs,zp,bias", SPLIT_CASES)
def test_split_k_gemm_matches_oracle(orc, dt, M, K, N, bs, zp, bias):
    """Few output tiles: K is split across workgroups and the float32
    partials (in the caller's workspace) are added in split order (+ bias);
    every output against the oracle, twice (the second call reuses the same
    workspace, left holding the first call's partials)."""
    log(f"split-K gemm {dt} M={M} K={K} N={N} bs={bs} zp={zp} bias={bias}")
    inp, g = _inputs(K, N, M, bs, dt, zp, bias, seed=M * 3 + K + N)
    pw = _packed(g, bs)
    need = mnb.workspace_bytes(pw.desc, M)
    assert need > 0
    ws = mnb.workspace(need)
    y_ref, S = oracle_ref(orc, inp)
    y1 = pw.matmul(g.a, workspace=ws).clone()
    y2 = pw.matmul(g.a, workspace=ws)
    assert_close(out_f64(y1), y_ref, S, dt, f"{dt} M={M} K={K} N={N}")
    assert torch.equal(y1, y2)


def test_split_k_captured_in_callers_graph_before_any_eager_call():
    """A split product whose first call ever is inside a graph the caller
    captures (torch.cuda.graph, workspace from the caller) gives the bits of
    the same product run eagerly afterwards, on every replay, with eager
    work between the replays."""
    dt, M, K, N, bs, zp, bias = "f32", 192, 3072, 200, 32, True, True
    _, g = _inputs(K, N, M, bs, dt, zp, bias, seed=77)
    pw = _packed(g, bs)
    ws_graph = mnb.workspace(mnb.workspace_bytes(pw.desc, M))
    y = torch.empty(M, N, device=DEV)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        pw.matmul(g.a, out=y, workspace=ws_graph)
    ws_eager = mnb.workspace(mnb.workspace_bytes(pw.desc, M))
    replays = []
    for rep in range(3):
        y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        replays.append(y.clone())
        pw.matmul(g.a, workspace=ws_eager)       # eager work between replays
        torch.cuda.synchronize()
    eager = pw.matmul(g.a, workspace=ws_eager)
    for rep, r in enumerate(replays):
        assert torch.equal(r, eager), rep


def test_split_k_graph_matches_direct():
    """A captured sequence of split products (the sequence's graph
    workspace) gives the bits of the same products run directly (its eager
    workspace), on every replay."""
    items = []
    for i, (dt, M, K, N, bs, zp, bias) in enumerate(SPLIT_CASES):
        _, g = _inputs(K, N, M, bs, dt, zp, bias, seed=100 + i)
        pw = _packed(g, bs)
        items.append((pw, g.a, torch.empty(M, N, device=DEV, dtype=g.a.dtype)))
    seq = mnb.Sequence(items)
    seq.run()
    direct = [y.clone() for _, _, y in items]
    for _, _, y in items:
        y.fill_(float("nan"))
    seq.capture()
    try:
        for rep in range(3):
            seq.replay()
            torch.cuda.synchronize()
            for (_, _, y), d in zip(items, direct):
                assert torch.equal(y, d), rep
            for _, _, y in items:
                y.fill_(float("nan"))
    finally:
        seq.close()


# ---------------------------------------------------------------------------
# small M (1 <= M <= 16, K % 32 == 0, block_size >= 32): matrix-core kernel
# ---------------------------------------------------------------------------

# 2..4 rows through the decode GEMV with split-K wavefront teams (W = 2 or 4
# wavefronts per column): K beyond one wavefront's 64 lanes x 4 / MR chunks.
ROW_TEAM_CASES = [  # (M, K, dt)
    (3, 2560, "f32"), (4, 2560, "f32"), (3, 3072, "f32"), (4, 3072, "f32"),
    (3, 4096, "f32"), (4, 4096, "f32"), (2, 6144, "f32"), (2, 8192, "f32"),
    (3, 2560, "bf16"), (4, 3072, "bf16"), (4, 4096, "bf16"), (4, 8192, "bf16"),
    (2, 16384, "bf16"),
]


@pytest.mark.parametrize("M,K,dt", ROW_TEAM_CASES)
def test_row_gemv_split_k_teams_random_weights(orc, M, K, dt):
    """Random weights, zero points, scales and bias (on and off) through the
    2-4-row GEMV where a column takes a team of several wavefronts (their
    partial sums meet in LDS per row): every output of a ragged N against
    the oracle, for block sizes 32 and 128."""
    worst = 0.0
    for bs, zp, bias in ((32, True, True), (128, False, False), (128, True, False)):
        N = 257
        log(f"row-team gemv {dt} M={M} K={K} N={N} bs={bs} zp={zp} bias={bias}")
        inp, g = _inputs(K, N, M, bs, dt, zp, bias, seed=M * 1000 + K + bs)
        pw = _packed(g, bs)
        assert mnb.workspace_bytes(pw.desc, M) == 0
        y = mnb.gemm(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=N, block_size=bs)
        y_ref, S = oracle_ref(orc, inp)
        worst = max(worst, assert_close(out_f64(y), y_ref, S, dt, f"M={M} K={K} bs={bs}"))
        # each row alone through the decode GEMV: same tolerance, and the
        # rows do not disturb one another (a row of zeros gives the bias)
        a0 = g.a.clone()
        a0[1:] = 0
        y0 = mnb.gemm(a0, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=N, block_size=bs)
        want = torch.zeros(N, device=DEV) if pw.bias is None else pw.bias
        for r in range(1, M):
            assert torch.equal(y0[r].float(), want.to(y0.dtype).float()), r
    log(f"row-team gemv {dt} M={M} K={K}: worst err/tol {worst:.3g}")


SMALL_M_CASES = [  # (M, K, N): ragged N, K not a multiple of the 128-value span
    (1, 32, 1), (2, 64, 17), (3, 96, 33), (4, 1024, 4096), (5, 160, 100),
    (8, 2048, 1024), (15, 3072, 130), (16, 1024, 515), (16, 128, 16), (7, 2560, 260),
    (9, 9728, 40), (12, 4096, 2049), (6, 224, 31),
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [32, 64, 128, 256])
def test_small_m_parity_sweep(orc, dt, bs):
    rng = np.random.default_rng(300 + bs)
    worst = 0.0
    for M, K, N in SMALL_M_CASES:
        zp, bias = bool(rng.integers(2)), bool(rng.integers(2))
        log(f"small-M {dt} bs={bs} M={M} K={K} N={N} zp={zp} bias={bias}")
        inp, g = _inputs(K, N, M, bs, dt, zp, bias, seed=M * 11 + K * 3 + N)
        pw = _packed(g, bs)
        y = mnb.gemm(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=N,
                     block_size=bs)
        y_ref, S = oracle_ref(orc, inp)
        worst = max(worst, assert_close(out_f64(y), y_ref, S, dt, f"M={M} K={K} N={N}"))
    log(f"small-M {dt} bs={bs}: worst err/tol {worst:.3g}")


@pytest.mark.parametrize("dt,M,K,N,bs,zp,bias", [("f32", 10, 3072, 12000, 64, True, True),
                                                  ("bf16", 16, 5120, 12000, 128, False, True)])
def test_small_m_passes_with_several_sets_per_workgroup(orc, dt, M, K, N, bs, zp, bias):
    """K longer than one staged pass and more column sets than resident
    workgroups: a workgroup stages every pass again for each further set.
    Sampled columns against the oracle, and a slice of the columns launched
    alone (where each is in a workgroup's first set) bit-identical."""
    log(f"small-M passes {dt} M={M} K={K} N={N} bs={bs}")
    inp, g = _inputs(K, N, M, bs, dt, zp, bias, seed=K + N + M)
    y = _packed(g, bs).matmul(g.a)
    rng = np.random.default_rng(K)
    cols = sorted({0, 16 * 300 + 5, N - 1, *map(int, rng.choice(N, size=40, replace=False))})
    y_ref, S = oracle_ref(orc, inp, cols=cols)
    assert_close(out_f64(y[:, torch.as_tensor(cols, device=DEV)]), y_ref, S, dt, f"M={M} K={K} N={N}")
    lo, hi = 16 * 700, 16 * 700 + 48
    part = mnb.PackedWeight.from_logical(g.q[lo:hi], g.scales[lo:hi], None if g.zp is None else g.zp[lo:hi],
                                         None if g.bias is None else g.bias[lo:hi], block_size=bs)
    assert torch.equal(part.matmul(g.a), y[:, lo:hi])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M", [2, 16])
def test_small_m_exact_arithmetic_bit_exact(orc, dt, M):
    for K, N, bs in [(1024, 70, 32), (2560, 33, 128), (352, 17, 64)]:
        log(f"small-M exact {dt} M={M} K={K} N={N} bs={bs}")
        q, zp, sc, a, bias = _exact_case(K, N, M, bs, dt, seed=K + 3 * M)
        pw = mnb.PackedWeight.from_logical(q.to(DEV), sc.to(DEV), zp.to(DEV), bias.to(DEV),
                                           block_size=bs)
        y = pw.matmul(a.to(DEV))
        y_ref, _ = orc.matmul(act_np(a), q.numpy(), zp.numpy(), act_np(sc), bs,
                              bias=bias.numpy())
        if dt == "f32":
            assert np.array_equal(y.cpu().numpy(), orc.round_to_f32(y_ref)), (K, N, M)
        else:
            assert np.array_equal(act_np(y), orc.round_to_bf16(y_ref)), (K, N, M)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_small_m_identity_rows_return_dequantized_weights(orc, dt):
    """A = the first 16 rows of I_K: row m of Y is column m of dequant(B),
    rounded once (float32, or bfloat16 for bfloat16 activations)."""
    K, N, bs = 160, 45, 32
    inp, g = _inputs(K, N, 1, bs, dt, True, False, seed=12)
    pw = _packed(g, bs)
    w = orc.dequant(inp.q.numpy(), inp.zp.numpy(), act_np(inp.scales), bs)   # [N][K] exact
    eye = torch.eye(K, device=DEV)[:16]
    if dt == "bf16":
        eye = eye.to(torch.bfloat16)
    y = mnb.gemm(eye, pw.b_packed, pw.scales, pw.zp_packed, K=K, N=N, block_size=bs)
    want = orc.round_to_f32(w) if dt == "f32" else orc.round_to_bf16(w)
    got = y.cpu().numpy() if dt == "f32" else act_np(y)
    assert np.array_equal(got, want[:, :16].T)


@pytest.mark.parametrize("M", [4, 16])
def test_small_m_fused_launch_bit_identical_to_separate(M):
    for K, bs, dt in [(1024, 32, "f32"), (2560, 128, "f32"), (2560, 128, "bf16")]:
        log(f"small-M fusion M={M} K={K} bs={bs} {dt}")
        _, g1 = _inputs(K, 300, M, bs, dt, True, False, seed=21)
        _, g2 = _inputs(K, 1700, M, bs, dt, True, False, seed=22)
        p1, p2 = _packed(g1, bs), _packed(g2, bs)
        a = g1.a
        q = torch.cat([g1.q, g2.q])
        fused = mnb.PackedWeight.from_logical(q, torch.cat([g1.scales, g2.scales]),
                                              torch.cat([g1.zp, g2.zp]), block_size=bs)
        assert torch.equal(fused.matmul(a), torch.cat([p1.matmul(a), p2.matmul(a)], 1))
