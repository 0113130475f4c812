"""GPU parity of the import, vocabulary and epilogue entry points against the
CPU oracle, through the C ABI.

Bit-exact: QDQ normalization (every byte of the three outputs), the tied
embedding gather, greedy ArgMax decided on the same values.  Within
tolerance: matmuls on imported weights against DequantizeLinear evaluated on
the QDQ tensors, the LM head over the full vocabulary (N = 151936, a ragged
last column group), the fused gate||up SiLU product.
"""

import numpy as np
import pytest
import torch

import weight_only_int4_matmulnbits_amd as mnb
from parity import ATOL, REL, act_np, assert_close, log, oracle_ref, out_f64
from workloads.generate import random_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _qdq_case(K, N, bs, dt, has_zp, seed):
    """Random QDQ tensors (flat packed uint4 streams, scales in the axis's
    shape are [nb*N] here and reshaped by the caller as needed)."""
    g = torch.Generator().manual_seed(seed)
    nb = -(-K // bs)
    w_q = torch.randint(0, 256, ((K * N + 1) // 2,), dtype=torch.uint8, generator=g)
    zp_q = torch.randint(0, 256, ((nb * N + 1) // 2,), dtype=torch.uint8, generator=g) if has_zp else None
    sc = torch.rand(nb * N, generator=g) * 0.02 + 0.005
    if dt == "bf16":
        sc = sc.to(torch.bfloat16)
    return w_q, zp_q, sc


def _np(t):
    return None if t is None else act_np(t)


# ---------------------------------------------------------------------------
# QDQ import
# ---------------------------------------------------------------------------

QDQ_SHAPES = [(3, 2, 16), (20, 2, 16), (37, 5, 16), (100, 33, 32), (64, 7, 32), (1000, 63, 128),
              (2560, 40, 128), (257, 129, 256), (1024, 3072, 32)]


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_qdq_import_bytes_match_oracle(orc, axis, dt):
    for i, (K, N, bs) in enumerate(QDQ_SHAPES):
        for has_zp in (True, False):
            log(f"qdq import axis={axis} {dt} K={K} N={N} bs={bs} zp={has_zp}")
            w_q, zp_q, sc = _qdq_case(K, N, bs, dt, has_zp, seed=100 * i + has_zp)
            b, s, z = mnb.import_qdq(w_q.to(DEV), sc.to(DEV), None if zp_q is None else zp_q.to(DEV),
                                     K=K, N=N, block_size=bs, axis=axis)
            rb, rs, rz = orc.qdq_import(w_q.numpy(), _np(zp_q), act_np(sc), K, N, bs, axis)
            assert np.array_equal(b.cpu().numpy(), rb), (K, N, bs)
            assert np.array_equal(act_np(s), rs), (K, N, bs)
            assert np.array_equal(z.cpu().numpy(), rz), (K, N, bs)


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M", [1, 5, 200])
def test_matmul_on_imported_weights_matches_dequantize_linear(orc, axis, dt, M):
    """Y = A x DequantizeLinear(W_qdq) with the dequantization evaluated by the
    oracle directly on the QDQ layout."""
    for K, N, bs, has_zp in [(1024, 96, 32, True), (1000, 70, 64, False), (2560, 33, 128, True)]:
        log(f"qdq matmul axis={axis} {dt} M={M} K={K} N={N} bs={bs} zp={has_zp}")
        w_q, zp_q, sc = _qdq_case(K, N, bs, dt, has_zp, seed=K + N + M)
        b, s, z = mnb.import_qdq(w_q.to(DEV), sc.to(DEV), None if zp_q is None else zp_q.to(DEV),
                                 K=K, N=N, block_size=bs, axis=axis)
        a = torch.randn(M, K, generator=torch.Generator().manual_seed(M + K))
        if dt == "bf16":
            a = a.to(torch.bfloat16)
        pw = mnb.PackedWeight(K, N, bs, a.dtype, b, s, z, None)
        y = pw.matmul(a.to(DEV))
        w = orc.qdq_dequant(w_q.numpy(), _np(zp_q), act_np(sc), K, N, bs, axis)   # [K][N] exact
        a64 = a.double().numpy()
        y_ref = a64 @ w
        S = np.abs(a64) @ np.abs(w)
        assert_close(out_f64(y), y_ref, S, dt, f"axis={axis} M={M} K={K} N={N}")


def test_tied_weight_serves_directly_when_native(orc):
    """Whole blocks and an even block count: the axis-1 QDQ tensors are used by
    the LM-head GEMV and the gather as they are, with no copy, bit-identically
    to the imported copy."""
    K, N, bs = 1024, 1000, 32
    assert mnb.qdq_is_native(K, N, bs, axis=1)
    w_q, zp_q, sc = _qdq_case(K, N, bs, "f32", True, seed=5)
    w_d, z_d, s_d = w_q.to(DEV), zp_q.to(DEV), sc.to(DEV).view(N, K // bs)
    b, s, z = mnb.import_qdq(w_d, s_d, z_d, K=K, N=N, block_size=bs, axis=1)
    assert torch.equal(b, w_d) and torch.equal(z, z_d) and torch.equal(s, s_d)
    a = torch.randn(1, K, device=DEV)
    y_direct = mnb.gemv(a, w_d, s_d, z_d, K=K, N=N, block_size=bs)
    assert torch.equal(y_direct, mnb.gemv(a, b, s, z, K=K, N=N, block_size=bs))
    ids = torch.tensor([0, 999, 17], device=DEV)
    rows = mnb.gather_rows(ids, w_d, s_d, z_d, K=K, N=N, block_size=bs)
    w = orc.qdq_dequant(w_q.numpy(), zp_q.numpy(), act_np(sc), K, N, bs, 1)   # [K][N]
    assert np.array_equal(rows.cpu().numpy(), orc.round_to_f32(w[:, [0, 999, 17]].T))


# ---------------------------------------------------------------------------
# tied embedding gather
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("K,N,bs,zp", [(1024, 500, 32, True), (100, 37, 64, False), (33, 9, 16, True),
                                       (2560, 300, 128, False)])
def test_gather_rows_bit_exact(orc, dt, K, N, bs, zp):
    inp = random_inputs(K, N, 1, bs, dt, zp, False, seed=K + N)
    g = inp.to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, block_size=bs)
    ids = [0, N - 1, 3 % N, -1, -N, 3 % N, N, -N - 1, 1 << 40]
    out = mnb.gather_rows(torch.tensor(ids, device=DEV), pw.b_packed, pw.scales, pw.zp_packed,
                          K=K, N=N, block_size=bs)
    w = orc.dequant(inp.q.numpy(), None if inp.zp is None else inp.zp.numpy(), act_np(inp.scales), bs)
    want = orc.round_to_f32(w) if dt == "f32" else orc.round_to_bf16(w)
    got = out.cpu().numpy() if dt == "f32" else act_np(out)
    for t, v in enumerate(ids):
        if -N <= v < N:
            assert np.array_equal(got[t], want[v % N]), (t, v)
        else:
            assert np.isnan(out[t].float().cpu().numpy()).all(), (t, v)


# ---------------------------------------------------------------------------
# greedy ArgMax and the LM head over the full vocabulary
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_argmax_matches_oracle(orc, dt):
    g = torch.Generator().manual_seed(7)
    for M, N in [(1, 1), (1, 151936), (3, 1000), (7, 1025), (2, 4096)]:
        x = torch.randint(-20, 21, (M, N), generator=g).float()     # many ties
        if N > 10:
            x[0, N // 2] = float("nan") if M > 2 else x[0, N // 2]
            x[-1, 5] = 1e6
        if dt == "bf16":
            x = x.to(torch.bfloat16)
        idx = mnb.argmax(x.to(DEV))
        assert idx.cpu().tolist() == orc.argmax(act_np(x)).tolist(), (M, N)
    # the first NaN wins, an all -inf row gives 0
    x = torch.tensor([[1.0, float("nan"), 5.0, float("nan")], [float("-inf")] * 4])
    if dt == "bf16":
        x = x.to(torch.bfloat16)
    assert mnb.argmax(x.to(DEV)).cpu().tolist() == [1, 0]


@pytest.mark.parametrize("dt,bs,K", [("f32", 32, 1024), ("bf16", 128, 2560)])
def test_lm_head_full_vocabulary_and_greedy_token(orc, dt, bs, K):
    """The tied weight as the LM head at N = 151936 (the last column group is
    partial), then the greedy token; and the same storage as the embedding."""
    N = 151936
    log(f"LM head {dt} K={K} N={N}")
    inp = random_inputs(K, N, 1, bs, dt, True, False, seed=11)
    g = inp.to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, block_size=bs)
    logits = pw.matmul(g.a)
    y_ref, S = oracle_ref(orc, inp)
    assert_close(out_f64(logits), y_ref, S, dt, "LM head")
    tok = int(mnb.argmax(logits)[0])
    # the decision taken on the GPU's own logits equals the oracle's decision
    # on those same values, and is a maximum of the exact logits within their
    # tolerance
    assert tok == int(orc.argmax(act_np(logits))[0])
    tol = REL[dt] * S[0] + ATOL
    assert y_ref[0, tok] >= y_ref[0].max() - tol[tok] - tol[int(np.argmax(y_ref[0]))]
    rows = mnb.gather_rows(torch.tensor([tok, N - 1], device=DEV), pw.b_packed, pw.scales,
                           pw.zp_packed, K=K, N=N, block_size=bs)
    w = orc.dequant(inp.q[[tok, N - 1]].numpy(), inp.zp[[tok, N - 1]].numpy(),
                    act_np(inp.scales[[tok, N - 1]]), bs)
    want = orc.round_to_f32(w) if dt == "f32" else orc.round_to_bf16(w)
    assert np.array_equal(rows.cpu().numpy() if dt == "f32" else act_np(rows), want)


# ---------------------------------------------------------------------------
# gate||up with the SiLU-gated product fused into the epilogue
# ---------------------------------------------------------------------------

def _silu_tol(dt, g_ref, u_ref, Sg, Su, h_ref):
    """Tolerance of h = silu(g) * u from those of g and u: |silu'| <= 1.1, the
    float32 evaluation (a few ulps), and the bfloat16 output rounding."""
    tg, tu = REL[dt] * Sg + ATOL, REL[dt] * Su + ATOL
    sil = g_ref / (1 + np.exp(-g_ref))
    t = 1.1 * np.abs(u_ref) * tg + np.abs(sil) * tu + 2.0 ** -20 * np.abs(h_ref) + ATOL
    if dt == "bf16":
        t += 2.0 ** -8 * np.abs(h_ref)
    return t


@pytest.mark.parametrize("dt,K,I,bs,zp,bias", [("f32", 1024, 3072, 32, True, False),
                                               ("bf16", 2560, 9728, 128, False, False),
                                               ("f32", 2560, 9728, 128, False, True),   # five chunks per lane
                                               ("f32", 1000, 333, 64, True, True),
                                               ("bf16", 96, 17, 16, True, True),
                                               ("f32", 8192, 40, 32, False, True),
                                               ("f32", 9728, 200, 128, True, False),
                                               ("f32", 12288, 64, 128, True, True),     # 2-wavefront teams
                                               ("bf16", 16384, 33, 32, False, True)])   # 2-wavefront teams
def test_gemv_silu_mul_matches_oracle(orc, dt, K, I, bs, zp, bias):
    log(f"silu gemv {dt} K={K} I={I} bs={bs} zp={zp} bias={bias}")
    inp = random_inputs(K, 2 * I, 1, bs, dt, zp, bias, seed=K + I)
    g = inp.to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs)
    h = mnb.gemv_silu_mul(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=2 * I,
                          block_size=bs)
    y_ref, S = oracle_ref(orc, inp)
    h_ref = orc.silu_mul(y_ref[0, :I], y_ref[0, I:])
    tol = _silu_tol(dt, y_ref[0, :I], y_ref[0, I:], S[0, :I], S[0, I:], h_ref)
    err = np.abs(out_f64(h)[0] - h_ref)
    assert np.isfinite(out_f64(h)).all()
    worst = float((err / tol).max())
    log(f"  worst err/tol {worst:.3g}")
    assert worst <= 1.0
    # run to run identical
    assert torch.equal(h, mnb.gemv_silu_mul(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias,
                                            K=K, N=2 * I, block_size=bs))


def test_gemv_silu_mul_beyond_register_kernel_is_refused():
    """K past mnb_gemv_max_k (the decode kernel's limit) is refused; every
    K up to it, split-K wavefront teams included, is served."""
    K, I, bs = 20000, 16, 128
    inp = random_inputs(K, 2 * I, 1, bs, "f32", False, False, seed=3)
    g = inp.to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, None, block_size=bs)
    assert K > mnb.gemv_max_k(pw.desc)
    with pytest.raises(mnb.MnbError) as e:
        mnb.gemv_silu_mul(g.a, pw.b_packed, pw.scales, K=K, N=2 * I, block_size=bs)
    assert e.value.status == -2
