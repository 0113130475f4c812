"""RMSNorm fused into the decode projection's input (mnb_gemv_rmsnorm)
against the oracle: a = x / sqrt(mean(x^2) + eps) * gamma in binary64, then
y = a x dequant(B) + bias, within the method's tolerance taken with the exact
normalized activations; exact invariants: scaling x by a power of two with
eps = 0 leaves y bit-identical, and a zero row gives exactly the bias."""

import numpy as np
import pytest
import torch

import weight_only_int4_matmulnbits_amd as mnb
from parity import REL, ATOL, act_np, log, out_f64
from workloads.generate import random_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gamma(K, dt, seed):
    g = torch.from_numpy(np.random.default_rng(seed).uniform(0.5, 1.5, K).astype(np.float32))
    return g if dt == "f32" else g.to(torch.bfloat16)


@pytest.mark.parametrize("K,N,bs,dt,zp,bias", [
    (1024, 4096, 32, "f32", True, False),      # Qwen3-0.6B qkv
    (2560, 6144, 128, "f32", False, False),    # Qwen3-4B qkv
    (2560, 19456, 128, "bf16", True, True),    # Qwen3-4B gate||up
    (12288, 65, 128, "bf16", True, True),      # two-wavefront teams
    (96, 33, 32, "f32", False, True),
])
def test_gemv_rmsnorm_matches_oracle(orc, K, N, bs, dt, zp, bias):
    log(f"rmsnorm gemv {dt} K={K} N={N} bs={bs} zp={zp} bias={bias}")
    inp = random_inputs(K, N, 1, bs, dt, zp, bias, seed=K + N)
    x = (inp.a.float() * 5.0).to(inp.a.dtype)
    gamma = _gamma(K, dt, K)
    eps = 1e-6
    g = inp.to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs)
    y = mnb.gemv_rmsnorm(x.to(DEV), gamma.to(DEV), eps, pw.b_packed, pw.scales, pw.zp_packed, pw.bias,
                         K=K, N=N, block_size=bs)
    a = orc.rmsnorm(act_np(x), act_np(gamma), eps)
    y_ref, S = orc.matmul_f64a(a, inp.q.numpy(), None if inp.zp is None else inp.zp.numpy(),
                               act_np(inp.scales), bs, None if inp.bias is None else inp.bias.numpy())
    err = np.abs(out_f64(y) - y_ref)
    tol = REL[dt] * S + ATOL
    worst = float((err / tol).max())
    log(f"  worst err/tol {worst:.3g}")
    assert np.isfinite(out_f64(y)).all() and worst <= 1.0


def test_gemv_rmsnorm_exact_invariants():
    K, N, bs = 2560, 300, 128
    inp = random_inputs(K, N, 1, bs, "f32", True, True, seed=8)
    g = inp.to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs)
    gamma = _gamma(K, "f32", 3).to(DEV)
    kw = dict(K=K, N=N, block_size=bs)
    y1 = mnb.gemv_rmsnorm(g.a, gamma, 0.0, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, **kw)
    y4 = mnb.gemv_rmsnorm(g.a * 4.0, gamma, 0.0, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, **kw)
    assert torch.equal(y1, y4)
    z = mnb.gemv_rmsnorm(torch.zeros_like(g.a), gamma, 1e-6, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, **kw)
    assert torch.equal(z[0], pw.bias)


@pytest.mark.parametrize("K,N,bs,dt", [(2560, 131072 + 37, 128, "f32"), (4096, 40000, 64, "bf16")])
def test_wide_rmsnorm_gemv_bit_identical_to_narrow_launches(K, N, bs, dt):
    """The columns of a wide launch (teams walking many column groups, grids
    past the resident workgroups) have the bits of the same columns in
    narrow launches: the normalization and the summation order depend on
    (K, block_size) only."""
    log(f"wide vs narrow rmsnorm gemv {dt} K={K} N={N} bs={bs}")
    inp = random_inputs(K, N, 1, bs, dt, True, False, seed=K + 3)
    g = inp.to(DEV)
    gamma = _gamma(K, dt, K + 1).to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, None, block_size=bs)
    y = mnb.gemv_rmsnorm(g.a, gamma, 1e-6, pw.b_packed, pw.scales, pw.zp_packed, None, K=K, N=N, block_size=bs)
    for lo, hi in [(0, 1000), (N - 517, N)]:
        part = mnb.PackedWeight.from_logical(g.q[lo:hi], g.scales[lo:hi], g.zp[lo:hi], None, block_size=bs)
        yp = mnb.gemv_rmsnorm(g.a, gamma, 1e-6, part.b_packed, part.scales, part.zp_packed, None,
                              K=K, N=hi - lo, block_size=bs)
        assert torch.equal(yp, y[:, lo:hi]), (lo, hi)
