"""The gated gate||up projection for any M (mnb_gemm_silu_mul) against the
oracle: h = silu(y_gate) * y_up with y = A x dequant(B) + bias, within the
tolerance derived from those of y_gate and y_up (|silu'| <= 1.1, the float32
evaluation and, for bfloat16, the output rounding).  Routes covered: the
prefill kernel with the gated epilogue (the Qwen3-4B prefill gate||up shape,
including its split last round of tiles; a ragged shape that takes direct
stores), the unfused standard path (float32 activations; bfloat16 with at most
128 rows), and one row through the gated decode GEMV."""

import numpy as np
import pytest
import torch

import weight_only_int4_matmulnbits_amd as mnb
from parity import log, oracle_ref, out_f64
from test_gpu_vocab import _silu_tol
from workloads.generate import random_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(orc, inp, h, I, rows, hcols):
    cols = np.concatenate([hcols, np.asarray(hcols) + I])
    y_ref, S = oracle_ref(orc, inp, rows, cols)
    k = len(hcols)
    g_ref, u_ref = y_ref[:, :k], y_ref[:, k:]
    h_ref = orc.silu_mul(g_ref, u_ref)
    tol = _silu_tol(inp.act_dtype, g_ref, u_ref, S[:, :k], S[:, k:], h_ref)
    hs = h if rows is None else h[torch.as_tensor(rows, device=DEV)]
    hs = hs[:, torch.as_tensor(hcols, device=DEV)]
    got = out_f64(hs)
    assert np.isfinite(got).all()
    worst = float((np.abs(got - h_ref) / tol).max())
    log(f"  worst err/tol {worst:.3g}")
    assert worst <= 1.0
    return worst


@pytest.mark.parametrize("zp,bias", [(True, True), (False, False)])
def test_gated_prefill_qwen3_4b_shape(orc, zp, bias):
    """M = 2048 bf16 rows through the 2560 -> 2 x 9728 gate||up weight: 608
    tiles, the last 96 (h columns 8192 .. 9727) split along K and reduced by
    the gated tail kernel; sampled rows x columns on both sides."""
    M, K, I, bs = 2048, 2560, 9728, 128
    log(f"gated prefill M={M} K={K} I={I} zp={zp} bias={bias}")
    inp = random_inputs(K, 2 * I, M, bs, "bf16", zp, bias, seed=55 + zp)
    g = inp.to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs)
    need = mnb.gemm_silu_workspace_bytes(pw.desc, M)
    assert need == 2 * 96 * 256 * 256 * 4
    h = mnb.gemm_silu_mul(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=2 * I, block_size=bs)
    h2 = mnb.gemm_silu_mul(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=2 * I, block_size=bs)
    assert torch.equal(h, h2)
    rng = np.random.default_rng(9)
    rows = sorted({0, 255, 256, M - 1, *rng.choice(M, 8, replace=False).tolist()})
    hcols = np.unique(np.concatenate([[0, 31, 32, 127, 128, 8191, 8192, I - 1],
                                      rng.integers(0, 8192, 24), rng.integers(8192, I, 24)]))
    _check(orc, inp, h, I, rows, hcols)


@pytest.mark.parametrize("M,K,I,bs,dt,zp,bias", [
    (300, 256, 200, 64, "bf16", True, True),     # ragged rows and columns, I % 8 != 0: direct stores
    (130, 1024, 64, 16, "bf16", False, True),    # 16-value blocks, one column tile
    (64, 512, 300, 32, "f32", True, True),       # float32: the unfused path
    (40, 640, 128, 128, "bf16", True, False),    # bfloat16 with at most 128 rows: the unfused path
    (5, 1024, 96, 32, "f32", False, False),      # small M, unfused
])
def test_gated_any_m_matches_oracle(orc, M, K, I, bs, dt, zp, bias):
    log(f"gated M={M} K={K} I={I} bs={bs} {dt} zp={zp} bias={bias}")
    inp = random_inputs(K, 2 * I, M, bs, dt, zp, bias, seed=M + K + I)
    g = inp.to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs)
    h = mnb.gemm_silu_mul(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=2 * I, block_size=bs)
    _check(orc, inp, h, I, None, np.arange(I))


def test_gated_single_row_is_the_decode_kernel(orc):
    """M = 1 takes the gated decode GEMV: no workspace, the same bits as
    mnb_gemv_silu_mul."""
    K, I, bs = 2560, 512, 128
    inp = random_inputs(K, 2 * I, 1, bs, "f32", True, True, seed=4)
    g = inp.to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs)
    assert mnb.gemm_silu_workspace_bytes(pw.desc, 1) == 0
    h = mnb.gemm_silu_mul(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=2 * I, block_size=bs)
    h1 = mnb.gemv_silu_mul(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=2 * I, block_size=bs)
    assert torch.equal(h, h1)
    _check(orc, inp, h, I, None, np.arange(I))
