"""Degenerate weights: every weight equal to its zero point (w = 0 exactly)
gives Y = bias exactly (bias-free: zeros), on every kernel path (decode GEMV,
2-4 row GEMV, small-M matrix cores, prefill GEMM), float32 and bfloat16."""

import numpy as np
import pytest
import torch

import weight_only_int4_matmulnbits_amd as mnb
from parity import assert_close, log, oracle_ref, out_f64
from workloads.generate import random_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M", [1, 3, 8, 64])
@pytest.mark.parametrize("K,N,bs", [(1024, 512, 32), (2560, 256, 128), (3072, 128, 32), (300, 70, 16)])
def test_weights_equal_to_zero_points_give_the_bias(orc, dt, M, K, N, bs):
    for bias in (False, True):
        log(f"zero weights {dt} M={M} K={K} N={N} bs={bs} bias={bias}")
        inp = random_inputs(K, N, M, bs, dt, True, bias, seed=K + N + M)
        inp.q = inp.zp.repeat_interleave(bs, dim=1)[:, :K].contiguous()
        g = inp.to(DEV)
        y = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs).matmul(g.a)
        y_ref, S = oracle_ref(orc, inp)
        assert_close(out_f64(y), y_ref, S, dt, f"zero weights M={M}")
        want = torch.zeros(M, N, dtype=y.dtype, device=DEV)
        if bias:
            want += g.bias.to(y.dtype)
        assert torch.equal(y, want), (M, K, N, bs, bias)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("K,bs,zp", [(4000, 32, True), (8192 + 96, 32, False), (9728, 128, True), (2560, 128, False)])
def test_infinite_last_activation_gives_infinities_of_the_exact_sign(dt, K, bs, zp):
    """One infinite activation at k = K - 1, every other value finite: each
    column's exact sum is +-inf with the sign of s * (q - zp) at that k.  The
    one-row GEMV's lanes whose chunks lie past K (K = 4000, 8288 and 9728 do
    not fill the team's lanes times its chunks) must add exactly nothing, not
    0 * inf = NaN."""
    N = 96
    log(f"infinite last activation {dt} K={K} bs={bs} zp={zp}")
    inp = random_inputs(K, N, 1, bs, dt, zp, False, seed=K + 7)
    blk = (K - 1) // bs
    z = inp.zp[:, blk].to(torch.int64) if zp else torch.full((N,), 8, dtype=torch.int64)
    q_last = torch.where(z < 8, z + 3, z - 3)        # never its zero point
    inp.q[:, K - 1] = q_last.to(inp.q.dtype)
    inp.a[0, K - 1] = float("inf")
    g = inp.to(DEV)
    y = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp if zp else None, None, block_size=bs).matmul(g.a)
    yy = y.double().cpu()[0]
    want = torch.sign(inp.scales[:, blk].double() * (q_last - z).double()) * float("inf")
    assert torch.equal(yy, want), (int(torch.isnan(yy).sum()), int((yy != want).sum()))
