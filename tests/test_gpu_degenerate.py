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
