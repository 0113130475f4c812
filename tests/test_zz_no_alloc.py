"""mnb_gemm_noalloc, the entry point for callers that cannot allocate, against
mnb_gemm (the same kernels and plan with a caller workspace), through the C
ABI: bit-identical outputs on two calls in a row, the second a smaller
product, so the static per-GPU scratch holds the first call's partials when
the second starts; also a product that needs no workspace.  Each result is
also checked against the oracle within the method's tolerance."""

import numpy as np
import pytest
import torch

import weight_only_int4_matmulnbits_amd as mnb
from parity import assert_close, log, oracle_ref, out_f64
from workloads.generate import random_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [  # (dt, M, K, N, bs, zp, bias): split products, then a smaller one, then none
    [("bf16", 512, 4096, 384, 128, True, True), ("f32", 256, 2048, 256, 32, True, False)],
    [("f32", 512, 3072, 1024, 32, True, True), ("bf16", 300, 1536, 520, 32, False, False)],
]


def _run_pair(orc, pair):
    for dt, M, K, N, bs, zp, bias in pair:
        log(f"noalloc {dt} M={M} K={K} N={N} bs={bs} zp={zp} bias={bias}")
        inp = random_inputs(K, N, M, bs, dt, zp, bias, seed=M + K + N)
        g = inp.to(DEV)
        pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs)
        need = mnb.workspace_bytes(pw.desc, M)
        assert 0 < need <= 64 << 20
        ws = mnb.workspace(need)
        y_ref_gpu = mnb.gemm(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=N,
                             block_size=bs, workspace=ws)
        out = torch.full((M, N), float("nan"), dtype=g.a.dtype, device=DEV)
        y = mnb.gemm_noalloc(g.a, pw.b_packed, pw.scales, pw.zp_packed, pw.bias, K=K, N=N,
                             block_size=bs, out=out)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref_gpu), (dt, M, K, N)
        y_ref, S = oracle_ref(orc, inp)
        assert_close(out_f64(y), y_ref, S, dt, f"noalloc {dt} M={M} K={K} N={N}")


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_gemm_two_calls(orc, case):
    _run_pair(orc, CASES[case])


def test_noalloc_without_split(orc):
    K, N, M, bs = 1024, 4096, 512, 32
    inp = random_inputs(K, N, M, bs, "f32", True, False, seed=3)
    g = inp.to(DEV)
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, block_size=bs)
    assert mnb.workspace_bytes(pw.desc, M) == 0
    y0 = mnb.gemm(g.a, pw.b_packed, pw.scales, pw.zp_packed, K=K, N=N, block_size=bs)
    y1 = mnb.gemm_noalloc(g.a, pw.b_packed, pw.scales, pw.zp_packed, K=K, N=N, block_size=bs)
    assert torch.equal(y0, y1)
    rows = [0, 1, 255, 511]
    y_ref, S = oracle_ref(orc, inp, rows=rows)
    assert_close(out_f64(y1[rows]), y_ref, S, "f32", "noalloc unsplit")
