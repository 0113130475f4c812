"""Shared helpers of the GPU parity tests: marshal torch tensors for the
oracle and compare the GPU results with it.

Tolerances (from the method's stated accuracy): float32 activations
|y - y_ref| <= 1e-4 * S + 1e-6, bfloat16 activations <= 8e-3 * S + 1e-6, with
S = sum_k |a_k * w_kn| + |bias_n| computed by the oracle in fp64.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

REL = {"f32": 1e-4, "bf16": 8e-3}
ATOL = 1e-6


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def act_np(t: torch.Tensor) -> np.ndarray:
    """float32 -> float32 array; bfloat16 -> uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def oracle_ref(orc, inp, rows=None, cols=None):
    """Oracle y and S for an inputs bundle (workloads.generate.ProjectionInputs,
    any device), optionally restricted to some rows of A / columns of B."""
    a = inp.a if rows is None else inp.a[torch.as_tensor(rows, device=inp.a.device)]
    sel = None if cols is None else torch.as_tensor(cols, device=inp.q.device)
    q = inp.q if sel is None else inp.q[sel]
    sc = inp.scales if sel is None else inp.scales[sel]
    zp = None if inp.zp is None else (inp.zp if sel is None else inp.zp[sel])
    bias = None if inp.bias is None else (inp.bias if sel is None else inp.bias[sel])
    return orc.matmul(act_np(a), q.cpu().numpy(), None if zp is None else zp.cpu().numpy(),
                      act_np(sc), inp.block_size,
                      bias=None if bias is None else bias.cpu().numpy(), nthreads=8)


def assert_close(y_gpu: np.ndarray, y_ref: np.ndarray, S: np.ndarray, dt: str,
                 what: str = "") -> float:
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.isfinite(y_gpu).all(), f"{what}: non-finite output"
    err = np.abs(y_gpu - y_ref)
    tol = REL[dt] * S + ATOL
    ratio = err / tol
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        i = np.unravel_index(int(ratio.argmax()), ratio.shape)
        raise AssertionError(
            f"{what}: max err/tol {worst:.3g} at {i}: gpu={y_gpu[i]!r} ref={y_ref[i]!r} "
            f"S={S[i]!r}")
    return worst
