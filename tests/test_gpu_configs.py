"""The five workloads at full size, run exactly as the benchmark runs them
(one Step: every projection packed once, then the whole step enqueued by the
library's sequence driver on one stream), checked against the oracle on
sampled outputs: all columns of the single GEMV; for the decode steps the
first, last and 30 random columns of every launch; for the prefill steps the
first, last and 6 random rows times the first, last and 14 random columns of
every launch; for the 0.6B step with 4, 8 and 16 rows per projection (the
bench's small-M rows: the 2-4-row GEMV, then the matrix-core small-M
kernel) all rows times the first, last and 30 random columns.  A
captured-graph replay must reproduce the eager step bit for bit, and so must
the decode steps' persistent launch.
"""

import numpy as np
import pytest
import torch

from parity import assert_close, log, oracle_ref, out_f64
from weight_only_int4_matmulnbits_amd.step import Step
from workloads import workload

pytestmark = pytest.mark.gpu


def _sample(n, k, rng):
    extra = rng.choice(n, size=min(k, n), replace=False) if n > 2 else []
    return sorted({0, n - 1, *map(int, extra)})


SMALL_M_STEPS = {"2m4": 4, "2m8": 8, "2m16": 16}     # the 0.6B step at M rows


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, *SMALL_M_STEPS])
def test_config_step_parity(orc, cfg):
    w = workload(2, M=SMALL_M_STEPS[cfg]) if cfg in SMALL_M_STEPS else workload(cfg)
    log(f"config {cfg}: building {w.title} ({len(w.launches)} launches)")
    step = Step(w, "cuda", seed=0)
    step.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(20 + SMALL_M_STEPS[cfg] if cfg in SMALL_M_STEPS else cfg)
    worst = 0.0
    for i, (pw, a, y) in enumerate(step.items):
        inp = step.logical_inputs(i)
        N = inp.N
        if cfg == 1:
            rows, cols = None, None
        elif w.M <= 16:
            rows, cols = None, _sample(N, 30, rng)
        else:
            rows, cols = _sample(w.M, 6, rng), _sample(N, 14, rng)
        y_ref, S = oracle_ref(orc, inp, rows, cols)
        yg = y
        if rows is not None:
            yg = yg[torch.as_tensor(rows, device=y.device)]
        if cols is not None:
            yg = yg[:, torch.as_tensor(cols, device=y.device)]
        worst = max(worst, assert_close(out_f64(yg), y_ref, S, w.act_dtype,
                                        f"config {cfg} launch {w.launches[i].name}"))
        del inp
    log(f"config {cfg}: worst err/tol {worst:.3g}")
    if cfg in (2, 4, *SMALL_M_STEPS):
        eager = [y.clone() for _, _, y in step.items]
        for _, _, y in step.items:
            y.fill_(float("nan"))
        step.capture()
        for rep in range(3):
            step.replay()
            torch.cuda.synchronize()
            for e, (_, _, y) in zip(eager, step.items):
                assert torch.equal(e, y), f"graph replay {rep} differs"
            step.run()            # eager work between replays
            torch.cuda.synchronize()
        if w.M == 1:
            # the persistent step kernel: the same bits in one launch, over
            # several launches with eager work between them
            log(f"config {cfg}: persistent step")
            step.make_persistent()
            for rep in range(3):
                for _, _, y in step.items:
                    y.fill_(float("nan"))
                step.launch_persistent()
                step.persistent.check()
                for i, (e, (_, _, y)) in enumerate(zip(eager, step.items)):
                    assert torch.equal(e, y), f"persistent launch {rep} differs at {w.launches[i].name}"
                step.run()
                torch.cuda.synchronize()
    step.close()


def test_config5_without_bias(orc):
    w = workload(5)
    step = Step(w, "cuda", seed=1, with_bias=False)
    step.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(55)
    for i in (0, 3, len(step.items) - 1):
        inp = step.logical_inputs(i)
        assert inp.bias is None
        rows, cols = _sample(w.M, 4, rng), _sample(inp.N, 8, rng)
        y_ref, S = oracle_ref(orc, inp, rows, cols)
        y = step.items[i][2][torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")]
        assert_close(out_f64(y), y_ref, S, "bf16", f"config 5 no-bias launch {i}")
    step.close()
