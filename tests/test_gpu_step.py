"""The persistent decode-step kernel (mnb_step_*): one cooperative launch for
a whole chain of M = 1 projections.

* Every column has the bits of mnb_gemv on the same inputs (same geometry,
  loads and summation order), so the references here are the per-projection
  GEMV run in order on one stream; the chain tests also check sampled columns
  of every projection against the oracle on the inputs that projection
  actually read.
* Chains where projection i + 1 reads projection i's output exercise the
  kernel's device-wide ordering: a projection that started before its input
  was complete would read stale or NaN-poisoned values.
* Launches repeat, with new inputs between them, so the arrival counters must
  be back at zero after every launch.
The full-size decode steps (configs 2 and 4) are compared with the eager
sequence in test_gpu_configs.py.
"""

import numpy as np
import pytest
import torch

import weight_only_int4_matmulnbits_amd as mnb
from parity import assert_close, log, oracle_ref, out_f64
from workloads.generate import random_inputs

pytestmark = pytest.mark.gpu


def _packed(K, N, bs, dt, zp, bias, seed, scale_range=(0.005, 0.02)):
    g = random_inputs(K, N, 1, bs, dt, zp, bias, seed=seed, scale_range=scale_range).to("cuda")
    pw = mnb.PackedWeight.from_logical(g.q, g.scales, g.zp, g.bias, block_size=bs)
    return g, pw


def _chain(shapes, bs, dt, zp, bias, seed):
    """Projections K_i -> N_i with K_{i+1} == N_i: entry i + 1 reads entry i's
    y.  Returns (inputs, packed weights, the first input, outputs)."""
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    ins, pws, ys = [], [], []
    for i, (K, N) in enumerate(shapes):
        g, pw = _packed(K, N, bs, dt, zp, bias, seed + i, scale_range=(0.002, 0.01))
        ins.append(g)
        pws.append(pw)
        ys.append(torch.empty(1, N, dtype=tdt, device="cuda"))
    a0 = ins[0].a.clone()
    return ins, pws, a0, ys


def _items(pws, a0, ys):
    return [(pw, a0 if i == 0 else ys[i - 1], y) for i, (pw, y) in enumerate(zip(pws, ys))]


def _reference(pws, a0):
    """The chain through mnb_gemv, one projection after the other."""
    outs, a = [], a0
    for pw in pws:
        y = torch.empty(1, pw.desc.N, dtype=a0.dtype, device="cuda")
        pw.matmul(a, out=y)
        outs.append(y)
        a = y
    torch.cuda.synchronize()
    return outs


CHAINS = [
    # a Qwen3-4B-like layer pair (qkv-sized, o, gate-sized, down) and a ragged tail
    ("f32", 128, False, False, [(2560, 4096), (4096, 2560), (2560, 9728), (9728, 2560),
                               (2560, 4096), (4096, 2560), (2560, 1000)]),
    # Qwen3-0.6B-like, block 32 with zero points
    ("f32", 32, True, False, [(1024, 2048), (2048, 1024), (1024, 3072), (3072, 1024), (1024, 777)]),
    # bfloat16, block 64, zero points and bias, odd widths
    ("bf16", 64, True, True, [(2048, 4096), (4096, 1536), (1536, 9728), (9728, 1024), (1024, 65)]),
]


@pytest.mark.parametrize("case", range(len(CHAINS)))
def test_chain_matches_sequential_gemv_and_oracle(orc, case):
    dt, bs, zp, bias, shapes = CHAINS[case]
    log(f"chain {case}: {dt} block {bs} zp={zp} bias={bias} {shapes}")
    ins, pws, a0, ys = _chain(shapes, bs, dt, zp, bias, seed=100 + 10 * case)
    ref = _reference(pws, a0)
    step = mnb.PersistentStep(_items(pws, a0, ys))
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        step.launch()
        step.check()
        for i, (r, y) in enumerate(zip(ref, ys)):
            assert torch.equal(r, y), f"chain {case} launch {rep}: projection {i} differs from mnb_gemv"
    # each projection against the oracle on the input it read
    rng = np.random.default_rng(case)
    for i, g in enumerate(ins):
        g.a = a0 if i == 0 else ys[i - 1]
        cols = sorted({0, g.N - 1, *map(int, rng.choice(g.N, size=min(24, g.N), replace=False))})
        y_ref, S = oracle_ref(orc, g, None, cols)
        assert_close(out_f64(ys[i][:, torch.as_tensor(cols, device="cuda")]), y_ref, S, dt,
                     f"chain {case} projection {i}")
    step.close()


SINGLES = [
    # (K, N, block, dtype, zp, bias)
    (32, 1, 32, "f32", True, True),
    (96, 3, 32, "f32", False, False),
    (1000, 65, 64, "bf16", True, False),
    (2560, 1, 128, "f32", False, True),
    (4096, 6144, 256, "bf16", False, True),
    (3072, 4097, 32, "f32", True, True),
    (9728, 129, 128, "f32", True, False),
    (2560, 151936, 128, "f32", False, False),    # a vocabulary-sized head
]


@pytest.mark.parametrize("shape", SINGLES)
def test_single_projection_is_mnb_gemv(shape):
    K, N, bs, dt, zp, bias = shape
    g, pw = _packed(K, N, bs, dt, zp, bias, seed=K + N)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    y_ref = torch.empty(1, N, dtype=tdt, device="cuda")
    pw.matmul(g.a, out=y_ref)
    y = torch.full((1, N), float("nan"), dtype=tdt, device="cuda")
    step = mnb.PersistentStep([(pw, g.a, y)])
    step.launch()
    step.check()
    assert torch.equal(y, y_ref), f"{shape}: differs from mnb_gemv"
    step.close()


def test_new_inputs_between_launches():
    """The counters return to zero and every launch reads the current input."""
    shapes = [(1024, 3072), (3072, 1024), (1024, 2048)]
    ins, pws, a0, ys = _chain(shapes, 32, "f32", True, False, seed=7)
    step = mnb.PersistentStep(_items(pws, a0, ys))
    gen = torch.Generator(device="cuda").manual_seed(11)
    for rep in range(5):
        a0.copy_(torch.randn(a0.shape, device="cuda", generator=gen))
        ref = _reference(pws, a0)
        for y in ys:
            y.fill_(float("nan"))
        step.launch()
        step.check()
        for i, (r, y) in enumerate(zip(ref, ys)):
            assert torch.equal(r, y), f"launch {rep}: projection {i}"
    step.close()


def test_unsupported_entries_are_refused():
    g, pw = _packed(1024, 64, 16, "f32", False, False, seed=3)        # block 16
    y = torch.empty(1, 64, device="cuda")
    with pytest.raises(mnb.MnbError) as e:
        mnb.PersistentStep([(pw, g.a, y)])
    assert e.value.status == -2
    g2, pw2 = _packed(1024, 64, 32, "bf16", False, False, seed=4)    # mixed activation types
    g3, pw3 = _packed(1024, 64, 32, "f32", False, False, seed=5)
    with pytest.raises(mnb.MnbError) as e:
        mnb.PersistentStep([(pw3, g3.a, torch.empty(1, 64, device="cuda")),
                            (pw2, g2.a, torch.empty(1, 64, dtype=torch.bfloat16, device="cuda"))])
    assert e.value.status == -2


def test_trace_timestamps_are_ordered_and_change_nothing():
    shapes = [(1024, 3072), (3072, 1024), (1024, 2048)]
    ins, pws, a0, ys = _chain(shapes, 32, "f32", True, False, seed=9)
    ref = _reference(pws, a0)
    step = mnb.PersistentStep(_items(pws, a0, ys))
    tr = step.trace_buffer()
    step.launch()
    step.check()
    for i, (r, y) in enumerate(zip(ref, ys)):
        assert torch.equal(r, y), f"projection {i} with tracing on"
    t = tr.cpu()
    assert t.shape[1:] == (len(shapes), 5) and t.shape[0] >= 1
    assert (t > 0).all()
    # per workgroup and projection the five phases are in order, and each
    # projection starts after the previous one's outputs are acknowledged
    assert (t[:, :, 1:] >= t[:, :, :-1]).all()
    assert (t[:, 1:, 0] >= t[:, :-1, 4]).all()
    # every workgroup saw every arrival of projection i - 1 before staging row
    # i (up to 1 us of skew between the clocks of different CUs)
    assert (t[:, 1:, 1].min(dim=0).values >= t[:, :-1, 4].max(dim=0).values - 100).all()
    step.close()
