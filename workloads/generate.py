"""Seeded synthetic inputs for one launch of a workload.

Distributions (from the workload descriptions in ``qwen3.py``):

* weights ``q``: uint4 values drawn uniformly from 0..15, logical layout
  [N][K] (one value per byte, not packed);
* zero points ``zp``: uniform 0..15, [N][n_blocks], or absent (the contract's
  default of 8 then applies);
* scales: uniform in [lo, hi), drawn in float32 and, for bf16 workloads,
  rounded to bfloat16 by torch's round-to-nearest-even cast;
* activations ``a``: standard normal, float32 (bf16 workloads: rounded to
  bfloat16 the same way);
* bias: fp32 drawn from N(0, 0.02) when the workload has one.

Every tensor comes from its own ``torch.Generator`` seeded by a hash of
(base seed, config, launch index, part index, tensor name), so any launch can be
regenerated alone. CPU and GPU generators produce different streams, so a test
that compares the two paths generates once and copies. This module performs
none of the method's arithmetic.
"""

from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import torch

from .qwen3 import Launch, Workload

_TENSORS = ("q", "zp", "scales", "a", "bias")


def seed_for(base: int, cfg: int, launch_idx: int, part_idx: int,
             tensor: str) -> int:
    key = f"{base}/{cfg}/{launch_idx}/{part_idx}/{tensor}".encode()
    return int.from_bytes(hashlib.blake2b(key, digest_size=8).digest(),
                          "little") & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


@dataclasses.dataclass
class ProjectionInputs:
    K: int
    N: int
    M: int
    block_size: int
    act_dtype: str
    q: torch.Tensor                    # uint8 [N][K], values 0..15
    zp: Optional[torch.Tensor]         # uint8 [N][nb] or None
    scales: torch.Tensor               # f32 / bf16 [N][nb]
    a: torch.Tensor                    # f32 / bf16 [M][K]
    bias: Optional[torch.Tensor]       # f32 [N] or None

    @property
    def n_blocks(self) -> int:
        return -(-self.K // self.block_size)

    def to(self, device) -> "ProjectionInputs":
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return dataclasses.replace(self, q=mv(self.q), zp=mv(self.zp),
                                   scales=mv(self.scales), a=mv(self.a),
                                   bias=mv(self.bias))


def random_inputs(K: int, N: int, M: int, block_size: int, act_dtype: str,
                  has_zp: bool, with_bias: bool, seed: int, device="cpu",
                  scale_range=(0.005, 0.02)) -> ProjectionInputs:
    """One projection with the standard distributions, from a single seed."""
    ws = Workload(0, "adhoc", M, block_size, act_dtype, scale_range[0],
                  scale_range[1], has_zp, with_bias,
                  (Launch("adhoc", K, N, (("adhoc", N),)),))
    return projection_inputs(ws, 0, base_seed=seed, device=device)


def projection_inputs(w: Workload, launch_idx: int, base_seed: int = 0,
                      device="cpu", with_bias: Optional[bool] = None
                      ) -> ProjectionInputs:
    """Inputs of launch ``launch_idx`` of workload ``w``.

    For a fused launch (QKV is already one projection; gate_up has two parts)
    the weights, scales and zero points of each part are drawn with the part's
    own seeds and concatenated along N; the activation and bias are drawn once
    per launch (the parts share their input).
    """
    L = w.launches[launch_idx]
    K, M, nb = L.K, w.M, w.n_blocks(L.K)
    bias_on = w.bias if with_bias is None else with_bias
    fdt = torch.float32 if w.act_dtype == "f32" else torch.bfloat16
    qs, zps, scs = [], [], []
    for p, (_, n_p) in enumerate(L.parts):
        s = lambda t: seed_for(base_seed, w.cfg, launch_idx, p, t)  # noqa: E731
        qs.append(torch.randint(0, 16, (n_p, K), dtype=torch.uint8,
                                device=device, generator=_gen(device, s("q"))))
        if w.has_zp:
            zps.append(torch.randint(0, 16, (n_p, nb), dtype=torch.uint8,
                                     device=device,
                                     generator=_gen(device, s("zp"))))
        u = torch.rand((n_p, nb), dtype=torch.float32, device=device,
                       generator=_gen(device, s("scales")))
        scs.append((w.scale_lo + (w.scale_hi - w.scale_lo) * u).to(fdt))
    s0 = lambda t: seed_for(base_seed, w.cfg, launch_idx, 0, t)  # noqa: E731
    a = torch.randn((M, K), dtype=torch.float32, device=device,
                    generator=_gen(device, s0("a"))).to(fdt)
    bias = None
    if bias_on:
        bias = 0.02 * torch.randn((L.N,), dtype=torch.float32, device=device,
                                  generator=_gen(device, s0("bias")))
    cat = lambda xs: xs[0] if len(xs) == 1 else torch.cat(xs, 0)  # noqa: E731
    return ProjectionInputs(K=K, N=L.N, M=M, block_size=w.block_size,
                            act_dtype=w.act_dtype, q=cat(qs),
                            zp=cat(zps) if w.has_zp else None,
                            scales=cat(scs), a=a, bias=bias)
