"""The five synthetic workloads, described by shape and value distribution.

Shapes follow the Qwen3 dense configurations listed on the page "Qwen3 CPU
Inference Critical Path" (section "Frozen model contract", model table:
0.6B = 28 layers, hidden 1,024, intermediate 3,072; 4B = 36 layers, hidden
2,560, intermediate 9,728; vocabulary 151,936) and the MatMulNBits shape list
in its "Exact kernel inventory" table (1024x3072 x56, 1024x4096 x28,
2048x1024 x28, 3072x1024 x28, 1024x151936 x1).

A decode or prefill *step* is the sequence of projections of every layer in
layer order, followed by the LM head. Q, K and V share one input and are one
fused projection of N = q + k + v columns (the same page's inventory splits the
fused QKV output by [2048, 1024, 1024]); gate and up share one input and run as
one launch over the concatenated N. Because the synthetic step has no attention
or normalization between projections, every launch receives its own seeded
input rather than the previous launch's output.

Nothing here computes anything: these are descriptions consumed by the seeded
generator in ``generate.py``.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Launch:
    """One matmul launch of a step: A[M,K] x dequant(B)[K,N] (+bias)."""

    name: str                 # e.g. "L3.qkv", "L3.gate_up", "lm_head"
    K: int
    N: int
    # Sub-projections whose weights are concatenated along N in this launch,
    # as (name, N_i). A single projection has one entry.
    parts: Tuple[Tuple[str, int], ...]


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    title: str
    M: int
    block_size: int
    act_dtype: str            # "f32" or "bf16"; scales and Y share it
    scale_lo: float
    scale_hi: float
    has_zp: bool
    bias: bool                # optional fp32 bias drawn from N(0, 0.02)
    launches: Tuple[Launch, ...]

    @property
    def n_projections(self) -> int:
        return sum(len(l.parts) for l in self.launches)

    def n_blocks(self, K: int) -> int:
        return -(-K // self.block_size)

    def weight_bytes(self, launch: Launch) -> int:
        """Packed nibbles + scales + packed zero points of one launch."""
        nb = self.n_blocks(launch.K)
        nib = launch.N * nb * self.block_size // 2
        sc = launch.N * nb * (4 if self.act_dtype == "f32" else 2)
        zp = launch.N * (-(-nb // 2)) if self.has_zp else 0
        return nib + sc + zp

    def step_weight_bytes(self) -> int:
        return sum(self.weight_bytes(l) for l in self.launches)

    def step_flops(self) -> int:
        return sum(2 * self.M * l.K * l.N for l in self.launches)


def _layer_launches(layers: int, hidden: int, inter: int, q_heads: int,
                    kv_heads: int, head: int) -> List[Launch]:
    q, kv = q_heads * head, kv_heads * head
    out: List[Launch] = []
    for i in range(layers):
        p = f"L{i}"
        out.append(Launch(f"{p}.qkv", hidden, q + 2 * kv,
                          ((f"{p}.qkv", q + 2 * kv),)))
        out.append(Launch(f"{p}.o", q, hidden, ((f"{p}.o", hidden),)))
        out.append(Launch(f"{p}.gate_up", hidden, 2 * inter,
                          ((f"{p}.gate", inter), (f"{p}.up", inter))))
        out.append(Launch(f"{p}.down", inter, hidden, ((f"{p}.down", hidden),)))
    return out


_VOCAB = 151936
_QWEN3_06B = _layer_launches(28, 1024, 3072, 16, 8, 128) + [
    Launch("lm_head", 1024, _VOCAB, (("lm_head", _VOCAB),))]
_QWEN3_4B = _layer_launches(36, 2560, 9728, 32, 8, 128) + [
    Launch("lm_head", 2560, _VOCAB, (("lm_head", _VOCAB),))]

CONFIGS = {
    1: Workload(1, "single MatMulNBits GEMV 1024->3072", 1, 32, "f32",
                0.005, 0.02, False, False,
                (Launch("gemv", 1024, 3072, (("gemv", 3072),)),)),
    2: Workload(2, "Qwen3-0.6B-shaped INT4 decode step", 1, 32, "f32",
                0.005, 0.02, True, False, tuple(_QWEN3_06B)),
    3: Workload(3, "Qwen3-0.6B-shaped INT4 prefill, 512 tokens", 512, 32,
                "f32", 0.005, 0.02, True, False, tuple(_QWEN3_06B)),
    4: Workload(4, "Qwen3-4B-shaped INT4 decode step", 1, 128, "f32",
                0.002, 0.01, False, False, tuple(_QWEN3_4B)),
    5: Workload(5, "Qwen3-4B-shaped INT4 prefill, 2048 tokens", 2048, 128,
                "bf16", 0.002, 0.01, True, True, tuple(_QWEN3_4B)),
}


def workload(cfg: int, M: Optional[int] = None) -> Workload:
    w = CONFIGS[cfg]
    return w if M is None else dataclasses.replace(w, M=M)
