"""A full decode or prefill step of a Qwen3-shaped workload on one stream.

Page "Qwen3 CPU Inference Critical Path": every projection of the model is a
MatMulNBits node ("Exact kernel inventory"); Q, K and V are one fused
projection whose output is later split ([2048, 1024, 1024] for 0.6B), and the
plan keeps packed weights for every token ("Phase Q1": plan-owned packed
weights reused by every token).  A step here is the model's projections in
layer order -- fused QKV, o, gate||up (one launch over the concatenated N),
down -- followed by the LM head, all enqueued on one stream by the library's
sequence driver (or replayed as one captured graph), or, for a decode step,
run as one launch of the persistent step kernel.

Inputs are the seeded synthetic tensors of ``workloads``; weights are packed
once on the GPU (the preparation step) and the logical values are dropped.
"""

from __future__ import annotations

import time
from typing import List, Optional, Tuple

import torch

from workloads.generate import projection_inputs
from workloads.qwen3 import Workload

from . import PackedWeight, PersistentStep, Sequence


class Step:
    def __init__(self, w: Workload, device="cuda", seed: int = 0,
                 with_bias: Optional[bool] = None):
        self.workload = w
        self.seed = seed
        self.with_bias = with_bias
        self.items: List[Tuple[PackedWeight, torch.Tensor, torch.Tensor]] = []
        dt = torch.float32 if w.act_dtype == "f32" else torch.bfloat16
        pack_s = 0.0
        for i, L in enumerate(w.launches):
            inp = projection_inputs(w, i, seed, device, with_bias=with_bias)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            pw = PackedWeight.from_logical(inp.q, inp.scales, inp.zp, inp.bias,
                                           block_size=w.block_size)
            torch.cuda.synchronize()
            pack_s += time.perf_counter() - t0
            y = torch.empty((w.M, L.N), dtype=dt, device=device)
            self.items.append((pw, inp.a, y))
            del inp
        self.pack_seconds = pack_s
        self.sequence = Sequence(self.items)
        self.persistent: Optional[PersistentStep] = None

    @property
    def weight_bytes(self) -> int:
        return sum(pw.weight_bytes for pw, _, _ in self.items)

    @property
    def launches(self) -> int:
        return len(self.items)

    def run(self, stream=None) -> None:
        self.sequence.run(stream)

    def capture(self) -> None:
        self.sequence.capture()

    def replay(self, stream=None) -> None:
        self.sequence.replay(stream)

    def make_persistent(self) -> PersistentStep:
        """The same projections as one persistent launch (decode steps only):
        launch_persistent() then computes what run() computes, bit for bit."""
        if self.persistent is None:
            self.persistent = PersistentStep(self.items)
        return self.persistent

    def launch_persistent(self, stream=None) -> None:
        self.make_persistent().launch(stream)

    def logical_inputs(self, launch_idx: int, device="cuda"):
        """Regenerate the logical (unpacked) inputs of one launch; identical to
        what was packed because the generator is seeded per tensor."""
        return projection_inputs(self.workload, launch_idx, self.seed, device,
                                 with_bias=self.with_bias)

    def close(self) -> None:
        self.sequence.close()
        if self.persistent is not None:
            self.persistent.close()
