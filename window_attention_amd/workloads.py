"""The five workloads (grids, window counts, shapes, layouts).  Data only."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    T: int
    H: int
    W: int
    nt: int
    nh: int
    nw: int
    batch: int
    heads: int
    head_dim: int
    sigma: float
    # layouts of the attention layers ("R" regular, "S" shifted), in order;
    # the canonical Q/K/V are gathered into `entry` and every layout change
    # (entry -> first layer, layer -> layer) is one fused transition
    schedule: Tuple[str, ...]
    entry: str = "R"
    input_dtype: str = "bf16"

    @property
    def L(self) -> int:
        return self.T * self.H * self.W


WORKLOADS = [
    Workload(0, "tiny_5x9x16", 5, 9, 16, 2, 3, 3, 1, 1, 64, 1.0, ("R", "S"), input_dtype="fp32"),
    Workload(1, "clip_4x45x80", 4, 45, 80, 4, 3, 3, 1, 24, 128, 1.0, ("R",)),
    Workload(2, "video_21x45x80", 21, 45, 80, 4, 3, 3, 1, 24, 128, 1.0, ("R", "S", "R", "S")),
    Workload(3, "hd_21x68x120", 21, 68, 120, 4, 3, 3, 2, 24, 128, 0.5, ("R", "S")),
    Workload(4, "long_31x90x160", 31, 90, 160, 4, 3, 3, 1, 24, 128, 1.0, ("S",), entry="R"),
]
BY_NAME = {w.name: w for w in WORKLOADS}
