"""The five measured workloads of the Fibonacci-offset sparse attention path (data only).

Shapes follow the pages' setting: 16 layers, hidden 512 = 8 heads x 64, training length
1024 and 4x extrapolation to 4096 ("Depth-Staggered Fibonacci Spacing for Sparse
Attention", Method and Results 3 - length extrapolation), plus one long-context shape
that fills one GPU. Alphas are produced by the per-layer schedules named here; the
schedule arithmetic itself lives in the library (and, independently, in the oracle).

Offset bases, as printed on the pages (Method, attended-set bullet; Controls):
* ``FIB_BASE``: the Fibonacci offsets 1, 2, 3, 5, ..., 987 (15 values, the repeated 1
  of the sequence dropped since a set of offsets is meant).
* ``POW2_BASE``: the log-sparse power-of-two control 1, 2, 4, ..., 2048 (12 values; the
  pages name 1024 and 2048 as its largest rungs at 4x length).
"""
from __future__ import annotations

from dataclasses import dataclass, field

FIB_BASE = (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987)
POW2_BASE = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048)

INT = 0
INTERP = 1
F32 = 0
BF16 = 1


@dataclass(frozen=True)
class Workload:
    config: int            # workload number, used in the seed recipe
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: int             # F32 or BF16
    windows: tuple         # W values swept
    bases: tuple           # tuple of (base_id, base tuple)
    mode: int              # INT or INTERP
    schedule: str          # "fixed1", "linear", "coprime", "uniform", "layer15_linear"
    layers: tuple          # layer indices run
    backward: bool
    theta: float = 10000.0
    extra_modes: tuple = field(default_factory=tuple)

    @property
    def rows(self) -> int:
        return self.B * self.H * self.N


WORKLOADS = (
    Workload(1, "single_head_fp32_n1024", 1, 1, 1024, 64, F32, (12,), ((0, FIB_BASE),),
             INT, "fixed1", (0,), False),
    Workload(2, "staggered_linear_16x_b8h8_n1024", 8, 8, 1024, 64, BF16, (6, 8, 10, 12),
             ((0, FIB_BASE),), INT, "linear", tuple(range(16)), False),
    Workload(3, "learned_dilation_16x_b8h8_n1024", 8, 8, 1024, 64, BF16, (12,),
             ((0, FIB_BASE),), INTERP, "uniform", tuple(range(16)), True),
    Workload(4, "coprime_extrapolation_b4h8_n4096", 4, 8, 4096, 64, BF16, (12,),
             ((0, FIB_BASE), (1, POW2_BASE)), INT, "coprime", tuple(range(16)), False),
    Workload(5, "long_context_b1h32_n131072", 1, 32, 131072, 64, BF16, (12,),
             ((0, FIB_BASE),), INT, "layer15_linear", (15,), True, extra_modes=(INTERP,)),
)

BY_CONFIG = {w.config: w for w in WORKLOADS}

# Learned-dilation alphas: U[0.95, 1.05] around the learned schedule's init of 1 (the pages
# report that learned alphas stay near 1), drawn with this seed.
UNIFORM_ALPHA_SEED = 3
UNIFORM_ALPHA_RANGE = (0.95, 1.05)
