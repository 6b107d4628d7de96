"""Seeded synthetic inputs for multi-scale retention.

This module holds no retention arithmetic: it draws numbers, rounds them to the
storage dtype and describes the workload shapes. Both the fp64 oracle (through
the tests and the bench) and the HIP library receive exactly these bits.

Recipe: numpy ``default_rng(seed)`` (PCG64) draws fp64 standard normals in the
order the caller asks for (Q, K, V, G, ...), each of shape [B, N, H, d]; the
draw is multiplied by its scale and rounded to fp32 (round-to-nearest-even) or
to bf16 (fp64 -> fp32 -> bf16, both round-to-nearest-even, by bit operations).
The oracle receives the rounded values upcast exactly to fp64.
"""

from .inputs import (  # noqa: F401
    Tensor,
    bf16_bits_to_f64,
    draw,
    f64_to_bf16_bits,
    round_to,
)
from .configs import CONFIGS, Workload, get  # noqa: F401
