"""fp64 CPU oracle for multi-scale retention.

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the HIP library and imports nothing from it.
"""

from .retention_oracle import (  # noqa: F401
    chunkwise,
    default_gammas,
    group_norm_swish,
    parallel,
    recurrent,
    recurrent_step,
    retention,
    retention_varlen,
    rotate,
    score_map,
)
from .retention_grad import chunkwise_state_grad, parallel_grad, unrotate  # noqa: F401
