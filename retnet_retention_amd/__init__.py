"""Multi-scale retention (RetNet) for AMD MI355X: hand-written HIP kernels for
gfx950 behind a C ABI (include/retention.h), with a thin ctypes binding.

    parallel_fwd     parallel form (training)
    chunkwise_fwd    chunkwise recurrent form (long sequences, prefill)
    chunkwise_fwd_noalloc the same without a workspace (a static scratch; allocates nothing)
    chunkwise_varlen_fwd  the same over packed sequences of different lengths
    recurrent_step   recurrent form, one decode step, state in place
    parallel_bwd     gradients of the parallel form (q, k, v and the gate)
    chunkwise_bwd    the same gradients, each product run as the chunkwise form
    score_map        one query token's retention weights, summed over heads
    check_chunkwise  raise if a chunkwise call's control word reports an error
"""

from .binding import (  # noqa: F401
    RetentionError,
    check_chunkwise,
    chunkwise_bwd,
    chunkwise_error,
    chunkwise_fwd,
    chunkwise_fwd_noalloc,
    chunkwise_varlen_fwd,
    chunkwise_varlen_workspace_bytes,
    chunkwise_workspace_bytes,
    lib,
    parallel_bwd,
    parallel_fwd,
    recurrent_step,
    score_map,
)
