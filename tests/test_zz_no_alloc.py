"""The chunkwise entry point that allocates nothing (its scratch is the
library's static device array) against the workspace entry point on the same
inputs: two calls in a row, the second smaller than the first, each
bit-identical to the workspace call (the same kernels run the same
arithmetic), with the error word clear."""

import numpy as np
import pytest
import torch

import retnet_retention_amd as rr
from tests.gpu_helpers import DEV, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # (batch, seqlen, heads, d, chunk, gate, rotary, state): the second is smaller
    (2, 1100, 4, 256, 512, True, True, True),
    (1, 300, 2, 128, 64, False, False, True),
]


def test_noalloc_matches_the_workspace_call():
    for b, n, h, d, chunk, gate, rot, state in CASES:
        print(f"case: noalloc b={b} n={n} h={h} d={d} chunk={chunk} gate={gate} rot={rot} state={state}", flush=True)
        q, k, v, g, s0 = make_inputs(171 + n, b, n, h, d, "bf16", 1 / 16, 1.0 if gate else None, state)
        tq, tk, tv = q.torch(DEV), k.torch(DEV), v.torch(DEV)
        tg = g.torch(DEV) if gate else None
        s_in = torch.from_numpy(s0.astype(np.float32)).to(DEV) if state else None
        base = 10000.0 if rot else 0.0
        s_ref = torch.empty((b, h, d, d), device=DEV)
        ref = rr.chunkwise_fwd(tq, tk, tv, tg, chunk=chunk, state_in=s_in, state_out=s_ref, rotary_base=base,
                               pos_offset=5)
        out = torch.full_like(tv, float("nan"))
        s_out = torch.full((b, h, d, d), float("nan"), device=DEV)
        err = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        rr.chunkwise_fwd_noalloc(tq, tk, tv, tg, chunk=chunk, state_in=s_in, state_out=s_out, rotary_base=base,
                                 pos_offset=5, out=out, error_word=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(out, ref)
        assert torch.equal(s_out, s_ref)
