"""GPU parity of the chunkwise form over packed sequences of different
lengths (a ragged prefill batch) against the fp64 oracle run on each
sequence alone: empty and one-token sequences, ragged last chunks, lengths
that are exact chunk multiples, a length bound above the longest sequence,
carried states, rotation and gate; bit-identity with the batched call when
the lengths are equal; and the kernels' clamping of invalid boundaries."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import retnet_retention_amd as rr
from retnet_retention_amd import binding as B
from synth import draw
from tests.gpu_helpers import DEV, assert_close, to64

pytestmark = pytest.mark.gpu


def _announce(**kw):
    print("case:", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _packed(seed, lens, h, d, dtype, gate, state):
    tot = int(sum(lens))
    specs = [((tot, h, d), 1 / 16)] * 3 + ([((tot, h, d), 1.0)] if gate else [])
    ts = draw(seed, specs, dtype)
    q, k, v = ts[:3]
    g = ts[3] if gate else None
    s0 = None
    if state:
        s0 = (np.random.default_rng(seed + 7).standard_normal((len(lens), h, d, d)) * 0.05)
        s0 = s0.astype(np.float32).astype(np.float64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, g, s0, cu


def _workspace(nseq, maxlen, h, d, dtype, chunk, base):
    desc, keep = B.make_desc(nseq, maxlen, h, d, d, dtype, rotary_base=base)
    need = B.lib().retention_chunkwise_varlen_workspace_bytes(ctypes.byref(desc), chunk)
    return torch.empty(need, dtype=torch.uint8, device=DEV)


def _run(q, k, v, g, s0, cu, maxlen, chunk, base, pos, dtype_code, workspace=None):
    tq, tk, tv = q.torch(DEV), k.torch(DEV), v.torch(DEV)
    tg = g.torch(DEV) if g is not None else None
    nseq, h, d = len(cu) - 1, tq.shape[1], tq.shape[2]
    s_in = torch.from_numpy(s0.astype(np.float32)).to(DEV) if s0 is not None else None
    s_out = torch.full((nseq, h, d, d), float("nan"), device=DEV)
    out = torch.full_like(tv, float("nan"))
    ws = workspace if workspace is not None else _workspace(nseq, maxlen, h, d, dtype_code, chunk, base)
    rr.chunkwise_varlen_fwd(tq, tk, tv, torch.from_numpy(cu).to(DEV), maxlen, tg, chunk=chunk, state_in=s_in,
                            state_out=s_out, rotary_base=base, pos_offset=pos, out=out, workspace=ws)
    torch.cuda.synchronize()
    word = rr.chunkwise_error(ws)  # the C ABI's reader of control word 1
    assert word == int(ws[4:8].view(torch.int32).item())
    return out, s_out, word


CASES = [
    # (lens, maxlen, heads, d, chunk, dtype, gate, rotary, state)
    ([0, 1, 63, 512, 513, 1000, 37], 1024, 2, 256, 512, "bf16", True, True, True),
    ([300, 17, 0, 520], 520, 2, 128, 128, "bf16", True, False, True),  # 8 (sequence, head) pairs: XCD classes
    ([5, 0, 130, 64, 1], 130, 3, 64, 64, "f32", False, True, True),
    ([200, 7], 256, 1, 256, 100, "f32", True, False, False),
    # 300 sequences x 8 heads: 300 pairs per ticket class, more than one tile of the schedule
    (list(np.random.default_rng(3).integers(0, 100, 300)), 100, 8, 64, 64, "f32", True, True, True),
    # 40 short sequences at chunk 7: eight slots, most sequences spread over a few of them
    (list(np.random.default_rng(4).integers(0, 50, 40)), 50, 2, 64, 7, "f32", False, False, True),
    # 16 heads (two per ticket class and sequence), rotation, a carried state, chunk 64
    ([130, 64, 0, 1, 200, 77, 5, 500], 512, 16, 128, 64, "bf16", True, True, True),
]


@pytest.mark.parametrize("lens,maxlen,h,d,chunk,dtype,gate,rot,state", CASES)
def test_varlen_parity(lens, maxlen, h, d, chunk, dtype, gate, rot, state):
    _announce(lens=lens if len(lens) < 10 else f"{len(lens)} sequences", maxlen=maxlen, h=h, d=d, chunk=chunk, dtype=dtype, gate=gate, rot=rot, state=state)
    q, k, v, g, s0, cu = _packed(41 + sum(lens), lens, h, d, dtype, gate, state)
    base = 10000.0 if rot else 0.0
    ref, ref_s = oracle.retention_varlen("chunkwise", q.f64, k.f64, v.f64, cu, g=None if g is None else g.f64,
                                         rotary_base=base, pos_offset=3, chunk=chunk, state_in=s0)
    code = B.RET_BF16 if dtype == "bf16" else B.RET_F32
    out, s_out, err = _run(q, k, v, g, s0, cu, maxlen, chunk, base, 3, code)
    assert err == 0
    assert_close(to64(out), ref, dtype, "out")
    assert_close(to64(s_out), ref_s, dtype, "state")


def test_varlen_equal_lengths_match_batched_call():
    """Equal lengths: the packed call runs the batched call's arithmetic, so
    outputs and states are bit-identical."""
    b, n, h, d, chunk = 2, 700, 2, 256, 512
    _announce(b=b, n=n, h=h, d=d, chunk=chunk)
    q, k, v, g, s0, cu = _packed(5, [n] * b, h, d, "bf16", True, True)
    out, s_out, err = _run(q, k, v, g, s0, cu, n, chunk, 10000.0, 3, B.RET_BF16)
    assert err == 0
    shp = (b, n, h, d)
    s_ref = torch.empty((b, h, d, d), device=DEV)
    ref = rr.chunkwise_fwd(q.torch(DEV).view(shp), k.torch(DEV).view(shp), v.torch(DEV).view(shp),
                           g.torch(DEV).view(shp), chunk=chunk,
                           state_in=torch.from_numpy(s0.astype(np.float32)).to(DEV), state_out=s_ref,
                           rotary_base=10000.0, pos_offset=3)
    torch.cuda.synchronize()
    assert torch.equal(out.view(shp), ref)
    assert torch.equal(s_out, s_ref)


def test_varlen_invalid_boundaries_are_clamped_and_reported():
    """Boundaries that run backwards or past the tensor: every access stays
    inside it (clamped), the control word reports the error, and the rows
    that only the valid first sequence writes are still right (the clamped
    third sequence overlaps its rows 50..99)."""
    h, d, chunk, maxlen = 2, 64, 64, 128
    q, k, v, g, _, _ = _packed(9, [200], h, d, "f32", True, False)
    cu = np.array([0, 100, 50, 300], dtype=np.int32)  # 100 -> 50 backwards; 300 past 200 rows
    _announce(cu=cu.tolist(), total=200, maxlen=maxlen)
    ws = _workspace(len(cu) - 1, maxlen, h, d, B.RET_F32, chunk, 0.0)
    out, _, err = _run(q, k, v, g, None, cu, maxlen, chunk, 0.0, 0, B.RET_F32, workspace=ws)
    assert err & 2
    with pytest.raises(rr.RetentionError) as info:
        rr.check_chunkwise(ws)
    assert info.value.word == err
    # a call with the binding's own workspace checks the word by itself
    with pytest.raises(rr.RetentionError):
        rr.chunkwise_varlen_fwd(q.torch(DEV), k.torch(DEV), v.torch(DEV), torch.from_numpy(cu).to(DEV), maxlen,
                                g.torch(DEV), chunk=chunk)
    ref, _ = oracle.retention_varlen("chunkwise", q.f64[:100], k.f64[:100], v.f64[:100], [0, 100],
                                     g=g.f64[:100], chunk=chunk)
    assert_close(to64(out[:50]), ref[:50], "f32", "valid sequence")


def test_varlen_bitwise_deterministic():
    """Workgroups take their items from tickets in whatever order the chip
    runs them, but each item's arithmetic is fixed: two calls agree bit for
    bit."""
    lens = [700, 3, 0, 512, 129]
    _announce(lens=lens, case="determinism")
    q, k, v, g, s0, cu = _packed(77, lens, 4, 256, "bf16", True, True)
    a = _run(q, k, v, g, s0, cu, 700, 256, 10000.0, 0, B.RET_BF16)
    b = _run(q, k, v, g, s0, cu, 700, 256, 10000.0, 0, B.RET_BF16)
    assert a[2] == 0 and b[2] == 0
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
