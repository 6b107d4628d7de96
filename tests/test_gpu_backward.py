"""GPU parity of the parallel form's backward (dq, dk, dv, dg) against the
fp64 gradient oracle, on the same input bits: single tokens, ragged lengths
over several query blocks, with and without the gate and the rotation, every
head dimension, fp32 and bf16, and the 3B workload's shape in full."""

import numpy as np
import pytest

import oracle
import retnet_retention_amd as rr
from synth import draw, get
from tests.gpu_helpers import DEV, assert_close, to64

pytestmark = pytest.mark.gpu


def _announce(**kw):
    print("case:", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _run(seed, b, n, h, d, dtype, scale, gate, rot, pos=0, gammas=None, gate_scale=1 / 16):
    specs = [((b, n, h, d), scale)] * 3 + [((b, n, h, d), 1 / 8)]  # q, k, v, dout
    if gate:
        specs.append(((b, n, h, d), gate_scale))
    ts = draw(seed, specs, dtype)
    q, k, v, dout = ts[:4]
    g = ts[4] if gate else None
    base = 10000.0 if rot else 0.0
    got = rr.parallel_bwd(q.torch(DEV), k.torch(DEV), v.torch(DEV), dout.torch(DEV),
                          g.torch(DEV) if gate else None, gammas=gammas, rotary_base=base, pos_offset=pos)
    ref = oracle.parallel_grad(q.f64, k.f64, v.f64, dout.f64, g=g.f64 if gate else None, gammas=gammas,
                               rotary_base=base, pos_offset=pos)
    return [None if x is None else to64(x) for x in got], ref


BF16_CASES = [
    # (batch, seqlen, heads, d, gate, rotary)
    (1, 1, 1, 64, True, False),
    (2, 63, 3, 64, True, True),
    (1, 300, 2, 256, True, True),
    (2, 130, 4, 128, False, False),
    (1, 700, 2, 256, False, True),
]


@pytest.mark.parametrize("b,n,h,d,gate,rot", BF16_CASES)
def test_bf16_parallel_backward(b, n, h, d, gate, rot):
    _announce(form="parallel backward", b=b, n=n, h=h, d=d, gate=gate, rot=rot)
    got, ref = _run(51 + n + d, b, n, h, d, "bf16", 1 / 16, gate, rot, pos=7)
    for name, x, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        if r is None:
            assert x is None
            continue
        assert_close(x, r, "bf16", name)


@pytest.mark.parametrize("d", [64, 256])
def test_f32_parallel_backward(d):
    _announce(form="parallel backward", dtype="f32", d=d)
    got, ref = _run(61 + d, 1, 130, 2, d, "f32", d ** -0.5, True, True, pos=3)
    for name, x, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert_close(x, r, "f32", name)


def test_backward_custom_gammas():
    """Decay 1 (linear attention), 1/2 and a vanishing one."""
    _announce(case="backward custom gammas")
    got, ref = _run(71, 1, 200, 3, 64, "bf16", 1 / 16, True, False, gammas=[1.0, 0.5, 2.0 ** -40])
    for name, x, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert_close(x, r, "bf16", name)


def test_3b_backward_full_size():
    """The 3B workload's shape (batch 4, 2048 tokens, 10 x 256, rotation,
    gate), every gradient against the oracle in full."""
    w = get("retention_3b")
    _announce(workload=w.name, form="parallel backward")
    got, ref = _run(w.seed + 100, w.batch, w.seqlen, w.heads, w.dk, "bf16", w.qkv_scale, True, True,
                    gate_scale=w.gate_scale)
    for name, x, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert_close(x, r, "bf16", name)


def _run_chunk(seed, b, n, h, d, chunk, dtype, scale, gate, rot):
    specs = [((b, n, h, d), scale)] * 3 + [((b, n, h, d), 1 / 8)]
    if gate:
        specs.append(((b, n, h, d), 1 / 16))
    ts = draw(seed, specs, dtype)
    q, k, v, dout = ts[:4]
    g = ts[4] if gate else None
    base = 10000.0 if rot else 0.0
    args = (q.torch(DEV), k.torch(DEV), v.torch(DEV), dout.torch(DEV), g.torch(DEV) if gate else None)
    got = rr.chunkwise_bwd(*args, chunk=chunk, rotary_base=base, pos_offset=11)
    par = rr.parallel_bwd(*args, rotary_base=base, pos_offset=11)
    ref = oracle.parallel_grad(q.f64, k.f64, v.f64, dout.f64, g=g.f64 if gate else None, rotary_base=base,
                               pos_offset=11)
    return [None if x is None else to64(x) for x in got], [None if x is None else to64(x) for x in par], ref


CHUNK_CASES = [
    # (batch, seqlen, heads, d, chunk, gate, rotary)
    (1, 1, 1, 64, 64, True, False),
    (2, 300, 2, 256, 64, True, True),
    (1, 700, 2, 128, 512, False, True),
    (2, 130, 4, 64, 7, True, False),
    (1, 8192, 2, 256, 512, True, False),
]


@pytest.mark.parametrize("b,n,h,d,chunk,gate,rot", CHUNK_CASES)
def test_bf16_chunkwise_backward(b, n, h, d, chunk, gate, rot):
    """The chunkwise backward against the fp64 gradients of the (same)
    function, and against the parallel backward on the GPU."""
    _announce(form="chunkwise backward", b=b, n=n, h=h, d=d, chunk=chunk, gate=gate, rot=rot)
    got, par, ref = _run_chunk(81 + n + chunk, b, n, h, d, chunk, "bf16", 1 / 16, gate, rot)
    for name, x, p, r in zip(("dq", "dk", "dv", "dg"), got, par, ref):
        if r is None:
            assert x is None
            continue
        assert_close(x, r, "bf16", name)
        assert_close(x, p, "bf16", name + " vs parallel backward")


def test_f32_chunkwise_backward():
    _announce(form="chunkwise backward", dtype="f32")
    got, _, ref = _run_chunk(91, 1, 200, 2, 128, 64, "f32", 128 ** -0.5, True, True)
    for name, x, r in zip(("dq", "dk", "dv", "dg"), got, ref):
        assert_close(x, r, "f32", name)


STATE_CASES = [
    # (batch, seqlen, heads, d, chunk, dtype, gate, rotary, state_in, d_state_out)
    (2, 300, 2, 256, 64, "bf16", True, True, True, True),
    (1, 130, 3, 128, 512, "bf16", False, False, True, False),
    (1, 200, 2, 64, 7, "bf16", True, False, False, True),
    (1, 150, 2, 128, 64, "f32", True, True, True, True),
    # two state workgroups per chunk (fp32, d = 256), each writing its rows
    # of the partner product's snapshots
    (1, 100, 2, 256, 32, "f32", True, False, True, True),
    (1, 200, 2, 64, 64, "bf16", False, True, False, True),
]


@pytest.mark.parametrize("b,n,h,d,chunk,dtype,gate,rot,s_in,dso", STATE_CASES)
def test_chunkwise_backward_with_state(b, n, h, d, chunk, dtype, gate, rot, s_in, dso):
    """Carried state: dq, dk, dv, dg and the state-in gradient, with the
    state-out gradient in the loss, against the fp64 oracle."""
    import torch

    _announce(form="chunkwise backward with state", b=b, n=n, h=h, d=d, chunk=chunk, dtype=dtype, gate=gate, rot=rot,
              state_in=s_in, d_state_out=dso)
    scale = d ** -0.5 if dtype == "f32" else 1 / 16
    specs = [((b, n, h, d), scale)] * 3 + [((b, n, h, d), 1 / 8)] + ([((b, n, h, d), 1 / 16)] if gate else [])
    ts = draw(123 + n + d, specs, dtype)
    q, k, v, dout = ts[:4]
    g = ts[4] if gate else None
    rng = np.random.default_rng(7 + n)
    s0 = (rng.standard_normal((b, h, d, d)) * 0.05).astype(np.float32) if s_in else None
    dso_a = (rng.standard_normal((b, h, d, d)) * 0.05).astype(np.float32) if dso else None
    base = 10000.0 if rot else 0.0
    t = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    got = rr.chunkwise_bwd(q.torch(DEV), k.torch(DEV), v.torch(DEV), dout.torch(DEV), g.torch(DEV) if gate else None,
                           chunk=chunk, state_in=t(s0), d_state_out=t(dso_a), rotary_base=base, pos_offset=4)
    ref = oracle.chunkwise_state_grad(q.f64, k.f64, v.f64, dout.f64, g=g.f64 if gate else None,
                                      state_in=None if s0 is None else s0.astype(np.float64),
                                      d_state_out=None if dso_a is None else dso_a.astype(np.float64),
                                      rotary_base=base, pos_offset=4)
    names = ("dq", "dk", "dv", "dg", "d_state_in")
    for i, name in enumerate(names[:len(got)]):
        r = ref[i]
        if r is None:
            assert got[i] is None
            continue
        assert_close(to64(got[i]), r, dtype, name)


GENERIC_GAMMAS = [1.0, 0.25, 2.0 ** -40, 0.999]


@pytest.mark.parametrize("chunk,s_in", [(512, True), (64, False)])
def test_chunkwise_backward_generic_decays(chunk, s_in):
    """Decays 0.25 and 2^-40 give |log2 g| x chunk > 64, so the three gradient
    products and the recomputed forward run the generic instantiations (an
    exact decay factor per score and the rescaled cross term), with the gate,
    a carried state and the state-out gradient; checked head by head against
    the fp64 oracle."""
    import torch

    b, n, h, d = 1, 700, 4, 256
    _announce(form="chunkwise backward, generic decays", chunk=chunk, state_in=s_in, gammas=GENERIC_GAMMAS)
    ts = draw(907 + chunk, [((b, n, h, d), 1 / 16)] * 3 + [((b, n, h, d), 1 / 8), ((b, n, h, d), 1 / 16)], "bf16")
    q, k, v, dout, g = ts
    rng = np.random.default_rng(31 + chunk)
    s0 = (rng.standard_normal((b, h, d, d)) * 0.05).astype(np.float32) if s_in else None
    dso = (rng.standard_normal((b, h, d, d)) * 0.05).astype(np.float32)
    t = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    got = rr.chunkwise_bwd(q.torch(DEV), k.torch(DEV), v.torch(DEV), dout.torch(DEV), g.torch(DEV), chunk=chunk,
                           state_in=t(s0), d_state_out=t(dso), gammas=GENERIC_GAMMAS, check=True)
    ref = oracle.chunkwise_state_grad(q.f64, k.f64, v.f64, dout.f64, g=g.f64,
                                      state_in=None if s0 is None else s0.astype(np.float64),
                                      d_state_out=dso.astype(np.float64), gammas=GENERIC_GAMMAS)
    for name, x, r in zip(("dq", "dk", "dv", "dg", "d_state_in"), got, ref):
        if r is None:
            assert x is None
            continue
        x = to64(x)
        assert_close(x, r, "bf16", name)
        if x.ndim == 4 and name != "d_state_in":
            for hd in range(h):
                assert_close(x[:, :, hd:hd + 1], r[:, :, hd:hd + 1], "bf16", f"{name} head {hd}")


def test_chunkwise_backward_repeatable_on_one_workspace():
    """Calls on one workspace return bit-identical gradients, with and without
    a carried state, whatever the workspace held before (it is filled with
    random bytes between calls): each call clears its control blocks, and the
    snapshots one product's state workgroups write for another are complete
    before that product reads them."""
    import torch

    b, n, h, d, chunk = 2, 2048, 8, 256, 256
    _announce(form="chunkwise backward, repeated on one workspace", b=b, n=n, h=h, d=d, chunk=chunk)
    ts = draw(501, [((b, n, h, d), 1 / 16)] * 3 + [((b, n, h, d), 1 / 8), ((b, n, h, d), 1 / 16)], "bf16")
    q, k, v, dout, g = (t.torch(DEV) for t in ts)
    rng = np.random.default_rng(17)
    s0 = torch.from_numpy((rng.standard_normal((b, h, d, d)) * 0.05).astype(np.float32)).to(DEV)
    dso = torch.from_numpy((rng.standard_normal((b, h, d, d)) * 0.05).astype(np.float32)).to(DEV)
    ws = torch.empty(256 << 20, dtype=torch.uint8, device=DEV)
    for kw in ({}, {"state_in": s0, "d_state_out": dso}):
        runs = []
        for _ in range(3):
            ws.random_(0, 256)
            runs.append([x.clone() for x in rr.chunkwise_bwd(q, k, v, dout, g, chunk=chunk, workspace=ws, check=True,
                                                             **kw)])
        for other in runs[1:]:
            for x, y in zip(runs[0], other):
                assert torch.equal(x, y)
