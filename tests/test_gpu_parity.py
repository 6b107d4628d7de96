"""GPU parity of the HIP library against the fp64 oracle, at sizes the oracle
finishes in seconds that still span several tiles and ragged tails, plus the
edge cases: a single token, chunk sizes that do not divide the sequence, a
carried state, custom decays (1, 1/2, vanishing), aliased state in/out,
decode after prefill, and bitwise run-to-run determinism."""

import numpy as np
import pytest
import torch

import oracle
import retnet_retention_amd as rr
from synth import get
from tests.gpu_helpers import DEV, assert_close, gpu_run, make_inputs, oracle_run, to64

pytestmark = pytest.mark.gpu


def _announce(**kw):
    print("case:", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


# --- the tiny fp32 workload: all three forms, max-abs 1e-4 -----------------
@pytest.mark.parametrize("form", ["parallel", "chunkwise", "recurrent"])
def test_tiny_fp32_workload(form):
    w = get("tiny_fp32")
    _announce(workload=w.name, form=form)
    q, k, v, g = w.inputs()
    ref, ref_s = oracle_run(form, q, k, v, g, chunk=w.chunk, rotary_base=w.rotary_base)
    out, st = gpu_run(form, q, k, v, g, chunk=w.chunk, rotary_base=w.rotary_base)
    assert_close(out, ref, "f32", f"{form} out")
    if ref_s is not None:
        assert_close(st, ref_s, "f32", f"{form} state")


# --- bf16 shapes: tiles, ragged tails, gate, rotation, carried state -------
BF16_CASES = [
    # (batch, seqlen, heads, d, chunk, gate, rotary, state)
    (1, 1, 1, 64, 64, True, True, False),
    (2, 63, 3, 64, 64, False, False, False),
    (1, 64, 1, 128, 64, True, False, True),
    (2, 65, 3, 256, 64, True, True, False),
    (1, 250, 2, 256, 64, True, True, True),
    (1, 250, 1, 128, 100, False, True, True),
    (2, 300, 2, 64, 7, True, False, True),
    (1, 700, 2, 256, 512, True, True, False),
    (1, 520, 1, 256, 128, False, False, False),
    (2, 600, 2, 256, 256, True, False, True),  # one full 256-row query block per chunk, ragged tail
    (1, 1500, 2, 256, 1024, True, True, True),
]


@pytest.mark.parametrize("b,n,h,d,chunk,gate,rot,state", BF16_CASES)
def test_bf16_chunkwise(b, n, h, d, chunk, gate, rot, state):
    _announce(form="chunkwise", b=b, n=n, h=h, d=d, chunk=chunk, gate=gate, rot=rot, state=state)
    q, k, v, g, s0 = make_inputs(11 + n + d, b, n, h, d, "bf16", 1 / 16, 1.0 if gate else None, state)
    base = 10000.0 if rot else 0.0
    ref, ref_s = oracle_run("chunkwise", q, k, v, g, chunk=chunk, rotary_base=base, pos_offset=3, state_in=s0)
    out, st = gpu_run("chunkwise", q, k, v, g, chunk=chunk, rotary_base=base, pos_offset=3, state_in=s0)
    assert_close(out, ref, "bf16", "out")
    assert_close(st, ref_s, "bf16", "state")


# (2, 300, 4, ...): 8 (sequence, head) pairs, so the grid takes its XCD-aware
# longest-first order, over two query blocks, with rotation from position 1000
@pytest.mark.parametrize("b,n,h,d,gate,rot,pos", [(1, 1, 1, 256, True, False, 0), (2, 63, 3, 64, True, True, 0),
                                                  (1, 200, 2, 128, False, True, 0), (1, 700, 2, 256, True, True, 0),
                                                  (2, 300, 4, 64, True, True, 1000)])
def test_bf16_parallel(b, n, h, d, gate, rot, pos):
    _announce(form="parallel", b=b, n=n, h=h, d=d, gate=gate, rot=rot, pos=pos)
    q, k, v, g, _ = make_inputs(23 + n, b, n, h, d, "bf16", 1 / 16, 1 / 16 if gate else None)
    base = 10000.0 if rot else 0.0
    ref, _ = oracle_run("parallel", q, k, v, g, rotary_base=base, pos_offset=pos)
    out, _ = gpu_run("parallel", q, k, v, g, rotary_base=base, pos_offset=pos)
    assert_close(out, ref, "bf16", "out")


@pytest.mark.parametrize("b,n,h,d,gate,state", [(2, 20, 3, 256, True, True), (3, 9, 2, 64, False, False),
                                                (1, 12, 1, 128, True, True)])
def test_bf16_recurrent(b, n, h, d, gate, state):
    _announce(form="recurrent", b=b, n=n, h=h, d=d, gate=gate, state=state)
    q, k, v, g, s0 = make_inputs(31 + n, b, n, h, d, "bf16", 1 / 16, 1.0 if gate else None, state)
    ref, ref_s = oracle_run("recurrent", q, k, v, g, rotary_base=10000.0, pos_offset=100, state_in=s0)
    out, st = gpu_run("recurrent", q, k, v, g, rotary_base=10000.0, pos_offset=100, state_in=s0)
    assert_close(out, ref, "bf16", "out")
    assert_close(st, ref_s, "bf16", "state")


# --- fp32 at larger head dims ----------------------------------------------
@pytest.mark.parametrize("form", ["parallel", "chunkwise"])
@pytest.mark.parametrize("d", [128, 256])
def test_f32_larger_heads(form, d):
    _announce(form=form, dtype="f32", d=d)
    q, k, v, g, s0 = make_inputs(41 + d, 1, 130, 2, d, "f32", d ** -0.5, None, form == "chunkwise")
    ref, ref_s = oracle_run(form, q, k, v, g, chunk=64, rotary_base=10000.0, state_in=s0)
    out, st = gpu_run(form, q, k, v, g, chunk=64, rotary_base=10000.0, state_in=s0)
    assert_close(out, ref, "f32", "out")
    if ref_s is not None:
        assert_close(st, ref_s, "f32", "state")


# --- decays: 1 (linear attention), 1/2, vanishing ---------------------------
def test_custom_gammas():
    _announce(case="custom gammas")
    gam = [1.0, 0.5, 2.0 ** -40, 0.999]
    q, k, v, g, _ = make_inputs(53, 1, 150, 4, 64, "f32", 1 / 8)
    for form in ("parallel", "chunkwise"):
        ref, _ = oracle_run(form, q, k, v, g, chunk=64, gammas=gam)
        out, _ = gpu_run(form, q, k, v, g, chunk=64, gammas=gam)
        assert_close(out, ref, "f32", form)


# --- bf16 with decays that take the generic decay path ---------------------
GENERIC_GAMMAS = [1.0, 0.25, 2.0 ** -40, 0.999]


@pytest.mark.parametrize("form,gate", [("chunkwise", True), ("chunkwise", False), ("parallel", True),
                                       ("parallel", False)])
def test_bf16_generic_decay_path(form, gate):
    """Decays 0.25 and 2^-40 give |log2 g| x span > 64 at chunk 512 (and over
    the parallel form's 256-row query blocks), so the host launches the
    generic instantiation: an exact decay factor per score, the cross term as
    O = xi (O / xi + Q R) with rows whose xi is below 2^-100 skipping it.
    bf16, d = 256, rotation, chunk 512 over 1100 tokens (a ragged last chunk),
    the chunkwise form from a carried state; every (sequence, head, 64-row
    block) is held to the bar on its own, with and without the gate."""
    b, n, h, d = 2, 1100, 4, 256
    _announce(case="generic decay path", form=form, gate=gate, gammas=GENERIC_GAMMAS)
    q, k, v, g, s0 = make_inputs(151 + gate, b, n, h, d, "bf16", 1 / 16, 1.0 if gate else None, form == "chunkwise")
    kw = dict(chunk=512, rotary_base=10000.0, pos_offset=9, gammas=GENERIC_GAMMAS, state_in=s0)
    ref, ref_s = oracle_run(form, q, k, v, g, **kw)
    out, st = gpu_run(form, q, k, v, g, **kw)
    assert_close(out, ref, "bf16", "out")
    for hh in range(h):
        assert_close(out[:, :, hh:hh + 1], ref[:, :, hh:hh + 1], "bf16", f"out head {hh}")
    if ref_s is not None:
        assert_close(st, ref_s, "bf16", "state")


# --- state in == state out (in place) ---------------------------------------
def test_state_in_out_alias():
    _announce(case="state alias")
    q, k, v, g, s0 = make_inputs(61, 2, 200, 2, 256, "bf16", 1 / 16, 1.0, True)
    ref_out, ref_s = oracle_run("chunkwise", q, k, v, g, chunk=64, state_in=s0)
    st = torch.from_numpy(s0.astype(np.float32)).to(DEV)
    out = rr.chunkwise_fwd(q.torch(DEV), k.torch(DEV), v.torch(DEV), g.torch(DEV), chunk=64, state_in=st,
                           state_out=st)
    torch.cuda.synchronize()
    assert_close(to64(out), ref_out, "bf16", "out")
    assert_close(to64(st), ref_s, "bf16", "state")


# --- many (sequence, head) pairs with a carried-in state --------------------
def test_many_pairs_with_carried_state():
    """1024 pairs, far more than the chip holds workgroups of this kernel at
    once, with a carried-in state: chunk 0's output workgroups wait for their
    state parts, which must not queue behind them. The control word stays
    clear (no wait gave up) and the results match."""
    b, n, h, d, chunk = 64, 77, 16, 64, 64
    _announce(case="many pairs with state", b=b, n=n, h=h, d=d, chunk=chunk)
    q, k, v, g, s0 = make_inputs(83, b, n, h, d, "bf16", 1 / 16, 1.0, True)
    ref, ref_s = oracle_run("chunkwise", q, k, v, g, chunk=chunk, state_in=s0)
    tq, tv = q.torch(DEV), v.torch(DEV)
    ws = torch.empty(rr.chunkwise_workspace_bytes(tq, tv, chunk), dtype=torch.uint8, device=DEV)
    st = torch.empty((b, h, d, d), device=DEV)
    out = rr.chunkwise_fwd(tq, k.torch(DEV), tv, g.torch(DEV), chunk=chunk,
                           state_in=torch.from_numpy(s0.astype(np.float32)).to(DEV), state_out=st, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[4:8].view(torch.int32).item()) == 0
    rr.check_chunkwise(ws)
    assert_close(to64(out), ref, "bf16", "out")
    assert_close(to64(st), ref_s, "bf16", "state")


# --- prefill, then decode steps: the state is the checkpoint ---------------
def test_decode_after_prefill_matches_longer_prefill():
    _announce(case="prefill+decode")
    b, n0, t, h, d = 2, 300, 12, 2, 256
    q, k, v, g, _ = make_inputs(71, b, n0 + t, h, d, "bf16", 1 / 16, 1 / 16)
    ref, _ = oracle_run("chunkwise", q, k, v, g, chunk=128, rotary_base=10000.0)
    tq, tk, tv, tg = q.torch(DEV), k.torch(DEV), v.torch(DEV), g.torch(DEV)
    st = torch.empty((b, h, d, d), device=DEV)
    rr.chunkwise_fwd(tq[:, :n0].contiguous(), tk[:, :n0].contiguous(), tv[:, :n0].contiguous(),
                     tg[:, :n0].contiguous(), chunk=128, state_out=st, rotary_base=10000.0)
    outs = []
    for i in range(t):
        sl = slice(n0 + i, n0 + i + 1)
        outs.append(rr.recurrent_step(tq[:, sl].contiguous(), tk[:, sl].contiguous(), tv[:, sl].contiguous(), st,
                                      tg[:, sl].contiguous(), rotary_base=10000.0, pos=n0 + i))
    torch.cuda.synchronize()
    got = np.concatenate([to64(o) for o in outs], axis=1)
    assert_close(got, ref[:, n0:], "bf16", "decode tail")
    # a split prefill with pos_offset continues the rotation and the state
    st2 = torch.empty_like(st)
    rr.chunkwise_fwd(tq[:, :n0].contiguous(), tk[:, :n0].contiguous(), tv[:, :n0].contiguous(),
                     tg[:, :n0].contiguous(), chunk=128, state_out=st2, rotary_base=10000.0)
    tail = rr.chunkwise_fwd(tq[:, n0:].contiguous(), tk[:, n0:].contiguous(), tv[:, n0:].contiguous(),
                            tg[:, n0:].contiguous(), chunk=128, state_in=st2, rotary_base=10000.0, pos_offset=n0)
    torch.cuda.synchronize()
    assert_close(to64(tail), ref[:, n0:], "bf16", "split prefill tail")


# --- determinism --------------------------------------------------------------
def test_bitwise_determinism():
    _announce(case="determinism")
    q, k, v, g, s0 = make_inputs(81, 2, 1100, 4, 256, "bf16", 1 / 16, 1.0, True)
    args = [x.torch(DEV) for x in (q, k, v, g)]
    s_in = torch.from_numpy(s0.astype(np.float32)).to(DEV)
    runs = []
    for _ in range(3):
        so = torch.empty_like(s_in)
        o = rr.chunkwise_fwd(*args, chunk=512, state_in=s_in, state_out=so)
        p = rr.parallel_fwd(*args, rotary_base=10000.0)
        torch.cuda.synchronize()
        runs.append((o.clone(), so.clone(), p.clone()))
    for r in runs[1:]:
        for a, b in zip(r, runs[0]):
            assert torch.equal(a, b)


# --- NaN in the input propagates instead of hanging or vanishing -------------
def test_nan_propagates_forward_only():
    """A NaN in v at the first token of a chunk reaches that column of every
    later output and no earlier one (inside a chunk 0 * NaN is NaN in IEEE
    arithmetic, for the oracle's matrix product as well)."""
    _announce(case="nan")
    q, k, v, g, _ = make_inputs(91, 1, 150, 1, 64, "f32", 1 / 8)
    tq, tk, tv = q.torch(DEV), k.torch(DEV), v.torch(DEV)
    tv[0, 64, 0, 5] = float("nan")
    out = rr.chunkwise_fwd(tq, tk, tv, chunk=64)
    torch.cuda.synchronize()
    o = out.cpu()
    assert torch.isfinite(o[0, :64]).all()
    assert torch.isnan(o[0, 64:, 0, 5]).all()
    assert torch.isfinite(o[0, 64:, 0, :5]).all()


# --- the chunk-to-chunk hand-off completes: every workgroup ran, no wait
# expired; with 8 | batch*heads the workgroups split into 8 classes (one ticket
# counter each), otherwise they share one counter
@pytest.mark.parametrize("b,h", [(2, 4), (1, 3)])
def test_chunkwise_handoff_completes(b, h):
    _announce(case=f"handoff control block b={b} h={h}")
    n, d, chunk = 1100, 256, 128
    q, k, v, g, s0 = make_inputs(97, b, n, h, d, "bf16", 1 / 16, 1.0, True)
    tq, tk, tv, tg = (x.torch(DEV) for x in (q, k, v, g))
    ws = torch.zeros(rr.chunkwise_workspace_bytes(tq, tv, chunk), dtype=torch.uint8, device=DEV)
    s_in = torch.from_numpy(s0.astype(np.float32)).to(DEV)
    s_out = torch.empty_like(s_in)
    out = rr.chunkwise_fwd(tq, tk, tv, tg, chunk=chunk, state_in=s_in, state_out=s_out, workspace=ws)
    torch.cuda.synchronize()
    ctrl = ws[:64].view(torch.int32).cpu()
    nchunks = -(-n // chunk)
    # one output workgroup (the whole 128-row chunk) and, this grid being
    # small (at most 384 workgroups with one state workgroup per chunk), two
    # state workgroups of 128 rows each per (sequence, head, chunk)
    assert nchunks * b * h * (1 + 1) <= 384
    total = nchunks * b * h * (2 + 1)
    assert int(ctrl[0]) == total
    assert int(ctrl[1]) == 0
    if (b * h) % 8 == 0:
        assert [int(x) for x in ctrl[8:16]] == [total // 8] * 8
    else:
        assert int(ctrl[8]) == total
    ref, ref_s = oracle_run("chunkwise", q, k, v, g, chunk=chunk, state_in=s0)
    assert_close(to64(out), ref, "bf16", "out")
    assert_close(to64(s_out), ref_s, "bf16", "state")


def test_step_with_per_sequence_positions():
    """Continuous batching: five sequences decode one token each at their own
    positions. Each row must equal the oracle step at its position, and be
    bit-identical to the single-position call made at that position."""
    _announce(case="step with per-sequence positions")
    b, h, d = 5, 3, 128
    positions = [0, 7, 100, 8191, 123456]
    q, k, v, g, s0 = make_inputs(97, b, 1, h, d, "bf16", 1 / 16, 1.0, True)
    base = 10000.0
    state = torch.from_numpy(s0.astype(np.float32)).to(DEV)
    pos_t = torch.tensor(positions, dtype=torch.int64, device=DEV)
    out = rr.recurrent_step(q.torch(DEV), k.torch(DEV), v.torch(DEV), state, g.torch(DEV), rotary_base=base,
                            positions=pos_t)
    torch.cuda.synchronize()
    gam = oracle.default_gammas(h)
    for i, pos in enumerate(positions):
        sl = slice(i, i + 1)
        ref_o, ref_s = oracle.recurrent_step(q.f64[sl], k.f64[sl], v.f64[sl], s0[sl], gam, g=g.f64[sl],
                                             rotary_base=base, pos=pos)
        assert_close(to64(out[sl]), ref_o, "bf16", f"out, position {pos}")
        assert_close(to64(state[sl]), ref_s, "bf16", f"state, position {pos}")
        one_state = torch.from_numpy(s0[sl].astype(np.float32)).to(DEV)
        one = rr.recurrent_step(q.torch(DEV)[sl].contiguous(), k.torch(DEV)[sl].contiguous(),
                                v.torch(DEV)[sl].contiguous(), one_state, g.torch(DEV)[sl].contiguous(),
                                rotary_base=base, pos=pos)
        torch.cuda.synchronize()
        assert torch.equal(one, out[sl]) and torch.equal(one_state, state[sl]), f"position {pos}"


@pytest.mark.parametrize("b,n,h,d,dtype,rot,query", [(1, 1, 1, 64, "bf16", False, -1), (2, 300, 3, 256, "bf16", True, -1),
                                                     (2, 130, 10, 128, "bf16", True, 57),
                                                     (1, 200, 2, 64, "f32", True, 150),
                                                     (4, 2048, 10, 256, "bf16", True, -1)])
def test_score_map(b, n, h, d, dtype, rot, query):
    """One query token's retention weights over the tokens before it, summed
    over heads (the last case is the 3B workload's shape)."""
    _announce(case="score map", b=b, n=n, h=h, d=d, dtype=dtype, rot=rot, query=query)
    q, k, _, _, _ = make_inputs(103 + n + d, b, n, h, d, dtype, d ** -0.5 if dtype == "f32" else 1 / 16)
    base = 10000.0 if rot else 0.0
    got = to64(rr.score_map(q.torch(DEV), k.torch(DEV), query=query, rotary_base=base, pos_offset=5))
    ref = oracle.score_map(q.f64, k.f64, rotary_base=base, pos_offset=5, query=query)
    assert_close(got, ref, dtype, "scores")
    last = n - 1 if query < 0 else query
    assert np.all(got[:, last + 1:] == 0.0)


@pytest.mark.parametrize("form", ["parallel", "chunkwise", "recurrent"])
def test_max_heads_and_far_positions(form):
    """128 heads (the most a call takes) at d = 64, rotation from position
    10^9 (the angle table is formed in fp64 before rounding), every form."""
    _announce(case="max heads, far positions", form=form)
    b, n, h, d = 1, 70 if form != "recurrent" else 5, 128, 64
    q, k, v, g, s0 = make_inputs(131, b, n, h, d, "bf16", 1 / 16, 1.0, form != "parallel")
    kw = dict(rotary_base=10000.0, pos_offset=10 ** 9)
    ref, ref_s = oracle_run(form, q, k, v, g, chunk=32, state_in=s0, **kw)
    out, st = gpu_run(form, q, k, v, g, chunk=32, state_in=s0, **kw)
    assert_close(out, ref, "bf16", "out")
    if ref_s is not None:
        assert_close(st, ref_s, "bf16", "state")


def test_step_inactive_slots():
    """A negative position marks an inactive slot: its state is untouched and
    its output is zero; the active rows match the oracle."""
    _announce(case="step with inactive slots")
    b, h, d = 4, 2, 64
    positions = [5, -1, 300, -7]
    q, k, v, g, s0 = make_inputs(111, b, 1, h, d, "bf16", 1 / 16, 1.0, True)
    state = torch.from_numpy(s0.astype(np.float32)).to(DEV)
    before = state.clone()
    pos_t = torch.tensor(positions, dtype=torch.int64, device=DEV)
    out = rr.recurrent_step(q.torch(DEV), k.torch(DEV), v.torch(DEV), state, g.torch(DEV), rotary_base=10000.0,
                            positions=pos_t)
    torch.cuda.synchronize()
    gam = oracle.default_gammas(h)
    for i, pos in enumerate(positions):
        if pos < 0:
            assert torch.equal(state[i], before[i]) and torch.count_nonzero(out[i]) == 0
            continue
        sl = slice(i, i + 1)
        ref_o, ref_s = oracle.recurrent_step(q.f64[sl], k.f64[sl], v.f64[sl], s0[sl], gam, g=g.f64[sl],
                                             rotary_base=10000.0, pos=pos)
        assert_close(to64(out[sl]), ref_o, "bf16", f"out, position {pos}")
        assert_close(to64(state[sl]), ref_s, "bf16", f"state, position {pos}")


def test_graph_replay_matches_eager():
    """A chunkwise prefill, a decode step and a packed (varlen) prefill
    captured into one HIP graph: every
    replay (with eager work and synchronizations in between) must give the
    eager results bit for bit (the control-block reset is a kernel, not a
    memset, and nothing in the calls allocates)."""
    _announce(case="graph replay")
    b, n, h, d, chunk = 2, 300, 2, 128, 64
    q, k, v, g, _ = make_inputs(141, b, n, h, d, "bf16", 1 / 16, 1.0)
    q1, k1, v1, g1, _ = make_inputs(142, b, 1, h, d, "bf16", 1 / 16, 1.0)
    tq, tk, tv, tg = (x.torch(DEV) for x in (q, k, v, g))
    sq, sk, sv, sg = (x.torch(DEV) for x in (q1, k1, v1, g1))
    out = torch.empty_like(tv)
    state = torch.empty((b, h, d, d), device=DEV)
    step_out = torch.empty_like(sv)
    ws = torch.empty(rr.chunkwise_workspace_bytes(tq, tv, chunk, rotary_base=10000.0), dtype=torch.uint8,
                     device=DEV)
    # the same tokens packed as three sequences of 300, 0 and 177 tokens
    lens = (300, 0, 177)
    cu = torch.tensor([0, 300, 300, 477], dtype=torch.int32, device=DEV)
    pq, pk, pv, pg = (x.reshape(b * n, h, d)[:477].contiguous() for x in (tq, tk, tv, tg))
    pout = torch.empty_like(pv)
    pstate = torch.empty((len(lens), h, d, d), device=DEV)
    pws = torch.empty(rr.chunkwise_varlen_workspace_bytes(len(lens), n, h, d, torch.bfloat16, chunk, 10000.0),
                      dtype=torch.uint8, device=DEV)

    def work():
        rr.chunkwise_fwd(tq, tk, tv, tg, chunk=chunk, state_out=state, out=out, workspace=ws, rotary_base=10000.0)
        rr.recurrent_step(sq, sk, sv, state, sg, rotary_base=10000.0, pos=n, out=step_out)
        rr.chunkwise_varlen_fwd(pq, pk, pv, cu, n, pg, chunk=chunk, state_out=pstate, out=pout, workspace=pws,
                                rotary_base=10000.0)

    work()
    torch.cuda.synchronize()
    ref = (out.clone(), state.clone(), step_out.clone(), pout.clone(), pstate.clone())
    # the packed call's first sequence is the batched call's first sequence
    assert torch.equal(pout[:300], out[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(3):
        out.zero_()
        state.fill_(7.0)
        step_out.zero_()
        pout.zero_()
        pstate.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((out, state, step_out, pout, pstate), ref,
                                   ("out", "state", "step", "packed out", "packed state")):
            assert torch.equal(got, want), f"replay {rep}: {name}"
        rr.parallel_fwd(tq, tk, tv, tg)  # eager work between replays
        torch.cuda.synchronize()
