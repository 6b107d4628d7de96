"""Pins of the fp64 oracle to things other than itself.

Each test fixes the oracle against a fact the pages or the mathematics fix:
the forms' equivalence (Spiral-RetNet-3b card, "Visualization of the retention
mechanism"; Elamur summary of "Retentive Network: A Successor to Transformer",
Summary), the per-head decay formula (same summary, Key points, fifth item),
closed forms, special cases that reduce to a library routine, brute force on
tiny exact inputs, and structural invariants. Pure CPU.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from synth import get

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, shape, scale=1.0):
    return rng.standard_normal(size=shape) * scale


def _qkv(seed, b, n, h, dk, dv, scale=0.5):
    rng = np.random.default_rng(seed)
    return _rand(rng, (b, n, h, dk), scale), _rand(rng, (b, n, h, dk), scale), _rand(rng, (b, n, h, dv), scale)


# ---------------------------------------------------------------------------
# P-d: per-head decay table, Key points (fifth item): gamma_i = 1 - 2^(-5-i)
# ---------------------------------------------------------------------------
def test_default_gamma_table_matches_page_formula():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "gamma_table.txt")) if not ln.startswith("#")]
    table = oracle.default_gammas(len(rows))
    for i, num, den in rows:
        assert table[int(i)] == int(num) / int(den)  # exact: both sides are dyadic
    assert table[0] == 0.96875 and table[1] == 0.984375
    assert table[15] == 1.0 - 2.0 ** -20
    # exact in fp32 as well for i <= 18 (24-bit significand)
    assert np.all(table[:19].astype(np.float32).astype(np.float64) == table[:19])


# ---------------------------------------------------------------------------
# P-b: brute force on tiny exact inputs. Small integers and dyadic decays make
# every operation exact in fp64, so all three forms must be bit-identical to
# the plain sum o_n = sum_{m<=n} g^(n-m) (q_n . k_m) v_m + g^(n+1) q_n S0,
# whatever order each form adds in.
# ---------------------------------------------------------------------------
def _brute(q, k, v, gammas, s0):
    bsz, n_tok, heads, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((bsz, n_tok, heads, dv))
    for b in range(bsz):
        for h in range(heads):
            gam = gammas[h]
            for n in range(n_tok):
                for j in range(dv):
                    acc = 0.0
                    for m in range(n + 1):
                        dot = sum(q[b, n, h, i] * k[b, m, h, i] for i in range(dk))
                        acc += gam ** (n - m) * dot * v[b, m, h, j]
                    acc += gam ** (n + 1) * sum(q[b, n, h, i] * s0[b, h, i, j] for i in range(dk))
                    out[b, n, h, j] = acc
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_all_forms_bit_exact_against_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    b, n, h, dk, dv = 2, 11, 2, 3, 4
    q = rng.integers(-3, 4, size=(b, n, h, dk)).astype(np.float64)
    k = rng.integers(-3, 4, size=(b, n, h, dk)).astype(np.float64)
    v = rng.integers(-3, 4, size=(b, n, h, dv)).astype(np.float64)
    s0 = rng.integers(-3, 4, size=(b, h, dk, dv)).astype(np.float64)
    gammas = np.array([0.5, 0.75])
    ref = _brute(q, k, v, gammas, s0)
    assert np.array_equal(oracle.parallel(q, k, v, gammas, state_in=s0), ref)
    out_r, _ = oracle.recurrent(q, k, v, gammas, state_in=s0)
    assert np.array_equal(out_r, ref)
    for chunk in (1, 3, 4, n):
        out_c, _ = oracle.chunkwise(q, k, v, gammas, chunk, state_in=s0)
        assert np.array_equal(out_c, ref), chunk


# ---------------------------------------------------------------------------
# P-a: the three forms agree (Spiral-RetNet card, "Visualization of the
# retention mechanism"; Elamur summary, Summary) to 1e-10, with rotation,
# ragged last chunks and a carried-in state.
# ---------------------------------------------------------------------------
def test_forms_agree_on_tiny_fp32_workload():
    w = get("tiny_fp32")
    q, k, v, _ = w.inputs()
    outs = {}
    for form in w.forms:
        outs[form], _ = oracle.retention(form, q.f64, k.f64, v.f64, rotary_base=w.rotary_base,
                                         chunk=w.chunk)
    assert np.max(np.abs(outs["parallel"] - outs["recurrent"])) <= 1e-10
    assert np.max(np.abs(outs["chunkwise"] - outs["recurrent"])) <= 1e-10


@pytest.mark.parametrize("n,chunk", [(63, 16), (100, 32), (130, 64)])
def test_forms_agree_ragged_with_state(n, chunk):
    q, k, v = _qkv(7 + n, 2, n, 3, 8, 5)
    rng = np.random.default_rng(n)
    s0 = rng.standard_normal((2, 3, 8, 5))
    gammas = oracle.default_gammas(3)
    par = oracle.parallel(q, k, v, gammas, state_in=s0)
    rec, st_r = oracle.recurrent(q, k, v, gammas, state_in=s0)
    chk, st_c = oracle.chunkwise(q, k, v, gammas, chunk, state_in=s0)
    assert np.max(np.abs(par - rec)) <= 1e-10
    assert np.max(np.abs(chk - rec)) <= 1e-10
    assert np.max(np.abs(st_c - st_r)) <= 1e-10


# ---------------------------------------------------------------------------
# P-c: decay 1 is causal linear attention with identity features and no
# normaliser (Linear Transformer, a comparison model on the Elamur summary):
# o_n = q_n . cumsum_m(k_m^T v_m), computed with numpy cumsum.
# ---------------------------------------------------------------------------
def test_gamma_one_is_causal_linear_attention():
    q, k, v = _qkv(3, 2, 40, 2, 6, 7)
    outer = k[..., :, None] * v[..., None, :]  # [B, N, H, dk, dv]
    prefix = np.cumsum(outer, axis=1)
    ref = np.einsum("bnhi,bnhij->bnhj", q, prefix)
    ones = np.ones(2)
    assert np.max(np.abs(oracle.parallel(q, k, v, ones) - ref)) <= 1e-12
    assert np.max(np.abs(oracle.recurrent(q, k, v, ones)[0] - ref)) <= 1e-12
    assert np.max(np.abs(oracle.chunkwise(q, k, v, ones, 9)[0] - ref)) <= 1e-12
    assert np.max(np.abs(oracle.recurrent(q, k, v, ones)[1] - prefix[:, -1])) <= 1e-12


# ---------------------------------------------------------------------------
# P-e: constant inputs. With q_m = q, k_m = k, v_m = v the sum is geometric:
# o_n = (q.k) v (1 - g^(n+1)) / (1 - g), final state k^T v (1 - g^N) / (1 - g).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("form", ["parallel", "recurrent", "chunkwise"])
def test_constant_inputs_geometric_closed_form(form):
    rng = np.random.default_rng(5)
    n_tok, heads, dk, dv = 50, 3, 4, 6
    qv, kv, vv = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
    q = np.broadcast_to(qv, (1, n_tok, heads, dk)).copy()
    k = np.broadcast_to(kv, (1, n_tok, heads, dk)).copy()
    v = np.broadcast_to(vv, (1, n_tok, heads, dv)).copy()
    gammas = oracle.default_gammas(heads)
    out, state = oracle.retention(form, q, k, v, gammas=gammas, chunk=16)
    n = np.arange(n_tok)
    for h in range(heads):
        gam = gammas[h]
        series = (1 - gam ** (n + 1)) / (1 - gam)
        ref = (qv @ kv) * series[:, None] * vv[None, :]
        assert np.max(np.abs(out[0, :, h] - ref)) <= 1e-11 * max(1.0, np.max(np.abs(ref)))
        if state is not None:
            ref_s = np.outer(kv, vv) * (1 - gam ** n_tok) / (1 - gam)
            assert np.max(np.abs(state[0, h] - ref_s)) <= 1e-11 * np.max(np.abs(ref_s))


# ---------------------------------------------------------------------------
# P-f: a vanishing decay leaves only the diagonal term: o_n -> (q_n.k_n) v_n.
# ---------------------------------------------------------------------------
def test_tiny_gamma_keeps_only_the_diagonal():
    q, k, v = _qkv(11, 1, 30, 2, 5, 5)
    gammas = np.array([2.0 ** -60, 2.0 ** -60])
    ref = np.einsum("bnhi,bnhi->bnh", q, k)[..., None] * v
    for form in ("parallel", "recurrent", "chunkwise"):
        out, _ = oracle.retention(form, q, k, v, gammas=gammas, chunk=7)
        assert np.max(np.abs(out - ref)) <= 1e-15, form


# ---------------------------------------------------------------------------
# P-g: the chunk size does not change the result; chunk 1 is the recurrent
# form and chunk N the parallel form (this pins the decay vectors xi, zeta and
# the g^b factor of the chunkwise form).
# ---------------------------------------------------------------------------
def test_chunk_size_invariance():
    q, k, v = _qkv(13, 2, 64, 2, 8, 8)
    gammas = oracle.default_gammas(2)
    ref, st_ref = oracle.recurrent(q, k, v, gammas)
    for chunk in (1, 7, 64, 1000):
        out, st = oracle.chunkwise(q, k, v, gammas, chunk)
        assert np.max(np.abs(out - ref)) <= 1e-10, chunk
        assert np.max(np.abs(st - st_ref)) <= 1e-10, chunk
    assert np.max(np.abs(oracle.chunkwise(q, k, v, gammas, 64)[0] - oracle.parallel(q, k, v, gammas))) <= 1e-10


# ---------------------------------------------------------------------------
# P-h: the state is a checkpoint. A split prefill (with the second part's
# positions continuing) equals the whole prefill; a prefill followed by
# single-token steps equals the tail of a longer prefill.
# ---------------------------------------------------------------------------
def test_split_prefill_and_decode_resume():
    q, k, v = _qkv(17, 2, 90, 2, 8, 6)
    g = np.random.default_rng(1).standard_normal(v.shape)
    base = 10000.0
    whole, st_whole = oracle.retention("chunkwise", q, k, v, g=g, rotary_base=base, chunk=16)
    n1 = 37
    a, st_a = oracle.retention("chunkwise", q[:, :n1], k[:, :n1], v[:, :n1], g=g[:, :n1], rotary_base=base,
                               chunk=16)
    b, st_b = oracle.retention("chunkwise", q[:, n1:], k[:, n1:], v[:, n1:], g=g[:, n1:], rotary_base=base,
                               pos_offset=n1, chunk=16, state_in=st_a)
    assert np.max(np.abs(np.concatenate([a, b], axis=1) - whole)) <= 1e-9
    assert np.max(np.abs(st_b - st_whole)) <= 1e-10
    # prefill 80 tokens, then 10 decode steps
    n0 = 80
    _, st = oracle.retention("chunkwise", q[:, :n0], k[:, :n0], v[:, :n0], rotary_base=base, chunk=16)
    for t in range(n0, 90):
        o, st = oracle.recurrent_step(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], st, oracle.default_gammas(2),
                                      g=g[:, t:t + 1], rotary_base=base, pos=t)
        assert np.max(np.abs(o[:, 0] - whole[:, t])) <= 1e-9
    assert np.max(np.abs(st - st_whole)) <= 1e-10


# ---------------------------------------------------------------------------
# P-i: without the GroupNorm epilogue the output is linear in V.
# ---------------------------------------------------------------------------
def test_linear_in_values():
    q, k, v1 = _qkv(19, 1, 33, 2, 4, 4)
    v2 = np.random.default_rng(2).standard_normal(v1.shape)
    gammas = oracle.default_gammas(2)
    for form in ("parallel", "recurrent", "chunkwise"):
        o1, _ = oracle.retention(form, q, k, v1, gammas=gammas, chunk=8)
        o2, _ = oracle.retention(form, q, k, v2, gammas=gammas, chunk=8)
        o12, _ = oracle.retention(form, q, k, v1 + v2, gammas=gammas, chunk=8)
        o3, _ = oracle.retention(form, q, k, -2.5 * v1, gammas=gammas, chunk=8)
        assert np.max(np.abs(o12 - (o1 + o2))) <= 1e-12
        assert np.max(np.abs(o3 + 2.5 * o1)) <= 1e-12


# ---------------------------------------------------------------------------
# P-j: rotation. Pairs turn like complex numbers multiplied by e^{i t theta_j}
# (checked with numpy complex arithmetic); the norm is kept; base 0 is the
# identity; and q_n . k_m depends only on n - m, so shifting every position
# leaves the parallel-form output unchanged.
# ---------------------------------------------------------------------------
def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((2, 9, 3, 8))
    base, off = 10000.0, 5
    y = oracle.rotate(x, base, off)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = np.array([base ** (-2.0 * j / 8) for j in range(4)])
    t = off + np.arange(9)
    rot = z * np.exp(1j * t[None, :, None, None] * theta[None, None, None, :])
    assert np.max(np.abs(y[..., 0::2] - rot.real)) <= 1e-14
    assert np.max(np.abs(y[..., 1::2] - rot.imag)) <= 1e-14
    assert np.max(np.abs(np.linalg.norm(y, axis=-1) - np.linalg.norm(x, axis=-1))) <= 1e-13
    assert np.array_equal(oracle.rotate(x, 0.0, 3), x)


def test_rotation_is_relative():
    q, k, v = _qkv(29, 1, 48, 2, 8, 4)
    a, _ = oracle.retention("parallel", q, k, v, rotary_base=10000.0, pos_offset=0)
    b, _ = oracle.retention("parallel", q, k, v, rotary_base=10000.0, pos_offset=1234)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))


# ---------------------------------------------------------------------------
# P-k: the epilogue equals torch's group_norm (one group per head, no affine)
# followed by silu, in fp64 on the CPU.
# ---------------------------------------------------------------------------
def test_epilogue_matches_torch_group_norm_and_silu():
    rng = np.random.default_rng(31)
    bsz, n_tok, heads, dv = 2, 5, 3, 16
    o = rng.standard_normal((bsz, n_tok, heads, dv)) * 3 + 1
    g = rng.standard_normal((bsz, n_tok, heads, dv))
    eps = 1e-5
    ours = oracle.group_norm_swish(o, g, eps)
    t = torch.from_numpy(o.reshape(bsz * n_tok, heads * dv))
    gn = torch.nn.functional.group_norm(t, heads, eps=eps).reshape(bsz, n_tok, heads, dv)
    ref = gn * torch.nn.functional.silu(torch.from_numpy(g))
    assert np.max(np.abs(ours - ref.numpy())) <= 1e-12


# ---------------------------------------------------------------------------
# P-l: causality: changing token t leaves every earlier output bit-identical.
# ---------------------------------------------------------------------------
def test_causality():
    q, k, v = _qkv(37, 1, 40, 2, 4, 4)
    g = np.random.default_rng(3).standard_normal(v.shape)
    t = 23
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, t] += 1.0
    k2[:, t] -= 2.0
    v2[:, t] *= 3.0
    for form in ("parallel", "recurrent", "chunkwise"):
        a, _ = oracle.retention(form, q, k, v, g=g, rotary_base=10000.0, chunk=8)
        b, _ = oracle.retention(form, q2, k2, v2, g=g, rotary_base=10000.0, chunk=8)
        assert np.array_equal(a[:, :t], b[:, :t]), form
        assert not np.allclose(a[:, t], b[:, t]), form


def test_score_map_pins():
    """The score map against the parallel form's weight matrix built
    independently (scores times the decay mask), and its closed form for
    identical tokens: w[m] = sum_h g_h^(n-m) |q.k|."""
    rng = np.random.default_rng(21)
    b, n, h, d = 2, 9, 3, 4
    q, k = rng.standard_normal((b, n, h, d)), rng.standard_normal((b, n, h, d))
    gam = oracle.default_gammas(h)
    w = oracle.score_map(q, k, rotary_base=100.0, pos_offset=4, query=6)
    qr, kr = oracle.rotate(q, 100.0, 4), oracle.rotate(k, 100.0, 4)
    pos = np.arange(n)
    want = np.zeros((b, n))
    for hh in range(h):
        decay = np.where(pos[:, None] >= pos[None, :], gam[hh] ** np.maximum(pos[:, None] - pos[None, :], 0), 0.0)
        a = np.einsum("bnd,bmd->bnm", qr[:, :, hh], kr[:, :, hh]) * decay[None]
        want += np.abs(a[:, 6, :])
    assert np.allclose(w, want, rtol=1e-13, atol=1e-14)
    assert np.all(w[:, 7:] == 0.0)
    # identical tokens, no rotation: every weight is |q.k| times the decay
    q1 = np.broadcast_to(rng.standard_normal((1, 1, h, d)), (1, n, h, d)).copy()
    k1 = np.broadcast_to(rng.standard_normal((1, 1, h, d)), (1, n, h, d)).copy()
    w1 = oracle.score_map(q1, k1)
    dots = np.abs(np.einsum("hd,hd->h", q1[0, 0], k1[0, 0]))
    for m in range(n):
        assert np.isclose(w1[0, m], np.sum(gam ** (n - 1 - m) * dots), rtol=1e-14)


def test_varlen_pins():
    """Packed sequences of different lengths: each slice against the brute
    force sum (integer inputs, dyadic decays: exact), an empty sequence
    passes its state through, positions restart at each sequence, and equal
    lengths reproduce the batched layout."""
    rng = np.random.default_rng(33)
    h, d = 2, 3
    lens = [4, 0, 1, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    tot = int(cu[-1])
    q, k, v = (rng.integers(-3, 4, size=(tot, h, d)).astype(np.float64) for _ in range(3))
    s0 = rng.integers(-3, 4, size=(len(lens), h, d, d)).astype(np.float64)
    gammas = np.array([0.5, 0.75])
    for form, chunk in (("chunkwise", 4), ("recurrent", None), ("parallel", None)):
        out, st = oracle.retention_varlen(form, q, k, v, cu, gammas=gammas, chunk=chunk,
                                          state_in=None if form == "parallel" else s0)
        for b in range(len(lens)):
            a, e = cu[b], cu[b + 1]
            if e > a:
                s_b = None if form == "parallel" else s0[b:b + 1]
                want = _brute(q[None, a:e], k[None, a:e], v[None, a:e], gammas,
                              s_b if s_b is not None else np.zeros((1, h, d, d)))
                assert np.array_equal(out[None, a:e], want), (form, b)
        if form != "parallel":
            assert np.array_equal(st[1], s0[1])  # the empty sequence
    # rotation positions count from each sequence's first token
    qf, kf, vf = (rng.standard_normal((tot, h, d + 1)) for _ in range(3))
    out, _ = oracle.retention_varlen("chunkwise", qf, kf, vf, cu, rotary_base=50.0, pos_offset=2, chunk=3)
    alone, _ = oracle.retention("chunkwise", qf[None, 5:11], kf[None, 5:11], vf[None, 5:11], rotary_base=50.0,
                                pos_offset=2, chunk=3)
    assert np.allclose(out[5:11], alone[0], rtol=0, atol=1e-14)
    # equal lengths: the packed layout of a batch
    qb, kb, vb, gb = (rng.standard_normal((2, 5, h, 4)) for _ in range(4))
    ref, ref_s = oracle.retention("chunkwise", qb, kb, vb, g=gb, rotary_base=10.0, chunk=2)
    out, st = oracle.retention_varlen("chunkwise", *(x.reshape(10, h, 4) for x in (qb, kb, vb)), [0, 5, 10],
                                      g=gb.reshape(10, h, 4), rotary_base=10.0, chunk=2)
    assert np.array_equal(out, ref.reshape(10, h, 4)) and np.array_equal(st, ref_s)
