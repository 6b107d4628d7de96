"""Pins of the fp64 gradient oracle (no GPU): finite differences of the
forward oracle, brute-force loops at decay 1, and the rotation's transpose.
A dropped term, a wrong sign, a transposed operand or a wrong decay exponent
anywhere in the gradients fails one of these."""

import numpy as np
import pytest

import oracle
from oracle.retention_grad import forward_for_check


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _fd_grad(f, x, h=1e-6):
    """Central differences of the scalar f at x, element by element."""
    out = np.zeros_like(x)
    flat = x.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        flat[i] = keep + h
        up = f()
        flat[i] = keep - h
        down = f()
        flat[i] = keep
        out.reshape(-1)[i] = (up - down) / (2 * h)
    return out


@pytest.mark.parametrize("gate,rot", [(True, True), (False, True), (True, False), (False, False)])
def test_gradients_match_finite_differences(gate, rot):
    rng = np.random.default_rng(3 + 2 * gate + rot)
    b, n, h, d = 1, 7, 2, 4
    q, k, v = _rand(rng, b, n, h, d) * 0.7, _rand(rng, b, n, h, d) * 0.7, _rand(rng, b, n, h, d)
    g = _rand(rng, b, n, h, d) if gate else None
    dout = _rand(rng, b, n, h, d)
    gam = [0.9, 0.55]
    base, pos = (10000.0, 5) if rot else (0.0, 0)

    def loss():
        return float((dout * forward_for_check(q, k, v, g, gammas=gam, rotary_base=base, pos_offset=pos)).sum())

    dq, dk, dv, dg = oracle.parallel_grad(q, k, v, dout, g=g, gammas=gam, rotary_base=base, pos_offset=pos)
    for name, x, an in (("q", q, dq), ("k", k, dk), ("v", v, dv)) + ((("g", g, dg),) if gate else ()):
        fd = _fd_grad(loss, x)
        assert np.max(np.abs(fd - an)) < 1e-6 * max(1.0, np.max(np.abs(fd))), name
    if not gate:
        assert dg is None


def test_gradients_of_the_recurrent_form():
    """The same gradients differentiate the recurrence (the forms are one
    function): finite differences through the recurrent oracle."""
    rng = np.random.default_rng(11)
    b, n, h, d = 2, 6, 1, 3
    q, k, v, dout = (_rand(rng, b, n, h, d) for _ in range(4))
    gam = [0.8]

    def loss():
        out, _ = oracle.retention("recurrent", q, k, v, gammas=gam)
        return float((dout * out).sum())

    dq, dk, dv, _ = oracle.parallel_grad(q, k, v, dout, gammas=gam)
    for x, an in ((q, dq), (k, dk), (v, dv)):
        assert np.max(np.abs(_fd_grad(loss, x) - an)) < 1e-6


def test_decay_one_against_loops():
    """Decay 1, no gate, no rotation: o_n = sum_{m<=n} (q_n.k_m) v_m, whose
    gradients written as plain loops are
        dv_m = sum_{n>=m} (q_n.k_m) dout_n
        dq_n = sum_{m<=n} (dout_n.v_m) k_m
        dk_m = sum_{n>=m} (dout_n.v_m) q_n
    With small integers every value is exact in fp64."""
    rng = np.random.default_rng(5)
    n, d = 6, 3
    q, k, v, dout = (rng.integers(-3, 4, size=(1, n, 1, d)).astype(np.float64) for _ in range(4))
    dq, dk, dv, _ = oracle.parallel_grad(q, k, v, dout, gammas=[1.0])
    Q, K, V, G = q[0, :, 0], k[0, :, 0], v[0, :, 0], dout[0, :, 0]
    for m in range(n):
        assert np.array_equal(dv[0, m, 0], sum(np.dot(Q[t], K[m]) * G[t] for t in range(m, n)))
        assert np.array_equal(dk[0, m, 0], sum(np.dot(G[t], V[m]) * Q[t] for t in range(m, n)))
    for t in range(n):
        assert np.array_equal(dq[0, t, 0], sum(np.dot(G[t], V[m]) * K[m] for m in range(t + 1)))


def test_unrotate_is_the_transpose_of_rotate():
    rng = np.random.default_rng(9)
    x, y = _rand(rng, 2, 5, 3, 8), _rand(rng, 2, 5, 3, 8)
    rx = oracle.rotate(x, 10000.0, 17)
    assert np.allclose(oracle.unrotate(rx, 10000.0, 17), x, atol=1e-13)
    assert abs((rx * y).sum() - (x * oracle.unrotate(y, 10000.0, 17)).sum()) < 1e-12


@pytest.mark.parametrize("gate,rot,dso", [(True, True, True), (False, False, True), (True, False, False)])
def test_state_gradients_match_finite_differences(gate, rot, dso):
    """Carried state: finite differences of sum(dout * out) + sum(dS * S_N)
    through the chunkwise oracle (its state in and state out)."""
    rng = np.random.default_rng(31 + 4 * gate + 2 * rot + dso)
    b, n, h, d, chunk = 1, 7, 2, 4, 3
    q, k, v = (_rand(rng, b, n, h, d) * 0.7 for _ in range(3))
    g = _rand(rng, b, n, h, d) if gate else None
    dout = _rand(rng, b, n, h, d)
    s0 = _rand(rng, b, h, d, d) * 0.5
    dso_t = _rand(rng, b, h, d, d) if dso else None
    gam = [0.9, 0.6]
    base = 100.0 if rot else 0.0

    def loss():
        out, st = oracle.retention("chunkwise", q, k, v, g=g, gammas=gam, rotary_base=base, pos_offset=2,
                                   chunk=chunk, state_in=s0)
        total = float((dout * out).sum())
        return total + (float((dso_t * st).sum()) if dso else 0.0)

    got = oracle.chunkwise_state_grad(q, k, v, dout, g=g, state_in=s0, d_state_out=dso_t, gammas=gam,
                                      rotary_base=base, pos_offset=2)
    for name, x, an in (("q", q, got[0]), ("k", k, got[1]), ("v", v, got[2]), ("s0", s0, got[4])) + \
            ((("g", g, got[3]),) if gate else ()):
        fd = _fd_grad(loss, x)
        assert np.max(np.abs(fd - an)) < 1e-6 * max(1.0, np.max(np.abs(fd))), name


def test_state_gradients_reduce_to_the_stateless_ones():
    rng = np.random.default_rng(41)
    q, k, v, dout, g = (_rand(rng, 2, 5, 2, 4) for _ in range(5))
    a = oracle.chunkwise_state_grad(q, k, v, dout, g=g, rotary_base=1000.0)
    b = oracle.parallel_grad(q, k, v, dout, g=g, rotary_base=1000.0)
    for x, y in zip(a[:4], b):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-13)
    assert a[4] is None
