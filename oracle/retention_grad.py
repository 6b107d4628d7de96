"""Plain fp64 CPU gradients of the parallel form of multi-scale retention,
with its position rotation, per-head GroupNorm and swish gate.

TEST INFRASTRUCTURE. Like ``retention_oracle``, this module exists only to
check the HIP library; only the test suite may call it, and it imports
nothing from the product.

What is differentiated is the forward definition of ``retention_oracle``
(the parallel form over whole sequences, no carried state):
    q' = rot(q), k' = rot(k)                       (rotation by position)
    o_n = sum_{m<=n} g^(n-m) (q'_n . k'_m) v_m      (per head)
    out = GN(o) (.) swish(G)                       (when a gate is given)
Given dout = dL/dout for a scalar loss L, every gradient below is the chain
rule taken step by step in the order of that definition, in fp64:
  * gate and GroupNorm (per token and head, over dv, biased variance, no
    affine): with y = (o - mu)/sigma, sigma = sqrt(var + eps),
        dG = dout (.) y (.) swish'(G),  swish'(x) = s(x) (1 + x (1 - s(x))),
        dy = dout (.) swish(G),
        do = (dy - mean(dy) - y mean(dy (.) y)) / sigma;
  * retention, A = (Q' K'^T) (.) D with D[n, m] = g^(n-m) for n >= m:
        dV = A^T dO,  dA = (dO V^T) (.) D,  dQ' = dA K',  dK' = dA^T Q';
  * rotation: each pair turns by a fixed angle, an orthogonal map, so the
    gradient turns back by the same angle: dq = rot(dq', -angle).
The finite-difference tests pin all of it to the forward oracle.
"""

import numpy as np

from .retention_oracle import default_gammas, group_norm_swish, rotate

__all__ = ["unrotate", "parallel_grad", "chunkwise_state_grad"]


def unrotate(x, rotary_base, pos_offset=0):
    """The transpose of ``rotate``: each adjacent pair turned back by its
    angle (x_{2j} c + x_{2j+1} s, -x_{2j} s + x_{2j+1} c)."""
    if not rotary_base:
        return x
    _, n_tok, _, d = x.shape
    j = np.arange(d // 2, dtype=np.float64)
    theta = float(rotary_base) ** (-2.0 * j / d)
    t = float(pos_offset) + np.arange(n_tok, dtype=np.float64)
    phi = t[:, None] * theta[None, :]
    cos = np.cos(phi)[None, :, None, :]
    sin = np.sin(phi)[None, :, None, :]
    even = x[..., 0::2]
    odd = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = even * cos + odd * sin
    out[..., 1::2] = -even * sin + odd * cos
    return out


def _decay_matrix(n_tok, gam):
    pos = np.arange(n_tok)
    dist = pos[:, None] - pos[None, :]
    return np.where(dist >= 0, float(gam) ** np.maximum(dist, 0), 0.0)


def parallel_grad(q, k, v, dout, g=None, gammas=None, rotary_base=0.0, pos_offset=0, eps=1e-5):
    """Gradients (dq, dk, dv, dg) of sum(dout * out) with out the parallel
    form (then GroupNorm + swish gate when ``g`` is given). dg is None
    without a gate. Layouts as in ``retention_oracle``."""
    heads = q.shape[2]
    gam = default_gammas(heads) if gammas is None else np.asarray(gammas, dtype=np.float64)
    qr = rotate(q, rotary_base, pos_offset)
    kr = rotate(k, rotary_base, pos_offset)
    n_tok = q.shape[1]

    # forward of the retention products, kept for the epilogue's gradient
    o = np.zeros(v.shape)
    for h in range(heads):
        dmat = _decay_matrix(n_tok, gam[h])
        a = (qr[:, :, h, :] @ np.swapaxes(kr[:, :, h, :], 1, 2)) * dmat[None]
        o[:, :, h, :] = a @ v[:, :, h, :]

    # gate and GroupNorm
    if g is not None:
        mu = o.mean(axis=-1, keepdims=True)
        var = ((o - mu) ** 2).mean(axis=-1, keepdims=True)
        sigma = np.sqrt(var + eps)
        y = (o - mu) / sigma
        sig = 1.0 / (1.0 + np.exp(-g))
        swish = g * sig
        dg = dout * y * (sig * (1.0 + g * (1.0 - sig)))
        dy = dout * swish
        do = (dy - dy.mean(axis=-1, keepdims=True) - y * (dy * y).mean(axis=-1, keepdims=True)) / sigma
    else:
        dg = None
        do = dout

    # retention products
    dqr = np.zeros(q.shape)
    dkr = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for h in range(heads):
        dmat = _decay_matrix(n_tok, gam[h])
        qh, kh, vh, doh = qr[:, :, h, :], kr[:, :, h, :], v[:, :, h, :], do[:, :, h, :]
        a = (qh @ np.swapaxes(kh, 1, 2)) * dmat[None]          # [B, N, N]
        dv[:, :, h, :] = np.swapaxes(a, 1, 2) @ doh
        da = (doh @ np.swapaxes(vh, 1, 2)) * dmat[None]
        dqr[:, :, h, :] = da @ kh
        dkr[:, :, h, :] = np.swapaxes(da, 1, 2) @ qh

    dq = unrotate(dqr, rotary_base, pos_offset)
    dk = unrotate(dkr, rotary_base, pos_offset)
    return dq, dk, dv, dg


def chunkwise_state_grad(q, k, v, dout, g=None, state_in=None, d_state_out=None, gammas=None, rotary_base=0.0,
                         pos_offset=0, eps=1e-5):
    """Gradients with a carried state: the forward is the chunkwise form
    (equivalently the recurrence) from state_in S0 (None: zeros), with output
    out (GroupNorm + gate when ``g`` is given) and final state S_N; the loss
    is sum(dout * out) + sum(d_state_out * S_N). Returns
    (dq, dk, dv, dg, d_state_in); d_state_in is None when state_in is.

    Each term follows the chain rule of the closed forms, per head:
        o_n = sum_{m<=n} g^(n-m) (q'_n . k'_m) v_m + g^(n+1) q'_n S0
        S_N = g^N S0 + sum_m g^(N-1-m) k'_m^T v_m
    so, with dO the gradient at o and dS = d_state_out,
        dq'_n += g^(n+1) S0 dO_n
        dk'_m += g^(N-1-m) dS v_m,   dv_m += g^(N-1-m) k'_m dS   (dS terms)
        dS0    = sum_n g^(n+1) q'_n^T dO_n + g^N dS."""
    heads = q.shape[2]
    n_tok = q.shape[1]
    gam = default_gammas(heads) if gammas is None else np.asarray(gammas, dtype=np.float64)
    qr = rotate(q, rotary_base, pos_offset)
    kr = rotate(k, rotary_base, pos_offset)
    bsz = q.shape[0]
    s0 = np.zeros((bsz, heads, q.shape[3], v.shape[3])) if state_in is None else state_in
    pos = np.arange(n_tok, dtype=np.float64)

    # forward of the retention output (with the carried state)
    o = np.zeros(v.shape)
    for h in range(heads):
        dmat = _decay_matrix(n_tok, gam[h])
        a = (qr[:, :, h, :] @ np.swapaxes(kr[:, :, h, :], 1, 2)) * dmat[None]
        o[:, :, h, :] = a @ v[:, :, h, :] + (gam[h] ** (pos + 1.0))[None, :, None] * (qr[:, :, h, :] @ s0[:, h])

    if g is not None:
        mu = o.mean(axis=-1, keepdims=True)
        var = ((o - mu) ** 2).mean(axis=-1, keepdims=True)
        sigma = np.sqrt(var + eps)
        y = (o - mu) / sigma
        sig = 1.0 / (1.0 + np.exp(-g))
        dg = dout * y * (sig * (1.0 + g * (1.0 - sig)))
        dy = dout * g * sig
        do = (dy - dy.mean(axis=-1, keepdims=True) - y * (dy * y).mean(axis=-1, keepdims=True)) / sigma
    else:
        dg, do = None, dout

    dqr = np.zeros(q.shape)
    dkr = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    ds0 = np.zeros(s0.shape)
    for h in range(heads):
        dmat = _decay_matrix(n_tok, gam[h])
        qh, kh, vh, doh = qr[:, :, h, :], kr[:, :, h, :], v[:, :, h, :], do[:, :, h, :]
        a = (qh @ np.swapaxes(kh, 1, 2)) * dmat[None]
        da = (doh @ np.swapaxes(vh, 1, 2)) * dmat[None]
        carry = gam[h] ** (pos + 1.0)                  # g^(n+1)
        tail = gam[h] ** (n_tok - 1.0 - pos)           # g^(N-1-m)
        dqr[:, :, h, :] = da @ kh + carry[None, :, None] * (doh @ np.swapaxes(s0[:, h], 1, 2))
        dkr[:, :, h, :] = np.swapaxes(da, 1, 2) @ qh
        dv[:, :, h, :] = np.swapaxes(a, 1, 2) @ doh
        ds0[:, h] = np.swapaxes(qh * carry[None, :, None], 1, 2) @ doh
        if d_state_out is not None:
            dsh = d_state_out[:, h]                    # [B, dk, dv]
            dkr[:, :, h, :] += tail[None, :, None] * (vh @ np.swapaxes(dsh, 1, 2))
            dv[:, :, h, :] += tail[None, :, None] * (kh @ dsh)
            ds0[:, h] += gam[h] ** n_tok * dsh
    dq = unrotate(dqr, rotary_base, pos_offset)
    dk = unrotate(dkr, rotary_base, pos_offset)
    return dq, dk, dv, dg, (None if state_in is None else ds0)


def forward_for_check(q, k, v, g=None, gammas=None, rotary_base=0.0, pos_offset=0, eps=1e-5):
    """The parallel forward of ``retention_oracle`` (rotation, products, and
    the epilogue when ``g`` is given), for finite differences."""
    from .retention_oracle import parallel

    heads = q.shape[2]
    gam = default_gammas(heads) if gammas is None else np.asarray(gammas, dtype=np.float64)
    o = parallel(rotate(q, rotary_base, pos_offset), rotate(k, rotary_base, pos_offset), v, gam)
    return group_norm_swish(o, g, eps) if g is not None else o
