"""Plain fp64 CPU oracle for multi-scale retention (parallel, recurrent and
chunkwise forms, position rotation, per-head GroupNorm and swish gate).

TEST INFRASTRUCTURE. This module exists only to check the HIP library. Only the
test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it; the product path (the C-ABI library and its
Python binding) never does, and it imports nothing from the product.

Sources (web pages on RetNet):
  [SUM]  "Retentive Network: A Successor to Transformer for Large Language
         Models", Elamur Research paper summary -- section "Summary" (retention
         replaces attention; it comes from a linear recurrence with exponential
         decay; positions are encoded like xPos; parallel, recurrent and
         chunkwise forms; one decay per head; swish gate and GroupNorm) and
         section "Key points" (fifth item: per-head decay 1 - 2^(-5-i); chunk
         cost O(dn(b+h)) with b = 512, h = 256).
  [RMB]  "Retentive Network (RetNet): Revolutionizing Neural Architecture for
         Language Models" -- section "representations" (parallel form for
         training, recurrent O(1) form for inference, chunkwise form that
         encodes chunks in parallel while recurrently summarising them).
  [CARD] "SpiralAI Spiral-RetNet-3b-base" model card -- "Visualization of the
         retention mechanism" (recurrent and parallel modes are mathematically
         equivalent).

The pages print no equations. What is computed here is the plainest reading
that fits everything they state (each step says which reading it takes):

  per head with decay g, for token n of a sequence (0-based),
      o_n = sum_{m<=n} g^(n-m) (q_n . k_m) v_m  +  g^(n+1) q_n S0
  which is the same as the linear recurrence with exponential decay
      S_n = g S_{n-1} + k_n^T v_n,  S_{-1} = S0,  o_n = q_n S_n,
  and, cutting the sequence into chunks that pass the recurrent state along,
      O_i = (Q_i K_i^T (.) D_i) V_i + (Q_i R_{i-1}) (.) xi
      R_i = K_i^T (V_i (.) zeta) + g^{b_i} R_{i-1},   R_{-1} = S0
  with D_i[r, c] = g^(r-c) for r >= c (else 0), xi_r = g^(r+1),
  zeta_r = g^(b_i-1-r), b_i the length of chunk i and r, c rows inside it.

Every power g^k below is formed with ``**`` in fp64 (no exp/log tricks), so
dyadic decays and small-integer inputs give exact results.

Layouts (all numpy float64):
  q, k  [B, N, H, dk]     v, g, out  [B, N, H, dv]     state  [B, H, dk, dv]
"""

import numpy as np

__all__ = [
    "default_gammas",
    "rotate",
    "parallel",
    "recurrent",
    "chunkwise",
    "recurrent_step",
    "group_norm_swish",
    "retention",
    "score_map",
]


def default_gammas(heads):
    """Per-head decay of multi-scale retention, [SUM] Key points (fifth item):
    head i (counted from 0) decays with g_i = 1 - 2^(-5-i).

    ``ldexp`` makes 2^(-5-i) exactly, so the table is exact in fp64."""
    i = np.arange(heads)
    return 1.0 - np.ldexp(1.0, -5 - i)


def rotate(x, rotary_base, pos_offset=0):
    """Position rotation of queries and keys, [SUM] Summary (the pages say the
    position encoding follows xPos, without a formula).

    Reading taken (the pages give no formula): the rotary scheme of the RoFormer
    reference that xPos builds on. Adjacent pairs (x_{2j}, x_{2j+1}) turn by the
    angle t * theta_j, theta_j = base^(-2j/d), t = pos_offset + n the absolute
    position, counter-clockwise:
        x'_{2j}   = x_{2j} cos - x_{2j+1} sin
        x'_{2j+1} = x_{2j} sin + x_{2j+1} cos
    There is no xPos amplitude factor: the per-head decay plays that role.
    ``rotary_base == 0`` means no rotation.
    """
    if not rotary_base:
        return x
    _, n_tok, _, d = x.shape
    j = np.arange(d // 2, dtype=np.float64)
    theta = float(rotary_base) ** (-2.0 * j / d)
    t = float(pos_offset) + np.arange(n_tok, dtype=np.float64)
    phi = t[:, None] * theta[None, :]  # [N, d/2]
    cos = np.cos(phi)[None, :, None, :]
    sin = np.sin(phi)[None, :, None, :]
    even = x[..., 0::2]
    odd = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = even * cos - odd * sin
    out[..., 1::2] = even * sin + odd * cos
    return out


def _zero_state(q, v):
    bsz, _, heads, dk = q.shape
    return np.zeros((bsz, heads, dk, v.shape[-1]))


def parallel(q, k, v, gammas, state_in=None):
    """Parallel form, [RMB] "representations" (the training form) and [SUM]
    Summary: O = (Q K^T (.) D) V over the whole sequence, D[n, m] = g^(n-m) for
    n >= m and 0 above the diagonal. The diagonal is included (g^0 = 1).

    ``state_in`` (optional, [B, H, dk, dv]) is a state carried in from earlier
    tokens; it adds g^(n+1) q_n S0, the closed form of the recurrence.
    """
    bsz, n_tok, heads, _ = q.shape
    out = np.zeros(v.shape)
    pos = np.arange(n_tok)
    dist = pos[:, None] - pos[None, :]
    for h in range(heads):
        gam = float(gammas[h])
        decay = np.where(dist >= 0, gam ** np.maximum(dist, 0), 0.0)  # [N, N]
        qh = q[:, :, h, :]  # [B, N, dk]
        kh = k[:, :, h, :]
        vh = v[:, :, h, :]
        scores = qh @ np.swapaxes(kh, 1, 2)  # [B, N, N]
        out[:, :, h, :] = (scores * decay[None]) @ vh
        if state_in is not None:
            carry = gam ** (pos + 1.0)  # g^(n+1)
            out[:, :, h, :] += carry[None, :, None] * (qh @ state_in[:, h])
    return out


def recurrent(q, k, v, gammas, state_in=None):
    """Recurrent form, [RMB] "representations" (O(1) per token) and [SUM]
    Summary (linear recurrence with exponential decay, no KV cache):
        S_n = g S_{n-1} + k_n^T v_n,   o_n = q_n S_n   (update, then read).
    Returns (out, final state)."""
    gam = np.asarray(gammas, dtype=np.float64)[None, :, None, None]
    state = _zero_state(q, v) if state_in is None else np.array(state_in, dtype=np.float64)
    out = np.zeros(v.shape)
    for n in range(q.shape[1]):
        outer = k[:, n, :, :, None] * v[:, n, :, None, :]  # [B, H, dk, dv]
        state = gam * state + outer
        out[:, n] = np.einsum("bhi,bhij->bhj", q[:, n], state)
    return out, state


def chunkwise(q, k, v, gammas, chunk, state_in=None):
    """Chunkwise recurrent form, [SUM] Summary (parallel work inside each
    chunk, a recurrent state carried from one chunk to the next) and [RMB]
    "representations". For chunk i of length b (the last one may be short):
        O_i = (Q_i K_i^T (.) D) V_i + (Q_i R_{i-1}) (.) xi
        R_i = K_i^T (V_i (.) zeta) + g^b R_{i-1}
    D[r, c] = g^(r-c) (r >= c), xi_r = g^(r+1), zeta_r = g^(b-1-r); these
    are what unrolling the recurrence over one chunk gives.
    Returns (out, final state)."""
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    bsz, n_tok, heads, _ = q.shape
    state = _zero_state(q, v) if state_in is None else np.array(state_in, dtype=np.float64)
    out = np.zeros(v.shape)
    for start in range(0, n_tok, chunk):
        blen = min(chunk, n_tok - start)
        rows = np.arange(blen)
        dist = rows[:, None] - rows[None, :]
        for h in range(heads):
            gam = float(gammas[h])
            decay = np.where(dist >= 0, gam ** np.maximum(dist, 0), 0.0)
            xi = gam ** (rows + 1.0)
            zeta = gam ** (blen - 1.0 - rows)
            qh = q[:, start:start + blen, h, :]  # [B, b, dk]
            kh = k[:, start:start + blen, h, :]
            vh = v[:, start:start + blen, h, :]
            inner = ((qh @ np.swapaxes(kh, 1, 2)) * decay[None]) @ vh
            cross = (qh @ state[:, h]) * xi[None, :, None]
            out[:, start:start + blen, h, :] = inner + cross
            state[:, h] = np.swapaxes(kh, 1, 2) @ (vh * zeta[None, :, None]) + gam ** blen * state[:, h]
    return out, state


def group_norm_swish(o, g, eps):
    """Output epilogue, [SUM] Summary and Key points (fourth item: removing the
    swish gate or GroupNorm hurts). Reading taken: GroupNorm with one group
    per head over that head's dv values of one token, biased variance, no
    affine parameters; swish(x) = x * sigmoid(x); out = swish(G) (.) GN(O)."""
    mu = o.mean(axis=-1, keepdims=True)
    var = ((o - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (o - mu) / np.sqrt(var + eps)
    return y * (g / (1.0 + np.exp(-g)))


def recurrent_step(q, k, v, state, gammas, g=None, rotary_base=0.0, pos=0, eps=1e-5):
    """One decode step for a batch of single tokens: q, k [B, 1, H, dk],
    v, g [B, 1, H, dv], state [B, H, dk, dv] (not modified).
    Returns (out [B, 1, H, dv], new state)."""
    qr = rotate(q, rotary_base, pos)
    kr = rotate(k, rotary_base, pos)
    out, new_state = recurrent(qr, kr, v, gammas, state_in=state)
    if g is not None:
        out = group_norm_swish(out, g, eps)
    return out, new_state


def retention(form, q, k, v, g=None, gammas=None, rotary_base=0.0, pos_offset=0,
              eps=1e-5, chunk=None, state_in=None):
    """Multi-scale retention over a batch of sequences: rotate Q and K, run the
    chosen form, then (when a gate G is given) GroupNorm + swish gate.
    ``form`` is "parallel", "recurrent" or "chunkwise".
    Returns (out, final state); the parallel form has no state output and
    returns None in its place."""
    heads = q.shape[2]
    gam = default_gammas(heads) if gammas is None else np.asarray(gammas, dtype=np.float64)
    qr = rotate(q, rotary_base, pos_offset)
    kr = rotate(k, rotary_base, pos_offset)
    if form == "parallel":
        out, state = parallel(qr, kr, v, gam, state_in=state_in), None
    elif form == "recurrent":
        out, state = recurrent(qr, kr, v, gam, state_in=state_in)
    elif form == "chunkwise":
        out, state = chunkwise(qr, kr, v, gam, chunk, state_in=state_in)
    else:
        raise ValueError(f"unknown form {form!r}")
    if g is not None:
        out = group_norm_swish(out, g, eps)
    return out, state


def retention_varlen(form, q, k, v, cu_seqlens, g=None, gammas=None, rotary_base=0.0, pos_offset=0, eps=1e-5,
                     chunk=None, state_in=None):
    """A ragged batch in packed layout: q, k, v, g are [T, H, d] and sequence
    b holds rows cu_seqlens[b] .. cu_seqlens[b+1]-1. Reading taken: every
    sequence is its own retention run (own state slot, positions counted from
    pos_offset at its first token), so this is ``retention`` applied to each
    slice alone; an empty sequence passes its state through. Returns
    (out [T, H, dv], final states [B, H, dk, dv]); rows outside every
    sequence stay zero."""
    cu = [int(x) for x in cu_seqlens]
    nseq, heads, dk, dv = len(cu) - 1, q.shape[1], q.shape[2], v.shape[2]
    out = np.zeros(v.shape[:2] + (dv,))
    states = np.zeros((nseq, heads, dk, dv))
    for b in range(nseq):
        a, e = cu[b], cu[b + 1]
        s0 = None if state_in is None else np.asarray(state_in[b:b + 1], dtype=np.float64)
        if e == a:
            if s0 is not None:
                states[b] = s0[0]
            continue
        piece = lambda x: None if x is None else np.asarray(x[a:e], dtype=np.float64)[None]
        o_b, s_b = retention(form, piece(q), piece(k), piece(v), g=piece(g), gammas=gammas,
                             rotary_base=rotary_base, pos_offset=pos_offset, eps=eps, chunk=chunk, state_in=s0)
        out[a:e] = o_b[0]
        if s_b is not None:
            states[b] = s_b[0]
    return out, states


def score_map(q, k, gammas=None, rotary_base=0.0, pos_offset=0, query=-1):
    """Retention weights of one query token over the tokens before it, summed
    over heads, the "Visualization of the retention mechanism" section of the
    SpiralAI model card page: the magnitude of each head's query-key dot
    product, summed across heads. Reading taken: the weights are
    those of the parallel form (Q K^T (.) D), so each carries its head's decay
    g^(n-m); for query token n (default: the last) and key token m <= n,
        w[b, m] = sum_h g_h^(n-m) |q'_{b,n,h} . k'_{b,m,h}|
    with q', k' rotated by position; w[b, m] = 0 for m > n. Returns [B, N]."""
    bsz, n_tok, heads, _ = q.shape
    gam = default_gammas(heads) if gammas is None else np.asarray(gammas, dtype=np.float64)
    n = n_tok - 1 if query < 0 else int(query)
    qr = rotate(q, rotary_base, pos_offset)
    kr = rotate(k, rotary_base, pos_offset)
    out = np.zeros((bsz, n_tok))
    for b in range(bsz):
        for m in range(n + 1):
            for h in range(heads):
                out[b, m] += float(gam[h]) ** (n - m) * abs(float(np.dot(qr[b, n, h], kr[b, m, h])))
    return out
