"""Shared helpers for the GPU parity tests: run the HIP library through its
binding on synthetic inputs and compare with the fp64 oracle."""

import numpy as np
import torch

import oracle
import retnet_retention_amd as rr
from synth import draw

DEV = "cuda:0"

# Bars: fp32 inputs max-abs 1e-4; bf16 inputs relative Frobenius 2e-2 (fp32 accumulation).
F32_MAX_ABS = 1e-4
BF16_REL_FROB = 2e-2


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_frob(got, ref):
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((got - ref).ravel()) / (den if den > 0 else 1.0))


# rows per block of the localized bf16 check
BLOCK_ROWS = 64


def _units(x, kind):
    """x split into the units of the localized check, as rows of a 2-D array:
    "state" [batch, heads, dk, dv] -> one unit per (sequence, head);
    "seq"   [batch, tokens, heads, d] -> per (sequence, block of BLOCK_ROWS
            tokens, head), the last block ragged (zero-padded);
    "packed" [tokens, heads, d] -> per (block of tokens, head);
    "rows"  anything [..., heads, d] -> per (leading index, head);
    "flat2" [batch, tokens] -> per (sequence, block of tokens)."""
    if kind == "state":
        return x.reshape(x.shape[0] * x.shape[1], -1)
    if kind == "rows":
        return x.reshape(-1, x.shape[-1])
    if kind == "packed":
        x = x[None]
        kind = "seq"
    if kind == "flat2":
        x = x[:, :, None, None]
        kind = "seq"
    assert kind == "seq" and x.ndim == 4, kind
    b, n, h, d = x.shape
    nb = -(-n // BLOCK_ROWS)
    pad = np.zeros((b, nb * BLOCK_ROWS, h, d), dtype=x.dtype)
    pad[:, :n] = x
    return pad.reshape(b, nb, BLOCK_ROWS, h, d).transpose(0, 1, 3, 2, 4).reshape(b * nb * h, BLOCK_ROWS * d)


def _default_kind(x, what):
    if x.ndim == 4 and "state" in what:
        return "state"
    return {2: "flat2", 3: "packed", 4: "seq"}.get(x.ndim, "rows")


def worst_block(got, ref, kind):
    """Largest relative Frobenius error over the units of `kind` (a unit whose
    reference is all zero is measured against a small floor instead), and
    the unit's index."""
    g, r = _units(got, kind), _units(ref, kind)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    floor = 1e-3 * max(float(np.sqrt(np.mean(den ** 2))), 1e-30)
    errs = num / np.maximum(den, floor)
    i = int(np.argmax(errs))
    return float(errs[i]), i, len(errs)


def assert_close(got, ref, dtype, what="", kind=None):
    """fp32: max-abs over every element. bf16: relative Frobenius over the
    whole tensor, and the same bar on every unit of the localized split
    (per (sequence, head, block of 64 rows) for outputs, per (sequence, head)
    for states), so that one wrong row, chunk boundary or head cannot hide in
    the norm of a large tensor."""
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if dtype == "f32":
        err = float(np.max(np.abs(got - ref)))
        print(f"  {what}: max-abs {err:.3e}", flush=True)
        assert err <= F32_MAX_ABS, f"{what}: max-abs {err:.3e} > {F32_MAX_ABS}"
    else:
        err = rel_frob(got, ref)
        kind = kind or _default_kind(got, what)
        worst, at, units = worst_block(got, ref, kind)
        print(f"  {what}: rel-Frobenius {err:.3e}; worst of {units} {kind} units {worst:.3e} (unit {at})",
              flush=True)
        assert err <= BF16_REL_FROB, f"{what}: rel-Frobenius {err:.3e} > {BF16_REL_FROB}"
        assert worst <= BF16_REL_FROB, f"{what}: unit {at} of {units} ({kind}): rel-Frobenius {worst:.3e}"
    return err


def make_inputs(seed, b, n, h, d, dtype, scale, gate_scale=None, state=False):
    specs = [((b, n, h, d), scale)] * 3
    if gate_scale is not None:
        specs.append(((b, n, h, d), gate_scale))
    ts = draw(seed, specs, dtype)
    q, k, v = ts[:3]
    g = ts[3] if gate_scale is not None else None
    s0 = None
    if state:
        rng = np.random.default_rng(seed + 1000)
        s0 = rng.standard_normal((b, h, d, d)) * 0.05
        s0 = s0.astype(np.float32).astype(np.float64)
    return q, k, v, g, s0


def gpu_run(form, q, k, v, g, *, chunk=64, rotary_base=0.0, pos_offset=0, state_in=None, gammas=None, eps=1e-5):
    """Run one form on the GPU; returns (out fp64, final state fp64 or None)."""
    tq, tk, tv = q.torch(DEV), k.torch(DEV), v.torch(DEV)
    tg = g.torch(DEV) if g is not None else None
    b, n, h, dk = tq.shape
    dv = tv.shape[-1]
    s_in = torch.from_numpy(state_in.astype(np.float32)).to(DEV) if state_in is not None else None
    state = None
    if form == "parallel":
        out = rr.parallel_fwd(tq, tk, tv, tg, gammas=gammas, rotary_base=rotary_base, pos_offset=pos_offset, eps=eps)
    elif form == "chunkwise":
        s_out = torch.full((b, h, dk, dv), float("nan"), device=DEV)
        out = rr.chunkwise_fwd(tq, tk, tv, tg, chunk=chunk, state_in=s_in, state_out=s_out, gammas=gammas,
                               rotary_base=rotary_base, pos_offset=pos_offset, eps=eps)
        state = s_out
    elif form == "recurrent":
        st = s_in.clone() if s_in is not None else torch.zeros((b, h, dk, dv), device=DEV)
        out = torch.empty_like(tv)
        for t in range(n):
            sl = slice(t, t + 1)
            o_t = rr.recurrent_step(tq[:, sl].contiguous(), tk[:, sl].contiguous(), tv[:, sl].contiguous(), st,
                                    tg[:, sl].contiguous() if tg is not None else None, gammas=gammas,
                                    rotary_base=rotary_base, pos=pos_offset + t, eps=eps)
            out[:, sl] = o_t
        state = st
    else:
        raise ValueError(form)
    torch.cuda.synchronize()
    return to64(out), (to64(state) if state is not None else None)


def oracle_run(form, q, k, v, g, *, chunk=64, rotary_base=0.0, pos_offset=0, state_in=None, gammas=None, eps=1e-5):
    """The fp64 oracle on the same bits; returns (out, final state or None)."""
    return oracle.retention(form, q.f64, k.f64, v.f64, g=None if g is None else g.f64, gammas=gammas,
                            rotary_base=rotary_base, pos_offset=pos_offset, eps=eps, chunk=chunk,
                            state_in=state_in)
