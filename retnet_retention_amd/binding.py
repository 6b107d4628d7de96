"""ctypes binding of libretention.so: torch tensors in, C-ABI calls out.

This layer only marshals arguments (shapes, dtypes, device pointers and the
current HIP stream); every step of the computation runs in the library's
kernels. It raises when the library has not been built: there is no fallback.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libretention.so")

RET_F32 = 0
RET_BF16 = 1

STATUS = {
    0: "RET_OK",
    1: "RET_ERR_NULL",
    2: "RET_ERR_SHAPE",
    3: "RET_ERR_UNSUPPORTED",
    4: "RET_ERR_GAMMA",
    5: "RET_ERR_ALIGN",
    6: "RET_ERR_WORKSPACE",
    7: "RET_ERR_HIP",
    8: "RET_ERR_ALIAS",
    9: "RET_ERR_ARG",
    10: "RET_ERR_SCRATCH",
}

# names declared in include/retention.h
EXPORTS = (
    "retention_parallel_workspace_bytes",
    "retention_parallel_fwd",
    "retention_chunkwise_workspace_bytes",
    "retention_chunkwise_fwd",
    "retention_chunkwise_fwd_timed",
    "retention_chunkwise_fwd_noalloc",
    "retention_chunkwise_varlen_workspace_bytes",
    "retention_chunkwise_varlen_fwd",
    "retention_recurrent_step",
    "retention_recurrent_step_positions",
    "retention_parallel_bwd_workspace_bytes",
    "retention_parallel_bwd",
    "retention_chunkwise_bwd_workspace_bytes",
    "retention_chunkwise_bwd",
    "retention_chunkwise_bwd_state_workspace_bytes",
    "retention_chunkwise_bwd_state",
    "retention_score_map_workspace_bytes",
    "retention_score_map",
    "retention_chunkwise_error",
    "retention_status_string",
    "retention_abi_version",
)


class RetDesc(ctypes.Structure):
    """Mirror of ret_desc_t."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("gamma", ctypes.POINTER(ctypes.c_double)),
        ("rotary_base", ctypes.c_double),
        ("pos_offset", ctypes.c_int64),
        ("gn_eps", ctypes.c_float),
    ]


class RetentionError(RuntimeError):
    """A call's status was not RET_OK, or a chunkwise call's control word
    reported an error (status "control", word in .word)."""

    def __init__(self, status, text, word=0):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status
        self.word = word


_lib = None


def lib():
    """The loaded library (loads it on first use; raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first (python -m retnet_retention_amd.build); "
                "there is no fallback implementation"
            )
        h = ctypes.CDLL(LIB_PATH)
        vp, sz, st, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int32
        pd = ctypes.POINTER(RetDesc)
        h.retention_parallel_workspace_bytes.argtypes = [pd]
        h.retention_parallel_workspace_bytes.restype = sz
        h.retention_parallel_fwd.argtypes = [pd, vp, vp, vp, vp, vp, vp, sz, vp]
        h.retention_parallel_fwd.restype = st
        h.retention_chunkwise_workspace_bytes.argtypes = [pd, i32]
        h.retention_chunkwise_workspace_bytes.restype = sz
        h.retention_chunkwise_fwd.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        h.retention_chunkwise_fwd.restype = st
        h.retention_chunkwise_fwd_timed.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        h.retention_chunkwise_fwd_timed.restype = st
        h.retention_chunkwise_fwd_noalloc.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        h.retention_chunkwise_fwd_noalloc.restype = st
        h.retention_chunkwise_varlen_workspace_bytes.argtypes = [pd, i32]
        h.retention_chunkwise_varlen_workspace_bytes.restype = sz
        h.retention_chunkwise_varlen_fwd.argtypes = [pd, i32, vp, ctypes.c_int64] + [vp] * 8 + [sz, vp]
        h.retention_chunkwise_varlen_fwd.restype = st
        h.retention_recurrent_step.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp]
        h.retention_recurrent_step.restype = st
        h.retention_recurrent_step_positions.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp]
        h.retention_recurrent_step_positions.restype = st
        h.retention_parallel_bwd_workspace_bytes.argtypes = [pd, i32]
        h.retention_parallel_bwd_workspace_bytes.restype = sz
        h.retention_parallel_bwd.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        h.retention_parallel_bwd.restype = st
        h.retention_chunkwise_bwd_workspace_bytes.argtypes = [pd, i32, i32]
        h.retention_chunkwise_bwd_workspace_bytes.restype = sz
        h.retention_chunkwise_bwd.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        h.retention_chunkwise_bwd.restype = st
        h.retention_chunkwise_bwd_state_workspace_bytes.argtypes = [pd, i32, i32]
        h.retention_chunkwise_bwd_state_workspace_bytes.restype = sz
        h.retention_chunkwise_bwd_state.argtypes = [pd, i32] + [vp] * 13 + [sz, vp]
        h.retention_chunkwise_bwd_state.restype = st
        h.retention_score_map_workspace_bytes.argtypes = [pd]
        h.retention_score_map_workspace_bytes.restype = sz
        h.retention_score_map.argtypes = [pd, vp, vp, i32, vp, vp, sz, vp]
        h.retention_score_map.restype = st
        h.retention_chunkwise_error.argtypes = [vp, sz, ctypes.POINTER(i32), vp]
        h.retention_chunkwise_error.restype = st
        h.retention_status_string.argtypes = [st]
        h.retention_status_string.restype = ctypes.c_char_p
        h.retention_abi_version.argtypes = []
        h.retention_abi_version.restype = i32
        _lib = h
    return _lib


def _check(status):
    if status != 0:
        raise RetentionError(status, lib().retention_status_string(status).decode())


def make_desc(batch, seqlen, heads, dk, dv, dtype, gammas=None, rotary_base=0.0, pos_offset=0, eps=1e-5):
    """Build a RetDesc; returns (desc, keepalive) -- keep the second alive
    while the descriptor is in use (it owns the gamma array)."""
    gam = None
    if gammas is not None:
        gam = (ctypes.c_double * heads)(*[float(x) for x in gammas])
    d = RetDesc(batch, seqlen, heads, dk, dv, dtype,
                ctypes.cast(gam, ctypes.POINTER(ctypes.c_double)) if gam is not None else None,
                float(rotary_base), int(pos_offset), float(eps))
    return d, gam


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return RET_BF16
    if t.dtype == torch.float32:
        return RET_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_device(name, t, like):
    """t (may be None) must be a GPU tensor on the device of `like`: its
    pointer goes to the kernels as a device address."""
    if t is not None and (not t.is_cuda or t.device != like.device):
        raise ValueError(f"{name} must be a GPU tensor on {like.device}")


def _workspace(ws, need, like):
    """The caller's workspace (checked), or a new one; returns (workspace,
    bytes, whether it is the binding's own)."""
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=like.device)
        return ws, ws.numel(), True
    _on_device("workspace", ws, like)
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws, ws.numel() * ws.element_size(), False


_CTRL_BITS = {1: "a wait between the chunk-to-chunk state workgroups gave up after its bound",
              2: "packed-sequence bounds (cu_seqlens) had to be clamped"}


def chunkwise_error(workspace):
    """Control word 1 of a chunkwise call's workspace (synchronizes the
    current stream first): 0 when the call that used it completed without an
    error, else bit 0 (1) a wait that gave up, bit 1 (2) clamped packed
    bounds; the outputs are then not valid."""
    word = ctypes.c_int32(0)
    _check(lib().retention_chunkwise_error(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                           ctypes.byref(word), _stream(workspace)))
    return int(word.value)


def check_chunkwise(workspace):
    """Raise RetentionError when the chunkwise call that used `workspace`
    reported an error in its control word (synchronizes)."""
    w = chunkwise_error(workspace)
    if w:
        why = "; ".join(t for b, t in _CTRL_BITS.items() if w & b) or "unknown bits"
        raise RetentionError("control", f"chunkwise control word 1 = {w} ({why}); the outputs are not valid", w)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _validate(q, k, v, g, out):
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("out", out)):
        if t is None:
            continue
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be a GPU tensor on q's device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [batch, seqlen, heads, d]")
    if k.shape != q.shape:
        raise ValueError("k must have the shape of q")
    if v.shape[:3] != q.shape[:3]:
        raise ValueError("v must agree with q on [batch, seqlen, heads]")
    for name, t in (("g", g), ("out", out)):
        if t is not None and t.shape != v.shape:
            raise ValueError(f"{name} must have the shape of v")


def _desc_for(q, v, gammas, rotary_base, pos_offset, eps):
    b, n, h, dk = q.shape
    return make_desc(b, n, h, dk, v.shape[-1], _dtype_code(q), gammas, rotary_base, pos_offset, eps)


def parallel_fwd(q, k, v, g=None, *, gammas=None, rotary_base=0.0, pos_offset=0, eps=1e-5, out=None,
                 workspace=None):
    """Parallel form over whole sequences; returns the output tensor."""
    out = torch.empty_like(v) if out is None else out
    _validate(q, k, v, g, out)
    desc, keep = _desc_for(q, v, gammas, rotary_base, pos_offset, eps)
    L = lib()
    need = L.retention_parallel_workspace_bytes(ctypes.byref(desc))
    ws_bytes = 0
    if need or workspace is not None:
        workspace, ws_bytes, _ = _workspace(workspace, need, q)
    _check(L.retention_parallel_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out),
                                    _ptr(workspace), ws_bytes, _stream(q)))
    del keep
    return out


def parallel_bwd(q, k, v, dout, g=None, *, gammas=None, rotary_base=0.0, pos_offset=0, eps=1e-5, workspace=None):
    """Gradients of sum(dout * parallel_fwd(q, k, v, g, ...)) with respect to
    q, k, v and g; returns (dq, dk, dv, dg), dg None without a gate."""
    _validate(q, k, v, g, dout)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(g) if g is not None else None
    desc, keep = _desc_for(q, v, gammas, rotary_base, pos_offset, eps)
    L = lib()
    need = L.retention_parallel_bwd_workspace_bytes(ctypes.byref(desc), int(g is not None))
    workspace, ws_bytes, _ = _workspace(workspace, need, q)
    _check(L.retention_parallel_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dout), _ptr(dq),
                                    _ptr(dk), _ptr(dv), _ptr(dg), _ptr(workspace), ws_bytes, _stream(q)))
    del keep
    return dq, dk, dv, dg


def chunkwise_bwd(q, k, v, dout, g=None, *, chunk=512, state_in=None, d_state_out=None, gammas=None,
                  rotary_base=0.0, pos_offset=0, eps=1e-5, workspace=None, check=None):
    """Gradients of sum(dout * out) (+ sum(d_state_out * state_out)) with
    out, state_out = chunkwise_fwd(q, k, v, g, chunk=chunk, state_in=state_in,
    ...), with respect to q, k, v, g and state_in. Returns (dq, dk, dv, dg)
    without a carried state, (dq, dk, dv, dg, d_state_in) with one; dg is
    None without a gate. check: as chunkwise_fwd (the control word covers
    all of the call's chunkwise launches)."""
    _validate(q, k, v, g, dout)
    if state_in is not None or d_state_out is not None:
        return _chunkwise_bwd_state(q, k, v, dout, g, chunk, state_in, d_state_out, gammas, rotary_base,
                                    pos_offset, eps, workspace, check)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(g) if g is not None else None
    desc, keep = _desc_for(q, v, gammas, rotary_base, pos_offset, eps)
    L = lib()
    need = L.retention_chunkwise_bwd_workspace_bytes(ctypes.byref(desc), int(chunk), int(g is not None))
    workspace, ws_bytes, own = _workspace(workspace, need, q)
    _check(L.retention_chunkwise_bwd(ctypes.byref(desc), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dout),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(workspace), ws_bytes, _stream(q)))
    del keep
    if check or (check is None and own):
        check_chunkwise(workspace)
    return dq, dk, dv, dg


def score_map(q, k, *, query=-1, gammas=None, rotary_base=0.0, pos_offset=0, workspace=None):
    """Retention score map of query token `query` (-1: the last) over the
    tokens before it, summed over heads; returns fp32 [batch, seqlen]."""
    _validate(q, k, k, None, k)
    out = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    desc, keep = _desc_for(q, k, gammas, rotary_base, pos_offset, 1e-5)
    L = lib()
    need = L.retention_score_map_workspace_bytes(ctypes.byref(desc))
    ws_bytes = 0
    if need or workspace is not None:
        workspace, ws_bytes, _ = _workspace(workspace, need, q)
    _check(L.retention_score_map(ctypes.byref(desc), _ptr(q), _ptr(k), int(query), _ptr(out), _ptr(workspace),
                                 ws_bytes, _stream(q)))
    del keep
    return out


def _chunkwise_bwd_state(q, k, v, dout, g, chunk, state_in, d_state_out, gammas, rotary_base, pos_offset, eps,
                         workspace, check):
    b, _, h, dk = q.shape
    for name, t in (("state_in", state_in), ("d_state_out", d_state_out)):
        _on_device(name, t, q)
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()
                              or tuple(t.shape) != (b, h, dk, v.shape[-1])):
            raise ValueError(f"{name} must be a contiguous fp32 [batch, heads, dk, dv] tensor")
    dq, dk_, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(g) if g is not None else None
    ds0 = torch.empty_like(state_in) if state_in is not None else None
    desc, keep = _desc_for(q, v, gammas, rotary_base, pos_offset, eps)
    L = lib()
    need = L.retention_chunkwise_bwd_state_workspace_bytes(ctypes.byref(desc), int(chunk), int(g is not None))
    workspace, ws_bytes, own = _workspace(workspace, need, q)
    _check(L.retention_chunkwise_bwd_state(ctypes.byref(desc), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                           _ptr(dout), _ptr(state_in), _ptr(d_state_out), _ptr(dq), _ptr(dk_),
                                           _ptr(dv), _ptr(dg), _ptr(ds0), _ptr(workspace), ws_bytes, _stream(q)))
    del keep
    if check or (check is None and own):
        check_chunkwise(workspace)
    return (dq, dk_, dv, dg) if state_in is None else (dq, dk_, dv, dg, ds0)


def chunkwise_workspace_bytes(q, v, chunk, rotary_base=0.0):
    desc, keep = _desc_for(q, v, None, rotary_base, 0, 1e-5)
    return lib().retention_chunkwise_workspace_bytes(ctypes.byref(desc), int(chunk))


def chunkwise_fwd(q, k, v, g=None, *, chunk=512, state_in=None, state_out=None, gammas=None, rotary_base=0.0,
                  pos_offset=0, eps=1e-5, out=None, workspace=None, kernel_events=None, check=None):
    """Chunkwise form; returns the output tensor (state_out, if given, is
    filled with the state after the last token). kernel_events: optional pair
    of torch.cuda.Event (timing enabled) recorded around the chunkwise kernel
    alone. check: synchronize and raise RetentionError if the call's control
    word reports an error; None checks only when the binding allocated the
    workspace (a caller's workspace can be checked later with
    check_chunkwise)."""
    out = torch.empty_like(v) if out is None else out
    _validate(q, k, v, g, out)
    for name, s in (("state_in", state_in), ("state_out", state_out)):
        if s is not None:
            b, _, h, dk = q.shape
            _on_device(name, s, q)
            if s.dtype != torch.float32 or not s.is_contiguous() or tuple(s.shape) != (b, h, dk, v.shape[-1]):
                raise ValueError(f"{name} must be a contiguous fp32 [batch, heads, dk, dv] tensor")
    desc, keep = _desc_for(q, v, gammas, rotary_base, pos_offset, eps)
    L = lib()
    need = L.retention_chunkwise_workspace_bytes(ctypes.byref(desc), int(chunk))
    workspace, ws_bytes, own = _workspace(workspace, need, q)
    if kernel_events is None:
        _check(L.retention_chunkwise_fwd(ctypes.byref(desc), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                         _ptr(out), _ptr(state_in), _ptr(state_out), _ptr(workspace), ws_bytes,
                                         _stream(q)))
    else:
        before, after = (ctypes.c_void_p(e.cuda_event) for e in kernel_events)
        _check(L.retention_chunkwise_fwd_timed(ctypes.byref(desc), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                               _ptr(out), _ptr(state_in), _ptr(state_out), _ptr(workspace),
                                               ws_bytes, _stream(q), before, after))
    del keep
    if check or (check is None and own):
        check_chunkwise(workspace)
    return out


def chunkwise_fwd_noalloc(q, k, v, g=None, *, chunk=512, state_in=None, state_out=None, gammas=None,
                          rotary_base=0.0, pos_offset=0, eps=1e-5, out=None, error_word=None):
    """The chunkwise form through the entry point that allocates nothing: the
    library's static scratch replaces the workspace (calls on one device must
    not overlap in time). `out` must be given (nothing is allocated here
    either); error_word: optional GPU int32 tensor [1] that receives the
    call's control word 1 in stream order."""
    if out is None:
        raise ValueError("chunkwise_fwd_noalloc allocates nothing: pass `out`")
    _validate(q, k, v, g, out)
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None:
            b, _, h, dk = q.shape
            _on_device(name, t, q)
            if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (b, h, dk, v.shape[-1]):
                raise ValueError(f"{name} must be a contiguous fp32 [batch, heads, dk, dv] tensor")
    if error_word is not None:
        _on_device("error_word", error_word, q)
        if error_word.dtype != torch.int32 or error_word.numel() < 1 or not error_word.is_contiguous():
            raise ValueError("error_word must be a contiguous GPU int32 tensor of at least one element")
    desc, keep = _desc_for(q, v, gammas, rotary_base, pos_offset, eps)
    _check(lib().retention_chunkwise_fwd_noalloc(ctypes.byref(desc), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                                 _ptr(out), _ptr(state_in), _ptr(state_out), _ptr(error_word),
                                                 _stream(q)))
    del keep
    return out


def chunkwise_varlen_fwd(q, k, v, cu_seqlens, max_seqlen, g=None, *, chunk=512, state_in=None, state_out=None,
                         gammas=None, rotary_base=0.0, pos_offset=0, eps=1e-5, out=None, workspace=None, check=None):
    """Chunkwise form over packed sequences of different lengths: q, k, v, g
    are [total_tokens, heads, d], sequence b holds rows cu_seqlens[b] ..
    cu_seqlens[b+1]-1 (cu_seqlens: GPU int32 [batch + 1]); max_seqlen bounds
    every length. state_in / state_out: fp32 [batch, heads, dk, dv] or None.
    Returns the output (rows outside every sequence are left as they were).
    check: as chunkwise_fwd (clamped cu_seqlens raise RetentionError)."""
    out = torch.empty_like(v) if out is None else out
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("out", out)):
        if t is None:
            continue
        if not t.is_cuda or t.device != q.device or not t.is_contiguous() or t.dtype != q.dtype or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous GPU [total_tokens, heads, d] tensor of q's dtype")
    if k.shape != q.shape or v.shape[:2] != q.shape[:2] or (g is not None and g.shape != v.shape) \
            or out.shape != v.shape:
        raise ValueError("q, k, v, g and out must agree on [total_tokens, heads]")
    _on_device("cu_seqlens", cu_seqlens, q)
    if not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 \
            or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous GPU int32 tensor [batch + 1]")
    batch = cu_seqlens.numel() - 1
    total, h, dk = q.shape
    for name, st in (("state_in", state_in), ("state_out", state_out)):
        _on_device(name, st, q)
        if st is not None and (st.dtype != torch.float32 or not st.is_contiguous()
                               or tuple(st.shape) != (batch, h, dk, v.shape[-1])):
            raise ValueError(f"{name} must be a contiguous fp32 [batch, heads, dk, dv] tensor")
    desc, keep = make_desc(batch, int(max_seqlen), h, dk, v.shape[-1], _dtype_code(q), gammas, rotary_base,
                           pos_offset, eps)
    L = lib()
    need = L.retention_chunkwise_varlen_workspace_bytes(ctypes.byref(desc), int(chunk))
    workspace, ws_bytes, own = _workspace(workspace, need, q)
    _check(L.retention_chunkwise_varlen_fwd(ctypes.byref(desc), int(chunk), _ptr(cu_seqlens), int(total), _ptr(q),
                                            _ptr(k), _ptr(v), _ptr(g), _ptr(out), _ptr(state_in), _ptr(state_out),
                                            _ptr(workspace), ws_bytes, _stream(q)))
    del keep
    if check or (check is None and own):
        check_chunkwise(workspace)
    return out


def chunkwise_varlen_workspace_bytes(batch, max_seqlen, heads, d, dtype, chunk, rotary_base=0.0):
    """Workspace bytes of chunkwise_varlen_fwd for `batch` sequences of at
    most max_seqlen tokens (dtype: torch.bfloat16 or torch.float32)."""
    code = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    desc, keep = make_desc(batch, max_seqlen, heads, d, d, code, rotary_base=rotary_base)
    return lib().retention_chunkwise_varlen_workspace_bytes(ctypes.byref(desc), int(chunk))


def recurrent_step(q, k, v, state, g=None, *, gammas=None, rotary_base=0.0, pos=0, eps=1e-5, out=None,
                   positions=None):
    """One decode step (q, k: [batch, 1, heads, dk]); updates `state` in place
    and returns the output [batch, 1, heads, dv]. `positions` (optional, a GPU
    int64 tensor [batch]): each sequence's rotation position, in place of
    `pos`."""
    out = torch.empty_like(v) if out is None else out
    _validate(q, k, v, g, out)
    if q.shape[1] != 1:
        raise ValueError("recurrent_step takes one token per sequence (seqlen 1)")
    b, _, h, dk = q.shape
    _on_device("state", state, q)
    if state.dtype != torch.float32 or not state.is_contiguous() or tuple(state.shape) != (b, h, dk, v.shape[-1]):
        raise ValueError("state must be a contiguous fp32 [batch, heads, dk, dv] tensor")
    desc, keep = _desc_for(q, v, gammas, rotary_base, pos, eps)
    if positions is None:
        _check(lib().retention_recurrent_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out),
                                              _ptr(state), _stream(q)))
    else:
        _on_device("positions", positions, q)
        if (positions.dtype != torch.int64 or not positions.is_cuda or not positions.is_contiguous()
                or tuple(positions.shape) != (b,)):
            raise ValueError("positions must be a contiguous GPU int64 tensor [batch]")
        _check(lib().retention_recurrent_step_positions(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                                        _ptr(out), _ptr(state), _ptr(positions), _stream(q)))
    del keep
    return out
