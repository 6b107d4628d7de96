"""The C-ABI library on the host: it loads without a GPU, exports every entry
point include/retention.h declares, sizes workspaces, and rejects invalid
arguments with the documented status before any HIP call. Only calls that
fail validation are made here, so no kernel is ever launched."""

import ctypes
import os
import re

import pytest

from retnet_retention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "retention.h")

ALIGNED = 1 << 32  # fake, never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libretention.so not built (run __graft_entry__.build())")
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(retention_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.retention_abi_version() == 1


def _desc(**kw):
    args = dict(batch=2, seqlen=100, heads=4, dk=256, dv=256, dtype=binding.RET_BF16)
    args.update(kw)
    gam = args.pop("gammas", None)
    rot = args.pop("rotary_base", 0.0)
    eps = args.pop("eps", 1e-5)
    d, keep = binding.make_desc(gammas=gam, rotary_base=rot, eps=eps, **args)
    return d, keep


def _par(L, d, q=ALIGNED, k=ALIGNED * 2, v=ALIGNED * 3, g=None, o=ALIGNED * 4, ws=None, wsb=0):
    return L.retention_parallel_fwd(ctypes.byref(d), q, k, v, g, o, ws, wsb, None)


def _chk(L, d, chunk=64, q=ALIGNED, k=ALIGNED * 2, v=ALIGNED * 3, g=None, o=ALIGNED * 4, si=None, so=None,
         ws=None, wsb=0):
    return L.retention_chunkwise_fwd(ctypes.byref(d), chunk, q, k, v, g, o, si, so, ws, wsb, None)


def _step(L, d, q=ALIGNED, k=ALIGNED * 2, v=ALIGNED * 3, g=None, o=ALIGNED * 4, s=ALIGNED * 5):
    return L.retention_recurrent_step(ctypes.byref(d), q, k, v, g, o, s, None)


def test_status_strings(L):
    for code in range(11):
        assert L.retention_status_string(code)
    assert b"scratch" in L.retention_status_string(10)
    assert L.retention_status_string(0) == b"ok"


def test_workspace_sizes(L):
    d, _ = _desc(batch=2, seqlen=1000, heads=3, dk=128, dv=128)
    assert L.retention_parallel_workspace_bytes(ctypes.byref(d)) == 0
    # control block (16 + batch*heads*(chunks+1)*4 ints) + fp32 state chain (2 slots per
    # sequence and head) + per-chunk states in bf16, each rounded up to 256 bytes
    up = lambda x: (x + 255) // 256 * 256
    ctrl = up((16 + 2 * 3 * 17 * 4) * 4)
    assert L.retention_chunkwise_workspace_bytes(ctypes.byref(d), 64) == (
        ctrl + up(2 * 3 * 2 * 128 * 128 * 4) + up(2 * 3 * 16 * 128 * 128 * 2))
    d, _ = _desc(batch=1, seqlen=10, heads=1, dk=64, dv=64, dtype=binding.RET_F32, rotary_base=10000.0)
    # rotation: angle table + a rotated copy of k (q is turned as the kernels
    # load it), each rounded up to 256 bytes
    rot = (10 * 32 * 8 + 255) // 256 * 256 + (10 * 64 * 4 + 255) // 256 * 256
    assert L.retention_parallel_workspace_bytes(ctypes.byref(d)) == rot
    # chunk larger than the sequence counts as one chunk
    assert L.retention_chunkwise_workspace_bytes(ctypes.byref(d), 4096) == (
        256 + rot + up(2 * 64 * 64 * 4) + up(64 * 64 * 4))
    assert L.retention_chunkwise_workspace_bytes(ctypes.byref(d), 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 2), (dict(seqlen=0), 2), (dict(heads=0), 2), (dict(heads=129), 2),
    (dict(dk=32, dv=32), 3), (dict(dk=128, dv=256), 3), (dict(dtype=7), 3),
    (dict(gammas=[0.9, 0.0, 0.5, 0.5]), 4), (dict(gammas=[0.9, 1.5, 0.5, 0.5]), 4),
    (dict(gammas=[0.9, float("nan"), 0.5, 0.5]), 4), (dict(rotary_base=-1.0), 9),
    (dict(rotary_base=float("inf")), 9),
    # batch * heads * seqlen past int64 in one product: rejected, not wrapped
    (dict(batch=2**31 - 1, seqlen=2**31 - 1, heads=16), 2),
    (dict(batch=2**31 - 1, heads=128), 2),
])
def test_descriptor_validation(L, kw, status):
    d, _ = _desc(**kw)
    assert _par(L, d) == status
    assert _chk(L, d) == status


def test_pointer_validation(L):
    d, _ = _desc()
    assert _par(L, d, q=None) == 1
    assert _par(L, d, o=None) == 1
    assert _par(L, d, k=ALIGNED + 8) == 5
    assert _par(L, d, g=ALIGNED * 6 + 4) == 5
    # the output overlaps q
    assert _par(L, d, o=ALIGNED + 256) == 8
    # gate given but eps invalid
    d2, _ = _desc(eps=0.0)
    assert _par(L, d2, g=ALIGNED * 6) == 9
    # rotation needs a workspace
    d3, _ = _desc(rotary_base=10000.0)
    assert _par(L, d3) == 6
    # chunkwise: chunk < 1, no workspace, workspace too small, misaligned state
    assert _chk(L, d, chunk=0) == 2
    assert _chk(L, d) == 6
    need = L.retention_chunkwise_workspace_bytes(ctypes.byref(d), 64)
    assert _chk(L, d, ws=ALIGNED * 8, wsb=need - 1) == 6
    assert _chk(L, d, ws=ALIGNED * 8, wsb=need, si=ALIGNED * 7 + 4) == 5
    assert _chk(L, d, ws=ALIGNED * 8 + 8, wsb=need) == 5


def test_timed_chunkwise_validates_like_the_plain_call(L):
    d, _ = _desc()
    need = L.retention_chunkwise_workspace_bytes(ctypes.byref(d), 64)
    args = (ctypes.byref(d), 64, ALIGNED, ALIGNED * 2, ALIGNED * 3, None, ALIGNED * 4, None, None)
    fake_events = (ALIGNED * 9, ALIGNED * 10)  # never recorded: validation fails first
    assert L.retention_chunkwise_fwd_timed(*args, None, 0, None, *fake_events) == 6
    assert L.retention_chunkwise_fwd_timed(*args, ALIGNED * 8, need - 1, None, *fake_events) == 6
    assert L.retention_chunkwise_fwd_timed(*args[:2], None, *args[3:], ALIGNED * 8, need, None, *fake_events) == 1


def test_step_validation(L):
    d, _ = _desc()  # seqlen 100: a step takes exactly one token
    assert _step(L, d) == 2
    d, _ = _desc(seqlen=1)
    assert _step(L, d, s=None) == 1
    assert _step(L, d, s=ALIGNED * 5 + 8) == 5
    assert _step(L, d, v=None) == 1


def test_product_path_never_touches_the_oracle():
    """No file of the package (Python or HIP/C++) imports or names the oracle."""
    pkg = os.path.join(ROOT, "retnet_retention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "retention_oracle" not in text, f


def test_backward_validates_before_any_device_call(L):
    d, _ = _desc(batch=1, seqlen=8, heads=2, dk=64, dv=64)
    ws_gate = L.retention_parallel_bwd_workspace_bytes(ctypes.byref(d), 1)
    ws_plain = L.retention_parallel_bwd_workspace_bytes(ctypes.byref(d), 0)
    up = lambda x: (x + 255) // 256 * 256
    tensor = up(1 * 8 * 2 * 64 * 2)
    # no rotation: the products read q (and, without a gate, dout) reversed;
    # with a gate the recomputed forward writes the reversed dO
    assert ws_plain == 0 and ws_gate == tensor
    p = [ALIGNED * i for i in range(1, 11)]
    bwd = L.retention_parallel_bwd
    # g and dg: both or neither
    assert bwd(ctypes.byref(d), p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], None, p[9], ws_gate, None) == 1
    # misaligned output
    assert bwd(ctypes.byref(d), p[0], p[1], p[2], None, p[4], p[5] + 8, p[6], p[7], None, p[9], ws_plain,
               None) == 5
    # an output overlapping an input
    assert bwd(ctypes.byref(d), p[0], p[1], p[2], None, p[4], p[0], p[6], p[7], None, p[9], ws_plain, None) == 8
    # workspace too small (with a gate: the reversed dO)
    assert bwd(ctypes.byref(d), p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], p[9], ws_gate - 1,
               None) == 6


def test_step_positions_validates(L):
    d, _ = _desc(batch=3, seqlen=1, heads=2, dk=64, dv=64, rotary_base=10000.0)
    step = L.retention_recurrent_step_positions
    a = [ALIGNED * i for i in range(1, 8)]
    # positions NULL
    assert step(ctypes.byref(d), a[0], a[1], a[2], None, a[3], a[4], None, None) == 1
    # positions not 8-byte aligned
    assert step(ctypes.byref(d), a[0], a[1], a[2], None, a[3], a[4], a[5] + 4, None) == 5
    # seqlen must be 1
    d2, _ = _desc(batch=3, seqlen=2, heads=2, dk=64, dv=64)
    assert step(ctypes.byref(d2), a[0], a[1], a[2], None, a[3], a[4], a[5], None) == 2


def test_score_map_validates(L):
    d, _ = _desc(batch=2, seqlen=10, heads=2, dk=64, dv=64)
    sm = L.retention_score_map
    assert L.retention_score_map_workspace_bytes(ctypes.byref(d)) == 0
    # query past the sequence
    assert sm(ctypes.byref(d), ALIGNED, ALIGNED * 2, 10, ALIGNED * 3, None, 0, None) == 9
    # scores overlapping q
    assert sm(ctypes.byref(d), ALIGNED, ALIGNED * 2, -1, ALIGNED, None, 0, None) == 8
    # rotation needs the angle table in the workspace
    d2, _ = _desc(batch=2, seqlen=10, heads=2, dk=64, dv=64, rotary_base=10000.0)
    assert L.retention_score_map_workspace_bytes(ctypes.byref(d2)) == 10 * 32 * 8 + (256 - 10 * 32 * 8 % 256) % 256
    assert sm(ctypes.byref(d2), ALIGNED, ALIGNED * 2, -1, ALIGNED * 3, None, 0, None) == 6


def test_stateful_backward_validates(L):
    d, _ = _desc(batch=1, seqlen=16, heads=2, dk=64, dv=64)
    bwd = L.retention_chunkwise_bwd_state
    need = L.retention_chunkwise_bwd_state_workspace_bytes(ctypes.byref(d), 8, 0)
    assert need > L.retention_chunkwise_bwd_workspace_bytes(ctypes.byref(d), 8, 0)
    a = [ALIGNED * i for i in range(1, 16)]
    # d_state_in without state_in
    assert bwd(ctypes.byref(d), 8, a[0], a[1], a[2], None, a[3], None, None, a[4], a[5], a[6], None, a[7], a[8],
               need, None) == 1
    # a decay below 2^-60 with a state-out gradient
    d2, _ = _desc(batch=1, seqlen=16, heads=2, dk=64, dv=64, gammas=[0.5, 2.0 ** -70])
    assert bwd(ctypes.byref(d2), 8, a[0], a[1], a[2], None, a[3], a[9], a[10], a[4], a[5], a[6], None, a[7], a[8],
               need, None) == 4


def _declared_param_counts():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    counts = {}
    for name, params in re.findall(r"\b(retention_\w+)\s*\(([^)]*)\)\s*;", text):
        params = params.strip()
        counts[name] = 0 if params in ("", "void") else params.count(",") + 1
    return counts


def test_binding_argtypes_match_the_header(L):
    """Every ctypes prototype has as many arguments as the C declaration."""
    counts = _declared_param_counts()
    assert sorted(counts) == sorted(binding.EXPORTS)
    for name, n in counts.items():
        assert len(getattr(L, name).argtypes) == n, name


def test_varlen_validates(L):
    d, keep = _desc(batch=3, seqlen=100)
    cu = ALIGNED * 9

    def call(d=d, chunk=64, cu=cu, total=250, q=ALIGNED, o=ALIGNED * 4, ws=ALIGNED * 8, wsb=1 << 40):
        return L.retention_chunkwise_varlen_fwd(ctypes.byref(d), chunk, cu, total, q, ALIGNED * 2, ALIGNED * 3,
                                                None, o, None, None, ws, wsb, None)

    assert call(total=301) == 2  # more rows than batch * seqlen
    assert call(total=-1) == 2
    assert call(chunk=0) == 2
    assert call(cu=None) == 1
    assert call(q=None) == 1
    assert call(cu=ALIGNED * 9 + 2) == 5
    assert call(o=ALIGNED + 16) == 8  # out overlaps q
    assert call(wsb=16) == 6
    assert call(ws=None) == 6


def test_written_buffers_must_not_overlap(L):
    """A state the call writes, the output and the workspace overlap nothing
    else (RET_ERR_ALIAS); state_in == state_out is the one allowed alias."""
    d, _ = _desc()
    need = L.retention_chunkwise_workspace_bytes(ctypes.byref(d), 64)
    ok = dict(ws=ALIGNED * 8, wsb=need)
    assert _chk(L, d, so=ALIGNED + 4096, **ok) == 8           # state_out inside q
    assert _chk(L, d, si=ALIGNED * 4 + 512, **ok) == 8        # state_in inside o
    assert _chk(L, d, si=ALIGNED * 6, so=ALIGNED * 6 + 1024, **ok) == 8  # partial state alias
    assert _chk(L, d, ws=ALIGNED * 3 + 256, wsb=need) == 8    # workspace inside v
    assert _chk(L, d, si=ALIGNED * 8 + 256, **ok) == 8        # state_in inside the workspace
    d1, _ = _desc(seqlen=1)
    assert _step(L, d1, s=ALIGNED * 4) == 8                    # state is the output
    assert _step(L, d1, s=ALIGNED * 2 + 512) == 8              # state inside k
    d3, _ = _desc(rotary_base=10000.0)
    nr = L.retention_parallel_workspace_bytes(ctypes.byref(d3))
    assert _par(L, d3, ws=ALIGNED * 4, wsb=nr) == 8            # rotation workspace is the output
    pos_bad = L.retention_recurrent_step_positions(ctypes.byref(d1), ALIGNED, ALIGNED * 2, ALIGNED * 3, None,
                                                   ALIGNED * 4, ALIGNED * 5, ALIGNED * 5 + 64, None)
    assert pos_bad == 8                                        # positions inside the state


def test_chunkwise_error_reader_validates(L):
    word = ctypes.c_int32(0)
    assert L.retention_chunkwise_error(None, 64, ctypes.byref(word), None) == 1
    assert L.retention_chunkwise_error(ALIGNED, 64, None, None) == 1
    assert L.retention_chunkwise_error(ALIGNED, 4, ctypes.byref(word), None) == 6
    assert L.retention_chunkwise_error(ALIGNED + 4, 64, ctypes.byref(word), None) == 5


def test_noalloc_validates_before_any_device_call(L):
    """The allocation-free chunkwise call checks its arguments like the
    workspace call and rejects calls needing more than its 128 MiB scratch
    (RET_ERR_SCRATCH) before it looks anything up on a device."""
    def call(d, q=ALIGNED, o=ALIGNED * 4, si=None, so=None, err=None, chunk=64):
        return L.retention_chunkwise_fwd_noalloc(ctypes.byref(d), chunk, q, ALIGNED * 2, ALIGNED * 3, None, o, si,
                                                 so, err, None)

    d, _ = _desc()
    assert call(d, chunk=0) == 2
    assert call(d, q=None) == 1
    assert call(d, o=ALIGNED + 256) == 8
    assert call(d, so=ALIGNED * 2 + 64) == 8
    assert call(d, err=ALIGNED * 7 + 2) == 5
    assert call(d, err=ALIGNED * 4 + 64) == 8  # the error word inside the output
    # 8 x 8192 tokens, 16 heads x 256: 268 MB of per-chunk states alone
    big, _ = _desc(batch=8, seqlen=8192, heads=16)
    assert L.retention_chunkwise_workspace_bytes(ctypes.byref(big), 512) > 128 << 20
    assert call(big, chunk=512) == 10
    # the 7B long-context shape fits
    d7, _ = _desc(batch=2, seqlen=8192, heads=16)
    assert L.retention_chunkwise_workspace_bytes(ctypes.byref(d7), 512) <= 128 << 20
