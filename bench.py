"""Throughput of multi-scale retention on one MI355X.

Headline (``value``): the chunkwise form over the 7B long-context workload
(batch 2, 8192 tokens, 16 heads x 256, chunk 512, bf16, GroupNorm + swish gate,
fp32 state out), in algorithmic TFLOP/s. One step = one chunkwise forward
over that batch (rotation-free workload: per-chunk states, intra- and
cross-chunk products, decay masks, GroupNorm, gate, state out).

Beside it, on the same run:
  decode    -- recurrent step, 16 heads x 256, fp32 state seeded by a chunkwise
               prefill of 8192 tokens, batch 1/8/64/256, tokens/s and GB/s;
  parallel  -- parallel form on the 3B workload (batch 4, 2048, 10 x 256,
               rotation, gate), TFLOP/s;
  roofline  -- the dominant kernel of the headline step against MI355X peak;
  cpu_baseline -- the fp64 oracle timed on this host on a bounded sample;
  chunkwise_detail -- kernel-time percentiles, a cold-cache run and the
               200M and 3B chunkwise workloads.
With --sweep (or --only sweep): the chunkwise kernel over 2k-64k tokens and
chunk sizes 64-1024.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only chunkwise|decode|parallel|sweep]
                       [--no-cpu-baseline] [--sweep]
"""

import argparse
import csv
import glob
import hashlib
import itertools
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E (published)

CSRC = os.path.join(ROOT, "retnet_retention_amd", "csrc")
# sources that define the chunkwise kernel: counters taken on another version
# of them no longer describe the kernel that runs
CHUNKWISE_SOURCES = ("retention_fwd.hip", "common.hpp", "launch.hpp")
CHUNKWISE_KERNEL = "retention_chunkwise_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunkwise_7b_8k_traffic.txt")
COPY_PROBE_BYTES = 512 << 20  # plain device-to-device copy of known size (counter calibration)


def source_hash(names=CHUNKWISE_SOURCES):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(n.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per chunkwise launch from the committed counter summary, or
    None when that summary is missing or was taken on other kernel sources."""
    try:
        fields = dict(ln.split(":", 1) for ln in open(TRAFFIC_FILE) if ":" in ln and not ln.startswith(" "))
    except OSError:
        return None
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("source_hash") != source_hash():
        return None
    try:
        return {"bytes": int(fields["traffic_bytes_per_launch"]), "fetch": int(fields["fetch_bytes_per_launch"]),
                "write": int(fields["write_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# algorithmic work (causal-counted; rotation, masks, GroupNorm, gate not counted)
# ---------------------------------------------------------------------------
def chunkwise_flops(batch, seqlen, heads, dk, dv, chunk):
    total = 0
    for start in range(0, seqlen, chunk):
        b = min(chunk, seqlen - start)
        total += b * (b + 1) * (dk + dv) + 4 * b * dk * dv
    return batch * heads * total


def chunkwise_dense_flops(batch, seqlen, heads, dk, dv, chunk):
    """The same work counted dense (every chunk's full b x b score block),
    reported beside the causal count, labelled."""
    total = 0
    for start in range(0, seqlen, chunk):
        b = min(chunk, seqlen - start)
        total += 2 * b * b * (dk + dv) + 4 * b * dk * dv
    return batch * heads * total


def chunkwise_split_flops(batch, seqlen, heads, dk, dv, chunk):
    """(state kernel, output kernel) shares of the chunkwise count."""
    state = out = 0
    for start in range(0, seqlen, chunk):
        b = min(chunk, seqlen - start)
        state += 2 * b * dk * dv
        out += b * (b + 1) * (dk + dv) + 2 * b * dk * dv
    return batch * heads * state, batch * heads * out


def parallel_flops(batch, seqlen, heads, dk, dv):
    return batch * heads * seqlen * (seqlen + 1) * (dk + dv)


def step_bytes(batch, heads, dk, dv, elem=2):
    """Per decode step: state read + write (fp32) and q, k, v, g in, o out."""
    return batch * heads * (8 * dk * dv + elem * (2 * dk + 3 * dv))


def chunkwise_bytes(batch, seqlen, heads, dk, dv, elem=2, gate=True, state_out=True):
    per_tok = heads * (2 * dk + dv * (2 + (1 if gate else 0))) * elem
    return batch * seqlen * per_tok + (batch * heads * dk * dv * 4 if state_out else 0)


# ---------------------------------------------------------------------------
# Every leg but the headline also warms until this much wall time of its own
# calls has passed: the GPU's clocks settle only after tens of milliseconds of
# sustained load, and a few warm-up calls of a short leg are far less.
SETTLE_MS = 150.0


def time_calls(fn, steps, warmup, settle_ms=0.0):
    """Average device time per call over `steps` back-to-back calls (events on
    torch's current stream, which is the stream the library launches on),
    after `warmup` calls and then, with settle_ms, more calls until that much
    wall time has passed."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall


def copy_probe():
    """Two plain copies of COPY_PROBE_BYTES: counter runs scale FETCH_SIZE and
    WRITE_SIZE by what they read for this kernel of known traffic."""
    import torch

    src = torch.ones(COPY_PROBE_BYTES // 4, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def chunkwise_inputs(name):
    """The workload's seeded inputs (drawn on the host), already on the GPU."""
    from synth import get

    w = get(name)
    return w, [t.torch("cuda:0") for t in w.inputs()]


def bench_chunkwise(steps, warmup, name="retention_7b_8k", cold_reps=0, prepared=None, settle_ms=0.0):
    """Chunkwise calls on one workload: per-call time (reset + kernel) and the
    kernel's own event time per call; with cold_reps, also the kernel after
    a 512 MiB write that evicts L2 and the Infinity Cache. prepared: the
    result of chunkwise_inputs(name), drawn earlier. settle_ms: as for
    time_calls (the headline leg takes exactly its `warmup` calls)."""
    import torch

    import retnet_retention_amd as rr

    w, (q, k, v, g) = prepared if prepared is not None else chunkwise_inputs(name)
    state = torch.empty((w.batch, w.heads, w.dk, w.dv), device="cuda:0")
    out = torch.empty_like(v)
    rot = getattr(w, "rotary_base", 0.0) or 0.0
    ws = torch.empty(rr.chunkwise_workspace_bytes(q, v, w.chunk, rotary_base=rot), dtype=torch.uint8,
                     device="cuda:0")

    def step(events=None):
        rr.chunkwise_fwd(q, k, v, g, chunk=w.chunk, state_out=state, out=out, workspace=ws, rotary_base=rot,
                         kernel_events=events)

    # the step rate: `steps` plain back-to-back calls (reset + kernel)
    for _ in range(warmup):
        step()
    ms, wall = time_calls(step, steps, 0, settle_ms=settle_ms)
    # then as many calls that each also record a pair of events around the
    # chunkwise kernel itself (after the control-block reset): the roofline's
    # duration (the event records add a little gap between calls, so these
    # calls do not time the step)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in pairs:  # creates the underlying events
        a.record()
        b.record()
    torch.cuda.synchronize()
    for ev in pairs:
        step(ev)
    torch.cuda.synchronize()
    kus = [a.elapsed_time(b) * 1e3 for a, b in pairs]
    kernel_ms = sum(kus) / steps / 1e3
    rr.check_chunkwise(ws)  # no wait of the timed calls gave up (control word clear)
    cold = []
    if cold_reps:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
        for _ in range(cold_reps):
            scratch.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()  # creates the events (the library records them again around the kernel)
            b.record()
            step((a, b))
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b) * 1e3)
        del scratch
    flops = chunkwise_flops(w.batch, w.seqlen, w.heads, w.dk, w.dv, w.chunk)
    st_f, out_f = chunkwise_split_flops(w.batch, w.seqlen, w.heads, w.dk, w.dv, w.chunk)
    return {
        "workload": w,
        "ms": ms,
        "kernel_ms": kernel_ms,
        "kernel_us_pct": (_pct(kus, 0.1), _pct(kus, 0.5), _pct(kus, 0.9)),
        "cold_kernel_us": _pct(cold, 0.5) if cold else None,
        "wall_s": wall,
        "flops": flops,
        "dense_flops": chunkwise_dense_flops(w.batch, w.seqlen, w.heads, w.dk, w.dv, w.chunk),
        "tflops": flops / (ms * 1e-3) / 1e12,
        "kernel_tflops": flops / (kernel_ms * 1e-3) / 1e12,
        "state_flops": st_f,
        "out_flops": out_f,
        "bytes": chunkwise_bytes(w.batch, w.seqlen, w.heads, w.dk, w.dv, gate=w.gate_scale is not None),
    }


def bench_parallel(steps, warmup):
    import torch

    import retnet_retention_amd as rr
    from synth import get

    w = get("retention_3b")
    q, k, v, g = (t.torch("cuda:0") for t in w.inputs())
    out = torch.empty_like(v)

    def step():
        rr.parallel_fwd(q, k, v, g, rotary_base=w.rotary_base, out=out)

    ms, _ = time_calls(step, steps, warmup, settle_ms=SETTLE_MS)
    flops = parallel_flops(w.batch, w.seqlen, w.heads, w.dk, w.dv)
    return {"workload": w, "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}


def bench_parallel_bwd(steps, warmup):
    """Backward of the parallel form on the 3B workload (rotation, gate):
    dq, dk, dv, dg from a seeded dout."""
    import torch

    import retnet_retention_amd as rr
    from synth import get

    w = get("retention_3b")
    q, k, v, g = (t.torch("cuda:0") for t in w.inputs())
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(w.seed + 7)
    dout = (torch.randn(v.shape, generator=gen, device="cuda:0") / 8).to(v.dtype)
    ws = torch.empty(_bwd_workspace_bytes(q, v, w.rotary_base), dtype=torch.uint8, device="cuda:0")

    def step():
        rr.parallel_bwd(q, k, v, dout, g, rotary_base=w.rotary_base, workspace=ws)

    ms, _ = time_calls(step, steps, warmup, settle_ms=SETTLE_MS)
    flops = 3 * parallel_flops(w.batch, w.seqlen, w.heads, w.dk, w.dv)
    return {"workload": w, "ms": ms, "flops": flops, "tflops": flops / (ms * 1e-3) / 1e12}


def bench_chunkwise_bwd(steps, warmup):
    """Backward of the chunkwise form on the 7B long-context workload (gate,
    no rotation, no carried state): dq, dk, dv, dg from a seeded dout."""
    import ctypes

    import torch

    import retnet_retention_amd as rr
    import retnet_retention_amd.binding as B
    from synth import get

    w = get("retention_7b_8k")
    q, k, v, g = (t.torch("cuda:0") for t in w.inputs())
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(w.seed + 7)
    dout = (torch.randn(v.shape, generator=gen, device="cuda:0") / 8).to(v.dtype)
    desc, keep = B._desc_for(q, v, None, 0.0, 0, 1e-5)
    need = B.lib().retention_chunkwise_bwd_workspace_bytes(ctypes.byref(desc), w.chunk, 1)
    del keep
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")

    def step():
        rr.chunkwise_bwd(q, k, v, dout, g, chunk=w.chunk, workspace=ws)

    ms, _ = time_calls(step, steps, warmup, settle_ms=SETTLE_MS)
    rr.check_chunkwise(ws)
    flops = 3 * chunkwise_flops(w.batch, w.seqlen, w.heads, w.dk, w.dv, w.chunk)
    return {"workload": w, "ms": ms, "flops": flops, "tflops": flops / (ms * 1e-3) / 1e12}


def bench_score_map(steps, warmup):
    """Score map of the last token on the 3B workload's q, k (rotation): a
    stream over k. Bytes: k once plus the query rows and the fp32 map."""
    import torch

    import retnet_retention_amd as rr
    from synth import get

    w = get("retention_3b")
    q, k, _, _ = (t.torch("cuda:0") for t in w.inputs())
    ws = torch.empty(w.seqlen * w.dk // 2 * 8 + 256, dtype=torch.uint8, device="cuda:0")
    ms, _ = time_calls(lambda: rr.score_map(q, k, rotary_base=w.rotary_base, workspace=ws), steps, warmup,
                       settle_ms=SETTLE_MS)
    nbytes = k.numel() * k.element_size() + w.batch * w.seqlen * 4
    return {"workload": w, "us": ms * 1e3, "gbps": nbytes / (ms * 1e-3) / 1e9}


def _bwd_workspace_bytes(q, v, rotary_base):
    import ctypes

    import retnet_retention_amd.binding as B

    desc, keep = B._desc_for(q, v, None, rotary_base, 0, 1e-5)
    n = B.lib().retention_parallel_bwd_workspace_bytes(ctypes.byref(desc), 1)
    del keep
    return n


def bench_decode(n_steps=256, warmup=16, batches=None, graph=True):
    """Prefill 8 distinct sequences of 8192 tokens (chunkwise, seeded GPU
    normals / 16 in bf16), tile the states to the batch, then time decode."""
    import torch

    import retnet_retention_amd as rr
    from synth import get

    w = get("retention_7b_decode")
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    distinct = 8
    shape = (distinct, w.seqlen, w.heads, w.dk)

    def normal(shp, scale):
        return (torch.randn(shp, generator=gen, device=dev, dtype=torch.float32) * scale).to(torch.bfloat16)

    pq, pk, pv, pg = (normal(shape, w.qkv_scale) for _ in range(4))
    base_state = torch.empty((distinct, w.heads, w.dk, w.dv), device=dev)
    rr.chunkwise_fwd(pq, pk, pv, pg, chunk=w.chunk, state_out=base_state)
    torch.cuda.synchronize()
    del pq, pk, pv, pg
    results = {}
    for bsz in batches or w.decode_batches:
        reps = (bsz + distinct - 1) // distinct
        state = base_state.repeat(reps, 1, 1, 1)[:bsz].contiguous()
        sshape = (bsz, 1, w.heads, w.dk)
        nin = 32  # distinct per-step inputs, cycled
        ins = [tuple(normal(sshape, s) for s in (w.qkv_scale, w.qkv_scale, w.qkv_scale, w.gate_scale))
               for _ in range(nin)]
        out = torch.empty(sshape, device=dev, dtype=torch.bfloat16)
        it = [0]

        def step():
            q, k, v, g = ins[it[0] % nin]
            it[0] += 1
            rr.recurrent_step(q, k, v, state, g, pos=w.seqlen + it[0], out=out)

        ms, _ = time_calls(step, n_steps, warmup, settle_ms=SETTLE_MS)
        nbytes = step_bytes(bsz, w.heads, w.dk, w.dv)
        results[bsz] = {"us_per_step": ms * 1e3, "tokens_per_s": bsz / (ms * 1e-3),
                        "gbps": nbytes / (ms * 1e-3) / 1e9}
        # the same steps replayed from a captured HIP graph (one graph of nin
        # steps, launched back to back): no per-launch host work between steps
        if graph:
            graph_ms = _graph_step_ms(step, nin, max(n_steps // nin, 2))
            results[bsz]["graph_us_per_step"] = graph_ms * 1e3
            results[bsz]["graph_gbps"] = nbytes / (graph_ms * 1e-3) / 1e9
        del state, ins
    return w, results


def bench_sweep(steps=10, warmup=20):
    """Chunkwise kernel time against context length (chunk 512) and against
    chunk size (8192 tokens), at the 7B layer's heads: batch 1, 16 heads x
    256, bf16, gate, state out. Inputs: seeded normals / 16 drawn on the GPU."""
    import torch

    import retnet_retention_amd as rr

    h, d = 16, 256
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(7)

    def run(n, chunk):
        q, k, v, g = ((torch.randn((1, n, h, d), generator=gen, device="cuda:0") / 16).to(torch.bfloat16)
                      for _ in range(4))
        state = torch.empty((1, h, d, d), device="cuda:0")
        out = torch.empty_like(v)
        ws = torch.empty(rr.chunkwise_workspace_bytes(q, v, chunk), dtype=torch.uint8, device="cuda:0")
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(steps)]
        for a, b in pairs:
            a.record()
            b.record()
        for _ in range(warmup):
            rr.chunkwise_fwd(q, k, v, g, chunk=chunk, state_out=state, out=out, workspace=ws)
        for ev in pairs:
            rr.chunkwise_fwd(q, k, v, g, chunk=chunk, state_out=state, out=out, workspace=ws, kernel_events=ev)
        torch.cuda.synchronize()
        rr.check_chunkwise(ws)
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)[steps // 2]
        flops = chunkwise_flops(1, n, h, d, d, chunk)
        row = {"tokens": n, "chunk": chunk, "kernel_us": round(us, 1), "us_per_1k_tokens": round(us * 1024 / n, 2),
               "tflops": round(flops / (us * 1e-6) / 1e12, 1),
               "hbm_frac": round(chunkwise_bytes(1, n, h, d, d) / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        print(f"sweep: {n} tokens, chunk {chunk}: {us:.1f} us, {row['us_per_1k_tokens']} us per 1k tokens, "
              f"{row['tflops']} TFLOP/s", file=sys.stderr, flush=True)
        del q, k, v, g, state, out, ws
        return row

    context = [run(n, 512) for n in (2048, 8192, 16384, 32768, 65536)]
    chunks = [run(8192, c) for c in (64, 128, 256, 512, 1024)]
    return {"shape": "batch 1, 16 heads x 256, bf16, gate, state out", "context_at_chunk_512": context,
            "chunk_at_8192_tokens": chunks}


VARLEN_LENS = (8192, 3000, 2048, 1500, 1024, 400, 200, 20)  # 16384 tokens in all


def bench_varlen(steps, warmup):
    """Chunkwise form over a packed ragged batch (prefill of sequences of
    different lengths) at the 7B layer's heads (16 x 256, bf16, gate, state
    out, chunk 512): eight sequences of VARLEN_LENS tokens, 16384 in all,
    beside the same 16384 tokens as two sequences of 8192. Both are timed
    per call (control reset and kernel). Inputs: seeded normals / 16 drawn on
    the GPU; the flops are the chunkwise count summed per sequence."""
    import torch

    import ctypes

    import retnet_retention_amd as rr
    from retnet_retention_amd import binding as B

    h, d, chunk = 16, 256, 512
    tot = sum(VARLEN_LENS)
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(11)
    q, k, v, g = ((torch.randn((tot, h, d), generator=gen, device="cuda:0") / 16).to(torch.bfloat16)
                  for _ in range(4))
    cu = torch.tensor([0] + list(itertools.accumulate(VARLEN_LENS)), dtype=torch.int32, device="cuda:0")
    out = torch.empty_like(v)
    st = torch.empty((len(VARLEN_LENS), h, d, d), device="cuda:0")
    maxlen = max(VARLEN_LENS)
    # the packed call's workspace (8 sequences of up to 8192) also covers the batched one
    desc, keep = B.make_desc(len(VARLEN_LENS), maxlen, h, d, d, B.RET_BF16)
    ws = torch.empty(B.lib().retention_chunkwise_varlen_workspace_bytes(ctypes.byref(desc), chunk),
                     dtype=torch.uint8, device="cuda:0")
    ms_var, _ = time_calls(lambda: rr.chunkwise_varlen_fwd(q, k, v, cu, maxlen, g, chunk=chunk, state_out=st, out=out,
                                                           workspace=ws), steps, warmup, settle_ms=SETTLE_MS)
    rr.check_chunkwise(ws)
    shp = (2, tot // 2, h, d)
    st2 = torch.empty((2, h, d, d), device="cuda:0")
    ms_fix, _ = time_calls(lambda: rr.chunkwise_fwd(q.view(shp), k.view(shp), v.view(shp), g.view(shp), chunk=chunk,
                                                    state_out=st2, out=out.view(shp), workspace=ws), steps, warmup,
                         settle_ms=SETTLE_MS)
    rr.check_chunkwise(ws)
    flops_var = sum(chunkwise_flops(1, n, h, d, d, chunk) for n in VARLEN_LENS)
    flops_fix = chunkwise_flops(2, tot // 2, h, d, d, chunk)
    return {"lens": list(VARLEN_LENS), "ms": ms_var, "tflops": flops_var / (ms_var * 1e-3) / 1e12,
            "tokens_per_s": tot / (ms_var * 1e-3), "equal_ms": ms_fix,
            "equal_tflops": flops_fix / (ms_fix * 1e-3) / 1e12}


def _graph_step_ms(step, per_graph, replays):
    """Device time per step of `per_graph` calls of `step` captured into one
    graph and replayed `replays` times (after two untimed replays)."""
    import torch

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capturing stream, as capture requires
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            step()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (replays * per_graph)
    del graph
    return ms


def cpu_baseline(sample_seqs=2, min_seconds=10.0, max_runs=20):
    """The fp64 oracle's chunkwise form on the headline workload (`sample_seqs`
    of its 2 sequences, all 16 heads, all 8192 tokens), repeated until at
    least `min_seconds` of CPU work; the rate is that of the mean run."""
    import oracle
    from synth import get

    w = get("retention_7b_8k")
    q, k, v, g = w.inputs(batch=sample_seqs)
    threads = None
    try:
        from threadpoolctl import threadpool_info

        threads = max((p.get("num_threads", 0) for p in threadpool_info()), default=None)
    except Exception:
        pass
    cores = len(os.sched_getaffinity(0))
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    runs, t0 = 0, time.perf_counter()
    while runs < max_runs and (runs == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.retention("chunkwise", q.f64, k.f64, v.f64, g=g.f64, chunk=w.chunk)
        runs += 1
    dt = (time.perf_counter() - t0) / runs
    flops = chunkwise_flops(sample_seqs, w.seqlen, w.heads, w.dk, w.dv, w.chunk)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads or cores,
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": f"chunkwise fp64 oracle on {sample_seqs} of 2 sequences of retention_7b_8k "
                  f"(8192 tokens, 16 heads x 256, chunk 512, gate), {runs} runs of {dt:.2f} s each on "
                  f"{threads or cores} BLAS threads ({cores} cores in the affinity mask)",
        "seconds": dt * runs,
    }


# ---------------------------------------------------------------------------
# rocprofv3 runs (children of this process, which never touches the GPU in
# this mode) and their text summaries
# ---------------------------------------------------------------------------
# counter passes: a few calls each (the counters are per dispatch)
LEG_ARGS = {
    "chunkwise": ["--only", "chunkwise", "--steps", "10", "--warmup", "2", "--no-other-chunkwise", "--cold-reps",
                  "0"],
    "decode": ["--only", "decode", "--decode-batches", "64", "--decode-steps", "64", "--no-decode-graph"],
    "parallel": ["--only", "parallel", "--steps", "10", "--warmup", "2"],
}
# kernel statistics: the benchmark's own default calls (warm-up included, so
# the averages are those of the timed, warmed-up calls to within a few %)
STATS_ARGS = {
    "chunkwise": ["--only", "chunkwise", "--no-other-chunkwise", "--cold-reps", "0"],
    "decode": ["--only", "decode", "--decode-batches", "64", "--no-decode-graph"],
    "parallel": ["--only", "parallel"],
    "parallel_bwd": ["--only", "parallel_bwd"],
    "chunkwise_bwd": ["--only", "chunkwise_bwd"],
    "varlen": ["--only", "varlen"],
}
SQ_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_LDS",
               "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS", "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE"]
# where the waves of the chunkwise kernel spend their cycles (one pass each)
SQ_STALL_SETS = [
    ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_LDS",
     "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM", "SQ_IFETCH"],
    ["SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL", "SQ_INST_LEVEL_LDS", "SQ_INSTS_MFMA", "SQ_INSTS_SALU",
     "SQ_ACTIVE_INST_MISC", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_VMEM"],
]


def _run_profiler(args, log, limit):
    print("$ " + " ".join(args), file=sys.stderr, flush=True)
    with open(log, "w") as f:
        r = subprocess.run(args, stdout=f, stderr=subprocess.STDOUT, timeout=limit, cwd="/tmp",
                           env={**os.environ, "TMPDIR": "/tmp"})
    if r.returncode != 0:
        tail = open(log).read()[-3000:]
        raise SystemExit(f"profiler run failed ({r.returncode}):\n{tail}")


def _bench_cmd(leg_args):
    return ["python3", os.path.join(ROOT, "bench.py"), *leg_args, "--no-cpu-baseline"]


PROFILE_OUT = [None]  # the --profile-out directory, shown as <out> in the recorded commands


def _rel(cmd):
    out = " ".join(cmd)
    if PROFILE_OUT[0]:
        out = out.replace(PROFILE_OUT[0], "<out>")
    return out.replace(ROOT + "/", "").replace(ROOT, ".")


def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        rows.extend(csv.DictReader(open(f)))
    return rows


def _per_dispatch(rows, counter, match):
    vals = {}
    for r in rows:
        if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
            key = (r.get("Dispatch_Id"), r.get("Agent_Id"))
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def profile_stats(out, raw):
    for leg, leg_args in STATS_ARGS.items():
        d = os.path.join(raw, f"stats_{leg}")
        cmd = ["rocprofv3", "--kernel-trace", "--stats", "-d", d, "-o", "run", "--output-format", "csv", "--",
               *_bench_cmd(leg_args)]
        _run_profiler(cmd, d + ".log", 600)
        line = [ln for ln in open(d + ".log") if ln.startswith("{")]
        stats = list(csv.DictReader(open(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)[0])))
        name = {"chunkwise": "chunkwise_7b_8k", "decode": "decode_step_7b_b64", "parallel": "parallel_3b",
                "parallel_bwd": "parallel_backward_3b", "chunkwise_bwd": "chunkwise_backward_7b_8k",
                "varlen": "chunkwise_varlen_ragged_16k"}[leg]
        with open(os.path.join(out, f"{name}_kernel_stats.txt"), "w") as f:
            f.write(f"rocprofv3 kernel statistics, {leg} leg of the benchmark\n")
            f.write("made by: python bench.py --profile stats --profile-out <out>\n")
            f.write(f"command: {_rel(cmd)}\n")
            f.write(f"kernel sources: {source_hash()} (chunkwise/parallel kernel), host {os.uname().nodename}\n\n")
            f.write(f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share%':>7s}\n")
            for r in stats[:12]:
                f.write(f"{r['Name'][:70]:70s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:10.2f} "
                        f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                        f"{float(r['Percentage']):7.2f}\n")
            if line:
                f.write("\nbenchmark line of the same (profiled) run, HIP-event timed:\n" + line[-1])
        print(f"wrote {name}_kernel_stats.txt", file=sys.stderr, flush=True)


def profile_traffic(out, raw):
    """Two counter passes (FETCH_SIZE, then WRITE_SIZE) over the chunkwise leg
    plus a plain copy of known size; each counter is scaled by what it reads
    for the copy."""
    leg = ["--only", "chunkwise", "--steps", "2", "--warmup", "1", "--no-other-chunkwise", "--cold-reps", "0",
           "--copy-probe"]
    res, cmds = {}, []
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = os.path.join(raw, f"pmc_{counter.lower()}")
        cmd = ["rocprofv3", "--pmc", counter, "-d", d, "-o", "run", "--output-format", "csv", "--",
               *_bench_cmd(leg)]
        _run_profiler(cmd, d + ".log", 180)
        cmds.append(cmd)
        rows = _counter_rows(d)
        kern = _per_dispatch(rows, counter, lambda n: CHUNKWISE_KERNEL in n)
        copy = _per_dispatch(rows, counter, lambda n: "copy" in n.lower() and "retention" not in n)
        if not kern or not copy:
            raise SystemExit(f"{counter}: kernel dispatches {len(kern)}, copy dispatches {len(copy)}")
        kib = sum(kern) / len(kern)
        copy_kib = max(copy)  # the copies are the largest non-retention dispatches
        scale = COPY_PROBE_BYTES / (copy_kib * 1024.0)
        res[counter] = (kib, copy_kib, scale, kib * 1024.0 * scale, len(kern))
    fetch, write = res["FETCH_SIZE"][3], res["WRITE_SIZE"][3]
    from synth import get

    w = get("retention_7b_8k")
    alg = chunkwise_bytes(w.batch, w.seqlen, w.heads, w.dk, w.dv)
    with open(os.path.join(out, "chunkwise_7b_8k_traffic.txt"), "w") as f:
        f.write("HBM traffic of the chunkwise kernel on the 7B long-context workload (batch 2, 8192 tokens,\n"
                "16 heads x 256, chunk 512, bf16, gate, state out), from two rocprofv3 counter passes\n")
        f.write("made by: python bench.py --profile traffic --profile-out <out>\n")
        for c in cmds:
            f.write(f"command: {_rel(c)}\n")
        f.write(f"kernel: {CHUNKWISE_KERNEL}<bf16, 256>\n")
        f.write(f"source_hash: {source_hash()}\n")
        for c, (kib, copy_kib, scale, b, n) in res.items():
            f.write(f"  {c}: {kib:.0f} KiB per dispatch (mean of {n}); copy of {COPY_PROBE_BYTES >> 20} MiB reads "
                    f"{copy_kib:.0f} KiB -> scale {scale:.4f} -> {b / 1e6:.1f} MB\n")
        f.write(f"fetch_bytes_per_launch: {int(fetch)}\n")
        f.write(f"write_bytes_per_launch: {int(write)}\n")
        f.write(f"traffic_bytes_per_launch: {int(fetch + write)}\n")
        f.write(f"algorithmic_bytes_per_launch: {alg}\n")
        f.write(f"  ratio measured/algorithmic: {(fetch + write) / alg:.3f}\n")
    print("wrote chunkwise_7b_8k_traffic.txt", file=sys.stderr, flush=True)


def profile_counters(out, raw):
    """SQ counter passes per leg: matrix-core activity and LDS behaviour, and
    for the chunkwise leg where its waves spend their cycles."""
    for leg in ("chunkwise", "parallel", "decode"):
        leg_args = [*LEG_ARGS[leg]]
        if leg != "decode":
            leg_args[leg_args.index("--steps") + 1] = "2"
        match = {"chunkwise": lambda n: CHUNKWISE_KERNEL in n, "parallel": lambda n: "retention_parallel" in n,
                 "decode": lambda n: "recurrent_step" in n}[leg]
        name = {"chunkwise": "chunkwise_7b_8k", "decode": "decode_step_7b_b64", "parallel": "parallel_3b"}[leg]
        sets = [SQ_COUNTERS] + (SQ_STALL_SETS if leg == "chunkwise" else [])
        lines, vals = [], {}
        for k, counters in enumerate(sets):
            d = os.path.join(raw, f"pmc_sq_{leg}_{k}")
            cmd = ["rocprofv3", "--pmc", *counters, "-d", d, "-o", "run", "--output-format", "csv", "--",
                   *_bench_cmd(leg_args)]
            _run_profiler(cmd, d + ".log", 180)
            rows = _counter_rows(d)
            lines.append(f"command: {_rel(cmd)}\n")
            for c in counters:
                v = _per_dispatch(rows, c, match)
                vals[c] = sum(v) / len(v) if v else float("nan")
                lines.append(f"  {c:32s} {vals[c]:.6g}  (dispatches {len(v)})\n")
        with open(os.path.join(out, f"{name}_sq_counters.txt"), "w") as f:
            f.write(f"rocprofv3 SQ counters, {leg} leg, mean per dispatch of the retention kernel\n")
            f.write("made by: python bench.py --profile counters --profile-out <out>\n")
            f.write(f"kernel sources: {source_hash()}\n")
            f.writelines(lines)
            xcds, cus, simds = 8, 256, 4
            gui = vals["GRBM_GUI_ACTIVE"] / xcds  # GRBM_GUI_ACTIVE sums the 8 XCDs
            f.write(f"derived: kernel cycles (GRBM_GUI_ACTIVE / {xcds} XCDs) = {gui:.4g}\n")
            f.write(f"derived: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {cus} CUs x {simds} SIMDs) = "
                    f"{vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * cus * simds):.4f}\n")
            f.write(f"derived: bf16 matrix flops executed = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 = "
                    f"{512 * vals['SQ_INSTS_VALU_MFMA_MOPS_BF16'] / 1e9:.2f} GFLOP per dispatch\n")
            if "SQ_WAVE_CYCLES" in vals:
                wc = vals["SQ_WAVE_CYCLES"]
                for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_LDS",
                          "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_MISC", "SQ_ACTIVE_INST_SCA"):
                    f.write(f"derived: {c} / SQ_WAVE_CYCLES = {vals[c] / wc:.4f}\n")
        print(f"wrote {name}_sq_counters.txt", file=sys.stderr, flush=True)


# memory-system passes (at most 4 TCC counters per pass): L2 hits, the EA
# read latency (requests in flight / requests), and back-pressure from DRAM
TCC_SETS = [
    ["TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_LEVEL_sum"],
    ["TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_EA0_WRREQ_STALL_sum", "TCC_EA0_WRREQ_sum", "TCC_BUSY_sum",
     "GRBM_GUI_ACTIVE"],
]


def profile_memory(out, raw):
    """TCC counter passes for the chunkwise and decode legs: how the memory
    system behaves under each (L2 hit rate, loaded read latency, stalls)."""
    for leg in ("chunkwise", "decode"):
        leg_args = [*LEG_ARGS[leg]]
        if leg != "decode":
            leg_args[leg_args.index("--steps") + 1] = "2"
        match = {"chunkwise": lambda n: CHUNKWISE_KERNEL in n, "decode": lambda n: "recurrent_step" in n}[leg]
        name = {"chunkwise": "chunkwise_7b_8k", "decode": "decode_step_7b_b64"}[leg]
        lines, vals = [], {}
        for k, counters in enumerate(TCC_SETS):
            d = os.path.join(raw, f"pmc_tcc_{leg}_{k}")
            cmd = ["rocprofv3", "--pmc", *counters, "-d", d, "-o", "run", "--output-format", "csv", "--",
                   *_bench_cmd(leg_args)]
            _run_profiler(cmd, d + ".log", 180)
            rows = _counter_rows(d)
            lines.append(f"command: {_rel(cmd)}\n")
            for c in counters:
                v = _per_dispatch(rows, c, match)
                vals[c] = sum(v) / len(v) if v else float("nan")
                lines.append(f"  {c:38s} {vals[c]:.6g}  (dispatches {len(v)})\n")
        with open(os.path.join(out, f"{name}_memory_counters.txt"), "w") as f:
            f.write(f"rocprofv3 TCC (L2 / memory interface) counters, {leg} leg, mean per dispatch\n")
            f.write("made by: python bench.py --profile memory --profile-out <out>\n")
            f.write(f"kernel sources: {source_hash()}\n")
            f.writelines(lines)
            xcds, channels = 8, 128  # 16 L2 channels per XCD
            gui = vals["GRBM_GUI_ACTIVE"] / xcds
            hit, miss = vals["TCC_HIT_sum"], vals["TCC_MISS_sum"]
            f.write(f"derived: kernel cycles (GRBM_GUI_ACTIVE / {xcds}) = {gui:.4g}\n")
            f.write(f"derived: L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS) = {hit / (hit + miss):.4f}\n")
            f.write(f"derived: mean EA read latency = TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ = "
                    f"{vals['TCC_EA0_RDREQ_LEVEL_sum'] / vals['TCC_EA0_RDREQ_sum']:.1f} cycles\n")
            f.write(f"derived: mean EA reads in flight per channel = TCC_EA0_RDREQ_LEVEL / (cycles x {channels}) = "
                    f"{vals['TCC_EA0_RDREQ_LEVEL_sum'] / (gui * channels):.1f}\n")
            for c in ("TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_EA0_WRREQ_STALL_sum", "TCC_BUSY_sum"):
                f.write(f"derived: {c} / (cycles x {channels} channels) = {vals[c] / (gui * channels):.4f}\n")
        print(f"wrote {name}_memory_counters.txt", file=sys.stderr, flush=True)


def roofline_object(cw, alg_gbps, traffic):
    """Roofline of the chunkwise kernel: bound by HBM when the workload's
    algorithmic intensity lies below the ridge point, else by the matrix
    cores; both fractions are given."""
    intensity = cw["flops"] / cw["bytes"]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    hbm = {"achieved": round(alg_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
           "frac": round(alg_gbps / PEAK_HBM_GBPS, 4)}
    mfma = {"achieved": round(cw["kernel_tflops"], 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(cw["kernel_tflops"] / PEAK_BF16_TFLOPS, 4)}
    bound, other = ("hbm", "mfma") if intensity < ridge else ("mfma", "hbm")
    main, side = (hbm, mfma) if bound == "hbm" else (mfma, hbm)
    return {"bound": bound, "kernel": f"{CHUNKWISE_KERNEL}<bf16,256>", **main,
            "traffic": traffic["bytes"] if traffic else None,
            "kernel_us": round(cw["kernel_ms"] * 1e3, 1),
            "algorithmic_bytes": cw["bytes"], "flops_per_launch": cw["flops"],
            "intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1),
            "attainable_tflops": round(min(PEAK_BF16_TFLOPS, intensity * PEAK_HBM_GBPS / 1e3), 1),
            other: side,
            "measured_gbps": (round(traffic["bytes"] / (cw["kernel_ms"] * 1e-3) / 1e9, 1) if traffic else None)}


def profile(kinds, out):
    PROFILE_OUT[0] = out
    os.makedirs(out, exist_ok=True)
    raw = os.path.join(out, "raw")
    os.makedirs(raw, exist_ok=True)
    if "stats" in kinds:
        profile_stats(out, raw)
    if "traffic" in kinds:
        profile_traffic(out, raw)
    if "counters" in kinds:
        profile_counters(out, raw)
    if "memory" in kinds:
        profile_memory(out, raw)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU's clocks take tens of milliseconds of load to settle: 5 warm-up
    # calls time the chunkwise call 14% slower than 200 do
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--only", choices=["chunkwise", "decode", "parallel", "parallel_bwd", "chunkwise_bwd", "score_map", "varlen",
                                       "sweep"],
                    default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-chunkwise", action="store_true",
                    help="skip the chunkwise timings of the 200M and 3B workloads")
    ap.add_argument("--no-decode-graph", action="store_true", help="skip the graph-replayed decode timing")
    ap.add_argument("--sweep", action="store_true",
                    help="also sweep the chunkwise kernel over context length and chunk size")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="chunkwise calls timed after evicting the caches (0: none)")
    ap.add_argument("--decode-batches", type=int, nargs="*", default=None)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--copy-probe", action="store_true", help="also run a plain copy of known size")
    ap.add_argument("--profile", nargs="+", choices=["stats", "traffic", "counters", "memory"], default=None,
                    help="run the named rocprofv3 passes over this benchmark and write text summaries")
    ap.add_argument("--profile-out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.profile:
        profile(args.profile, os.path.abspath(args.profile_out))
        return

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)
    import retnet_retention_amd as rr

    rr.lib()  # fail loudly if the HIP library is missing

    line = {}
    # The headline leg runs last: the legs before it keep the GPU busy for
    # seconds, so its W warm-up and K timed calls run at settled clocks (with
    # a cold GPU, 5 warm-up calls time the chunkwise call about 14% slower
    # than 200 do). Its inputs are drawn on the host first, so that no host
    # work stands between the last GPU leg and its calls.
    headline_inputs = chunkwise_inputs("retention_7b_8k") if args.only in (None, "chunkwise") else None
    if args.only in (None, "decode"):
        wd, dec = bench_decode(args.decode_steps, batches=args.decode_batches, graph=not args.no_decode_graph)
        for b, r in dec.items():
            print(f"decode batch {b}: {r['us_per_step']:.2f} us/step, {r['tokens_per_s']:.0f} tok/s, "
                  f"{r['gbps']:.0f} GB/s", file=sys.stderr, flush=True)
        ref_b = 64 if 64 in dec else max(dec)
        line["decode"] = {
            "workload": f"{wd.name}: 16 heads x 256, fp32 state from an 8192-token chunkwise prefill, bf16 steps",
            "per_batch": {str(b): {k: round(v, 2) for k, v in r.items()} for b, r in dec.items()},
            f"tokens_per_s_b{ref_b}": round(dec[ref_b]["tokens_per_s"], 1),
            f"hbm_gbps_b{ref_b}": round(dec[ref_b]["gbps"], 1),
            f"hbm_frac_b{ref_b}": round(dec[ref_b]["gbps"] / PEAK_HBM_GBPS, 4),
        }
    if args.only in (None, "parallel"):
        par = bench_parallel(max(args.steps // 2, 3), args.warmup)
        print(f"parallel {par['workload'].name}: {par['ms']:.3f} ms, {par['tflops']:.1f} TFLOP/s", file=sys.stderr,
              flush=True)
        line["parallel"] = {"workload": f"{par['workload'].name}: batch 4, 2048 tokens, 10 x 256, rotation, gate",
                            "ms": round(par["ms"], 4), "tflops": round(par["tflops"], 2),
                            "mfma_frac": round(par["tflops"] / PEAK_BF16_TFLOPS, 4)}
    if args.only in (None, "parallel_bwd"):
        pb = bench_parallel_bwd(max(args.steps // 2, 3), max(args.warmup // 4, 3))
        print(f"parallel backward {pb['workload'].name}: {pb['ms']:.3f} ms, {pb['tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        line["parallel_backward"] = {
            "workload": f"{pb['workload'].name}: batch 4, 2048 tokens, 10 x 256, rotation, gate; dq, dk, dv, dg",
            "ms": round(pb["ms"], 4), "tflops": round(pb["tflops"], 2),
            "mfma_frac": round(pb["tflops"] / PEAK_BF16_TFLOPS, 4),
            "flops": "3 x the forward's algorithmic count (dQ, dK, dV products); the recomputed forward "
                     "for the GroupNorm gradient is not counted"}
    if args.only in (None, "chunkwise_bwd"):
        cb2 = bench_chunkwise_bwd(max(args.steps // 5, 3), max(args.warmup // 10, 3))
        print(f"chunkwise backward {cb2['workload'].name}: {cb2['ms']:.3f} ms, {cb2['tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        line["chunkwise_backward"] = {
            "workload": f"{cb2['workload'].name}: batch 2, 8192 tokens, 16 x 256, chunk 512, gate; dq, dk, dv, dg",
            "ms": round(cb2["ms"], 4), "tflops": round(cb2["tflops"], 2),
            "mfma_frac": round(cb2["tflops"] / PEAK_BF16_TFLOPS, 4),
            "flops": "3 x the chunkwise form's algorithmic count; the recomputed forward is not counted"}
    if args.only in (None, "score_map"):
        sm = bench_score_map(max(args.steps, 10), max(args.warmup // 4, 10))
        print(f"score map {sm['workload'].name}: {sm['us']:.1f} us, {sm['gbps']:.0f} GB/s", file=sys.stderr,
              flush=True)
        line["score_map"] = {"workload": f"{sm['workload'].name}: last token over 2048, 10 heads x 256, rotation",
                             "us": round(sm["us"], 2), "gbps": round(sm["gbps"], 1),
                             "hbm_frac": round(sm["gbps"] / PEAK_HBM_GBPS, 4),
                             "note": "includes the angle-table kernel (rotation) and launch gaps"}
    if args.only in (None, "varlen"):
        vl = bench_varlen(max(args.steps // 2, 10), max(args.warmup // 4, 10))
        print(f"varlen {vl['lens']}: {vl['ms']:.3f} ms, {vl['tflops']:.1f} TFLOP/s; two x 8192: {vl['equal_ms']:.3f} ms",
              file=sys.stderr, flush=True)
        line["varlen"] = {
            "workload": "packed ragged batch: 8 sequences of " + "/".join(map(str, vl["lens"])) +
                        " tokens (16384 in all), 16 x 256, chunk 512, bf16, gate, state out",
            "ms": round(vl["ms"], 4), "tflops": round(vl["tflops"], 2), "tokens_per_s": round(vl["tokens_per_s"]),
            "same_tokens_as_2x8192_ms": round(vl["equal_ms"], 4),
            "same_tokens_as_2x8192_tflops": round(vl["equal_tflops"], 2),
            "note": "per call: control reset and kernel; flops are the chunkwise count summed per sequence"}
    if args.only in (None, "chunkwise"):
        cw = bench_chunkwise(args.steps, args.warmup, cold_reps=args.cold_reps, prepared=headline_inputs)
        del headline_inputs
        w = cw["workload"]
        print(f"chunkwise {w.name}: {cw['ms']:.3f} ms/step, {cw['tflops']:.1f} TFLOP/s; kernel alone "
              f"{cw['kernel_ms'] * 1e3:.1f} us, {cw['kernel_tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        alg_gbps = cw["bytes"] / (cw["kernel_ms"] * 1e-3) / 1e9
        # the same form on the two smaller chunkwise workloads (warm, reported
        # beside the headline workload, not as its value)
        others = {}
        if not args.no_other_chunkwise:
            for oname in ("retention_200m", "retention_3b"):
                o = bench_chunkwise(max(args.steps // 2, 3), max(args.warmup // 4, 3), name=oname,
                                    settle_ms=SETTLE_MS)
                ow = o["workload"]
                print(f"chunkwise {oname}: {o['ms']:.3f} ms/step, {o['tflops']:.1f} TFLOP/s; kernel alone "
                      f"{o['kernel_ms'] * 1e3:.1f} us, {o['kernel_tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
                others[oname] = {
                    "workload": f"batch {ow.batch}, {ow.seqlen} tokens, {ow.heads} x {ow.dk}, chunk {ow.chunk}"
                                + (", rotation" if ow.rotary_base else "") + ", gate",
                    "ms": round(o["ms"], 4), "kernel_us": round(o["kernel_ms"] * 1e3, 1),
                    "kernel_tflops": round(o["kernel_tflops"], 2),
                    "mfma_frac": round(o["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
                    "hbm_frac": round(o["bytes"] / (o["kernel_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        traffic = recorded_traffic()
        line.update({
            "metric": "chunkwise retention TFLOP/s (+% MFMA peak); decode-step tokens/s and HBM GB/s",
            "value": round(cw["tflops"], 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(cw["ms"], 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": w.name, "form": "chunkwise", "batch": w.batch, "seq_len": w.seqlen,
                       "heads": w.heads, "head_dim": w.dk, "chunk": w.chunk, "gate": True, "rotary": False,
                       "state_out": True, "parallelism": "single GPU"},
            # One chunkwise call = a control-block reset (a few microseconds)
            # and the fused chunkwise kernel; `value` charges the whole call,
            # the roofline the kernel's own duration (events recorded around
            # it on the same stream, averaged over the timed calls). The bound
            # is the roofline's own: the workload's algorithmic intensity
            # (flop per HBM byte) against the ridge point peak flops / peak
            # bandwidth; the other ceiling is reported beside it.
            "roofline": roofline_object(cw, alg_gbps, traffic),
        })
        line["chunkwise_detail"] = {
            "kernel_us_p10_p50_p90": [round(x, 1) for x in cw["kernel_us_pct"]],
            "cold_kernel_us_p50": round(cw["cold_kernel_us"], 1) if cw["cold_kernel_us"] else None,
            "cold": "each cold call follows a 512 MiB write that evicts L2 and the Infinity Cache",
            "dense_equivalent_flops_per_launch": cw["dense_flops"],
            "other_workloads": others,
        }
    if args.sweep or args.only == "sweep":
        line["sweep"] = bench_sweep()
    if args.copy_probe:
        copy_probe()
    if args.only is None and not args.no_cpu_baseline:
        cb = cpu_baseline()
        print(f"cpu baseline: {cb['value'] * 1e3:.2f} GFLOP/s ({cb['seconds']:.1f} s in all)", file=sys.stderr,
              flush=True)
        cb.pop("seconds")
        if "value" in line:
            cb["gpu_speedup"] = round(line["value"] / cb["value"], 1)
        line["cpu_baseline"] = cb
    # the contract's keys first, then the legs
    first = [k for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                         "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline") if k in line]
    line = {**{k: line[k] for k in first}, **{k: v for k, v in line.items() if k not in first}}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
