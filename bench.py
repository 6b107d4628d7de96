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
  cpu_baseline -- the fp64 oracle timed on this host on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only chunkwise|decode|parallel]
                       [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E (published)


# ---------------------------------------------------------------------------
# algorithmic work (causal-counted; rotation, masks, GroupNorm, gate not counted)
# ---------------------------------------------------------------------------
def chunkwise_flops(batch, seqlen, heads, dk, dv, chunk):
    total = 0
    for start in range(0, seqlen, chunk):
        b = min(chunk, seqlen - start)
        total += b * (b + 1) * (dk + dv) + 4 * b * dk * dv
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
def time_calls(fn, steps, warmup):
    """Average device time per call over `steps` back-to-back calls (events on
    torch's current stream, which is the stream the library launches on)."""
    import torch

    for _ in range(warmup):
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


def bench_chunkwise(steps, warmup):
    import torch

    import retnet_retention_amd as rr
    from synth import get

    w = get("retention_7b_8k")
    q, k, v, g = (t.torch("cuda:0") for t in w.inputs())
    state = torch.empty((w.batch, w.heads, w.dk, w.dv), device="cuda:0")
    out = torch.empty_like(v)
    ws = torch.empty(rr.chunkwise_workspace_bytes(q, v, w.chunk), dtype=torch.uint8, device="cuda:0")

    def step():
        rr.chunkwise_fwd(q, k, v, g, chunk=w.chunk, state_out=state, out=out, workspace=ws)

    ms, wall = time_calls(step, steps, warmup)
    flops = chunkwise_flops(w.batch, w.seqlen, w.heads, w.dk, w.dv, w.chunk)
    st_f, out_f = chunkwise_split_flops(w.batch, w.seqlen, w.heads, w.dk, w.dv, w.chunk)
    return {
        "workload": w,
        "ms": ms,
        "wall_s": wall,
        "flops": flops,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "state_flops": st_f,
        "out_flops": out_f,
        "bytes": chunkwise_bytes(w.batch, w.seqlen, w.heads, w.dk, w.dv),
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

    ms, _ = time_calls(step, steps, warmup)
    flops = parallel_flops(w.batch, w.seqlen, w.heads, w.dk, w.dv)
    return {"workload": w, "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}


def bench_decode(n_steps=256, warmup=16):
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
    for bsz in w.decode_batches:
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

        ms, _ = time_calls(step, n_steps, warmup)
        nbytes = step_bytes(bsz, w.heads, w.dk, w.dv)
        results[bsz] = {"us_per_step": ms * 1e3, "tokens_per_s": bsz / (ms * 1e-3),
                        "gbps": nbytes / (ms * 1e-3) / 1e9}
        del state, ins
    return w, results


def cpu_baseline(sample_seqs=2):
    """The fp64 oracle's chunkwise form on a bounded sample of the headline
    workload: `sample_seqs` of its 2 sequences, all 16 heads, all 8192 tokens."""
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
    t0 = time.perf_counter()
    oracle.retention("chunkwise", q.f64, k.f64, v.f64, g=g.f64, chunk=w.chunk)
    dt = time.perf_counter() - t0
    flops = chunkwise_flops(sample_seqs, w.seqlen, w.heads, w.dk, w.dv, w.chunk)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads or cores,
        "kind": "oracle",
        "sample": f"chunkwise fp64 oracle on {sample_seqs} of 2 sequences of retention_7b_8k "
                  f"(8192 tokens, 16 heads x 256, chunk 512, gate): {dt:.2f} s on {threads or cores} BLAS threads "
                  f"({cores} cores in affinity mask)",
        "seconds": dt,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["chunkwise", "decode", "parallel"], default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)
    import retnet_retention_amd as rr

    rr.lib()  # fail loudly if the HIP library is missing

    line = {}
    if args.only in (None, "chunkwise"):
        cw = bench_chunkwise(args.steps, args.warmup)
        w = cw["workload"]
        print(f"chunkwise {w.name}: {cw['ms']:.3f} ms/step, {cw['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
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
            "mfma_frac_step": round(cw["tflops"] / PEAK_BF16_TFLOPS, 4),
            "hbm_gbps_step": round(cw["bytes"] / (cw["ms"] * 1e-3) / 1e9, 1),
            # The chunkwise call runs two kernels (per-chunk states, then the
            # fused output); the whole call is timed on its stream.
            "roofline": {"bound": "mfma", "kernel": "chunkwise call (state + output kernels)",
                         "achieved": round(cw["tflops"], 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(cw["tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": None},
        })
    if args.only in (None, "decode"):
        wd, dec = bench_decode()
        for b, r in dec.items():
            print(f"decode batch {b}: {r['us_per_step']:.2f} us/step, {r['tokens_per_s']:.0f} tok/s, "
                  f"{r['gbps']:.0f} GB/s", file=sys.stderr, flush=True)
        line["decode"] = {
            "workload": f"{wd.name}: 16 heads x 256, fp32 state from an 8192-token chunkwise prefill, bf16 steps",
            "per_batch": {str(b): {k: round(v, 2) for k, v in r.items()} for b, r in dec.items()},
            "tokens_per_s_b64": round(dec[64]["tokens_per_s"], 1),
            "hbm_gbps_b64": round(dec[64]["gbps"], 1),
            "hbm_frac_b64": round(dec[64]["gbps"] / PEAK_HBM_GBPS, 4),
        }
    if args.only in (None, "parallel"):
        par = bench_parallel(max(args.steps // 2, 3), args.warmup)
        print(f"parallel {par['workload'].name}: {par['ms']:.3f} ms, {par['tflops']:.1f} TFLOP/s", file=sys.stderr,
              flush=True)
        line["parallel"] = {"workload": f"{par['workload'].name}: batch 4, 2048 tokens, 10 x 256, rotation, gate",
                            "ms": round(par["ms"], 4), "tflops": round(par["tflops"], 2),
                            "mfma_frac": round(par["tflops"] / PEAK_BF16_TFLOPS, 4)}
    if args.only is None and not args.no_cpu_baseline:
        cb = cpu_baseline()
        print(f"cpu baseline: {cb['value'] * 1e3:.2f} GFLOP/s ({cb['seconds']:.1f} s)", file=sys.stderr, flush=True)
        cb.pop("seconds")
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
