"""Host logic of bench.py that needs no GPU: the flop and byte counts the
roofline uses, and how the roofline picks its bound."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_chunkwise_counts_on_the_7b_workload():
    # causal intra-chunk products (Q K^T and P V over the lower triangle of
    # each 512 x 512 chunk, diagonal included), the cross term Q R and the
    # state update K^T V, each 2 flops per multiply-add, at d = 256
    b, n, h, d, c = 2, 8192, 16, 256, 512
    chunks = n // c
    intra = c * (c + 1) // 2 * d * 2 * 2
    per_chunk = intra + c * d * d * 2 + c * d * d * 2
    assert bench.chunkwise_flops(b, n, h, d, d, c) == b * h * chunks * per_chunk
    # q, k, v, g read, o written (bf16), fp32 state out
    assert bench.chunkwise_bytes(b, n, h, d, d) == 5 * b * n * h * d * 2 + b * h * d * d * 4


def _cw(flops, nbytes, us):
    return {"flops": flops, "bytes": nbytes, "kernel_ms": us * 1e-3,
            "kernel_tflops": flops / (us * 1e-6) / 1e12}


def test_roofline_bound_follows_the_ridge_point():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBPS * 1e9)
    below = _cw(flops=int(0.5 * ridge * 1e9), nbytes=10**9, us=500.0)
    r = bench.roofline_object(below, below["bytes"] / 500e-6 / 1e9, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["frac"] - r["achieved"] / bench.PEAK_HBM_GBPS) < 1e-3
    assert r["mfma"]["unit"] == "TFLOP/s" and r["traffic"] is None
    assert abs(r["attainable_tflops"] - 0.5 * bench.PEAK_BF16_TFLOPS) < 1.0
    above = _cw(flops=int(2 * ridge * 1e9), nbytes=10**9, us=500.0)
    r = bench.roofline_object(above, above["bytes"] / 500e-6 / 1e9, {"bytes": 123})
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["hbm"]["unit"] == "GB/s"
    assert r["traffic"] == 123 and r["attainable_tflops"] == bench.PEAK_BF16_TFLOPS


def test_packed_batch_leg_and_profile_names():
    # the ragged batch holds the same 16384 tokens as 2 x 8192
    assert sum(bench.VARLEN_LENS) == 16384 and max(bench.VARLEN_LENS) == 8192
    # its flops are the chunkwise count summed per sequence: less than the
    # two full sequences' (shorter chunks hold fewer causal pairs)
    per_seq = sum(bench.chunkwise_flops(1, n, 16, 256, 256, 512) for n in bench.VARLEN_LENS)
    assert 0 < per_seq < bench.chunkwise_flops(2, 8192, 16, 256, 256, 512)
    # every kernel-statistics leg runs a benchmark leg that --only accepts
    for leg, args in bench.STATS_ARGS.items():
        assert args[:2] == ["--only", leg]


def test_gpus_above_one_exits_with_a_message():
    import subprocess
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)
