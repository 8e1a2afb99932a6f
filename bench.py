"""Benchmark of libbitlinear (BitLinear W1.58A8) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--part ...]

A step is one decode pass over the four 2B-class BitLinear shapes (M = 1
token, bf16 activations -> per-token int8 -> ternary GEMV -> fp32):
K2560->N2560, K2560->N640, K2560->N6912, K6912->N2560.  Weights are rotated
over enough distinct packed copies (> 2 x the 256 MB Infinity Cache) that
every step reads its weights from HBM.  ``value`` is the GEMV algorithmic
bytes moved per step (packed weights + int8 activations + fp32 outputs +
scales) over the measured step time, in GB/s.

Also measured in the same run and reported beside it: the prefill GEMM
(M = 2048, K2560->N6912, int8 TOPS against the int8 MFMA peak), the prefill
FFN tail (gate/up, ReLU² + subln + requant, down) and the CPU oracle on a
bounded sample of the decode step.

Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BitLinear M=1 GEMV GB/s (% HBM peak); M=2048 GEMM int8 TOPS (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
I8_MFMA_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA
COLD_BYTES = 600 * 2 ** 20     # > 2 x 256 MB Infinity Cache


def gemv_bytes(M, K, N):
    """Algorithmic bytes of one BitLinear: packed W + int8 X + fp32 Y + d + gamma."""
    return N * K // 4 + M * K + 4 * M * N + 4 * M + 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--part", default="all", choices=["all", "decode", "gemm", "ffn"],
                    help="restrict the GPU legs (for profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def decode_setup(bl, torch, workloads):
    shapes = workloads.DECODE_SHAPES
    per_step = sum(s.N * s.K // 4 for s in shapes)
    reps = max(2, math.ceil(COLD_BYTES / per_step))
    sets = []
    for i, s in enumerate(shapes):
        W, X = workloads.bitlinear_problem(i, 1, s.K, s.N)
        Wp, g = bl.quant_weight_absmean_pack(W.cuda())
        copies = [Wp] + [Wp.clone() for _ in range(reps - 1)]
        sets.append(dict(shape=s, Wp=copies, g=g, X=X.cuda(),
                         Xq=torch.empty((1, s.K), dtype=torch.int8, device="cuda"),
                         d=torch.empty((1,), dtype=torch.float32, device="cuda"),
                         Y=torch.empty((1, s.N), dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()
    return sets, reps


def decode_step(bl, sets, r):
    for p in sets:
        bl.quant_act_absmax_i8(p["X"], Xq=p["Xq"], d=p["d"])
        bl.bitlinear_gemv(p["Xq"], p["d"], p["Wp"][r], p["g"], Y=p["Y"])


def bench_decode(bl, torch, workloads, steps, warmup):
    """Step time from HIP-graph replays (one graph per weight copy, so the
    host issues one launch per step), then the GEMV kernel's own duration
    from event pairs around eager launches queued behind a sleep kernel (the
    queue is full when they run, so no host gap enters the pairs)."""
    sets, reps = decode_setup(bl, torch, workloads)
    for i in range(2 * reps):
        decode_step(bl, sets, i % reps)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(side):
        for r in range(reps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                decode_step(bl, sets, r)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % reps].replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        graphs[(warmup + i) % reps].replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)

    # kernel durations: 3 queue packets per GEMV, kept well under the queue depth
    per_pass = 48
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in sets]
           for _ in range(per_pass)]
    torch.cuda._sleep(200_000_000)
    for i in range(per_pass):
        for j, p in enumerate(sets):
            evs[i][j][0].record()
            bl.bitlinear_gemv(p["Xq"], p["d"], p["Wp"][i % reps], p["g"], Y=p["Y"])
            evs[i][j][1].record()
    torch.cuda.synchronize()
    per_shape_us = [1000.0 * sum(evs[i][j][0].elapsed_time(evs[i][j][1])
                                 for i in range(per_pass)) / per_pass
                    for j in range(len(sets))]
    step_bytes = sum(gemv_bytes(1, p["shape"].K, p["shape"].N) for p in sets)
    shapes = []
    for p, us in zip(sets, per_shape_us):
        b = gemv_bytes(1, p["shape"].K, p["shape"].N)
        shapes.append(dict(shape=p["shape"].name, K=p["shape"].K, N=p["shape"].N,
                           bytes=b, us=round(us, 3), GBs=round(b / us / 1e3, 1)))
    kernel_us = sum(per_shape_us) / len(per_shape_us)
    achieved = (step_bytes / len(sets)) / kernel_us / 1e3
    return dict(ms_total=ms, ms_per_step=ms / steps, step_bytes=step_bytes,
                value=step_bytes * steps / (ms * 1e-3) / 1e9, reps=reps,
                kernel_us=kernel_us, achieved=achieved, shapes=shapes)


def bench_gemm(bl, torch, workloads, steps, warmup):
    p = workloads.PREFILL
    M, K, N = p["M"], p["K"], p["F"]
    W, X = workloads.bitlinear_problem(p["seed"], M, K, N)
    Wp, g = bl.quant_weight_absmean_pack(W.cuda())
    Xq, d = bl.quant_act_absmax_i8(X.cuda())
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        bl.bitlinear_gemm(Xq, d, Wp, g, Y=Y)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:
        e[0].record()
        bl.bitlinear_gemm(Xq, d, Wp, g, Y=Y)
        e[1].record()
    torch.cuda.synchronize()
    us = 1000.0 * sum(a.elapsed_time(b) for a, b in evs) / steps
    ops = 2.0 * M * N * K
    tops = ops / us / 1e6
    return dict(M=M, K=K, N=N, us=round(us, 2), TOPS=round(tops, 1),
                frac=round(tops / I8_MFMA_PEAK_TOPS, 4))


def bench_ffn(bl, torch, workloads, steps, warmup):
    p = workloads.PREFILL
    M, K, F, N = p["M"], p["K"], p["F"], p["N"]
    Wg, Wu, Wd, X = workloads.ffn_problem(p["seed"], M, K, F, N)
    (Wgp, gg), (Wup, gu), (Wdp, gd) = [bl.quant_weight_absmean_pack(w.cuda()) for w in (Wg, Wu, Wd)]
    Xq, d = bl.quant_act_absmax_i8(X.cuda())
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty((bl.workspace_bytes(bl.BL_OP_FFN_RELU2, M, N, K, F),), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warmup):
        bl.bitlinear_ffn_relu2(Xq, d, Wgp, gg, Wup, gu, Wdp, gd, Y=Y, ws=ws)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        bl.bitlinear_ffn_relu2(Xq, d, Wgp, gg, Wup, gu, Wdp, gd, Y=Y, ws=ws)
    t1.record()
    torch.cuda.synchronize()
    us = 1000.0 * t0.elapsed_time(t1) / steps
    ops = 2.0 * M * K * F * 2 + 2.0 * M * F * N
    return dict(M=M, K=K, F=F, N=N, us=round(us, 2), TOPS=round(ops / us / 1e6, 1))


def cpu_baseline(torch, workloads, seconds):
    """The oracle, as it stands, on the decode step's four shapes, repeated
    for about `seconds` of wall time."""
    import numpy as np
    import oracle
    probs = []
    for i, s in enumerate(workloads.DECODE_SHAPES):
        W, X = workloads.bitlinear_problem(i, 1, s.K, s.N)
        Wp, g = oracle.quantize_weight(W.numpy())
        probs.append((s, Wp, g, workloads.bf16_bits(X)))
    step_bytes = sum(gemv_bytes(1, s.K, s.N) for s, _, _, _ in probs)
    passes = 0
    t0 = time.perf_counter()
    while True:
        for s, Wp, g, xb in probs:
            Xq, d = oracle.quant_act(oracle.bf16_to_f32(xb))
            oracle.bitlinear(Xq, d, Wp, g, s.K)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(step_bytes * passes / el / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{passes} decode steps (4 shapes, M=1, act quant + add/sub/skip "
                      f"accumulate + fp64 rescale) in {el:.1f} s, one process"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import ternary_weight_linear_absmean_amd as bl
    import workloads
    bl.load()
    torch.cuda.set_device(0)

    out = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
           "config": {"workload": "decode GEMV M=1 bf16 activations, 2B-class BitLinear shapes "
                                  "K2560->N2560, K2560->N640, K2560->N6912, K6912->N2560; "
                                  "weights N(0,0.02) absmean-ternary 2-bit packed, rotated "
                                  "cold past the 256 MB Infinity Cache",
                      "M": 1, "shapes": [[s.K, s.N] for s in workloads.DECODE_SHAPES]}}
    if args.part in ("all", "decode"):
        dec = bench_decode(bl, torch, workloads, args.steps, args.warmup)
        out["value"] = round(dec["value"], 2)
        out["ms_per_step"] = round(dec["ms_per_step"], 5)
        out["roofline"] = {"bound": "hbm", "achieved": round(dec["achieved"], 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(dec["achieved"] / HBM_PEAK_GBS, 4), "traffic": None,
                           "kernel": "gemv_kernel (bitlinear_gemv, M=1)",
                           "avg_launch_us": round(dec["kernel_us"], 3)}
        out["decode_shapes"] = dec["shapes"]
        out["config"]["weight_copies"] = dec["reps"]
        out["config"]["step_bytes"] = dec["step_bytes"]
    if args.part in ("all", "gemm"):
        out["gemm"] = bench_gemm(bl, torch, workloads, max(10, args.steps // 8), 5)
    if args.part in ("all", "ffn"):
        out["ffn"] = bench_ffn(bl, torch, workloads, max(5, args.steps // 40), 2)
    if not args.no_cpu and args.part == "all":
        out["cpu_baseline"] = cpu_baseline(torch, workloads, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
