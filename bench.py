"""Benchmark of libbitlinear (BitLinear W1.58A8) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--part ...]

A step is one decode pass over the four 2B-class BitLinear shapes (M = 1
token, bf16 activations -> per-token int8 -> ternary GEMV -> fp32):
K2560->N2560, K2560->N640, K2560->N6912, K6912->N2560, as one fused launch
(bitlinear_gemv_fused) replayed from a HIP graph.  Weights are rotated over
enough distinct packed copies (> 2 x the 256 MB Infinity Cache) that every
step reads its weights from HBM.  ``value`` is the algorithmic bytes moved
per step (packed weights + bf16 activations + fp32 outputs + gamma: 10,975,248
B for the four shapes) over the
measured step time, in GB/s.  The same step as separate quant + GEMV calls
is reported as ``decode_unfused``.

Also measured in the same run and reported beside it: batched decode
(bitlinear_gemv on M = 8 / 32 / 64 tokens, K2560->N6912 and K6912->N2560,
cold weights, per launch), the prefill GEMM
(M = 2048, K2560->N6912, int8 TOPS against the int8 MFMA peak), the prefill
FFN tail (gate/up, ReLU² + subln + requant, down), one decode token through
the full 30-layer linear stack (bitlinear_decode_stack: 521 MB of packed
weights per token, tokens/s and GB/s), the QAT backward (dX and dW at
M = 2048 for the FFN shapes, the absmean quantiser, a whole training step),
the decode step's products on five-weights-per-byte rows against the 2-bit
rows (``t5_storage``: four launches each, pre-quantised tokens, cold weights),
measured ceilings (a device copy; hipBLASLt's int8 GEMM at the prefill
shape) with the decode and GEMM figures as fractions of them, and the CPU
oracle on bounded samples (all threads, then one) of the decode step, the
prefill GEMM (32 of its 2048 token rows), batched decode (M = 32,
K2560->N6912) and the prefill FFN block (8 of its 2048 token rows).

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
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
COLD_BYTES = 600 * 2 ** 20     # > 2 x 256 MB Infinity Cache


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_fused_decode_m1.md")
GEMV_SOURCE = os.path.join(ROOT, "ternary_weight_linear_absmean_amd", "csrc", "gemv.hip")


def measured_traffic():
    """HBM bytes per launch of the fused decode kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (calibrated on a plain copy),
    or None when that summary was taken on a different gemv.hip."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
        src = hashlib.sha256(open(GEMV_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line)
    key = "source_sha256(ternary_weight_linear_absmean_amd/csrc/gemv.hip)"
    if fields.get(key, "").strip() != src:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def decode_bytes(K, N):
    """Algorithmic bytes of one M = 1 BitLinear from bf16 activations: packed
    2-bit W + bf16 X + fp32 Y + gamma."""
    return N * K // 4 + 2 * K + 4 * N + 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--part", default="all",
                    choices=["all", "decode", "batched", "gemm", "ffn", "stack", "qat", "t5",
                             "a4", "copy"],
                    help="restrict the GPU legs (for profiling runs); 'copy' (not in 'all') "
                         "times a plain device copy of 256 MiB, the reference for the "
                         "byte counters")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def decode_setup(bl, torch, workloads):
    shapes = workloads.DECODE_SHAPES
    per_step = sum(s.N * s.K // 4 for s in shapes)
    reps = max(2, math.ceil(COLD_BYTES / per_step))
    reps = STEPS_PER_GRAPH * math.ceil(reps / STEPS_PER_GRAPH)
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


def fused_step(bl, sets, r):
    """One decode step: a single launch, act quant fused into the four GEMVs."""
    bl.bitlinear_gemv_fused([dict(X=p["X"], Wp=p["Wp"][r], gamma=p["g"], Y=p["Y"])
                             for p in sets])


def unfused_step(bl, sets, r):
    """The same step as two calls per shape (quant_act_absmax_i8 + bitlinear_gemv)."""
    for p in sets:
        bl.quant_act_absmax_i8(p["X"], Xq=p["Xq"], d=p["d"])
        bl.bitlinear_gemv(p["Xq"], p["d"], p["Wp"][r], p["g"], Y=p["Y"])


STEPS_PER_GRAPH = 10


def capture(torch, fn, reps, per_graph):
    """HIP graphs over the weight copies: graph i holds `per_graph` consecutive
    steps (copies i*per_graph ...), plus one single-step graph per copy for
    step counts that are not a multiple.  A graph only changes how the host
    launches the steps, not the work each step does."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    multi, single = [], []
    with torch.cuda.stream(side):
        for start in range(0, reps, per_graph):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for r in range(start, start + per_graph):
                    fn(r)
            multi.append(g)
        for r in range(reps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                fn(r)
            single.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return multi, single


def replay_ms(torch, graphs, steps, warmup, per_graph):
    """Replay exactly `steps` steps after `warmup` warm-up steps; returns ms."""
    multi, single = graphs

    def run(n, first):
        done = 0
        i = first
        while n - done >= per_graph:
            multi[i % len(multi)].replay()
            done += per_graph
            i += 1
        while done < n:
            single[(i * per_graph + done) % len(single)].replay()
            done += 1
        return i

    nxt = run(warmup, 0)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    run(steps, nxt)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def bench_decode(bl, torch, workloads, steps, warmup):
    """The decode step replayed from HIP graphs over cold weight copies.  With
    the fused call a step is exactly one kernel, so the event-timed region
    over K steps gives that kernel's average launch duration (with the
    dispatch gap between back-to-back kernels) directly."""
    sets, reps = decode_setup(bl, torch, workloads)
    for r in range(reps):
        fused_step(bl, sets, r)
        unfused_step(bl, sets, r)
    torch.cuda.synchronize()
    g_fused = capture(torch, lambda r: fused_step(bl, sets, r), reps, STEPS_PER_GRAPH)
    ms = replay_ms(torch, g_fused, steps, warmup, STEPS_PER_GRAPH)
    g_unfused = capture(torch, lambda r: unfused_step(bl, sets, r), reps, STEPS_PER_GRAPH)
    ms_unfused = replay_ms(torch, g_unfused, steps, warmup, STEPS_PER_GRAPH)
    # bf16 activations are read by the fused kernel (quantisation is fused)
    step_bytes = sum(decode_bytes(p["shape"].K, p["shape"].N) for p in sets)
    us = 1000.0 * ms / steps
    return dict(ms_per_step=ms / steps, step_bytes=step_bytes,
                value=step_bytes / us / 1e3, reps=reps, kernel_us=us,
                achieved=step_bytes / us / 1e3,
                unfused=dict(us_per_step=round(1000.0 * ms_unfused / steps, 3),
                             GBs=round(step_bytes * steps / (ms_unfused * 1e-3) / 1e9, 1),
                             launches_per_step=2 * len(sets)))


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
    # back-to-back launches between two events: the average launch period,
    # dispatch gaps included, with no timing work between the kernels
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        bl.bitlinear_gemm(Xq, d, Wp, g, Y=Y)
    t1.record()
    torch.cuda.synchronize()
    us = 1000.0 * t0.elapsed_time(t1) / steps
    ops = 2.0 * M * N * K
    tops = ops / us / 1e6
    out = dict(M=M, K=K, N=N, us=round(us, 2), TOPS=round(tops, 1),
               frac=round(tops / I8_MFMA_PEAK_TOPS, 4))
    # the prefill down-projection shape, K6912 -> N2560
    K2, N2 = p["F"], p["N"]
    W2, X2 = workloads.bitlinear_problem(p["seed"] + 1, M, K2, N2)
    Wp2, g2 = bl.quant_weight_absmean_pack(W2.cuda())
    Xq2, d2 = bl.quant_act_absmax_i8(X2.cuda())
    Y2 = torch.empty((M, N2), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        bl.bitlinear_gemm(Xq2, d2, Wp2, g2, Y=Y2)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        bl.bitlinear_gemm(Xq2, d2, Wp2, g2, Y=Y2)
    t1.record()
    torch.cuda.synchronize()
    us2 = 1000.0 * t0.elapsed_time(t1) / steps
    t2 = 2.0 * M * N2 * K2 / us2 / 1e6
    out["down_shape"] = dict(M=M, K=K2, N=N2, us=round(us2, 2), TOPS=round(t2, 1),
                             frac=round(t2 / I8_MFMA_PEAK_TOPS, 4))
    return out


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


def bench_qat(bl, torch, workloads, steps, warmup):
    """QAT at M = 2048 tokens for the FFN shapes: dX and dW, each timed over
    back-to-back calls (operand preparation + product) between two events,
    the absmean weight quantiser, and a whole training step of the layer
    (fresh absmean weights, activation quant, forward, dX, dW).  TFLOPs and
    frac_bf16 count the 2 M N K algorithmic flops of each gradient; the bf16
    MFMA issues twice that (the hi and lo halves of the fp32 gradient), which
    issued_frac_bf16 reports."""
    out = []
    for sh in workloads.QAT_SHAPES:
        M, K, N = workloads.QAT_M, sh.K, sh.N
        W, X, dY = workloads.qat_problem(600 + K, M, K, N)
        Wp, g = bl.quant_weight_absmean_pack(W.cuda())
        Xq, d = bl.quant_act_absmax_i8(X.cuda())
        dY = dY.cuda()
        dX = torch.empty((M, K), dtype=torch.float32, device="cuda")
        dW = torch.empty((N, K), dtype=torch.float32, device="cuda")
        wsi = torch.empty((bl.workspace_bytes(bl.BL_OP_BACKWARD_INPUT, M, N, K),),
                          dtype=torch.uint8, device="cuda")
        wsw = torch.empty((bl.workspace_bytes(bl.BL_OP_BACKWARD_WEIGHT, M, N, K),),
                          dtype=torch.uint8, device="cuda")
        Wd = W.cuda()
        Xd = X.cuda()
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        wsq = torch.empty((max(16, bl.workspace_bytes(bl.BL_OP_QUANT_WEIGHT, 0, N, K)),),
                          dtype=torch.uint8, device="cuda")

        def step():
            # one training step of the layer: fresh absmean weights, per-token
            # activations, forward, both straight-through gradients
            bl.quant_weight_absmean_pack(Wd, Wp=Wp, gamma=g, ws=wsq)
            bl.quant_act_absmax_i8(Xd, Xq=Xq, d=d)
            bl.bitlinear_gemm(Xq, d, Wp, g, Y=Y)
            bl.bitlinear_backward_input(dY, Wp, g, dX=dX, ws=wsi)
            bl.bitlinear_backward_weight(dY, Xq, d, dW=dW, ws=wsw)

        row = dict(M=M, K=K, N=N)
        for name, fn in (("dX", lambda: bl.bitlinear_backward_input(dY, Wp, g, dX=dX, ws=wsi)),
                         ("dW", lambda: bl.bitlinear_backward_weight(dY, Xq, d, dW=dW, ws=wsw)),
                         ("weight_quant", lambda: bl.quant_weight_absmean_pack(Wd, Wp=Wp, gamma=g,
                                                                               ws=wsq)),
                         ("step", step)):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(steps):
                fn()
            t1.record()
            torch.cuda.synchronize()
            us = 1000.0 * t0.elapsed_time(t1) / steps
            if name in ("dX", "dW"):
                tf = 2.0 * M * N * K / us / 1e6
                # frac: the algorithmic 2 M N K flops over the bf16 peak;
                # issued_frac: the MFMA work issued (hi and lo halves: twice that)
                row[name] = dict(us=round(us, 2), TFLOPs=round(tf, 1),
                                 frac_bf16=round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                 issued_frac_bf16=round(2.0 * tf / BF16_MFMA_PEAK_TFLOPS, 4))
            elif name == "weight_quant":
                # fp32 W read twice (sum, then ternarise) + packed codes written
                byts = 2 * 4 * N * K + N * K // 4
                row[name] = dict(us=round(us, 2), GBs=round(byts / us / 1e3, 1))
            else:
                row[name] = dict(us=round(us, 2))
        out.append(row)
    return out


STACK_SEED = 4242


def stack_bytes(H, KV, F, layers):
    """Algorithmic HBM bytes of one token through the stack: the packed
    weights (the dominant term) plus the 7 gammas and the subln gain of each
    layer; activations stay in L2-sized fp32 vectors and are not counted."""
    per_layer = (2 * H * H + 2 * KV * H + 3 * F * H) // 4 + 7 * 4 + 4 * F
    return layers * per_layer


def bench_stack(bl, torch, workloads, steps, warmup):
    """One decode token through the 30-layer 2B-class linear stack
    (bitlinear_decode_stack), replayed from a HIP graph.  Each replay first
    resets the residual stream to the same input token (a 10 KB copy standing
    in for the embedding lookup), so every token does identical work; the
    521 MB of packed weights exceed the Infinity Cache, so every token streams
    them from HBM."""
    H, KV, F, D, L = workloads.HIDDEN, workloads.KV, workloads.FFN, workloads.HEAD_DIM, \
        workloads.LAYERS
    layers = []
    for l in range(L):
        W = workloads.stack_layer_weights(STACK_SEED, l, H, KV, F, device="cuda")
        Ld = {}
        for name, gname in zip(bl.LAYER_WEIGHTS, bl.LAYER_GAMMAS):
            Ld[name], Ld[gname] = bl.quant_weight_absmean_pack(W[name])
        Ld["ffn_norm"] = torch.ones(F, dtype=torch.float32, device="cuda")
        layers.append(Ld)
        del W
    torch.cuda.synchronize()
    x0 = workloads.stack_token(STACK_SEED, H).cuda()
    x = x0.clone()
    ws = torch.empty((bl.workspace_bytes(bl.BL_OP_DECODE_STACK, 1, H, KV, F),),
                     dtype=torch.uint8, device="cuda")

    def timed(path, n):
        def token(stream):
            x.copy_(x0)
            bl.bitlinear_decode_stack(layers, x, H, KV, F, D, ws=ws, stream=stream, path=path)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            token(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                token(side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(x).all())
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(n):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return 1000.0 * t0.elapsed_time(t1) / n

    nbytes = stack_bytes(H, KV, F, L)
    us = timed(bl.BL_STACK_PERSISTENT, steps)
    us_l = timed(bl.BL_STACK_LAUNCHES, max(10, steps // 4))
    return dict(layers=L, H=H, KV=KV, F=F, head_dim=D, tokens=steps,
                path="persistent", launches_per_token=2 + (L - 1) // 16,
                us_per_token=round(us, 2), tokens_per_s=round(1e6 / us, 1),
                bytes_per_token=nbytes, GBs=round(nbytes / us / 1e3, 1),
                frac=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                launches_path=dict(us_per_token=round(us_l, 2),
                                   GBs=round(nbytes / us_l / 1e3, 1),
                                   launches_per_token=2 + 8 * L))


def bench_batched(bl, torch, workloads):
    """Batched decode: bitlinear_gemv on M in {8, 32, 64} pre-quantised
    tokens against K2560->N6912 and K6912->N2560, weights rotated over
    copies past the Infinity Cache, launches replayed from HIP graphs; the
    time per launch includes the dispatch gap."""
    shapes = workloads.BATCHED_SHAPES
    reps = STEPS_PER_GRAPH * math.ceil(max(2, math.ceil(COLD_BYTES / min(
        s.N * s.K // 4 for s in shapes))) / STEPS_PER_GRAPH)
    rows = []
    for i, s in enumerate(shapes):
        W, _ = workloads.bitlinear_problem(70 + i, 1, s.K, s.N)
        Wp, g = bl.quant_weight_absmean_pack(W.cuda())
        copies = [Wp] + [Wp.clone() for _ in range(reps - 1)]
        for M in workloads.BATCHED_M:
            _, X = workloads.bitlinear_problem(80 + M, M, s.K, 1)
            Xq, d = bl.quant_act_absmax_i8(X.cuda())
            Y = torch.empty((M, s.N), dtype=torch.float32, device="cuda")

            def step(r):
                bl.bitlinear_gemv(Xq, d, copies[r], g, Y=Y)
            for r in range(reps):
                step(r)
            torch.cuda.synchronize()
            graphs = capture(torch, step, reps, STEPS_PER_GRAPH)
            ms = replay_ms(torch, graphs, 2 * reps, STEPS_PER_GRAPH, STEPS_PER_GRAPH)
            us = 1000.0 * ms / (2 * reps)
            nbytes = s.N * s.K // 4 + M * s.K + 4 * M * s.N + 4 * M + 4
            rows.append(dict(M=M, K=s.K, N=s.N, us=round(us, 2), GBs=round(nbytes / us / 1e3, 1)))
        del copies
    return rows


def bench_t5(bl, torch, workloads, steps, warmup):
    """Five weights per byte against two bits per weight: the decode step's
    four products at M = 1 from pre-quantised tokens, as four
    bitlinear_gemv_t5 launches and as four bitlinear_gemv launches (both on
    v_dot4), weights rotated over copies past the Infinity Cache, replayed
    from HIP graphs.  GB/s counts each format's own bytes (weights, int8
    codes, fp32 outputs, scales)."""
    shapes = workloads.DECODE_SHAPES
    base = []
    for i, s in enumerate(shapes):
        W, X = workloads.bitlinear_problem(i, 1, s.K, s.N)
        Wp, g = bl.quant_weight_absmean_pack(W.cuda())
        Xq, d = bl.quant_act_absmax_i8(X.cuda())
        base.append(dict(shape=s, Wp=Wp, Wt5=bl.bitlinear_repack_t5(Wp), g=g, Xq=Xq, d=d,
                         Y=torch.empty((1, s.N), dtype=torch.float32, device="cuda")))
    out = {}
    for name, key, call in (("2bit", "Wp", bl.bitlinear_gemv), ("t5", "Wt5", bl.bitlinear_gemv_t5)):
        per_step = sum(p[key].numel() for p in base)
        reps = STEPS_PER_GRAPH * math.ceil(max(2, math.ceil(COLD_BYTES / per_step)) / STEPS_PER_GRAPH)
        copies = [[p[key]] + [p[key].clone() for _ in range(reps - 1)] for p in base]

        def step(r):
            for p, c in zip(base, copies):
                call(p["Xq"], p["d"], c[r], p["g"], Y=p["Y"])
        for r in range(reps):
            step(r)
        torch.cuda.synchronize()
        graphs = capture(torch, step, reps, STEPS_PER_GRAPH)
        ms = replay_ms(torch, graphs, steps, warmup, STEPS_PER_GRAPH)
        us = 1000.0 * ms / steps
        nbytes = per_step + sum(p["shape"].K + 4 * p["shape"].N + 8 for p in base)
        out[name] = dict(us_per_step=round(us, 3), weight_bytes=per_step, step_bytes=nbytes,
                         GBs=round(nbytes / us / 1e3, 1), launches_per_step=len(base))
        del copies, graphs
    Y2 = [p["Y"].clone() for p in base]
    for p in base:
        bl.bitlinear_gemv_t5(p["Xq"], p["d"], p["Wt5"], p["g"], Y=p["Y"])
    torch.cuda.synchronize()
    out["identical_outputs"] = all(torch.equal(a.view(torch.int32), p["Y"].view(torch.int32))
                                   for a, p in zip(Y2, base))
    out["time_ratio_t5_over_2bit"] = round(out["t5"]["us_per_step"] / out["2bit"]["us_per_step"], 3)
    return out


def bench_a4(bl, torch, workloads, steps, warmup):
    """4-bit activations (BitNet a4.8) against 8-bit: the decode step's four
    products at M = 1 from pre-quantised tokens, as four bitlinear_a4 and as
    four bitlinear_gemv launches, weights rotated over copies past the
    Infinity Cache, replayed from HIP graphs; and the prefill product at
    M = 2048, K2560 -> N6912, bitlinear_a4 against bitlinear_gemm.  GB/s and
    TOPS count each format's own bytes and 2 M N K."""
    shapes = workloads.DECODE_SHAPES
    base = []
    for i, s in enumerate(shapes):
        W, X = workloads.bitlinear_problem(i, 1, s.K, s.N)
        Wp, g = bl.quant_weight_absmean_pack(W.cuda())
        Xq, d = bl.quant_act_absmax_i8(X.cuda())
        P, d4 = bl.quant_act_absmax_i4(X.cuda())
        base.append(dict(shape=s, Wp=Wp, g=g, Xq=Xq, d=d, P=P, d4=d4,
                         Y=torch.empty((1, s.N), dtype=torch.float32, device="cuda")))
    per_step = sum(p["Wp"].numel() for p in base)
    reps = STEPS_PER_GRAPH * math.ceil(max(2, math.ceil(COLD_BYTES / per_step)) / STEPS_PER_GRAPH)
    copies = [[p["Wp"]] + [p["Wp"].clone() for _ in range(reps - 1)] for p in base]
    out = {}
    for name, xk, dk, call, abytes in (("a8", "Xq", "d", bl.bitlinear_gemv, 1.0),
                                       ("a4", "P", "d4", bl.bitlinear_a4, 0.5)):
        def step(r):
            for p, c in zip(base, copies):
                call(p[xk], p[dk], c[r], p["g"], Y=p["Y"])
        for r in range(reps):
            step(r)
        torch.cuda.synchronize()
        graphs = capture(torch, step, reps, STEPS_PER_GRAPH)
        ms = replay_ms(torch, graphs, steps, warmup, STEPS_PER_GRAPH)
        us = 1000.0 * ms / steps
        nbytes = per_step + sum(int(abytes * p["shape"].K) + 4 * p["shape"].N + 8 for p in base)
        out[name] = dict(us_per_step=round(us, 3), step_bytes=nbytes, GBs=round(nbytes / us / 1e3, 1),
                         launches_per_step=len(base))
        del graphs
    del copies
    p = workloads.PREFILL
    M, K, N = p["M"], p["K"], p["F"]
    W, X = workloads.bitlinear_problem(p["seed"], M, K, N)
    Wp, g = bl.quant_weight_absmean_pack(W.cuda())
    Xq, d = bl.quant_act_absmax_i8(X.cuda())
    P4, d4 = bl.quant_act_absmax_i4(X.cuda())
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    pre = {}
    for name, fn in (("a8", lambda: bl.bitlinear_gemm(Xq, d, Wp, g, Y=Y)),
                     ("a4", lambda: bl.bitlinear_a4(P4, d4, Wp, g, Y=Y))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        n = max(10, steps // 8)
        t0.record()
        for _ in range(n):
            fn()
        t1.record()
        torch.cuda.synchronize()
        us = 1000.0 * t0.elapsed_time(t1) / n
        tops = 2.0 * M * N * K / us / 1e6
        pre[name] = dict(us=round(us, 2), TOPS=round(tops, 1), frac=round(tops / I8_MFMA_PEAK_TOPS, 4))
    out["prefill_M2048_K2560_N6912"] = pre
    return out


def bench_copy(torch, steps):
    """A plain device-to-device copy of 256 MiB: the kernel whose HBM byte
    counters (FETCH_SIZE, WRITE_SIZE) calibrate the ones read for the GEMV."""
    n = 256 * 2 ** 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    us = 1000.0 * t0.elapsed_time(t1) / steps
    return dict(bytes_read=n, bytes_written=n, us=round(us, 2), GBs=round(2 * n / us / 1e3, 1))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(torch, workloads, seconds):
    """The oracle, as it stands, on the decode step's four shapes, repeated
    for about `seconds` of wall time: the first half on all the threads its
    OpenMP loops take, the second half on one thread."""
    import oracle
    probs = []
    for i, s in enumerate(workloads.DECODE_SHAPES):
        W, X = workloads.bitlinear_problem(i, 1, s.K, s.N)
        Wp, g = oracle.quantize_weight(W.numpy())
        probs.append((s, Wp, g, workloads.bf16_bits(X)))
    step_bytes = sum(decode_bytes(s.K, s.N) for s, _, _, _ in probs)

    def timed(limit):
        passes = 0
        t0 = time.perf_counter()
        while True:
            for s, Wp, g, xb in probs:
                Xq, d = oracle.quant_act(oracle.bf16_to_f32(xb))
                oracle.bitlinear(Xq, d, Wp, g, s.K)
            passes += 1
            el = time.perf_counter() - t0
            if el >= limit:
                return passes, el

    # a bounded sample of the prefill GEMM: 32 of its 2048 token rows
    p = workloads.PREFILL
    Mg, Kg, Ng = 32, p["K"], p["F"]
    Wg, Xg = workloads.bitlinear_problem(p["seed"], Mg, Kg, Ng)
    Wpg, gg = oracle.quantize_weight(Wg.numpy())
    Xqg, dg = oracle.quant_act(oracle.bf16_to_f32(workloads.bf16_bits(Xg)))
    gemm_ops = 2.0 * Mg * Kg * Ng

    # batched decode: 32 tokens against K2560 -> N6912
    sb = workloads.BATCHED_SHAPES[0]
    Wb, Xb = workloads.bitlinear_problem(70, 32, sb.K, sb.N)
    Wpb, gb = oracle.quantize_weight(Wb.numpy())
    Xqb, db = oracle.quant_act(oracle.bf16_to_f32(workloads.bf16_bits(Xb)))
    batched_ops = 2.0 * 32 * sb.K * sb.N
    # the prefill FFN block on 8 of its 2048 token rows (gate, up, tail, down)
    F, Nd = p["F"], p["N"]
    gf = workloads.generator(p["seed"] + 1)
    Wgf, Wuf, Wdf = (workloads.weight(gf, F, Kg), workloads.weight(gf, F, Kg),
                     workloads.weight(gf, Nd, F))
    Xf = workloads.activations(gf, 8, Kg)
    (Wpgf, ggf), (Wpuf, guf), (Wpdf, gdf) = (oracle.quantize_weight(w.numpy())
                                            for w in (Wgf, Wuf, Wdf))
    Xqf, df = oracle.quant_act(oracle.bf16_to_f32(workloads.bf16_bits(Xf)))
    ffn_ops = 2.0 * 8 * (2 * Kg * F + F * Nd)

    def timed_call(fn, limit):
        reps = 0
        t0 = time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= limit:
                return reps, el

    def timed_gemm(limit):
        return timed_call(lambda: oracle.bitlinear(Xqg, dg, Wpg, gg, Kg), limit)

    def batched():
        oracle.bitlinear(Xqb, db, Wpb, gb, sb.K)

    def ffn():
        oracle.ffn_relu2(Xqf, df, Wpgf, ggf, Wpuf, guf, None, 1e-5, Wpdf, gdf, Kg, F, Nd)

    cores = oracle.num_threads()
    passes, el = timed(seconds / 2)
    greps, gel = timed_gemm(0.5)
    breps, bel = timed_call(batched, 0.5)
    freps, fel = timed_call(ffn, 0.5)
    oracle.set_num_threads(1)
    passes1, el1 = timed(seconds / 2)
    greps1, gel1 = timed_gemm(1.0)
    breps1, bel1 = timed_call(batched, 1.0)
    freps1, fel1 = timed_call(ffn, 1.0)
    oracle.set_num_threads(cores)
    batched_row = {"TOPS": round(batched_ops * breps / bel / 1e12, 5),
                   "TOPS_1_thread": round(batched_ops * breps1 / bel1 / 1e12, 5),
                   "sample": f"M=32 K{sb.K}->N{sb.N} ({batched_ops / 1e9:.2f} G int ops per pass): "
                             f"{breps} passes in {bel:.1f} s on {cores} threads, {breps1} in "
                             f"{bel1:.1f} s on 1 thread"}
    ffn_row = {"TOPS": round(ffn_ops * freps / fel / 1e12, 5),
               "TOPS_1_thread": round(ffn_ops * freps1 / fel1 / 1e12, 5),
               "sample": f"8 of the {p['M']} token rows of the prefill FFN block "
                         f"({ffn_ops / 1e9:.2f} G int ops per pass): {freps} passes in "
                         f"{fel:.1f} s on {cores} threads, {freps1} in {fel1:.1f} s on 1 thread"}
    prefill = {"TOPS": round(gemm_ops * greps / gel / 1e12, 5),
               "TOPS_1_thread": round(gemm_ops * greps1 / gel1 / 1e12, 5),
               "sample": f"{Mg} of the {p['M']} token rows of the M={p['M']} K{Kg}->N{Ng} "
                         f"prefill GEMM ({gemm_ops / 1e9:.2f} G int ops per pass): {greps} "
                         f"passes in {gel:.1f} s on {cores} threads, {greps1} in {gel1:.1f} s "
                         f"on 1 thread"}
    return {"value": round(step_bytes * passes / el / 1e9, 3), "unit": "GB/s",
            "prefill_gemm": prefill, "batched_decode": batched_row, "prefill_ffn": ffn_row,
            "cores": cores, "kind": "oracle",
            "value_1_thread": round(step_bytes * passes1 / el1 / 1e9, 3),
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"{passes} decode steps (4 shapes, M=1, act quant + add/sub/skip "
                      f"accumulate + fp64 rescale) in {el:.1f} s on {cores} threads, then "
                      f"{passes1} in {el1:.1f} s on 1 thread, one process"}


def bench_ceilings(torch, workloads):
    """Measured achievable peaks: a 256 MiB device copy (HBM read + write) and
    hipBLASLt's int8 GEMM (torch._int_mm, int32 out) at the prefill shape
    M = 2048, K2560 -> N6912, with B given in both layouts: K x N row-major,
    and the transpose of N x K row-major (the [N][K] layout of the packed
    weights).  The faster one is the ceiling."""
    copy = bench_copy(torch, 20)
    p = workloads.PREFILL
    M, K, N = p["M"], p["K"], p["F"]
    g = workloads.generator(0)
    A = torch.randint(-127, 128, (M, K), generator=g, dtype=torch.int8).cuda()
    B_kn = torch.randint(-1, 2, (K, N), generator=g, dtype=torch.int8).cuda()
    B_nk = torch.randint(-1, 2, (N, K), generator=g, dtype=torch.int8).cuda().t()
    out = dict(hbm_copy_GBs=copy["GBs"])
    try:
        times = {}
        for name, B in (("b_kxn_rowmajor", B_kn), ("b_nxk_rowmajor_transposed", B_nk)):
            for _ in range(3):
                torch._int_mm(A, B)
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(20):
                torch._int_mm(A, B)
            t1.record()
            torch.cuda.synchronize()
            times[name] = round(1000.0 * t0.elapsed_time(t1) / 20, 2)
        us = min(times.values())
        out["hipblaslt_int8_gemm_us_by_layout"] = times
        out["hipblaslt_int8_gemm_us"] = us
        out["hipblaslt_int8_gemm_TOPS"] = round(2.0 * M * N * K / us / 1e6, 1)
    except RuntimeError as e:                     # not every build ships the int8 GEMM
        out["hipblaslt_int8_gemm_error"] = str(e)[:120]
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on one GPU only; --gpus must be 1", file=sys.stderr)
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
                           "frac": round(dec["achieved"] / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic(),
                           "kernel": "gemv_fused_kernel<1, true> (bitlinear_gemv_fused, 4 jobs, M=1)",
                           "avg_launch_us": round(dec["kernel_us"], 3),
                           "bytes_per_launch": dec["step_bytes"]}
        out["decode_unfused"] = dec["unfused"]
        out["config"]["weight_copies"] = dec["reps"]
        out["config"]["step_bytes"] = dec["step_bytes"]
    if args.part in ("all", "batched"):
        out["batched_decode"] = bench_batched(bl, torch, workloads)
    if args.part in ("all", "gemm"):
        out["gemm"] = bench_gemm(bl, torch, workloads, max(10, args.steps // 8), 5)
    if args.part in ("all", "ffn"):
        out["ffn"] = bench_ffn(bl, torch, workloads, max(5, args.steps // 40), 2)
    if args.part in ("all", "qat"):
        out["qat_backward"] = bench_qat(bl, torch, workloads, max(5, args.steps // 40), 2)
    if args.part in ("all", "t5"):
        out["t5_storage"] = bench_t5(bl, torch, workloads, max(20, args.steps // 2), 10)
    if args.part in ("all", "a4"):
        out["a4_activations"] = bench_a4(bl, torch, workloads, max(20, args.steps // 2), 10)
    if args.part == "copy":
        out["copy"] = bench_copy(torch, 10)
    if args.part in ("all", "stack"):
        out["stack"] = bench_stack(bl, torch, workloads, max(20, args.steps // 4), 5)
    if args.part == "all":
        ceil = bench_ceilings(torch, workloads)
        out["ceilings"] = ceil
        if "roofline" in out and ceil.get("hbm_copy_GBs"):
            out["roofline"]["frac_of_measured_copy"] = round(
                out["roofline"]["achieved"] / ceil["hbm_copy_GBs"], 4)
        if "gemm" in out and ceil.get("hipblaslt_int8_gemm_TOPS"):
            out["gemm"]["frac_of_hipblaslt"] = round(
                out["gemm"]["TOPS"] / ceil["hipblaslt_int8_gemm_TOPS"], 4)
    if not args.no_cpu and args.part == "all":
        out["cpu_baseline"] = cpu_baseline(torch, workloads, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
