"""GPU parity of bitlinear_decode_stack against the oracle's decode stack.

Teacher-forced (the primary check): the GPU runs the whole stack with its
per-layer trace; the oracle then runs each layer alone from the GPU's input
to that layer (oracle.decode_stack on one layer).  Every value that feeds a
later per-token quantisation is carried in fp32 on both sides, so q, k, v, o
and x_mid must be bit-identical in every layer; the FFN output y carries the
subln RMS, an fp64 sum whose order is each side's own, and must be within
1e-3 relative of the oracle's, element by element; the next layer's input
and the final x must be the fp32 sums x_mid + y of the GPU's own values.

Free-running (secondary): the oracle runs the whole stack on its own
activations; the first layer must be bit-identical, later layers within 1e-3
of each trace segment's largest magnitude (a y that differs in its last bit
can move a later int8 decision by one step).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

RTOL = 1e-3
NAMES = workloads.STACK_NAMES
GAMMAS = ("gq", "gk", "gv", "go", "gg", "gu", "gd")


def _build(bl, seed, n_layers, H, KV, F, gain=True):
    """Quantise every weight on both sides; the packed bytes and gamma bits
    must agree before the stack is compared."""
    gpu_layers, ref_layers = [], []
    for l in range(n_layers):
        W = workloads.stack_layer_weights(seed, l, H, KV, F)
        norm = workloads.stack_norm_gain(seed, l, F, gain) if gain is not None else None
        G, R = {}, {}
        for name, gname in zip(NAMES, GAMMAS):
            Wp, g = bl.quant_weight_absmean_pack(W[name].cuda())
            rp, rg = oracle.quantize_weight(W[name].numpy())
            torch.cuda.synchronize()
            assert np.array_equal(Wp.cpu().numpy(), rp), (l, name)
            assert np.float32(g.item()).view(np.uint32) == np.float32(rg).view(np.uint32)
            G[name], G[gname] = Wp, g
            R[name], R[gname] = rp, rg
        G["ffn_norm"] = norm.cuda() if norm is not None else None
        R["ffn_norm"] = norm.numpy() if norm is not None else None
        gpu_layers.append(G)
        ref_layers.append(R)
    return gpu_layers, ref_layers


SEGMENTS = ("x_in", "q", "k", "v", "o", "x_mid", "y")


def _segments(row, H, KV):
    cuts = np.cumsum([0, H, H, KV, KV, H, H, H])
    return {n: row[cuts[i]:cuts[i + 1]] for i, n in enumerate(SEGMENTS)}


def _teacher_forced(trace, x_final, layers, H, KV, F, D, eps=1e-5):
    """Each layer of the GPU trace against the oracle run on that layer alone,
    from the GPU's input to it."""
    n = trace.shape[0]
    u = lambda a: np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    for l in range(n):
        got = _segments(trace[l], H, KV)
        _, ref_row = oracle.decode_stack(got["x_in"].copy(), [layers[l]], H, KV, F, D, eps)
        ref = _segments(ref_row[0], H, KV)
        for name in ("q", "k", "v", "o", "x_mid"):
            diff = u(got[name]) != u(ref[name])
            assert not diff.any(), (l, name, int(diff.sum()))
        err = np.abs(got["y"].astype(np.float64) - ref["y"].astype(np.float64))
        bad = err > RTOL * np.abs(ref["y"].astype(np.float64))
        assert not bad.any(), (l, "y", int(bad.sum()), float(err.max()))
        x_next = np.add(got["x_mid"], got["y"], dtype=np.float32)
        following = trace[l + 1, :H] if l + 1 < n else x_final
        assert np.array_equal(u(following), u(x_next)), (l, "x_next")


def _compare(trace, ref_trace, H, KV):
    cuts = np.cumsum([0, H, H, KV, KV, H, H, H])
    names = ("x_in", "q", "k", "v", "o", "x_mid", "y")
    for l in range(ref_trace.shape[0]):
        for i, name in enumerate(names):
            got = trace[l, cuts[i]:cuts[i + 1]]
            ref = ref_trace[l, cuts[i]:cuts[i + 1]]
            if l == 0 and name != "y":
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (l, name)
                continue
            scale = np.abs(ref).max()
            err = np.abs(got.astype(np.float64) - ref).max()
            assert err <= RTOL * scale, (l, name, err, scale)
    same = np.mean(trace.view(np.uint32) == ref_trace.view(np.uint32))
    assert same >= 0.999, same


PATHS = pytest.mark.parametrize("path", [1, 2], ids=["launches", "persistent"])


@PATHS
@pytest.mark.parametrize("H,KV,F,D,n_layers,gain", [
    (256, 128, 512, 64, 3, True),      # 4 query heads on 2 key/value heads
    (192, 192, 320, 64, 2, True),      # one query head per key/value head; F % 128 = 64
    (256, 64, 448, 32, 2, None),       # 8 query heads on 2; no subln gain
    (2560, 640, 6912, 128, 2, True),   # 2B-class layer dimensions
], ids=["grouped", "mha_ragged", "gqa8_nogain", "full_dims"])
def test_decode_stack_matches_oracle(gpu, H, KV, F, D, n_layers, gain, path):
    bl = gpu
    seed = 11 + H + n_layers
    gl, rl = _build(bl, seed, n_layers, H, KV, F, gain)
    x0 = workloads.stack_token(seed, H)
    x = x0.cuda()
    trace = bl.bitlinear_decode_stack(gl, x, H, KV, F, D, eps=1e-5, trace=True, path=path)
    torch.cuda.synchronize()
    ref_x, ref_trace = oracle.decode_stack(x0.numpy(), rl, H, KV, F, D, 1e-5)
    _compare(trace.cpu().numpy(), ref_trace, H, KV)
    got = x.cpu().numpy()
    err = np.abs(got.astype(np.float64) - ref_x).max()
    assert err <= RTOL * np.abs(ref_x).max()


@PATHS
def test_decode_stack_trace_off_and_no_layers(gpu, path):
    bl = gpu
    H, KV, F, D = 256, 128, 512, 64
    gl, _ = _build(bl, 5, 2, H, KV, F)
    x0 = workloads.stack_token(5, H).cuda()
    x1 = x0.clone()
    t = bl.bitlinear_decode_stack(gl, x1, H, KV, F, D, trace=True, path=path)
    x2 = x0.clone()
    assert bl.bitlinear_decode_stack(gl, x2, H, KV, F, D, path=path) is None
    x3 = x0.clone()
    bl.bitlinear_decode_stack([], x3, H, KV, F, D, path=path)
    torch.cuda.synchronize()
    assert torch.equal(x1, x2)                       # the trace does not change the result
    assert torch.equal(x3, x0)                       # no layers: x untouched
    assert torch.equal(t[0, :H], x0)
    assert not torch.equal(x1, x0)


@PATHS
def test_decode_stack_graph_replay(gpu, path):
    # The stack records no memset and no host synchronisation, so it can be
    # captured once and replayed; every replay must equal the eager result.
    bl = gpu
    H, KV, F, D = 256, 64, 512, 32
    gl, _ = _build(bl, 9, 2, H, KV, F)
    x0 = workloads.stack_token(9, H).cuda()
    ref = x0.clone()
    ws = torch.empty(bl.workspace_bytes(bl.BL_OP_DECODE_STACK, 1, H, KV, F),
                     dtype=torch.uint8, device="cuda")
    bl.bitlinear_decode_stack(gl, ref, H, KV, F, D, ws=ws, path=path)
    torch.cuda.synchronize()
    x = x0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bl.bitlinear_decode_stack(gl, x, H, KV, F, D, ws=ws, stream=s, path=path)   # warm-up
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bl.bitlinear_decode_stack(gl, x, H, KV, F, D, ws=ws,
                                  stream=torch.cuda.current_stream(), path=path)
    for _ in range(3):
        x.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x, ref)
        _ = (x0 * 2).sum().item()                    # eager work between replays


def test_decode_stack_chunked_layers(gpu):
    # 18 layers span two persistent launches (16 layers each at most); the
    # second launch picks the residual stream up from the workspace.
    bl = gpu
    H, KV, F, D, n = 128, 64, 256, 32, 18
    gl, rl = _build(bl, 21, n, H, KV, F)
    x0 = workloads.stack_token(21, H)
    x = x0.cuda()
    trace = bl.bitlinear_decode_stack(gl, x, H, KV, F, D, trace=True,
                                      path=bl.BL_STACK_PERSISTENT)
    torch.cuda.synchronize()
    ref_x, ref_trace = oracle.decode_stack(x0.numpy(), rl, H, KV, F, D, 1e-5)
    _compare(trace.cpu().numpy(), ref_trace, H, KV)
    err = np.abs(x.cpu().numpy().astype(np.float64) - ref_x).max()
    assert err <= RTOL * np.abs(ref_x).max()


@PATHS
def test_decode_stack_teacher_forced_30_layers(gpu, path):
    """The 2B-class stack as timed (30 layers at 2560 / 640 / 6912, head size
    128; the persistent path runs it as 16 + 14 layers in two launches, and
    reuses its 16 layer slots), every layer checked teacher-forced.  Three
    quantised layers are cycled over the 30 to keep the setup short."""
    bl = gpu
    H, KV, F, D = workloads.HIDDEN, workloads.KV, workloads.FFN, workloads.HEAD_DIM
    n = workloads.LAYERS
    gl, rl = _build(bl, 41, 3, H, KV, F)
    gl = [gl[l % 3] for l in range(n)]
    rl = [rl[l % 3] for l in range(n)]
    x0 = workloads.stack_token(41, H)
    x = x0.cuda()
    ws = torch.empty(bl.workspace_bytes(bl.BL_OP_DECODE_STACK, 1, H, KV, F), dtype=torch.uint8,
                     device="cuda")
    trace = bl.bitlinear_decode_stack(gl, x, H, KV, F, D, eps=1e-5, trace=True, ws=ws, path=path)
    torch.cuda.synchronize()
    assert bl.bitlinear_decode_stack_status(ws, H, KV, F, D, path=path) == 0
    trace = trace.cpu().numpy()
    assert np.array_equal(trace[0, :H].view(np.uint32), x0.numpy().view(np.uint32))
    _teacher_forced(trace, x.cpu().numpy(), rl, H, KV, F, D)


@PATHS
def test_decode_stack_teacher_forced_small(gpu, path):
    """Teacher-forced on the small dimension sets, 18 layers (two persistent
    launches), subln gain on."""
    bl = gpu
    H, KV, F, D, n = 256, 64, 448, 32, 18
    gl, rl = _build(bl, 45, n, H, KV, F)
    x0 = workloads.stack_token(45, H)
    x = x0.cuda()
    trace = bl.bitlinear_decode_stack(gl, x, H, KV, F, D, trace=True, path=path)
    torch.cuda.synchronize()
    _teacher_forced(trace.cpu().numpy(), x.cpu().numpy(), rl, H, KV, F, D)


def test_decode_stack_status_after_time_out(gpu):
    """A wait limit of 1 us, far shorter than one exchange of the persistent
    path, makes waits give up: the kernel still exits, x is NaN and the status
    call reports it; the next call with the default limit clears the status."""
    bl = gpu
    H, KV, F, D = 512, 128, 1024, 64
    gl, _ = _build(bl, 47, 2, H, KV, F)
    x0 = workloads.stack_token(47, H).cuda()
    ws = torch.empty(bl.workspace_bytes(bl.BL_OP_DECODE_STACK, 1, H, KV, F), dtype=torch.uint8,
                     device="cuda")
    x = x0.clone()
    bl.bitlinear_decode_stack(gl, x, H, KV, F, D, ws=ws, path=bl.BL_STACK_PERSISTENT, wait_us=1)
    torch.cuda.synchronize()
    assert bl.bitlinear_decode_stack_status(ws, H, KV, F, D) == 1
    assert torch.isnan(x).all()
    x = x0.clone()
    bl.bitlinear_decode_stack(gl, x, H, KV, F, D, ws=ws, path=bl.BL_STACK_PERSISTENT)
    torch.cuda.synchronize()
    assert bl.bitlinear_decode_stack_status(ws, H, KV, F, D) == 0
    assert torch.isfinite(x).all()
    x = x0.clone()
    bl.bitlinear_decode_stack(gl, x, H, KV, F, D, ws=ws, path=bl.BL_STACK_LAUNCHES)
    torch.cuda.synchronize()
    assert bl.bitlinear_decode_stack_status(ws, H, KV, F, D) == 0


def test_decode_stack_paths_agree_full_dims(gpu):
    # Both paths on the 2B-class dimensions (3 layers): identical up to the
    # order of the fp64 sum of H^2 in the subln RMS.
    bl = gpu
    H, KV, F, D = workloads.HIDDEN, workloads.KV, workloads.FFN, workloads.HEAD_DIM
    gl, _ = _build(bl, 31, 3, H, KV, F)
    x0 = workloads.stack_token(31, H).cuda()
    xa, xb = x0.clone(), x0.clone()
    ta = bl.bitlinear_decode_stack(gl, xa, H, KV, F, D, trace=True, path=bl.BL_STACK_LAUNCHES)
    tb = bl.bitlinear_decode_stack(gl, xb, H, KV, F, D, trace=True,
                                   path=bl.BL_STACK_PERSISTENT)
    torch.cuda.synchronize()
    _compare(tb.cpu().numpy(), ta.cpu().numpy().astype(np.float32), H, KV)
    assert torch.isfinite(xb).all()
    assert (xa - xb).abs().max().item() <= RTOL * xa.abs().max().item()
