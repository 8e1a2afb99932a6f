"""GPU parity: libbitlinear (through its C ABI) against the CPU oracle.

Bar: every integer result (packed weights, gamma's bits, int8 activations and
their scales, int32 accumulators, the FFN's int8 intermediate and its scale)
is bit-exact; a BitLinear's fp32 output Y = fl(float(acc) * fl(gamma * d)) is
bit-exact too (the oracle's fp32 rescale of its own accumulators), and within
1e-3 relative of the oracle's fp64 value; the FFN's fp32 output, which carries
a summation of H^2 whose order is the library's, is within 1e-3 relative,
element by element.  Inputs are the seeded synthetic workloads of
workloads.py, at small sizes that span several tiles with ragged tails, and at
the full 2B-class shapes (every output row, prefill included).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

RTOL = 1e-3          # fp32 outputs against the oracle's fp64 values
CANARY = -12345.678  # fills guard bands after every output


def _f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def _gpu_weight(bl, W):
    Wp, g = bl.quant_weight_absmean_pack(W.cuda())
    torch.cuda.synchronize()
    return Wp, g


def _ref_act(X):
    if X.dtype == torch.bfloat16:
        x32 = oracle.bf16_to_f32(workloads.bf16_bits(X))
    else:
        x32 = X.numpy()
    return oracle.quant_act(x32)


def _assert_close(Y, ref, rtol=RTOL):
    Y = np.asarray(Y, dtype=np.float64)
    err = np.abs(Y - ref)
    bad = err > rtol * np.abs(ref)
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outside rel {rtol}; "
                           f"worst {np.max(err / np.maximum(np.abs(ref), 1e-300)):.3e}")


def _assert_y_bits(Y, acc_ref, d_ref, g_ref):
    """Y bit for bit equal to the oracle's fp32 rescale of its accumulators."""
    Y32 = oracle.dequant_f32(acc_ref, d_ref, g_ref)
    diff = _f32_bits(Y) != _f32_bits(Y32)
    assert not diff.any(), f"{diff.sum()} of {diff.size} fp32 outputs differ in their bits"


def _guarded(shape, dtype, fill):
    """An output tensor followed by a guard band; returns (view, guard)."""
    n = int(np.prod(shape)) if len(shape) else 1
    buf = torch.full((n + 256,), fill, dtype=dtype, device="cuda")
    return buf[:n].view(*shape), buf[n:]


# ---------------------------------------------------------------- weights
@pytest.mark.parametrize("N,K,seed", [(256, 256, 0), (67, 260, 1), (640, 2560, 2),
                                      (6912, 2560, 3), (2560, 6912, 4), (1, 4, 5),
                                      (20000, 64, 6), (16385, 8, 7), (13000, 2600, 8)])
def test_quant_weight_bit_exact(gpu, N, K, seed):
    """Ragged block tails (N*K not a multiple of 2048); above 2^24 weights the
    block sums span 2 (6912 x 2560) and 3 (13000 x 2600) chunks of the upper
    pairwise levels."""
    W = workloads.weight(workloads.generator(seed), N, K)
    Wp, g = _gpu_weight(gpu, W)
    Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
    assert _f32_bits(g.cpu().numpy()[0]) == _f32_bits(g_ref)
    assert np.array_equal(Wp.cpu().numpy(), Wp_ref)


@pytest.mark.parametrize("N,K,lo,hi", [(300, 1028, -6, 3), (9000, 12, -6, 3), (4100, 4100, -33, 27)])
def test_quant_weight_wide_range_bit_exact(gpu, N, K, lo, hi):
    """Magnitudes over 9 or 60 decades (weights times 10^j, j in [lo, hi))
    make the fp64 sum depend on its order: gamma must still match the
    oracle's bits."""
    g = workloads.generator(800 + N)
    W = workloads.weight(g, N, K) * torch.pow(
        10.0, torch.randint(lo, hi, (N, K), generator=g).double()).float()
    Wp, gam = _gpu_weight(gpu, W)
    Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
    assert _f32_bits(gam.cpu().numpy()[0]) == _f32_bits(g_ref)
    assert np.array_equal(Wp.cpu().numpy(), Wp_ref)


def test_quant_weight_golden_and_ties(gpu):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "handworked.json")) as f:
        cases = json.load(f)["weights"]
    for c in cases:
        W = torch.tensor(c["W"], dtype=torch.float32)
        Wp, g = _gpu_weight(gpu, W)
        assert g.item() == c["gamma"], c["derivation"]
        assert Wp.cpu().tolist() == c["Wp"], c["derivation"]
    # constant magnitude with random signs: gamma == |w|, Wq == sign
    s = torch.randint(0, 2, (96, 128), generator=workloads.generator(8)).float() * 2 - 1
    Wp, g = _gpu_weight(gpu, s * 0.0173)
    assert g.item() == np.float32(0.0173)
    Wp_ref, g_ref = oracle.quantize_weight((s * 0.0173).numpy())
    assert np.array_equal(oracle.unpack(Wp_ref, 128), s.numpy().astype(np.int8))
    assert np.array_equal(Wp.cpu().numpy(), Wp_ref) and g.item() == g_ref


def test_quant_weight_empty(gpu):
    g = torch.full((1,), 7.0, device="cuda")
    for N, K in ((0, 64), (5, 0)):
        W = torch.zeros(N, K, device="cuda")
        Wp = torch.zeros(N, K // 4, dtype=torch.uint8, device="cuda")
        gpu.quant_weight_absmean_pack(W, Wp=Wp, gamma=g)
        torch.cuda.synchronize()
        assert g.item() == 0.0


# ------------------------------------------------------------ activations
@pytest.mark.parametrize("M,K,dtype,seed", [
    (4, 256, torch.float32, 0), (1, 2560, torch.bfloat16, 1), (1, 6912, torch.bfloat16, 2),
    (64, 6912, torch.bfloat16, 3), (2048, 2560, torch.bfloat16, 4), (3, 257, torch.float32, 5),
    (5, 260, torch.bfloat16, 6), (2, 1, torch.float32, 7),
    (3, 8192, torch.bfloat16, 8), (2, 8200, torch.float32, 9), (7, 6912, torch.float32, 10),
    (3, 8, torch.bfloat16, 11)])
def test_quant_act_bit_exact(gpu, M, K, dtype, seed):
    X = workloads.activations(workloads.generator(seed), M, K, dtype=dtype)
    if M > 1:
        X[1] = 0                       # an all-zero token
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    Xq_ref, d_ref = _ref_act(X)
    assert np.array_equal(Xq.cpu().numpy(), Xq_ref)
    assert np.array_equal(_f32_bits(d.cpu().numpy()), _f32_bits(d_ref))


def test_quant_act_golden(gpu):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "handworked.json")) as f:
        cases = json.load(f)["activations"]
    for c in cases:
        Xq, d = gpu.quant_act_absmax_i8(torch.tensor(c["X"], dtype=torch.float32).cuda())
        assert Xq.cpu().tolist() == c["Xq"], c["derivation"]
        assert d.cpu().tolist() == c["d"], c["derivation"]


# ------------------------------------------------------------------ products
def _product_case(gpu, call, M, K, N, seed, dtype=torch.bfloat16):
    W, X = workloads.bitlinear_problem(seed, M, K, N, dtype=dtype)
    Wp, g = _gpu_weight(gpu, W)
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    Y, Yguard = _guarded((M, N), torch.float32, CANARY)
    acc, Aguard = _guarded((M, N), torch.int32, -7)
    getattr(gpu, call)(Xq, d, Wp, g, Y=Y, acc=acc)
    torch.cuda.synchronize()
    assert torch.all(Yguard == CANARY) and torch.all(Aguard == -7), "write past the output"
    Xq_ref, d_ref = _ref_act(X)
    Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
    acc_ref, Y_ref = oracle.bitlinear(Xq_ref, d_ref, Wp_ref, g_ref, K)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    _assert_y_bits(Y.cpu().numpy(), acc_ref, d_ref, g_ref)
    _assert_close(Y.cpu().numpy(), Y_ref)
    return Y, acc


@pytest.mark.parametrize("shape", workloads.DECODE_SHAPES, ids=lambda s: s.name)
def test_gemv_decode_shapes(gpu, shape):
    _product_case(gpu, "bitlinear_gemv", 1, shape.K, shape.N, 10 + shape.N)


@pytest.mark.parametrize("M", [2, 3, 4, 5, 8, 9, 13, 32, 64])
def test_gemv_token_counts(gpu, M):
    _product_case(gpu, "bitlinear_gemv", M, 2560, 640, 100 + M)


@pytest.mark.parametrize("M", workloads.BATCHED_M)
@pytest.mark.parametrize("shape", workloads.BATCHED_SHAPES, ids=lambda s: s.name)
def test_gemv_batched_decode(gpu, M, shape):
    _product_case(gpu, "bitlinear_gemv", M, shape.K, shape.N, 200 + M)


@pytest.mark.parametrize("M,K,N", [(1, 64, 1), (1, 64, 7), (3, 320, 641), (1, 6912, 97),
                                   (7, 4096, 65), (1, 25600, 33), (8, 12288, 50),
                                   (1, 131072, 9)])
def test_gemv_ragged(gpu, M, K, N):
    _product_case(gpu, "bitlinear_gemv", M, K, N, 300 + N)


@pytest.mark.parametrize("call,M,K,N", [
    # the role-split MFMA kernel (M < 128, K <= 8192): rounds of 2048 k,
    # 16-token blocks, 16 RB weight rows per workgroup
    ("bitlinear_gemm", 1, 6912, 100),     # one token; four rounds, the last partial
    ("bitlinear_gemm", 17, 6912, 65),     # two token blocks, the second with one token
    ("bitlinear_gemm", 33, 576, 97),      # three blocks; one partial round
    ("bitlinear_gemv", 3, 320, 641),      # v_dot4 hands over to the MFMA kernel at M = 3
    ("bitlinear_gemv", 64, 8192, 50),     # the largest K the kernel takes
    ("bitlinear_gemm", 8, 6912, 4160),    # codes past M staged as zeros; RB = 2
    ("bitlinear_gemm", 9, 6912, 4110),    # ragged N inside a row block
    ("bitlinear_gemm", 20, 2560, 4200),   # two blocks, RB = 4 (grid past 256 otherwise)
    ("bitlinear_gemm", 40, 576, 4200),    # a round of 36 groups
    ("bitlinear_gemm", 100, 8192, 40),    # seven blocks, three row groups (the last ragged)
    ("bitlinear_gemm", 127, 64, 33),      # one unit per row, eight blocks, ragged N
    ("bitlinear_gemm", 16, 2048, 16),     # one round exactly, one workgroup
    ("bitlinear_gemm", 5, 64, 300),       # one unit per row: only one lane group holds weights
    ("bitlinear_gemm", 17, 2112, 4097),   # a 1-unit last round; two blocks; RB = 4, idle slots
    ("bitlinear_gemv", 48, 4096, 1000),   # three token blocks (grid order by XCD)
    ("bitlinear_gemm", 127, 6144, 2050),  # three rounds, eight blocks, RB capped at 4
    ("bitlinear_gemv", 64, 2560, 6912),   # RB = 8
    # K past 8192: the earlier paths
    ("bitlinear_gemm", 5, 8256, 64),      # the 128 x 128 tile kernel
    ("bitlinear_gemv", 40, 8256, 30),     # v_dot4
], ids=lambda v: str(v))
def test_few_token_kernel_paths(gpu, call, M, K, N):
    _product_case(gpu, call, M, K, N, 500 + M + N)


def test_tiny_config(gpu):
    t = workloads.TINY
    for call in ("bitlinear_gemv", "bitlinear_gemm"):
        _product_case(gpu, call, t["M"], t["K"], t["N"], t["seed"], dtype=t["dtype"])


@pytest.mark.parametrize("M,K,N", [(1, 64, 1), (130, 192, 131), (129, 2560, 257),
                                   (256, 640, 384), (17, 6912, 100), (64, 2560, 640),
                                   (513, 128, 257), (300, 6912, 300), (1024, 64, 512)])
def test_gemm_ragged(gpu, M, K, N):
    _product_case(gpu, "bitlinear_gemm", M, K, N, 400 + M)


@pytest.mark.parametrize("K,N", [(2560, 6912), (6912, 2560)], ids=["gate_up", "down"])
def test_gemm_prefill_full_size(gpu, K, N):
    """M = 2048 at both prefill shapes, as timed; every output is compared."""
    p = workloads.PREFILL
    M = p["M"]
    W, X = workloads.bitlinear_problem(p["seed"] + K, M, K, N)
    Wp, g = _gpu_weight(gpu, W)
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    Y, acc = gpu.bitlinear_gemm(Xq, d, Wp, g, want_acc=True)
    torch.cuda.synchronize()
    Xq_ref, d_ref = _ref_act(X)
    assert np.array_equal(Xq.cpu().numpy(), Xq_ref)
    Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
    assert np.array_equal(Wp.cpu().numpy(), Wp_ref)
    acc_ref, Y_ref = oracle.bitlinear(Xq_ref, d_ref, Wp_ref, g_ref, K)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    _assert_y_bits(Y.cpu().numpy(), acc_ref, d_ref, g_ref)
    _assert_close(Y.cpu().numpy(), Y_ref)


def test_gemv_equals_gemm(gpu):
    """Both kernels give identical bits for every M the decode call takes."""
    W, X = workloads.bitlinear_problem(31, 64, 2560, 1000)
    Wp, g = _gpu_weight(gpu, W)
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    for M in (1, 2, 5, 8, 9, 64):
        Y1, a1 = gpu.bitlinear_gemv(Xq[:M], d[:M], Wp, g, want_acc=True)
        Y2, a2 = gpu.bitlinear_gemm(Xq[:M], d[:M], Wp, g, want_acc=True)
        torch.cuda.synchronize()
        assert torch.equal(a1, a2) and torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))


def test_determinism(gpu):
    W, X = workloads.bitlinear_problem(32, 300, 2560, 700)
    Wp, g = _gpu_weight(gpu, W)
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    outs = [gpu.bitlinear_gemm(Xq, d, Wp, g) for _ in range(2)]
    outs += [gpu.bitlinear_gemv(Xq[:8], d[:8], Wp, g) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[2], outs[3])


def test_empty_products(gpu):
    Xq = torch.zeros(0, 64, dtype=torch.int8, device="cuda")
    d = torch.zeros(0, device="cuda")
    Wp = torch.zeros(5, 16, dtype=torch.uint8, device="cuda")
    g = torch.ones(1, device="cuda")
    assert gpu.bitlinear_gemm(Xq, d, Wp, g).shape == (0, 5)
    assert gpu.bitlinear_gemv(Xq, d, Wp, g).shape == (0, 5)


# ------------------------------------------------------------------------ FFN
def _ffn_case(gpu, M, K, F, N, seed, gated=True, gain=True, eps=1e-5, rows=None):
    Wg, Wu, Wd, X = workloads.ffn_problem(seed, M, K, F, N)
    Wgp, gg = _gpu_weight(gpu, Wg)
    Wup, gu = _gpu_weight(gpu, Wu)
    Wdp, gd = _gpu_weight(gpu, Wd)
    nw = None
    if gain:
        nw = 1.0 + 0.5 * torch.randn(F, generator=workloads.generator(seed + 99))
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    Y, Hq, dh = gpu.bitlinear_ffn_relu2(Xq, d, Wgp, gg, Wup if gated else None,
                                        gu if gated else None, Wdp, gd,
                                        norm_w=nw.cuda() if gain else None, eps=eps,
                                        want_debug=True)
    torch.cuda.synchronize()
    Xq_ref, d_ref = _ref_act(X)
    ref_w = {}
    for name, W, Wp_gpu, g_gpu in (("g", Wg, Wgp, gg), ("u", Wu, Wup, gu), ("d", Wd, Wdp, gd)):
        Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
        assert np.array_equal(Wp_gpu.cpu().numpy(), Wp_ref) and g_gpu.item() == g_ref
        ref_w[name] = (Wp_ref, g_ref)
    if rows is None:
        rows = np.arange(M)
    ref = oracle.ffn_relu2(Xq_ref[rows], d_ref[rows], ref_w["g"][0], ref_w["g"][1],
                           ref_w["u"][0] if gated else None, ref_w["u"][1],
                           nw.numpy() if gain else None, eps, ref_w["d"][0], ref_w["d"][1],
                           K, F, N)
    assert np.array_equal(Hq.cpu().numpy()[rows], ref["Hq"])
    assert np.array_equal(_f32_bits(dh.cpu().numpy()[rows]), _f32_bits(ref["dh"]))
    _assert_close(Y.cpu().numpy()[rows], ref["Y"])


@pytest.mark.parametrize("gated,gain", [(True, True), (True, False), (False, True)])
def test_ffn_tiny(gpu, gated, gain):
    _ffn_case(gpu, 4, 256, 512, 256, 40, gated=gated, gain=gain)


@pytest.mark.parametrize("M", [1, 3, 37, 130])
def test_ffn_token_counts(gpu, M):
    _ffn_case(gpu, M, 320, 384, 200, 50 + M)


def test_ffn_decode_shape(gpu):
    _ffn_case(gpu, 1, 2560, 6912, 2560, 60)


def test_ffn_prefill_full_size(gpu):
    """The M = 2048 FFN block as timed; every row is compared."""
    p = workloads.PREFILL
    _ffn_case(gpu, p["M"], p["K"], p["F"], p["N"], p["seed"])


@pytest.mark.parametrize("M,K,F,N,gated,gain", [
    (256, 256, 320, 192, True, True),     # one M-tile; F % 128 = 64: a half-empty column tile
    (300, 128, 512, 64, True, False),     # ragged M (two M-tiles), no subln gain
    (129, 192, 448, 100, True, True),     # K % 128 = 64 tail, 3.5 column tiles
    (200, 256, 384, 96, False, True),     # no gate: separate product and tail
    (128, 64, 256, 64, True, True),       # K = 64: no full k-step, the tail step only
], ids=["one_tile_ragged_f", "ragged_m_nogain", "k_tail", "ungated", "k64"])
def test_ffn_prefill_paths(gpu, M, K, F, N, gated, gain):
    """M >= 128 with a gate runs the fused gate/up kernel and the partial-sum
    tail; every row is compared with the oracle."""
    _ffn_case(gpu, M, K, F, N, 80 + M, gated=gated, gain=gain)


def test_ffn_prefill_zero_token_and_determinism(gpu):
    M, K, F, N = 260, 128, 384, 64
    Wg, Wu, Wd, X = workloads.ffn_problem(71, M, K, F, N)
    Wgp, gg = _gpu_weight(gpu, Wg)
    Wup, gu = _gpu_weight(gpu, Wu)
    Wdp, gd = _gpu_weight(gpu, Wd)
    X[5] = 0
    X[259] = 0
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    out1 = gpu.bitlinear_ffn_relu2(Xq, d, Wgp, gg, Wup, gu, Wdp, gd, want_debug=True)
    out2 = gpu.bitlinear_ffn_relu2(Xq, d, Wgp, gg, Wup, gu, Wdp, gd, want_debug=True)
    torch.cuda.synchronize()
    Y, Hq, dh = out1
    for r in (5, 259):
        assert dh[r].item() == 0 and not Hq[r].any() and not Y[r].any()
    for a, b in zip(out1, out2):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.int8 else a.view(torch.int32),
                           b.view(torch.uint8) if b.dtype == torch.int8 else b.view(torch.int32))


def test_ffn_zero_token(gpu):
    """An all-zero token gives zero codes, dh = 0 and a zero output row."""
    M, K, F, N = 3, 128, 256, 64
    Wg, Wu, Wd, X = workloads.ffn_problem(70, M, K, F, N)
    Wgp, gg = _gpu_weight(gpu, Wg)
    Wup, gu = _gpu_weight(gpu, Wu)
    Wdp, gd = _gpu_weight(gpu, Wd)
    X[1] = 0
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    Y, Hq, dh = gpu.bitlinear_ffn_relu2(Xq, d, Wgp, gg, Wup, gu, Wdp, gd, want_debug=True)
    torch.cuda.synchronize()
    assert dh[1].item() == 0 and not Hq[1].any() and not Y[1].any()
    assert math.isfinite(Y.abs().max().item())


# --------------------------------------------------------------- fused decode
def _fused_case(gpu, M, shapes, dtype, seed, share_x=False, want_q=True):
    jobs, refs = [], []
    Xshared = None
    for i, (K, N) in enumerate(shapes):
        W, X = workloads.bitlinear_problem(seed + i, M, K, N, dtype=dtype)
        if share_x:
            Xshared = X if Xshared is None else Xshared
            X = Xshared
        Wp, g = _gpu_weight(gpu, W)
        job = dict(X=X.cuda(), Wp=Wp, gamma=g)
        if want_q:
            job["Xq"] = None
            job["d"] = None
        jobs.append(job)
        refs.append((X, W))
    out = gpu.bitlinear_gemv_fused(jobs)
    torch.cuda.synchronize()
    for (X, W), j in zip(refs, out):
        K = X.shape[1]
        Xq_ref, d_ref = _ref_act(X)
        Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
        acc_ref, Y_ref = oracle.bitlinear(Xq_ref, d_ref, Wp_ref, g_ref, K)
        if want_q:
            assert np.array_equal(j["Xq"].cpu().numpy(), Xq_ref)
            assert np.array_equal(_f32_bits(j["d"].cpu().numpy()), _f32_bits(d_ref))
        _assert_y_bits(j["Y"].cpu().numpy(), acc_ref, d_ref, g_ref)
        _assert_close(j["Y"].cpu().numpy(), Y_ref)
        # bit-identical to the two-call path
        Xq2, d2 = gpu.quant_act_absmax_i8(j["X"])
        Y2 = gpu.bitlinear_gemv(Xq2, d2, j["Wp"], j["gamma"])
        torch.cuda.synchronize()
        assert torch.equal(j["Y"].view(torch.int32), Y2.view(torch.int32))


def test_fused_decode_step(gpu):
    shapes = [(s.K, s.N) for s in workloads.DECODE_SHAPES]
    _fused_case(gpu, 1, shapes, torch.bfloat16, 500)


def _fused_fits(M, K, dtype):
    tile = 1 if M == 1 else 2 if M == 2 else 4 if M <= 4 else 8
    es = 4 if dtype == torch.float32 else 2
    return tile * K * (1 + es) <= 128 * 1024


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_fused_tokens_and_dtypes(gpu, M, dtype):
    big = 6912 if _fused_fits(M, 6912, dtype) else 1024
    _fused_case(gpu, M, [(2560, 640), (big, 97), (128, 1)], dtype, 600 + M)


@pytest.mark.parametrize("M,K,dtype", [(1, 16384, torch.float32), (4, 6912, torch.bfloat16),
                                       (8, 2560, torch.bfloat16)])
def test_fused_large_lds(gpu, M, K, dtype):
    """Staged activations above 64 KB of LDS (80, 83 and 61 KB)."""
    assert _fused_fits(M, K, dtype)
    _fused_case(gpu, M, [(K, 300)], dtype, 650 + M)


@pytest.mark.parametrize("K,N", [(64, 1), (4160, 33), (6208, 130), (8256, 17)])
def test_fused_one_token_unit_slots(gpu, K, N):
    """One token runs its dot products on MFMA with the lanes of a row taking
    units s, s + L, ...: rows of 1 unit, of 65 units (9 slots of 8 lanes: a
    second batch whose slot is 1/8 valid), 97 units (16 lanes, last slot 1/16
    valid) and 129 units (16 lanes, 9 slots)."""
    _fused_case(gpu, 1, [(K, N), (2560, 7)], torch.bfloat16, 660 + K)


def test_fused_shared_input_qkv(gpu):
    _fused_case(gpu, 1, [(2560, 2560), (2560, 640), (2560, 640)], torch.bfloat16, 700,
                share_x=True)


def test_fused_eight_jobs_no_q_outputs(gpu):
    shapes = [(64 * (i + 1), 33 * (i + 1)) for i in range(8)]
    _fused_case(gpu, 2, shapes, torch.bfloat16, 800, want_q=False)


def test_fused_zero_rows_job_still_quantises(gpu):
    X = workloads.activations(workloads.generator(900), 1, 320)
    Wp = torch.zeros(0, 80, dtype=torch.uint8, device="cuda")
    g = torch.ones(1, device="cuda")
    out = gpu.bitlinear_gemv_fused([dict(X=X.cuda(), Wp=Wp, gamma=g, Xq=None, d=None)])
    torch.cuda.synchronize()
    Xq_ref, d_ref = _ref_act(X)
    assert np.array_equal(out[0]["Xq"].cpu().numpy(), Xq_ref)
    assert out[0]["Y"].shape == (1, 0)


def test_fused_mixed_order_with_quantise_only_job(gpu):
    """The launch orders the jobs by decreasing K (stable); a quantise-only
    job (no rows) between product jobs of equal and unequal K keeps its own
    Xq and d, and every product job its own Y."""
    specs = [(2560, 100), (6912, 0), (1024, 33), (2560, 64), (6912, 40)]
    jobs, refs = [], []
    for i, (K, N) in enumerate(specs):
        if N == 0:
            X = workloads.activations(workloads.generator(950 + i), 1, K)
            job = dict(X=X.cuda(), Wp=torch.zeros(0, K // 4, dtype=torch.uint8, device="cuda"),
                       gamma=torch.ones(1, device="cuda"), Xq=None, d=None)
            refs.append((X, None))
        else:
            W, X = workloads.bitlinear_problem(950 + i, 1, K, N, dtype=torch.bfloat16)
            Wp, g = _gpu_weight(gpu, W)
            job = dict(X=X.cuda(), Wp=Wp, gamma=g, Xq=None, d=None)
            refs.append((X, W))
        jobs.append(job)
    out = gpu.bitlinear_gemv_fused(jobs)
    torch.cuda.synchronize()
    for (X, W), j in zip(refs, out):
        K = X.shape[1]
        Xq_ref, d_ref = _ref_act(X)
        assert np.array_equal(j["Xq"].cpu().numpy(), Xq_ref)
        assert np.array_equal(_f32_bits(j["d"].cpu().numpy()), _f32_bits(d_ref))
        if W is None:
            assert j["Y"].shape == (1, 0)
            continue
        Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
        acc_ref, Y_ref = oracle.bitlinear(Xq_ref, d_ref, Wp_ref, g_ref, K)
        _assert_y_bits(j["Y"].cpu().numpy(), acc_ref, d_ref, g_ref)
        _assert_close(j["Y"].cpu().numpy(), Y_ref)
