"""GPU parity of the QAT backward (bitlinear_backward_input / _weight) against
the oracle (oracle.backward_input / backward_weight, fp64).

The forward operands are quantised on the GPU, checked bit-exact against the
oracle's own quantisation, and the oracle then takes its own operands.  Bar
for the fp32 gradients: each element within 2^-12 of the exact value relative
to sum_c |term_c| (the magnitudes of the products it adds).  That is a bound
of the kernels' arithmetic with room to spare: each fp32 operand value is
split into bf16 hi + lo (2^-17 of the value), every product is then exact,
and the fp32 accumulator takes one rounding (2^-24 of the running sum) per
16 terms of the contraction plus a few more for the split partials and the
rescale: at most ~(2^-17 + (c/16 + 8) 2^-24) sum |terms| = 3.4e-5 sum |terms|
for the longest contraction tested (c = 6912), 7x below the bar.  Plus two
checks that the fp32 gradient is not rounded to bf16 on the way (outputs made
of a single term must be right to 2^-16, and the median error must sit far
below bf16's).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

BAR = 2.0 ** -12      # |err| <= BAR * sum_c |term_c|, every element
SINGLE_TERM = 2.0 ** -16
CANARY = -12345.678


def _guarded(shape):
    n = int(np.prod(shape))
    buf = torch.full((n + 256,), CANARY, dtype=torch.float32, device="cuda")
    return buf[:n].view(*shape), buf[n:]


def _ref_act(X):
    if X.dtype == torch.bfloat16:
        return oracle.quant_act(oracle.bf16_to_f32(workloads.bf16_bits(X)))
    return oracle.quant_act(X.numpy())


def _assert_bar(out, ref, bound, median_max=1e-5):
    out = np.asarray(out, dtype=np.float64)
    assert np.all(np.isfinite(out))
    err = np.abs(out - ref)
    bad = err > BAR * bound
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside the bar"
    nz = bound > 0
    if nz.any():
        med = float(np.median(err[nz] / bound[nz]))
        assert med <= median_max, f"median relative error {med:.3e}"
    assert np.all(out[~nz] == 0)


def _problem(gpu, M, K, N, seed, dtype=torch.bfloat16):
    """GPU forward operands (checked against the oracle's) and the oracle's."""
    W, X, dY = workloads.qat_problem(seed, M, K, N, dtype=dtype)
    Wp, g = gpu.quant_weight_absmean_pack(W.cuda())
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    torch.cuda.synchronize()
    Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
    Xq_ref, d_ref = _ref_act(X)
    assert np.array_equal(Wp.cpu().numpy(), Wp_ref) and g.item() == g_ref
    assert np.array_equal(Xq.cpu().numpy(), Xq_ref)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), d_ref.view(np.uint32))
    return dict(dY=dY, Wp=Wp, g=g, Xq=Xq, d=d, Wp_ref=Wp_ref, g_ref=g_ref, Xq_ref=Xq_ref,
                d_ref=d_ref)


def _input_bound(dY, Wp_ref, g_ref, K):
    """sum_n |dY[m, n] gamma Wq[n, k]|."""
    return (np.abs(dY.astype(np.float64)) @ np.abs(oracle.unpack(Wp_ref, K).astype(np.float64))
            * float(g_ref))


def _weight_bound(dY, Xq_ref, d_ref):
    """sum_m |dY[m, n] d[m] Xq[m, k]|."""
    G = np.abs(dY.astype(np.float64) * d_ref.astype(np.float64)[:, None])
    return G.T @ np.abs(Xq_ref.astype(np.float64))


def _check_case(gpu, M, K, N, seed, dtype=torch.bfloat16):
    p = _problem(gpu, M, K, N, seed, dtype)
    dY = p["dY"].numpy()
    dX, gx = _guarded((M, K))
    dW, gw = _guarded((N, K))
    gpu.bitlinear_backward_input(p["dY"].cuda(), p["Wp"], p["g"], dX=dX)
    gpu.bitlinear_backward_weight(p["dY"].cuda(), p["Xq"], p["d"], dW=dW)
    torch.cuda.synchronize()
    assert bool((gx == CANARY).all()) and bool((gw == CANARY).all())
    ref = oracle.backward_input(dY, p["Wp_ref"], p["g_ref"], K)
    _assert_bar(dX.cpu().numpy(), ref, _input_bound(dY, p["Wp_ref"], p["g_ref"], K))
    ref = oracle.backward_weight(dY, p["Xq_ref"], p["d_ref"])
    _assert_bar(dW.cpu().numpy(), ref, _weight_bound(dY, p["Xq_ref"], p["d_ref"]))


@pytest.mark.parametrize("M,K,N", [
    (1, 64, 4),          # one token, one k-block: every tile ragged
    (3, 192, 68),        # N % 32 = 4: a partial 32-wide contraction step
    (130, 320, 260),     # ragged in every dimension, several tiles
    (257, 128, 132),     # M just past two row tiles
    (64, 640, 2560),     # long contraction, 3 tiles: dX split 4 ways
    (200, 2560, 640),    # k/v projection: dX split 2 ways
    (128, 2560, 2560),   # q/o projection
    (1000, 320, 200),    # many tokens, few tiles: dW split 4 ways
    (4096, 128, 64),     # one dW tile, 128 c-steps: split 8 ways
    (3, 131072, 64),     # the largest K the calls take
])
def test_backward_ragged(gpu, M, K, N):
    _check_case(gpu, M, K, N, 500 + M)


def test_backward_fp32_inputs(gpu):
    _check_case(gpu, 37, 256, 100, 540, dtype=torch.float32)


@pytest.mark.parametrize("shape", workloads.QAT_SHAPES, ids=lambda s: s.name)
def test_backward_full_size_sampled(gpu, shape):
    """M = 2048 tokens at the 2B-class FFN shapes, in the launch the benchmark
    times; the oracle recomputes sampled rows of dX (rows of dY) and of dW
    (columns of dY) in full."""
    M, K, N = workloads.QAT_M, shape.K, shape.N
    p = _problem(gpu, M, K, N, 560 + K)
    dY = p["dY"].numpy()
    dX = gpu.bitlinear_backward_input(p["dY"].cuda(), p["Wp"], p["g"])
    dW = gpu.bitlinear_backward_weight(p["dY"].cuda(), p["Xq"], p["d"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(K)
    rows = np.unique(np.concatenate([[0, 127, 128, M - 1], rng.integers(0, M, 12)]))
    ref = oracle.backward_input(dY[rows], p["Wp_ref"], p["g_ref"], K)
    _assert_bar(dX.cpu().numpy()[rows], ref,
                _input_bound(dY[rows], p["Wp_ref"], p["g_ref"], K))
    cols = np.unique(np.concatenate([[0, 127, 128, N - 1], rng.integers(0, N, 12)]))
    ref = oracle.backward_weight(dY[:, cols], p["Xq_ref"], p["d_ref"])
    _assert_bar(dW.cpu().numpy()[cols], ref,
                _weight_bound(dY[:, cols], p["Xq_ref"], p["d_ref"]))


def test_backward_single_term_outputs_keep_fp32(gpu):
    """With one nonzero per row (dX) or per column (dW) of dY, every output is
    a single product: the fp32 gradient must survive to 2^-16, which a bf16
    rounding of it (2^-9) would not."""
    M, K, N = 96, 256, 128
    p = _problem(gpu, M, K, N, 570)
    dY = np.zeros((M, N), np.float32)
    vals = (1.0 + np.arange(M) * 2.0 ** -12).astype(np.float32) * 1e-3
    dY[np.arange(M), np.arange(M) % N] = vals                   # one per row and per column
    dYt = torch.from_numpy(dY).cuda()
    dX = gpu.bitlinear_backward_input(dYt, p["Wp"], p["g"]).cpu().numpy()
    dW = gpu.bitlinear_backward_weight(dYt, p["Xq"], p["d"]).cpu().numpy()
    ref = oracle.backward_input(dY, p["Wp_ref"], p["g_ref"], K)
    nz = ref != 0
    assert nz.any()
    assert np.all(np.abs(dX[nz] - ref[nz]) <= SINGLE_TERM * np.abs(ref[nz]))
    assert np.all(dX[~nz] == 0)
    ref = oracle.backward_weight(dY, p["Xq_ref"], p["d_ref"])
    nz = ref != 0
    assert nz.any()
    assert np.all(np.abs(dW[nz] - ref[nz]) <= SINGLE_TERM * np.abs(ref[nz]))
    assert np.all(dW[~nz] == 0)


def test_backward_empty_sums_write_zeros(gpu):
    """N = 0: dX = 0 (no output features); M = 0: dW = 0 (no tokens)."""
    dX, gx = _guarded((3, 128))
    gpu.bitlinear_backward_input(torch.zeros(3, 0, device="cuda"),
                                 torch.zeros(0, 32, dtype=torch.uint8, device="cuda"),
                                 torch.ones(1, device="cuda"), dX=dX)
    dW, gw = _guarded((5, 64))
    gpu.bitlinear_backward_weight(torch.zeros(0, 5, device="cuda"),
                                  torch.zeros(0, 64, dtype=torch.int8, device="cuda"),
                                  torch.zeros(0, device="cuda"), dW=dW)
    torch.cuda.synchronize()
    assert not dX.any() and not dW.any()
    assert bool((gx == CANARY).all()) and bool((gw == CANARY).all())
    # empty outputs: nothing to do
    assert gpu.bitlinear_backward_input(torch.zeros(0, 8, device="cuda"),
                                        torch.zeros(8, 16, dtype=torch.uint8, device="cuda"),
                                        torch.ones(1, device="cuda")).shape == (0, 64)
    assert gpu.bitlinear_backward_weight(torch.zeros(4, 0, device="cuda"),
                                         torch.zeros(4, 64, dtype=torch.int8, device="cuda"),
                                         torch.ones(4, device="cuda")).shape == (0, 64)


def test_backward_zero_token_and_determinism(gpu):
    """An all-zero token (d = 0) adds nothing to dW; two runs are bit-identical."""
    M, K, N = 150, 192, 72
    W, X, dY = workloads.qat_problem(580, M, K, N)
    X[7] = 0
    Wp, g = gpu.quant_weight_absmean_pack(W.cuda())
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    dYc = dY.cuda()
    a = [gpu.bitlinear_backward_input(dYc, Wp, g) for _ in range(2)]
    b = [gpu.bitlinear_backward_weight(dYc, Xq, d) for _ in range(2)]
    dY2 = dYc.clone()
    dY2[7] = 0
    c = gpu.bitlinear_backward_weight(dY2, Xq, d)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int32), a[1].view(torch.int32))
    assert torch.equal(b[0].view(torch.int32), b[1].view(torch.int32))
    assert d[7].item() == 0
    assert torch.equal(b[0], c)


def test_backward_rejects_bad_shapes(gpu):
    dY = torch.zeros(2, 6, device="cuda")
    with pytest.raises(gpu.BitLinearError):
        gpu.bitlinear_backward_input(dY, torch.zeros(6, 16, dtype=torch.uint8, device="cuda"),
                                     torch.ones(1, device="cuda"))          # N % 4
    with pytest.raises(gpu.BitLinearError):
        gpu.bitlinear_backward_weight(torch.zeros(2, 8, device="cuda"),
                                      torch.zeros(2, 96, dtype=torch.int8, device="cuda"),
                                      torch.ones(2, device="cuda"))         # K % 64


def test_backward_split_products_are_deterministic(gpu):
    """Products split along the contraction add their partial sums in a
    fixed order: repeated calls give identical bits."""
    for M, K, N in ((64, 640, 2560), (1000, 320, 200)):
        W, X, dY = workloads.qat_problem(590 + M, M, K, N)
        Wp, g = gpu.quant_weight_absmean_pack(W.cuda())
        Xq, d = gpu.quant_act_absmax_i8(X.cuda())
        dYc = dY.cuda()
        a = [gpu.bitlinear_backward_input(dYc, Wp, g) for _ in range(3)]
        b = [gpu.bitlinear_backward_weight(dYc, Xq, d) for _ in range(3)]
        torch.cuda.synchronize()
        for r in (1, 2):
            assert torch.equal(a[0].view(torch.int32), a[r].view(torch.int32))
            assert torch.equal(b[0].view(torch.int32), b[r].view(torch.int32))
