"""GPU parity of the 4-bit activation path (BitNet a4.8: "Microsoft BitNet
深度研究报告", §3 论文演进时间线 and §10 关键资源) against the oracle:
quant_act_absmax_i4 (codes, packed bytes and scales bit-exact) and
bitlinear_a4 (int32 accumulators and fp32 outputs bit-exact: Y equals the
oracle's fp32 rescale of its own accumulators; and within 1e-3 of the fp64
value), through every product kernel the call dispatches to: the decode
kernel (M <= 8, with its LDS chunking past 64 KiB of staged codes), the
16x16x64 MFMA tiles (8 < M < 128) and both 32x32x32 MFMA tile shapes
(M >= 128, N below and above 4096), with ragged M, N and K.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

RTOL = 1e-3
CANARY = -12345.678


def _bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def _ref4(X):
    if X.dtype == torch.bfloat16:
        x32 = oracle.bf16_to_f32(workloads.bf16_bits(X))
    else:
        x32 = X.numpy()
    q, d = oracle.quant_act4(x32)
    return q, d, oracle.pack_act4(q)


@pytest.mark.parametrize("M,K,dtype,seed", [
    (4, 256, torch.float32, 0), (1, 2560, torch.bfloat16, 1), (1, 6912, torch.bfloat16, 2),
    (64, 6912, torch.bfloat16, 3), (2048, 2560, torch.bfloat16, 4), (3, 258, torch.float32, 5),
    (5, 262, torch.bfloat16, 6), (2, 2, torch.float32, 7), (3, 8200, torch.bfloat16, 8)])
def test_quant_act4_bit_exact(gpu, M, K, dtype, seed):
    X = workloads.activations(workloads.generator(900 + seed), M, K, dtype=dtype)
    if M > 1:
        X[1] = 0
    P, d = gpu.quant_act_absmax_i4(X.cuda())
    torch.cuda.synchronize()
    q_ref, d_ref, P_ref = _ref4(X)
    assert np.array_equal(P.cpu().numpy(), P_ref)
    assert np.array_equal(_bits(d.cpu().numpy()), _bits(d_ref))


def test_quant_act4_golden(gpu):
    with open(os.path.join(os.path.dirname(__file__), "golden", "handworked.json")) as f:
        cases = json.load(f)["activations4"]
    for c in cases:
        P, d = gpu.quant_act_absmax_i4(torch.tensor(c["X"], dtype=torch.float32).cuda())
        torch.cuda.synchronize()
        assert P.cpu().tolist() == c["P"], c["derivation"]
        assert d.cpu().tolist() == c["d"], c["derivation"]


def _a4_case(gpu, M, K, N, seed, dtype=torch.bfloat16):
    W, X = workloads.bitlinear_problem(1000 + seed, M, K, N, dtype=dtype)
    Wp, g = gpu.quant_weight_absmean_pack(W.cuda())
    P, d = gpu.quant_act_absmax_i4(X.cuda())
    Ybuf = torch.full((M * N + 256,), CANARY, dtype=torch.float32, device="cuda")
    Abuf = torch.full((M * N + 256,), -7, dtype=torch.int32, device="cuda")
    Y, acc = Ybuf[:M * N].view(M, N), Abuf[:M * N].view(M, N)
    gpu.bitlinear_a4(P, d, Wp, g, Y=Y, acc=acc)
    torch.cuda.synchronize()
    assert torch.all(Ybuf[M * N:] == CANARY) and torch.all(Abuf[M * N:] == -7), "write past the output"
    q_ref, d_ref, P_ref = _ref4(X)
    assert np.array_equal(P.cpu().numpy(), P_ref)
    Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
    assert np.array_equal(Wp.cpu().numpy(), Wp_ref)
    acc_ref, Y_ref = oracle.bitlinear_a4(P_ref, d_ref, Wp_ref, g_ref, K)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    Y32 = oracle.dequant_f32(acc_ref, d_ref, g_ref)
    assert np.array_equal(_bits(Y.cpu().numpy()), _bits(Y32))
    err = np.abs(Y.cpu().numpy().astype(np.float64) - Y_ref)
    assert np.all(err <= RTOL * np.abs(Y_ref))


@pytest.mark.parametrize("shape", workloads.DECODE_SHAPES, ids=lambda s: s.name)
def test_a4_decode_shapes(gpu, shape):
    _a4_case(gpu, 1, shape.K, shape.N, shape.N)


@pytest.mark.parametrize("M,K,N", [
    (2, 2560, 640), (3, 320, 641), (5, 6912, 97), (8, 12288, 50), (1, 64, 1), (7, 4096, 65),
    (9, 2560, 130), (33, 576, 97), (127, 64, 33), (64, 6912, 300),
    (128, 192, 131), (300, 2560, 700), (257, 640, 4200), (513, 128, 257)],
    ids=lambda v: str(v))
def test_a4_kernel_paths(gpu, M, K, N):
    _a4_case(gpu, M, K, N, M + N)


def test_a4_tiny_fp32(gpu):
    t = workloads.TINY
    _a4_case(gpu, t["M"], t["K"], t["N"], 5, dtype=torch.float32)


@pytest.mark.parametrize("K,N", [(2560, 6912), (6912, 2560)], ids=["gate_up", "down"])
def test_a4_prefill_full_size(gpu, K, N):
    """M = 2048 at both prefill shapes; every output is compared."""
    _a4_case(gpu, workloads.PREFILL["M"], K, N, 7 + K)


def test_a4_zero_token_and_empty(gpu):
    W, X = workloads.bitlinear_problem(1500, 3, 256, 64, dtype=torch.float32)
    X[1] = 0
    Wp, g = gpu.quant_weight_absmean_pack(W.cuda())
    P, d = gpu.quant_act_absmax_i4(X.cuda())
    Y = gpu.bitlinear_a4(P, d, Wp, g)
    torch.cuda.synchronize()
    assert d[1].item() == 0 and not P[1].any() and not Y[1].any()
    P0 = torch.zeros(0, 128, dtype=torch.uint8, device="cuda")
    assert gpu.bitlinear_a4(P0, torch.zeros(0, device="cuda"), Wp, g).shape == (0, 64)
