"""GPU parity of the five-weights-per-byte storage (bitlinear_repack_t5,
bitlinear_gemv_t5) against the oracle: repacking is byte-exact, and the
product's int32 accumulator and fp32 output are bit-exact (the same values
as the 2-bit product on the same ternary weights).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

CANARY = 77


def _random_wp(seed, N, K):
    """Random 2-bit rows [N, K/4]: every byte value, code 3 included."""
    g = workloads.generator(seed)
    return torch.randint(0, 256, (N, K // 4), generator=g, dtype=torch.int32).to(torch.uint8)


def _repack(gpu, Wp, K):
    N = Wp.shape[0]
    rb = gpu.t5_row_bytes(K)
    buf = torch.full((N * rb + 256,), CANARY, dtype=torch.uint8, device="cuda")
    Wt5 = buf[:N * rb].view(N, rb)
    gpu.bitlinear_repack_t5(Wp.cuda(), K, Wt5=Wt5)
    torch.cuda.synchronize()
    assert torch.all(buf[N * rb:] == CANARY), "write past Wt5"
    return Wt5


@pytest.mark.parametrize("N,K", [(1, 4), (3, 20), (5, 84), (33, 260), (130, 2560), (64, 6912),
                                 (7, 6916), (2, 131072)])
def test_repack_bit_exact(gpu, N, K):
    Wp = _random_wp(1000 + K, N, K)
    Wt5 = _repack(gpu, Wp, K)
    ref = oracle.pack_t5(oracle.unpack(Wp.numpy(), K))
    assert np.array_equal(Wt5.cpu().numpy(), ref)


def _t5_case(gpu, M, K, N, seed, zero_token=False):
    g = workloads.generator(seed)
    Wp = torch.randint(0, 256, (N, K // 4), generator=g, dtype=torch.int32).to(torch.uint8)
    Xq = torch.randint(-127, 128, (M, K), generator=g, dtype=torch.int32).to(torch.int8)
    d = torch.rand(M, generator=g, dtype=torch.float32) * 0.05
    if zero_token:
        Xq[0] = 0
        d[0] = 0.0
    gamma = torch.tensor([0.0137], dtype=torch.float32)
    Wt5 = _repack(gpu, Wp, K)
    Y = torch.full((M * N + 64,), float(CANARY), dtype=torch.float32, device="cuda")
    acc = torch.full((M * N + 64,), CANARY, dtype=torch.int32, device="cuda")
    gpu.bitlinear_gemv_t5(Xq.cuda(), d.cuda(), Wt5, gamma.cuda(), Y=Y[:M * N].view(M, N),
                          acc=acc[:M * N].view(M, N))
    torch.cuda.synchronize()
    assert torch.all(Y[M * N:] == CANARY) and torch.all(acc[M * N:] == CANARY), "write past Y"
    acc_ref = oracle.ternary_acc(Xq.numpy(), Wp.numpy(), K)
    Y_ref = oracle.dequant_f32(acc_ref, d.numpy(), gamma.numpy()[0])
    assert np.array_equal(acc[:M * N].view(M, N).cpu().numpy(), acc_ref)
    Yg = Y[:M * N].view(M, N).cpu().numpy()
    assert np.array_equal(Yg.view(np.uint32), Y_ref.view(np.uint32))
    return Wp, Xq, d, gamma, Yg


@pytest.mark.parametrize("M,K,N", [
    (1, 4, 1), (1, 20, 7), (2, 84, 33), (3, 260, 65), (5, 2560, 130), (8, 6912, 97),
    (4, 6916, 50),                      # K % 5 != 0: a partial last byte
    (1, 65520, 9),                      # the largest K one token stages
    (8, 8160, 5),                       # the largest K eight tokens stage
    (6, 1280, 300),                     # M in the 8-token tile, ragged rows per workgroup
], ids=lambda v: str(v))
def test_gemv_t5_bit_exact(gpu, M, K, N):
    _t5_case(gpu, M, K, N, 2000 + K + N)


def test_gemv_t5_zero_token(gpu):
    _, _, _, _, Y = _t5_case(gpu, 3, 2560, 64, 7, zero_token=True)
    assert np.all(Y[0] == 0.0)


@pytest.mark.parametrize("shape", workloads.DECODE_SHAPES, ids=lambda s: s.name)
def test_gemv_t5_decode_shapes_equal_2bit(gpu, shape):
    """The decode shapes at full size, weights from the GPU quantiser: the
    five-per-byte product returns exactly the 2-bit product's outputs."""
    W, X = workloads.bitlinear_problem(40 + shape.N, 1, shape.K, shape.N)
    Wp, g = gpu.quant_weight_absmean_pack(W.cuda())
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    Wt5 = gpu.bitlinear_repack_t5(Wp)
    Y2, a2 = gpu.bitlinear_gemv(Xq, d, Wp, g, want_acc=True)
    Y5, a5 = gpu.bitlinear_gemv_t5(Xq, d, Wt5, g, want_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(a2, a5)
    assert torch.equal(Y2.view(torch.int32), Y5.view(torch.int32))
    rows = np.arange(0, shape.N, 97)
    acc_ref = oracle.ternary_acc(Xq.cpu().numpy(), Wp.cpu().numpy()[rows], shape.K)
    assert np.array_equal(a5.cpu().numpy()[:, rows], acc_ref)


def test_gemv_t5_rejects(gpu):
    Wp = _random_wp(5, 4, 64)
    Wt5 = gpu.bitlinear_repack_t5(Wp.cuda())
    d = torch.ones(9, device="cuda")
    g = torch.ones(1, device="cuda")
    with pytest.raises(gpu.BitLinearError):                          # M > 8
        gpu.bitlinear_gemv_t5(torch.zeros(9, 64, dtype=torch.int8, device="cuda"), d, Wt5, g)
    big = gpu.bitlinear_repack_t5(_random_wp(6, 1, 8164).cuda())
    with pytest.raises(gpu.BitLinearError):                          # codes exceed 64 KiB
        gpu.bitlinear_gemv_t5(torch.zeros(8, 8164, dtype=torch.int8, device="cuda"), d[:8],
                              big, g)
    with pytest.raises(ValueError):                                  # row length
        gpu.bitlinear_gemv_t5(torch.zeros(1, 128, dtype=torch.int8, device="cuda"), d[:1],
                              Wt5, g)


def test_gemv_t5_graph_replays_match_eager(gpu):
    """Repack + product captured in a HIP graph, replayed three times with
    eager work between the replays: every replay equals the eager result."""
    W, X = workloads.bitlinear_problem(77, 3, 2560, 640)
    Wp, g = gpu.quant_weight_absmean_pack(W.cuda())
    Xq, d = gpu.quant_act_absmax_i8(X.cuda())
    Wt5 = gpu.bitlinear_repack_t5(Wp)
    Y_eager = gpu.bitlinear_gemv_t5(Xq, d, Wt5, g)
    torch.cuda.synchronize()
    Wt5_g = torch.empty_like(Wt5)
    Y_g = torch.empty_like(Y_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            gpu.bitlinear_repack_t5(Wp, Wt5=Wt5_g, stream=side)
            gpu.bitlinear_gemv_t5(Xq, d, Wt5_g, g, Y=Y_g, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        Wt5_g.zero_()
        Y_g.fill_(float(CANARY))
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(Wt5_g, Wt5)
        assert torch.equal(Y_g.view(torch.int32), Y_eager.view(torch.int32))
        gpu.bitlinear_gemv_t5(Xq, d, Wt5, g)                 # eager work between replays
        torch.cuda.synchronize()
