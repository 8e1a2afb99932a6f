"""The allocation-free weight quantiser (quant_weight_absmean_pack_noalloc)
against quant_weight_absmean_pack, the entry point whose kernels it shares,
and against the oracle.

Its block sums live in a library-owned device array that every call on the
GPU reuses, so the cases run one after another on the same array: a large
call, then smaller ones (which must not see the larger call's leftovers), the
largest size the array takes, and replays from a HIP graph.  Packed bytes and
gamma's bits must be identical to the workspace entry point's and to the
oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _bits(g):
    return np.float32(g.item()).view(np.uint32)


def _both(gpu, W):
    N, K = W.shape
    Wp = torch.full((N, K // 4), 0xEE, dtype=torch.uint8, device="cuda")
    g = torch.full((1,), -1.0, device="cuda")
    gpu.quant_weight_absmean_pack_noalloc(W, Wp=Wp, gamma=g)
    Wp_ws, g_ws = gpu.quant_weight_absmean_pack(W)
    torch.cuda.synchronize()
    assert torch.equal(Wp, Wp_ws)
    assert _bits(g) == _bits(g_ws)
    return Wp, g


@pytest.mark.parametrize("seed", [0])
def test_noalloc_matches_workspace_call_then_smaller(gpu, seed):
    """Two calls in a row on the shared scratch, the second smaller."""
    for N, K, s in ((6912, 2560, seed + 1), (67, 260, seed + 2), (1, 4, seed + 3)):
        W = workloads.weight(workloads.generator(s), N, K)
        Wp, g = _both(gpu, W.cuda())
        Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
        assert np.array_equal(Wp.cpu().numpy(), Wp_ref)
        assert _bits(g) == np.float32(g_ref).view(np.uint32)


def test_noalloc_largest_size_and_limit(gpu):
    """N * K = 2^27 fills the scratch array exactly; one more row is refused
    before anything is launched."""
    N, K = 32768, 4096
    W = workloads.weight(workloads.generator(9), N, K)
    Wp, g = _both(gpu, W.cuda())
    Wp_ref, g_ref = oracle.quantize_weight(W.numpy())
    assert np.array_equal(Wp.cpu().numpy(), Wp_ref)
    assert _bits(g) == np.float32(g_ref).view(np.uint32)
    del W, Wp
    big = torch.zeros((N + 1, K), dtype=torch.float32, device="cuda")
    gam = torch.full((1,), 5.0, device="cuda")
    with pytest.raises(gpu.BitLinearError) as e:
        gpu.quant_weight_absmean_pack_noalloc(big, gamma=gam)
    assert e.value.status == 2                       # BL_ERR_SHAPE
    torch.cuda.synchronize()
    assert gam.item() == 5.0                         # nothing launched


def test_noalloc_empty_and_golden(gpu):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "handworked.json")) as f:
        cases = json.load(f)["weights"]
    for c in cases:
        W = torch.tensor(c["W"], dtype=torch.float32, device="cuda")
        Wp, g = _both(gpu, W)
        assert g.item() == c["gamma"], c["derivation"]
        assert Wp.cpu().tolist() == c["Wp"], c["derivation"]
    g = torch.full((1,), 7.0, device="cuda")
    gpu.quant_weight_absmean_pack_noalloc(torch.zeros((0, 64), device="cuda"),
                                          Wp=torch.zeros((0, 16), dtype=torch.uint8, device="cuda"),
                                          gamma=g)
    torch.cuda.synchronize()
    assert g.item() == 0.0


def test_noalloc_graph_replays(gpu):
    """Captured in a HIP graph (the call allocates nothing, so it can be) and
    replayed with eager work between the replays: every replay gives the
    eager result."""
    N, K = 2560, 2560
    W0 = workloads.weight(workloads.generator(21), N, K).cuda()
    W1 = workloads.weight(workloads.generator(22), N, K).cuda()
    Wp_ref0, g_ref0 = gpu.quant_weight_absmean_pack(W0)
    Wp_ref1, g_ref1 = gpu.quant_weight_absmean_pack(W1)
    W = W0.clone()
    Wp = torch.empty((N, K // 4), dtype=torch.uint8, device="cuda")
    g = torch.empty((1,), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gpu.quant_weight_absmean_pack_noalloc(W, Wp=Wp, gamma=g, stream=s)     # warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu.quant_weight_absmean_pack_noalloc(W, Wp=Wp, gamma=g,
                                              stream=torch.cuda.current_stream())
    for i in range(4):
        src, Wp_ref, g_ref = (W0, Wp_ref0, g_ref0) if i % 2 == 0 else (W1, Wp_ref1, g_ref1)
        W.copy_(src)
        Wp.fill_(0xEE)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Wp, Wp_ref) and _bits(g) == _bits(g_ref)
        _ = (W0 * 2).sum().item()                   # eager work between replays
