"""Pins for the oracle's QAT backward (oracle.backward_input / backward_weight).

The straight-through estimator makes the backward the adjoint of the forward's
linear map at the quantised operands.  The pins check exactly that, against
the forward oracle's own int32 accumulation (the C ternary_acc, a separate
code path), plus the special cases the definitions fix.  Nothing here re-types
the backward's formula.
"""
import numpy as np

import oracle


def _ternary(seed, N, K):
    rng = np.random.default_rng(seed)
    W = rng.normal(0.0, 0.02, (N, K)).astype(np.float32)
    return oracle.quantize_weight(W)


def test_backward_input_is_the_adjoint_of_the_forward():
    """<dY, gamma * (Xq Wq^T)> == <dX, Xq> for every Xq: pins orientation,
    the ternary decode and the gamma factor of dX."""
    M, N, K = 5, 48, 320
    Wp, g = _ternary(1, N, K)
    rng = np.random.default_rng(2)
    dY = rng.normal(size=(M, N)).astype(np.float32)
    dX = oracle.backward_input(dY, Wp, g, K)
    assert dX.shape == (M, K)
    for s in range(3):
        Xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
        acc = oracle.ternary_acc(Xq, Wp, K).astype(np.float64)        # Xq Wq^T, exact
        lhs = np.sum(dY.astype(np.float64) * float(g) * acc)
        rhs = np.sum(dX * Xq.astype(np.float64))
        assert abs(lhs - rhs) <= 1e-9 * np.sum(np.abs(dY)) * 127 * K * float(g)


def test_backward_weight_is_the_adjoint_of_the_forward():
    """<dY, (Xq d) Wq^T> == <dW, Wq> for every ternary Wq: pins the
    orientation of dW and the per-token scale d."""
    M, N, K = 6, 40, 256
    rng = np.random.default_rng(3)
    X = rng.normal(size=(M, K)).astype(np.float32)
    Xq, d = oracle.quant_act(X)
    dY = rng.normal(size=(M, N)).astype(np.float32)
    dW = oracle.backward_weight(dY, Xq, d)
    assert dW.shape == (N, K)
    for s in range(3):
        Wp, g = _ternary(10 + s, N, K)
        Wq = oracle.unpack(Wp, K).astype(np.float64)
        acc = oracle.ternary_acc(Xq, Wp, K).astype(np.float64)        # Xq Wq^T, exact
        lhs = np.sum(dY.astype(np.float64) * d.astype(np.float64)[:, None] * acc)
        rhs = np.sum(dW * Wq)
        assert abs(lhs - rhs) <= 1e-9 * np.sum(np.abs(dY)) * 127 * K * float(np.max(d))


def test_backward_special_cases():
    M, N, K = 3, 8, 64
    rng = np.random.default_rng(4)
    dY = rng.normal(size=(M, N)).astype(np.float32)
    # W = +c everywhere: gamma = c, Wq = +1, so every dX[m, k] = c * sum_n dY[m, n]
    c = np.float32(0.015625)
    Wp, g = oracle.quantize_weight(np.full((N, K), c, dtype=np.float32))
    assert np.float32(g) == c
    dX = oracle.backward_input(dY, Wp, g, K)
    row = float(c) * dY.astype(np.float64).sum(axis=1)
    assert np.allclose(dX, np.repeat(row[:, None], K, axis=1), rtol=1e-12, atol=0)
    # W = 0: gamma = 0 and no gradient reaches X
    Wp0, g0 = oracle.quantize_weight(np.zeros((N, K), dtype=np.float32))
    assert not oracle.backward_input(dY, Wp0, g0, K).any()
    # an all-zero token (d = 0, Xq = 0) contributes nothing to dW; dW is
    # linear in dY, so doubling dY doubles dW exactly
    X = rng.normal(size=(M, K)).astype(np.float32)
    X[1] = 0
    Xq, d = oracle.quant_act(X)
    assert d[1] == 0 and not Xq[1].any()
    dW = oracle.backward_weight(dY, Xq, d)
    dY2 = dY.copy()
    dY2[1] = 1000.0
    assert np.array_equal(oracle.backward_weight(dY2, Xq, d), dW)
    assert np.array_equal(oracle.backward_weight(2 * dY, Xq, d), 2 * dW)
