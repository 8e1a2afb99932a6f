"""Pins of the oracle's 4-bit activation path (BitNet a4.8: "Microsoft BitNet
深度研究报告", §3 论文演进时间线, row 2024-11, and §10 关键资源), CPU only.

The pages give the name and "activations at 4 bits" only; the reading (absmax
to [-7, 7], s = 7/a, d = a/7, two codes per byte, low nibble first) is pinned
here by values worked by hand, exact rational arithmetic, invariants of the
rule, every byte value of the storage, and the product against an int64
matmul.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked.json")


def test_golden_activations4():
    with open(GOLDEN) as f:
        cases = json.load(f)["activations4"]
    for c in cases:
        X = np.array(c["X"], dtype=np.float32)
        q, d = oracle.quant_act4(X)
        assert q.tolist() == c["q"], c["derivation"]
        assert d.tolist() == c["d"], c["derivation"]
        P = oracle.pack_act4(q)
        assert P.tolist() == c["P"], c["derivation"]
        assert oracle.unpack_act4(P, X.shape[1]).tolist() == c["q"]


def _rne(t):
    return round(t)          # Fraction: round half to even


def _inputs():
    g = workloads.generator(77)
    X = workloads.activations(g, 6, 2560).float().numpy()
    X[2] = 0.0
    X[3, :] = np.float32(1e-30) * np.arange(2560, dtype=np.float32)   # tiny magnitudes
    return X


def test_act4_against_exact_rational():
    """q = rne(7 x / a) in exact arithmetic except within 2^-20 of a half
    (where the fp32 product may fall on either side); |7x/a - q| <= 1/2."""
    X = _inputs()
    q, d = oracle.quant_act4(X)
    near = 0
    for m in range(X.shape[0]):
        a = max(Fraction(float(v)) for v in np.abs(X[m]))
        if a == 0:
            assert not q[m].any() and d[m] == 0
            continue
        for k in range(0, X.shape[1], 7):
            t = Fraction(float(X[m, k])) * 7 / a
            ex = max(-7, min(7, _rne(t)))
            if q[m, k] != ex:
                frac = abs(t - (t.numerator // t.denominator)) - Fraction(1, 2)
                assert abs(frac) < Fraction(1, 2 ** 20), (m, k, float(t), q[m, k])
                near += 1
            assert abs(t - int(q[m, k])) <= Fraction(1, 2) + Fraction(1, 2 ** 20)
    assert near <= 2


def test_act4_invariants():
    X = _inputs()
    q, d = oracle.quant_act4(X)
    assert q.min() >= -7 and q.max() <= 7
    for m in range(X.shape[0]):
        if d[m] == 0:
            continue
        k = int(np.argmax(np.abs(X[m])))
        assert abs(int(q[m, k])) == 7                      # the absmax element maps to +-7
        assert d[m] == np.float32(np.float32(np.abs(X[m]).max()) / np.float32(7))
    qn, dn = oracle.quant_act4(-X)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d)
    q2, d2 = oracle.quant_act4(X * np.float32(4))             # exact power-of-two scaling
    assert np.array_equal(q2, q) and np.array_equal(d2, d * np.float32(4))


def test_act4_storage_every_byte():
    P = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = oracle.unpack_act4(P, 512)
    for b in range(256):
        lo, hi = b & 15, b >> 4
        assert q[0, 2 * b] == (lo if lo < 8 else lo - 16)
        assert q[0, 2 * b + 1] == (hi if hi < 8 else hi - 16)
    assert np.array_equal(oracle.pack_act4(q), P)


def test_act4_product_against_int64_matmul():
    g = workloads.generator(78)
    W = workloads.weight(g, 96, 320).numpy()
    X = workloads.activations(g, 5, 320).float().numpy()
    Wp, gam = oracle.quantize_weight(W)
    q, d = oracle.quant_act4(X)
    P = oracle.pack_act4(q)
    acc, Y = oracle.bitlinear_a4(P, d, Wp, gam, 320)
    ref = q.astype(np.int64) @ oracle.unpack(Wp, 320).astype(np.int64).T
    assert np.array_equal(acc, ref)
    Yref = ref.astype(np.float64) * float(gam) * d.astype(np.float64)[:, None]
    assert np.all(np.abs(Y - Yref) <= 1e-12 * np.abs(Yref) + 1e-300)
