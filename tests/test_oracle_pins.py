"""Pins for the CPU oracle: each test checks the oracle against something other
than itself -- values worked by hand from the printed formulas, closed forms,
exact rational arithmetic, a library routine (numpy int64 / fp64 matmul,
torch's bf16 conversion), brute force over every small input, and the
statistics a Gaussian weight matrix must show.  A plausible slip in the oracle
(a dropped term, a wrong sign, index or threshold, a transposed operand, a
wrong bit order or code) fails at least one of them.

Runs on the CPU only (no GPU marker).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ------------------------------------------------------------------ golden
def test_golden_weights(golden):
    for case in golden["weights"]:
        W = np.array(case["W"], dtype=np.float32)
        g = oracle.absmean_gamma(W)
        assert g == np.float32(case["gamma"]), case["derivation"]
        Wq = oracle.ternarize(W, g)
        assert Wq.tolist() == case["Wq"], case["derivation"]
        Wp = oracle.pack(Wq)
        assert Wp.tolist() == case["Wp"], case["derivation"]
        assert oracle.unpack(Wp, W.shape[1]).tolist() == case["Wq"]


def test_golden_activations(golden):
    for case in golden["activations"]:
        X = np.array(case["X"], dtype=np.float32)
        Xq, d = oracle.quant_act(X)
        assert Xq.tolist() == case["Xq"], case["derivation"]
        assert d.tolist() == case["d"], case["derivation"]


def test_golden_accumulate(golden):
    for case in golden["accumulate"]:
        Xq = np.array(case["Xq"], dtype=np.int8)
        Wq = np.array(case["Wq"], dtype=np.int8)
        K = Xq.shape[1]
        acc = oracle.ternary_acc(Xq, oracle.pack(Wq), K)
        assert acc.tolist() == case["acc"], case["derivation"]


# ------------------------------------------------------------ weight quant
def test_constant_magnitude_closed_form():
    """|W| == c with random signs: gamma == c exactly and Wq == sign(W)."""
    rng = np.random.default_rng(1)
    for c in (0.0173, 1.0, 3.0e-5, 123.5):
        c32 = np.float32(c)
        signs = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=(37, 64))
        W = signs * c32
        g = oracle.absmean_gamma(W)
        assert g == c32
        assert np.array_equal(oracle.ternarize(W, g), signs.astype(np.int8))


def _exact_q(w, gamma):
    """round(clamp(w / gamma, -1, 1)) in exact rational arithmetic, ties to even."""
    w, gamma = Fraction(float(w)), Fraction(float(gamma))
    if w == 0:
        return 0
    if gamma == 0:
        return 1 if w > 0 else -1
    t = max(Fraction(-1), min(Fraction(1), w / gamma))
    return round(t)          # Python's round on Fraction is half-to-even


def test_ternarize_matches_exact_rational():
    rng = np.random.default_rng(2)
    W = (rng.standard_normal(3000) * 0.02).astype(np.float32)
    g = np.float32(0.0159)
    # crafted exact ties and near ties around |w| = gamma / 2
    half = np.float32(g / 2)
    crafted = np.array([half, -half, np.nextafter(half, 1), np.nextafter(half, 0),
                        -np.nextafter(half, 1), -np.nextafter(half, 0),
                        g, -g, 2 * g, 0.0, np.float32(1e-30)], dtype=np.float32)
    W = np.concatenate([W, crafted])
    Wq = oracle.ternarize(W, g)
    expect = np.array([_exact_q(w, g) for w in W], dtype=np.int8)
    assert np.array_equal(Wq, expect)
    # tie |w| == gamma / 2 rounds to 0, just above rounds away
    assert Wq[len(W) - 11] == 0 and Wq[len(W) - 10] == 0
    assert Wq[len(W) - 9] == 1 and Wq[len(W) - 8] == 0


def test_ternarize_threshold_form_random():
    """Equivalent exact threshold: Wq = sign(w) iff 2|w| > gamma (fp64, exact)."""
    W = workloads.weight(workloads.generator(5), 300, 256).numpy()
    g = oracle.absmean_gamma(W)
    Wq = oracle.ternarize(W, g)
    w64 = W.astype(np.float64)
    expect = np.where(2 * np.abs(w64) > np.float64(g), np.sign(w64), 0).astype(np.int8)
    assert np.array_equal(Wq, expect)


def _exact_abs_sum(W):
    """sum |w| over W exactly, as a Fraction.  Every fp32 |w| is m * 2^e with
    an integer m < 2^24; the integers of one exponent are added in int64
    (exact), then the per-exponent sums as rationals."""
    a = np.abs(np.asarray(W, dtype=np.float32).astype(np.float64)).ravel()
    m, e = np.frexp(a)
    mi = np.round(m * 2.0 ** 24).astype(np.int64)
    ee = (e - 24).astype(np.int64)
    assert np.array_equal(np.ldexp(mi.astype(np.float64), ee), a)   # decomposition exact
    total = Fraction(0)
    for ev in np.unique(ee[mi != 0]):
        total += Fraction(int(mi[ee == ev].sum())) * Fraction(2) ** int(ev)
    return total


def _nearest_f32(q):
    """The fp32 nearest the rational q >= 0, ties to the even significand."""
    if q == 0:
        return np.float32(0.0)
    c = np.float32(float(q))
    cands = [np.nextafter(c, np.float32(0.0)), c, np.nextafter(c, np.float32(np.inf))]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - q), int(v.view(np.uint32)) & 1))


def _spread_weights(seed, N, K):
    """Gaussian weights times 10^u, u uniform in [-30, 30] per element."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K)) * 0.02 * 10.0 ** rng.uniform(-30, 30, size=(N, K))
    return W.astype(np.float32)


@pytest.mark.parametrize("N,K,seed,spread", [
    (512, 768, 3, False), (7, 12, 4, False), (333, 260, 5, False), (3, 20, 6, False),
    (64, 6912, 7, False), (300, 100, 8, True), (5, 2560, 9, True)])
def test_gamma_is_nearest_fp32_of_exact_mean(N, K, seed, spread):
    """The pairwise fp64 sum is within ~log2(n) * 2^-53 of the exact sum, far
    inside half an fp32 ulp: away from an fp32 midpoint gamma must be the fp32
    nearest the exact rational mean (computed here without any floating-point
    addition).  The golden cases cover inputs that sit on a midpoint."""
    W = _spread_weights(seed, N, K) if spread else workloads.weight(
        workloads.generator(seed), N, K).numpy()
    q = _exact_abs_sum(W) / (N * K)
    ref = _nearest_f32(q)
    lo, hi = np.nextafter(ref, np.float32(0.0)), np.nextafter(ref, np.float32(np.inf))
    mids = [(Fraction(float(lo)) + Fraction(float(ref))) / 2,
            (Fraction(float(ref)) + Fraction(float(hi))) / 2]
    assert min(abs(q - m) for m in mids) > q * Fraction(1, 2 ** 40)   # not a near-midpoint case
    assert oracle.absmean_gamma(W) == ref


def test_gaussian_statistics():
    """W ~ N(0, s^2): E|w| = s sqrt(2/pi); P(Wq = 0) = P(|Z| <= sqrt(2/pi)/2)
    = 2 Phi(sqrt(2/pi)/2) - 1 = 0.31006; +1 and -1 share the rest equally."""
    N, K = 256, 256
    W = workloads.weight(workloads.generator(0), N, K).numpy()
    g = float(oracle.absmean_gamma(W))
    s = workloads.W_STD
    n = N * K
    mean_abs = s * math.sqrt(2 / math.pi)
    sd_abs = s * math.sqrt(1 - 2 / math.pi) / math.sqrt(n)
    assert abs(g - mean_abs) < 4 * sd_abs
    Wq = oracle.ternarize(W, g)
    p0 = 2 * 0.5 * (1 + math.erf(math.sqrt(2 / math.pi) / 2 / math.sqrt(2))) - 1
    assert abs(p0 - 0.31006) < 1e-4
    f0 = np.mean(Wq == 0)
    fp = np.mean(Wq == 1)
    fm = np.mean(Wq == -1)
    tol = 4 * math.sqrt(p0 * (1 - p0) / n)
    assert abs(f0 - p0) < tol
    assert abs(fp - (1 - p0) / 2) < tol and abs(fm - (1 - p0) / 2) < tol


def test_pack_invariants_roundtrip():
    rng = np.random.default_rng(4)
    Wq = rng.integers(-1, 2, size=(33, 128)).astype(np.int8)
    Wp = oracle.pack(Wq)
    assert Wp.shape == (33, 32)
    codes = np.stack([(Wp >> (2 * j)) & 3 for j in range(4)], axis=-1)
    assert codes.max() <= 2                       # code 3 never written
    assert np.array_equal(oracle.unpack(Wp, 128), Wq)
    # bit order: weight 4b+j sits in bits 2j..2j+1 of byte b
    for n in range(3):
        for k in range(0, 128, 7):
            code = (int(Wp[n, k // 4]) >> (2 * (k % 4))) & 3
            assert code == {0: 0, 1: 1, -1: 2}[int(Wq[n, k])]


def test_unpack_every_byte():
    """All 256 byte values decode; code 3 reads as 0."""
    Wp = np.arange(256, dtype=np.uint8).reshape(256, 1)
    Wq = oracle.unpack(Wp, 4)
    for b in range(256):
        for j in range(4):
            c = (b >> (2 * j)) & 3
            assert Wq[b, j] == {0: 0, 1: 1, 2: -1, 3: 0}[c]


# ------------------------------------------------- five weights per byte
# Pins of the base-3 storage (oracle.c, ob_pack_t5): a bijection on the 243
# five-weight patterns, ordered with weight 5b as the most significant digit,
# decoded identically by an independent method (repeated multiplication of
# the byte, read as a fraction of 256, by 3: the integer part of each product
# is the next digit), 16-byte rows at 1.6 bits per weight, zero-weight pads.

def _t5_patterns():
    return [p for p in itertools.product((-1, 0, 1), repeat=5)]


def _digits_by_multiplication(q):
    r, out = q, []
    for _ in range(5):
        t = 3 * r
        out.append(t >> 8)
        r = t & 255
    return out


def test_t5_every_pattern_is_a_distinct_ordered_byte():
    pats = _t5_patterns()                         # lexicographic, first weight most significant
    Wq = np.array(pats, dtype=np.int8)            # [243, 5]
    Wt5 = oracle.pack_t5(Wq)
    assert Wt5.shape == (243, 16)
    q = Wt5[:, 0].astype(int)
    assert len(set(q.tolist())) == 243            # injective
    assert np.all(np.diff(q) > 0)                 # order follows the base-3 value
    assert np.all(Wt5[:, 1:] == Wt5[0, 1])        # pad bytes: five zero weights
    assert np.array_equal(oracle.unpack_t5(Wt5, 5), Wq)
    for i, pat in enumerate(pats):
        assert _digits_by_multiplication(int(q[i])) == [w + 1 for w in pat]


def test_t5_every_byte_value_decodes_as_by_multiplication():
    Wt5 = np.arange(256, dtype=np.uint8).reshape(1, 256)
    Wq = oracle.unpack_t5(Wt5, 1280)
    for b in range(256):
        assert [int(w) + 1 for w in Wq[0, 5 * b:5 * b + 5]] == _digits_by_multiplication(b)


def test_t5_row_layout_and_padding():
    for K in (1, 4, 5, 6, 79, 80, 81, 2560, 6912):
        rb = oracle.t5_row_bytes(K)
        assert rb % 16 == 0 and 5 * rb >= K and 5 * rb < K + 80
    assert oracle.t5_row_bytes(2560) * 8 == 2560 * 8 // 5        # 1.6 bits per weight
    zero_byte = oracle.pack_t5(np.zeros((1, 5), dtype=np.int8))[0, 0]
    assert zero_byte == 128                       # v = 11111 base 3 = 121, ceil(256 * 121 / 243)
    rng = np.random.default_rng(11)
    for K in (7, 13, 6912):
        Wq = rng.integers(-1, 2, size=(4, K)).astype(np.int8)
        Wt5 = oracle.pack_t5(Wq)
        assert np.array_equal(oracle.unpack_t5(Wt5, K), Wq)
        # the digits past K are zero weights, in the last partial byte and after
        wide = oracle.unpack_t5(Wt5, 5 * Wt5.shape[1])
        assert np.array_equal(wide[:, :K], Wq) and np.all(wide[:, K:] == 0)
        assert np.all(Wt5[:, (K + 4) // 5:] == 128)


def test_t5_product_equals_2bit_product():
    rng = np.random.default_rng(12)
    for M, N, K in ((1, 7, 20), (3, 33, 2560), (2, 5, 6912)):
        Wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        Xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        d = rng.random(M).astype(np.float32)
        g = np.float32(0.37)
        acc2, Y2 = oracle.bitlinear(Xq, d, oracle.pack(Wq), g, K)
        acc5, Y5 = oracle.bitlinear_t5(Xq, d, oracle.pack_t5(Wq), g, K)
        assert np.array_equal(acc2, acc5)
        assert np.array_equal(acc5, Xq.astype(np.int64) @ Wq.astype(np.int64).T)
        assert np.array_equal(Y2, Y5)


# -------------------------------------------------------- activation quant
def test_bf16_widening_matches_torch():
    X = torch.randn(64, 96, generator=workloads.generator(9)).to(torch.bfloat16)
    X[0, :4] = torch.tensor([0.0, -0.0, float("inf"), 1e-40]).to(torch.bfloat16)
    got = oracle.bf16_to_f32(workloads.bf16_bits(X))
    ref = X.to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_act_quant_against_exact_rounding():
    """Xq == rne(127 x / a) computed exactly, except within 1e-4 of a .5 tie
    (where the fp32 steps s = fl(127/a), fl(x*s) may land either side)."""
    X = workloads.activations(workloads.generator(11), 16, 2560).float().numpy()
    Xq, d = oracle.quant_act(X)
    x64 = X.astype(np.float64)
    a = np.abs(x64).max(axis=1, keepdims=True)
    t = 127.0 * x64 / a
    exact = np.clip(np.round(t), -127, 127)          # numpy rounds half to even
    near_tie = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-4
    diff = Xq.astype(np.float64) != exact
    assert not np.any(diff & ~near_tie)
    assert np.all(np.abs(Xq[diff].astype(np.float64) - exact[diff]) <= 1)
    assert diff.sum() <= max(3, near_tie.sum())
    # the absmax element maps to +-127; d reproduces a
    idx = np.abs(x64).argmax(axis=1)
    assert np.all(np.abs(Xq[np.arange(16), idx]) == 127)
    assert np.allclose(d.astype(np.float64) * 127.0, a[:, 0], rtol=2e-7, atol=0)
    # dequantisation error bound |x - Xq d| <= d / 2 (+ fp32 slack)
    err = np.abs(x64 - Xq.astype(np.float64) * d[:, None].astype(np.float64))
    assert np.all(err <= d[:, None].astype(np.float64) * (0.5 + 1e-5))


def test_act_quant_symmetry_and_scaling():
    X = workloads.activations(workloads.generator(12), 8, 512).float().numpy()
    Xq, d = oracle.quant_act(X)
    Xn, dn = oracle.quant_act(-X)
    assert np.array_equal(Xn, -Xq) and np.array_equal(dn, d)
    # multiplying a token by a power of two changes only its scale
    X2 = X.copy()
    X2[3] *= 4.0
    Xq2, d2 = oracle.quant_act(X2)
    assert np.array_equal(Xq2, Xq)
    assert d2[3] == 4 * d[3] and np.array_equal(np.delete(d2, 3), np.delete(d, 3))
    assert Xq.min() >= -127 and Xq.max() <= 127


def test_act_quant_zero_row():
    X = np.zeros((2, 64), dtype=np.float32)
    X[1, 5] = -3.0
    Xq, d = oracle.quant_act(X)
    assert not Xq[0].any() and d[0] == 0
    assert Xq[1, 5] == -127 and np.count_nonzero(Xq[1]) == 1


# ------------------------------------------------------------- accumulate
def test_brute_force_k1_every_pair():
    """K = 1... padded to the 4-weight byte with zero weights: every (trit,
    int8) pair gives acc = trit * x."""
    xs = np.arange(-128, 128, dtype=np.int64)
    Xq = np.zeros((256, 4), dtype=np.int8)
    Xq[:, 0] = xs
    Xq[:, 1:] = np.int8(77)          # must be ignored: their weights are 0
    Wq = np.zeros((3, 4), dtype=np.int8)
    Wq[:, 0] = [-1, 0, 1]
    acc = oracle.ternary_acc(Xq, oracle.pack(Wq), 4)
    assert np.array_equal(acc, np.outer(xs, [-1, 0, 1]))


def test_brute_force_k4_all_trit_rows():
    """All 81 ternary rows of length 4 against 2000 random int8 rows."""
    import itertools
    Wq = np.array(list(itertools.product([-1, 0, 1], repeat=4)), dtype=np.int8)
    rng = np.random.default_rng(6)
    Xq = rng.integers(-128, 128, size=(2000, 4)).astype(np.int8)
    acc = oracle.ternary_acc(Xq, oracle.pack(Wq), 4)
    ref = Xq.astype(np.int64) @ Wq.astype(np.int64).T
    assert np.array_equal(acc, ref)


@pytest.mark.parametrize("M,K,N", [(4, 256, 256), (3, 2560, 640), (1, 6912, 96),
                                   (5, 64, 7)])
def test_acc_matches_int64_matmul(M, K, N):
    rng = np.random.default_rng(M * 1000 + N)
    Wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    Xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    acc = oracle.ternary_acc(Xq, oracle.pack(Wq), K)
    assert np.array_equal(acc, Xq.astype(np.int64) @ Wq.astype(np.int64).T)


def test_acc_special_cases():
    rng = np.random.default_rng(7)
    Xq = rng.integers(-127, 128, size=(6, 128)).astype(np.int8)
    ones = np.ones((5, 128), dtype=np.float32) * np.float32(0.3)
    Wp, g = oracle.quantize_weight(ones)                 # W = +c -> all +1
    assert g == np.float32(0.3)
    acc = oracle.ternary_acc(Xq, Wp, 128)
    assert np.array_equal(acc, np.repeat(Xq.astype(np.int64).sum(1, keepdims=True), 5, 1))
    Wp0, g0 = oracle.quantize_weight(np.zeros((5, 128), dtype=np.float32))
    assert g0 == 0 and not oracle.ternary_acc(Xq, Wp0, 128).any()
    d = np.full(6, 0.5, np.float32)
    assert not oracle.dequant_f64(oracle.ternary_acc(Xq, Wp0, 128), d, g0).any()


# --------------------------------------------------------------- dequant
def test_dequant_is_dequantised_matmul():
    """Y = (Xq d) (Wq gamma)^T computed by numpy in fp64 on dequantised operands."""
    M, K, N = 4, 256, 256
    W, X = workloads.bitlinear_problem(0, M, K, N, dtype=torch.float32, outliers=False)
    Wp, g = oracle.quantize_weight(W.numpy())
    Xq, d = oracle.quant_act(X.numpy())
    acc, Y = oracle.bitlinear(Xq, d, Wp, g, K)
    Xhat = Xq.astype(np.float64) * d[:, None].astype(np.float64)
    What = oracle.unpack(Wp, K).astype(np.float64) * np.float64(g)
    ref = Xhat @ What.T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-300)
    # the fp32 evaluation is two roundings away from the fp64 one
    Y32 = oracle.dequant_f32(acc, d, g).astype(np.float64)
    nz = Y != 0
    assert np.all(np.abs(Y32[nz] - Y[nz]) / np.abs(Y[nz]) <= 2.0 ** -23 * 1.01)
    assert np.array_equal(Y32 == 0, Y == 0)


def test_int32_to_fp32_exact_bound():
    """float(acc) is exact for |acc| <= 127 K while K <= 132104 (127 K <= 2^24)."""
    assert 127 * 132104 <= 2 ** 24 < 127 * 132105
    acc = np.array([[2 ** 24, -(2 ** 24) + 1, 877824, -877824]], dtype=np.int32)
    Y = oracle.dequant_f32(acc, np.ones(1, np.float32), np.float32(1.0))
    assert np.array_equal(Y.astype(np.int64), acc.astype(np.int64))


# -------------------------------------------------------------------- FFN
def _ffn_inputs(seed, M, K, F, N, gain=True):
    Wg, Wu, Wd, X = workloads.ffn_problem(seed, M, K, F, N, dtype=torch.float32)
    Wgp, gg = oracle.quantize_weight(Wg.numpy())
    Wup, gu = oracle.quantize_weight(Wu.numpy())
    Wdp, gd = oracle.quantize_weight(Wd.numpy())
    Xq, d = oracle.quant_act(X.numpy())
    nw = None
    if gain:
        nw = (1.0 + 0.5 * torch.randn(F, generator=workloads.generator(seed + 99))).numpy()
    return Xq, d, Wgp, gg, Wup, gu, nw, Wdp, gd


def _ffn_literal_fp64(Xq, d, Wgp, gg, Wup, gu, nw, eps, Wdp, gd, K, F):
    """The FFN as written (RMSNorm applied, then absmax requant), all in
    numpy fp64 with dense matmuls on unpacked weights."""
    x = Xq.astype(np.float64) * d[:, None].astype(np.float64)
    G = x @ (oracle.unpack(Wgp, K).astype(np.float64) * gg).T
    U = x @ (oracle.unpack(Wup, K).astype(np.float64) * gu).T if Wup is not None else 1.0
    H = np.maximum(G, 0.0) ** 2 * U
    rms = np.sqrt((H * H).mean(axis=1, keepdims=True) + eps)
    Z = H / rms * (nw.astype(np.float64) if nw is not None else 1.0)
    a = np.abs(Z).max(axis=1, keepdims=True)
    Zq = np.clip(np.round(Z * 127.0 / a), -127, 127)
    Y = (Zq * (a / 127.0)) @ (oracle.unpack(Wdp, F).astype(np.float64) * gd).T
    return Y, Zq.astype(np.int8), rms[:, 0]


@pytest.mark.parametrize("gated,gain", [(True, True), (True, False), (False, True)])
def test_ffn_against_literal_fp64(gated, gain):
    M, K, F, N = 5, 256, 384, 192
    eps = 1e-5
    Xq, d, Wgp, gg, Wup, gu, nw, Wdp, gd = _ffn_inputs(21, M, K, F, N, gain)
    if not gated:
        Wup = None
    out = oracle.ffn_relu2(Xq, d, Wgp, gg, Wup, gu, nw, eps, Wdp, gd, K, F, N)
    Y, Zq, rms = _ffn_literal_fp64(Xq, d, Wgp, gg, Wup, gu, nw, eps, Wdp, gd, K, F)
    assert np.allclose(out["rms"], rms, rtol=1e-6)
    diff = out["Hq"].astype(np.int64) - Zq.astype(np.int64)
    assert np.abs(diff).max() <= 1 and np.count_nonzero(diff) <= 0.002 * diff.size + 1
    rel = np.linalg.norm(out["Y"] - Y) / np.linalg.norm(Y)
    assert rel < 1e-3


def test_ffn_scale_invariance():
    """Doubling gamma_u doubles U and H exactly: Hq is unchanged, dh doubles,
    and (with eps = 0) rms doubles, so Y is unchanged."""
    M, K, F, N = 4, 128, 256, 128
    Xq, d, Wgp, gg, Wup, gu, nw, Wdp, gd = _ffn_inputs(22, M, K, F, N)
    a = oracle.ffn_relu2(Xq, d, Wgp, gg, Wup, gu, nw, 0.0, Wdp, gd, K, F, N)
    b = oracle.ffn_relu2(Xq, d, Wgp, gg, Wup, np.float32(2 * gu), nw, 0.0, Wdp, gd, K, F, N)
    assert np.array_equal(a["Hq"], b["Hq"])
    assert np.array_equal(b["dh"], 2 * a["dh"])
    assert np.allclose(b["Y"], a["Y"], rtol=1e-12)


def test_ffn_requant_is_act_quant_of_h():
    """With unit gain the int8 intermediate is the per-token absmax quant of H."""
    M, K, F, N = 3, 128, 256, 64
    Xq, d, Wgp, gg, Wup, gu, _, Wdp, gd = _ffn_inputs(23, M, K, F, N, gain=False)
    out = oracle.ffn_relu2(Xq, d, Wgp, gg, Wup, gu, None, 1e-5, Wdp, gd, K, F, N)
    G = oracle.dequant_f32(oracle.ternary_acc(Xq, Wgp, K), d, gg)
    U = oracle.dequant_f32(oracle.ternary_acc(Xq, Wup, K), d, gu)
    H = (np.maximum(G, 0) * np.maximum(G, 0)) * U          # fp32, same op order
    Hq, dh = oracle.quant_act(H.astype(np.float32))
    assert np.array_equal(out["Hq"], Hq) and np.array_equal(out["dh"], dh)
