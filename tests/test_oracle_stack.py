"""Pins for the oracle's decode-stack composition (oracle.decode_stack).

The stack chains BitLinears that are pinned on their own elsewhere.  These
tests pin what the composition adds: which vector feeds which projection, the
query-head grouping of the one-key attention stand-in, the fp32 residual
adds, the order of the trace, and the fp32 FFN output that feeds the next
layer.  Each expected value comes from a property fixed by the construction,
not from the oracle's own code.
"""
import numpy as np
import pytest

import oracle
import workloads

H, KV, F, D = 128, 64, 256, 32          # 4 query heads, 2 key/value heads


def _layer(W, gain=None):
    L = {}
    for name, g in zip(("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd"),
                       ("gq", "gk", "gv", "go", "gg", "gu", "gd")):
        L[name], L[g] = oracle.quantize_weight(W[name])
    L["ffn_norm"] = gain
    return L


def _random(seed, layer=0):
    return {k: v.numpy().astype(np.float64)
            for k, v in workloads.stack_layer_weights(seed, layer, H, KV, F).items()}


def _segments(row):
    cuts = np.cumsum([H, H, KV, KV, H, H, H])
    names = ("x_in", "q", "k", "v", "o", "x_mid", "y")
    parts = np.split(row, cuts[:-1])
    assert cuts[-1] == 5 * H + 2 * KV
    return dict(zip(names, parts))


def test_expand_heads_by_hand():
    # 4 query heads of size 2 share 2 key/value heads: heads 0, 1 read kv head
    # 0 and heads 2, 3 read kv head 1.
    v = np.array([1, 2, 3, 4], dtype=np.float32)
    got = oracle.expand_heads(v, H=8, D=2)
    assert got.tolist() == [1, 2, 1, 2, 3, 4, 3, 4]
    # one key/value head per query head: the identity
    assert oracle.expand_heads(v, H=4, D=2).tolist() == [1, 2, 3, 4]


def test_zero_weights_leave_the_stream_unchanged():
    # All-zero weights quantise to all-zero codes: every BitLinear gives 0,
    # the FFN's H is 0 (a zero row, whose down projection is 0), so both
    # residual adds return x bit for bit.
    W = {k: np.zeros_like(v) for k, v in _random(0).items()}
    x0 = workloads.stack_token(0, H).numpy()
    x, trace = oracle.decode_stack(x0, [_layer(W), _layer(W)], H, KV, F, D, 1e-5)
    assert np.array_equal(x.view(np.uint32), x0.view(np.uint32))
    for row in trace:
        s = _segments(row)
        assert np.array_equal(s["x_in"], x0) and np.array_equal(s["x_mid"], x0)
        for k in ("q", "k", "v", "o", "y"):
            assert not s[k].any(), k


def _identity_value_path(seed):
    """A layer whose v-projection copies x[:KV] and whose o-projection copies
    its input (ternary identities with gamma exactly 1), with random q, k,
    gate, up and a zero down projection."""
    W = _random(seed)
    W["Wv"] = np.zeros((KV, H))
    W["Wv"][np.arange(KV), np.arange(KV)] = H      # mean |W| = KV*H/(KV*H) = 1
    W["Wo"] = H * np.eye(H)                          # mean |W| = 1
    W["Wd"] = np.zeros((H, F))
    return W


def test_value_path_copies_grouped_heads():
    # With the identities above, v = x[:KV] and o = expand(v), each up to one
    # int8 quantisation step (half the scale amax/127 per rounding), and the
    # zero down projection makes y = 0.  The layer's output is therefore
    # x + expand(x[:KV]) within those two half-steps: a wrong head index, a
    # wrong input to v or o, or a missing residual add all break it.
    W = _identity_value_path(3)
    x0 = workloads.stack_token(3, H).numpy()
    x, trace = oracle.decode_stack(x0, [_layer(W)], H, KV, F, D, 1e-5)
    s = _segments(trace[0])
    d_x = np.abs(x0).max() / 127.0
    assert np.max(np.abs(s["v"] - x0[:KV])) <= 0.5 * d_x * (1 + 1e-6)
    a = np.concatenate([x0[:KV][(h // 2) * D:(h // 2 + 1) * D] for h in range(H // D)])
    d_a = np.abs(s["v"]).max() / 127.0
    bound = 0.5 * d_x + 0.5 * d_a + 1e-6 * np.abs(x0).max()
    assert np.max(np.abs(s["o"] - a)) <= bound
    assert not s["y"].any()
    assert np.max(np.abs(x - (x0 + a))) <= bound * (1 + 1e-5)
    assert np.array_equal(s["x_in"], x0)


def test_ffn_output_matches_the_fp64_tail():
    # With o = 0 the FFN sees x itself; its fp32 output must equal the fp64
    # FFN tail's Y up to fp32 rounding of the rescale (a few ulp).
    W = _random(5)
    W["Wo"] = np.zeros((H, H))
    gain = workloads.stack_norm_gain(5, 0, F).numpy()
    L = _layer(W, gain)
    x0 = workloads.stack_token(5, H).numpy()
    x, trace = oracle.decode_stack(x0, [L], H, KV, F, D, 1e-5)
    s = _segments(trace[0])
    Xq, d = oracle.quant_act(x0[None, :])
    ref = oracle.ffn_relu2(Xq, d, L["Wg"], L["gg"], L["Wu"], L["gu"], gain, 1e-5,
                           L["Wd"], L["gd"], H, F, H)
    assert np.any(ref["Y"] != 0)
    np.testing.assert_allclose(s["y"], ref["Y"][0], rtol=1e-6, atol=0)
    np.testing.assert_array_equal(s["x_mid"], x0)


@pytest.mark.parametrize("n_layers", [3])
def test_trace_chains_fp32_residual_adds(n_layers):
    layers = [_layer(_random(7, l), workloads.stack_norm_gain(7, l, F).numpy())
              for l in range(n_layers)]
    x0 = workloads.stack_token(7, H).numpy()
    x, trace = oracle.decode_stack(x0, layers, H, KV, F, D, 1e-5)
    assert trace.shape == (n_layers, 5 * H + 2 * KV) and trace.dtype == np.float32
    prev = x0
    for row in trace:
        s = _segments(row)
        assert np.array_equal(s["x_in"], prev)
        assert np.array_equal(s["x_mid"], (s["x_in"] + s["o"]).astype(np.float32))
        prev = (s["x_mid"] + s["y"]).astype(np.float32)
        for k in ("q", "k", "v", "o", "y"):
            assert np.abs(s[k]).max() > 0, k
    assert np.array_equal(x, prev)
