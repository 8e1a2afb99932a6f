"""CPU oracle for the BitLinear W1.58A8 layer (numpy front end of oracle.c).

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
and its Python binding never import it and share no code with it.

Every function is a thin call into ``liboracle.so`` (plain C, see oracle.c for
the definition each one follows and the page passage it cites).  Arrays are
numpy; the shapes follow nn.Linear: X [M, K], W [N, K], Y [M, N].
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("BITLINEAR_ORACLE_LIB")   # mutation tests only
    if not path:
        if (not os.path.exists(_build.LIB)
                or os.path.getmtime(_build.SRC) > os.path.getmtime(_build.LIB)):
            _build.build()
        path = _build.LIB
    lib = ctypes.CDLL(path)
    lib.ob_num_threads.restype = ctypes.c_int
    lib.ob_num_threads.argtypes = []
    lib.ob_set_num_threads.restype = None
    lib.ob_set_num_threads.argtypes = [ctypes.c_int]
    lib.ob_absmean_gamma.restype = _f32
    lib.ob_absmean_gamma.argtypes = [_p, _i64, _i64]
    lib.ob_ternarize.restype = None
    lib.ob_ternarize.argtypes = [_p, _i64, _f32, _p]
    lib.ob_pack.restype = None
    lib.ob_pack.argtypes = [_p, _i64, _i64, _p]
    lib.ob_unpack.restype = None
    lib.ob_unpack.argtypes = [_p, _i64, _i64, _p]
    lib.ob_t5_row_bytes.restype = _i64
    lib.ob_t5_row_bytes.argtypes = [_i64]
    lib.ob_pack_t5.restype = None
    lib.ob_pack_t5.argtypes = [_p, _i64, _i64, _p]
    lib.ob_unpack_t5.restype = None
    lib.ob_unpack_t5.argtypes = [_p, _i64, _i64, _p]
    lib.ob_bf16_to_f32.restype = None
    lib.ob_bf16_to_f32.argtypes = [_p, _i64, _p]
    lib.ob_quant_act.restype = None
    lib.ob_quant_act.argtypes = [_p, _i64, _i64, _p, _p]
    lib.ob_quant_act4.restype = None
    lib.ob_quant_act4.argtypes = [_p, _i64, _i64, _p, _p]
    lib.ob_pack_act4.restype = None
    lib.ob_pack_act4.argtypes = [_p, _i64, _i64, _p]
    lib.ob_unpack_act4.restype = None
    lib.ob_unpack_act4.argtypes = [_p, _i64, _i64, _p]
    lib.ob_ternary_acc.restype = None
    lib.ob_ternary_acc.argtypes = [_p, _p, _i64, _i64, _i64, _p]
    lib.ob_dequant_f64.restype = None
    lib.ob_dequant_f64.argtypes = [_p, _p, _f32, _i64, _i64, _p]
    lib.ob_dequant_f32.restype = None
    lib.ob_dequant_f32.argtypes = [_p, _p, _f32, _i64, _i64, _p]
    lib.ob_ffn_relu2.restype = None
    lib.ob_ffn_relu2.argtypes = [_p, _p, _i64, _i64, _i64,
                                 _p, _f32, _p, _f32, _p, _f32,
                                 _p, _f32, _i64,
                                 _p, _p, _p, _p, _p, _p, _p, _p, _p]
    _lib = lib
    return lib


def _c(a, dtype):
    """Contiguous array of exactly ``dtype`` (copies only when needed)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return a.ctypes.data_as(_p) if a is not None else None


def num_threads():
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().ob_num_threads())


def set_num_threads(n):
    """Threads for the oracle's later parallel loops (CPU timing only)."""
    _load().ob_set_num_threads(int(n))


def absmean_gamma(W):
    """gamma = mean |W| over the whole tensor (fp64 sum, fixed order) -> float32."""
    W = _c(W, np.float32)
    N, K = W.shape
    return np.float32(_load().ob_absmean_gamma(_ptr(W), N, K))


def ternarize(W, gamma):
    """Wq = round(clamp(W / gamma, -1, 1)) -> int8 array of W's shape."""
    W = _c(W, np.float32)
    out = np.empty(W.shape, dtype=np.int8)
    _load().ob_ternarize(_ptr(W), W.size, float(np.float32(gamma)), _ptr(out))
    return out


def pack(Wq):
    """int8 ternary [N, K] -> packed codes uint8 [N, K/4]."""
    Wq = _c(Wq, np.int8)
    N, K = Wq.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    out = np.empty((N, K // 4), dtype=np.uint8)
    _load().ob_pack(_ptr(Wq), N, K, _ptr(out))
    return out


def unpack(Wp, K):
    """packed uint8 [N, K/4] -> int8 ternary [N, K]."""
    Wp = _c(Wp, np.uint8)
    N = Wp.shape[0]
    out = np.empty((N, K), dtype=np.int8)
    _load().ob_unpack(_ptr(Wp), N, K, _ptr(out))
    return out


def t5_row_bytes(K):
    """Bytes per row of the five-per-byte format (oracle.c, ob_pack_t5)."""
    return int(_load().ob_t5_row_bytes(int(K)))


def pack_t5(Wq):
    """int8 ternary [N, K] -> five weights per byte, uint8 [N, t5_row_bytes(K)]."""
    Wq = _c(Wq, np.int8)
    N, K = Wq.shape
    out = np.empty((N, t5_row_bytes(K)), dtype=np.uint8)
    _load().ob_pack_t5(_ptr(Wq), N, K, _ptr(out))
    return out


def unpack_t5(Wt5, K):
    """uint8 [N, t5_row_bytes(K)] -> int8 ternary [N, K]."""
    Wt5 = _c(Wt5, np.uint8)
    N = Wt5.shape[0]
    if Wt5.shape[1] != t5_row_bytes(K):
        raise ValueError("row length does not match K")
    out = np.empty((N, K), dtype=np.int8)
    _load().ob_unpack_t5(_ptr(Wt5), N, K, _ptr(out))
    return out


def bitlinear_t5(Xq, d, Wt5, gamma, K):
    """(acc int32 [M, N], Y float64 [M, N]) of the five-per-byte format: the
    weights decoded, then the same BitLinear product as the 2-bit format."""
    Wq = unpack_t5(Wt5, K)
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    return bitlinear(Xq, d, pack(Wq), gamma, K)


def quantize_weight(W):
    """The offline weight path: (packed uint8 [N, K/4], gamma float32)."""
    g = absmean_gamma(W)
    return pack(ternarize(W, g)), g


def bf16_to_f32(bits):
    """bf16 given as its uint16 bit patterns -> float32 (exact)."""
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    _load().ob_bf16_to_f32(_ptr(bits), bits.size, _ptr(out))
    return out


def quant_act(X):
    """Per-token absmax int8: X float32 [M, K] -> (Xq int8 [M, K], d float32 [M])."""
    X = _c(X, np.float32)
    M, K = X.shape
    Xq = np.empty((M, K), dtype=np.int8)
    d = np.empty((M,), dtype=np.float32)
    _load().ob_quant_act(_ptr(X), M, K, _ptr(Xq), _ptr(d))
    return Xq, d


def quant_act4(X):
    """Per-token absmax to signed 4-bit codes: X float32 [M, K] ->
    (codes int8 [M, K] in [-7, 7], d float32 [M])."""
    X = _c(X, np.float32)
    M, K = X.shape
    Xq = np.empty((M, K), dtype=np.int8)
    d = np.empty((M,), dtype=np.float32)
    _load().ob_quant_act4(_ptr(X), M, K, _ptr(Xq), _ptr(d))
    return Xq, d


def pack_act4(Xq):
    """int8 codes [M, K] (K even) -> two per byte, uint8 [M, K/2]."""
    Xq = _c(Xq, np.int8)
    M, K = Xq.shape
    if K % 2:
        raise ValueError("K must be even")
    out = np.empty((M, K // 2), dtype=np.uint8)
    _load().ob_pack_act4(_ptr(Xq), M, K, _ptr(out))
    return out


def unpack_act4(P, K):
    """uint8 [M, K/2] -> int8 codes [M, K] in [-8, 7]."""
    P = _c(P, np.uint8)
    M = P.shape[0]
    if P.shape[1] * 2 != K:
        raise ValueError("shape mismatch")
    out = np.empty((M, K), dtype=np.int8)
    _load().ob_unpack_act4(_ptr(P), M, K, _ptr(out))
    return out


def bitlinear_a4(P, d, Wp, gamma, K):
    """One BitLinear from 4-bit packed activation codes: (acc int32 [M, N],
    Y float64 [M, N]); the codes are unpacked, then the product and rescale
    are those of the 8-bit codes."""
    return bitlinear(unpack_act4(P, K), d, Wp, gamma, K)


def ternary_acc(Xq, Wp, K):
    """int32 acc [M, N] = Xq [M, K] . unpack(Wp)^T by add / subtract / skip."""
    Xq = _c(Xq, np.int8)
    Wp = _c(Wp, np.uint8)
    M = Xq.shape[0]
    N = Wp.shape[0]
    if Xq.shape[1] != K or Wp.shape[1] * 4 != K:
        raise ValueError("shape mismatch")
    acc = np.empty((M, N), dtype=np.int32)
    _load().ob_ternary_acc(_ptr(Xq), _ptr(Wp), M, N, K, _ptr(acc))
    return acc


def dequant_f64(acc, d, gamma):
    acc = _c(acc, np.int32)
    d = _c(d, np.float32)
    M, N = acc.shape
    Y = np.empty((M, N), dtype=np.float64)
    _load().ob_dequant_f64(_ptr(acc), _ptr(d), float(np.float32(gamma)), M, N, _ptr(Y))
    return Y


def dequant_f32(acc, d, gamma):
    acc = _c(acc, np.int32)
    d = _c(d, np.float32)
    M, N = acc.shape
    Y = np.empty((M, N), dtype=np.float32)
    _load().ob_dequant_f32(_ptr(acc), _ptr(d), float(np.float32(gamma)), M, N, _ptr(Y))
    return Y


def bitlinear(Xq, d, Wp, gamma, K):
    """One BitLinear from quantised operands: (acc int32 [M, N], Y float64 [M, N])."""
    acc = ternary_acc(Xq, Wp, K)
    return acc, dequant_f64(acc, d, gamma)


def ffn_relu2(Xq, d, Wg, gamma_g, Wu, gamma_u, norm_w, eps, Wd, gamma_d, K, F, N):
    """ReLU^2 FFN tail with subln RMSNorm and int8 requant; see oracle.c.

    Returns dict(Y=float64 [M, N], Hq=int8 [M, F], dh=float32 [M], rms=float64 [M],
    Y32=float32 [M, N]: Y as the fp32 value that feeds a later quantisation).
    """
    Xq = _c(Xq, np.int8)
    d = _c(d, np.float32)
    M = Xq.shape[0]
    Wg = _c(Wg, np.uint8)
    Wu = _c(Wu, np.uint8) if Wu is not None else None
    Wd = _c(Wd, np.uint8)
    nw = _c(norm_w, np.float32) if norm_w is not None else None
    Y = np.empty((M, N), dtype=np.float64)
    Hq = np.empty((M, F), dtype=np.int8)
    dh = np.empty((M,), dtype=np.float32)
    rms = np.empty((M,), dtype=np.float64)
    scratch = np.empty((M, max(F, N)), dtype=np.int32)
    G = np.empty((M, F), dtype=np.float32)
    U = np.empty((M, F), dtype=np.float32)
    Zp = np.empty((M, F), dtype=np.float32)
    Y32 = np.empty((M, N), dtype=np.float32)
    _load().ob_ffn_relu2(_ptr(Xq), _ptr(d), M, K, F,
                         _ptr(Wg), float(np.float32(gamma_g)),
                         _ptr(Wu), float(np.float32(gamma_u)),
                         _ptr(nw), float(eps),
                         _ptr(Wd), float(np.float32(gamma_d)), N,
                         _ptr(Y), _ptr(Hq), _ptr(dh), _ptr(rms),
                         _ptr(scratch), _ptr(G), _ptr(U), _ptr(Zp), _ptr(Y32))
    return dict(Y=Y, Hq=Hq, dh=dh, rms=rms, Y32=Y32)


def expand_heads(v, H, D):
    """Attention over a single key returns v: query head h (of H / D) reads
    key/value head h // g, g = (H / D) / (len(v) / D)."""
    v = np.asarray(v, dtype=np.float32)
    group = (H // D) // (v.shape[0] // D)
    heads = v.reshape(-1, D)
    return np.concatenate([heads[h // group] for h in range(H // D)]).astype(np.float32)


def _bitlinear_f32(x, Wp, gamma, K):
    """One M = 1 BitLinear on an fp32 activation row, output as fp32 (the
    value a later quantisation sees)."""
    Xq, d = quant_act(np.asarray(x, dtype=np.float32)[None, :])
    return dequant_f32(ternary_acc(Xq, Wp, K), d, gamma)[0]


def decode_stack(x0, layers, H, KV, F, D, eps):
    """One decode token through the layers of a BitNet b1.58 stack (the
    one-token stand-ins of attention as documented for bitlinear_decode_stack):
        q, k, v = BitLinear(x); a = expand_heads(v); o = BitLinear(a);
        x_mid = x + o; y = ffn_relu2(x_mid); x = x_mid + y.
    Every value that feeds a later per-token quantisation (q, k, v, o, y and
    the fp32 residual stream) is carried in fp32 with the rescale order of
    dequant_f32, so the int8 decisions are those of the method in that
    precision.  Returns (x_final, trace [n_layers, 5 H + 2 KV]) with the
    per-layer x_in, q, k, v, o, x_mid, y."""
    x = np.asarray(x0, dtype=np.float32).copy()
    rows = []
    for L in layers:
        q = _bitlinear_f32(x, L["Wq"], L["gq"], H)
        k = _bitlinear_f32(x, L["Wk"], L["gk"], H)
        v = _bitlinear_f32(x, L["Wv"], L["gv"], H)
        o = _bitlinear_f32(expand_heads(v, H, D), L["Wo"], L["go"], H)
        x_mid = np.add(x, o, dtype=np.float32)
        Xq, d = quant_act(x_mid[None, :])
        f = ffn_relu2(Xq, d, L["Wg"], L["gg"], L["Wu"], L["gu"], L.get("ffn_norm"), eps,
                      L["Wd"], L["gd"], H, F, H)
        y = f["Y32"][0]
        rows.append(np.concatenate([x, q, k, v, o, x_mid, y]))
        x = np.add(x_mid, y, dtype=np.float32)
    trace = np.stack(rows) if rows else np.zeros((0, 5 * H + 2 * KV), np.float32)
    return x, trace


# ------------------------------------------------------------------ QAT backward
# "Microsoft BitNet 深度研究报告", §2 (4) 量化感知训练: the forward uses the
# quantised weights, the backward passes the gradient through the quantisers
# with the straight-through estimator, and the optimiser updates the original
# (latent) weights.  Reading taken: the forward is Y = X~ W~^T with
# X~ = Xq * d (per-token absmax) and W~ = gamma * Wq (absmean); the STE treats
# both quantisers as the identity, so the gradients of the latent X and W are
# those of the linear map at X~, W~.  Plain fp64; numpy matmul is the
# contraction.

def backward_input(dY, Wp, gamma, K):
    """dX = dY . W~, W~ = gamma * Wq: fp64 [M, K] from dY [M, N]."""
    Wq = unpack(Wp, K).astype(np.float64)                     # [N, K] in {-1, 0, 1}
    return (np.asarray(dY, dtype=np.float64) @ Wq) * float(np.float32(gamma))


def backward_weight(dY, Xq, d):
    """dW = dY^T . X~, X~ = Xq * d (row m scaled by d[m]): fp64 [N, K]."""
    G = np.asarray(dY, dtype=np.float64) * np.asarray(d, dtype=np.float64)[:, None]
    return G.T @ np.asarray(Xq, dtype=np.float64)
