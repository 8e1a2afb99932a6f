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
        if not os.path.exists(_build.LIB):
            _build.build()
        path = _build.LIB
    lib = ctypes.CDLL(path)
    lib.ob_num_threads.restype = ctypes.c_int
    lib.ob_num_threads.argtypes = []
    lib.ob_absmean_gamma.restype = _f32
    lib.ob_absmean_gamma.argtypes = [_p, _i64, _i64]
    lib.ob_ternarize.restype = None
    lib.ob_ternarize.argtypes = [_p, _i64, _f32, _p]
    lib.ob_pack.restype = None
    lib.ob_pack.argtypes = [_p, _i64, _i64, _p]
    lib.ob_unpack.restype = None
    lib.ob_unpack.argtypes = [_p, _i64, _i64, _p]
    lib.ob_bf16_to_f32.restype = None
    lib.ob_bf16_to_f32.argtypes = [_p, _i64, _p]
    lib.ob_quant_act.restype = None
    lib.ob_quant_act.argtypes = [_p, _i64, _i64, _p, _p]
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
                                 _p, _p, _p, _p, _p, _p, _p, _p]
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

    Returns dict(Y=float64 [M, N], Hq=int8 [M, F], dh=float32 [M], rms=float64 [M]).
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
    _load().ob_ffn_relu2(_ptr(Xq), _ptr(d), M, K, F,
                         _ptr(Wg), float(np.float32(gamma_g)),
                         _ptr(Wu), float(np.float32(gamma_u)),
                         _ptr(nw), float(eps),
                         _ptr(Wd), float(np.float32(gamma_d)), N,
                         _ptr(Y), _ptr(Hq), _ptr(dh), _ptr(rms),
                         _ptr(scratch), _ptr(G), _ptr(U), _ptr(Zp))
    return dict(Y=Y, Hq=Hq, dh=dh, rms=rms)
