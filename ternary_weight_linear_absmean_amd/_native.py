"""ctypes binding of libbitlinear (include/bitlinear.h).

Argument marshalling only: each function checks that its torch tensors are on
the GPU, contiguous and of the right dtype, allocates outputs (and the
workspace) with torch when the caller gives none, and passes raw device
pointers and the current HIP stream to the C entry point of the same name.
Every step of the computation runs in libbitlinear's kernels.  There is no
fallback: if the library is missing, ``load()`` raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbitlinear.so")

BL_F32 = 0
BL_BF16 = 1
BL_OP_QUANT_WEIGHT = 0
BL_OP_FFN_RELU2 = 1
BL_MAX_K = 131072

STATUS = {0: "BL_OK", 1: "BL_ERR_NULL", 2: "BL_ERR_SHAPE", 3: "BL_ERR_DTYPE",
          4: "BL_ERR_ALIGN", 5: "BL_ERR_WORKSPACE", 6: "BL_ERR_ARCH", 7: "BL_ERR_HIP"}

EXPORTS = ["quant_weight_absmean_pack", "quant_weight_absmean_pack_noalloc", "quant_act_absmax_i8",
           "quant_act_absmax_i4", "bitlinear_a4", "bitlinear_gemv",
           "bitlinear_gemm", "bitlinear_gemv_fused", "bitlinear_ffn_relu2",
           "bitlinear_decode_stack", "bitlinear_decode_stack_status",
           "bitlinear_backward_input", "bitlinear_backward_weight",
           "bitlinear_t5_row_bytes", "bitlinear_repack_t5", "bitlinear_gemv_t5",
           "bl_workspace_bytes", "bl_status_string", "bl_last_error", "bl_abi_version"]
BL_OP_DECODE_STACK = 2
BL_OP_BACKWARD_INPUT = 3
BL_OP_BACKWARD_WEIGHT = 4
LAYER_WEIGHTS = ("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd")
LAYER_GAMMAS = ("gq", "gk", "gv", "go", "gg", "gu", "gd")


class Layer(ctypes.Structure):
    """bl_layer (include/bitlinear.h)."""
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHTS + LAYER_GAMMAS + ("ffn_norm",)]


class StackDims(ctypes.Structure):
    """bl_stack_dims (include/bitlinear.h)."""
    _fields_ = [("H", ctypes.c_int64), ("KV", ctypes.c_int64), ("F", ctypes.c_int64),
                ("D", ctypes.c_int64), ("eps", ctypes.c_float), ("path", ctypes.c_int32),
                ("wait_us", ctypes.c_int32), ("reserved", ctypes.c_int32)]


BL_STACK_AUTO = 0
BL_STACK_LAUNCHES = 1
BL_STACK_PERSISTENT = 2
BL_MAX_JOBS = 8


class GemvJob(ctypes.Structure):
    """bl_gemv_job (include/bitlinear.h)."""
    _fields_ = [("X", ctypes.c_void_p), ("Wp", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("Xq", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

_lib = None
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class BitLinearError(RuntimeError):
    def __init__(self, call, status, detail):
        self.call, self.status, self.detail = call, status, detail
        super().__init__(f"{call}: {STATUS.get(status, status)}: {detail}")


def load():
    """Load libbitlinear.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python -m ternary_weight_linear_absmean_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    lib.quant_weight_absmean_pack.restype = st
    lib.quant_weight_absmean_pack.argtypes = [_p, _i64, _i64, _p, _p, _p, _sz, _p]
    lib.quant_weight_absmean_pack_noalloc.restype = st
    lib.quant_weight_absmean_pack_noalloc.argtypes = [_p, _i64, _i64, _p, _p, _p]
    lib.quant_act_absmax_i8.restype = st
    lib.quant_act_absmax_i8.argtypes = [_p, ctypes.c_int, _i64, _i64, _p, _p, _p]
    lib.quant_act_absmax_i4.restype = st
    lib.quant_act_absmax_i4.argtypes = [_p, ctypes.c_int, _i64, _i64, _p, _p, _p]
    for name in ("bitlinear_gemv", "bitlinear_gemm", "bitlinear_a4"):
        f = getattr(lib, name)
        f.restype = st
        f.argtypes = [_p, _p, _i64, _p, _p, _i64, _i64, _p, _p, _p]
    lib.bitlinear_gemv_fused.restype = st
    lib.bitlinear_gemv_fused.argtypes = [ctypes.POINTER(GemvJob), ctypes.c_int, _i64, _p]
    lib.bitlinear_decode_stack.restype = st
    lib.bitlinear_decode_stack.argtypes = [ctypes.POINTER(Layer), ctypes.c_int,
                                           ctypes.POINTER(StackDims), _p, _p, _p, _sz, _p]
    lib.bitlinear_decode_stack_status.restype = st
    lib.bitlinear_decode_stack_status.argtypes = [_p, _sz, ctypes.POINTER(StackDims),
                                                  ctypes.POINTER(ctypes.c_int32)]
    lib.bitlinear_ffn_relu2.restype = st
    lib.bitlinear_ffn_relu2.argtypes = [_p, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p,
                                        ctypes.c_float, _p, _p, _i64, _p, _p, _p, _p, _sz, _p]
    lib.bl_workspace_bytes.restype = _sz
    for name in ("bitlinear_backward_input", "bitlinear_backward_weight"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [_p, _i64, _i64, _p, _p, _i64, _p, _p, _sz, _p]
    lib.bl_workspace_bytes.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64]
    lib.bitlinear_t5_row_bytes.restype = _sz
    lib.bitlinear_t5_row_bytes.argtypes = [_i64]
    lib.bitlinear_repack_t5.restype = st
    lib.bitlinear_repack_t5.argtypes = [_p, _i64, _i64, _p, _p]
    lib.bitlinear_gemv_t5.restype = st
    lib.bitlinear_gemv_t5.argtypes = [_p, _p, _i64, _p, _p, _i64, _i64, _p, _p, _p]
    lib.bl_status_string.restype = ctypes.c_char_p
    lib.bl_status_string.argtypes = [ctypes.c_int]
    lib.bl_last_error.restype = ctypes.c_char_p
    lib.bl_last_error.argtypes = []
    lib.bl_abi_version.restype = ctypes.c_int
    lib.bl_abi_version.argtypes = []
    _lib = lib
    return lib


def _check(call, status):
    if status != 0:
        raise BitLinearError(call, status, load().bl_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def workspace_bytes(op, M=0, N=0, K=0, F=0):
    return int(load().bl_workspace_bytes(op, M, N, K, F))


def quant_weight_absmean_pack(W, Wp=None, gamma=None, ws=None, stream=None):
    """fp32 W [N, K] -> (packed uint8 [N, K/4], gamma fp32 [1]) on the GPU."""
    _dev(W, torch.float32, "W")
    N, K = W.shape
    dev = W.device
    Wp = _dev(Wp, torch.uint8, "Wp") if Wp is not None else torch.empty(
        (N, K // 4), dtype=torch.uint8, device=dev)
    gamma = _dev(gamma, torch.float32, "gamma") if gamma is not None else torch.empty(
        (1,), dtype=torch.float32, device=dev)
    need = workspace_bytes(BL_OP_QUANT_WEIGHT, 0, N, K, 0)
    if ws is None:
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _check("quant_weight_absmean_pack", load().quant_weight_absmean_pack(
        _ptr(W), N, K, _ptr(Wp), _ptr(gamma), _ptr(ws), ws.numel(), _stream(stream)))
    return Wp, gamma


def quant_weight_absmean_pack_noalloc(W, Wp=None, gamma=None, stream=None):
    """quant_weight_absmean_pack with the library's own scratch (no workspace);
    N * K <= 2^27.  Pass Wp and gamma to keep the call itself free of
    allocation (torch allocates them here when they are absent)."""
    _dev(W, torch.float32, "W")
    N, K = W.shape
    dev = W.device
    Wp = _dev(Wp, torch.uint8, "Wp") if Wp is not None else torch.empty(
        (N, K // 4), dtype=torch.uint8, device=dev)
    gamma = _dev(gamma, torch.float32, "gamma") if gamma is not None else torch.empty(
        (1,), dtype=torch.float32, device=dev)
    _check("quant_weight_absmean_pack_noalloc", load().quant_weight_absmean_pack_noalloc(
        _ptr(W), N, K, _ptr(Wp), _ptr(gamma), _stream(stream)))
    return Wp, gamma


def quant_act_absmax_i8(X, Xq=None, d=None, stream=None):
    """X [M, K] (fp32 or bf16) -> (Xq int8 [M, K], d fp32 [M])."""
    if X.dtype == torch.float32:
        dt = BL_F32
    elif X.dtype == torch.bfloat16:
        dt = BL_BF16
    else:
        raise TypeError("X must be float32 or bfloat16")
    _dev(X, X.dtype, "X")
    M, K = X.shape
    Xq = _dev(Xq, torch.int8, "Xq") if Xq is not None else torch.empty(
        (M, K), dtype=torch.int8, device=X.device)
    d = _dev(d, torch.float32, "d") if d is not None else torch.empty(
        (M,), dtype=torch.float32, device=X.device)
    _check("quant_act_absmax_i8", load().quant_act_absmax_i8(
        _ptr(X), dt, M, K, _ptr(Xq), _ptr(d), _stream(stream)))
    return Xq, d


def _product(call, Xq, d, Wp, gamma, Y, acc, want_acc, stream, a4=False):
    _dev(Xq, torch.uint8 if a4 else torch.int8, "Xq4" if a4 else "Xq")
    _dev(d, torch.float32, "d")
    _dev(Wp, torch.uint8, "Wp")
    _dev(gamma, torch.float32, "gamma")
    M, K = Xq.shape
    if a4:
        K *= 2
    N = Wp.shape[0]
    if Wp.dim() != 2 or Wp.shape[1] * 4 != K:
        raise ValueError(f"Wp must be [N, K/4] = [*, {K // 4}], got {tuple(Wp.shape)}")
    if d.shape != (M,):
        raise ValueError("d must be [M]")
    Y = _dev(Y, torch.float32, "Y") if Y is not None else torch.empty(
        (M, N), dtype=torch.float32, device=Xq.device)
    if acc is None and want_acc:
        acc = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    _dev(acc, torch.int32, "acc")
    _check(call, getattr(load(), call)(_ptr(Xq), _ptr(d), M, _ptr(Wp), _ptr(gamma), N, K,
                                       _ptr(Y), _ptr(acc), _stream(stream)))
    return (Y, acc) if want_acc or acc is not None else Y


def bitlinear_gemv(Xq, d, Wp, gamma, Y=None, acc=None, want_acc=False, stream=None):
    """Y [M, N] fp32 for 1 <= M <= 64 tokens; with want_acc also int32 acc."""
    return _product("bitlinear_gemv", Xq, d, Wp, gamma, Y, acc, want_acc, stream)


def bitlinear_gemm(Xq, d, Wp, gamma, Y=None, acc=None, want_acc=False, stream=None):
    """Y [M, N] fp32 for any M on int8 MFMA; with want_acc also int32 acc."""
    return _product("bitlinear_gemm", Xq, d, Wp, gamma, Y, acc, want_acc, stream)


def quant_act_absmax_i4(X, Xq4=None, d=None, stream=None):
    """X [M, K] (fp32 or bf16, K even) -> (Xq4 uint8 [M, K/2] 4-bit codes, d fp32 [M])."""
    if X.dtype == torch.float32:
        dt = BL_F32
    elif X.dtype == torch.bfloat16:
        dt = BL_BF16
    else:
        raise TypeError("X must be float32 or bfloat16")
    _dev(X, X.dtype, "X")
    M, K = X.shape
    Xq4 = _dev(Xq4, torch.uint8, "Xq4") if Xq4 is not None else torch.empty(
        (M, K // 2), dtype=torch.uint8, device=X.device)
    d = _dev(d, torch.float32, "d") if d is not None else torch.empty(
        (M,), dtype=torch.float32, device=X.device)
    _check("quant_act_absmax_i4", load().quant_act_absmax_i4(
        _ptr(X), dt, M, K, _ptr(Xq4), _ptr(d), _stream(stream)))
    return Xq4, d


def bitlinear_a4(Xq4, d, Wp, gamma, Y=None, acc=None, want_acc=False, stream=None):
    """Y [M, N] fp32 from 4-bit activation codes Xq4 uint8 [M, K/2]; with
    want_acc also the int32 accumulator."""
    return _product("bitlinear_a4", Xq4, d, Wp, gamma, Y, acc, want_acc, stream, a4=True)


def t5_row_bytes(K):
    """Bytes per row of the five-weights-per-byte format (0 if K is out of range)."""
    return int(load().bitlinear_t5_row_bytes(K))


def bitlinear_repack_t5(Wp, K=None, Wt5=None, stream=None):
    """2-bit packed Wp [N, K/4] -> Wt5 uint8 [N, t5_row_bytes(K)] (same weights)."""
    _dev(Wp, torch.uint8, "Wp")
    N = Wp.shape[0]
    K = Wp.shape[1] * 4 if K is None else K
    if Wp.dim() != 2 or Wp.shape[1] * 4 != K:
        raise ValueError(f"Wp must be [N, K/4], got {tuple(Wp.shape)} for K={K}")
    rb = t5_row_bytes(K)
    Wt5 = _dev(Wt5, torch.uint8, "Wt5") if Wt5 is not None else torch.empty(
        (N, rb), dtype=torch.uint8, device=Wp.device)
    if tuple(Wt5.shape) != (N, rb):
        raise ValueError(f"Wt5 must be [{N}, {rb}]")
    _check("bitlinear_repack_t5", load().bitlinear_repack_t5(_ptr(Wp), N, K, _ptr(Wt5),
                                                             _stream(stream)))
    return Wt5


def bitlinear_gemv_t5(Xq, d, Wt5, gamma, Y=None, acc=None, want_acc=False, stream=None):
    """Y [M, N] fp32 from five-per-byte weights, 1 <= M <= 8; with want_acc
    also the int32 accumulator."""
    _dev(Xq, torch.int8, "Xq")
    _dev(d, torch.float32, "d")
    _dev(Wt5, torch.uint8, "Wt5")
    _dev(gamma, torch.float32, "gamma")
    M, K = Xq.shape
    N = Wt5.shape[0]
    if Wt5.dim() != 2 or Wt5.shape[1] != t5_row_bytes(K):
        raise ValueError(f"Wt5 must be [N, {t5_row_bytes(K)}], got {tuple(Wt5.shape)}")
    if d.shape != (M,):
        raise ValueError("d must be [M]")
    Y = _dev(Y, torch.float32, "Y") if Y is not None else torch.empty(
        (M, N), dtype=torch.float32, device=Xq.device)
    if acc is None and want_acc:
        acc = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    _dev(acc, torch.int32, "acc")
    _check("bitlinear_gemv_t5", load().bitlinear_gemv_t5(
        _ptr(Xq), _ptr(d), M, _ptr(Wt5), _ptr(gamma), N, K, _ptr(Y), _ptr(acc),
        _stream(stream)))
    return (Y, acc) if want_acc or acc is not None else Y


def bitlinear_gemv_fused(jobs, stream=None):
    """Fused decode step: each job is a dict with X ([M, K] fp32 / bf16), Wp,
    gamma and optional Y, Xq, d (allocated when absent; Xq / d only when the
    key is present with None meaning "allocate").  Returns the list of jobs
    with their output tensors filled in."""
    if not 1 <= len(jobs) <= BL_MAX_JOBS:
        raise ValueError(f"1..{BL_MAX_JOBS} jobs")
    arr = (GemvJob * len(jobs))()
    M = None
    out = []
    for i, j in enumerate(jobs):
        X = j["X"]
        if X.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("X must be float32 or bfloat16")
        _dev(X, X.dtype, "X")
        _dev(j["Wp"], torch.uint8, "Wp")
        _dev(j["gamma"], torch.float32, "gamma")
        m, K = X.shape
        if M is None:
            M = m
        elif m != M:
            raise ValueError("all jobs must have the same number of tokens")
        N = j["Wp"].shape[0]
        if j["Wp"].shape[1] * 4 != K:
            raise ValueError("Wp must be [N, K/4]")
        dev = X.device
        r = dict(j)
        r["Y"] = _dev(j.get("Y"), torch.float32, "Y") if j.get("Y") is not None else \
            torch.empty((M, N), dtype=torch.float32, device=dev)
        if "Xq" in j:
            r["Xq"] = j["Xq"] if j["Xq"] is not None else torch.empty((M, K), dtype=torch.int8,
                                                                        device=dev)
            _dev(r["Xq"], torch.int8, "Xq")
        if "d" in j:
            r["d"] = j["d"] if j["d"] is not None else torch.empty((M,), dtype=torch.float32,
                                                                     device=dev)
            _dev(r["d"], torch.float32, "d")
        arr[i] = GemvJob(X.data_ptr(), j["Wp"].data_ptr(), j["gamma"].data_ptr(),
                         r["Y"].data_ptr(), r["Xq"].data_ptr() if r.get("Xq") is not None else None,
                         r["d"].data_ptr() if r.get("d") is not None else None, N, K,
                         BL_BF16 if X.dtype == torch.bfloat16 else BL_F32, 0)
        out.append(r)
    _check("bitlinear_gemv_fused", load().bitlinear_gemv_fused(arr, len(jobs), M, _stream(stream)))
    return out


def bitlinear_ffn_relu2(Xq, d, Wg, gamma_g, Wu, gamma_u, Wd, gamma_d, norm_w=None, eps=1e-5,
                        Y=None, Hq=None, dh=None, want_debug=False, ws=None, stream=None):
    """ReLU^2 FFN tail; returns Y [M, N] (and Hq int8 [M, F], dh fp32 [M] with
    want_debug)."""
    _dev(Xq, torch.int8, "Xq")
    _dev(d, torch.float32, "d")
    for t, n in ((Wg, "Wg"), (Wd, "Wd")):
        _dev(t, torch.uint8, n)
    _dev(Wu, torch.uint8, "Wu")
    _dev(gamma_g, torch.float32, "gamma_g")
    _dev(gamma_d, torch.float32, "gamma_d")
    _dev(gamma_u, torch.float32, "gamma_u")
    _dev(norm_w, torch.float32, "norm_w")
    M, K = Xq.shape
    F = Wg.shape[0]
    N = Wd.shape[0]
    if Wg.shape[1] * 4 != K or (Wu is not None and tuple(Wu.shape) != tuple(Wg.shape)) \
            or Wd.shape[1] * 4 != F:
        raise ValueError("weight shapes do not chain: Wg/Wu [F, K/4], Wd [N, F/4]")
    dev = Xq.device
    Y = _dev(Y, torch.float32, "Y") if Y is not None else torch.empty(
        (M, N), dtype=torch.float32, device=dev)
    if want_debug:
        Hq = Hq if Hq is not None else torch.empty((M, F), dtype=torch.int8, device=dev)
        dh = dh if dh is not None else torch.empty((M,), dtype=torch.float32, device=dev)
    _dev(Hq, torch.int8, "Hq")
    _dev(dh, torch.float32, "dh")
    need = workspace_bytes(BL_OP_FFN_RELU2, M, N, K, F)
    if ws is None:
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _check("bitlinear_ffn_relu2", load().bitlinear_ffn_relu2(
        _ptr(Xq), _ptr(d), M, K, F, _ptr(Wg), _ptr(gamma_g), _ptr(Wu), _ptr(gamma_u),
        _ptr(norm_w), float(eps), _ptr(Wd), _ptr(gamma_d), N, _ptr(Y), _ptr(Hq), _ptr(dh),
        _ptr(ws), ws.numel(), _stream(stream)))
    return (Y, Hq, dh) if want_debug else Y


def bitlinear_decode_stack(layers, x, H, KV, F, D, eps=1e-5, trace=False, ws=None, stream=None,
                           path=BL_STACK_AUTO, wait_us=0):
    """One decode token through len(layers) layers; x fp32 [H] is updated in
    place.  Each layer is a dict with packed weights Wq..Wd (uint8), gammas
    gq..gd (fp32 [1]) and optional ffn_norm (fp32 [F]).  With trace=True
    returns the per-layer trace [n_layers, 5 H + 2 KV] (x_in, q, k, v, o,
    x_mid, y).  path: BL_STACK_AUTO, BL_STACK_LAUNCHES or BL_STACK_PERSISTENT;
    wait_us: limit of each wait of the persistent path (0 = 1 s)."""
    _dev(x, torch.float32, "x")
    n = len(layers)
    arr = (Layer * max(1, n))()
    for i, L in enumerate(layers):
        vals = []
        for k in LAYER_WEIGHTS:
            vals.append(_dev(L[k], torch.uint8, k).data_ptr())
        for k in LAYER_GAMMAS:
            vals.append(_dev(L[k], torch.float32, k).data_ptr())
        nw = L.get("ffn_norm")
        vals.append(_dev(nw, torch.float32, "ffn_norm").data_ptr() if nw is not None else None)
        arr[i] = Layer(*vals)
    dims = StackDims(H, KV, F, D, float(eps), int(path), int(wait_us), 0)
    tr = None
    if trace:
        tr = torch.empty((n, 5 * H + 2 * KV), dtype=torch.float32, device=x.device)
    need = workspace_bytes(BL_OP_DECODE_STACK, 1, H, KV, F)
    if ws is None:
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=x.device)
    _check("bitlinear_decode_stack", load().bitlinear_decode_stack(
        arr, n, ctypes.byref(dims), _ptr(x), _ptr(tr), _ptr(ws), ws.numel(), _stream(stream)))
    return tr


def bitlinear_decode_stack_status(ws, H, KV, F, D, path=BL_STACK_AUTO):
    """Status of the last bitlinear_decode_stack call on workspace ws (uint8
    device tensor): 0 = it ran to the end, 1 = a wait gave up (x holds NaN).
    Blocking read; call it once that call's work has finished."""
    _dev(ws, torch.uint8, "ws")
    dims = StackDims(H, KV, F, D, 0.0, int(path), 0, 0)
    out = ctypes.c_int32(-1)
    _check("bitlinear_decode_stack_status", load().bitlinear_decode_stack_status(
        _ptr(ws), ws.numel(), ctypes.byref(dims), ctypes.byref(out)))
    return int(out.value)


def bitlinear_backward_input(dY, Wp, gamma, dX=None, ws=None, stream=None):
    """Straight-through gradient of the layer input: dX [M, K] = gamma (dY . Wq)
    for dY fp32 [M, N] and the forward's packed Wp [N, K/4], gamma [1]."""
    _dev(dY, torch.float32, "dY")
    _dev(Wp, torch.uint8, "Wp")
    _dev(gamma, torch.float32, "gamma")
    M, N = dY.shape
    if Wp.dim() != 2 or Wp.shape[0] != N:
        raise ValueError(f"Wp must be [N, K/4] with N = {N}, got {tuple(Wp.shape)}")
    K = Wp.shape[1] * 4
    dX = _dev(dX, torch.float32, "dX") if dX is not None else torch.empty(
        (M, K), dtype=torch.float32, device=dY.device)
    if tuple(dX.shape) != (M, K):
        raise ValueError(f"dX must be [{M}, {K}]")
    need = workspace_bytes(BL_OP_BACKWARD_INPUT, M, N, K, 0)
    if ws is None:
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=dY.device)
    _check("bitlinear_backward_input", load().bitlinear_backward_input(
        _ptr(dY), M, N, _ptr(Wp), _ptr(gamma), K, _ptr(dX), _ptr(ws), ws.numel(), _stream(stream)))
    return dX


def bitlinear_backward_weight(dY, Xq, d, dW=None, ws=None, stream=None):
    """Straight-through gradient of the latent weights: dW [N, K] =
    (dY o d)^T . Xq for dY fp32 [M, N] and the forward's Xq int8 [M, K], d [M]."""
    _dev(dY, torch.float32, "dY")
    _dev(Xq, torch.int8, "Xq")
    _dev(d, torch.float32, "d")
    M, N = dY.shape
    if Xq.dim() != 2 or Xq.shape[0] != M or tuple(d.shape) != (M,):
        raise ValueError(f"Xq must be [{M}, K] and d [{M}]")
    K = Xq.shape[1]
    dW = _dev(dW, torch.float32, "dW") if dW is not None else torch.empty(
        (N, K), dtype=torch.float32, device=dY.device)
    if tuple(dW.shape) != (N, K):
        raise ValueError(f"dW must be [{N}, {K}]")
    need = workspace_bytes(BL_OP_BACKWARD_WEIGHT, M, N, K, 0)
    if ws is None:
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=dY.device)
    _check("bitlinear_backward_weight", load().bitlinear_backward_weight(
        _ptr(dY), M, N, _ptr(Xq), _ptr(d), K, _ptr(dW), _ptr(ws), ws.numel(), _stream(stream)))
    return dW
