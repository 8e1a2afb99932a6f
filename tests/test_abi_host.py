"""Host-side checks of the C ABI (CPU only, no GPU needed).

The library must load, export every function include/bitlinear.h declares,
and reject bad arguments with the documented status before it touches a
device: every call below fails validation (or is an empty no-op), so no
kernel is launched and no device memory is read.
"""
import ctypes
import os
import re

import pytest

import ternary_weight_linear_absmean_amd as bl
from ternary_weight_linear_absmean_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")

OK, NULL, SHAPE, DTYPE, ALIGN, WS = 0, 1, 2, 3, 4, 5

# fake, never-dereferenced addresses: validation fails before any use
A16 = ctypes.c_void_p(0x10000)
A4 = ctypes.c_void_p(0x10004)
A1 = ctypes.c_void_p(0x10001)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return bl.load()


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("quant_weight_absmean_pack", "quant_act_absmax_i8", "bitlinear_gemv",
              "bitlinear_gemm", "bitlinear_ffn_relu2"):
        assert n in names
    assert sorted(names) == sorted(_native.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert lib.bl_abi_version() == 2
    for code, name in _native.STATUS.items():
        assert lib.bl_status_string(code).decode() == name
    assert lib.bl_status_string(99).decode() == "BL_ERR_UNKNOWN"


def test_workspace_sizes(lib):
    # one fp64 sum per block of 2048 row-major weights, rounded up to 256 bytes
    assert lib.bl_workspace_bytes(bl.BL_OP_QUANT_WEIGHT, 0, 6912, 2560, 0) == 6912 * 2560 // 2048 * 8
    assert lib.bl_workspace_bytes(bl.BL_OP_QUANT_WEIGHT, 0, 7, 2560, 0) == 256
    assert lib.bl_workspace_bytes(bl.BL_OP_QUANT_WEIGHT, 0, 40, 4096, 0) == 768
    M, F = 2048, 6912
    ws = lib.bl_workspace_bytes(bl.BL_OP_FFN_RELU2, M, 2560, 2560, F)
    assert ws >= M * F * (4 + 4 + 1) + 2 * M * 4
    assert ws % 256 == 0
    assert lib.bl_workspace_bytes(99, 1, 1, 1, 1) == 0


def _err(lib):
    return lib.bl_last_error().decode()


def test_product_validation(lib):
    for fn in (lib.bitlinear_gemv, lib.bitlinear_gemm):
        # negative and unsupported sizes
        assert fn(A16, A4, -1, A16, A4, 8, 64, A4, None, None) == SHAPE
        assert "negative" in _err(lib)
        assert fn(A16, A4, 1, A16, A4, 8, 96, A4, None, None) == SHAPE       # K % 64
        assert fn(A16, A4, 1, A16, A4, 8, 2 * bl.BL_MAX_K, A4, None, None) == SHAPE
        # empty problems are no-ops, even with NULL pointers
        assert fn(None, None, 0, None, None, 8, 64, None, None, None) == OK
        assert fn(None, None, 3, None, None, 0, 64, None, None, None) == OK
        # NULL and misaligned pointers
        assert fn(None, A4, 1, A16, A4, 8, 64, A4, None, None) == NULL
        assert fn(A16, A4, 1, A16, None, 8, 64, A4, None, None) == NULL
        assert fn(A1, A4, 1, A16, A4, 8, 64, A4, None, None) == ALIGN
        assert fn(A16, A4, 1, A4, A4, 8, 64, A4, None, None) == ALIGN
        assert fn(A16, A1, 1, A16, A4, 8, 64, A4, None, None) == ALIGN
        assert fn(A16, A4, 1, A16, A4, 8, 64, A4, A1, None) == ALIGN
    # the decode call takes at most 64 tokens
    assert lib.bitlinear_gemv(A16, A4, 65, A16, A4, 8, 64, A4, None, None) == SHAPE


def test_a4_validation(lib):
    q4, a4 = lib.quant_act_absmax_i4, lib.bitlinear_a4
    assert q4(A16, 0, -1, 64, A16, A4, None) == SHAPE
    assert q4(A16, 0, 2, 65, A16, A4, None) == SHAPE                     # K odd
    assert q4(A16, 0, 2, 2 * bl.BL_MAX_K, A16, A4, None) == SHAPE
    assert q4(A16, 9, 2, 64, A16, A4, None) == DTYPE
    assert q4(None, 0, 0, 64, None, None, None) == OK                    # no rows
    assert q4(None, 0, 2, 64, A16, A4, None) == NULL
    assert q4(A16, 0, 2, 64, None, A4, None) == NULL
    assert q4(A16, 0, 2, 64, A16, None, None) == NULL
    assert q4(A4, 0, 2, 64, A16, A4, None) == ALIGN
    assert q4(A16, 0, 2, 64, A4, A4, None) == ALIGN
    assert q4(A16, 0, 2, 64, A16, A1, None) == ALIGN
    assert a4(A16, A4, -1, A16, A4, 8, 64, A4, None, None) == SHAPE
    assert a4(A16, A4, 1, A16, A4, 8, 96, A4, None, None) == SHAPE         # K % 64
    assert a4(None, None, 0, None, None, 8, 64, None, None, None) == OK
    assert a4(None, A4, 1, A16, A4, 8, 64, A4, None, None) == NULL
    assert a4(A4, A4, 1, A16, A4, 8, 64, A4, None, None) == ALIGN


def test_noalloc_quant_validation(lib):
    """The allocation-free quantiser's host checks: its scratch holds the
    block sums of at most 2^27 weights."""
    f = lib.quant_weight_absmean_pack_noalloc
    assert f(A16, -1, 64, A16, A4, None) == SHAPE
    assert f(A16, 2, 66, A16, A4, None) == SHAPE                          # K % 4
    assert f(A16, 2, 2 * bl.BL_MAX_K, A16, A4, None) == SHAPE
    assert f(A16, 32769, 4096, A16, A4, None) == SHAPE                    # N K > 2^27
    assert "2^27" in _err(lib) or "134217728" in _err(lib)
    assert f(A16, 2, 64, A16, None, None) == NULL
    assert f(None, 2, 64, A16, A4, None) == NULL
    assert f(A16, 2, 64, None, A4, None) == NULL
    assert f(A4, 2, 64, A16, A4, None) == ALIGN
    assert f(A16, 2, 64, A4, A4, None) == ALIGN
    assert f(A16, 2, 64, A16, A1, None) == ALIGN


def test_t5_validation(lib):
    rb, rp, gv = lib.bitlinear_t5_row_bytes, lib.bitlinear_repack_t5, lib.bitlinear_gemv_t5
    # rows: ceil(K / 5) bytes rounded up to 16
    assert [rb(k) for k in (0, 1, 5, 80, 81, 2560, 6912)] == [0, 16, 16, 16, 32, 512, 1392]
    assert rb(-1) == 0 and rb(2 * bl.BL_MAX_K) == 0
    # repack
    assert rp(A16, -1, 64, A16, None) == SHAPE
    assert rp(A16, 2, 66, A16, None) == SHAPE                            # K % 4
    assert rp(A16, 2, 2 * bl.BL_MAX_K, A16, None) == SHAPE
    assert rp(A16, 2 ** 31 - 1, bl.BL_MAX_K, A16, None) == SHAPE         # grid size
    assert rp(None, 0, 64, None, None) == OK and rp(None, 3, 0, None, None) == OK
    assert rp(None, 2, 64, A16, None) == NULL
    assert rp(A16, 2, 64, None, None) == NULL
    assert rp(A4, 2, 64, A16, None) == ALIGN
    assert rp(A16, 2, 64, A4, None) == ALIGN
    # product
    assert gv(A16, A4, -1, A16, A4, 8, 64, A4, None, None) == SHAPE
    assert gv(A16, A4, 9, A16, A4, 8, 64, A4, None, None) == SHAPE       # M <= 8
    assert gv(A16, A4, 1, A16, A4, 8, 66, A4, None, None) == SHAPE       # K % 4
    assert gv(A16, A4, 1, A16, A4, 8, 0, A4, None, None) == SHAPE        # K > 0
    assert gv(A16, A4, 1, A16, A4, 8, 65524, A4, None, None) == SHAPE    # staged codes > 64 KiB
    assert gv(A16, A4, 5, A16, A4, 8, 8164, A4, None, None) == SHAPE
    assert gv(None, None, 0, None, None, 8, 64, None, None, None) == OK
    assert gv(None, None, 3, None, None, 0, 64, None, None, None) == OK
    assert gv(None, A4, 1, A16, A4, 8, 64, A4, None, None) == NULL
    assert gv(A16, A4, 1, None, A4, 8, 64, A4, None, None) == NULL
    assert gv(A4, A4, 1, A16, A4, 8, 64, A4, None, None) == ALIGN
    assert gv(A16, A4, 1, A4, A4, 8, 64, A4, None, None) == ALIGN
    assert gv(A16, A1, 1, A16, A4, 8, 64, A4, None, None) == ALIGN
    assert gv(A16, A4, 1, A16, A4, 8, 64, A4, A1, None) == ALIGN


def test_quant_validation(lib):
    f = lib.quant_weight_absmean_pack
    assert f(A16, 4, 6, A16, A4, A16, 1 << 20, None) == SHAPE            # K % 4
    assert f(A16, -1, 8, A16, A4, A16, 1 << 20, None) == SHAPE
    assert f(A16, 4, 8, A16, None, A16, 1 << 20, None) == NULL
    assert f(None, 4, 8, A16, A4, A16, 1 << 20, None) == NULL
    assert f(A4, 4, 8, A16, A4, A16, 1 << 20, None) == ALIGN
    assert f(A16, 4, 8, A16, A4, A16, 8, None) == WS                      # needs 4 * 8
    assert f(A16, 4, 8, A16, A4, None, 1 << 20, None) == WS
    g = lib.quant_act_absmax_i8
    assert g(A16, 0, -1, 8, A16, A4, None) == SHAPE
    assert g(A16, 7, 1, 8, A16, A4, None) == DTYPE
    assert g(None, 0, 0, 8, None, None, None) == OK
    assert g(None, 0, 1, 8, A16, A4, None) == NULL
    assert g(A4, 1, 1, 8, A16, A4, None) == ALIGN


def test_ffn_validation(lib):
    f = lib.bitlinear_ffn_relu2
    big = 1 << 40
    args = dict(Xq=A16, d=A4, M=2, K=64, F=128, Wg=A16, gg=A4, Wu=A16, gu=A4, nw=None,
                eps=1e-5, Wd=A16, gd=A4, N=64, Y=A4, Hq=None, dh=None, ws=A16, wsb=big, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["Xq"], a["d"], a["M"], a["K"], a["F"], a["Wg"], a["gg"], a["Wu"], a["gu"],
                 a["nw"], ctypes.c_float(a["eps"]), a["Wd"], a["gd"], a["N"], a["Y"], a["Hq"],
                 a["dh"], a["ws"], a["wsb"], a["s"])

    assert call(F=100) == SHAPE
    assert call(K=-64) == SHAPE
    assert call(eps=-1.0) == SHAPE
    assert call(M=0, Xq=None, d=None) == OK
    assert call(Wg=None) == NULL
    assert call(Wu=A16, gu=None) == NULL
    assert call(Hq=A4) == ALIGN
    assert call(nw=A4) == ALIGN
    assert call(wsb=16) == WS
    assert call(ws=None) == WS


def test_python_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        bl.quant_act_absmax_i8(torch.zeros(2, 64))
    with pytest.raises(TypeError):
        bl.bitlinear_backward_input(torch.zeros(2, 8), torch.zeros(8, 16, dtype=torch.uint8),
                                    torch.ones(1))
    with pytest.raises(TypeError):
        bl.bitlinear_backward_weight(torch.zeros(2, 8), torch.zeros(2, 64, dtype=torch.int8),
                                     torch.ones(2))
    with pytest.raises(TypeError):
        bl.quant_weight_absmean_pack(torch.zeros(4, 64))
    with pytest.raises(TypeError):
        bl.bitlinear_repack_t5(torch.zeros(4, 16, dtype=torch.uint8))
    with pytest.raises(TypeError):
        bl.bitlinear_gemv_t5(torch.zeros(1, 64, dtype=torch.int8), torch.ones(1),
                             torch.zeros(4, 16, dtype=torch.uint8), torch.ones(1))


def test_fused_validation(lib):
    J = _native.GemvJob

    def job(**kw):
        a = dict(X=0x10000, Wp=0x20000, gamma=0x30000, Y=0x40000, Xq=None, d=None, N=8,
                 K=128, dtype=1, reserved=0)
        a.update(kw)
        return J(a["X"], a["Wp"], a["gamma"], a["Y"], a["Xq"], a["d"], a["N"], a["K"],
                 a["dtype"], a["reserved"])

    def call(jobs, M=1):
        arr = (J * max(1, len(jobs)))(*jobs)
        return lib.bitlinear_gemv_fused(arr, len(jobs), M, None)

    assert lib.bitlinear_gemv_fused(None, 1, 1, None) == NULL
    assert call([]) == SHAPE
    assert call([job()] * 9) == SHAPE
    assert call([job()], M=0) == SHAPE
    assert call([job()], M=9) == SHAPE
    assert call([job(K=96)]) == SHAPE
    assert call([job(K=0)]) == SHAPE
    assert call([job(K=16384)], M=8) == SHAPE          # LDS: 8 * 16384 * 3 > 128 KB
    assert call([job(K=6912)], M=8) == SHAPE           # 8 * 6912 * 3 > 128 KB
    assert call([job(K=6912, dtype=0)], M=4) == SHAPE  # 4 * 6912 * 5 > 128 KB
    assert call([job(N=-1)]) == SHAPE
    assert call([job(reserved=1)]) == SHAPE
    assert call([job(dtype=5)]) == DTYPE
    assert call([job(X=None)]) == NULL
    assert call([job(Y=None)]) == NULL
    assert call([job(X=0x10004)]) == ALIGN
    assert call([job(Xq=0x50004)]) == ALIGN
    assert call([job(d=0x50002)]) == ALIGN
    assert call([job(), job(K=100)]) == SHAPE          # second job checked too


def test_stack_validation(lib):
    Lr = _native.Layer
    D = _native.StackDims

    def layer(**kw):
        a = {k: 0x100000 + 0x1000 * i for i, k in enumerate(_native.LAYER_WEIGHTS)}
        a.update({k: 0x200000 + 0x1000 * i for i, k in enumerate(_native.LAYER_GAMMAS)})
        a["ffn_norm"] = None
        a.update(kw)
        return Lr(*[a[k] for k in _native.LAYER_WEIGHTS + _native.LAYER_GAMMAS + ("ffn_norm",)])

    need = bl.workspace_bytes(bl.BL_OP_DECODE_STACK, 1, 256, 128, 512)
    assert need >= 4 * (2 * 256 + 2 * 128 + 2 * 512) + 512

    def call(layers=None, n=None, H=256, KV=128, F=512, Dh=64, eps=1e-5, path=0,
             x=A16, trace=None, ws=A16, wsb=1 << 20, wait_us=0, reserved=0):
        layers = [layer()] if layers is None else layers
        arr = (Lr * max(1, len(layers)))(*layers)
        dims = D(H, KV, F, Dh, eps, path, wait_us, reserved)
        return lib.bitlinear_decode_stack(arr, len(layers) if n is None else n,
                                          ctypes.byref(dims), x, trace, ws, wsb, None)

    assert lib.bitlinear_decode_stack(None, 1, None, A16, None, A16, 1 << 20, None) == NULL
    assert call(n=-1) == SHAPE
    assert call(H=200) == SHAPE
    assert call(KV=96) == SHAPE
    assert call(F=500) == SHAPE
    assert call(H=32768, KV=128) == SHAPE
    assert call(Dh=48) == SHAPE                       # D does not divide H
    assert call(H=384, KV=256, Dh=128) == SHAPE       # 2 kv heads do not divide 3 query heads
    assert call(eps=-1.0) == SHAPE
    assert call(eps=float("nan")) == SHAPE
    assert call(path=3) == SHAPE
    assert call(path=-1) == SHAPE
    assert call(wait_us=-1) == SHAPE
    assert call(reserved=1) == SHAPE
    assert call(n=0, x=None) == OK                    # no layers: nothing to do
    assert call(x=None) == NULL
    assert call(layers=[layer(), layer(Wd=None)]) == NULL
    assert call(layers=[layer(gk=None)]) == NULL
    assert call(x=A4) == ALIGN
    assert call(trace=A4) == ALIGN
    assert call(layers=[layer(Wv=0x100004)]) == ALIGN
    assert call(layers=[layer(gq=0x200002)]) == ALIGN
    assert call(layers=[layer(ffn_norm=0x300004)]) == ALIGN
    assert call(wsb=need - 1) == WS
    assert call(ws=None) == WS
    assert call(ws=A4) == ALIGN


def test_stack_status_validation(lib):
    """The status call checks everything on the host before it reads a byte."""
    D = _native.StackDims
    need = bl.workspace_bytes(bl.BL_OP_DECODE_STACK, 1, 256, 128, 512)
    out = ctypes.c_int32(-5)

    def call(H=256, ws=A16, wsb=1 << 20, status=True, wait_us=0, reserved=0, dims=True):
        d = D(H, 128, 512, 64, 1e-5, 0, wait_us, reserved)
        return lib.bitlinear_decode_stack_status(ws, wsb, ctypes.byref(d) if dims else None,
                                                 ctypes.byref(out) if status else None)

    assert call(dims=False) == NULL
    assert call(H=200) == SHAPE
    assert call(wait_us=-2) == SHAPE
    assert call(reserved=3) == SHAPE
    assert call(status=False) == NULL
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(ws=A4) == ALIGN
    assert out.value == -5                            # nothing written on an error


def test_backward_validation(lib):
    big = 1 << 40
    fi, fw = lib.bitlinear_backward_input, lib.bitlinear_backward_weight
    # workspace: Wq^T bf16 with rows padded to 64; (dY o d)^T as two bf16
    # planes + Xq^T bf16; plus fp32 partial tiles (128 x 256) when the last
    # round of tiles over the 512 two-per-CU slots is at most half full and
    # there are >= 16 c-steps of 32: that tail is split up to 8 ways of >= 8
    # steps, aiming at the 512 slots.
    tile = 128 * 256 * 4
    # M = 8, K = 6912: 27 tiles, 80 steps -> 8 splits of 10 steps
    assert lib.bl_workspace_bytes(bl.BL_OP_BACKWARD_INPUT, 8, 2560, 6912, 0) == \
        6912 * 2560 * 2 + 8 * 27 * tile
    # 4 steps: no split
    assert lib.bl_workspace_bytes(bl.BL_OP_BACKWARD_INPUT, 8, 100, 128, 0) == 128 * 128 * 2
    assert lib.bl_workspace_bytes(bl.BL_OP_BACKWARD_WEIGHT, 100, 6, 128, 0) == \
        2 * ((6 * 128 * 2 + 255) // 256 * 256) + 128 * 128 * 2
    # the QAT shapes at M = 2048: dX 2560 <- 6912 has 160 tiles, 216 steps -> 3
    # splits; dX 6912 <- 2560 has 432 tiles, more than half the slots: none;
    # dW has 540 tiles = 512 + a tail of 28, 64 steps -> 8 splits
    assert lib.bl_workspace_bytes(bl.BL_OP_BACKWARD_INPUT, 2048, 6912, 2560, 0) == \
        2560 * 6912 * 2 + 3 * 160 * tile
    assert lib.bl_workspace_bytes(bl.BL_OP_BACKWARD_INPUT, 2048, 2560, 6912, 0) == 6912 * 2560 * 2
    assert lib.bl_workspace_bytes(bl.BL_OP_BACKWARD_WEIGHT, 2048, 6912, 2560, 0) == \
        2 * 6912 * 2048 * 2 + 2560 * 2048 * 2 + 8 * 28 * tile
    for f in (fi, fw):
        assert f(A16, -1, 8, A16, A4, 64, A4, A16, big, None) == SHAPE
        assert f(A16, 2, 8, A16, A4, 96, A4, A16, big, None) == SHAPE           # K % 64
        assert f(A16, 2, 8, A16, A4, 2 * bl.BL_MAX_K, A4, A16, big, None) == SHAPE
        assert f(A16, 2 ** 31 - 1, 8, A16, A4, 64, A4, A16, big, None) == SHAPE
        assert f(None, 2, 8, A16, A4, 64, A4, A16, big, None) == NULL
        assert f(A16, 2, 8, None, A4, 64, A4, A16, big, None) == NULL
        assert f(A16, 2, 8, A16, None, 64, A4, A16, big, None) == NULL
        assert f(A16, 2, 8, A16, A4, 64, None, A16, big, None) == NULL
        assert f(A4, 2, 8, A16, A4, 64, A4, A16, big, None) == ALIGN
        assert f(A16, 2, 8, A4, A4, 64, A4, A16, big, None) == ALIGN
        assert f(A16, 2, 8, A16, A1, 64, A4, A16, big, None) == ALIGN
        assert f(A16, 2, 8, A16, A4, 64, A1, A16, big, None) == ALIGN
        assert f(A16, 2, 8, A16, A4, 64, A4, A16, 16, None) == WS
        assert f(A16, 2, 8, A16, A4, 64, A4, None, big, None) == WS
        assert f(A16, 2, 8, A16, A4, 64, A4, A4, big, None) == ALIGN
        assert f(None, 0, 0, None, None, 0, None, None, 0, None) == OK
    assert fi(A16, 2, 6, A16, A4, 64, A4, A16, big, None) == SHAPE             # N % 4
    # empty outputs are no-ops, even with NULL pointers
    assert fi(None, 0, 8, None, None, 64, None, None, 0, None) == OK
    assert fw(None, 3, 0, None, None, 64, None, None, 0, None) == OK
