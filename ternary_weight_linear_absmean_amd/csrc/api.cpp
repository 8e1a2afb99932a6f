// api.cpp -- the C ABI of libbitlinear (declared in include/bitlinear.h).
//
// Every entry point validates its arguments on the host, in a fixed order
// (sizes, then the no-op case, then pointers, alignment, workspace, device
// architecture), and only then enqueues kernels on the caller's stream.  No
// entry point allocates, frees or synchronises.  The only global state is a
// per-device cache of "is this device gfx950", filled on first use.
#include "bitlinear.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.h"

#define BL_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512];

bl_status fail(bl_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

bl_status ok() {
    g_last_error[0] = '\0';
    return BL_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_arch_mutex;
signed char g_arch_state[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

bl_status check_arch() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(BL_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(BL_ERR_ARCH, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_arch_mutex);
    if (g_arch_state[dev] == 0) {
        hipDeviceProp_t p;
        e = hipGetDeviceProperties(&p, dev);
        if (e != hipSuccess)
            return fail(BL_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
        g_arch_state[dev] = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
        if (g_arch_state[dev] < 0)
            return fail(BL_ERR_ARCH, "device %d is %s, not gfx950", dev, p.gcnArchName);
    }
    if (g_arch_state[dev] < 0)
        return fail(BL_ERR_ARCH, "device %d is not gfx950", dev);
    return BL_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bl_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess)
        return fail(BL_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

constexpr int64_t kI32Max = 2147483647;
constexpr int64_t kBackwardMax = kI32Max - 63;     // row lengths padded to 64 stay in int

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// FFN workspace: G [M][F] f32 | U [M][F] f32 | Hq [M][F] i8 | dh [M] f32 | dz [M] f32.
// With the fused gate/up kernel (gated, M >= 128) G holds Z and U's region the
// per-tile row partials: max |Z| f32 [M][T] then, 256-byte aligned, sum H^2
// f64 [M][T], T = ceil(F / 128); 12 T <= 4 F bytes per row for any F >= 64.
struct FfnWs {
    size_t g, u, hq, dh, dz, total;
};

FfnWs ffn_ws(int64_t M, int64_t F) {
    FfnWs w;
    const size_t mf = (size_t)M * (size_t)F;
    w.g = 0;
    w.u = round_up(w.g + mf * 4, 256);
    w.hq = round_up(w.u + mf * 4, 256);
    w.dh = round_up(w.hq + mf, 256);
    w.dz = round_up(w.dh + (size_t)M * 4, 256);
    w.total = round_up(w.dz + (size_t)M * 4, 256);
    return w;
}

// Shared checks of the BitLinear product calls.
bl_status check_product(const char *name, const int8_t *Xq, const float *d, int64_t M,
                        int64_t max_m, const uint8_t *Wp, const float *gamma, int64_t N,
                        int64_t K, float *Y, int32_t *acc, bool *noop) {
    *noop = false;
    if (M < 0 || N < 0 || K < 0)
        return fail(BL_ERR_SHAPE, "%s: negative size (M=%lld N=%lld K=%lld)", name,
                    (long long)M, (long long)N, (long long)K);
    if (M > max_m)
        return fail(BL_ERR_SHAPE, "%s: M=%lld exceeds %lld", name, (long long)M,
                    (long long)max_m);
    if (N > kI32Max)
        return fail(BL_ERR_SHAPE, "%s: N=%lld exceeds 2^31-1", name, (long long)N);
    if (K > BL_MAX_K || K % 64 != 0)
        return fail(BL_ERR_SHAPE, "%s: K=%lld must be a multiple of 64 and <= %d", name,
                    (long long)K, BL_MAX_K);
    if (M == 0 || N == 0) {
        *noop = true;
        return ok();
    }
    if (!Xq || !d || !Wp || !gamma || !Y)
        return fail(BL_ERR_NULL, "%s: NULL pointer (Xq=%p d=%p Wp=%p gamma=%p Y=%p)", name,
                    (const void *)Xq, (const void *)d, (const void *)Wp, (const void *)gamma,
                    (const void *)Y);
    if (!aligned(Xq, 16) || !aligned(Wp, 16))
        return fail(BL_ERR_ALIGN, "%s: Xq and Wp must be 16-byte aligned", name);
    if (!aligned(d, 4) || !aligned(gamma, 4) || !aligned(Y, 4) || (acc && !aligned(acc, 4)))
        return fail(BL_ERR_ALIGN, "%s: d, gamma, Y and acc must be 4-byte aligned", name);
    return check_arch();
}

}  // namespace

BL_EXPORT const char *bl_status_string(bl_status st) {
    switch (st) {
    case BL_OK: return "BL_OK";
    case BL_ERR_NULL: return "BL_ERR_NULL";
    case BL_ERR_SHAPE: return "BL_ERR_SHAPE";
    case BL_ERR_DTYPE: return "BL_ERR_DTYPE";
    case BL_ERR_ALIGN: return "BL_ERR_ALIGN";
    case BL_ERR_WORKSPACE: return "BL_ERR_WORKSPACE";
    case BL_ERR_ARCH: return "BL_ERR_ARCH";
    case BL_ERR_HIP: return "BL_ERR_HIP";
    }
    return "BL_ERR_UNKNOWN";
}

BL_EXPORT const char *bl_last_error(void) { return g_last_error; }

BL_EXPORT int bl_abi_version(void) { return BL_ABI_VERSION; }

BL_EXPORT size_t bl_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int64_t F) {
    if (M < 0 || N < 0 || F < 0)
        return 0;
    switch (op) {
    case BL_OP_QUANT_WEIGHT:
        if (K < 0 || K > BL_MAX_K || N > kI32Max) return 0;
        return round_up((size_t)bl::quant_weight_blocks(N, K) * sizeof(double), 256);
    case BL_OP_FFN_RELU2: return ffn_ws(M, F).total;
    case BL_OP_DECODE_STACK:
        if (N < 0 || K < 0 || F < 0 || N > 16384 || K > 16384 || F > 16384) return 0;
        return round_up(bl::stack_ws_floats((int)N, (int)K, (int)F) * sizeof(float), 256);
    case BL_OP_BACKWARD_INPUT:
        if (K < 0 || N < 0 || N > kBackwardMax) return 0;
        if (M < 0 || M > kBackwardMax) return 0;
        return round_up(bl::backward_input_ws_bytes(M, N, K), 256);
    case BL_OP_BACKWARD_WEIGHT:
        if (K < 0 || M < 0 || N < 0 || M > kBackwardMax || N > kBackwardMax) return 0;
        return round_up(bl::backward_weight_ws_bytes(M, N, K), 256);
    default: return 0;
    }
}

BL_EXPORT bl_status quant_weight_absmean_pack(const float *W, int64_t N, int64_t K, uint8_t *Wp,
                                              float *gamma, void *ws, size_t ws_bytes,
                                              void *stream) {
    const char *name = "quant_weight_absmean_pack";
    if (N < 0 || K < 0 || K % 4 != 0 || K > BL_MAX_K || N > kI32Max)
        return fail(BL_ERR_SHAPE, "%s: need N in [0, 2^31), K in [0, %d] with K %% 4 == 0 "
                    "(N=%lld K=%lld)", name, BL_MAX_K, (long long)N, (long long)K);
    if (N * K > ((int64_t)1 << 40))   // keeps every grid of the three kernels below 2^31
        return fail(BL_ERR_SHAPE, "%s: N*K=%lld exceeds 2^40 weights", name, (long long)(N * K));
    if (!gamma)
        return fail(BL_ERR_NULL, "%s: gamma is NULL", name);
    if (!aligned(gamma, 4))
        return fail(BL_ERR_ALIGN, "%s: gamma must be 4-byte aligned", name);
    const bool empty = (N == 0 || K == 0);
    if (!empty) {
        if (!W || !Wp)
            return fail(BL_ERR_NULL, "%s: NULL pointer (W=%p Wp=%p)", name, (const void *)W,
                        (const void *)Wp);
        if (!aligned(W, 16) || !aligned(Wp, 16))
            return fail(BL_ERR_ALIGN, "%s: W and Wp must be 16-byte aligned", name);
        const size_t need = bl_workspace_bytes(BL_OP_QUANT_WEIGHT, 0, N, K, 0);
        if (!ws || ws_bytes < need)
            return fail(BL_ERR_WORKSPACE, "%s: workspace %zu bytes at %p, need %zu", name,
                        ws_bytes, ws, need);
        if (!aligned(ws, 16))
            return fail(BL_ERR_ALIGN, "%s: ws must be 16-byte aligned", name);
    }
    bl_status st = check_arch();
    if (st != BL_OK)
        return st;
    return launched(bl::launch_quant_weight(W, N, K, Wp, gamma, static_cast<double *>(ws),
                                            static_cast<hipStream_t>(stream)),
                    name);
}

BL_EXPORT bl_status quant_weight_absmean_pack_noalloc(const float *W, int64_t N, int64_t K,
                                                      uint8_t *Wp, float *gamma, void *stream) {
    const char *name = "quant_weight_absmean_pack_noalloc";
    if (N < 0 || K < 0 || K % 4 != 0 || K > BL_MAX_K || N > kI32Max)
        return fail(BL_ERR_SHAPE, "%s: need N in [0, 2^31), K in [0, %d] with K %% 4 == 0 "
                    "(N=%lld K=%lld)", name, BL_MAX_K, (long long)N, (long long)K);
    if (N * K > BL_NOALLOC_MAX_WEIGHTS)
        return fail(BL_ERR_SHAPE, "%s: N*K=%lld exceeds the %lld weights its scratch holds",
                    name, (long long)(N * K), (long long)BL_NOALLOC_MAX_WEIGHTS);
    if (!gamma)
        return fail(BL_ERR_NULL, "%s: gamma is NULL", name);
    if (!aligned(gamma, 4))
        return fail(BL_ERR_ALIGN, "%s: gamma must be 4-byte aligned", name);
    if (N > 0 && K > 0) {
        if (!W || !Wp)
            return fail(BL_ERR_NULL, "%s: NULL pointer (W=%p Wp=%p)", name, (const void *)W,
                        (const void *)Wp);
        if (!aligned(W, 16) || !aligned(Wp, 16))
            return fail(BL_ERR_ALIGN, "%s: W and Wp must be 16-byte aligned", name);
    }
    bl_status st = check_arch();
    if (st != BL_OK)
        return st;
    static_assert(BL_NOALLOC_MAX_WEIGHTS / 2048 <= bl::kNoAllocQuantMaxBlocks,
                  "the scratch array holds every block sum");
    double *bsum = nullptr;
    const hipError_t e = bl::noalloc_quant_scratch(&bsum);
    if (e != hipSuccess)
        return fail(BL_ERR_HIP, "%s: scratch address lookup failed: %s", name,
                    hipGetErrorString(e));
    return launched(bl::launch_quant_weight(W, N, K, Wp, gamma, bsum,
                                            static_cast<hipStream_t>(stream)),
                    name);
}

BL_EXPORT bl_status quant_act_absmax_i8(const void *X, bl_dtype dtype, int64_t M, int64_t K,
                                        int8_t *Xq, float *d, void *stream) {
    const char *name = "quant_act_absmax_i8";
    if (M < 0 || K < 0 || K > BL_MAX_K || M > kI32Max)
        return fail(BL_ERR_SHAPE, "%s: need M in [0, 2^31), K in [0, %d] (M=%lld K=%lld)", name,
                    BL_MAX_K, (long long)M, (long long)K);
    if (dtype != BL_F32 && dtype != BL_BF16)
        return fail(BL_ERR_DTYPE, "%s: unknown dtype %d", name, (int)dtype);
    if (M == 0)
        return ok();
    if (!d || (K > 0 && (!X || !Xq)))
        return fail(BL_ERR_NULL, "%s: NULL pointer (X=%p Xq=%p d=%p)", name, X, (void *)Xq,
                    (void *)d);
    if ((K > 0 && (!aligned(X, 16) || !aligned(Xq, 16))) || !aligned(d, 4))
        return fail(BL_ERR_ALIGN, "%s: X and Xq must be 16-byte aligned, d 4-byte", name);
    bl_status st = check_arch();
    if (st != BL_OK)
        return st;
    return launched(bl::launch_quant_act(X, dtype == BL_BF16 ? 1 : 0, M, K, Xq, d,
                                         static_cast<hipStream_t>(stream)),
                    name);
}

BL_EXPORT bl_status quant_act_absmax_i4(const void *X, bl_dtype dtype, int64_t M, int64_t K,
                                        uint8_t *Xq4, float *d, void *stream) {
    const char *name = "quant_act_absmax_i4";
    if (M < 0 || K < 0 || K % 2 != 0 || K > BL_MAX_K || M > kI32Max)
        return fail(BL_ERR_SHAPE, "%s: need M in [0, 2^31), K in [0, %d] and even (M=%lld K=%lld)",
                    name, BL_MAX_K, (long long)M, (long long)K);
    if (dtype != BL_F32 && dtype != BL_BF16)
        return fail(BL_ERR_DTYPE, "%s: unknown dtype %d", name, (int)dtype);
    if (M == 0)
        return ok();
    if (!d || (K > 0 && (!X || !Xq4)))
        return fail(BL_ERR_NULL, "%s: NULL pointer (X=%p Xq4=%p d=%p)", name, X, (void *)Xq4,
                    (void *)d);
    if ((K > 0 && (!aligned(X, 16) || !aligned(Xq4, 16))) || !aligned(d, 4))
        return fail(BL_ERR_ALIGN, "%s: X and Xq4 must be 16-byte aligned, d 4-byte", name);
    bl_status st = check_arch();
    if (st != BL_OK)
        return st;
    return launched(bl::launch_quant_act4(X, dtype == BL_BF16 ? 1 : 0, M, K, Xq4, d,
                                          static_cast<hipStream_t>(stream)),
                    name);
}

BL_EXPORT bl_status bitlinear_a4(const uint8_t *Xq4, const float *d, int64_t M, const uint8_t *Wp,
                                 const float *gamma, int64_t N, int64_t K, float *Y, int32_t *acc,
                                 void *stream) {
    bool noop = false;
    bl_status st = check_product("bitlinear_a4", reinterpret_cast<const int8_t *>(Xq4), d, M,
                                 kI32Max, Wp, gamma, N, K, Y, acc, &noop);
    if (st != BL_OK || noop)
        return st;
    return launched(bl::launch_bitlinear_a4(Xq4, d, (int)M, Wp, gamma, (int)N, (int)K, Y, acc,
                                            static_cast<hipStream_t>(stream)),
                    "bitlinear_a4");
}

BL_EXPORT bl_status bitlinear_gemv(const int8_t *Xq, const float *d, int64_t M, const uint8_t *Wp,
                                   const float *gamma, int64_t N, int64_t K, float *Y,
                                   int32_t *acc, void *stream) {
    bool noop = false;
    bl_status st = check_product("bitlinear_gemv", Xq, d, M, 64, Wp, gamma, N, K, Y, acc, &noop);
    if (st != BL_OK || noop)
        return st;
    return launched(bl::launch_bitlinear(Xq, d, (int)M, Wp, gamma, (int)N, (int)K, Y, acc,
                                         static_cast<hipStream_t>(stream)),
                    "bitlinear_gemv");
}

BL_EXPORT bl_status bitlinear_gemm(const int8_t *Xq, const float *d, int64_t M, const uint8_t *Wp,
                                   const float *gamma, int64_t N, int64_t K, float *Y,
                                   int32_t *acc, void *stream) {
    bool noop = false;
    bl_status st =
        check_product("bitlinear_gemm", Xq, d, M, kI32Max, Wp, gamma, N, K, Y, acc, &noop);
    if (st != BL_OK || noop)
        return st;
    return launched(bl::launch_gemm(Xq, d, (int)M, Wp, gamma, (int)N, (int)K, Y, acc,
                                    static_cast<hipStream_t>(stream)),
                    "bitlinear_gemm");
}

// Shared checks of the two backward calls; *noop is set when the output has
// no elements.  An empty contraction (N == 0 for dX, M == 0 for dW) still
// runs, with no operand read: the product kernel writes the zeros.
static bl_status check_backward(const char *name, const float *dY, int64_t M, int64_t N, int64_t K,
                                const void *w, const float *scale, float *out, void *ws,
                                size_t ws_bytes, size_t need, bool out_empty, bool sum_empty,
                                bool *noop) {
    *noop = false;
    if (M < 0 || N < 0 || K < 0 || M > kBackwardMax || N > kBackwardMax)
        return fail(BL_ERR_SHAPE, "%s: negative or too large size (M=%lld N=%lld K=%lld)", name,
                    (long long)M, (long long)N, (long long)K);
    if (K % 64 != 0 || K > BL_MAX_K)
        return fail(BL_ERR_SHAPE, "%s: K=%lld must be a multiple of 64 and <= %d", name,
                    (long long)K, BL_MAX_K);
    if (out_empty) {
        *noop = true;
        return ok();
    }
    if (!out || (!sum_empty && (!dY || !w || !scale)))
        return fail(BL_ERR_NULL, "%s: NULL pointer", name);
    if (!sum_empty && (!aligned(dY, 16) || !aligned(w, 16)))
        return fail(BL_ERR_ALIGN, "%s: dY and the integer operand must be 16-byte aligned", name);
    if ((!sum_empty && !aligned(scale, 4)) || !aligned(out, 4))
        return fail(BL_ERR_ALIGN, "%s: the scale and the output must be 4-byte aligned", name);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(BL_ERR_WORKSPACE, "%s: workspace %zu bytes at %p, need %zu", name, ws_bytes, ws,
                    need);
    if (!aligned(ws, 16))
        return fail(BL_ERR_ALIGN, "%s: ws must be 16-byte aligned", name);
    return check_arch();
}

BL_EXPORT bl_status bitlinear_backward_input(const float *dY, int64_t M, int64_t N, const uint8_t *Wp,
                                             const float *gamma, int64_t K, float *dX, void *ws,
                                             size_t ws_bytes, void *stream) {
    const char *name = "bitlinear_backward_input";
    if (N % 4 != 0)
        return fail(BL_ERR_SHAPE, "%s: N=%lld must be a multiple of 4", name, (long long)N);
    bool noop = false;
    const size_t need = bl_workspace_bytes(BL_OP_BACKWARD_INPUT, M, N, K, 0);
    bl_status st = check_backward(name, dY, M, N, K, Wp, gamma, dX, ws, ws_bytes, need,
                                  M == 0 || K == 0, N == 0, &noop);
    if (st != BL_OK || noop)
        return st;
    return launched(bl::launch_backward_input(dY, (int)M, (int)N, Wp, gamma, (int)K, dX, ws,
                                              static_cast<hipStream_t>(stream)),
                    name);
}

BL_EXPORT bl_status bitlinear_backward_weight(const float *dY, int64_t M, int64_t N, const int8_t *Xq,
                                              const float *d, int64_t K, float *dW, void *ws,
                                              size_t ws_bytes, void *stream) {
    const char *name = "bitlinear_backward_weight";
    bool noop = false;
    const size_t need = bl_workspace_bytes(BL_OP_BACKWARD_WEIGHT, M, N, K, 0);
    bl_status st = check_backward(name, dY, M, N, K, Xq, d, dW, ws, ws_bytes, need,
                                  N == 0 || K == 0, M == 0, &noop);
    if (st != BL_OK || noop)
        return st;
    return launched(bl::launch_backward_weight(dY, (int)M, (int)N, Xq, d, (int)K, dW, ws,
                                               static_cast<hipStream_t>(stream)),
                    name);
}

BL_EXPORT bl_status bitlinear_gemv_fused(const bl_gemv_job *jobs, int count, int64_t M,
                                         void *stream) {
    const char *name = "bitlinear_gemv_fused";
    if (!jobs)
        return fail(BL_ERR_NULL, "%s: jobs is NULL", name);
    if (count < 1 || count > BL_MAX_JOBS)
        return fail(BL_ERR_SHAPE, "%s: count=%d must be in [1, %d]", name, count, BL_MAX_JOBS);
    if (M < 1 || M > bl::kGemvMaxTokens)
        return fail(BL_ERR_SHAPE, "%s: M=%lld must be in [1, %d]", name, (long long)M,
                    bl::kGemvMaxTokens);
    bl::GemvJob gj[BL_MAX_JOBS];
    for (int j = 0; j < count; ++j) {
        const bl_gemv_job &b = jobs[j];
        if (b.dtype != BL_F32 && b.dtype != BL_BF16)
            return fail(BL_ERR_DTYPE, "%s: job %d: unknown dtype %d", name, j, (int)b.dtype);
        const int esize = b.dtype == BL_F32 ? 4 : 2;
        if (b.N < 0 || b.N > kI32Max || b.K <= 0 || b.K % 64 != 0 || b.K > 16384 ||
            bl::fused_lds_bytes(bl::fused_tile((int)M), (int)b.K, esize) > bl::kFusedMaxLds)
            return fail(BL_ERR_SHAPE, "%s: job %d: need N >= 0, 0 < K <= 16384, K %% 64 == 0 "
                        "and tile(M) * K * (1 + element size) <= %zu (M=%lld N=%lld K=%lld)",
                        name, j, bl::kFusedMaxLds, (long long)M, (long long)b.N, (long long)b.K);
        if (b.reserved != 0)
            return fail(BL_ERR_SHAPE, "%s: job %d: reserved must be 0", name, j);
        if (!b.X || (b.N > 0 && (!b.Wp || !b.gamma || !b.Y)))
            return fail(BL_ERR_NULL, "%s: job %d: NULL pointer", name, j);
        if (!aligned(b.X, 16) || (b.Wp && !aligned(b.Wp, 16)) || (b.Xq && !aligned(b.Xq, 16)) ||
            (b.gamma && !aligned(b.gamma, 4)) || (b.Y && !aligned(b.Y, 4)) ||
            (b.d && !aligned(b.d, 4)))
            return fail(BL_ERR_ALIGN, "%s: job %d: X, Wp, Xq need 16-byte alignment, "
                        "gamma, Y, d 4-byte", name, j);
        gj[j] = bl::GemvJob{b.X, b.Wp, b.gamma, b.Y, b.Xq, b.d, (int)b.N, (int)b.K,
                            b.dtype == BL_BF16 ? 1 : 0};
    }
    bl_status st = check_arch();
    if (st != BL_OK)
        return st;
    return launched(bl::launch_gemv_fused(gj, count, (int)M, static_cast<hipStream_t>(stream)),
                    name);
}

BL_EXPORT bl_status bitlinear_ffn_relu2(const int8_t *Xq, const float *d, int64_t M, int64_t K,
                                        int64_t F, const uint8_t *Wg, const float *gamma_g,
                                        const uint8_t *Wu, const float *gamma_u,
                                        const float *norm_w, float eps, const uint8_t *Wd,
                                        const float *gamma_d, int64_t N, float *Y, int8_t *Hq,
                                        float *dh, void *ws, size_t ws_bytes, void *stream) {
    const char *name = "bitlinear_ffn_relu2";
    if (M < 0 || N < 0 || K < 0 || F < 0 || M > kI32Max || N > kI32Max)
        return fail(BL_ERR_SHAPE, "%s: negative or too large size (M=%lld K=%lld F=%lld N=%lld)",
                    name, (long long)M, (long long)K, (long long)F, (long long)N);
    if (K % 64 != 0 || F % 64 != 0 || K > BL_MAX_K || F > BL_MAX_K)
        return fail(BL_ERR_SHAPE, "%s: K=%lld and F=%lld must be multiples of 64 and <= %d", name,
                    (long long)K, (long long)F, BL_MAX_K);
    if (!(eps >= 0.0f))
        return fail(BL_ERR_SHAPE, "%s: eps must be >= 0", name);
    if (M == 0)
        return ok();
    if (!Xq || !d || !Wg || !gamma_g || !Wd || !gamma_d || (N > 0 && !Y) || (Wu && !gamma_u))
        return fail(BL_ERR_NULL, "%s: NULL pointer", name);
    if (!aligned(Xq, 16) || !aligned(Wg, 16) || !aligned(Wd, 16) || (Wu && !aligned(Wu, 16)) ||
        (Hq && !aligned(Hq, 16)))
        return fail(BL_ERR_ALIGN, "%s: Xq, Wg, Wu, Wd and Hq must be 16-byte aligned", name);
    if (!aligned(d, 4) || !aligned(gamma_g, 4) || !aligned(gamma_d, 4) ||
        (gamma_u && !aligned(gamma_u, 4)) || (norm_w && !aligned(norm_w, 16)) ||
        (Y && !aligned(Y, 4)) || (dh && !aligned(dh, 4)))
        return fail(BL_ERR_ALIGN, "%s: fp32 vectors must be 4-byte aligned (norm_w 16)", name);
    const FfnWs w = ffn_ws(M, F);
    if (!ws || ws_bytes < w.total)
        return fail(BL_ERR_WORKSPACE, "%s: workspace %zu bytes at %p, need %zu", name, ws_bytes,
                    ws, w.total);
    if (!aligned(ws, 16))
        return fail(BL_ERR_ALIGN, "%s: ws must be 16-byte aligned", name);
    bl_status st = check_arch();
    if (st != BL_OK)
        return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char *base = static_cast<char *>(ws);
    float *G = reinterpret_cast<float *>(base + w.g);
    float *U = Wu ? reinterpret_cast<float *>(base + w.u) : nullptr;
    int8_t *hq = Hq ? Hq : reinterpret_cast<int8_t *>(base + w.hq);
    float *dhb = dh ? dh : reinterpret_cast<float *>(base + w.dh);
    float *dz = reinterpret_cast<float *>(base + w.dz);
    const int m = (int)M, k = (int)K, f = (int)F, n = (int)N;

    hipError_t e;
    if (Wu && m >= 128) {
        // one MFMA kernel for gate and up with the ReLU^2 product, gain and
        // row partials in its epilogue; Z takes G's region, the partials U's
        const int tiles = bl::ffn_gate_up_tiles(f);
        float *pmax = reinterpret_cast<float *>(base + w.u);
        double *psum = reinterpret_cast<double *>(base + w.u + round_up((size_t)M * tiles * 4, 256));
        e = bl::launch_ffn_gate_up(Xq, d, m, k, Wg, gamma_g, Wu, gamma_u, norm_w, f, G, pmax, psum, s);
        if (e == hipSuccess)
            e = bl::launch_ffn_tail_z(G, pmax, psum, tiles, eps, m, f, hq, dhb, dz, s);
    } else {
        e = bl::launch_bitlinear(Xq, d, m, Wg, gamma_g, f, k, G, nullptr, s);
        if (e == hipSuccess && Wu)
            e = bl::launch_bitlinear(Xq, d, m, Wu, gamma_u, f, k, U, nullptr, s);
        if (e == hipSuccess)
            e = bl::launch_ffn_tail(G, U, norm_w, eps, m, f, hq, dhb, dz, s);
    }
    if (e == hipSuccess && n > 0)
        e = bl::launch_bitlinear(hq, dz, m, Wd, gamma_d, n, f, Y, nullptr, s);
    return launched(e, name);
}

// Checks of bl_stack_dims shared by the stack call and its status call.
static bl_status check_stack_dims(const char *name, const bl_stack_dims *dims) {
    if (!dims)
        return fail(BL_ERR_NULL, "%s: dims is NULL", name);
    const int64_t H = dims->H, KV = dims->KV, F = dims->F, D = dims->D;
    if (H <= 0 || KV <= 0 || F <= 0 || D <= 0 || H % 64 || KV % 64 ||
        F % 64 || H > 16384 || KV > 16384 || F > 16384 || H % D || KV % D ||
        (H / D) % (KV / D) || dims->path < BL_STACK_AUTO || dims->path > BL_STACK_PERSISTENT ||
        !(dims->eps >= 0.0f) || dims->wait_us < 0 || dims->reserved != 0)
        return fail(BL_ERR_SHAPE, "%s: need H, KV, F multiples of 64 up to 16384; D dividing "
                    "H and KV; KV/D dividing H/D; eps >= 0; path 0..2; wait_us >= 0; "
                    "reserved == 0 (H=%lld KV=%lld F=%lld D=%lld)", name, (long long)H,
                    (long long)KV, (long long)F, (long long)D);
    return BL_OK;
}

BL_EXPORT bl_status bitlinear_decode_stack(const bl_layer *layers, int n_layers,
                                           const bl_stack_dims *dims, float *x, float *trace,
                                           void *ws, size_t ws_bytes, void *stream) {
    const char *name = "bitlinear_decode_stack";
    bl_status st0 = check_stack_dims(name, dims);
    if (st0 != BL_OK)
        return st0;
    const int64_t H = dims->H, KV = dims->KV, F = dims->F, D = dims->D;
    if (n_layers < 0)
        return fail(BL_ERR_SHAPE, "%s: n_layers=%d must be >= 0", name, n_layers);
    if (n_layers == 0)
        return ok();
    if (!layers || !x)
        return fail(BL_ERR_NULL, "%s: NULL layers or x", name);
    if (!aligned(x, 16) || (trace && !aligned(trace, 16)))
        return fail(BL_ERR_ALIGN, "%s: x and trace must be 16-byte aligned", name);
    for (int l = 0; l < n_layers; ++l) {
        const bl_layer &L = layers[l];
        const uint8_t *w[7] = {L.Wq, L.Wk, L.Wv, L.Wo, L.Wg, L.Wu, L.Wd};
        const float *g[7] = {L.gq, L.gk, L.gv, L.go, L.gg, L.gu, L.gd};
        for (int i = 0; i < 7; ++i) {
            if (!w[i] || !g[i])
                return fail(BL_ERR_NULL, "%s: layer %d: NULL weight or gamma %d", name, l, i);
            if (!aligned(w[i], 16) || !aligned(g[i], 4))
                return fail(BL_ERR_ALIGN, "%s: layer %d: weights need 16-byte, gammas 4-byte "
                            "alignment", name, l);
        }
        if (L.ffn_norm && !aligned(L.ffn_norm, 16))
            return fail(BL_ERR_ALIGN, "%s: layer %d: ffn_norm must be 16-byte aligned", name, l);
    }
    const size_t need = bl_workspace_bytes(BL_OP_DECODE_STACK, 1, H, KV, F);
    if (!ws || ws_bytes < need)
        return fail(BL_ERR_WORKSPACE, "%s: workspace %zu bytes at %p, need %zu", name, ws_bytes,
                    ws, need);
    if (!aligned(ws, 16))
        return fail(BL_ERR_ALIGN, "%s: ws must be 16-byte aligned", name);
    bl_status st = check_arch();
    if (st != BL_OK)
        return st;
    if (dims->path == BL_STACK_PERSISTENT && !bl::stack_persistent_fits((int)H, (int)KV, (int)F, (int)D))
        return fail(BL_ERR_SHAPE, "%s: H=%lld KV=%lld F=%lld exceed the persistent path's "
                    "per-workgroup limits on this device", name, (long long)H, (long long)KV,
                    (long long)F);
    return launched(bl::launch_decode_stack(layers, n_layers, (int)H, (int)KV, (int)F, (int)D,
                                            dims->eps, dims->wait_us, x, trace,
                                            static_cast<float *>(ws), dims->path,
                                            static_cast<hipStream_t>(stream)),
                    name);
}

BL_EXPORT bl_status bitlinear_decode_stack_status(const void *ws, size_t ws_bytes,
                                                  const bl_stack_dims *dims, int32_t *status) {
    const char *name = "bitlinear_decode_stack_status";
    bl_status st = check_stack_dims(name, dims);
    if (st != BL_OK)
        return st;
    if (!status)
        return fail(BL_ERR_NULL, "%s: status is NULL", name);
    const size_t need = bl_workspace_bytes(BL_OP_DECODE_STACK, 1, dims->H, dims->KV, dims->F);
    if (!ws || ws_bytes < need)
        return fail(BL_ERR_WORKSPACE, "%s: workspace %zu bytes at %p, need %zu", name, ws_bytes,
                    ws, need);
    if (!aligned(ws, 16))
        return fail(BL_ERR_ALIGN, "%s: ws must be 16-byte aligned", name);
    st = check_arch();
    if (st != BL_OK)
        return st;
    const bl::StackWs w = bl::stack_ws(static_cast<float *>(const_cast<void *>(ws)), (int)dims->H,
                                       (int)dims->KV, (int)dims->F);
    unsigned word = 0;
    const hipError_t e = hipMemcpy(&word, bl::stack_status_word(w, (int)dims->H, (int)dims->KV,
                                                                (int)dims->F),
                                   sizeof word, hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return fail(BL_ERR_HIP, "%s: reading the status word failed: %s", name,
                    hipGetErrorString(e));
    *status = word != 0u ? 1 : 0;
    return ok();
}

BL_EXPORT size_t bitlinear_t5_row_bytes(int64_t K) {
    if (K < 0 || K > BL_MAX_K)
        return 0;
    return (size_t)bl::t5_row_bytes(K);
}

BL_EXPORT bl_status bitlinear_repack_t5(const uint8_t *Wp, int64_t N, int64_t K, uint8_t *Wt5,
                                        void *stream) {
    const char *name = "bitlinear_repack_t5";
    if (N < 0 || K < 0 || K % 4 != 0 || K > BL_MAX_K || N > kI32Max)
        return fail(BL_ERR_SHAPE, "%s: need N in [0, 2^31), K in [0, %d] with K %% 4 == 0 "
                    "(N=%lld K=%lld)", name, BL_MAX_K, (long long)N, (long long)K);
    if (N == 0 || K == 0)
        return ok();
    // one thread per 16 output bytes, 256 per workgroup, a 1-D grid
    const int64_t blocks = (N * (bl::t5_row_bytes(K) / 16) + 255) / 256;
    if (blocks > kI32Max)
        return fail(BL_ERR_SHAPE, "%s: N=%lld K=%lld needs %lld workgroups (max 2^31-1)", name,
                    (long long)N, (long long)K, (long long)blocks);
    if (!Wp || !Wt5)
        return fail(BL_ERR_NULL, "%s: NULL pointer (Wp=%p Wt5=%p)", name, (const void *)Wp,
                    (void *)Wt5);
    if (!aligned(Wp, 16) || !aligned(Wt5, 16))
        return fail(BL_ERR_ALIGN, "%s: Wp and Wt5 must be 16-byte aligned", name);
    bl_status st = check_arch();
    if (st != BL_OK)
        return st;
    return launched(bl::launch_repack_t5(Wp, (int)N, (int)K, Wt5, static_cast<hipStream_t>(stream)),
                    name);
}

BL_EXPORT bl_status bitlinear_gemv_t5(const int8_t *Xq, const float *d, int64_t M,
                                      const uint8_t *Wt5, const float *gamma, int64_t N, int64_t K,
                                      float *Y, int32_t *acc, void *stream) {
    const char *name = "bitlinear_gemv_t5";
    if (M < 0 || N < 0 || K < 0)
        return fail(BL_ERR_SHAPE, "%s: negative size (M=%lld N=%lld K=%lld)", name, (long long)M,
                    (long long)N, (long long)K);
    if (M > bl::kT5MaxTokens)
        return fail(BL_ERR_SHAPE, "%s: M=%lld exceeds %d", name, (long long)M, bl::kT5MaxTokens);
    if (N > kI32Max)
        return fail(BL_ERR_SHAPE, "%s: N=%lld exceeds 2^31-1", name, (long long)N);
    if (K == 0 || K % 4 != 0 || K > BL_MAX_K)
        return fail(BL_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 4, <= %d", name,
                    (long long)K, BL_MAX_K);
    if (M == 0 || N == 0)
        return ok();
    if (bl::t5_lds_bytes((int)M, K) > bl::kT5MaxLds)
        return fail(BL_ERR_SHAPE, "%s: M=%lld K=%lld stages %zu bytes of codes (max %zu)", name,
                    (long long)M, (long long)K, bl::t5_lds_bytes((int)M, K), bl::kT5MaxLds);
    if (!Xq || !d || !Wt5 || !gamma || !Y)
        return fail(BL_ERR_NULL, "%s: NULL pointer (Xq=%p d=%p Wt5=%p gamma=%p Y=%p)", name,
                    (const void *)Xq, (const void *)d, (const void *)Wt5, (const void *)gamma,
                    (const void *)Y);
    if (!aligned(Xq, 16) || !aligned(Wt5, 16))
        return fail(BL_ERR_ALIGN, "%s: Xq and Wt5 must be 16-byte aligned", name);
    if (!aligned(d, 4) || !aligned(gamma, 4) || !aligned(Y, 4) || (acc && !aligned(acc, 4)))
        return fail(BL_ERR_ALIGN, "%s: d, gamma, Y and acc must be 4-byte aligned", name);
    bl_status st = check_arch();
    if (st != BL_OK)
        return st;
    return launched(bl::launch_gemv_t5(Xq, d, (int)M, Wt5, gamma, (int)N, (int)K, Y, acc,
                                       static_cast<hipStream_t>(stream)),
                    name);
}
