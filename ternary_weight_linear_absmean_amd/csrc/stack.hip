// stack.hip -- one decode token through a stack of BitNet b1.58 layers.
//
// Each layer is a chain of W1.58A8 BitLinears ([CARD] 模型详情: every linear
// layer is a BitLinear without bias, ReLU² FFN, subln) with the parts that
// are not BitLinears reduced to their one-token stand-ins:
//   q, k, v = BitLinear(x)                 (one fused launch, x quantised once
//                                           per workgroup)
//   a       = v repeated per query group   (attention over a single key:
//                                           softmax of one score is 1)
//   o       = BitLinear(a);   x = x + o    (fp32 residual)
//   G, U    = BitLinear(x)                 (one fused launch)
//   y       = down(requant(subln(relu(G)^2 * U)));   x = x + y
// q and k are computed (their weights are streamed like every other
// projection) but, with one key, do not change a.
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

constexpr int kThreads = 256;

// a[h * D + i] = v[(h / group) * D + i]
__global__ __launch_bounds__(kThreads) void expand_heads_kernel(const float *__restrict__ v,
                                                                float *__restrict__ a, int H,
                                                                int D, int group) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= H) return;
    const int h = i / D;
    a[i] = v[(h / group) * D + (i - h * D)];
}

// x = x + y (fp32), optionally recording the input and the result.
__global__ __launch_bounds__(kThreads) void residual_kernel(float *__restrict__ x,
                                                            const float *__restrict__ y, int H,
                                                            float *__restrict__ before,
                                                            float *__restrict__ after) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= H) return;
    const float xi = x[i];
    const float r = __fadd_rn(xi, y[i]);
    x[i] = r;
    if (before) before[i] = xi;
    if (after) after[i] = r;
}

}  // namespace

namespace {
size_t r64(size_t n) { return (n + 63) / 64 * 64; }
}  // namespace

size_t stack_ws_floats(int H, int KV, int F) {
    // q, a, o, y: H each; k, v: KV each; G, U: F each; dh, dz: 1 each; Hq: F
    // bytes = F / 4 floats; then the persistent path's tagged vectors.
    return 4 * r64(H) + 2 * r64(KV) + 2 * r64(F) + 2 * r64(1) + r64(F / 4 + 1) +
           r64(stack_persistent_ws_floats(H, KV, F));
}

StackWs stack_ws(float *ws, int H, int KV, int F) {
    StackWs w;
    float *p = ws;
    auto take = [&](size_t n) { float *r = p; p += r64(n); return r; };
    w.q = take(H); w.a = take(H); w.o = take(H); w.y = take(H);
    w.k = take(KV); w.v = take(KV);
    w.G = take(F); w.U = take(F);
    w.dh = take(1); w.dz = take(1);
    w.Hq = reinterpret_cast<int8_t *>(take(F / 4 + 1));
    w.tagged = take(stack_persistent_ws_floats(H, KV, F));
    return w;
}

hipError_t launch_decode_stack(const StackLayer *layers, int n_layers, int H, int KV, int F,
                               int D, float eps, int wait_us, float *x, float *trace, float *ws,
                               int path, hipStream_t s) {
    const StackWs w = stack_ws(ws, H, KV, F);
    if (path == kStackPersistent || (path == kStackAuto && stack_persistent_fits(H, KV, F, D)))
        return launch_decode_stack_persistent(layers, n_layers, H, KV, F, D, eps, wait_us, x,
                                              trace, w, s);
    // this path has no bounded waits: its status is always 0
    hipError_t e0 = launch_stack_clear_status(stack_status_word(w, H, KV, F), s);
    if (e0 != hipSuccess) return e0;
    float *q = w.q, *a = w.a, *o = w.o, *y = w.y, *k = w.k, *v = w.v, *G = w.G, *U = w.U;
    float *dh = w.dh, *dz = w.dz;
    int8_t *Hq = w.Hq;
    const int group = (H / D) / (KV / D);
    const size_t stride = (size_t)5 * H + 2 * KV;     // x_in q k v o x_mid y
    const dim3 eb((H + kThreads - 1) / kThreads);
    for (int l = 0; l < n_layers; ++l) {
        const StackLayer &L = layers[l];
        float *t = trace ? trace + (size_t)l * stride : nullptr;
        float *tq = t ? t + H : q;
        float *tk = t ? t + 2 * H : k;
        float *tv = t ? t + 2 * H + KV : v;
        float *to = t ? t + 2 * H + 2 * KV : o;
        float *ty = t ? t + 4 * H + 2 * KV : y;
        GemvJob qkv[3] = {
            {x, L.Wq, L.gq, tq, nullptr, nullptr, H, H, 0},
            {x, L.Wk, L.gk, tk, nullptr, nullptr, KV, H, 0},
            {x, L.Wv, L.gv, tv, nullptr, nullptr, KV, H, 0},
        };
        hipError_t e = launch_gemv_fused(qkv, 3, 1, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(expand_heads_kernel, eb, dim3(kThreads), 0, s, (const float *)tv, a, H,
                           D, group);
        GemvJob oj[1] = {{a, L.Wo, L.go, to, nullptr, nullptr, H, H, 0}};
        e = launch_gemv_fused(oj, 1, 1, s);
        if (e != hipSuccess) return e;
        // x is unchanged since the layer began, so `before` records x_in
        hipLaunchKernelGGL(residual_kernel, eb, dim3(kThreads), 0, s, x, (const float *)to, H,
                           t ? t : nullptr, t ? t + 3 * H + 2 * KV : nullptr);
        GemvJob gu[2] = {
            {x, L.Wg, L.gg, G, nullptr, nullptr, F, H, 0},
            {x, L.Wu, L.gu, U, nullptr, nullptr, F, H, 0},
        };
        e = launch_gemv_fused(gu, 2, 1, s);
        if (e != hipSuccess) return e;
        e = launch_ffn_tail(G, U, L.ffn_norm, eps, 1, F, Hq, dh, dz, s);
        if (e != hipSuccess) return e;
        e = launch_gemv(Hq, dz, 1, L.Wd, L.gd, H, F, ty, nullptr, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(residual_kernel, eb, dim3(kThreads), 0, s, x, (const float *)ty, H,
                           nullptr, nullptr);
    }
    return hipGetLastError();
}

}  // namespace bl
