// ffn.hip -- ReLU² + subln + int8 requantisation between the gate/up and the
// down BitLinears of a BitNet b1.58 feed-forward block.
//
// The iaiol.com article (权重映射为三元值) and the model card (模型详情) give
// the block's pieces: ReLU² in place of SwiGLU, subln normalisation, int8
// per-token absmax activations into every BitLinear.  Readings taken: gated
// H = relu(G)^2 * U; subln is RMSNorm over the F features with optional gain
// g; its output is requantised per token.  Absmax codes are unchanged by the
// per-row factor 1/rms > 0, so the codes are taken from fp32(H * g) and the
// down projection's activation scale becomes dz = dh / rms.
//
// One workgroup per token row: pass 1 forms max |H * g| (exact) and the fp64
// sum of H^2 (fixed reduction tree, so run-to-run identical); pass 2
// recomputes H * g from G and U (still in L2) and writes the int8 codes.
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

constexpr int kThreads = 256;

struct HZ {
    float h;
    float z;
};

__device__ __forceinline__ HZ h_and_z(float g, float u, bool gated, float gain) {
    const float r = g > 0.0f ? g : 0.0f;
    const float r2 = __fmul_rn(r, r);
    const float h = gated ? __fmul_rn(r2, u) : r2;
    return HZ{h, __fmul_rn(h, gain)};
}


__global__ __launch_bounds__(kThreads) void ffn_tail_kernel(
    const float *__restrict__ G, const float *__restrict__ U, const float *__restrict__ norm_w,
    float eps, int F, int8_t *__restrict__ Hq, float *__restrict__ dh, float *__restrict__ dz) {
    __shared__ float red_a[kThreads / 64];
    __shared__ double red_s[kThreads / 64];
    const int64_t m = blockIdx.x;
    const float *g_row = G + m * F;
    const float *u_row = U ? U + m * F : nullptr;
    const bool gated = U != nullptr;
    float a = 0.0f;
    double ss = 0.0;
    for (int f = 4 * threadIdx.x; f < F; f += 4 * kThreads) {     // F % 64 == 0
        const float4 gv = *reinterpret_cast<const float4 *>(g_row + f);
        const float4 uv = gated ? *reinterpret_cast<const float4 *>(u_row + f)
                                : make_float4(1.f, 1.f, 1.f, 1.f);
        const float4 wv = norm_w ? *reinterpret_cast<const float4 *>(norm_w + f)
                                 : make_float4(1.f, 1.f, 1.f, 1.f);
        const HZ e0 = h_and_z(gv.x, uv.x, gated, wv.x);
        const HZ e1 = h_and_z(gv.y, uv.y, gated, wv.y);
        const HZ e2 = h_and_z(gv.z, uv.z, gated, wv.z);
        const HZ e3 = h_and_z(gv.w, uv.w, gated, wv.w);
        a = fmaxf(a, fmaxf(fmaxf(fabsf(e0.z), fabsf(e1.z)), fmaxf(fabsf(e2.z), fabsf(e3.z))));
        ss += (double)e0.h * e0.h + (double)e1.h * e1.h + (double)e2.h * e2.h + (double)e3.h * e3.h;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a = fmaxf(a, __shfl_xor(a, off));
        ss += __shfl_xor(ss, off);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red_a[wave] = a;
        red_s[wave] = ss;
    }
    __syncthreads();
    a = red_a[0];
    ss = red_s[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
        a = fmaxf(a, red_a[w]);
        ss += red_s[w];
    }
    const bool zero = !(a > 0.0f);
    const float s = act_inv_scale(a);
    int8_t *q_row = Hq + m * F;
    for (int f = 4 * threadIdx.x; f < F; f += 4 * kThreads) {
        const float4 gv = *reinterpret_cast<const float4 *>(g_row + f);
        const float4 uv = gated ? *reinterpret_cast<const float4 *>(u_row + f)
                                : make_float4(1.f, 1.f, 1.f, 1.f);
        const float4 wv = norm_w ? *reinterpret_cast<const float4 *>(norm_w + f)
                                 : make_float4(1.f, 1.f, 1.f, 1.f);
        const uint32_t q = (uint32_t)(act_code(h_and_z(gv.x, uv.x, gated, wv.x).z, s) & 0xFF) |
                           ((uint32_t)(act_code(h_and_z(gv.y, uv.y, gated, wv.y).z, s) & 0xFF) << 8) |
                           ((uint32_t)(act_code(h_and_z(gv.z, uv.z, gated, wv.z).z, s) & 0xFF) << 16) |
                           ((uint32_t)(act_code(h_and_z(gv.w, uv.w, gated, wv.w).z, s) & 0xFF) << 24);
        *reinterpret_cast<uint32_t *>(q_row + f) = q;
    }
    if (threadIdx.x == 0) {
        const float dhm = act_scale(a);
        dh[m] = dhm;
        // a row whose H * g is all zero has zero codes and scale 0
        dz[m] = zero ? 0.0f : (float)((double)dhm / sqrt(ss / (double)F + (double)eps));
    }
}

// Tail after the fused gate/up kernel (M >= 128): Z = fl(H * g) is already
// in memory and the gate/up epilogue left, per row and 128-column tile,
// max |Z| and the fp64 sum of H^2.  One workgroup per row reduces those
// partials in tile order (the same order in every thread, uniform addresses),
// so max |Z| is exact and the sum is run-to-run identical; then it writes the
// int8 codes of Z.  Z is read once, with non-temporal loads.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void ffn_tail_z_kernel(
    const float *__restrict__ Z, const float *__restrict__ pmax, const double *__restrict__ psum,
    int tiles, float eps, int F, int8_t *__restrict__ Hq, float *__restrict__ dh,
    float *__restrict__ dz) {
    const int64_t m = blockIdx.x;
    float a = 0.0f;
    double ss = 0.0;
    for (int t = 0; t < tiles; ++t) {
        a = fmaxf(a, scalar_load(pmax + m * tiles + t));
        ss += scalar_load(psum + m * tiles + t);
    }
    const bool zero = !(a > 0.0f);
    const float s = act_inv_scale(a);
    const float *z_row = Z + m * F;
    int8_t *q_row = Hq + m * F;
    for (int f = 4 * threadIdx.x; f < F; f += 4 * kThreads) {     // F % 64 == 0
        const f32x4 z = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(z_row + f));
        const uint32_t q = (uint32_t)(act_code(z.x, s) & 0xFF) |
                           ((uint32_t)(act_code(z.y, s) & 0xFF) << 8) |
                           ((uint32_t)(act_code(z.z, s) & 0xFF) << 16) |
                           ((uint32_t)(act_code(z.w, s) & 0xFF) << 24);
        *reinterpret_cast<uint32_t *>(q_row + f) = q;
    }
    if (threadIdx.x == 0) {
        const float dhm = act_scale(a);
        dh[m] = dhm;
        // a row whose Z is all zero has zero codes and scale 0
        dz[m] = zero ? 0.0f : (float)((double)dhm / sqrt(ss / (double)F + (double)eps));
    }
}

}  // namespace

hipError_t launch_ffn_tail_z(const float *Z, const float *pmax, const double *psum, int tiles,
                             float eps, int M, int F, int8_t *Hq, float *dh, float *dz,
                             hipStream_t s) {
    if (M == 0)
        return hipSuccess;
    hipLaunchKernelGGL(ffn_tail_z_kernel, dim3(M), dim3(kThreads), 0, s, Z, pmax, psum, tiles,
                       eps, F, Hq, dh, dz);
    return hipGetLastError();
}

hipError_t launch_ffn_tail(const float *G, const float *U, const float *norm_w, float eps,
                           int M, int F, int8_t *Hq, float *dh, float *dz, hipStream_t s) {
    if (M == 0)
        return hipSuccess;
    hipLaunchKernelGGL(ffn_tail_kernel, dim3(M), dim3(kThreads), 0, s, G, U, norm_w, eps, F, Hq,
                       dh, dz);
    return hipGetLastError();
}

}  // namespace bl
