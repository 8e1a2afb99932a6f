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


// One workgroup per token row.  A thread's share of the row (up to
// kTailU 16-byte units of G, U and the gains per chunk of kTailChunk features)
// is loaded in one batch, every load unconditional (an absent U or gain
// reads G and is not used), and z stays in registers for the codes: one
// round trip instead of one per unit and a second pass over the row (7.7 us
// for M = 1, F = 6912 before).  Each thread adds its fp64 H^2 terms in the
// same order as a unit-by-unit loop would.
constexpr int kTailU = 8;
constexpr int kTailChunk = 4 * kThreads * kTailU;

__global__ __launch_bounds__(kThreads) void ffn_tail_kernel(
    const float *__restrict__ G, const float *__restrict__ U, const float *__restrict__ norm_w,
    float eps, int F, int8_t *__restrict__ Hq, float *__restrict__ dh, float *__restrict__ dz) {
    __shared__ float red_a[kThreads / 64];
    __shared__ double red_s[kThreads / 64];
    const int64_t m = blockIdx.x;
    const float *g_row = G + m * F;
    const bool gated = U != nullptr;
    const float *u_src = gated ? U + m * F : g_row;        // a valid row either way
    const float *w_src = norm_w ? norm_w : g_row;
    const int tid = threadIdx.x;
    if (F == 0) {                                          // no features: zero scales
        if (tid == 0) { dh[m] = 0.0f; dz[m] = 0.0f; }
        return;
    }
    float a = 0.0f;
    double ss = 0.0;
    float4 zk[kTailU];                                      // z of the first chunk
    auto chunk_z = [&](int f0, float4 (&z)[kTailU], bool reduce) {
        float4 gv[kTailU], uv[kTailU], wv[kTailU];
#pragma unroll
        for (int j = 0; j < kTailU; ++j) {                  // F % 64 == 0, F >= 64
            const int fc = min(f0 + 4 * tid + 4 * kThreads * j, F - 4);
            gv[j] = *reinterpret_cast<const float4 *>(g_row + fc);
            uv[j] = *reinterpret_cast<const float4 *>(u_src + fc);
            wv[j] = *reinterpret_cast<const float4 *>(w_src + fc);
        }
#pragma unroll
        for (int j = 0; j < kTailU; ++j) {
            const float4 u = gated ? uv[j] : make_float4(1.f, 1.f, 1.f, 1.f);
            const float4 w = norm_w ? wv[j] : make_float4(1.f, 1.f, 1.f, 1.f);
            const HZ e0 = h_and_z(gv[j].x, u.x, gated, w.x);
            const HZ e1 = h_and_z(gv[j].y, u.y, gated, w.y);
            const HZ e2 = h_and_z(gv[j].z, u.z, gated, w.z);
            const HZ e3 = h_and_z(gv[j].w, u.w, gated, w.w);
            z[j] = make_float4(e0.z, e1.z, e2.z, e3.z);
            if (reduce && f0 + 4 * tid + 4 * kThreads * j < F) {
                a = fmaxf(a, fmaxf(fmaxf(fabsf(e0.z), fabsf(e1.z)), fmaxf(fabsf(e2.z), fabsf(e3.z))));
                ss += (double)e0.h * e0.h + (double)e1.h * e1.h + (double)e2.h * e2.h +
                      (double)e3.h * e3.h;
            }
        }
    };
    chunk_z(0, zk, true);
    for (int f0 = kTailChunk; f0 < F; f0 += kTailChunk) {  // F > 8192 only
        float4 zt[kTailU];
        chunk_z(f0, zt, true);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a = fmaxf(a, __shfl_xor(a, off));
        ss += __shfl_xor(ss, off);
    }
    const int wave = tid >> 6;
    if ((tid & 63) == 0) {
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
    auto put = [&](const float4 (&z)[kTailU], int f0) {
#pragma unroll
        for (int j = 0; j < kTailU; ++j) {
            const int f = f0 + 4 * tid + 4 * kThreads * j;
            if (f < F)
                *reinterpret_cast<uint32_t *>(q_row + f) =
                    (uint32_t)(act_code(z[j].x, s) & 0xFF) | ((uint32_t)(act_code(z[j].y, s) & 0xFF) << 8) |
                    ((uint32_t)(act_code(z[j].z, s) & 0xFF) << 16) |
                    ((uint32_t)(act_code(z[j].w, s) & 0xFF) << 24);
        }
    };
    put(zk, 0);
    for (int f0 = kTailChunk; f0 < F; f0 += kTailChunk) {  // F > 8192 only
        float4 zt[kTailU];
        chunk_z(f0, zt, false);
        put(zt, f0);
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
// max |Z| and the fp64 sum of H^2.  One workgroup per row: each thread loads
// one tile's partials, then issues every 16-byte load of its share of the Z
// row before it uses any of them (vector loads retire in order, so the
// partials arrive first); max |Z| is reduced across the workgroup (exact),
// and one thread adds the fp64 sums in tile order, so the sum is run-to-run
// identical.  Then the int8 codes of Z are written.  Z is read once, with
// non-temporal loads.  (Reading the partials with one dependent scalar load
// per tile, and each 16-byte Z load waited for before the next was issued,
// took 16.0 us at M = 2048, F = 6912.)
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kZUnits = 8;                                // 16-byte Z loads in flight per thread
constexpr int kMaxTiles = BL_MAX_K / 128;                  // 128-column tiles per row

__global__ __launch_bounds__(kThreads) void ffn_tail_z_kernel(
    const float *__restrict__ Z, const float *__restrict__ pmax, const double *__restrict__ psum,
    int tiles, float eps, int F, int8_t *__restrict__ Hq, float *__restrict__ dh,
    float *__restrict__ dz) {
    __shared__ double s_sum[kMaxTiles > kThreads ? kMaxTiles : kThreads];
    __shared__ float s_max[kThreads / 64];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const float *pm = pmax + m * tiles;
    const double *ps = psum + m * tiles;
    if (F == 0) {                                          // no features: zero scales
        if (tid == 0) { dh[m] = 0.0f; dz[m] = 0.0f; }
        return;
    }
    // Every load below is unconditional, at an in-bounds (clamped) address,
    // so the compiler counts them and waits for the partials alone.
    const bool has_t = tid < tiles;
    const float pa0 = pm[min(tid, tiles - 1)];             // requested first
    const double pss0 = ps[min(tid, tiles - 1)];
    const float *z_row = Z + m * F;
    int8_t *q_row = Hq + m * F;
    constexpr int kChunk = 4 * kThreads * kZUnits;         // row elements per chunk
    f32x4 zr[kZUnits];
#pragma unroll
    for (int j = 0; j < kZUnits; ++j)                      // F % 64 == 0
        zr[j] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(z_row + min(4 * tid + 4 * kThreads * j, F - 4)));
    float pa = has_t ? pa0 : 0.0f;
    s_sum[tid] = has_t ? pss0 : 0.0;                       // slots past the tiles: unused
    for (int t = tid + kThreads; t < tiles; t += kThreads) {   // F > 32768 only
        pa = fmaxf(pa, pm[t]);
        s_sum[t] = ps[t];
    }
    pa = group_max(pa, 64);
    if ((tid & 63) == 0) s_max[tid >> 6] = pa;
    __syncthreads();
    float a = s_max[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) a = fmaxf(a, s_max[w]);
    const float s = act_inv_scale(a);
    auto put = [&](const f32x4 &z, int f) {
        const uint32_t q = (uint32_t)(act_code(z.x, s) & 0xFF) |
                           ((uint32_t)(act_code(z.y, s) & 0xFF) << 8) |
                           ((uint32_t)(act_code(z.z, s) & 0xFF) << 16) |
                           ((uint32_t)(act_code(z.w, s) & 0xFF) << 24);
        *reinterpret_cast<uint32_t *>(q_row + f) = q;
    };
#pragma unroll
    for (int j = 0; j < kZUnits; ++j) {
        const int f = 4 * tid + 4 * kThreads * j;
        if (f < F) put(zr[j], f);
    }
    for (int f0 = kChunk; f0 < F; f0 += kChunk) {          // F > 8192 only
#pragma unroll
        for (int j = 0; j < kZUnits; ++j)
            zr[j] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4 *>(z_row + min(f0 + 4 * tid + 4 * kThreads * j, F - 4)));
#pragma unroll
        for (int j = 0; j < kZUnits; ++j) {
            const int f = f0 + 4 * tid + 4 * kThreads * j;
            if (f < F) put(zr[j], f);
        }
    }
    if (tid == 0) {                                        // after its own codes
        double ss = 0.0;
        for (int t = 0; t < tiles; ++t) ss += s_sum[t];
        const float dhm = act_scale(a);
        dh[m] = dhm;
        // a row whose Z is all zero has zero codes and scale 0
        dz[m] = !(a > 0.0f) ? 0.0f : (float)((double)dhm / sqrt(ss / (double)F + (double)eps));
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
