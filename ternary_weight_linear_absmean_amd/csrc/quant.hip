// quant.hip -- quantisers of the BitLinear W1.58A8 layer on gfx950.
//
// Weights ("Microsoft BitNet 深度研究报告", §2 (2) AbsMean 量化):
//   gamma = (1/n) sum |w_i| over the whole tensor, Q(w) = round(clamp(w /
//   gamma, -1, 1)), stored as 2-bit codes {0: 0, +1: 1, -1: 2}, four per byte
//   (technical-report copy, 推理完满 / GPU端).
// Activations (iaiol.com article, 权重映射为三元值; model card, 模型详情):
//   per-token absmax int8.
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

// ---------------------------------------------------------------------------
// gamma = (1/n) sum |W| in fp64, in one fixed order (the pages fix none):
// within a row, element k goes to partial (k / 4) mod 64 and each partial adds
// its elements in ascending k; the 64 partials are added in consecutive pairs,
// level by level; the row sums, zero-extended to a power of two, are added in
// consecutive pairs the same way; then / n in fp64 and one rounding to fp32.
// Every term is >= 0, so adding +0.0 (tails, padding) changes nothing.

// Row sums, one wave per row: lane l is partial l, reading the float4 units
// l, l + 64, ... of its row (coalesced, eight units in flight), and the
// partials are added in consecutive pairs by shuffles (after the step with
// offset h, lane i * 2h holds the pair sum of its 2h-lane group).
constexpr int kRowsumWaves = 4;
constexpr int kRowsumUnroll = 8;

__global__ __launch_bounds__(64 * kRowsumWaves) void rowsum_abs_kernel(const float *__restrict__ W,
                                                                       int64_t N, int64_t K,
                                                                       double *__restrict__ rowsum) {
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * kRowsumWaves + (threadIdx.x >> 6);
    if (n >= N)
        return;                                   // whole wave; no barrier follows
    const float *row = W + n * K;
    const int64_t units = K / 4;                  // K % 4 == 0
    double p = 0.0;
    for (int64_t u0 = lane; u0 < units; u0 += 64 * kRowsumUnroll) {
        float4 v[kRowsumUnroll];
#pragma unroll
        for (int i = 0; i < kRowsumUnroll; ++i) {
            const int64_t u = u0 + 64 * i;
            v[i] = u < units ? *reinterpret_cast<const float4 *>(row + 4 * u)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < kRowsumUnroll; ++i) {
            p += fabs((double)v[i].x);
            p += fabs((double)v[i].y);
            p += fabs((double)v[i].z);
            p += fabs((double)v[i].w);
        }
    }
#pragma unroll
    for (int h = 1; h < 64; h *= 2) p += __shfl_down(p, h);
    if (lane == 0)
        rowsum[n] = p;
}

// Total: one workgroup of 1024 threads takes the row sums in chunks of 8192
// (thread t: 8 consecutive values, added in pairs in registers; then lanes by
// shuffles; then the 16 wave sums in wave 0) -- each chunk sum is a subtree
// of the zero-extended pair tree.  The chunk sums are combined with a carry
// stack, as in binary counting: chunk c is pushed, and while the subtree at
// the top has a left sibling of the same size they are added, left + right.
// At the end the stack is folded from the top (a missing right sibling is a
// zero subtree, and x + 0 = x).
constexpr int kGammaThreads = 1024;
constexpr int kGammaChunk = 8 * kGammaThreads;

__global__ __launch_bounds__(kGammaThreads) void gamma_kernel(const double *__restrict__ rowsum,
                                                              int64_t N, int64_t K,
                                                              float *__restrict__ gamma) {
    __shared__ double wsum[kGammaThreads / 64];
    __shared__ double stack[48];                  // thread 0's carry stack, one entry per level
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int depth = 0;                                // meaningful in thread 0
    const int64_t chunks = (N + kGammaChunk - 1) / kGammaChunk;
    for (int64_t c = 0; c < chunks; ++c) {
        double e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t idx = c * kGammaChunk + 8 * t + i;
            e[i] = idx < N ? rowsum[idx] : 0.0;
        }
        double s = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
#pragma unroll
        for (int h = 1; h < 64; h *= 2) s += __shfl_down(s, h);
        if (lane == 0)
            wsum[wave] = s;
        __syncthreads();
        double w = lane < kGammaThreads / 64 ? wsum[lane] : 0.0;
#pragma unroll
        for (int h = 1; h < kGammaThreads / 64; h *= 2) w += __shfl_down(w, h);
        __syncthreads();                          // wsum is rewritten by the next chunk
        if (t == 0) {                             // lane 0 of wave 0 holds the chunk sum
            double sub = w;
            for (int64_t k = c; k & 1; k >>= 1) sub = stack[--depth] + sub;
            stack[depth++] = sub;
        }
    }
    if (t == 0) {
        double total = 0.0;
        if (depth > 0) {
            total = stack[--depth];
            while (depth > 0) total = stack[--depth] + total;
        }
        gamma[0] = (N * K == 0) ? 0.0f : (float)(total / (double)(N * K));
    }
}

// Ternarise and pack: one output byte (four weights) per thread.
// round(clamp(w / gamma, -1, 1)) is +-1 exactly when |w / gamma| > 1/2 (a
// tie |w / gamma| == 1/2 rounds to the even 0), i.e. when 2|w| > gamma.  The
// comparison is done in fp64, where 2|w| is exact, so no division is needed.
__global__ __launch_bounds__(256) void ternarize_pack_kernel(const float *__restrict__ W,
                                                             int64_t N, int64_t K,
                                                             const float *__restrict__ gamma,
                                                             uint8_t *__restrict__ Wp) {
    const int64_t KB = K / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= N * KB)
        return;
    const double g = (double)gamma[0];
    const float4 v = *reinterpret_cast<const float4 *>(W + 4 * idx);   // row-major: byte idx
    const float w[4] = {v.x, v.y, v.z, v.w};
    uint32_t byte = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double aw = fabs((double)w[j]);
        uint32_t code = 0;
        if (2.0 * aw > g)
            code = (w[j] > 0.0f) ? 1u : 2u;
        byte |= code << (2 * j);
    }
    Wp[idx] = (uint8_t)byte;
}

// ---------------------------------------------------------------------------
// Per-token absmax int8: one workgroup per token row.
//   a = max |x|;  s = fl(127 / a);  q = clamp(rne(fl(x * s)), -127, 127);
//   d = fl(a / 127);  a == 0 -> q = 0, d = 0.
constexpr int kActThreads = 256;

template <int DT>
__device__ __forceinline__ float load_x(const void *X, int64_t i) {
    if constexpr (DT == 0) {
        return reinterpret_cast<const float *>(X)[i];
    } else {
        const uint32_t b = reinterpret_cast<const uint16_t *>(X)[i];
        return __uint_as_float(b << 16);
    }
}

template <int DT>
__device__ __forceinline__ float4 load_x4(const void *X, int64_t i) {  // i % 4 == 0
    if constexpr (DT == 0) {
        return *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(X) + i);
    } else {
        const uint2 b = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(X) + i);
        return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                           __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u));
    }
}


__device__ __forceinline__ float block_max(float v, float *red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kActThreads / 64; ++w)
        r = fmaxf(r, red[w]);
    return r;
}

// One pass for rows of at most 8192 elements, K % 8 == 0: thread t holds the
// 8-element groups t, t + 256, ... of its row in registers (all loads in
// flight at once: 16 bytes per load for bf16, 2 x 16 for fp32), so X is
// read once; the codes go out as 8-byte words.  Same arithmetic as below.
constexpr int kActGroups = 4;                     // groups per thread: K <= 8192

template <int DT>
__global__ __launch_bounds__(kActThreads) void quant_act_row_kernel(const void *__restrict__ X,
                                                                    int64_t K,
                                                                    int8_t *__restrict__ Xq,
                                                                    float *__restrict__ d) {
    __shared__ float red[kActThreads / 64];
    const int64_t m = blockIdx.x;
    const int groups = (int)(K / 8);
    float x[kActGroups][8];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kActGroups; ++i) {
        const int g = threadIdx.x + kActThreads * i;
        const int gc = min(g, groups - 1);            // a valid address; unused when g >= groups
        if constexpr (DT == 0) {
            const float4 *src = reinterpret_cast<const float4 *>(X) + ((size_t)m * K + 8 * gc) / 4;
            const float4 v0 = src[0], v1 = src[1];
            x[i][0] = v0.x; x[i][1] = v0.y; x[i][2] = v0.z; x[i][3] = v0.w;
            x[i][4] = v1.x; x[i][5] = v1.y; x[i][6] = v1.z; x[i][7] = v1.w;
        } else {
            const uint4 b = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(X) +
                                                           (size_t)m * K + 8 * gc);
            const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[i][2 * t] = __uint_as_float(w[t] << 16);
                x[i][2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
            }
        }
        if (g < groups) {
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[i][e]));
        }
    }
    a = block_max(a, red);
    const float s = act_inv_scale(a);
#pragma unroll
    for (int i = 0; i < kActGroups; ++i) {
        const int g = threadIdx.x + kActThreads * i;
        if (g < groups) {
            uint32_t q[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                q[h] = (uint32_t)(act_code(x[i][4 * h], s) & 0xFF) |
                       ((uint32_t)(act_code(x[i][4 * h + 1], s) & 0xFF) << 8) |
                       ((uint32_t)(act_code(x[i][4 * h + 2], s) & 0xFF) << 16) |
                       ((uint32_t)(act_code(x[i][4 * h + 3], s) & 0xFF) << 24);
            *reinterpret_cast<uint2 *>(Xq + (size_t)m * K + 8 * g) = make_uint2(q[0], q[1]);
        }
    }
    if (threadIdx.x == 0)
        d[m] = act_scale(a);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kActThreads) void quant_act_kernel(const void *__restrict__ X,
                                                                int64_t K,
                                                                int8_t *__restrict__ Xq,
                                                                float *__restrict__ d) {
    __shared__ float red[kActThreads / 64];
    const int64_t m = blockIdx.x;
    const int64_t base = m * K;
    float a = 0.0f;
    if constexpr (VEC) {
        for (int64_t k = 4 * (int64_t)threadIdx.x; k < K; k += 4 * kActThreads) {
            const float4 v = load_x4<DT>(X, base + k);
            a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    } else {
        for (int64_t k = threadIdx.x; k < K; k += kActThreads)
            a = fmaxf(a, fabsf(load_x<DT>(X, base + k)));
    }
    a = block_max(a, red);
    const float s = act_inv_scale(a);
    if constexpr (VEC) {
        for (int64_t k = 4 * (int64_t)threadIdx.x; k < K; k += 4 * kActThreads) {
            const float4 v = load_x4<DT>(X, base + k);
            const uint32_t q = (uint32_t)(act_code(v.x, s) & 0xFF) |
                               ((uint32_t)(act_code(v.y, s) & 0xFF) << 8) |
                               ((uint32_t)(act_code(v.z, s) & 0xFF) << 16) |
                               ((uint32_t)(act_code(v.w, s) & 0xFF) << 24);
            *reinterpret_cast<uint32_t *>(Xq + base + k) = q;
        }
    } else {
        for (int64_t k = threadIdx.x; k < K; k += kActThreads)
            Xq[base + k] = (int8_t)act_code(load_x<DT>(X, base + k), s);
    }
    if (threadIdx.x == 0)
        d[m] = act_scale(a);
}

}  // namespace

hipError_t launch_quant_weight(const float *W, int64_t N, int64_t K, uint8_t *Wp, float *gamma,
                               double *rowsum, hipStream_t s) {
    if (N == 0 || K == 0) {   // gamma = 0, nothing to pack
        hipLaunchKernelGGL(gamma_kernel, dim3(1), dim3(kGammaThreads), 0, s, rowsum, (int64_t)0, K, gamma);
        return hipGetLastError();
    }
    const unsigned nb_rows = (unsigned)((N + kRowsumWaves - 1) / kRowsumWaves);
    hipLaunchKernelGGL(rowsum_abs_kernel, dim3(nb_rows), dim3(64 * kRowsumWaves), 0, s, W, N, K, rowsum);
    hipLaunchKernelGGL(gamma_kernel, dim3(1), dim3(kGammaThreads), 0, s, rowsum, N, K, gamma);
    const int64_t bytes = N * (K / 4);
    const unsigned nb = (unsigned)((bytes + 255) / 256);
    hipLaunchKernelGGL(ternarize_pack_kernel, dim3(nb), dim3(256), 0, s, W, N, K, gamma, Wp);
    return hipGetLastError();
}

hipError_t launch_quant_act(const void *X, int dtype, int64_t M, int64_t K, int8_t *Xq, float *d,
                            hipStream_t s) {
    if (M == 0)
        return hipSuccess;
    const bool vec = (K % 4) == 0;
    const dim3 grid((unsigned)M), block(kActThreads);
    if (K > 0 && K % 8 == 0 && K <= 8 * kActThreads * kActGroups) {
        if (dtype == 0) hipLaunchKernelGGL(quant_act_row_kernel<0>, grid, block, 0, s, X, K, Xq, d);
        else            hipLaunchKernelGGL(quant_act_row_kernel<1>, grid, block, 0, s, X, K, Xq, d);
        return hipGetLastError();
    }
    if (dtype == 0) {
        if (vec) hipLaunchKernelGGL((quant_act_kernel<0, true>), grid, block, 0, s, X, K, Xq, d);
        else     hipLaunchKernelGGL((quant_act_kernel<0, false>), grid, block, 0, s, X, K, Xq, d);
    } else {
        if (vec) hipLaunchKernelGGL((quant_act_kernel<1, true>), grid, block, 0, s, X, K, Xq, d);
        else     hipLaunchKernelGGL((quant_act_kernel<1, false>), grid, block, 0, s, X, K, Xq, d);
    }
    return hipGetLastError();
}

}  // namespace bl
