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
// gamma, step 1: fp64 sum of |W[n][k]| over k in ascending order, one row per
// thread.  A wave stages a 64-row x 64-column tile through LDS (coalesced
// float4 loads, 16 per thread), then each thread adds its row's 64 values in
// k order.  The next tile's loads are all issued before the current tile is
// summed, so memory latency overlaps the (inherently sequential) fp64 adds.
// Tail columns are read as 0, and adding +0.0 to a non-negative sum is
// exact, so the result is the plain ascending-k sum.
constexpr int kRowsumRows = 64;
constexpr int kRowsumCols = 64;
constexpr int kRowsumLoads = kRowsumRows * (kRowsumCols / 4) / 64;   // float4 per thread

__global__ __launch_bounds__(64) void rowsum_abs_kernel(const float *__restrict__ W, int64_t N,
                                                        int64_t K, double *__restrict__ rowsum) {
    __shared__ float tile[kRowsumRows][kRowsumCols + 1];
    const int t = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * kRowsumRows;
    // thread t's float4 i covers row (t + 64 i) / 16, columns 4 ((t + 64 i) % 16)..+3
    auto load_tile = [&](int64_t k0, float4 (&v)[kRowsumLoads]) {
#pragma unroll
        for (int i = 0; i < kRowsumLoads; ++i) {
            const int j = t + 64 * i;
            const int64_t n = n0 + j / (kRowsumCols / 4);
            const int64_t k = k0 + 4 * (j % (kRowsumCols / 4));
            v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (n < N && k < K)   // K % 4 == 0, so a float4 never straddles K
                v[i] = *reinterpret_cast<const float4 *>(W + n * K + k);
        }
    };
    float4 v[kRowsumLoads];
    load_tile(0, v);
    double sum = 0.0;
    for (int64_t k0 = 0; k0 < K; k0 += kRowsumCols) {
#pragma unroll
        for (int i = 0; i < kRowsumLoads; ++i) {
            const int j = t + 64 * i;
            const int r = j / (kRowsumCols / 4), c = 4 * (j % (kRowsumCols / 4));
            tile[r][c + 0] = v[i].x;
            tile[r][c + 1] = v[i].y;
            tile[r][c + 2] = v[i].z;
            tile[r][c + 3] = v[i].w;
        }
        __syncthreads();
        if (k0 + kRowsumCols < K) load_tile(k0 + kRowsumCols, v);
        for (int c = 0; c < kRowsumCols; ++c)
            sum += fabs((double)tile[t][c]);
        __syncthreads();
    }
    const int64_t n = n0 + t;
    if (n < N)
        rowsum[n] = sum;
}

// gamma, step 2: add the row sums in ascending n, divide by n in fp64, round
// once to fp32.  The wave stages chunks of row sums in LDS (all loads of a
// chunk in flight together) and lane 0 adds them in order.
constexpr int kGammaChunk = 2048;

__global__ __launch_bounds__(64) void gamma_kernel(const double *__restrict__ rowsum, int64_t N,
                                                   int64_t K, float *__restrict__ gamma) {
    __shared__ double buf[kGammaChunk];
    const int lane = threadIdx.x;
    double total = 0.0;
    for (int64_t c0 = 0; c0 < N; c0 += kGammaChunk) {
        const int cnt = (N - c0) < kGammaChunk ? (int)(N - c0) : kGammaChunk;
        double v[kGammaChunk / 64];
#pragma unroll
        for (int i = 0; i < kGammaChunk / 64; ++i) {
            const int j = lane + 64 * i;
            v[i] = j < cnt ? rowsum[c0 + j] : 0.0;
        }
#pragma unroll
        for (int i = 0; i < kGammaChunk / 64; ++i) buf[lane + 64 * i] = v[i];
        __syncthreads();
        if (lane == 0)
            for (int j = 0; j < cnt; ++j) total += buf[j];
        __syncthreads();
    }
    if (lane == 0)   // mean of an empty tensor: gamma = 0
        gamma[0] = (N * K == 0) ? 0.0f : (float)(total / (double)(N * K));
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
        hipLaunchKernelGGL(gamma_kernel, dim3(1), dim3(64), 0, s, rowsum, (int64_t)0, K, gamma);
        return hipGetLastError();
    }
    const unsigned nb_rows = (unsigned)((N + kRowsumRows - 1) / kRowsumRows);
    hipLaunchKernelGGL(rowsum_abs_kernel, dim3(nb_rows), dim3(64), 0, s, W, N, K, rowsum);
    hipLaunchKernelGGL(gamma_kernel, dim3(1), dim3(64), 0, s, rowsum, N, K, gamma);
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
