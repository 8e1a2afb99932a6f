// gemv.hip -- W1.58A8 product for a handful of tokens (decode), on the VALU.
//
// The product is the add / subtract / skip accumulation of "Microsoft BitNet
// 深度研究报告", §2 (3) 查找表优化, over the packed 2-bit weights of the
// technical-report copy's GPU端 section (load the packed weights, unpack in
// registers, compute).  On gfx950 one v_perm_b32 turns four 2-bit codes into
// four int8 values {0, +1, -1} and one v_dot4_i32_i8 adds the four signed
// products into an int32: about 0.8 VALU instructions per weight, below the
// rate at which HBM delivers packed weights to a CU.
//
// Layout of the work: a workgroup is 4 waves; each wave owns R = 64 / L rows
// and each row is split over L lanes.  Lane s of a row reads the 16-byte
// units (64 weights each) s, s + L, s + 2L, ... of that row, so every load
// instruction of a wave covers R runs of L consecutive 16-byte units.  The
// activations are staged once per workgroup in LDS, put into the transposed
// order that the unpacked weights come out in.  The int32 partial sums of a
// row are added across its L lanes with cross-lane shuffles, and the lane
// that ends with the row's sum applies the fp32 rescale.
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kUnitsInFlight = 4;           // 16-byte loads issued before use
constexpr int kXBytes = 64 * 1024;          // LDS budget for staged activations

template <int L, int MT>
__device__ __forceinline__ void dot_unit(const uint4 &w, const uint4 *xs, int gpc, int ul,
                                         int (&acc)[MT]) {
    const uint32_t dws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t v0, v1, v2, v3;
        unpack16(dws[t], v0, v1, v2, v3);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4 xv = xs[m * gpc + 4 * ul + t];
            int a = acc[m];
            a = dot4(v0, xv.x, a);
            a = dot4(v1, xv.y, a);
            a = dot4(v2, xv.z, a);
            a = dot4(v3, xv.w, a);
            acc[m] = a;
        }
    }
}

template <int L>
__device__ __forceinline__ void load_units(uint4 (&w)[kUnitsInFlight], const uint4 *wrow, int u,
                                           int ue) {
#pragma unroll
    for (int j = 0; j < kUnitsInFlight; ++j)
        w[j] = wrow[min(u + j * L, ue - 1)];            // clamped: always in bounds
}

template <int L, int MT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ d, int M,
    const uint8_t *__restrict__ Wp, const float *__restrict__ gamma, int N, int K, int KC,
    float *__restrict__ Y, int32_t *__restrict__ acc_out) {
    constexpr int R = 64 / L;
    extern __shared__ uint4 xs[];                     // [MT][KC / 16], transposed groups
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int r = lane / L;
    const int s = lane % L;
    const int row = (blockIdx.x * (kThreads / 64) + (tid >> 6)) * R + r;
    const int m0 = blockIdx.y * MT;
    const int mt = min(MT, M - m0);
    const int gpc = KC / 16;                           // 16-byte groups per staged row
    // Rows past N read the last row (in bounds) and are never stored.
    const uint4 *wrow = reinterpret_cast<const uint4 *>(Wp + (size_t)min(row, N - 1) * (K / 4));

    int acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0;

    for (int kc0 = 0; kc0 < K; kc0 += KC) {
        const int kc = min(KC, K - kc0);
        const int ub = kc0 / 64;
        const int ue = ub + kc / 64;
        // The first weight loads do not depend on the activations: issue them
        // before staging, so the two memory latencies overlap.
        uint4 w[kUnitsInFlight];
        load_units<L>(w, wrow, ub + s, ue);
        const int groups = kc / 16;
        __syncthreads();                               // previous chunk consumed
        for (int i = tid; i < mt * groups; i += kThreads) {
            const int m = i / groups;
            const int g = i - m * groups;
            const uint4 v = *reinterpret_cast<const uint4 *>(Xq + (size_t)(m0 + m) * K + kc0 + 16 * g);
            xs[m * gpc + g] = transpose16(v);
        }
        __syncthreads();
        for (int u = ub + s; u < ue; u += L * kUnitsInFlight) {
            // software pipeline: the next batch is in flight while this one computes
            uint4 wn[kUnitsInFlight];
            const int un = u + L * kUnitsInFlight;
            if (un < ue)
                load_units<L>(wn, wrow, un, ue);
#pragma unroll
            for (int j = 0; j < kUnitsInFlight; ++j)
                if (u + j * L < ue)
                    dot_unit<L, MT>(w[j], xs, gpc, u + j * L - ub, acc);
            if (un < ue) {
#pragma unroll
                for (int j = 0; j < kUnitsInFlight; ++j) w[j] = wn[j];
            }
        }
    }

#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int off = L / 2; off > 0; off >>= 1)
            acc[m] += __shfl_xor(acc[m], off);
    }
    if (row < N && s == 0) {
        const float g = gamma[0];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < mt) {
                const size_t o = (size_t)(m0 + m) * N + row;
                Y[o] = rescale(acc[m], __fmul_rn(g, d[m0 + m]));
                if (acc_out) acc_out[o] = acc[m];
            }
        }
    }
}

template <int L, int MT>
hipError_t launch_lm(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                     const float *gamma, int N, int K, float *Y, int32_t *acc, hipStream_t s) {
    constexpr int rows_per_wg = (kThreads / 64) * (64 / L);
    int KC = (kXBytes / MT) / 64 * 64;
    if (KC > K) KC = K;
    const dim3 grid((N + rows_per_wg - 1) / rows_per_wg, (M + MT - 1) / MT);
    const size_t lds = (size_t)MT * KC;
    hipLaunchKernelGGL((gemv_kernel<L, MT>), grid, dim3(kThreads), lds, s,
                       Xq, d, M, Wp, gamma, N, K, KC, Y, acc);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_m(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                    const float *gamma, int N, int K, float *Y, int32_t *acc, hipStream_t s) {
    const int U = K / 64;                               // 16-byte units per row
    int L = U >= 96 ? 64 : U >= 48 ? 32 : 16;
#ifdef BL_GEMV_FORCE_L
    L = BL_GEMV_FORCE_L;                                // tuning builds only
#endif
    switch (L) {
    case 8: return launch_lm<8, MT>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    case 16: return launch_lm<16, MT>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    case 32: return launch_lm<32, MT>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    default: return launch_lm<64, MT>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    }
}

}  // namespace

hipError_t launch_gemv(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                       const float *gamma, int N, int K, float *Y, int32_t *acc,
                       hipStream_t s) {
    if (M == 0 || N == 0)
        return hipSuccess;
    if (M == 1) return launch_m<1>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    if (M == 2) return launch_m<2>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    if (M <= 4) return launch_m<4>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    return launch_m<8>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
}

}  // namespace bl
