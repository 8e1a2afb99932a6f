// gemm.hip -- W1.58A8 product for many tokens (prefill) on int8 MFMA.
//
// The technical-report copy (推理完满 / GPU端) describes the W1.58A8 kernel as
// pack, store, load, unpack, compute over four ternary weights per int8.  At
// M = 2048 the product is compute-bound, so on gfx950 the unpacked ternary
// tile goes through v_mfma_i32_16x16x64_i8 with int32 accumulation: the
// ternary values {-1, 0, +1} are exact int8 operands and every int32 sum is
// exact.  The rescale Y = float(acc) * fl(gamma * d[m]) is applied in the
// epilogue.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of Y as a 2 x 2
// grid of waves, each owning 64 x 64 = 4 x 4 MFMA blocks of 16 x 16.  Per
// 64-wide k-step the activation tile (128 rows x 64 int8) and the packed
// weight tile (128 rows x 16 bytes) are read from global memory; the
// weights are unpacked (v_perm byte lookup) into int8 in LDS.  Both operands
// use the same transposed order inside every 16-byte group (see
// device_common.h), so each MFMA lane multiplies matching k.
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kPitch = BK / 16 + 1;      // uint4 per LDS row: 4 groups + 1 pad

__device__ __forceinline__ v4i as_v4i(uint4 v) {
    v4i r;
    r.x = (int)v.x; r.y = (int)v.y; r.z = (int)v.z; r.w = (int)v.w;
    return r;
}

__global__ __launch_bounds__(256) void gemm_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ d, int M,
    const uint8_t *__restrict__ Wp, const float *__restrict__ gamma, int N, int K,
    float *__restrict__ Y, int32_t *__restrict__ acc_out) {
    __shared__ uint4 As[BM * kPitch];
    __shared__ uint4 Bs[BN * kPitch];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int m_base = blockIdx.y * BM;
    const int n_base = blockIdx.x * BN;
    const int KB = K / 4;

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = v4i{0, 0, 0, 0};

    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx >> 2;
            const int g = idx & 3;
            const int gm = m_base + r;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (gm < M)
                v = *reinterpret_cast<const uint4 *>(Xq + (size_t)gm * K + k0 + 16 * g);
            As[r * kPitch + g] = transpose16(v);
        }
        if (tid < BN) {
            const int gn = n_base + tid;
            uint4 w = make_uint4(0u, 0u, 0u, 0u);
            if (gn < N)
                w = *reinterpret_cast<const uint4 *>(Wp + (size_t)gn * KB + k0 / 4);
            const uint32_t dws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint4 o;
                unpack16(dws[g], o.x, o.y, o.z, o.w);
                Bs[tid * kPitch + g] = o;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v4i a = as_v4i(As[(wm * 64 + i * 16 + (lane & 15)) * kPitch + (lane >> 4)]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4i b = as_v4i(Bs[(wn * 64 + j * 16 + (lane & 15)) * kPitch + (lane >> 4)]);
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[i][j], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // 16 x 16 int32 result block: lane l holds column l % 16, rows 4 (l / 16) + 0..3.
    const float g = gamma[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = m_base + wm * 64 + i * 16 + 4 * (lane >> 4) + rr;
            if (row >= M) continue;
            const float c = __fmul_rn(g, d[row]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n_base + wn * 64 + j * 16 + (lane & 15);
                if (col < N) {
                    const size_t o = (size_t)row * N + col;
                    Y[o] = rescale(acc[i][j][rr], c);
                    if (acc_out) acc_out[o] = acc[i][j][rr];
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                       const float *gamma, int N, int K, float *Y, int32_t *acc,
                       hipStream_t s) {
    if (M == 0 || N == 0)
        return hipSuccess;
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, s, Xq, d, M, Wp, gamma, N, K, Y, acc);
    return hipGetLastError();
}

hipError_t launch_bitlinear(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                            const float *gamma, int N, int K, float *Y, int32_t *acc,
                            hipStream_t s) {
    if (M <= kGemvMaxTokens)
        return launch_gemv(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    return launch_gemm(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
}

}  // namespace bl
