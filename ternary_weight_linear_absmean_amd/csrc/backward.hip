// backward.hip -- QAT backward through BitLinear on bf16 MFMA.
//
// "Microsoft BitNet 深度研究报告", §2 (4) 量化感知训练: the forward runs on the
// quantised weights and the backward passes the gradient through the
// quantisers with the straight-through estimator; the optimiser updates the
// latent weights.  With X~ = Xq d and W~ = gamma Wq the forward operands, the
// gradients of the latent X and W are
//     dX = dY . W~ = gamma (dY . Wq)          [M][K]
//     dW = dY^T . X~ = (dY o d)^T . Xq        [N][K]
// Both multiply fp32 gradients by small integers ({-1, 0, +1} or int8
// codes), which bf16 holds exactly.  Each fp32 value a is split into
// hi = bf16(a) and lo = bf16(a - hi) (a = hi + lo to about 2^-17 relative)
// and v_mfma_f32_32x32x16_bf16 takes both halves against the same integer
// operand: every product is exact in fp32, only the fp32 accumulation rounds.
//
// One product kernel, C[i][j] = s . sum_c A[i][c] B[j][c], A fp32 and B int8,
// both contraction-contiguous.  Transpose kernels put the operands in that
// form (rows padded to a multiple of 64, pads written as zeros):
//     dX:  A = dY [M][N],              B = Wq^T [K][Np],   s = gamma
//     dW:  A = (dY o d)^T [N][Mp],     B = Xq^T [K][Mp],   s = 1
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;                         // transpose tile (elements)

// Wq^T [K][ld] (int8) from the packed rows Wp [N][K/4]: tile of 64 rows n x
// 64 weights k; codes {0, 1, 2} -> {0, +1, -1}; columns n >= N are zeros.
__global__ __launch_bounds__(256) void unpack_transpose_kernel(const uint8_t *__restrict__ Wp, int N,
                                                               int K, int8_t *__restrict__ WT,
                                                               int ld) {
    __shared__ int8_t s[kTile][kTile + 16];      // 80-byte rows: 16-byte aligned reads
    const int t = threadIdx.x;
    const int n0 = blockIdx.x * kTile, k0 = blockIdx.y * kTile;
    {
        const int r = t >> 2, q = t & 3;                  // row n0 + r, 16 weights per dword q
        uint32_t dw = 0u;
        if (n0 + r < N)
            dw = *reinterpret_cast<const uint32_t *>(Wp + (size_t)(n0 + r) * (K / 4) + k0 / 4 + 4 * q);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t c = (dw >> (2 * j)) & 3u;
            s[16 * q + j][r] = (int8_t)((int)(c & 1u) - (int)(c >> 1));
        }
    }
    __syncthreads();
    const int k = t >> 2, seg = t & 3;                    // row k0 + k, 16 columns per segment
    const uint4 v = *reinterpret_cast<const uint4 *>(&s[k][16 * seg]);
    *reinterpret_cast<uint4 *>(WT + (size_t)(k0 + k) * ld + n0 + 16 * seg) = v;
}

// G^T [N][ld] (fp32) = (dY o d)^T: G^T[n][m] = fl(dY[m][n] * d[m]); columns
// m >= M are zeros.
__global__ __launch_bounds__(256) void transpose_scale_kernel(const float *__restrict__ dY,
                                                              const float *__restrict__ d, int M,
                                                              int N, float *__restrict__ GT, int ld) {
    __shared__ float s[kTile][kTile + 1];
    const int t = threadIdx.x;
    const int m0 = blockIdx.x * kTile, n0 = blockIdx.y * kTile;
#pragma unroll
    for (int p = 0; p < kTile * kTile / 256; ++p) {
        const int e = t + 256 * p;
        const int r = e >> 6, c = e & 63;                 // dY row m0 + r, column n0 + c
        float v = 0.0f;
        if (m0 + r < M && n0 + c < N) v = __fmul_rn(dY[(size_t)(m0 + r) * N + n0 + c], d[m0 + r]);
        s[c][r] = v;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kTile * kTile / 256; ++p) {
        const int e = t + 256 * p;
        const int r = e >> 6, c = e & 63;                 // G^T row n0 + r, column m0 + c
        if (n0 + r < N) GT[(size_t)(n0 + r) * ld + m0 + c] = s[r][c];
    }
}

// Xq^T [K][ld] (int8); columns m >= M are zeros.
__global__ __launch_bounds__(256) void transpose_i8_kernel(const int8_t *__restrict__ Xq, int M,
                                                           int K, int8_t *__restrict__ XT, int ld) {
    __shared__ int8_t s[kTile][kTile + 16];      // 80-byte rows: 16-byte aligned reads
    const int t = threadIdx.x;
    const int m0 = blockIdx.x * kTile, k0 = blockIdx.y * kTile;
    {
        const int r = t >> 2, seg = t & 3;                // Xq row m0 + r, 16 columns k per segment
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (m0 + r < M)
            v = *reinterpret_cast<const uint4 *>(Xq + (size_t)(m0 + r) * K + k0 + 16 * seg);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) s[16 * seg + j][r] = (int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFF);
    }
    __syncthreads();
    const int k = t >> 2, seg = t & 3;
    const uint4 v = *reinterpret_cast<const uint4 *>(&s[k][16 * seg]);
    *reinterpret_cast<uint4 *>(XT + (size_t)(k0 + k) * ld + m0 + 16 * seg) = v;
}

// ------------------------------------------------------------- the product
constexpr int kBI = 128, kBJ = 128, kBC = 32;
constexpr int kLP = kBC + 8;                      // bf16 per staged row (+8 pad: 80 bytes)

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;   // finite inputs
}
__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }

struct StageNT {
    float4 a[4];                                  // 128 x 32 fp32 of A: 4 float4 per thread
    uint4 b;                                      // 128 x 32 int8 of B: 16 bytes per thread
};

__device__ __forceinline__ void load_nt(StageNT &st, const float *__restrict__ A, int lda,
                                        const int8_t *__restrict__ B, int ldb, int I, int J, int C,
                                        int i0, int j0, int c0, int t) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int e = t + 256 * p;
        const int r = e >> 3, q = e & 7;                  // row i0 + r, columns c0 + 4q .. + 3
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i0 + r < I && c0 + 4 * q < C)                 // C % 4 == 0
            v = *reinterpret_cast<const float4 *>(A + (size_t)(i0 + r) * lda + c0 + 4 * q);
        st.a[p] = v;
    }
    const int r = t >> 1, h = t & 1;                      // row j0 + r, columns c0 + 16h .. + 15
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (j0 + r < J) v = *reinterpret_cast<const uint4 *>(B + (size_t)(j0 + r) * ldb + c0 + 16 * h);
    st.b = v;
}

// A -> hi / lo bf16 planes, B -> bf16 (exact: |b| <= 127), into LDS rows of kLP.
__device__ __forceinline__ void store_nt(const StageNT &st, uint32_t *Ahi, uint32_t *Alo, uint32_t *Bs,
                                         int t) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int e = t + 256 * p;
        const int r = e >> 3, q = e & 7;
        const float x[4] = {st.a[p].x, st.a[p].y, st.a[p].z, st.a[p].w};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            hi[u] = bf16_rne(x[u]);
            lo[u] = bf16_rne(x[u] - __uint_as_float(hi[u] << 16));   // exact difference
        }
        uint32_t *ph = Ahi + r * (kLP / 2) + 2 * q;
        uint32_t *pl = Alo + r * (kLP / 2) + 2 * q;
        *reinterpret_cast<uint2 *>(ph) = make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
        *reinterpret_cast<uint2 *>(pl) = make_uint2(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
    }
    const int r = t >> 1, h = t & 1;
    const uint32_t w[4] = {st.b.x, st.b.y, st.b.z, st.b.w};
    uint32_t o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int b0 = (int)(int8_t)((w[u >> 1] >> (16 * (u & 1))) & 0xFF);
        const int b1 = (int)(int8_t)((w[u >> 1] >> (16 * (u & 1) + 8)) & 0xFF);
        o[u] = pack2(__float_as_uint((float)b0) >> 16, __float_as_uint((float)b1) >> 16);
    }
    uint4 *pb = reinterpret_cast<uint4 *>(Bs + r * (kLP / 2) + 8 * h);
    pb[0] = make_uint4(o[0], o[1], o[2], o[3]);
    pb[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// C[i][j] = s . sum_{c < C} A[i][c] B[j][c]; 128 x 128 tiles, 4 waves of
// 64 x 64 (2 x 2 blocks of 32 x 32); 32-wide c-steps, LDS double-buffered,
// the next step's operands loaded while the current one computes.
__global__ __launch_bounds__(256) void gemm_nt_f32i8_kernel(
    const float *__restrict__ A, int lda, const int8_t *__restrict__ B, int ldb, int I, int J, int C,
    const float *__restrict__ scale, float *__restrict__ Out, int ldo) {
    constexpr int kPlane = kBI * kLP / 2;                 // dwords per 128-row bf16 plane
    __shared__ uint32_t lds[2][3][kPlane];                // [buffer][A hi, A lo, B]
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wi = wave >> 1, wj = wave & 1;
    const int i0 = blockIdx.x * kBI, j0 = blockIdx.y * kBJ;
    const int steps = (C + kBC - 1) / kBC;

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    StageNT st;
    if (steps > 0) {
        load_nt(st, A, lda, B, ldb, I, J, C, i0, j0, 0, t);
        store_nt(st, lds[0][0], lds[0][1], lds[0][2], t);
        if (steps > 1) load_nt(st, A, lda, B, ldb, I, J, C, i0, j0, kBC, t);
    }
    __syncthreads();
    for (int s = 0; s < steps; ++s) {
        const int buf = s & 1;
        const uint32_t *Ahi = lds[buf][0], *Alo = lds[buf][1], *Bs = lds[buf][2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {               // 16 c per MFMA
            const int col = (16 * sub + 8 * (lane >> 5)) / 2;      // dword offset in a row
            bf16x8 ah[2], al[2], bb[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int row = wi * 64 + a * 32 + (lane & 31);
                ah[a] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Ahi + row * (kLP / 2) + col));
                al[a] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Alo + row * (kLP / 2) + col));
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int row = wj * 64 + b * 32 + (lane & 31);
                bb[b] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(Bs + row * (kLP / 2) + col));
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[a], bb[b], acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[a], bb[b], acc[a][b], 0, 0, 0);
                }
        }
        if (s + 1 < steps) {
            store_nt(st, lds[buf ^ 1][0], lds[buf ^ 1][1], lds[buf ^ 1][2], t);
            if (s + 2 < steps) load_nt(st, A, lda, B, ldb, I, J, C, i0, j0, (s + 2) * kBC, t);
        }
        __syncthreads();
    }

    const float sc = scale ? scalar_load(scale) : 1.0f;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = i0 + wi * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (i >= I) continue;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int j = j0 + wj * 64 + b * 32 + (lane & 31);
                if (j < J) Out[(size_t)i * ldo + j] = scale ? __fmul_rn(acc[a][b][r], sc) : acc[a][b][r];
            }
        }
}

int64_t pad64(int64_t v) { return (v + 63) / 64 * 64; }
size_t round256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t backward_input_ws_bytes(int64_t N, int64_t K) { return (size_t)K * (size_t)pad64(N); }

size_t backward_weight_ws_bytes(int64_t M, int64_t N, int64_t K) {
    const size_t mp = (size_t)pad64(M);
    return round256((size_t)N * mp * 4) + (size_t)K * mp;
}

// Sizes as validated by the entry points: M, N < 2^31 - 63, K % 64 == 0.
// An empty contraction (N == 0 for dX, M == 0 for dW) reads no operand: the
// product kernel then writes zeros.
hipError_t launch_backward_input(const float *dY, int M, int N, const uint8_t *Wp, const float *gamma,
                                 int K, float *dX, void *ws, hipStream_t s) {
    if (M == 0 || K == 0)
        return hipSuccess;
    const int np = (int)pad64(N);
    int8_t *WT = static_cast<int8_t *>(ws);
    if (np > 0)
        hipLaunchKernelGGL(unpack_transpose_kernel, dim3(np / kTile, K / kTile), dim3(256), 0, s, Wp,
                           N, K, WT, np);
    hipLaunchKernelGGL(gemm_nt_f32i8_kernel, dim3((M + kBI - 1) / kBI, (K + kBJ - 1) / kBJ), dim3(256),
                       0, s, dY, N, WT, np, M, K, N, np > 0 ? gamma : nullptr, dX, K);
    return hipGetLastError();
}

hipError_t launch_backward_weight(const float *dY, int M, int N, const int8_t *Xq, const float *d,
                                  int K, float *dW, void *ws, hipStream_t s) {
    if (N == 0 || K == 0)
        return hipSuccess;
    const int mp = (int)pad64(M);
    float *GT = static_cast<float *>(ws);
    int8_t *XT = static_cast<int8_t *>(ws) + round256((size_t)N * mp * 4);
    if (mp > 0) {
        hipLaunchKernelGGL(transpose_scale_kernel, dim3(mp / kTile, (N + kTile - 1) / kTile), dim3(256),
                           0, s, dY, d, M, N, GT, mp);
        hipLaunchKernelGGL(transpose_i8_kernel, dim3(mp / kTile, K / kTile), dim3(256), 0, s, Xq, M, K,
                           XT, mp);
    }
    hipLaunchKernelGGL(gemm_nt_f32i8_kernel, dim3((N + kBI - 1) / kBI, (K + kBJ - 1) / kBJ), dim3(256),
                       0, s, GT, mp, XT, mp, N, K, mp, nullptr, dW, K);
    return hipGetLastError();
}

}  // namespace bl
