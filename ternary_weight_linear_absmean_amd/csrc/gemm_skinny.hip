// gemm_skinny.hip -- W1.58A8 product for a few tokens (M < 128, K <= 8192) on
// int8 MFMA, each workgroup reading its weight rows once.
//
// Same product as gemm.hip (the technical-report copy's GPU端 pack / load /
// unpack / compute, int32 accumulation, rescale fl(float(acc) * fl(gamma d))),
// laid out for small M, where the packed weights are most of the bytes and a
// launch is bound by load latency rather than by MFMA work.
// Integer sums are exact, so the result does not depend on how k is split.
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i as_v4i(uint4 v) {
    v4i r;
    r.x = (int)v.x; r.y = (int)v.y; r.z = (int)v.z; r.w = (int)v.w;
    return r;
}

// A workgroup owns 16 tokens (one token block) and 16 RB weight rows,
// K <= 2048 NR.  Its waves have two roles, as in the fused one-token GEMV:
//   * four staging waves copy the block's 16 code rows into LDS as
//     transposed 16-byte groups, in rounds of 2048 k (128 groups), and count
//     up the round's LDS word after each round; all their loads are issued
//     at once;
//   * eight compute waves request every packed-weight unit they use at
//     kernel start, then per round wait for the count and run the MFMAs.
// A wave's vector loads complete in issue order, so activation loads that a
// wave issues behind its weight requests wait for the whole weight stream;
// with the roles split, the codes reach LDS as the first weights land.
// (Kernels that staged the codes behind their own weight loads took 7.3 /
// 9.7 / 14.4 us at M = 8 / 32 / 64, K6912 -> N2560, against 5.5 / 6.4 / 8.6.)
//
// k layout: unit u of a row is weights [64 u, +64), packed bytes [16 u, +16).
// Compute wave cw takes the unit quads qd = cw + 8 rho (rho = round); lane
// (r = lane % 16, g = lane / 16) holds unit 4 qd + g of row r of each row
// block and feeds its dword t to MFMA step t: weights k in
// [256 qd + 64 g + 16 t, +16) against activation group 16 qd + 4 g + t of
// token r (the A operand of v_mfma_i32_16x16x64_i8).  Codes past M or past
// K are staged as zeros (each staging load's buffer range is one token row),
// so the weight units past K may hold anything: their products are zero.
// Each token block re-reads the row group's weights; the grid puts all
// token blocks of a row group on one XCD (workgroup x runs on XCD x % 8), so
// those re-reads meet one L2.
constexpr int kFwStageThreads = 256;              // four staging waves
constexpr int kFwComputeWaves = 8;
constexpr int kFwThreads = kFwStageThreads + 64 * kFwComputeWaves;
constexpr int kFwRoundGroups = 128;               // 16-code groups per round: 8 waves x 4 units x 4
constexpr int kFwMaxRounds = 4;                   // K <= 8192
// Buffer resource word 3 for raw (untyped, unswizzled) loads: 32-bit data
// format; a load at or past num_records bytes returns zeros.
constexpr int kRawBufferWord3 = 0x00020000;

template <int RB, int NR>
__global__ __launch_bounds__(kFwThreads) void gemm_few_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ d, int M,
    const uint8_t *__restrict__ Wp, const float *__restrict__ gamma, int N, int K,
    float *__restrict__ Y, int32_t *__restrict__ acc_out, int ntb, int nrg) {
    constexpr int P = kFwRoundGroups * NR + 1;             // uint4 per staged token row (odd)
    constexpr int kXsU4 = 16 * P;
    __shared__ uint4 xs[kXsU4];
    __shared__ int red[RB * 4 * 64];                       // the compute waves' sums, [RB][4][64]
    __shared__ float cS[16];                               // fl(gamma * d[token])
    // staging waves past each round, one word per round: a single count
    // could reach 4 (rho + 1) while a slow wave is still in round rho
    __shared__ unsigned n_staged[NR];
    const int tid = threadIdx.x, lane = tid & 63;
    const int slot = (int)blockIdx.x >> 3;
    const int tb = slot % ntb, rg = (slot / ntb) * 8 + ((int)blockIdx.x & 7);
    if (rg >= nrg)
        return;                                            // the whole workgroup, before any barrier
    const int m0 = 16 * tb, mt = min(16, M - m0);
    const int n0 = 16 * RB * rg;
    if (tid < NR)
        n_staged[tid] = 0u;
    for (int i = tid; i < RB * 4 * 64; i += kFwThreads) red[i] = 0;
    __syncthreads();                                       // nothing is in flight yet

    v4i acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = v4i{0, 0, 0, 0};
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (__builtin_expect(wave < kFwStageThreads / 64, 1)) {
        // ---- staging waves: load i of a round covers 64 consecutive groups
        //      of token (tid / 128) + 2 i, wave-uniform, so each load's buffer
        //      range is that token's row (empty past M)
        const int half = __builtin_amdgcn_readfirstlane(tid >> 7), e = tid & 127;
        __amdgpu_buffer_rsrc_t rs[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = half + 2 * i;
            rs[i] = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<int8_t *>(Xq + (size_t)(m0 + min(t, mt - 1)) * K), (short)0,
                t < mt ? K : 0, kRawBufferWord3);
        }
        uint4 a[NR][8];                                    // round-major: round 0 lands first
#pragma unroll
        for (int rho = 0; rho < NR; ++rho) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const v4u v = __builtin_amdgcn_raw_buffer_load_b128(
                    rs[i], 16 * (kFwRoundGroups * rho + e), 0, 0);
                a[rho][i] = make_uint4(v.x, v.y, v.z, v.w);
            }
            __builtin_amdgcn_sched_barrier(0);             // keep the rounds in issue order
        }
#pragma unroll
        for (int rho = 0; rho < NR; ++rho) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                xs[(half + 2 * i) * P + kFwRoundGroups * rho + e] = transpose16(a[rho][i]);
            // this wave's groups of the round in LDS before the count
            if (lane == 0)
                __hip_atomic_fetch_add(&n_staged[rho], 1u, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        // the row factors, needed only by the epilogue (behind the final barrier)
        if (tid < 16)
            cS[tid] = tid < mt ? __fmul_rn(scalar_load(gamma), d[m0 + tid]) : 0.0f;
    } else {
        // ---- compute waves: every unit requested at once, round 0's first
        const int cw = wave - kFwStageThreads / 64;
        const int r = lane & 15, g = lane >> 4;
        const int U = K >> 6, KB = K >> 2;
        uint4 w[NR][RB];
#pragma unroll
        for (int rho = 0; rho < NR; ++rho) {
            const int u = min(4 * (cw + 8 * rho) + g, U - 1);   // past K: any unit (zero codes)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int row = min(n0 + 16 * rb + r, N - 1);    // past N: discarded outputs
                w[rho][rb] = *reinterpret_cast<const uint4 *>(Wp + (size_t)row * KB + 16 * u);
            }
        }
#pragma unroll
        for (int rho = 0; rho < NR; ++rho) {
            const int qd = cw + 8 * rho;
            if (4 * qd >= U)
                break;                                     // wave-uniform: no unit left
            while (__hip_atomic_load(&n_staged[rho], __ATOMIC_ACQUIRE,
                                     __HIP_MEMORY_SCOPE_WORKGROUP) < 4u)
                __builtin_amdgcn_s_sleep(1);
            const uint4 *A = xs + r * P + 16 * qd + 4 * g;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const v4i af = as_v4i(A[t]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const uint32_t dw = t == 0 ? w[rho][rb].x : t == 1 ? w[rho][rb].y
                                      : t == 2 ? w[rho][rb].z : w[rho][rb].w;
                    uint4 bv;
                    unpack16(dw, bv.x, bv.y, bv.z, bv.w);
                    acc[rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, as_v4i(bv), acc[rb], 0, 0, 0);
                }
            }
        }
    }

    // the eight compute waves' sums (disjoint k) added into LDS with
    // ds_add (int32 sums are exact, so the order of the adds does not
    // matter), then the 16 RB x mt outputs, a token's columns on consecutive
    // threads.  (Each wave's partials written out and summed eight at a time
    // behind a second barrier: 6.15 / 8.50 against 5.92 / 8.15 us at
    // K2560 -> N6912, M = 32 / 64.)
    if (wave >= kFwStageThreads / 64) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                __hip_atomic_fetch_add(&red[(rb * 4 + v) * 64 + lane], acc[rb][v], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    for (int o = tid; o < 256 * RB; o += kFwThreads) {
        const int tok = o / (16 * RB), c = o % (16 * RB);
        const int rb = c >> 4, l = 16 * (tok >> 2) + (c & 15), v = tok & 3;
        const int sum = red[(rb * 4 + v) * 64 + l];
        const int col = n0 + c;
        if (tok < mt && col < N) {
            const size_t off = (size_t)(m0 + tok) * N + col;
            Y[off] = rescale(sum, cS[tok]);
            if (acc_out) acc_out[off] = sum;
        }
    }
}

template <int RB, int NR>
void launch_few(const int8_t *Xq, const float *d, int M, const uint8_t *Wp, const float *gamma,
                int N, int K, float *Y, int32_t *acc, hipStream_t s) {
    const int ntb = (M + 15) / 16, nrg = (N + 16 * RB - 1) / (16 * RB);
    const dim3 grid(8 * ntb * ((nrg + 7) / 8));
    hipLaunchKernelGGL((gemm_few_kernel<RB, NR>), grid, dim3(kFwThreads), 0, s, Xq, d, M, Wp,
                       gamma, N, K, Y, acc, ntb, nrg);
}

template <int NR>
void launch_few_rb(int rb, const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                   const float *gamma, int N, int K, float *Y, int32_t *acc, hipStream_t s) {
    if (rb == 1) launch_few<1, NR>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    else if (rb == 2) launch_few<2, NR>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    else if constexpr (NR <= 2) {
        if (rb == 4) launch_few<4, NR>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
        else launch_few<8, NR>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    } else {
        launch_few<4, NR>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    }
}

}  // namespace

bool gemm_skinny_fits(int M, int K) {
    return M >= 1 && M < 128 && K >= 64 && K <= kFwMaxRounds * 16 * kFwRoundGroups;
}

hipError_t launch_gemm_skinny(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                              const float *gamma, int N, int K, float *Y, int32_t *acc,
                              hipStream_t s) {
    if (M == 0 || N == 0)
        return hipSuccess;
    // Rows per workgroup 16 RB: the fewest that keep the grid within one
    // workgroup per CU (at most 256), capped so that a lane's weight units
    // (RB per round) fit in 64 registers.  Measured at K2560 -> N6912, M = 8:
    // 5.2 us; half the rows and two workgroups per CU, 6.0; twice the rows
    // (at most 128 workgroups), 6.0.
    const int nr = (K + 16 * kFwRoundGroups - 1) / (16 * kFwRoundGroups);   // rounds of 2048 k, <= 4
    const int ntb = (M + 15) / 16;
    const int rb_max = nr <= 2 ? 8 : 4;
    int rb = 1;
    while (rb < rb_max && ntb * ((N + 16 * rb - 1) / (16 * rb)) > 256) rb *= 2;
    switch (nr) {
    case 1: launch_few_rb<1>(rb, Xq, d, M, Wp, gamma, N, K, Y, acc, s); break;
    case 2: launch_few_rb<2>(rb, Xq, d, M, Wp, gamma, N, K, Y, acc, s); break;
    case 3: launch_few_rb<3>(rb, Xq, d, M, Wp, gamma, N, K, Y, acc, s); break;
    default: launch_few_rb<4>(rb, Xq, d, M, Wp, gamma, N, K, Y, acc, s); break;
    }
    return hipGetLastError();
}

}  // namespace bl
