// t5.hip -- ternary weights at five per byte (base 3): repacking from the
// 2-bit format, and a decode-sized product that reads the denser rows.
//
// The pages put a ternary weight at about 1.58 bits (log2 3: iaiol.com
// article, "权重映射为三元值"; the 0.4 GB model of the aigc.izzi.cn news
// page), while the format they store is 2 bits per weight ("Microsoft BitNet
// 深度研究报告", §2 (2) 实际存储, and the int2 I2_S kernel of its 内核类型
// table).  Five base-3 digits fit one byte (3^5 = 243 <= 256): 1.6 bits per
// weight, 20% fewer bytes than 2 bits.  Format (the pages give none):
//   digit d = w + 1; byte b of a row holds weights 5b .. 5b + 4 as
//   v = sum_j d_j 3^(4 - j) (weight 5b the most significant digit), stored as
//   q = ceil(256 v / 243); weights past K are 0 (digit 1), and rows are
//   padded with such bytes to a multiple of 16.
// Decoding without a division: q / 256 is a fraction just above v / 243, so
// multiplying it by 3 five times and keeping the integer part each time
// yields the digits, most significant first: with r_0 = q, t = 3 r_j,
// d_j = t >> 8, r_(j+1) = t & 255.  For the four bytes of a dword the even
// and the odd bytes sit in two 16-bit fields each (3 * 255 < 2^16, so a
// 32-bit multiply by 3 does not carry from one field into the next); after
// each multiply the four digits are bytes 1 and 3 of the two dwords, and one
// v_perm_b32 gathers them.  The digits are w + 1, so sum_k x d = sum_k x w +
// sum_k x: the product subtracts each token's sum of codes once.
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

// 2-bit code -> base-3 digit w + 1 (code 3, never written, reads as 0)
__device__ __forceinline__ int digit_of_code(unsigned c) {
    return 1 + (int)(c & 1u) - (int)(c >> 1);
}

// One thread per 16 output bytes (80 weights) of a row.
__global__ __launch_bounds__(256) void repack_t5_kernel(const uint8_t *__restrict__ Wp, int N, int K,
                                                       uint8_t *__restrict__ Wt5, int RB) {
    const int chunks = RB / 16;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)N * chunks) return;
    const int n = (int)(i / chunks), c = (int)(i - (int64_t)n * chunks);
    const uint8_t *row = Wp + (size_t)n * (K / 4);
    uint32_t out[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t dw = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            int v = 0;
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                const int k = 80 * c + 20 * w + 5 * b + j;
                const int digit = k < K ? digit_of_code((row[k >> 2] >> (2 * (k & 3))) & 3u) : 1;
                v = 3 * v + digit;
            }
            dw |= (uint32_t)((256 * v + 242) / 243) << (8 * b);
        }
        out[w] = dw;
    }
    *reinterpret_cast<uint4 *>(Wt5 + (size_t)n * RB + 16 * c) =
        make_uint4(out[0], out[1], out[2], out[3]);
}

constexpr int kT5Threads = 256;
constexpr int kT5InFlight = 4;              // 16-byte weight loads issued before use

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The digits of the four bytes of dw: byte c of D[j] = digit j of byte c.
__device__ __forceinline__ void digits20(uint32_t dw, uint32_t (&D)[5]) {
    uint32_t e = dw & 0x00FF00FFu, o = (dw >> 8) & 0x00FF00FFu;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        e *= 3u;
        o *= 3u;
        D[j] = perm(o, e, 0x07030501u);      // bytes: e.1, o.1, e.3, o.3
        e &= 0x00FF00FFu;
        o &= 0x00FF00FFu;
    }
}

// One 16-byte unit (80 weights) against the staged codes of MT tokens.  The
// codes of a unit are 20 dwords: dword 5t + j holds the activations of the
// weights that digit j of packed dword t encodes, k = 80u + 20t + 5c + j in
// byte c.
template <int MT>
__device__ __forceinline__ void t5_unit(const uint4 &w, const uint4 *xs, int U, int u,
                                        int (&acc)[MT]) {
    const uint32_t dws[4] = {w.x, w.y, w.z, w.w};
    uint32_t D[4][5];
#pragma unroll
    for (int t = 0; t < 4; ++t) digits20(dws[t], D[t]);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const uint4 *x4 = xs + ((size_t)m * U + u) * 5;
        uint32_t x[20];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const uint4 v = x4[i];
            x[4 * i] = v.x;
            x[4 * i + 1] = v.y;
            x[4 * i + 2] = v.z;
            x[4 * i + 3] = v.w;
        }
        int a = acc[m];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < 5; ++j) a = dot4(D[t][j], x[5 * t + j], a);
        acc[m] = a;
    }
}

// Layout as the 2-bit VALU product: 4 waves, each owning R = 64 / L rows
// with a row split over L lanes; lane s reads units s, s + L, ...  The codes
// of MT tokens are staged once per workgroup in the digit order above,
// together with each token's sum of codes.
template <int L, int MT>
__global__ __launch_bounds__(kT5Threads) void gemv_t5_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ d, int M,
    const uint8_t *__restrict__ Wt5, const float *__restrict__ gamma, int N, int K, int RB,
    float *__restrict__ Y, int32_t *__restrict__ acc_out) {
    // every argument from the kernarg segment in one batch of scalar loads
    // (one wait), not each batch where it is first used
    asm volatile("" ::"s"(Xq), "s"(d), "s"(M), "s"(Wt5), "s"(gamma), "s"(N), "s"(K), "s"(RB), "s"(Y), "s"(acc_out));
    constexpr int R = 64 / L;
    extern __shared__ uint4 xs[];                 // [MT][U][5]
    __shared__ int sx[MT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int r = lane / L, s = lane % L;
    const int row = (blockIdx.x * (kT5Threads / 64) + (tid >> 6)) * R + r;
    const int m0 = blockIdx.y * MT;
    const int mt = min(MT, M - m0);
    const int U = RB / 16;
    // Rows past N read the last row (in bounds) and are never stored.
    const uint4 *wrow = reinterpret_cast<const uint4 *>(Wt5 + (size_t)min(row, N - 1) * RB);
    // the epilogue's scales, loaded now on the vector path: scalar loads
    // would put their round trip (pointer, then value) in front of the
    // weight loads, since every wait for a scalar load waits for all of them
    const float gam = __hip_atomic_load(gamma, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float dv[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        dv[m] = m < mt ? __hip_atomic_load(d + m0 + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;

    uint4 w[kT5InFlight];
#pragma unroll
    for (int j = 0; j < kT5InFlight; ++j) w[j] = ld_stream(wrow + min(s + j * L, U - 1));

    if (tid < MT) sx[tid] = 0;
    __syncthreads();
    // staging: item (m, P) = the 20 codes k = 20P .. 20P + 19 of token m
    uint32_t *xd = reinterpret_cast<uint32_t *>(xs);
    const int P4 = 4 * U;
    for (int i = tid; i < mt * P4; i += kT5Threads) {
        const int m = i / P4, P = i - m * P4;
        const int8_t *xr = Xq + (size_t)(m0 + m) * K;
        uint32_t in[5];
#pragma unroll
        for (int t = 0; t < 5; ++t) {
            const int k = 20 * P + 4 * t;               // K % 4 == 0: all or none of a dword
            in[t] = k < K ? *reinterpret_cast<const uint32_t *>(xr + k) : 0u;
        }
        int sum = 0;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            uint32_t v = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int e = 5 * c + j;                // code 20P + e
                const uint32_t byte = (in[e >> 2] >> (8 * (e & 3))) & 0xFFu;
                v |= byte << (8 * c);
                sum += (int)(int8_t)byte;
            }
            xd[((size_t)m * U * 20) + 5 * P + j] = v;
        }
        atomicAdd(&sx[m], sum);
    }
    __syncthreads();

    int acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0;
    for (int u = s; u < U; u += L * kT5InFlight) {
        uint4 wn[kT5InFlight];
        const int un = u + L * kT5InFlight;
        if (un < U) {
#pragma unroll
            for (int j = 0; j < kT5InFlight; ++j) wn[j] = ld_stream(wrow + min(un + j * L, U - 1));
        }
#pragma unroll
        for (int j = 0; j < kT5InFlight; ++j)
            if (u + j * L < U) t5_unit<MT>(w[j], xs, U, u + j * L, acc);
        if (un < U) {
#pragma unroll
            for (int j = 0; j < kT5InFlight; ++j) w[j] = wn[j];
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = group_sum(acc[m], L);
    if (row < N && s == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < mt) {
                const int a = acc[m] - sx[m];
                const size_t o = (size_t)(m0 + m) * N + row;
                Y[o] = rescale(a, __fmul_rn(gam, dv[m]));
                if (acc_out) acc_out[o] = a;
            }
        }
    }
}

template <int L, int MT>
hipError_t launch_t5_lm(const int8_t *Xq, const float *d, int M, const uint8_t *Wt5,
                        const float *gamma, int N, int K, float *Y, int32_t *acc, hipStream_t s) {
    constexpr int rows_per_wg = (kT5Threads / 64) * (64 / L);
    const int RB = (int)t5_row_bytes(K);
    const dim3 grid((N + rows_per_wg - 1) / rows_per_wg, (M + MT - 1) / MT);
    hipLaunchKernelGGL((gemv_t5_kernel<L, MT>), grid, dim3(kT5Threads), t5_lds_bytes(M, K), s,
                       Xq, d, M, Wt5, gamma, N, K, RB, Y, acc);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_t5_m(const int8_t *Xq, const float *d, int M, const uint8_t *Wt5,
                       const float *gamma, int N, int K, float *Y, int32_t *acc, hipStream_t s) {
    const int U = (int)(t5_row_bytes(K) / 16);
#ifndef BL_T5_L64_UNITS
#define BL_T5_L64_UNITS 96
#endif
    int L = U >= BL_T5_L64_UNITS ? 64 : U >= 48 ? 32 : 16;   // the 2-bit product's rule
#ifdef BL_T5_FORCE_L
    L = BL_T5_FORCE_L;                             // tuning builds only
#endif
    switch (L) {
    case 8: return launch_t5_lm<8, MT>(Xq, d, M, Wt5, gamma, N, K, Y, acc, s);
    case 16: return launch_t5_lm<16, MT>(Xq, d, M, Wt5, gamma, N, K, Y, acc, s);
    case 32: return launch_t5_lm<32, MT>(Xq, d, M, Wt5, gamma, N, K, Y, acc, s);
    default: return launch_t5_lm<64, MT>(Xq, d, M, Wt5, gamma, N, K, Y, acc, s);
    }
}

}  // namespace

hipError_t launch_repack_t5(const uint8_t *Wp, int N, int K, uint8_t *Wt5, hipStream_t s) {
    const int RB = (int)t5_row_bytes(K);
    const int64_t total = (int64_t)N * (RB / 16);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(repack_t5_kernel, dim3((unsigned)blocks), dim3(256), 0, s, Wp, N, K, Wt5, RB);
    return hipGetLastError();
}

hipError_t launch_gemv_t5(const int8_t *Xq, const float *d, int M, const uint8_t *Wt5,
                          const float *gamma, int N, int K, float *Y, int32_t *acc, hipStream_t s) {
    if (M == 0 || N == 0)
        return hipSuccess;
    if (M == 1) return launch_t5_m<1>(Xq, d, M, Wt5, gamma, N, K, Y, acc, s);
    if (M == 2) return launch_t5_m<2>(Xq, d, M, Wt5, gamma, N, K, Y, acc, s);
    if (M <= 4) return launch_t5_m<4>(Xq, d, M, Wt5, gamma, N, K, Y, acc, s);
    return launch_t5_m<8>(Xq, d, M, Wt5, gamma, N, K, Y, acc, s);
}

}  // namespace bl
