// gemv.hip -- W1.58A8 product for a handful of tokens (decode): v_dot4 on the
// VALU, and for one token in the fused kernel the int8 MFMA.
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
#include <algorithm>
#include <climits>

#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kUnitsInFlight = 4;           // 16-byte loads issued before use

// Packed weights are read exactly once per call: non-temporal loads stream
// them through the caches without displacing what is reused (the staged
// activations, which every workgroup of a job reads).  On the four decode
// shapes with weights cold in HBM this took the fused step from 8.2 to 7.4 us.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
constexpr int kXBytes = 64 * 1024;          // LDS budget for staged activations
constexpr int kMaxJobs = kGemvMaxJobs;

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
        w[j] = ld_stream(wrow + min(u + j * L, ue - 1));   // clamped: always in bounds
}

// A4: the activations are 4-bit codes, two per byte ([M][K/2]); only the
// staging differs (eight bytes of codes per 16-element group, sign-extended
// into the same transposed int8 group).
template <int L, int MT, bool A4 = false>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ d, int M,
    const uint8_t *__restrict__ Wp, const float *__restrict__ gamma, int N, int K, int KC,
    float *__restrict__ Y, int32_t *__restrict__ acc_out) {
    // every argument from the kernarg segment in one batch of scalar loads
    // (one wait), not each batch where it is first used
    asm volatile("" ::"s"(Xq), "s"(d), "s"(M), "s"(Wp), "s"(gamma), "s"(N), "s"(K), "s"(KC), "s"(Y), "s"(acc_out));
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
    // the epilogue's scales, loaded now on the vector path: scalar loads
    // would put their round trip (pointer, then value) in front of the
    // weight loads, since every wait for a scalar load waits for all of them
    const float gam = __hip_atomic_load(gamma, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float dv[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        dv[m] = m < mt ? __hip_atomic_load(d + m0 + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;

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
            if constexpr (A4) {
                const uint2 v = *reinterpret_cast<const uint2 *>(
                    Xq + ((size_t)(m0 + m) * K + kc0 + 16 * g) / 2);
                xs[m * gpc + g] = a4_to_t16(v);
            } else {
                const uint4 v = *reinterpret_cast<const uint4 *>(Xq + (size_t)(m0 + m) * K + kc0 + 16 * g);
                xs[m * gpc + g] = transpose16(v);
            }
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
    for (int m = 0; m < MT; ++m) acc[m] = group_sum(acc[m], L);
    if (row < N && s == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < mt) {
                const size_t o = (size_t)(m0 + m) * N + row;
                Y[o] = rescale(acc[m], __fmul_rn(gam, dv[m]));
                if (acc_out) acc_out[o] = acc[m];
            }
        }
    }
}

template <int L, int MT, bool A4 = false>
hipError_t launch_lm(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                     const float *gamma, int N, int K, float *Y, int32_t *acc, hipStream_t s) {
    constexpr int rows_per_wg = (kThreads / 64) * (64 / L);
    int KC = (kXBytes / MT) / 64 * 64;
    if (KC > K) KC = K;
    const dim3 grid((N + rows_per_wg - 1) / rows_per_wg, (M + MT - 1) / MT);
    const size_t lds = (size_t)MT * KC;
    hipLaunchKernelGGL((gemv_kernel<L, MT, A4>), grid, dim3(kThreads), lds, s,
                       Xq, d, M, Wp, gamma, N, K, KC, Y, acc);
    return hipGetLastError();
}

template <int MT, bool A4 = false>
hipError_t launch_m(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                    const float *gamma, int N, int K, float *Y, int32_t *acc, hipStream_t s) {
    const int U = K / 64;                               // 16-byte units per row
    int L = U >= 96 ? 64 : U >= 48 ? 32 : 16;
#ifdef BL_GEMV_FORCE_L
    L = BL_GEMV_FORCE_L;                                // tuning builds only
#endif
    switch (L) {
    case 8: return launch_lm<8, MT, A4>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    case 16: return launch_lm<16, MT, A4>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    case 32: return launch_lm<32, MT, A4>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    default: return launch_lm<64, MT, A4>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    }
}

// ---------------------------------------------------------------------------
// Fused decode kernel: per-token absmax int8 quantisation folded into the
// GEMV, for several independent BitLinears in one launch.  Workgroups are
// dealt to the jobs in order of decreasing K, so the longest run first (job
// j of that order owns workgroups [wg_begin_j, wg_begin_j+1)).
// A workgroup's waves have two roles:
//   quantising waves (4) read the job's activation rows (L2-resident after
//     the first workgroup) into LDS, form max |x| per token (counting up an
//     LDS word), then write the int8 codes into LDS in transposed 16-byte
//     groups (the job's first workgroup also stores Xq and d to memory) and
//     count up a second word;
//   compute waves (8) issue all their packed-weight loads at once, unpack
//     the first units as they land while the codes are being formed, and once
//     the second count reaches four run the unit loop and lane reduction of
//     gemv_kernel, with the lane split L chosen per job.
// The roles are split because a wave cannot issue past a load instruction
// the memory pipeline has not accepted: with the weight requests of the whole
// launch in flight, a wave that issued weight loads reaches the next
// instruction only as the earliest of them return.  A workgroup barrier
// between the activation and the weight phases therefore delayed the codes
// to about when the weights had landed (codes 3.1 us after the workgroup
// start, 2.9 us of which waiting); with the quantising waves issuing no
// weight loads and no barrier, the four decode shapes' step went from 7.2 to
// 6.35 us.  For the same reason the compute waves form no codes: some of them
// are still held at their weight-load issue when max |x| is known, and codes
// that waited for all twelve waves came about 1 us after the quantising
// waves' own.
// The arguments sit in the kernarg segment, which the waves read with scalar
// loads whose every wait is a round trip to L2.  The token count and each
// job's first workgroup come first, as separate scalar parameters, and the
// library is built to preload the leading kernel arguments into SGPRs at wave
// launch (gfx950 kernarg preload; on firmware without it, a prologue loads
// them): the workgroup picks its job with no memory access and reads the job
// record (64 bytes, on one 64-byte line) in one load, one round trip before
// the first weight and activation loads (5.41-5.43 against 5.51-5.54 us per
// step on the four decode shapes with the header loaded from the segment;
// preloading the first job's pointers as well ran 5.45-5.47).  Gamma is read
// on the vector path instead, behind the weights.
struct FusedJob {
    const void *X;
    const uint8_t *Wp;
    const float *gamma;
    float *Y;
    int8_t *Xq;
    float *d;
    int N, K, dtype, lshift;          // lanes per row L = 1 << lshift
};

struct alignas(64) FusedArgs {                 // the job records; the header is passed before it
    FusedJob job[kMaxJobs];
};
static_assert(sizeof(FusedJob) == 64, "one 64-byte scalar load per job record");


// 512 compute threads: every workgroup quantises its job's whole activation
// row, so fewer, larger workgroups repeat that less; on the four 2B-class
// decode shapes (M = 1) 512 measured 9.3 us per step against 9.7 us for 256
// and 11.4 us for 1024 (before the role split).
constexpr int kQWaves = 4;                     // waves that quantise the activations
constexpr int kQThreads = 64 * kQWaves;
constexpr int kCThreads = 512;                 // waves that load weights and form the products
constexpr int kFThreads = kQThreads + kCThreads;
// Every 16-byte weight unit of a lane is requested at once: with the lane
// splits below a lane owns at most 108 / 16 < 8 units of a row.
constexpr int kFUnits = 8;
constexpr int kXPre = 2;            // activation groups per thread loaded ahead of the weights
// Weight units a compute wave unpacks while the codes are being formed (as
// far as they have landed): two measured 5.81-5.83 us per step on the four
// decode shapes, three 5.84-5.86, four 5.88, none 5.95-5.97; the unpacked
// units stay in registers (16 each) until the codes are there.
constexpr int kPreUnits = 2;

// Token counts that take the MFMA dot products (the rest use v_dot4).
#ifndef BL_FUSED_MFMA_MAX_MT
#define BL_FUSED_MFMA_MAX_MT 1
#endif
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i as_v4i(uint4 v) { return v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}; }

// 16 consecutive activations as fp32 from their raw 16-byte words: four
// words of fp32, or two words of bf16 (widening is exact).
__device__ __forceinline__ void unpack_x16(const uint4 (&raw)[4], int dtype, float (&x)[16]) {
    if (dtype == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x[4 * t] = __uint_as_float(raw[t].x);
            x[4 * t + 1] = __uint_as_float(raw[t].y);
            x[4 * t + 2] = __uint_as_float(raw[t].z);
            x[4 * t + 3] = __uint_as_float(raw[t].w);
        }
    } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t w4[4] = {raw[t].x, raw[t].y, raw[t].z, raw[t].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[8 * t + 2 * i] = bf16_lo(w4[i]);
                x[8 * t + 2 * i + 1] = bf16_hi(w4[i]);
            }
        }
    }
}

// kMfma (one token): the dot products run on v_mfma_i32_16x16x64_i8 instead
// of v_dot4, with the lanes reading the same units as the v_dot4 loop (L
// lanes per row, lane s of a row on units s, s + L, ...).  Column i of the
// 16-column B operand is lane i % 16 of a lane group g = lane / 16; with
// c = L / 4 columns per row, column i belongs to row i / c of the wave and
// its lane group g holds unit (i % c) + c g of the current slot, so the 4
// lane groups of the c columns of a row cover the slot's L units.  Row j of
// the A operand carries, on lane group g, the activations of unit
// (j % c) + c g: the k layout of A and B then matches wherever j = i (mod c),
// and D[i % c][i] (accumulator i % c of lane i) is column i's partial sum
// over its 4 units.  One MFMA does the work of 64 lanes x 4 v_dot4 on the
// matrix core, beside the other wave's unpacking; the c partials of a row
// are added with shuffles.
template <int MT, bool kMfma>
__global__ __launch_bounds__(kFThreads) void gemv_fused_kernel(int Mtok, int b1, int b2, int b3, int b4, int b5, int b6, int b7,
                                                                const FusedArgs args) {
    // job t starts at workgroup b_t (job 0 at 0; unused jobs at INT_MAX)
    const int wgb[kMaxJobs] = {0, b1, b2, b3, b4, b5, b6, b7};
    extern __shared__ uint4 xs[];   // [MT][K / 16] transposed code groups, then the raw activations
    __shared__ float red[kQWaves][MT];
    __shared__ unsigned n_amax, n_codes;        // quantising waves past each step
    int j = 0, jbegin = 0;
#pragma unroll
    for (int t = 1; t < kMaxJobs; ++t)
        if ((int)blockIdx.x >= wgb[t]) {
            j = t;
            jbegin = wgb[t];
        }
    const FusedJob jb = args.job[j];                // the record, copied by one load
    const int K = jb.K, N = jb.N, dtype = jb.dtype, lshift = jb.lshift;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wg = (int)blockIdx.x - jbegin;
    const int m0 = blockIdx.y * MT;
    const int mt = min(MT, Mtok - m0);
    const int U = K / 64;
    const int gpc = K / 16;
    if (tid == 0) {
        n_amax = 0u;
        n_codes = 0u;
    }
    __syncthreads();                            // nothing is in flight yet

    const int gsz = dtype == 0 ? 4 : 2;                           // uint4 per 16 elements
    uint4 *xraw = xs + MT * gpc;                                   // [MT][K / 16][gsz]
    const bool writer = (wg == 0);
    // The int8 codes of groups g = first, first + kQThreads, ... from the raw
    // rows in LDS, once every quantising wave's maximum is in red[][].
    auto form_codes = [&](int first) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float a = red[0][m];
#pragma unroll
            for (int v = 1; v < kQWaves; ++v) a = fmaxf(a, red[v][m]);
            if (m < mt) {
                const float sc = act_inv_scale(a);
                for (int g = first; g < gpc; g += kQThreads) {
                    uint4 raw[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (t < gsz) raw[t] = xraw[((size_t)m * gpc + g) * gsz + t];
                    float x[16];
                    unpack_x16(raw, dtype, x);
                    uint32_t q4[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        q4[t] = (uint32_t)(act_code(x[4 * t], sc) & 0xFF) |
                                ((uint32_t)(act_code(x[4 * t + 1], sc) & 0xFF) << 8) |
                                ((uint32_t)(act_code(x[4 * t + 2], sc) & 0xFF) << 16) |
                                ((uint32_t)(act_code(x[4 * t + 3], sc) & 0xFF) << 24);
                    const uint4 qv = make_uint4(q4[0], q4[1], q4[2], q4[3]);
                    if (writer && jb.Xq)
                        *reinterpret_cast<uint4 *>(jb.Xq + (size_t)(m0 + m) * K + 16 * g) = qv;
                    xs[m * gpc + g] = transpose16(qv);
                }
                if (writer && jb.d && first == 0)
                    jb.d[m0 + m] = act_scale(a);
            }
        }
    };

    // The quantising waves' code is laid out first, right after the common
    // prologue: the instruction cache is cold at each launch, and a far jump
    // costs a fetch from L2.  The compute waves take that jump instead, which
    // also puts the activation requests ahead of the weight stream on the
    // CU (5.55-5.62 against 5.82 us per step with the compute path first;
    // issuing the weight loads before the role split: 6.56 us).
    if (__builtin_expect(tid < kQThreads, 1)) {
        // ---- quantising waves: the job's activation rows -> max |x| in LDS
        const char *xbase = reinterpret_cast<const char *>(jb.X);
        const int ng = mt * gpc;                                   // (token, group) pairs
        uint4 xr[kXPre][4];
#pragma unroll
        for (int p = 0; p < kXPre; ++p) {
            const int e = min(tid + p * kQThreads, ng - 1);
            const int m = MT == 1 ? 0 : e / gpc, g = e - m * gpc;   // one token: no division
            const uint4 *src = reinterpret_cast<const uint4 *>(xbase + (size_t)(m0 + m) * K * gsz) +
                               (size_t)g * gsz;
            if (dtype == 0) {
#pragma unroll
                for (int t = 0; t < 4; ++t) xr[p][t] = src[t];
            } else {
                xr[p][0] = src[0];
                xr[p][1] = src[1];
            }
        }
        float amax[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) amax[m] = 0.0f;
        auto stage = [&](const uint4 (&raw)[4], int e) {
            const int m = MT == 1 ? 0 : e / gpc, g = e - m * gpc;   // one token: no division
            float x[16];
            unpack_x16(raw, dtype, x);
            uint4 *dst = xraw + ((size_t)m * gpc + g) * gsz;
            dst[0] = raw[0];
            dst[1] = raw[1];
            if (dtype == 0) { dst[2] = raw[2]; dst[3] = raw[3]; }
            float a = 0.0f;
#pragma unroll
            for (int i2 = 0; i2 < 16; ++i2) a = fmaxf(a, fabsf(x[i2]));
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
                if (mm == m) amax[mm] = fmaxf(amax[mm], a);
        };
#pragma unroll
        for (int p = 0; p < kXPre; ++p) {
            const int e = tid + p * kQThreads;
            if (e < ng) stage(xr[p], e);
        }
        for (int e = tid + kXPre * kQThreads; e < ng; e += kQThreads) {
            const int m = MT == 1 ? 0 : e / gpc, g = e - m * gpc;   // one token: no division
            const uint4 *src = reinterpret_cast<const uint4 *>(xbase + (size_t)(m0 + m) * K * gsz) +
                               (size_t)g * gsz;
            uint4 raw[4];
            raw[0] = src[0];
            raw[1] = src[1];
            if (dtype == 0) { raw[2] = src[2]; raw[3] = src[3]; }
            stage(raw, e);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            amax[m] = group_max(amax[m], 64);
        }
        if (lane == 0) {
#pragma unroll
            for (int m = 0; m < MT; ++m) red[tid >> 6][m] = amax[m];
        }
        // every quantising wave's maximum (and raw words) in LDS before the count
        if (lane == 0)
            __hip_atomic_fetch_add(&n_amax, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        while (__hip_atomic_load(&n_amax, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kQWaves)
            __builtin_amdgcn_s_sleep(1);
        form_codes(tid);
        // the codes in LDS before the count the compute waves wait for
        if (lane == 0)
            __hip_atomic_fetch_add(&n_codes, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        return;
    }

    // ---- compute waves: issue the packed-weight loads, then wait for the codes
    const int ct = tid - kQThreads;
    const int L = 1 << lshift;
    const int r = lane >> lshift;
    const int s = lane & (L - 1);
    const int rows_wg = (kCThreads / 64) * (64 >> lshift);
    int row, sig;
    if constexpr (kMfma) {
        // c = L / 4 columns per row (a power of two), column i
        const int cs = lshift - 2, c = 1 << cs, i = lane & 15;
        row = wg * rows_wg + (ct >> 6) * (64 >> lshift) + (i >> cs);
        sig = (i & (c - 1)) + c * (lane >> 4);
    } else {
        row = wg * rows_wg + (ct >> 6) * (64 >> lshift) + r;
        sig = s;
    }
    const uint4 *wrow = reinterpret_cast<const uint4 *>(jb.Wp + (size_t)max(min(row, N - 1), 0) * (K / 4));
    uint4 w[kFUnits];
#pragma unroll
    for (int q = 0; q < kFUnits; ++q)
        w[q] = ld_stream(wrow + min(sig + q * L, U - 1));  // a job with N == 0 reads its own X here
    // gamma on the vector path, behind the weights (the products need it
    // only after every weight has landed; a job with no rows has none)
    const float gam = N > 0 ? __builtin_nontemporal_load(jb.gamma) : 0.0f;
    auto codes_ready = [&]() {
        return __hip_atomic_load(&n_codes, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >=
               (unsigned)kQWaves;
    };

    if constexpr (kMfma) {
        // dot products on MFMA over the lane's units; slots past the row's
        // last unit take zero weights (the loop is wave-uniform)
        static_assert(MT == 1, "the MFMA mapping carries one token");
        const int nslot = (U + L - 1) >> lshift;
        // Until the codes are complete, unpack the first units as they land
        // (the test between units is wave-uniform: one LDS word).
        uint4 bpre[kPreUnits][4];
        int npre = kPreUnits;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
        for (int q = 0; q < kPreUnits; ++q) {
            if (__builtin_amdgcn_readfirstlane((int)codes_ready())) {
                npre = q;
                break;
            }
            const bool ok = q < nslot && sig + q * L < U;
            const uint32_t dws[4] = {ok ? w[q].x : 0u, ok ? w[q].y : 0u, ok ? w[q].z : 0u,
                                     ok ? w[q].w : 0u};
#pragma unroll
            for (int t = 0; t < 4; ++t) unpack16(dws[t], bpre[q][t].x, bpre[q][t].y, bpre[q][t].z, bpre[q][t].w);
        }
        while (!codes_ready())
            __builtin_amdgcn_s_sleep(1);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        v4i acc4 = v4i{0, 0, 0, 0};
        for (int i0 = 0; i0 < nslot; i0 += kFUnits) {
            uint4 wn[kFUnits];
            const bool more = i0 + kFUnits < nslot;
            if (more) {
#pragma unroll
                for (int q = 0; q < kFUnits; ++q)
                    wn[q] = ld_stream(wrow + min(sig + (i0 + kFUnits + q) * L, U - 1));
            }
#pragma unroll
            for (int q = 0; q < kFUnits; ++q) {
                if (i0 + q < nslot) {
                    const int u = sig + (i0 + q) * L;
                    const bool ok = u < U;
                    const int uc = min(u, U - 1);
                    uint4 bv[4];
                    if (q < kPreUnits && i0 == 0 && q < npre) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) bv[t] = bpre[q < kPreUnits ? q : 0][t];
                    } else {
                        // selects rather than a branch on the last slot: branches
                        // keep the compiler from interleaving consecutive units
                        const uint32_t dws[4] = {ok ? w[q].x : 0u, ok ? w[q].y : 0u, ok ? w[q].z : 0u,
                                                 ok ? w[q].w : 0u};
#pragma unroll
                        for (int t = 0; t < 4; ++t) unpack16(dws[t], bv[t].x, bv[t].y, bv[t].z, bv[t].w);
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        acc4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(xs[4 * uc + t]), as_v4i(bv[t]),
                                                                     acc4, 0, 0, 0);
                }
            }
            if (more) {
#pragma unroll
                for (int q = 0; q < kFUnits; ++q) w[q] = wn[q];
            }
        }
        // lane i < 16: D[i % c][i], then the sum over the row's c columns
        const int c = L >> 2;
        const int jc = lane & (c - 1);
        const int v01 = (jc & 1) ? acc4[1] : acc4[0];
        const int v23 = (jc & 1) ? acc4[3] : acc4[2];
        int v = (jc & 2) ? v23 : v01;
        v = group_sum(v, c);
        if (lane < 16 && jc == 0 && row < N) {
            float a = red[0][0];
#pragma unroll
            for (int vv = 1; vv < kQWaves; ++vv) a = fmaxf(a, red[vv][0]);
            jb.Y[(size_t)m0 * N + row] = rescale(v, __fmul_rn(gam, act_scale(a)));
        }
        return;
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    while (!codes_ready())
        __builtin_amdgcn_s_sleep(1);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);

    // dot products over this lane's units, software-pipelined
    int acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0;
    if (row < N) {
        for (int u = s; u < U; u += L * kFUnits) {
            uint4 wn[kFUnits];
            const int un = u + L * kFUnits;
            if (un < U) {
#pragma unroll
                for (int q = 0; q < kFUnits; ++q) wn[q] = ld_stream(wrow + min(un + q * L, U - 1));
            }
#pragma unroll
            for (int q = 0; q < kFUnits; ++q)
                if (u + q * L < U)
                    dot_unit<16, MT>(w[q], xs, gpc, u + q * L, acc);
            if (un < U) {
#pragma unroll
                for (int q = 0; q < kFUnits; ++q) w[q] = wn[q];
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = group_sum(acc[m], L);
    if (row < N && s == 0) {
        const float g = gam;
        float dm[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float a = red[0][m];
#pragma unroll
            for (int v = 1; v < kQWaves; ++v) a = fmaxf(a, red[v][m]);
            dm[m] = act_scale(a);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < mt)
                jb.Y[(size_t)(m0 + m) * N + row] = rescale(acc[m], __fmul_rn(g, dm[m]));
    }
}

}  // namespace

// 4-bit activation codes, 1 <= M <= 8, on the v_dot4 kernel.
hipError_t launch_gemv_a4(const uint8_t *Xq4, const float *d, int M, const uint8_t *Wp,
                          const float *gamma, int N, int K, float *Y, int32_t *acc,
                          hipStream_t s) {
    if (M == 0 || N == 0)
        return hipSuccess;
    const int8_t *X = reinterpret_cast<const int8_t *>(Xq4);
    if (M == 1) return launch_m<1, true>(X, d, M, Wp, gamma, N, K, Y, acc, s);
    if (M == 2) return launch_m<2, true>(X, d, M, Wp, gamma, N, K, Y, acc, s);
    if (M <= 4) return launch_m<4, true>(X, d, M, Wp, gamma, N, K, Y, acc, s);
    return launch_m<8, true>(X, d, M, Wp, gamma, N, K, Y, acc, s);
}

hipError_t launch_gemv(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                       const float *gamma, int N, int K, float *Y, int32_t *acc,
                       hipStream_t s) {
    if (M == 0 || N == 0)
        return hipSuccess;
    // From 3 tokens on, the MFMA kernel that reads the weights once is faster
    // (K6912 -> N2560: 7.4 against 8.1 us at M = 4, 8.5 against 17.8 us at
    // M = 8); at M = 2 the v_dot4 path wins (5.9 against 6.9 us).
    if (M >= 3 && gemm_skinny_fits(M, K))
        return launch_gemm_skinny(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    if (M == 1) return launch_m<1>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    if (M == 2) return launch_m<2>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    if (M <= 4) return launch_m<4>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    return launch_m<8>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
}

}  // namespace bl

namespace bl {
namespace {
template <int MT>
hipError_t launch_fused_mt(const FusedArgs &a, const int *wgb, int M, int grid_x, int max_k, int max_es,
                           hipStream_t s) {
    const dim3 grid(grid_x, (M + MT - 1) / MT);
    hipLaunchKernelGGL((gemv_fused_kernel<MT, (MT <= BL_FUSED_MFMA_MAX_MT)>), grid, dim3(kFThreads),
                       fused_lds_bytes(MT, max_k, max_es), s, M, wgb[1], wgb[2], wgb[3], wgb[4], wgb[5],
                       wgb[6], wgb[7], a);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemv_fused(const GemvJob *jobs, int count, int M, hipStream_t s) {
    FusedArgs a = {};
    int wg_begin[kMaxJobs];
    for (int j = 0; j < kMaxJobs; ++j) wg_begin[j] = INT_MAX;
    int wg = 0, max_k = 0, max_es = 2;
    // Jobs in order of decreasing K (stable): the longest workgroups are
    // dispatched first.  Each job keeps its own outputs, so the order changes
    // no result.
    int order[kMaxJobs];
    for (int j = 0; j < count; ++j) order[j] = j;
    std::stable_sort(order, order + count, [&](int x, int y) { return jobs[x].K > jobs[y].K; });
    for (int j = 0; j < count; ++j) {
        FusedJob &f = a.job[j];
        const GemvJob &src = jobs[order[j]];
        f.X = src.X; f.Wp = src.Wp; f.gamma = src.gamma; f.Y = src.Y;
        f.Xq = src.Xq; f.d = src.d;
        f.N = src.N; f.K = src.K; f.dtype = src.dtype;
        // Lanes per row: 8 below K = 6144 (64 rows, 40 KB of K = 2560 weights
        // per workgroup), 16 above (32 rows, 54 KB at K = 6912).  Few, large
        // workgroups repeat the activation quantisation fewer times; on the
        // four decode shapes this measured 8.2 us per step against 9.3 us
        // for 16 / 32 / 64 lanes.
        const int U = f.K / 64;
        f.lshift = U >= 96 ? 4 : 3;
#ifdef BL_FUSED_LSHIFT
        f.lshift = BL_FUSED_LSHIFT;                     // tuning builds only
#endif
        const int rows_per_wg = (kCThreads / 64) * (64 >> f.lshift);
        wg_begin[j] = wg;
        // a job with N == 0 still gets one workgroup when it must write Xq / d
        const int n_wg = f.N > 0 ? (f.N + rows_per_wg - 1) / rows_per_wg : ((f.Xq || f.d) ? 1 : 0);
        // A job with no output rows only quantises; its weight-row pointer
        // aims at its own activations (K / 4 <= 2 K valid bytes) so the
        // kernel's unconditional first loads stay in bounds.
        if (f.N == 0)
            f.Wp = static_cast<const uint8_t *>(f.X);
        wg += n_wg;
        max_k = f.K > max_k ? f.K : max_k;
        max_es = (f.dtype == 0 ? 4 : 2) > max_es ? (f.dtype == 0 ? 4 : 2) : max_es;
    }
    if (wg == 0)
        return hipSuccess;
    if (M == 1) return launch_fused_mt<1>(a, wg_begin, M, wg, max_k, max_es, s);
    if (M == 2) return launch_fused_mt<2>(a, wg_begin, M, wg, max_k, max_es, s);
    if (M <= 4) return launch_fused_mt<4>(a, wg_begin, M, wg, max_k, max_es, s);
    return launch_fused_mt<8>(a, wg_begin, M, wg, max_k, max_es, s);
}

}  // namespace bl
