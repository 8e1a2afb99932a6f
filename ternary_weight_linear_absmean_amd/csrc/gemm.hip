// gemm.hip -- W1.58A8 product for many tokens (prefill) on int8 MFMA.
//
// The technical-report copy (推理完满 / GPU端) describes the W1.58A8 kernel as
// pack, store, load, unpack, compute over four ternary weights per int8.  At
// M = 2048 the product is compute-bound, so on gfx950 the unpacked ternary
// tile goes through int8 MFMA with int32 accumulation: the values
// {-1, 0, +1} are exact int8 operands and every int32 sum is exact.  The
// rescale Y = float(acc) * fl(gamma * d[m]) is applied in the epilogue.
// Both operands use the same transposed order inside every 16-byte group
// (see device_common.h), so each MFMA lane multiplies matching k.
//
// Two kernels:
//   gemm_kernel     M < 128: 128 x 128 tiles of v_mfma_i32_16x16x64_i8,
//                   4 waves, single-buffered LDS (A transposed, B unpacked).
//   gemm256_kernel  M >= 128: see below.
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

// A4: the activations are 4-bit codes, two per byte ([M][K/2]); only the
// staging differs (eight bytes per 16-element group, sign-extended into the
// same transposed int8 group).
template <bool A4>
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
            if constexpr (A4) {
                uint2 v = make_uint2(0u, 0u);
                if (gm < M)
                    v = *reinterpret_cast<const uint2 *>(Xq + ((size_t)gm * K + k0 + 16 * g) / 2);
                As[r * kPitch + g] = a4_to_t16(v);
            } else {
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (gm < M)
                    v = *reinterpret_cast<const uint4 *>(Xq + (size_t)gm * K + k0 + 16 * g);
                As[r * kPitch + g] = transpose16(v);
            }
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


// ---------------------------------------------------------------------------
// Large-M kernel on v_mfma_i32_32x32x32_i8 (on gfx950 the 32x32x32 int8 form
// sustains about twice the throughput of 16x16x64 in a plain MFMA loop).
// Workgroup = WM x WN waves, each wave owns MI x NJ blocks of 32 x 32 of Y
// (16 MI NJ int32 accumulators per lane); tile = 32 MI WM x 32 NJ WN.
//   <1, 4, 4, 2>: 128 x 256 tiles, 256 threads, two workgroups per CU (wide
//                 N, e.g. K2560 -> N6912): each SIMD runs one wave of each
//                 workgroup, and the two workgroups meet at their own
//                 barriers, so a SIMD's two waves are not held in step;
//                 44.0-44.8 us at M = 2048 against 45.5-46.1 us for
//                 256 x 256 tiles of 8 waves (<2, 4, 4, 2>) with the same loop
//   <2, 4, 2, 2>: 128 x 256 tiles, 512 threads (narrow N, e.g. K6912 -> N2560,
//                 where 256 x 256 tiles would leave most CUs idle): measured
//                 59 us on M2048 K6912 N2560 against 73 us for 128 x 128
//                 tiles of 128 threads, with the same epilogue
//   <2, 4, 4, 2> in gate/up mode (GU): the FFN's gate and up products in one
//                 kernel, 256 x 128 outputs per tile (see GateUp below)
// k-step 128: the activation tile (transposed 16-byte groups, see
// device_common.h) and the packed weight tile (2-bit codes, 4x smaller than
// int8) are staged in LDS, double-buffered, from registers loaded two
// k-steps ahead; each wave unpacks its B operands (one v_perm per four
// weights) right after reading the packed dwords from LDS.  One barrier per
// k-step; __builtin_amdgcn_iglp_opt(1) asks the scheduler to interleave the
// LDS reads with the MFMAs.  A K tail of 64 (K % 128 == 64) is one extra
// half step.  Rows past M and columns past N read clamped (valid) addresses
// and their outputs are never stored.
//
// Workgroup i runs M-tile i % m_tiles and N-tile i / m_tiles: workgroups are
// dealt to the 8 XCDs round-robin, so with 8 M-tiles each XCD keeps one
// M-tile of activations resident in its L2 while it streams packed weights.
constexpr int BK2 = 128;
constexpr int kAPitch = BK2 / 16 + 1;          // uint4 per A row (8 + 1 pad)
constexpr int kBPitch = BK2 / 16 + 1;          // dwords per B column (8 + 1 pad)
typedef int v16i __attribute__((ext_vector_type(16)));

template <int AG, int BG> struct Stage2 { uint4 a[AG]; uint4 b[BG]; };
template <int AG, int BG> struct SrcPtr { const int8_t *a[AG]; const uint8_t *b[BG]; };

// Per k-step a workgroup of T threads stages BM rows x 128 bytes of A (BM * 8
// groups of 16 bytes, AG = BM * 8 / T per thread) and BN columns x 32 packed
// bytes of B (BN * 2 groups of 16 bytes, BG = BN * 2 / T per thread).
// With A4 the activation rows are 4-bit codes, K / 2 bytes each, and a
// 16-element group is 8 bytes.
template <int BM, int BN, int T, int AG, int BG, bool A4>
__device__ __forceinline__ SrcPtr<AG, BG> src_ptrs(const int8_t *__restrict__ Xq,
        const uint8_t *__restrict__ Wp, int M, int N, int K, int KB, int m_base, int n_base, int tid) {
    SrcPtr<AG, BG> p;
#pragma unroll
    for (int i = 0; i < AG; ++i) {
        const int idx = tid + T * i;
        const int r = min(m_base + (idx >> 3), M - 1);
        p.a[i] = A4 ? Xq + ((size_t)r * K + 16 * (idx & 7)) / 2 : Xq + (size_t)r * K + 16 * (idx & 7);
    }
#pragma unroll
    for (int i = 0; i < BG; ++i) {
        const int idx = tid + T * i;
        const int gn = min(n_base + (idx >> 1), N - 1);
        p.b[i] = Wp + (size_t)gn * KB + 16 * (idx & 1);
    }
    return p;
}
// Gate/up mode (the FFN block's first two BitLinears in one kernel).  The
// B tile's 256 columns interleave the two weights in 32-row blocks: LDS
// column b belongs to wave b / 64, block j = (b / 32) % 2 takes W_gate
// (j = 0) or W_up (j = 1), row f = f0 + 32 (b / 64) + b % 32.  A wave's two
// accumulator blocks then hold the gate and the up sums of the same 128 x 32
// outputs in the same registers, and the epilogue forms
// H = relu(G)^2 * U and Z = H * g without leaving the lane.
struct GateUp {
    const uint8_t *Wu;
    const float *gamma_u;
    const float *norm_w;     // [F] or null (ones)
    float *Z;                // [M][F] fp32
    float *pmax;             // [M][n_tiles]: max |Z| over the tile's columns
    double *psum;            // [M][n_tiles]: sum of H^2 over the tile's columns
    int n_tiles;
};

template <int BN, int T, int AG, int BG>
__device__ __forceinline__ void gate_up_b_ptrs(SrcPtr<AG, BG> &p, const uint8_t *__restrict__ Wg,
        const uint8_t *__restrict__ Wu, int F, int KB, int f0, int tid) {
    static_assert(BN == 256, "gate/up tiles are 256 B-columns wide");
#pragma unroll
    for (int i = 0; i < BG; ++i) {
        const int idx = tid + T * i;
        const int b = idx >> 1;
        const int f = min(f0 + 32 * (b >> 6) + (b & 31), F - 1);
        p.b[i] = ((b >> 5) & 1 ? Wu : Wg) + (size_t)f * KB + 16 * (idx & 1);
    }
}

template <int AG, int BG, bool A4>
__device__ __forceinline__ void load_stage2(Stage2<AG, BG> &st, const SrcPtr<AG, BG> &sp, int k0) {
#pragma unroll
    for (int i = 0; i < AG; ++i) {
        if constexpr (A4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(sp.a[i] + k0 / 2);
            st.a[i] = make_uint4(v.x, v.y, 0u, 0u);
        } else {
            st.a[i] = *reinterpret_cast<const uint4 *>(sp.a[i] + k0);
        }
    }
#pragma unroll
    for (int i = 0; i < BG; ++i) st.b[i] = *reinterpret_cast<const uint4 *>(sp.b[i] + k0 / 4);
}
template <int T, int AG, int BG, bool A4>
__device__ __forceinline__ void store_stage2(const Stage2<AG, BG> &st, uint4 *As, uint32_t *Bs, int tid) {
#pragma unroll
    for (int i = 0; i < AG; ++i) {
        const int idx = tid + T * i;
        As[(idx >> 3) * kAPitch + (idx & 7)] =
            A4 ? a4_to_t16(make_uint2(st.a[i].x, st.a[i].y)) : transpose16(st.a[i]);
    }
#pragma unroll
    for (int i = 0; i < BG; ++i) {
        const int idx = tid + T * i;
        uint32_t *b = Bs + (idx >> 1) * kBPitch + 4 * (idx & 1);
        b[0] = st.b[i].x; b[1] = st.b[i].y; b[2] = st.b[i].z; b[3] = st.b[i].w;
    }
}

// Gate/up epilogue.  Each lane turns its gate / up sums into
// G = fl(acc_g * fl(gamma_g d)), U = fl(acc_u * fl(gamma_u d)) and
// H = fl(fl(relu(G)^2) * U), exactly as two separate products and the tail
// would, and parks H in LDS.  Then every wave takes 32 rows, two per step:
// a lane owns 4 consecutive columns, forms Z = fl(H * g), stores 16 bytes of
// Z (a wave store covers two whole 512-byte row segments), and the 32 lanes
// of a row reduce max |Z| and the fp64 sum of H^2 over the tile's columns in
// a fixed order (4 terms per lane, then a butterfly), so a partial depends
// only on the data.
template <int WM, int MI2, int BM2, int BNO, int kHPitch>
__device__ __forceinline__ void gate_up_epilogue(const v16i (&acc)[MI2][2], float *hS,
        const float *cS, const float *cSu, const GateUp &gu, int M, int F, int m_base, int f0,
        int wm, int wn, int lane, int wave) {
    static_assert(BNO == 128 && BM2 == 32 * (WM * 4), "one 32-row band per wave in pass 2");
    __syncthreads();                           // every wave is done with the operand stages
#pragma unroll
    for (int i = 0; i < MI2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int lrow = wm * 32 * MI2 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const float G = rescale(acc[i][0][r], cS[lrow]);
            const float U = rescale(acc[i][1][r], cSu[lrow]);
            const float rg = G > 0.0f ? G : 0.0f;
            hS[lrow * kHPitch + wn * 32 + (lane & 31)] = __fmul_rn(__fmul_rn(rg, rg), U);
        }
    }
    __syncthreads();
    const int c4 = 4 * (lane & 31);            // this lane's 4 columns of the tile
    const bool col_ok = f0 + c4 < F;           // F % 64 == 0: 4 columns are all in or all out
    float4 gain = make_float4(1.f, 1.f, 1.f, 1.f);
    if (gu.norm_w && col_ok) gain = *reinterpret_cast<const float4 *>(gu.norm_w + f0 + c4);
    const int nt = (int)(f0 / BNO);
#pragma unroll 2
    for (int k = 0; k < 16; ++k) {
        const int lrow = 32 * wave + 2 * k + (lane >> 5);
        const int row = m_base + lrow;
        const float4 h = *reinterpret_cast<const float4 *>(hS + lrow * kHPitch + c4);
        float4 z;
        z.x = __fmul_rn(h.x, gain.x);
        z.y = __fmul_rn(h.y, gain.y);
        z.z = __fmul_rn(h.z, gain.z);
        z.w = __fmul_rn(h.w, gain.w);
        const bool ok = col_ok && row < M;
        float a = 0.0f;
        double ss = 0.0;
        if (ok) {
            *reinterpret_cast<float4 *>(gu.Z + (size_t)row * F + f0 + c4) = z;
            a = fmaxf(fmaxf(fabsf(z.x), fabsf(z.y)), fmaxf(fabsf(z.z), fabsf(z.w)));
            ss = (double)h.x * h.x;
            ss += (double)h.y * h.y;
            ss += (double)h.z * h.z;
            ss += (double)h.w * h.w;
        }
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) {
            a = fmaxf(a, __shfl_xor(a, off));
            ss += __shfl_xor(ss, off);
        }
        if ((lane & 31) == 0 && row < M) {
            gu.pmax[(size_t)row * gu.n_tiles + nt] = a;
            gu.psum[(size_t)row * gu.n_tiles + nt] = ss;
        }
    }
}

template <int WM, int WN, int MI2, int NJ2, bool GU, bool A4 = false>
__global__ __launch_bounds__(64 * WM * WN, WM * WN == 4 ? 2 : 1) void gemm256_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ d, int M,
    const uint8_t *__restrict__ Wp, const float *__restrict__ gamma, int N, int K,
    float *__restrict__ Y, int32_t *__restrict__ acc_out, int m_tiles, const GateUp gu) {
    constexpr int BM2 = 32 * MI2 * WM, BN2 = 32 * NJ2 * WN, kThreads2 = 64 * WM * WN;
    static_assert(BM2 * 8 % kThreads2 == 0 && BN2 * 2 % kThreads2 == 0,
                  "every thread stages whole 16-byte groups of A and B");
    static_assert(!GU || (NJ2 == 2 && WN == 4),
                  "gate/up mode: 4 waves across, one gate and one up block each");
    constexpr int AG = BM2 * 8 / kThreads2, BG = BN2 * 2 / kThreads2;
    // 128 x 256 tiles: a wave raises its priority while it issues its MFMAs
    // (K6912 -> N2560 at M = 2048: 52.5 against 53.6-54.5 us); the 256 x 256
    // tiles run slower with it (47.8-48.8 against 43.4-44.2 us).
    constexpr bool kPrio = MI2 == 2;
    constexpr int kStageA = BM2 * kAPitch, kStageB = BN2 * kBPitch;
    constexpr int BNO = GU ? BN2 / 2 : BN2;    // output columns of a tile
    // LDS: the double-buffered operand stages; in gate/up mode the epilogue
    // reuses the same bytes for the tile's H values [BM2][BNO + 8].
    constexpr int kHPitch = BNO + 8;
    constexpr int kMainBytes = 2 * kStageA * 16 + 2 * kStageB * 4;
    constexpr int kEpiBytes = GU ? BM2 * kHPitch * 4 : 0;
    constexpr int kLdsBytes = kMainBytes > kEpiBytes ? kMainBytes : kEpiBytes;
    __shared__ uint4 smem[kLdsBytes / 16];
    uint4 *const As = smem;
    uint32_t *const Bs = reinterpret_cast<uint32_t *>(smem + 2 * kStageA);
    __shared__ float cS[BM2];                  // fl(gamma * d[row]) of the tile's rows
    __shared__ float cSu[GU ? BM2 : 1];        // fl(gamma_u * d[row]) (gate/up mode)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int m_base = (blockIdx.x % m_tiles) * BM2;
    const int n_base = (blockIdx.x / m_tiles) * BNO;
    const int KB = K / 4;
    const int KT = K / BK2;                    // full 128-wide steps
    v16i acc[MI2][NJ2];
#pragma unroll
    for (int i = 0; i < MI2; ++i)
#pragma unroll
        for (int j = 0; j < NJ2; ++j) acc[i][j] = v16i{};
    SrcPtr<AG, BG> sp = src_ptrs<BM2, BN2, kThreads2, AG, BG, A4>(Xq, Wp, M, N, K, KB, m_base, n_base, tid);
    if constexpr (GU) gate_up_b_ptrs<BN2, kThreads2, AG, BG>(sp, Wp, gu.Wu, N, KB, n_base, tid);
    const int a_off = (wm * 32 * MI2 + (lane & 31)) * kAPitch + (lane >> 5);
    const int b_off = (wn * 32 * NJ2 + (lane & 31)) * kBPitch + (lane >> 5);
    // The loads for k-step kt + 2 are issued on every step, past the end
    // from the last k-step again (a valid address, never stored to LDS):
    // with no branch around them the compiler knows that exactly one
    // stage's loads are in flight behind the stage it stores, and waits for
    // that stage only instead of draining everything issued this step.
    // The row factors are read once, ahead of the operand loads, and kept in
    // LDS: the epilogue then issues no global load, so its stores never wait
    // behind one (the vector-memory counter retires loads and stores in order).
    float d_row[(BM2 + kThreads2 - 1) / kThreads2];
#pragma unroll
    for (int t = 0; t * kThreads2 < BM2; ++t)
        if (t * kThreads2 + tid < BM2) d_row[t] = d[min(m_base + t * kThreads2 + tid, M - 1)];
    const float g = scalar_load(gamma);
    const float gu_scale = GU ? scalar_load(gu.gamma_u) : 0.0f;
    auto put_row_factors = [&]() {
#pragma unroll
        for (int t = 0; t * kThreads2 < BM2; ++t)
            if (t * kThreads2 + tid < BM2) {
                cS[t * kThreads2 + tid] = __fmul_rn(g, d_row[t]);
                if constexpr (GU) cSu[t * kThreads2 + tid] = __fmul_rn(gu_scale, d_row[t]);
            }
    };
    const int kt_last = KT - 1;
    if (KT > 0) {
        Stage2<AG, BG> s0, s1;
        load_stage2<AG, BG, A4>(s0, sp, 0);
        load_stage2<AG, BG, A4>(s1, sp, min(1, kt_last) * BK2);
        put_row_factors();
        store_stage2<kThreads2, AG, BG, A4>(s0, As, Bs, tid);
        __syncthreads();
#define BL_STEP(KT_, MINE, NEXT)                                                              \
        {                                                                                         \
            const int kt_ = (KT_);                                                                \
            load_stage2<AG, BG, A4>(MINE, sp, min(kt_ + 2, kt_last) * BK2);                      \
            const int buf = kt_ & 1;                                                              \
            __builtin_amdgcn_iglp_opt(1);                                                       \
            const uint4 *A = As + buf * kStageA + a_off;                                          \
            const uint32_t *B = Bs + buf * kStageB + b_off;                                       \
            _Pragma("unroll") for (int h = 0; h < 4; ++h) {                                       \
                v4i bf[NJ2];                                                                      \
                _Pragma("unroll") for (int j = 0; j < NJ2; ++j) {                                 \
                    uint4 v;                                                                      \
                    unpack16(B[j * 32 * kBPitch + 2 * h], v.x, v.y, v.z, v.w);                    \
                    bf[j] = as_v4i(v);                                                            \
                }                                                                                 \
                v4i af[MI2];                                                                      \
                _Pragma("unroll") for (int i = 0; i < MI2; ++i)                                   \
                    af[i] = as_v4i(A[i * 32 * kAPitch + 2 * h]);                                  \
                if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);                              \
                _Pragma("unroll") for (int i = 0; i < MI2; ++i)                                   \
                    _Pragma("unroll") for (int j = 0; j < NJ2; ++j)                               \
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0); \
                if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);                              \
            }                                                                                     \
            if (kt_ + 1 < KT) store_stage2<kThreads2, AG, BG, A4>(NEXT, As + (buf ^ 1) * kStageA, Bs + (buf ^ 1) * kStageB, tid); \
            __syncthreads();                                                                      \
        }
        int kt = 0;
#pragma unroll 1
        for (; kt + 2 <= KT; kt += 2) {
            BL_STEP(kt, s0, s1)
            BL_STEP(kt + 1, s1, s0)
        }
        if (kt < KT) BL_STEP(kt, s0, s1)
    }
#undef BL_STEP
    if (KT == 0) {                             // K < 128: no prologue ran
        put_row_factors();
        __syncthreads();
    }
    // K % 128 == 64: one last 64-wide half step straight from global memory
    if (K % BK2) {
        const int k0 = KT * BK2;
        Stage2<AG, BG> st;
#pragma unroll
        for (int i = 0; i < AG; ++i) {
            const int idx = tid + kThreads2 * i;
            if constexpr (A4) {
                uint2 v = make_uint2(0u, 0u);
                if ((idx & 7) < 4) v = *reinterpret_cast<const uint2 *>(sp.a[i] + k0 / 2);
                st.a[i] = make_uint4(v.x, v.y, 0u, 0u);
            } else {
                st.a[i] = (idx & 7) < 4 ? *reinterpret_cast<const uint4 *>(sp.a[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int i = 0; i < BG; ++i) {
            const int idx = tid + kThreads2 * i;
            st.b[i] = (idx & 1) == 0 ? *reinterpret_cast<const uint4 *>(sp.b[i] + k0 / 4) : make_uint4(0u, 0u, 0u, 0u);
        }
        store_stage2<kThreads2, AG, BG, A4>(st, As, Bs, tid);
        __syncthreads();
        const uint4 *A = As + a_off;
        const uint32_t *B = Bs + b_off;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4i bf[NJ2];
#pragma unroll
            for (int j = 0; j < NJ2; ++j) {
                uint4 v;
                unpack16(B[j * 32 * kBPitch + 2 * h], v.x, v.y, v.z, v.w);
                bf[j] = as_v4i(v);
            }
#pragma unroll
            for (int i = 0; i < MI2; ++i) {
                const v4i a = as_v4i(A[i * 32 * kAPitch + 2 * h]);
#pragma unroll
                for (int j = 0; j < NJ2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bf[j], acc[i][j], 0, 0, 0);
            }
        }
    }

    if constexpr (GU) {
        gate_up_epilogue<WM, MI2, BM2, BNO, kHPitch>(acc, reinterpret_cast<float *>(smem), cS, cSu,
                                                    gu, M, N, m_base, n_base, wm, wn, lane, wave);
        return;
    }
    // Whole tile inside Y and no int32 copy: branch-free stores from one
    // per-lane base pointer (row offsets are uniform multiples of N).
    if (!acc_out && m_base + BM2 <= M && n_base + BN2 <= N) {
        float *yl = Y + (size_t)(m_base + wm * 32 * MI2 + 4 * (lane >> 5)) * N +
                    (n_base + wn * 32 * NJ2 + (lane & 31));
        const float *cl = cS + wm * 32 * MI2 + 4 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < MI2; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = i * 32 + 8 * (r >> 2) + (r & 3);
                const float c = cl[lr];
                float *y = yl + (size_t)lr * N;
#pragma unroll
                for (int j = 0; j < NJ2; ++j) y[j * 32] = rescale(acc[i][j][r], c);
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < MI2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int lrow = wm * 32 * MI2 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int row = m_base + lrow;
            if (row >= M) continue;
            const float c = cS[lrow];
#pragma unroll
            for (int j = 0; j < NJ2; ++j) {
                const int col = n_base + wn * 32 * NJ2 + j * 32 + (lane & 31);
                if (col < N) {
                    const size_t o = (size_t)row * N + col;
                    Y[o] = rescale(acc[i][j][r], c);
                    if (acc_out) acc_out[o] = acc[i][j][r];
                }
            }
        }
    }
}

}  // namespace

namespace {
template <bool A4>
hipError_t launch_gemm_t(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                         const float *gamma, int N, int K, float *Y, int32_t *acc,
                         hipStream_t s) {
    if (M == 0 || N == 0)
        return hipSuccess;
    if (!A4 && M < 128 && gemm_skinny_fits(M, K))
        return launch_gemm_skinny(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
    if (M >= 128) {
        int cfg = (N >= 4096 && M >= 256) ? 0 : 1;
#ifdef BL_GEMM_CFG
        cfg = BL_GEMM_CFG;                        // tuning builds only
#endif
        if (cfg == 0) {
            const int m_tiles = (M + 127) / 128, n_tiles = (N + 255) / 256;
            hipLaunchKernelGGL((gemm256_kernel<1, 4, 4, 2, false, A4>), dim3(m_tiles * n_tiles), dim3(256), 0,
                               s, Xq, d, M, Wp, gamma, N, K, Y, acc, m_tiles, GateUp{});
        } else {
            const int m_tiles = (M + 127) / 128, n_tiles = (N + 255) / 256;
            hipLaunchKernelGGL((gemm256_kernel<2, 4, 2, 2, false, A4>), dim3(m_tiles * n_tiles), dim3(512), 0,
                               s, Xq, d, M, Wp, gamma, N, K, Y, acc, m_tiles, GateUp{});
        }
        return hipGetLastError();
    }
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
    hipLaunchKernelGGL(gemm_kernel<A4>, grid, dim3(256), 0, s, Xq, d, M, Wp, gamma, N, K, Y, acc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                       const float *gamma, int N, int K, float *Y, int32_t *acc,
                       hipStream_t s) {
    return launch_gemm_t<false>(Xq, d, M, Wp, gamma, N, K, Y, acc, s);
}

hipError_t launch_bitlinear_a4(const uint8_t *Xq4, const float *d, int M, const uint8_t *Wp,
                               const float *gamma, int N, int K, float *Y, int32_t *acc,
                               hipStream_t s) {
    if (M <= kGemvMaxTokens)
        return launch_gemv_a4(Xq4, d, M, Wp, gamma, N, K, Y, acc, s);
    return launch_gemm_t<true>(reinterpret_cast<const int8_t *>(Xq4), d, M, Wp, gamma, N, K, Y, acc, s);
}

hipError_t launch_ffn_gate_up(const int8_t *Xq, const float *d, int M, int K, const uint8_t *Wg,
                              const float *gamma_g, const uint8_t *Wu, const float *gamma_u,
                              const float *norm_w, int F, float *Z, float *pmax, double *psum,
                              hipStream_t s) {
    if (M == 0 || F == 0)
        return hipSuccess;
    const int m_tiles = (M + 255) / 256, n_tiles = ffn_gate_up_tiles(F);
    const GateUp gu{Wu, gamma_u, norm_w, Z, pmax, psum, n_tiles};
    hipLaunchKernelGGL((gemm256_kernel<2, 4, 4, 2, true>), dim3(m_tiles * n_tiles), dim3(512), 0, s,
                       Xq, d, M, Wg, gamma_g, F, K, nullptr, nullptr, m_tiles, gu);
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
