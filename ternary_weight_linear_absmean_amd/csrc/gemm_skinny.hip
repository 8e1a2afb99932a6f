// gemm_skinny.hip -- W1.58A8 product for a few tokens (M < 128) on int8
// MFMA, reading every packed weight once.
//
// Same product as gemm.hip (the technical-report copy's GPU端 pack / load /
// unpack / compute, int32 accumulation, rescale fl(float(acc) * fl(gamma d))),
// laid out for small M, where the weights dominate the bytes and there are
// too few token tiles to fill the chip:
//
//   * a workgroup (4 waves) owns 32 weight rows -- one 32-column block of Y --
//     for every token: MB blocks of 32 tokens, the rows past M are zero;
//   * K is cut into chunks of 512; wave w takes the chunk's 128-wide quarter
//     w, so a lane needs one 16-byte unit of its row per chunk: lane
//     (r = lane % 32, h = lane / 32) reads bytes [32 q + 16 h, +16) of row r
//     for quarter q.  Every unit of the workgroup is requested at kernel
//     start (K <= 8192: at most 16 per lane), so the whole weight stream is in
//     flight at once;
//   * the tokens' codes of each chunk are staged in LDS (transposed 16-byte
//     groups, double-buffered, loaded one chunk ahead);
//   * k-step t of quarter q takes dword t of each lane's unit, i.e. weights
//     k in [128 q + 64 h + 16 t, +16) on lane half h; the matching activation
//     group (8 w + 4 h + t of the chunk) is the A operand of
//     v_mfma_i32_32x32x32_i8, so each MFMA sums the 32 k of its two halves;
//   * the four waves' int32 partial sums (disjoint k) are added through LDS
//     and the epilogue rescales and stores the 32 x M block.
// Integer sums are exact, so the result does not depend on how k is split.
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kSkThreads = 256;
constexpr int kSkChunk = 512;                     // k per chunk: 4 waves x 128
constexpr int kSkMaxChunks = 16;                  // K <= 8192
constexpr int kSkPitch = kSkChunk / 16 + 1;       // uint4 per staged token row (+1 pad)

__device__ __forceinline__ v4i as_v4i(uint4 v) {
    v4i r;
    r.x = (int)v.x; r.y = (int)v.y; r.z = (int)v.z; r.w = (int)v.w;
    return r;
}

// Activation groups of one chunk: token rows 32 MB, 32 groups of 16 codes.
// Thread tid stages groups e = tid + 256 i (token e / 32, group e % 32).
template <int MB>
__device__ __forceinline__ void load_chunk(uint4 (&a)[MB * 4], const int8_t *__restrict__ Xq, int M,
                                           int K, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < MB * 4; ++i) {
        const int e = tid + kSkThreads * i;
        const int tk = e >> 5, k = k0 + 16 * (e & 31);
        // groups past M or K are zeros (whole waves of them issue no load)
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (tk < M && k < K) v = *reinterpret_cast<const uint4 *>(Xq + (size_t)tk * K + k);
        a[i] = v;
    }
}
template <int MB>
__device__ __forceinline__ void store_chunk(const uint4 (&a)[MB * 4], uint4 *buf, int tid) {
#pragma unroll
    for (int i = 0; i < MB * 4; ++i) {
        const int e = tid + kSkThreads * i;
        buf[(e >> 5) * kSkPitch + (e & 31)] = transpose16(a[i]);
    }
}

template <int MB>
__global__ __launch_bounds__(kSkThreads) void gemm_skinny_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ d, int M,
    const uint8_t *__restrict__ Wp, const float *__restrict__ gamma, int N, int K,
    float *__restrict__ Y, int32_t *__restrict__ acc_out) {
    constexpr int kStage = 32 * MB * kSkPitch;                  // uint4 per chunk buffer
    __shared__ uint4 As[2 * kStage];
    __shared__ float cS[32 * MB];                               // fl(gamma * d[token])
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 32;
    const int nch = (K + kSkChunk - 1) / kSkChunk;
    const int KB = K / 4;

    // 1. every packed-weight unit of this lane, requested before anything else
    const uint8_t *wrow = Wp + (size_t)min(n0 + (lane & 31), N - 1) * KB;
    uint4 w[kSkMaxChunks];
#pragma unroll
    for (int c = 0; c < kSkMaxChunks; ++c) {
        if (c < nch) {
            const int q = 4 * c + wave;                          // 128-wide quarter
            const int off = 32 * q + 16 * (lane >> 5);           // byte offset in the row
            const bool ok = off < KB;                            // K % 64 == 0: whole units
            const uint4 v = *reinterpret_cast<const uint4 *>(wrow + min(off, KB - 16));
            w[c] = ok ? v : make_uint4(0u, 0u, 0u, 0u);         // code 0 = weight 0
        }
    }

    // 2. row factors and the first activation chunks: PF chunks are held in
    //    registers ahead of the one in LDS (two where registers allow)
    constexpr int PF = MB <= 2 ? 2 : 1;
    const float g = scalar_load(gamma);
    if (tid < 32 * MB) cS[tid] = tid < M ? __fmul_rn(g, d[tid]) : 0.0f;
    uint4 a[PF][MB * 4];
    load_chunk<MB>(a[0], Xq, M, K, 0, tid);
    if constexpr (PF == 2) {
        if (nch > 1) load_chunk<MB>(a[1], Xq, M, K, kSkChunk, tid);
    }
    store_chunk<MB>(a[0], As, tid);
    if (nch > PF) load_chunk<MB>(a[0], Xq, M, K, PF * kSkChunk, tid);
    __syncthreads();

    v16i acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b] = v16i{};

    // 3. chunk loop: MFMAs on chunk c while chunks c + 1 .. c + PF sit in
    //    registers; register set (c + 1) % PF holds chunk c + 1
#pragma unroll
    for (int c = 0; c < kSkMaxChunks; ++c) {
        if (c < nch) {
            const uint4 *A = As + (c & 1) * kStage;
            const uint32_t dws[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint4 bv;
                unpack16(dws[t], bv.x, bv.y, bv.z, bv.w);
                const v4i bf = as_v4i(bv);
                const int grp = 8 * wave + 4 * (lane >> 5) + t;
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    const v4i af = as_v4i(A[(32 * b + (lane & 31)) * kSkPitch + grp]);
                    acc[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf, acc[b], 0, 0, 0);
                }
            }
            if (c + 1 < nch) {
                store_chunk<MB>(a[(c + 1) % PF], As + ((c + 1) & 1) * kStage, tid);
                if (c + 1 + PF < nch)
                    load_chunk<MB>(a[(c + 1) % PF], Xq, M, K, (c + 1 + PF) * kSkChunk, tid);
            }
            __syncthreads();
        }
    }

    // 4. add the four waves' partial sums through LDS (the stages are free now)
    int *red = reinterpret_cast<int *>(As);                     // [4][MB][16][64]
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wave * MB + b) * 16 + r) * 64 + lane] = acc[b][r];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MB * 4; ++i) {
        const int e = tid + kSkThreads * i;                      // (b, r, l) = e / 1024, ...
        const int b = e >> 10, r = (e >> 6) & 15, l = e & 63;
        int s = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) s += red[((v * MB + b) * 16 + r) * 64 + l];
        const int lt = 32 * b + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);   // token in the block
        const int col = n0 + (l & 31);
        if (lt < M && col < N) {
            const size_t o = (size_t)lt * N + col;
            Y[o] = rescale(s, cS[lt]);
            if (acc_out) acc_out[o] = s;
        }
    }
}

// Resident variant for M * K <= 64 KB (e.g. up to 9 tokens at K = 6912):
// every activation group is requested together with the weights at kernel
// start and staged once, [M][K / 16 + 1] groups in LDS, so the chunk loop
// runs with no barrier.  A lanes of token rows past M take zeros; groups
// past K in the last chunk meet zero weights (and stay inside the array,
// see res_fits).
constexpr int kResGroups = 4096;                 // 64 KB of LDS
constexpr int kResLoads = kResGroups / kSkThreads;

__global__ __launch_bounds__(kSkThreads) void gemm_skinny_res_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ d, int M,
    const uint8_t *__restrict__ Wp, const float *__restrict__ gamma, int N, int K,
    float *__restrict__ Y, int32_t *__restrict__ acc_out) {
    __shared__ uint4 As[kResGroups];
    __shared__ float cS[32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 32;
    const int nch = (K + kSkChunk - 1) / kSkChunk;
    const int KB = K / 4, G = K / 16, P = G + 1;

    const uint8_t *wrow = Wp + (size_t)min(n0 + (lane & 31), N - 1) * KB;
    uint4 w[kSkMaxChunks];
#pragma unroll
    for (int c = 0; c < kSkMaxChunks; ++c) {
        if (c < nch) {
            const int off = 32 * (4 * c + wave) + 16 * (lane >> 5);
            const uint4 v = *reinterpret_cast<const uint4 *>(wrow + min(off, KB - 16));
            w[c] = off < KB ? v : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    const int total = M * G;
    uint4 a[kResLoads];
#pragma unroll
    for (int i = 0; i < kResLoads; ++i) {
        const int e = tid + kSkThreads * i;
        a[i] = make_uint4(0u, 0u, 0u, 0u);
        if (e < total) {
            const int tk = e / G, grp = e - tk * G;
            a[i] = *reinterpret_cast<const uint4 *>(Xq + (size_t)tk * K + 16 * grp);
        }
    }
    const float g = scalar_load(gamma);
    if (tid < 32) cS[tid] = tid < M ? __fmul_rn(g, d[tid]) : 0.0f;
#pragma unroll
    for (int i = 0; i < kResLoads; ++i) {
        const int e = tid + kSkThreads * i;
        if (e < total) {
            const int tk = e / G, grp = e - tk * G;
            As[tk * P + grp] = transpose16(a[i]);
        }
    }
    __syncthreads();

    v16i acc = v16i{};
    const int m = lane & 31;
    const bool live = m < M;
#pragma unroll
    for (int c = 0; c < kSkMaxChunks; ++c) {
        if (c < nch) {
            const uint32_t dws[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint4 bv;
                unpack16(dws[t], bv.x, bv.y, bv.z, bv.w);
                const int grp = 32 * c + 8 * wave + 4 * (lane >> 5) + t;
                const uint4 av = live ? As[m * P + grp] : make_uint4(0u, 0u, 0u, 0u);
                acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(as_v4i(av), as_v4i(bv), acc, 0, 0, 0);
            }
        }
    }

    __syncthreads();                              // every wave is done reading As
    int *red = reinterpret_cast<int *>(As);       // [4][16][64]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid + kSkThreads * i;
        const int r = e >> 6, l = e & 63;
        const int s = red[r * 64 + l] + red[(16 + r) * 64 + l] + red[(32 + r) * 64 + l] +
                      red[(48 + r) * 64 + l];
        const int lt = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        const int col = n0 + (l & 31);
        if (lt < M && col < N) {
            const size_t o = (size_t)lt * N + col;
            Y[o] = rescale(s, cS[lt]);
            if (acc_out) acc_out[o] = s;
        }
    }
}

// Narrow-N variant on v_mfma_i32_16x16x64_i8: 16 weight rows per workgroup,
// so N = 2560 spreads over 160 workgroups instead of 80 (each CU streams half
// as many bytes).  Chunks are 1024 wide and wave w takes the 256-wide quarter
// w: lane (r = lane % 16, g = lane / 16) reads the 64 weights
// [kq + 64 g, +64) of row r as one 16-byte unit and uses its dword t in
// MFMA step t (k in [kq + 64 g + 16 t, +16) on lane group g, kq the quarter's
// first k); the A operand of token m on lane group g is activation group
// kq / 16 + 4 g + t.  Tokens come in MB blocks of 16.
constexpr int kS16Chunk = 1024;
constexpr int kS16MaxChunks = 8;                  // K <= 8192
constexpr int kS16Pitch = kS16Chunk / 16 + 1;     // uint4 per staged token row (+1 pad)

template <int MB>
__device__ __forceinline__ void load_chunk16(uint4 (&a)[MB * 4], const int8_t *__restrict__ Xq,
                                             int M, int K, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < MB * 4; ++i) {
        const int e = tid + kSkThreads * i;                      // token e / 64, group e % 64
        const int tk = e >> 6, k = k0 + 16 * (e & 63);
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (tk < M && k < K) v = *reinterpret_cast<const uint4 *>(Xq + (size_t)tk * K + k);
        a[i] = v;
    }
}
template <int MB>
__device__ __forceinline__ void store_chunk16(const uint4 (&a)[MB * 4], uint4 *buf, int tid) {
#pragma unroll
    for (int i = 0; i < MB * 4; ++i) {
        const int e = tid + kSkThreads * i;
        buf[(e >> 6) * kS16Pitch + (e & 63)] = transpose16(a[i]);
    }
}

template <int MB>
__global__ __launch_bounds__(kSkThreads) void gemm_skinny16_kernel(
    const int8_t *__restrict__ Xq, const float *__restrict__ d, int M,
    const uint8_t *__restrict__ Wp, const float *__restrict__ gamma, int N, int K,
    float *__restrict__ Y, int32_t *__restrict__ acc_out) {
    constexpr int kStage = 16 * MB * kS16Pitch;
    __shared__ uint4 As[2 * kStage];
    __shared__ float cS[16 * MB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 16;
    const int nch = (K + kS16Chunk - 1) / kS16Chunk;
    const int KB = K / 4;

    const uint8_t *wrow = Wp + (size_t)min(n0 + (lane & 15), N - 1) * KB;
    uint4 w[kS16MaxChunks];
#pragma unroll
    for (int c = 0; c < kS16MaxChunks; ++c) {
        if (c < nch) {
            const int off = 256 * c + 64 * wave + 16 * (lane >> 4);   // bytes: quarter + unit
            const uint4 v = *reinterpret_cast<const uint4 *>(wrow + min(off, KB - 16));
            w[c] = off < KB ? v : make_uint4(0u, 0u, 0u, 0u);
        }
    }

    constexpr int PF = MB <= 2 ? 2 : 1;
    const float g = scalar_load(gamma);
    if (tid < 16 * MB) cS[tid] = tid < M ? __fmul_rn(g, d[tid]) : 0.0f;
    uint4 a[PF][MB * 4];
    load_chunk16<MB>(a[0], Xq, M, K, 0, tid);
    if constexpr (PF == 2) {
        if (nch > 1) load_chunk16<MB>(a[1], Xq, M, K, kS16Chunk, tid);
    }
    store_chunk16<MB>(a[0], As, tid);
    if (nch > PF) load_chunk16<MB>(a[0], Xq, M, K, PF * kS16Chunk, tid);
    __syncthreads();

    v4i acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < kS16MaxChunks; ++c) {
        if (c < nch) {
            const uint4 *A = As + (c & 1) * kStage;
            const uint32_t dws[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint4 bv;
                unpack16(dws[t], bv.x, bv.y, bv.z, bv.w);
                const v4i bf = as_v4i(bv);
                const int grp = 16 * wave + 4 * (lane >> 4) + t;
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    const v4i af = as_v4i(A[(16 * b + (lane & 15)) * kS16Pitch + grp]);
                    acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf, acc[b], 0, 0, 0);
                }
            }
            if (c + 1 < nch) {
                store_chunk16<MB>(a[(c + 1) % PF], As + ((c + 1) & 1) * kStage, tid);
                if (c + 1 + PF < nch)
                    load_chunk16<MB>(a[(c + 1) % PF], Xq, M, K, (c + 1 + PF) * kS16Chunk, tid);
            }
            __syncthreads();
        }
    }

    // the four waves' sums: [4][MB][4][64] through LDS, then 16 x M outputs
    int *red = reinterpret_cast<int *>(As);
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * MB + b) * 4 + r) * 64 + lane] = acc[b][r];
    __syncthreads();
    if (tid < MB * 64) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int b = tid >> 6, l = tid & 63;
            int sum = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) sum += red[((v * MB + b) * 4 + r) * 64 + l];
            const int lt = 16 * b + 4 * (l >> 4) + r;            // token
            const int col = n0 + (l & 15);
            if (lt < M && col < N) {
                const size_t o = (size_t)lt * N + col;
                Y[o] = rescale(sum, cS[lt]);
                if (acc_out) acc_out[o] = sum;
            }
        }
    }
}

// The resident layout holds M rows of K / 16 + 1 groups, and the last chunk
// may read up to 31 groups past a row's end: M (K / 16 + 1) + 32 <= 4096.
bool res_fits(int M, int K) { return M <= 32 && M * (K / 16 + 1) + 32 <= kResGroups; }

}  // namespace

bool gemm_skinny_fits(int M, int K) {
    return M >= 1 && M < 128 && K >= 64 && K <= kSkMaxChunks * kSkChunk;
}

hipError_t launch_gemm_skinny(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                              const float *gamma, int N, int K, float *Y, int32_t *acc,
                              hipStream_t s) {
    if (M == 0 || N == 0)
        return hipSuccess;
    // Narrow N: 16-row workgroups when 32-row ones would leave most CUs idle.
    if (N <= 4096 && M <= 64) {
        const dim3 grid16((N + 15) / 16);
        if (M <= 16)
            hipLaunchKernelGGL(gemm_skinny16_kernel<1>, grid16, dim3(kSkThreads), 0, s, Xq, d, M, Wp,
                               gamma, N, K, Y, acc);
        else if (M <= 32)
            hipLaunchKernelGGL(gemm_skinny16_kernel<2>, grid16, dim3(kSkThreads), 0, s, Xq, d, M, Wp,
                               gamma, N, K, Y, acc);
        else
            hipLaunchKernelGGL(gemm_skinny16_kernel<4>, grid16, dim3(kSkThreads), 0, s, Xq, d, M, Wp,
                               gamma, N, K, Y, acc);
        return hipGetLastError();
    }
    const dim3 grid((N + 31) / 32);
    if (res_fits(M, K))
        hipLaunchKernelGGL(gemm_skinny_res_kernel, grid, dim3(kSkThreads), 0, s, Xq, d, M, Wp, gamma,
                           N, K, Y, acc);
    else if (M <= 32)
        hipLaunchKernelGGL(gemm_skinny_kernel<1>, grid, dim3(kSkThreads), 0, s, Xq, d, M, Wp, gamma,
                           N, K, Y, acc);
    else if (M <= 64)
        hipLaunchKernelGGL(gemm_skinny_kernel<2>, grid, dim3(kSkThreads), 0, s, Xq, d, M, Wp, gamma,
                           N, K, Y, acc);
    else
        hipLaunchKernelGGL(gemm_skinny_kernel<4>, grid, dim3(kSkThreads), 0, s, Xq, d, M, Wp, gamma,
                           N, K, Y, acc);
    return hipGetLastError();
}

}  // namespace bl
