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
// hi = bf16(a) and lo = bf16(a - hi) (a = hi + lo to about 2^-17 relative;
// both roundings to nearest even, v_cvt_pk_bf16_f32), and
// v_mfma_f32_32x32x16_bf16 takes both halves against the same integer
// operand: every product is exact in fp32, only the fp32 accumulation rounds.
//
// One product kernel, C[i][j] = s . sum_c A[i][c] B[j][c], B bf16 and A
// either fp32 (split while it is staged into LDS) or already split into two
// bf16 planes, both operands contraction-contiguous.  Preparation kernels put
// the operands in that form (rows padded to a multiple of 64, pads written as
// zeros):
//     dX:  A = dY [M][N] fp32,                 B = Wq^T [K][Np] bf16,  s = gamma
//     dW:  A = (dY o d)^T [N][Mp] hi/lo bf16,  B = Xq^T [K][Mp] bf16,  s = 1
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;                         // preparation tile (elements)

// bf16 bits of small integers (|v| <= 127, exact): the top half of the fp32.
__device__ __forceinline__ uint32_t bf16_of_int(int v) { return __float_as_uint((float)v) >> 16; }

// Two fp32 values -> their bf16 pair (round to nearest even), low half first.
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
    const bf16x2 h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// hi / lo split of two fp32 values: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = cvt_pk(a, b);
    lo = cvt_pk(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

// Wq^T [K][ld] (bf16) from the packed rows Wp [N][K/4]: tile of 64 rows n x
// 64 weights k; codes {0, 1, 2} -> {0, +1, -1}; columns n >= N are zeros.
__global__ __launch_bounds__(256) void unpack_transpose_kernel(const uint8_t *__restrict__ Wp, int N,
                                                               int K, uint16_t *__restrict__ WT,
                                                               int ld) {
    __shared__ uint16_t s[kTile][kTile + 8];     // 144-byte rows: 16-byte aligned reads
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
            s[16 * q + j][r] = (uint16_t)bf16_of_int((int)(c & 1u) - (int)(c >> 1));
        }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int e = t + 256 * p;
        const int k = e >> 3, seg = e & 7;                // row k0 + k, 8 columns per segment
        const uint4 v = *reinterpret_cast<const uint4 *>(&s[k][8 * seg]);
        *reinterpret_cast<uint4 *>(WT + (size_t)(k0 + k) * ld + n0 + 8 * seg) = v;
    }
}

// (dY o d)^T split into bf16 planes GH, GL [N][ld]: G^T[n][m] = fl(dY[m][n] d[m]),
// GH = bf16(G^T), GL = bf16(G^T - GH); columns m >= M are zeros.  A 1-D grid
// of m_tiles x n-tiles 64 x 64 tiles (either count may pass grid.y's limit).
__global__ __launch_bounds__(256) void transpose_scale_split_kernel(const float *__restrict__ dY,
                                                                    const float *__restrict__ d,
                                                                    int M, int N,
                                                                    uint16_t *__restrict__ GH,
                                                                    uint16_t *__restrict__ GL,
                                                                    int ld, int m_tiles) {
    __shared__ float s[kTile][kTile + 1];
    const int t = threadIdx.x;
    const int m0 = (int)(blockIdx.x % m_tiles) * kTile, n0 = (int)(blockIdx.x / m_tiles) * kTile;
    // Every load first, unconditional at clamped (in-bounds) addresses
    // (M, N >= 1 here), then the products: with a branch around each load
    // the compiler waited for every load before issuing the next.
    constexpr int kPer = kTile * kTile / 256;
    float yv[kPer], dv[kPer];
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
        const int e = t + 256 * p;
        const int r = e >> 6, c = e & 63;                 // dY row m0 + r, column n0 + c
        const int rr = min(m0 + r, M - 1), cc = min(n0 + c, N - 1);
        yv[p] = dY[(size_t)rr * N + cc];
        dv[p] = d[rr];
    }
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
        const int e = t + 256 * p;
        const int r = e >> 6, c = e & 63;
        s[c][r] = (m0 + r < M && n0 + c < N) ? __fmul_rn(yv[p], dv[p]) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kTile * kTile / 512; ++p) {
        const int e = t + 256 * p;
        const int r = e >> 5, c = 2 * (e & 31);           // G^T row n0 + r, columns m0 + c, + 1
        if (n0 + r < N) {
            uint32_t hi, lo;
            split2(s[r][c], s[r][c + 1], hi, lo);
            const size_t o = (size_t)(n0 + r) * ld + m0 + c;
            *reinterpret_cast<uint32_t *>(GH + o) = hi;
            *reinterpret_cast<uint32_t *>(GL + o) = lo;
        }
    }
}

// Xq^T [K][ld] (bf16); columns m >= M are zeros.
__global__ __launch_bounds__(256) void transpose_i8_kernel(const int8_t *__restrict__ Xq, int M,
                                                           int K, uint16_t *__restrict__ XT, int ld) {
    __shared__ uint16_t s[kTile][kTile + 8];     // 144-byte rows: 16-byte aligned reads
    const int t = threadIdx.x;
    const int m0 = blockIdx.x * kTile, k0 = blockIdx.y * kTile;
    {
        const int r = t >> 2, seg = t & 3;                // Xq row m0 + r, 16 columns k per segment
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (m0 + r < M)
            v = *reinterpret_cast<const uint4 *>(Xq + (size_t)(m0 + r) * K + k0 + 16 * seg);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 16; ++j)
            s[16 * seg + j][r] = (uint16_t)bf16_of_int((int)(int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFF));
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int e = t + 256 * p;
        const int k = e >> 3, seg = e & 7;
        const uint4 v = *reinterpret_cast<const uint4 *>(&s[k][8 * seg]);
        *reinterpret_cast<uint4 *>(XT + (size_t)(k0 + k) * ld + m0 + 8 * seg) = v;
    }
}

// ------------------------------------------------------------- the product
// 128 x 256 tiles of C, 4 waves of 64 x 128 (2 x 4 blocks of 32 x 32); 32-wide
// c-steps, double-buffered in LDS, the next step's operands loaded while the
// current one computes.  LDS rows hold 32 bf16 + 8 pad (80 bytes: the 16-byte
// fragment reads of 16 consecutive rows hit distinct banks).
constexpr int kTI = 128, kTJ = 256, kBC = 32;
constexpr int kRowDw = (kBC + 8) / 2;             // dwords per LDS row
constexpr int kAhiRow = 0, kAloRow = kTI, kBRow = 2 * kTI;
constexpr int kStageDw = (2 * kTI + kTJ) * kRowDw;

struct Operands {
    const float *a32;                             // fp32 A, split in the kernel (or null)
    const uint16_t *ahi, *alo;                    // bf16 planes of A (when a32 is null)
    int lda;
    const uint16_t *b;
    int ldb;
};

template <bool kF32A> struct Staged;
template <> struct Staged<true> { float4 a[4]; uint4 b[4]; };
template <> struct Staged<false> { uint4 ah[2], al[2]; uint4 b[4]; };

// Row and 16-byte chunk that staged element e of a 16-byte-per-lane operand
// (A planes, B) takes.  One wave store covers 16 rows of 64 bytes; each
// 16-lane quarter takes rows {k, k + 4, k + 8, k + 12}, whose 80-byte-pitch
// bank ranges tile the 64 banks exactly (rows k .. k + 3 would wrap onto
// each other).  The global load uses the same map, 4 lanes per 64-byte row.
__device__ __forceinline__ void chunk_of(int e, int &r, int &q) {
    const int l = e & 63;
    r = ((e >> 6) << 4) + (l >> 4) + 4 * ((l >> 2) & 3);
    q = l & 3;
}

// The same for fp32 A, 8 lanes per 32-float row, each lane storing 8 bytes
// per plane: a half-wave store covers 4 rows, taken as {k, k + 4, k + 8,
// k + 12} of a 16-row group that two consecutive 64-lane groups share.
__device__ __forceinline__ void chunk8_of(int e, int &r, int &q) {
    const int g = e >> 6, l = e & 63;
    r = ((g >> 1) << 4) + (((g & 1) << 1) | (l >> 5)) + 4 * ((l >> 3) & 3);
    q = l & 7;
}

// Branch-free loads: rows past I (J) read row I - 1 (J - 1), whose products
// land only in outputs that are never stored; fp32 columns past C read column
// C - 4, and meet B's zero pad columns.  Planes and B have zero pad columns
// up to the row length, a multiple of 64.
template <bool kF32A>
__device__ __forceinline__ void load_stage(Staged<kF32A> &st, const Operands &op, int I, int J, int C,
                                           int i0, int j0, int c0, int t) {
    if constexpr (kF32A) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            int r, q;                                     // row i0 + r, columns c0 + 4q .. + 3
            chunk8_of(t + 256 * p, r, q);
            const int rr = min(i0 + r, I - 1), cc = min(c0 + 4 * q, C - 4);
            st.a[p] = *reinterpret_cast<const float4 *>(op.a32 + (size_t)rr * op.lda + cc);
        }
    } else {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            int r, q;                                     // row i0 + r, columns c0 + 8q .. + 7
            chunk_of(t + 256 * p, r, q);
            const size_t o = (size_t)min(i0 + r, I - 1) * op.lda + c0 + 8 * q;
            const uint4 h = *reinterpret_cast<const uint4 *>(op.ahi + o);
            const uint4 l = *reinterpret_cast<const uint4 *>(op.alo + o);
            st.ah[p] = h;
            st.al[p] = l;
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        int r, q;                                         // row j0 + r, columns c0 + 8q .. + 7
        chunk_of(t + 256 * p, r, q);
        const uint4 v = *reinterpret_cast<const uint4 *>(op.b + (size_t)min(j0 + r, J - 1) * op.ldb +
                                                         c0 + 8 * q);
        st.b[p] = v;
    }
}

template <bool kF32A>
__device__ __forceinline__ void store_stage(const Staged<kF32A> &st, uint32_t *lds, int t) {
    if constexpr (kF32A) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            int r, q;
            chunk8_of(t + 256 * p, r, q);
            uint32_t h0, l0, h1, l1;
            split2(st.a[p].x, st.a[p].y, h0, l0);
            split2(st.a[p].z, st.a[p].w, h1, l1);
            *reinterpret_cast<uint2 *>(lds + (kAhiRow + r) * kRowDw + 2 * q) = make_uint2(h0, h1);
            *reinterpret_cast<uint2 *>(lds + (kAloRow + r) * kRowDw + 2 * q) = make_uint2(l0, l1);
        }
    } else {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            int r, q;
            chunk_of(t + 256 * p, r, q);
            *reinterpret_cast<uint4 *>(lds + (kAhiRow + r) * kRowDw + 4 * q) = st.ah[p];
            *reinterpret_cast<uint4 *>(lds + (kAloRow + r) * kRowDw + 4 * q) = st.al[p];
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        int r, q;
        chunk_of(t + 256 * p, r, q);
        *reinterpret_cast<uint4 *>(lds + (kBRow + r) * kRowDw + 4 * q) = st.b[p];
    }
}

__device__ __forceinline__ bf16x8 frag(const uint32_t *lds, int row, int col) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(lds + row * kRowDw + col));
}

// Tile order: the 8 XCDs receive workgroups round-robin; each XCD takes a
// contiguous run of row-major tiles, so the row panels of A it streams stay
// in its own L2.
__device__ __forceinline__ int xcd_tile(int L, int T) {
    const int q = T / 8, rem = T % 8, x = L % 8;
    return x * q + min(x, rem) + L / 8;
}

struct Frags {
    bf16x8 ah[2], al[2], bb[4];
};

// One 16-wide sub-step's fragments of a wave: A hi / lo rows arow + 32a and B
// rows brow + 32b, columns col .. col + 3 (dwords).
__device__ __forceinline__ void read_frags(Frags &f, const uint32_t *L, int arow, int brow, int col) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        f.ah[a] = frag(L, kAhiRow + arow + 32 * a, col);
        f.al[a] = frag(L, kAloRow + arow + 32 * a, col);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) f.bb[b] = frag(L, brow + 32 * b, col);
}

__device__ __forceinline__ void mfma_substep(f32x16 (&acc)[2][4], const Frags &f) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.ah[a], f.bb[b], acc[a][b], 0, 0, 0);
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.al[a], f.bb[b], acc[a][b], 0, 0, 0);
        }
}

// kPipe: sub-step 1's fragments are read before sub-step 0's MFMAs, and the
// next step's sub-step 0 fragments right after the barrier, under sub-step
// 1's MFMAs, so LDS latency hides behind matrix work.  It needs both
// sub-steps' fragments live, which with fp32 A does not fit two workgroups
// per CU; both loops add the same products in the same order.
//
// Work units.  The first `full` units are whole tiles (scaled and stored to
// Out).  The remaining `tail` tiles -- a last round that would leave most
// slots idle -- are split into `splits` contraction ranges of split_steps
// c-steps: unit full + z tail + t takes tile full + t over the c-steps
// [z split_steps, (z + 1) split_steps) and stores its raw partial tile
// (kTI x kTJ floats) to part + (z tail + t) kTI kTJ, for split_sum_kernel.
// Whole tiles are dispatched first, so the split units fill the slots the
// last whole round frees; each group runs in XCD-chunked order (full is a
// multiple of 8).
template <bool kF32A, bool kPipe>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gemm_bf16x2_kernel(
    const Operands op, int I, int J, int C, int full, int tail, int tiles_j, int split_steps,
    float *__restrict__ part, const float *__restrict__ scale, float *__restrict__ Out, int ldo) {
    __shared__ uint32_t lds[2 * kStageDw];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wi = wave >> 1, wj = wave & 1;
    const int total_steps = (C + kBC - 1) / kBC;
    const int L = blockIdx.x;
    const bool whole = L < full;
    int tile, z = 0;
    if (whole) {
        tile = xcd_tile(L, full);
    } else {
        const int v = xcd_tile(L - full, gridDim.x - full);
        z = v / tail;
        tile = full + (v - z * tail);
    }
    const int i0 = (tile / tiles_j) * kTI, j0 = (tile % tiles_j) * kTJ;
    const int cb = z * split_steps * kBC;                 // first column of this unit
    const int steps = whole ? total_steps : min(split_steps, total_steps - z * split_steps);

    f32x16 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    const int arow = wi * 64 + (lane & 31), brow = kBRow + wj * 128 + (lane & 31);
    const int col0 = 4 * (lane >> 5), col1 = 8 + 4 * (lane >> 5);
    Staged<kF32A> st;
    if (steps > 0) {
        load_stage<kF32A>(st, op, I, J, C, i0, j0, cb, t);
        store_stage<kF32A>(st, lds, t);
        if (steps > 1) load_stage<kF32A>(st, op, I, J, C, i0, j0, cb + kBC, t);
    }
    __syncthreads();
    if constexpr (kPipe) {
        Frags f0, f1;
        if (steps > 0) read_frags(f0, lds, arow, brow, col0);
        for (int s = 0; s < steps; ++s) {
            read_frags(f1, lds + (s & 1) * kStageDw, arow, brow, col1);
            mfma_substep(acc, f0);
            if (s + 1 < steps) {
                store_stage<kF32A>(st, lds + ((s + 1) & 1) * kStageDw, t);
                if (s + 2 < steps) load_stage<kF32A>(st, op, I, J, C, i0, j0, cb + (s + 2) * kBC, t);
            }
            __syncthreads();
            if (s + 1 < steps) read_frags(f0, lds + ((s + 1) & 1) * kStageDw, arow, brow, col0);
            mfma_substep(acc, f1);
        }
    } else {
        for (int s = 0; s < steps; ++s) {
            const uint32_t *L = lds + (s & 1) * kStageDw;
            Frags f;
            read_frags(f, L, arow, brow, col0);
            mfma_substep(acc, f);
            read_frags(f, L, arow, brow, col1);
            mfma_substep(acc, f);
            if (s + 1 < steps) {
                store_stage<kF32A>(st, lds + ((s + 1) & 1) * kStageDw, t);
                if (s + 2 < steps) load_stage<kF32A>(st, op, I, J, C, i0, j0, cb + (s + 2) * kBC, t);
            }
            __syncthreads();
        }
    }

    if (!whole) {                                         // raw partial, tile layout
        float *P = part + (size_t)(z * tail + (tile - full)) * (kTI * kTJ);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int il = wi * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
#pragma unroll
                for (int b = 0; b < 4; ++b) P[il * kTJ + wj * 128 + b * 32 + (lane & 31)] = acc[a][b][r];
            }
        return;
    }
    const float sc = scale ? scalar_load(scale) : 1.0f;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = i0 + wi * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (i >= I) continue;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int j = j0 + wj * 128 + b * 32 + (lane & 31);
                if (j < J) Out[(size_t)i * ldo + j] = scale ? __fmul_rn(acc[a][b][r], sc) : acc[a][b][r];
            }
        }
}

constexpr int kCUs = 256;

// Adds a split tile's partial sums in split order, then scales:
// Out = s . (((P0 + P1) + P2) + ...).  Block (t, y): tail tile t, rows
// 16 y .. 16 y + 15; each thread 4 float4 of partials, scalar output stores.
__global__ __launch_bounds__(256) void split_sum_kernel(const float *__restrict__ part, int splits,
                                                        int full, int tail, int tiles_j, int I, int J,
                                                        const float *__restrict__ scale,
                                                        float *__restrict__ Out, int ldo) {
    const float sc = scale ? scalar_load(scale) : 1.0f;
    const int tt = blockIdx.x, tile = full + tt;
    const int i0 = (tile / tiles_j) * kTI, j0 = (tile % tiles_j) * kTJ;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int e = threadIdx.x + 256 * p;
        const int row = 16 * blockIdx.y + (e >> 6), col = 4 * (e & 63);
        const size_t off = (size_t)row * kTJ + col;
        float4 a = *reinterpret_cast<const float4 *>(part + (size_t)tt * (kTI * kTJ) + off);
        for (int z = 1; z < splits; ++z) {
            const float4 b =
                *reinterpret_cast<const float4 *>(part + (size_t)(z * tail + tt) * (kTI * kTJ) + off);
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        if (scale) {
            a.x = __fmul_rn(a.x, sc);
            a.y = __fmul_rn(a.y, sc);
            a.z = __fmul_rn(a.z, sc);
            a.w = __fmul_rn(a.w, sc);
        }
        const int i = i0 + row, j = j0 + col;             // J % 64 == 0: 4 columns in or out
        if (i < I && j < J) {
            float *o = Out + (size_t)i * ldo + j;
            o[0] = a.x;
            o[1] = a.y;
            o[2] = a.z;
            o[3] = a.w;
        }
    }
}

// Schedule of an I x J x C product over the 2 x 256 workgroup slots (two
// per CU): whole rounds of tiles run unsplit; a last round that would fill at
// most half the slots is split along the contraction, up to 8 ways of at
// least 8 c-steps each.  The same rule sizes the workspace.
constexpr int kSlots = 2 * kCUs;
struct Plan {
    int full, tail, splits, split_steps;
};
Plan plan_product(int64_t I, int64_t J, int64_t C) {
    const int64_t tiles = ((I + kTI - 1) / kTI) * ((J + kTJ - 1) / kTJ);
    const int64_t steps = (C + kBC - 1) / kBC;
    const int64_t full = tiles / kSlots * kSlots, tail = tiles - full;
    int64_t s = 1;
    if (tail > 0 && tail <= kSlots / 2 && steps >= 16)
        s = std::max<int64_t>(1, std::min<int64_t>({8, kSlots / tail, steps / 8}));
    if (s == 1)
        return Plan{(int)tiles, 0, 1, (int)steps};
    const int64_t per = (steps + s - 1) / s;
    return Plan{(int)full, (int)tail, (int)((steps + per - 1) / per), (int)per};
}

// fp32 A: the plain loop; bf16 planes: the pipelined loop.  `part` holds
// splits x tail x kTI x kTJ floats when the tail is split.
template <bool kF32A>
hipError_t launch_product(const Operands &op, int I, int J, int C, const float *scale, float *Out,
                          int ldo, float *part, hipStream_t s) {
    const int64_t ti = (I + kTI - 1) / kTI, tj = (J + kTJ - 1) / kTJ;
    if (ti * tj * 8 > INT32_MAX)
        return hipErrorInvalidConfiguration;      // more units than a 1-D grid holds
    const Plan pl = plan_product(I, J, C);
    const int64_t units = (int64_t)pl.full + (int64_t)pl.tail * pl.splits;
    const dim3 block(256);
    hipLaunchKernelGGL((gemm_bf16x2_kernel<kF32A, !kF32A>), dim3((unsigned)units), block, 0, s, op, I,
                       J, C, pl.full, pl.tail, (int)tj, pl.split_steps, part, scale, Out, ldo);
    if (pl.tail > 0)
        hipLaunchKernelGGL(split_sum_kernel, dim3(pl.tail, kTI / 16), block, 0, s, part, pl.splits,
                           pl.full, pl.tail, (int)tj, I, J, scale, Out, ldo);
    return hipGetLastError();
}

int64_t pad64(int64_t v) { return (v + 63) / 64 * 64; }
size_t round256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

// Partial tiles of a product's split tail (none when nothing is split).
size_t partial_bytes(int64_t I, int64_t J, int64_t C) {
    const Plan pl = plan_product(I, J, C);
    return pl.tail > 0 ? (size_t)pl.splits * (size_t)pl.tail * (kTI * kTJ) * 4 : 0;
}

size_t backward_input_ws_bytes(int64_t M, int64_t N, int64_t K) {
    return round256((size_t)K * (size_t)pad64(N) * 2) + partial_bytes(M, K, N);
}

size_t backward_weight_ws_bytes(int64_t M, int64_t N, int64_t K) {
    const size_t mp = (size_t)pad64(M);
    return 2 * round256((size_t)N * mp * 2) + round256((size_t)K * mp * 2) +
           partial_bytes(N, K, (int64_t)mp);
}

// Sizes as validated by the entry points: M, N < 2^31 - 63, K % 64 == 0.
// An empty contraction (N == 0 for dX, M == 0 for dW) reads no operand: the
// product kernel then writes zeros.
hipError_t launch_backward_input(const float *dY, int M, int N, const uint8_t *Wp, const float *gamma,
                                 int K, float *dX, void *ws, hipStream_t s) {
    if (M == 0 || K == 0)
        return hipSuccess;
    const int np = (int)pad64(N);
    uint16_t *WT = static_cast<uint16_t *>(ws);
    if (np > 0)
        hipLaunchKernelGGL(unpack_transpose_kernel, dim3(np / kTile, K / kTile), dim3(256), 0, s, Wp,
                           N, K, WT, np);
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + round256((size_t)K * np * 2));
    const Operands op{dY, nullptr, nullptr, N, WT, np};
    return launch_product<true>(op, M, K, N, np > 0 ? gamma : nullptr, dX, K, part, s);
}

hipError_t launch_backward_weight(const float *dY, int M, int N, const int8_t *Xq, const float *d,
                                  int K, float *dW, void *ws, hipStream_t s) {
    if (N == 0 || K == 0)
        return hipSuccess;
    const int mp = (int)pad64(M);
    const size_t plane = round256((size_t)N * mp * 2);
    uint16_t *GH = static_cast<uint16_t *>(ws);
    uint16_t *GL = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + plane);
    uint16_t *XT = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + 2 * plane);
    if (mp > 0) {
        const int64_t blocks = (int64_t)(mp / kTile) * ((N + kTile - 1) / kTile);
        if (blocks > INT32_MAX)
            return hipErrorInvalidConfiguration;  // more tiles than a 1-D grid holds
        hipLaunchKernelGGL(transpose_scale_split_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dY, d,
                           M, N, GH, GL, mp, mp / kTile);
        hipLaunchKernelGGL(transpose_i8_kernel, dim3(mp / kTile, K / kTile), dim3(256), 0, s, Xq, M, K,
                           XT, mp);
    }
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + 2 * plane +
                                            round256((size_t)K * mp * 2));
    const Operands op{nullptr, GH, GL, mp, XT, mp};
    return launch_product<false>(op, N, K, mp, nullptr, dW, K, part, s);
}

}  // namespace bl
