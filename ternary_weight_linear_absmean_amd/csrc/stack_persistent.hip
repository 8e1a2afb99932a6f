// stack_persistent.hip -- the decode stack as one persistent launch per
// chunk of layers.
//
// The one-token stack is a chain of small dependent steps: every BitLinear
// needs the whole previous vector before it can quantise (per-token absmax,
// [NEWS] 权重映射为三元值).  With one launch per step the chain pays a kernel
// boundary per step.  Here one workgroup per compute unit stays resident for
// up to kMaxLayers layers.  Per layer there are four phases, each a set of
// BitLinear rows split evenly over the workgroups:
//   P0  q, k, v = BitLinear(x)        prologue: x = x_mid + y of the layer
//                                     before (the second residual add)
//   P1  o = BitLinear(a)              prologue: a = v repeated per query group
//   P2  (gate f, up f) pairs          prologue: x_mid = x + o (first residual
//                                     add); epilogue: H_f = relu(G_f)^2 U_f
//   P3  y = BitLinear_down(Zq)        prologue: z = H * g, max |z|, sum H^2,
//                                     dz = (max|z| / 127) / rms (subln)
// Each workgroup quantises the phase input itself (every workgroup computes
// the same max and the same codes), so only phase outputs cross workgroups.
//
// Synchronisation is carried by the data.  Every value that crosses
// workgroups is stored as an 8-byte (value, tag) pair with one device-
// coherent 64-bit store; the tag names the layer and phase that produced it.
// A consumer loads its elements of the input vector with device-coherent
// 64-bit loads until every tag is the expected one (the XCDs' L2s are
// bypassed by these accesses, so no L2 write-back or invalidate is needed),
// so reading the input is the barrier: there is no separate flag round trip.
// A producer can never overwrite a value a consumer has yet to read: it
// reaches the next write of the same buffer only after every workgroup has
// produced outputs that come after that read in its program order.  The tags
// are cleared at the start of every call, so a stale value never matches.
//
// The workgroup's waves have two roles.  Receiver waves poll the phase input
// into LDS; compute waves hold the packed weights and form the dot products.
// A wave's vector loads complete in issue order, so polls issued behind a
// phase's weight loads would wait for all of them; with the roles split, the
// compute waves issue the next phase's weight loads (and gammas) as soon as
// their dot products are done, and those stream from HBM while the receivers
// wait for the next input; once they have arrived the compute waves unpack
// up to four units each to int8 values, still before the input is there.
//
// Every wait is bounded by a real-time limit (the caller's, 1 s by default).
// A workgroup that runs out of time (only possible if the grid is not all
// resident, or if the caller set a limit shorter than a phase) raises an
// error word, fills x with NaN and leaves; the others then see the error word
// and leave.  The host reads the word back through the status call.
// The host launches at most one workgroup per compute unit.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

constexpr int kRecvWaves = 4;
constexpr int kR = 64 * kRecvWaves;           // receiver threads
constexpr int kC = 512;                       // compute threads
constexpr int kT = kR + kC;                   // threads per workgroup
constexpr int kS = 6;                         // packed 16-byte weight units per compute thread
constexpr int kPU = 4;                        // of them unpacked while the phase input is awaited
constexpr int kMaxH = 3072;                   // longest H (P0, P1, P2 inputs)
constexpr int kMaxF = 7168;                   // longest F (P3 input)
constexpr int kNH = kMaxH / 2 / kR;           // 2-element chunks per receiver, length H
constexpr int kNF = kMaxF / 2 / kR;           // 2-element chunks per receiver, length F
constexpr int kMaxLayers = 16;                // layers per launch (kernel-argument table)
constexpr int kMaxGrid = 512;
constexpr uint64_t kTicksPerUs = 100;        // the real-time counter runs at 100 MHz
constexpr uint64_t kDefaultWaitUs = 1000000;  // 1 s
constexpr int kSC1 = 16;                      // buffer cache policy: coherent at device scope

typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

struct PLayer {
    const uint8_t *W[7];                      // q k v o gate up down
    const float *g[7];
    const float *norm;
};

struct PArgs {
    PLayer layer[kMaxLayers];
    int n_layers, l0, H, KV, F, D, group;
    float eps;
    int first, last;                          // this launch holds the call's first / last layer
    int lshift[4];                            // log2 lanes per row group, per phase
    int nslot[4];                             // weight units per lane per matrix, per phase
    const float *x_in;
    float *x_out;
    float *trace;                             // row of this launch's first layer, or null
    int trace_stride;
    float *q, *k;                             // outputs nothing reads back
    uint2 *xa, *xm, *v, *o, *h, *y;           // tagged (value bits, tag), slot 0
    int slot_stride;                          // tagged values per layer slot
    unsigned *err;
    uint64_t wait_ticks;                      // limit of every wait
};

// tag of the values produced in phase p of global layer lg (0 = cleared)
__device__ __forceinline__ unsigned tag_of(int lg, int p) { return 4u * lg + p + 1u; }

// Each of kMaxLayers layer slots has its own tagged vectors (layer lg uses
// slot lg % kMaxLayers): within a launch no vector is written twice, so a
// line that a consumer's L2 cached early is never mistaken later (its tag
// would not match anyway; this keeps such misses rare).
__device__ __forceinline__ uint2 *slot(const PArgs &a, uint2 *p, int lg) {
    return p + (size_t)(lg % kMaxLayers) * a.slot_stride;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void st_tag(uint2 *p, float v, unsigned tag) {
    const unsigned long long w = ((unsigned long long)tag << 32) | __float_as_uint(v);
    __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), w, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_u(unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// phase geometry: row groups R and input length K
__device__ __forceinline__ int phase_rows(const PArgs &a, int P) {
    return P == 0 ? a.H + 2 * a.KV : P == 2 ? a.F : a.H;
}
__device__ __forceinline__ int phase_k(const PArgs &a, int P) { return P == 3 ? a.F : a.H; }

// this workgroup's row groups [r0, r0 + nr) of R (b R < 2^31 for the sizes allowed)
__device__ __forceinline__ void wg_rows(int R, int &r0, int &nr) {
    const unsigned G = gridDim.x, b = blockIdx.x;
    r0 = (int)((b * (unsigned)R) / G);
    nr = (int)(((b + 1) * (unsigned)R) / G) - r0;
}

// A pointer every lane holds the same value of, as a uniform (scalar) value.
__device__ __forceinline__ const uint8_t *uniform(const uint8_t *p) {
    const unsigned long long v = (unsigned long long)p;
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v >> 32));
    return (const uint8_t *)(((unsigned long long)hi << 32) | lo);
}

// packed row pointer of row group gr (second matrix of a pair in *second)
template <int P>
__device__ __forceinline__ const uint4 *row_ptr(const PArgs &a, const PLayer &L, int gr,
                                                const uint4 **second) {
    const int H = a.H, KV = a.KV;
    const size_t rb = (size_t)(P == 3 ? a.F : H) / 4;      // bytes per packed row
    if (P == 0) {
        // the three base pointers are loaded as uniform values first, then
        // picked per lane (a per-lane pick of the address to load from would
        // be a vector load of the argument table)
        const uint8_t *wq = uniform(L.W[0]);
        const uint8_t *wk = uniform(L.W[1]);
        const uint8_t *wv = uniform(L.W[2]);
        const uint8_t *base = gr < H ? wq + (size_t)gr * rb
                            : gr < H + KV ? wk + (size_t)(gr - H) * rb
                                          : wv + (size_t)(gr - H - KV) * rb;
        return reinterpret_cast<const uint4 *>(base);
    }
    if (P == 1) return reinterpret_cast<const uint4 *>(L.W[3] + (size_t)gr * rb);
    if (P == 2) {
        *second = reinterpret_cast<const uint4 *>(L.W[5] + (size_t)gr * rb);
        return reinterpret_cast<const uint4 *>(L.W[4] + (size_t)gr * rb);
    }
    return reinterpret_cast<const uint4 *>(L.W[6] + (size_t)gr * rb);
}

// What a compute thread needs before the phase input arrives: its packed
// weight units and the phase's gammas.
struct Pre {
    uint4 w[kS];
    uint4 v[kPU][4];                          // units i < kPU unpacked: v[i][t] from dword t
    float g0, g1, g2;
};

// Compute thread ct issues the loads of phase P: row group ct >> lshift of
// the workgroup's range, units s, s + L, ... (row and unit clamped).
template <int P>
__device__ __forceinline__ void prefetch(const PArgs &a, const PLayer &L, int ct, Pre &pre) {
    const int R = phase_rows(a, P), K = phase_k(a, P);
    int r0, nr;
    wg_rows(R, r0, nr);
    const int ls = a.lshift[P], ns = a.nslot[P];
    const int s = ct & ((1 << ls) - 1);
    const bool live = (ct >> ls) < nr;
    const int gr = min(r0 + min(ct >> ls, max(nr - 1, 0)), R - 1);
    const int upr = K / 64;
    const uint4 *second = nullptr;
    const uint4 *row = row_ptr<P>(a, L, gr, &second);
    constexpr int half = P == 2 ? kS / 2 : kS;
#pragma unroll
    for (int i = 0; i < half; ++i) {
        if (i < ns && live) {
            const int u = min(s + (i << ls), upr - 1);
            pre.w[i] = row[u];
            if (P == 2) pre.w[half + i] = second[u];
        }
    }
    if (P == 0) { pre.g0 = scalar_load(L.g[0]); pre.g1 = scalar_load(L.g[1]); pre.g2 = scalar_load(L.g[2]); }
    if (P == 1) pre.g0 = scalar_load(L.g[3]);
    if (P == 2) { pre.g0 = scalar_load(L.g[4]); pre.g1 = scalar_load(L.g[5]); }
    if (P == 3) pre.g0 = scalar_load(L.g[6]);
}

// Unpacks the first kPU loaded units of phase P (the first matrix of a
// pair) into int8 values, so that after the input arrives only the v_dot4
// work remains for them.  Run between the loads and the wait for the input.
template <int P>
__device__ __forceinline__ void unpack_pre(const PArgs &a, Pre &pre) {
    const int ns = a.nslot[P];
    constexpr int half = P == 2 ? kS / 2 : kS;
    constexpr int nu = half < kPU ? half : kPU;
#pragma unroll
    for (int i = 0; i < nu; ++i) {
        if (i < ns) {
            const uint32_t dw[4] = {pre.w[i].x, pre.w[i].y, pre.w[i].z, pre.w[i].w};
#pragma unroll
            for (int t = 0; t < 4; ++t)
                unpack16(dw[t], pre.v[i][t].x, pre.v[i][t].y, pre.v[i][t].z, pre.v[i][t].w);
        }
    }
}

struct Smem {
    float vals[kMaxF];                       // the phase input (fp32), staged by the receivers
    float gain[kMaxF];                       // the subln gain of the current layer
    uint4 xs[kMaxF / 16];                    // its int8 codes, transposed groups, [4][K / 64]
    float red_a[kRecvWaves];
    double red_s[kRecvWaves];
    unsigned fail;
};

// ------------------------------------------------------------- receivers
// Receiver r holds chunks c = r + i kR (2 elements each: 2c, 2c + 1).

// Poll chunks of one or two tagged vectors (element index map idx, which
// keeps a chunk's two elements adjacent) until both halves of every chunk
// carry the expected tag; emit(c, w0, w1) is called once per chunk as it
// completes.  false on time-out or a raised error.
template <int NC, bool TWO, typename Index, typename Emit>
__device__ __forceinline__ bool receive(const PArgs &a, const uint2 *p0, unsigned t0,
                                        const uint2 *p1, unsigned t1, int n_src, int n,
                                        Index idx, Emit emit) {
    const int r = threadIdx.x;
    const __amdgpu_buffer_rsrc_t r0 = rsrc(p0, n_src * 8);
    const __amdgpu_buffer_rsrc_t r1 = rsrc(TWO ? p1 : p0, n_src * 8);
    const int nch = n / 2;
    const int nj = (nch + kR - 1) / kR;       // uniform
    unsigned pending = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i)
        if (i < nj && r + i * kR < nch) pending |= 1u << i;
    const uint64_t start = __builtin_amdgcn_s_memrealtime();
    // While the producers are still working, only lane 0 of each wave polls,
    // on its last chunk (produced by one of the later workgroups: probing
    // the first chunk, from an early producer, started the sweep while much
    // of the input was still missing, 585-591 against 568-572 us per token;
    // every wave probing the input's very last chunk, 585); a sweep by every
    // lane each round would flood the memory side with re-reads.  The sweep
    // below then reads every chunk.
    {
        int ip = 0;
#pragma unroll
        for (int i = 0; i < NC; ++i)
            if (pending >> i & 1u) ip = i;
        const int off = idx(2 * (r + ip * kR)) * 8;
        for (;;) {
            int rdy = 1;
            if ((threadIdx.x & 63) == 0 && (pending & 1u)) {
                const v4u w0 = __builtin_amdgcn_raw_buffer_load_b128(r0, off, 0, kSC1);
                v4u w1 = w0;
                if (TWO) w1 = __builtin_amdgcn_raw_buffer_load_b128(r1, off, 0, kSC1);
                rdy = w0.y == t0 && w0.w == t0 && (!TWO || (w1.y == t1 && w1.w == t1));
            }
            if (__shfl(rdy, 0)) break;
            if (ld_u(a.err) != 0u || __builtin_amdgcn_s_memrealtime() - start > a.wait_ticks)
                return false;
        }
    }
    // One sweep through the L2 (plain loads: after the proxy most chunks are
    // in memory, and the workgroups of an XCD then share one fetch of each
    // line), then device-coherent re-polls of whatever is still stale.
    auto sweep = [&](auto aux) {
        constexpr int kAux = decltype(aux)::value;
        v4u w0[NC], w1[NC];
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            if (pending >> i & 1u) {
                const int off = idx(2 * (r + i * kR)) * 8;
                w0[i] = __builtin_amdgcn_raw_buffer_load_b128(r0, off, 0, kAux);
                if (TWO) w1[i] = __builtin_amdgcn_raw_buffer_load_b128(r1, off, 0, kAux);
            }
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const bool ready = (pending >> i & 1u) && w0[i].y == t0 && w0[i].w == t0 &&
                               (!TWO || (w1[i].y == t1 && w1[i].w == t1));
            if (ready) {
                emit(r + i * kR, w0[i], TWO ? w1[i] : w0[i]);
                pending &= ~(1u << i);
            }
        }
    };
    sweep(std::integral_constant<int, 0>{});
    while (pending) {
        sweep(std::integral_constant<int, kSC1>{});
        if (pending && (ld_u(a.err) != 0u ||
                        __builtin_amdgcn_s_memrealtime() - start > a.wait_ticks))
            return false;
    }
    return true;
}

struct Same {
    __device__ int operator()(int e) const { return e; }
};
// a[h D + i] = v[(h / group) D + i]; D is even, so a chunk stays in one head
struct Expand {
    int D, group;
    __device__ int operator()(int e) const {
        const int h = e / D;
        return (h / group) * D + (e - h * D);
    }
};

__device__ __forceinline__ float2 halves(const v4u &w) {
    return make_float2(__uint_as_float(w.x), __uint_as_float(w.z));
}

// Workgroup 0 keeps a tagged copy of a phase input chunk (and the trace copy).
__device__ __forceinline__ void keep(uint2 *dst, int n, int c, float2 x, unsigned tag, float *tr) {
    if (blockIdx.x != 0) return;
    const v4u w = {__float_as_uint(x.x), tag, __float_as_uint(x.y), tag};
    __builtin_amdgcn_raw_buffer_store_b128(w, rsrc(dst, n * 8), c * 16, 0, kSC1);
    if (tr) *reinterpret_cast<float2 *>(tr + 2 * c) = x;
}

__device__ __forceinline__ float wave_max(float a) { return group_max(a, 64); }

// P0 input: x of global layer lg (x_in for the call's first layer, else
// x_mid + y of the layer before); workgroup 0 keeps it as xa.
__device__ __forceinline__ bool receive_p0(const PArgs &a, Smem &sm, int lg, float *tr) {
    const int K = a.H;
    float am = 0.0f;
    bool ok = true;
    const unsigned tag = tag_of(lg, 0);
    if (a.first && lg == a.l0) {
        const __amdgpu_buffer_rsrc_t r = rsrc(a.x_in, K * 4);
        const int nj = (K / 2 + kR - 1) / kR;
        v2u w[kNH];
#pragma unroll
        for (int i = 0; i < kNH; ++i)         // all loads first; past the end: 0
            if (i < nj) w[i] = __builtin_amdgcn_raw_buffer_load_b64(
                            r, ((int)threadIdx.x + i * kR) * 8, 0, 0);
#pragma unroll
        for (int i = 0; i < kNH; ++i) {
            const int c = threadIdx.x + i * kR;
            if (i < nj && c < K / 2) {
                const float2 x = make_float2(__uint_as_float(w[i].x), __uint_as_float(w[i].y));
                *reinterpret_cast<float2 *>(sm.vals + 2 * c) = x;
                keep(slot(a, a.xa, lg), K, c, x, tag, tr);
                am = fmaxf(am, fmaxf(fabsf(x.x), fabsf(x.y)));
            }
        }
    } else {
        ok = receive<kNH, true>(a, slot(a, a.xm, lg - 1), tag_of(lg - 1, 2), slot(a, a.y, lg - 1),
                                tag_of(lg - 1, 3), K, K, Same{},
                                [&](int c, const v4u &m, const v4u &y) {
            const float2 mm = halves(m), yy = halves(y);
            const float2 x = make_float2(__fadd_rn(mm.x, yy.x), __fadd_rn(mm.y, yy.y));
            *reinterpret_cast<float2 *>(sm.vals + 2 * c) = x;
            keep(slot(a, a.xa, lg), K, c, x, tag, tr);
            am = fmaxf(am, fmaxf(fabsf(x.x), fabsf(x.y)));
        });
    }
    am = wave_max(am);
    if ((threadIdx.x & 63) == 0) sm.red_a[threadIdx.x >> 6] = am;
    return ok;
}

// P1 input: a = v repeated per query group
__device__ __forceinline__ bool receive_p1(const PArgs &a, Smem &sm, int lg) {
    float am = 0.0f;
    const bool ok = receive<kNH, false>(a, slot(a, a.v, lg), tag_of(lg, 0), nullptr, 0u, a.KV, a.H,
                                        Expand{a.D, a.group},
                                        [&](int c, const v4u &w, const v4u &) {
        const float2 x = halves(w);
        *reinterpret_cast<float2 *>(sm.vals + 2 * c) = x;
        am = fmaxf(am, fmaxf(fabsf(x.x), fabsf(x.y)));
    });
    am = wave_max(am);
    if ((threadIdx.x & 63) == 0) sm.red_a[threadIdx.x >> 6] = am;
    return ok;
}

// P2 input: x_mid = x + o (fp32); workgroup 0 keeps it as xm.
__device__ __forceinline__ bool receive_p2(const PArgs &a, Smem &sm, int lg, float *tr) {
    const int K = a.H;
    float am = 0.0f;
    const unsigned tag = tag_of(lg, 2);
    const bool ok = receive<kNH, true>(a, slot(a, a.xa, lg), tag_of(lg, 0), slot(a, a.o, lg),
                                       tag_of(lg, 1), K, K, Same{},
                                       [&](int c, const v4u &x, const v4u &o) {
        const float2 xx = halves(x), oo = halves(o);
        const float2 m = make_float2(__fadd_rn(xx.x, oo.x), __fadd_rn(xx.y, oo.y));
        *reinterpret_cast<float2 *>(sm.vals + 2 * c) = m;
        keep(slot(a, a.xm, lg), K, c, m, tag, tr);
        am = fmaxf(am, fmaxf(fabsf(m.x), fabsf(m.y)));
    });
    am = wave_max(am);
    if ((threadIdx.x & 63) == 0) sm.red_a[threadIdx.x >> 6] = am;
    return ok;
}

// P3 input: Z = H * g (subln codes) staged, with max |Z| and sum H^2 (fp64,
// each receiver in chunk order, then a fixed tree: every workgroup gets the
// same bits).
__device__ __forceinline__ bool receive_p3(const PArgs &a, Smem &sm, int lg, const float *norm) {
    const int K = a.F;
    const int nj = (K / 2 + kR - 1) / kR;     // uniform
    // The gains go through LDS (each chunk's callback reads its own two back).
    // All loads are issued before any is used (buffer loads: past the end
    // they give 0, never written).
    if (norm) {
        const __amdgpu_buffer_rsrc_t rg = rsrc(norm, K * 4);
        v2u g[kNF];
#pragma unroll
        for (int i = 0; i < kNF; ++i)
            if (i < nj)
                g[i] = __builtin_amdgcn_raw_buffer_load_b64(rg, ((int)threadIdx.x + i * kR) * 8, 0, 0);
#pragma unroll
        for (int i = 0; i < kNF; ++i) {
            const int c = threadIdx.x + i * kR;
            if (i < nj && c < K / 2)
                *reinterpret_cast<float2 *>(sm.gain + 2 * c) =
                    make_float2(__uint_as_float(g[i].x), __uint_as_float(g[i].y));
        }
    } else {
#pragma unroll
        for (int i = 0; i < kNF; ++i) {
            const int c = threadIdx.x + i * kR;
            if (i < nj && c < K / 2)
                *reinterpret_cast<float2 *>(sm.gain + 2 * c) = make_float2(1.0f, 1.0f);
        }
    }
    // z = H g, max |z| and each chunk's H^2 are formed as the chunks arrive
    // (in the emit callback, not in a pass over the staged row afterwards:
    // 586-591 against 599-602 us per token); the fp64 sum then runs over the
    // chunks in their fixed order, so every workgroup gets the same bits.
    // (Parking the per-chunk terms in LDS instead of registers, which avoids
    // a few register spills, measured 605-607 us.)
    float am = 0.0f;
    double ssc[kNF];
#pragma unroll
    for (int i = 0; i < kNF; ++i) ssc[i] = 0.0;
    const bool ok = receive<kNF, false>(a, slot(a, a.h, lg), tag_of(lg, 2), nullptr, 0u, K, K, Same{},
                                        [&](int c, const v4u &w, const v4u &) {
        const float2 hv = halves(w);
        const float2 g = *reinterpret_cast<const float2 *>(sm.gain + 2 * c);
        const float2 z = make_float2(__fmul_rn(hv.x, g.x), __fmul_rn(hv.y, g.y));
        *reinterpret_cast<float2 *>(sm.vals + 2 * c) = z;
        am = fmaxf(am, fmaxf(fabsf(z.x), fabsf(z.y)));
        ssc[(c - (int)threadIdx.x) >> 8] = (double)hv.x * hv.x + (double)hv.y * hv.y;
    });
    static_assert(kR == 256, "chunk slot = (c - thread) / kR");
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < kNF; ++i) ss += ssc[i];
    am = wave_max(am);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) {
        sm.red_a[threadIdx.x >> 6] = am;
        sm.red_s[threadIdx.x >> 6] = ss;
    }
    return ok;
}

// After the receivers: every thread quantises one 16-element group of the
// staged input into the transposed layout xs[t * (K / 64) + u] (group
// g = 4 u + t), so the lanes of a row, which read units u, u + 1, ..., read
// consecutive 16 bytes.  Returns false (x filled with NaN) if a receiver failed.
__device__ __forceinline__ bool quantise(const PArgs &a, Smem &sm, int K, float &am) {
    __syncthreads();
    if (sm.fail) {
        if (threadIdx.x == 0)
            __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = threadIdx.x; i < a.H; i += kT) a.x_out[i] = __builtin_nanf("");
        return false;
    }
    am = sm.red_a[0];
#pragma unroll
    for (int w = 1; w < kRecvWaves; ++w) am = fmaxf(am, sm.red_a[w]);
    const float sc = act_inv_scale(am);
    const int U = K / 64;
    // One code dword per thread and step (all waves take part): dword t of
    // group g holds elements 16 g + t + 4 j in byte j, the transposed order.
    uint32_t *xd = reinterpret_cast<uint32_t *>(sm.xs);
    for (int q = threadIdx.x; q < K / 4; q += kT) {
        const int g = q >> 2, t = q & 3;
        const float *src = sm.vals + 16 * g + t;
        xd[((g & 3) * U + (g >> 2)) * 4 + t] =
            (uint32_t)(act_code(src[0], sc) & 0xFF) |
            ((uint32_t)(act_code(src[4], sc) & 0xFF) << 8) |
            ((uint32_t)(act_code(src[8], sc) & 0xFF) << 16) |
            ((uint32_t)(act_code(src[12], sc) & 0xFF) << 24);
    }
    __syncthreads();
    return true;
}

// one 16-byte weight unit (64 weights) against activation groups 4u..4u+3,
// into four independent accumulators: from the packed unit, or (dot_unit)
// from its values unpacked ahead
__device__ __forceinline__ void dot_unit_packed(const uint4 &w, const uint4 *xs, int U, int u,
                                                int (&acc)[4]) {
    const uint32_t dws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t v0, v1, v2, v3;
        unpack16(dws[t], v0, v1, v2, v3);
        const uint4 xv = xs[t * U + u];
        acc[0] = dot4(v0, xv.x, acc[0]);
        acc[1] = dot4(v1, xv.y, acc[1]);
        acc[2] = dot4(v2, xv.z, acc[2]);
        acc[3] = dot4(v3, xv.w, acc[3]);
    }
}
__device__ __forceinline__ void dot_unit(const uint4 (&v)[4], const uint4 *xs, int U, int u,
                                         int (&acc)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint4 xv = xs[t * U + u];
        acc[0] = dot4(v[t].x, xv.x, acc[0]);
        acc[1] = dot4(v[t].y, xv.y, acc[1]);
        acc[2] = dot4(v[t].z, xv.z, acc[2]);
        acc[3] = dot4(v[t].w, xv.w, acc[3]);
    }
}

// Dot products of phase P with the loaded units, reduced over the lane group;
// returns true on the lane that holds the row group's sums.
template <int P>
__device__ __forceinline__ bool dot_phase(const PArgs &a, const Smem &sm, const Pre &pre, int ct,
                                          int nr, int &acc0, int &acc1) {
    const int K = phase_k(a, P);
    const int ls = a.lshift[P], ns = a.nslot[P];
    const int s = ct & ((1 << ls) - 1);
    const int rg = ct >> ls;
    const int U = K / 64;
    constexpr int half = P == 2 ? kS / 2 : kS;
    int c0[4] = {0, 0, 0, 0}, c1[4] = {0, 0, 0, 0};
    if (rg < nr) {
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const int u = s + (i << ls);
            if (i < ns && u < U) {
                if (i < kPU) dot_unit(pre.v[i < kPU ? i : 0], sm.xs, U, u, c0);
                else dot_unit_packed(pre.w[i], sm.xs, U, u, c0);
                if (P == 2) dot_unit_packed(pre.w[half + i], sm.xs, U, u, c1);
            }
        }
    }
    // Every weight load of this phase is complete here (lanes that skipped a
    // unit included): without this wait the compiler would wait for them
    // behind the output stores that follow, i.e. for those stores too.
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
    acc0 = (c0[0] + c0[1]) + (c0[2] + c0[3]);
    acc1 = (c1[0] + c1[1]) + (c1[2] + c1[3]);
    acc0 = group_sum(acc0, 1 << ls);
    if (P == 2) acc1 = group_sum(acc1, 1 << ls);
    return rg < nr && s == 0;
}

// Receiver waves: per phase, poll the input into LDS, then join the two
// workgroup barriers of quantise().
__device__ __forceinline__ void receiver_loop(const PArgs &a, Smem &sm) {
    const int H = a.H, KV = a.KV, F = a.F;
    float am;
    for (int l = 0; l < a.n_layers; ++l) {
        const int lg = a.l0 + l;
        float *tr = a.trace ? a.trace + (size_t)l * a.trace_stride : nullptr;
        if (!receive_p0(a, sm, lg, tr)) sm.fail = 1u;
        if (!quantise(a, sm, H, am)) return;
        if (!receive_p1(a, sm, lg)) sm.fail = 1u;
        if (!quantise(a, sm, H, am)) return;
        if (!receive_p2(a, sm, lg, tr ? tr + 3 * H + 2 * KV : nullptr)) sm.fail = 1u;
        if (!quantise(a, sm, H, am)) return;
        if (!receive_p3(a, sm, lg, a.layer[l].norm)) sm.fail = 1u;
        if (!quantise(a, sm, F, am)) return;
    }
    // the residual stream after the call's last layer: x = x_mid + y
    if (a.last && blockIdx.x == 0) {
        const int lg = a.l0 + a.n_layers - 1;
        const bool ok = receive<kNH, true>(a, slot(a, a.xm, lg), tag_of(lg, 2), slot(a, a.y, lg),
                                           tag_of(lg, 3), H, H,
                                           Same{}, [&](int c, const v4u &m, const v4u &y) {
            const float2 mm = halves(m), yy = halves(y);
            *reinterpret_cast<float2 *>(a.x_out + 2 * c) =
                make_float2(__fadd_rn(mm.x, yy.x), __fadd_rn(mm.y, yy.y));
        });
        if (!ok)
            for (int i = threadIdx.x; i < H; i += kR) a.x_out[i] = __builtin_nanf("");
    }
}

// Compute waves: per phase, join quantise(), then the dot products, the
// phase outputs and the next phase's weight loads.
__device__ __forceinline__ void compute_loop(const PArgs &a, Smem &sm) {
    const int H = a.H, KV = a.KV, F = a.F;
    const int ct = (int)threadIdx.x - kR;
    Pre pre;
    prefetch<0>(a, a.layer[0], ct, pre);
    for (int l = 0; l < a.n_layers; ++l) {
        const PLayer &L = a.layer[l];
        const int lg = a.l0 + l;
        float *tr = a.trace ? a.trace + (size_t)l * a.trace_stride : nullptr;
        int r0, nr, acc0, acc1;
        float am;

        // P0: q, k, v
        unpack_pre<0>(a, pre);
        if (!quantise(a, sm, H, am)) return;
        float d = act_scale(am);
        wg_rows(H + 2 * KV, r0, nr);
        if (dot_phase<0>(a, sm, pre, ct, nr, acc0, acc1)) {
            const int gr = r0 + (ct >> a.lshift[0]);
            const int seg = gr < H ? 0 : gr < H + KV ? 1 : 2;
            const float gm = seg == 0 ? pre.g0 : seg == 1 ? pre.g1 : pre.g2;
            const float y = rescale(acc0, __fmul_rn(gm, d));
            if (seg == 0) {
                a.q[gr] = y;
                if (tr) tr[H + gr] = y;
            } else if (seg == 1) {
                a.k[gr - H] = y;
                if (tr) tr[2 * H + gr - H] = y;
            } else {
                st_tag(slot(a, a.v, lg) + gr - H - KV, y, tag_of(lg, 0));
                if (tr) tr[2 * H + KV + gr - H - KV] = y;
            }
        }
        prefetch<1>(a, L, ct, pre);

        // P1: o
        unpack_pre<1>(a, pre);
        if (!quantise(a, sm, H, am)) return;
        d = act_scale(am);
        wg_rows(H, r0, nr);
        if (dot_phase<1>(a, sm, pre, ct, nr, acc0, acc1)) {
            const int gr = r0 + (ct >> a.lshift[1]);
            const float y = rescale(acc0, __fmul_rn(pre.g0, d));
            st_tag(slot(a, a.o, lg) + gr, y, tag_of(lg, 1));
            if (tr) tr[2 * H + 2 * KV + gr] = y;
        }
        prefetch<2>(a, L, ct, pre);

        // P2: gate/up pairs -> H
        unpack_pre<2>(a, pre);
        if (!quantise(a, sm, H, am)) return;
        d = act_scale(am);
        wg_rows(F, r0, nr);
        if (dot_phase<2>(a, sm, pre, ct, nr, acc0, acc1)) {
            const int gr = r0 + (ct >> a.lshift[2]);
            const float G = rescale(acc0, __fmul_rn(pre.g0, d));
            const float U = rescale(acc1, __fmul_rn(pre.g1, d));
            const float r = G > 0.0f ? G : 0.0f;
            st_tag(slot(a, a.h, lg) + gr, __fmul_rn(__fmul_rn(r, r), U), tag_of(lg, 2));
        }
        prefetch<3>(a, L, ct, pre);

        // P3: down -> y, with dz = (max|Z| / 127) / rms(H)
        unpack_pre<3>(a, pre);
        if (!quantise(a, sm, F, am)) return;
        double ss = sm.red_s[0];
#pragma unroll
        for (int w = 1; w < kRecvWaves; ++w) ss += sm.red_s[w];
        const float dh = act_scale(am);
        d = !(am > 0.0f) ? 0.0f : (float)((double)dh / sqrt(ss / (double)F + (double)a.eps));
        wg_rows(H, r0, nr);
        if (dot_phase<3>(a, sm, pre, ct, nr, acc0, acc1)) {
            const int gr = r0 + (ct >> a.lshift[3]);
            const float y = rescale(acc0, __fmul_rn(pre.g0, d));
            st_tag(slot(a, a.y, lg) + gr, y, tag_of(lg, 3));
            if (tr) tr[4 * H + 2 * KV + gr] = y;
        }
        if (l + 1 < a.n_layers) prefetch<0>(a, a.layer[l + 1], ct, pre);
    }
}

// The two roles run separate loops; each calls quantise() (two workgroup
// barriers) exactly once per phase, so every wave passes the same barriers.
__global__ __launch_bounds__(kT) void stack_persistent_kernel(const PArgs args) {
    // The arguments are read in place from the kernel-argument segment (a
    // reference to the by-value parameter would be copied to scratch).
    (void)args;
    const PArgs &a = *(const PArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    __shared__ Smem sm;
    if (threadIdx.x == 0) sm.fail = 0u;
    __syncthreads();
    if (threadIdx.x < kR)
        receiver_loop(a, sm);
    else
        compute_loop(a, sm);
}

// Clears every tag (and the error word) before a call.
__global__ __launch_bounds__(256) void stack_reset_kernel(uint2 *tagged, int n, unsigned *err) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
        tagged[i] = make_uint2(0u, 0u);
    if (blockIdx.x == 0 && threadIdx.x == 0) *err = 0u;
}

int grid_for_device() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus < kMaxGrid ? cus : kMaxGrid;
}

// lanes per row group for R row groups over G workgroups; false if a
// workgroup's rows do not fit one pass of the compute threads with <= slots
// units each
bool plan_phase(int G, int R, int K, bool pair, int &lshift, int &nslot) {
    const int rows = (R + G - 1) / G;
    if (rows > kC) return false;
    int ls = 6;
    while (ls > 0 && (kC >> ls) < rows) --ls;
    const int upr = K / 64;
    const int ns = (upr + (1 << ls) - 1) >> ls;
    lshift = ls;
    nslot = ns;
    return ns <= (pair ? kS / 2 : kS);
}

bool plan(int G, int H, int KV, int F, int D, int (&ls)[4], int (&ns)[4]) {
    if (G <= 0 || G > kMaxGrid || H > kMaxH || F > kMaxF || D % 2) return false;
    return plan_phase(G, H + 2 * KV, H, false, ls[0], ns[0]) &&
           plan_phase(G, H, H, false, ls[1], ns[1]) &&
           plan_phase(G, F, H, true, ls[2], ns[2]) &&
           plan_phase(G, H, F, false, ls[3], ns[3]);
}

}  // namespace

size_t stack_persistent_ws_floats(int H, int KV, int F) {
    // per layer slot tagged xa, xm, o, y [H], v [KV], h [F] (2 floats each),
    // then err
    return 2 * (size_t)kMaxLayers * (4 * (size_t)H + KV + F) + 64;
}

unsigned *stack_status_word(const StackWs &ws, int H, int KV, int F) {
    uint2 *t = reinterpret_cast<uint2 *>(ws.tagged);
    return reinterpret_cast<unsigned *>(t + (size_t)kMaxLayers * (4 * (size_t)H + KV + F));
}

hipError_t launch_stack_clear_status(unsigned *err, hipStream_t s) {
    hipLaunchKernelGGL(stack_reset_kernel, dim3(1), dim3(256), 0, s, (uint2 *)nullptr, 0, err);
    return hipGetLastError();
}

bool stack_persistent_fits(int H, int KV, int F, int D) {
    int ls[4], ns[4];
    return plan(grid_for_device(), H, KV, F, D, ls, ns);
}

hipError_t launch_decode_stack_persistent(const StackLayer *layers, int n_layers, int H, int KV,
                                          int F, int D, float eps, int wait_us, float *x,
                                          float *trace, const StackWs &ws, hipStream_t s) {
    const int G = grid_for_device();
    PArgs a = {};
    if (!plan(G, H, KV, F, D, a.lshift, a.nslot))
        return hipErrorInvalidValue;
    a.H = H; a.KV = KV; a.F = F; a.D = D; a.group = (H / D) / (KV / D); a.eps = eps;
    a.x_in = x; a.x_out = x;
    a.trace_stride = 5 * H + 2 * KV;
    a.q = ws.q; a.k = ws.k;
    uint2 *t = reinterpret_cast<uint2 *>(ws.tagged);
    a.xa = t; a.xm = t + H; a.o = t + 2 * H; a.y = t + 3 * H; a.v = t + 4 * H; a.h = t + 4 * H + KV;
    a.slot_stride = 4 * H + KV + F;
    const int n_tagged = kMaxLayers * a.slot_stride;
    a.err = stack_status_word(ws, H, KV, F);
    a.wait_ticks = (wait_us > 0 ? (uint64_t)wait_us : kDefaultWaitUs) * kTicksPerUs;
    hipLaunchKernelGGL(stack_reset_kernel, dim3(256), dim3(256), 0, s, t, n_tagged, a.err);
    for (int l0 = 0; l0 < n_layers; l0 += kMaxLayers) {
        const int n = n_layers - l0 < kMaxLayers ? n_layers - l0 : kMaxLayers;
        for (int i = 0; i < n; ++i) {
            const StackLayer &L = layers[l0 + i];
            PLayer &P = a.layer[i];
            P.W[0] = L.Wq; P.W[1] = L.Wk; P.W[2] = L.Wv; P.W[3] = L.Wo;
            P.W[4] = L.Wg; P.W[5] = L.Wu; P.W[6] = L.Wd;
            P.g[0] = L.gq; P.g[1] = L.gk; P.g[2] = L.gv; P.g[3] = L.go;
            P.g[4] = L.gg; P.g[5] = L.gu; P.g[6] = L.gd;
            P.norm = L.ffn_norm;
        }
        a.n_layers = n;
        a.l0 = l0;
        a.first = l0 == 0;
        a.last = l0 + n == n_layers;
        a.trace = trace ? trace + (size_t)l0 * a.trace_stride : nullptr;
        hipLaunchKernelGGL(stack_persistent_kernel, dim3(G), dim3(kT), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace bl
