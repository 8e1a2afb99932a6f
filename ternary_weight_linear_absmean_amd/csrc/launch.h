// launch.h -- internal kernel launchers of libbitlinear (not part of the ABI).
// Callers have validated every argument; launchers only enqueue work on the
// given stream and return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bitlinear.h"

namespace bl {

// Offline weight path: fp64 sums of |W| over blocks of 2048 row-major terms
// into `bsum` [quant_weight_blocks(N, K)], gamma, packing.
int64_t quant_weight_blocks(int64_t N, int64_t K);
hipError_t launch_quant_weight(const float *W, int64_t N, int64_t K, uint8_t *Wp,
                               float *gamma, double *bsum, hipStream_t s);
// The allocation-free variant's block sums live in a library-owned device
// array of kNoAllocQuantMaxBlocks doubles (512 KiB: N*K <= 2^27 weights);
// noalloc_quant_scratch gives the current device's address of it.
constexpr int64_t kNoAllocQuantMaxBlocks = 65536;
hipError_t noalloc_quant_scratch(double **out);

// Per-token absmax int8 quantisation; dtype 0 = fp32, 1 = bf16.
hipError_t launch_quant_act(const void *X, int dtype, int64_t M, int64_t K,
                            int8_t *Xq, float *d, hipStream_t s);
// Per-token absmax to 4-bit codes, two per byte [M][K/2]; K even.
hipError_t launch_quant_act4(const void *X, int dtype, int64_t M, int64_t K,
                             uint8_t *Xq4, float *d, hipStream_t s);
// Y = float(acc) * fl(gamma * d[m]) with the activations given as 4-bit codes
// [M][K/2] (any M, K % 64 == 0): the product kernels with their activation
// staging reading nibbles.
hipError_t launch_bitlinear_a4(const uint8_t *Xq4, const float *d, int M, const uint8_t *Wp,
                               const float *gamma, int N, int K, float *Y, int32_t *acc,
                               hipStream_t s);

// Y = float(acc) * fl(gamma * d[m]), acc = Xq . unpack(Wp)^T.  VALU kernel
// (v_dot4) for a handful of tokens.
hipError_t launch_gemv(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                       const float *gamma, int N, int K, float *Y, int32_t *acc,
                       hipStream_t s);

// The same for 4-bit activation codes ([M][K/2]), 1 <= M <= 8.
hipError_t launch_gemv_a4(const uint8_t *Xq4, const float *d, int M, const uint8_t *Wp,
                          const float *gamma, int N, int K, float *Y, int32_t *acc,
                          hipStream_t s);

// Same product on int8 MFMA tiles, any M.
hipError_t launch_gemm(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                       const float *gamma, int N, int K, float *Y, int32_t *acc,
                       hipStream_t s);

// Few-token product on int8 MFMA that reads every packed weight once
// (gemm_skinny.hip): 1 <= M < 128, 64 <= K <= 8192, K % 64 == 0.
bool gemm_skinny_fits(int M, int K);
hipError_t launch_gemm_skinny(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                              const float *gamma, int N, int K, float *Y, int32_t *acc,
                              hipStream_t s);

// Largest M the VALU kernel takes in one pass over the weights.
constexpr int kGemvMaxTokens = 8;

// One job of the fused decode kernel (validated by the caller).
struct GemvJob {
    const void *X;
    const uint8_t *Wp;
    const float *gamma;
    float *Y;
    int8_t *Xq;
    float *d;
    int N, K, dtype;
};
constexpr int kGemvMaxJobs = 8;

// Tokens per fused-kernel tile for M tokens, and its LDS bytes: the int8
// codes (tile x K) plus the raw activations (tile x K x element size).
constexpr int fused_tile(int M) { return M == 1 ? 1 : M == 2 ? 2 : M <= 4 ? 4 : 8; }
constexpr size_t fused_lds_bytes(int tile, int K, int esize) {
    return (size_t)tile * K * (1 + esize);
}
constexpr size_t kFusedMaxLds = 128 * 1024;

// Per-token int8 quantisation of each job's X fused into its GEMV; all jobs
// in one launch.  M <= 8, count <= kGemvMaxJobs,
// fused_lds_bytes(fused_tile(M), K, esize) <= kFusedMaxLds for every job.
hipError_t launch_gemv_fused(const GemvJob *jobs, int count, int M, hipStream_t s);

// FFN block, M >= 128 with a gate: both first BitLinears in one MFMA kernel
// (gemm.hip) whose epilogue writes Z = fl(fl(relu(G)^2 * U) * g) [M][F] and,
// per row and 128-column tile, max |Z| and the fp64 sum of H^2 ([M][tiles]);
// then the tail (ffn.hip) reduces the partials and writes the int8 codes.
constexpr int ffn_gate_up_tiles(int F) { return (F + 127) / 128; }
hipError_t launch_ffn_gate_up(const int8_t *Xq, const float *d, int M, int K, const uint8_t *Wg,
                              const float *gamma_g, const uint8_t *Wu, const float *gamma_u,
                              const float *norm_w, int F, float *Z, float *pmax, double *psum,
                              hipStream_t s);
hipError_t launch_ffn_tail_z(const float *Z, const float *pmax, const double *psum, int tiles,
                             float eps, int M, int F, int8_t *Hq, float *dh, float *dz,
                             hipStream_t s);

// QAT backward (backward.hip): dX = gamma (dY . Wq) and dW = (dY o d)^T . Xq
// on bf16 MFMA; the workspace holds the transposed operands.
size_t backward_input_ws_bytes(int64_t M, int64_t N, int64_t K);
size_t backward_weight_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_backward_input(const float *dY, int M, int N, const uint8_t *Wp, const float *gamma,
                                 int K, float *dX, void *ws, hipStream_t s);
hipError_t launch_backward_weight(const float *dY, int M, int N, const int8_t *Xq, const float *d,
                                  int K, float *dW, void *ws, hipStream_t s);

// Five ternary weights per byte (t5.hip): bytes per row (a multiple of 16),
// the token tile of the product, and its LDS bytes (the staged codes of a
// tile: 80 bytes per 16-byte weight unit and token).
constexpr int64_t t5_row_bytes(int64_t K) { return ((K + 4) / 5 + 15) / 16 * 16; }
constexpr int kT5MaxTokens = 8;
constexpr int t5_tile(int M) { return M == 1 ? 1 : M == 2 ? 2 : M <= 4 ? 4 : 8; }
constexpr size_t t5_lds_bytes(int M, int64_t K) {
    return (size_t)t5_tile(M) * (size_t)(t5_row_bytes(K) / 16) * 80;
}
constexpr size_t kT5MaxLds = 64 * 1024;
// Wp [N][K/4] (2-bit codes) -> Wt5 [N][t5_row_bytes(K)]; K % 4 == 0.
hipError_t launch_repack_t5(const uint8_t *Wp, int N, int K, uint8_t *Wt5, hipStream_t s);
// Y = float(acc) * fl(gamma * d[m]) from the five-per-byte rows; 1 <= M <= 8,
// K % 4 == 0, K > 0, t5_lds_bytes(M, K) <= kT5MaxLds.
hipError_t launch_gemv_t5(const int8_t *Xq, const float *d, int M, const uint8_t *Wt5,
                          const float *gamma, int N, int K, float *Y, int32_t *acc, hipStream_t s);

// Picks the VALU kernel for M <= kGemvMaxTokens and MFMA otherwise.
hipError_t launch_bitlinear(const int8_t *Xq, const float *d, int M, const uint8_t *Wp,
                            const float *gamma, int N, int K, float *Y, int32_t *acc,
                            hipStream_t s);

// One layer's weights for the decode stack (device pointers): the ABI's
// bl_layer itself.
using StackLayer = bl_layer;

// Workspace of launch_decode_stack, carved from the caller's buffer: every
// region starts on a 64-float boundary.  The per-step path uses q..Hq, the
// persistent path q, k and the tagged region.
struct StackWs {
    float *q, *a, *o, *y, *k, *v, *G, *U, *dh, *dz;
    int8_t *Hq;
    float *tagged;
};
size_t stack_ws_floats(int H, int KV, int F);
StackWs stack_ws(float *ws, int H, int KV, int F);

// Decode-stack paths (bl_stack_dims.path).
enum StackPath { kStackAuto = 0, kStackLaunches = 1, kStackPersistent = 2 };

// One token (M = 1) through n_layers layers; x [H] fp32 is updated in place.
// trace: NULL or [n_layers][5 H + 2 KV] = x_in, q, k, v, o, x_mid, y.
hipError_t launch_decode_stack(const StackLayer *layers, int n_layers, int H, int KV, int F,
                               int D, float eps, int wait_us, float *x, float *trace, float *ws,
                               int path, hipStream_t s);

// The persistent path: one launch per 16 layers, one workgroup per compute
// unit of the current device.  fits() says whether these sizes fit its
// per-workgroup limits on the current device.
size_t stack_persistent_ws_floats(int H, int KV, int F);
bool stack_persistent_fits(int H, int KV, int F, int D);
hipError_t launch_decode_stack_persistent(const StackLayer *layers, int n_layers, int H, int KV,
                                          int F, int D, float eps, int wait_us, float *x,
                                          float *trace, const StackWs &ws, hipStream_t s);
// The call's status word in the workspace (0: every wait ended in time), and
// a launch that clears it.
unsigned *stack_status_word(const StackWs &ws, int H, int KV, int F);
hipError_t launch_stack_clear_status(unsigned *err, hipStream_t s);

// FFN tail on fp32 G, U [M][F]: H = relu(G)^2 * U, Hq / dh = absmax int8 of
// H * g, dz = dh / rms(H).  U == NULL: ungated; norm_w == NULL: unit gain.
hipError_t launch_ffn_tail(const float *G, const float *U, const float *norm_w,
                           float eps, int M, int F, int8_t *Hq, float *dh, float *dz,
                           hipStream_t s);

}  // namespace bl
