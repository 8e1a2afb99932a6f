/*
 * bitlinear.h -- C ABI of libbitlinear, the BitLinear W1.58A8 layer of
 * BitNet b1.58 on AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (nn.Linear convention, no bias):
 *     X [M][K] activations, W [N][K] weights, Y [M][N] = X W^T.
 * W is quantised by absmean to ternary codes with one scale gamma per tensor,
 * X is quantised per token (row) by absmax to int8 with one scale d[m], the
 * product is an exact int32 sum and Y = acc * gamma * d[m].
 *
 * Passages defining the operations (pages by title, section):
 *   [RPT]  "Microsoft BitNet 深度研究报告", §2 技术原理:
 *          (1) 三元量化 -- weights take the values {-1, 0, +1};
 *          (2) AbsMean 量化 -- Q(w) = round(clamp(w / gamma, -1, 1)),
 *              gamma = (1/n) sum |w_i|; 实际存储 -- 2-bit codes
 *              {0: 0, +1: 1, -1: 2};
 *          (3) 查找表优化 -- W = +1: C += A, W = -1: C -= A, W = 0: skip.
 *   [CARD] "BitNet b1.58 2B4T - 原生1比特大语言模型规模化实践", 模型详情 --
 *          W1.58A8; absmean ternary weights; per-token absmax int8
 *          activations; ReLU² FFN; subln; no bias in linear or norm layers.
 *   [NEWS] iaiol.com BitNet b1.58 2B4T article, "权重映射为三元值{-1, 0, +1}"
 *          -- per-token absmax 8-bit activations, subln, ReLU² instead of
 *          SwiGLU; "微软在1 bit LLM上的探索" -- BitLinear replaces nn.Linear,
 *          W1.58A8 needs its own matmul kernel.
 *   [TR]   copy of the "BitNet b1.58 2B4T Technical Report", 推理完满 /
 *          GPU端 -- four ternary weights packed into one int8; pack, store,
 *          load, unpack, compute.
 *
 * Data formats (readings of what the pages leave open):
 *   packed weights Wp: uint8 [N][K/4], row-major.  Byte b of row n holds the
 *     weights k = 4b..4b+3; weight 4b+j sits in bits 2j..2j+1; code 0 = 0,
 *     1 = +1, 2 = -1 (code 3 is never written and reads as 0).
 *   gamma: one fp32 per weight tensor, = fp32(S / (N*K)) with S = sum |W|
 *     in fp64 over the N*K weights in row-major order, by pairwise summation:
 *     neighbouring terms are added in pairs, then neighbouring pair sums, and
 *     so on until one sum is left (a sum with no right neighbour at its level
 *     is carried up unchanged); the division is in fp64, rounded once.
 *     Wq = sign(w) where 2|w| > gamma, else 0 (round half to even).
 *   Xq: int8 [M][K] row-major, d: fp32 [M].  Per row: a = max|x|,
 *     s = fp32(127 / a), Xq = clamp(rne(fp32(x * s)), -127, 127),
 *     d = fp32(a / 127); an all-zero row gives Xq = 0, d = 0.
 *   acc: int32 [M][N], exact (|acc| <= 127 K < 2^31).
 *   Y: fp32 [M][N], Y = fp32(float(acc) * fp32(gamma * d[m])).
 *
 * Calling conventions, for every call below:
 *   - Every tensor pointer is a DEVICE pointer (hipMalloc / torch CUDA
 *     memory) on the current HIP device; the caller owns all memory and the
 *     stream.  The library keeps no pointer after it returns and never
 *     allocates or frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it; no call synchronises the host.
 *   - Validation runs on the host before anything is enqueued.  On a non-OK
 *     return nothing was launched and no output was written;
 *     bl_last_error() then gives a readable reason (per thread).
 *   - Tensor pointers must be 16-byte aligned (BL_ERR_ALIGN), except d,
 *     gamma and the fp32 vectors, which need 4-byte alignment.
 *   - Device faults inside a kernel surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - Inputs with NaN or Inf give unspecified (but memory-safe) results.
 *   - The current device must be gfx950 (BL_ERR_ARCH).
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BL_ABI_VERSION 2

typedef enum {
    BL_OK = 0,
    BL_ERR_NULL = 1,      /* a required pointer is NULL */
    BL_ERR_SHAPE = 2,     /* a size is negative, too large, or not a required multiple */
    BL_ERR_DTYPE = 3,     /* unknown bl_dtype */
    BL_ERR_ALIGN = 4,     /* a pointer is not aligned as required */
    BL_ERR_WORKSPACE = 5, /* ws is NULL or ws_bytes < bl_workspace_bytes(...) */
    BL_ERR_ARCH = 6,      /* the current HIP device is not gfx950 */
    BL_ERR_HIP = 7        /* a HIP runtime call or a kernel launch failed */
} bl_status;

typedef enum {
    BL_F32 = 0,           /* IEEE binary32 */
    BL_BF16 = 1           /* bfloat16 (upper half of binary32) */
} bl_dtype;

typedef enum {
    BL_OP_QUANT_WEIGHT = 0,   /* quant_weight_absmean_pack */
    BL_OP_FFN_RELU2 = 1,      /* bitlinear_ffn_relu2 */
    BL_OP_DECODE_STACK = 2,   /* bitlinear_decode_stack: N = H, K = KV, F = F */
    BL_OP_BACKWARD_INPUT = 3, /* bitlinear_backward_input */
    BL_OP_BACKWARD_WEIGHT = 4 /* bitlinear_backward_weight */
} bl_op;

/* Largest K (and F) any call accepts: keeps |acc| <= 127 K exact in int32
 * and float(acc) exact in fp32 (127 K <= 2^24). */
#define BL_MAX_K 131072

/* ------------------------------------------------------------------------
 * quant_weight_absmean_pack -- offline weight path.
 * [RPT] §2 (2) AbsMean 量化 (gamma, Q(w)) and 实际存储 (codes);
 * [TR] GPU端 (four weights per int8).
 *
 *   W      in   fp32 [N][K], row-major (the nn.Linear weight, out x in).
 *   N, K        N >= 0, K >= 0, K % 4 == 0, K <= BL_MAX_K.
 *   Wp     out  uint8 [N][K/4], the packed codes (format above).
 *   gamma  out  fp32 [1]; N*K == 0 gives gamma = 0 and writes no Wp byte.
 *   ws          device workspace of >= bl_workspace_bytes(BL_OP_QUANT_WEIGHT,
 *               0, N, K, 0) bytes (one fp64 sum per block of 2048 row-major
 *               weights), 16-byte aligned.
 *   N*K <= 2^40 (BL_ERR_SHAPE otherwise).
 * gamma is reproducible to the bit (the fixed pairwise order above).
 */
bl_status quant_weight_absmean_pack(const float *W, int64_t N, int64_t K,
                                    uint8_t *Wp, float *gamma,
                                    void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * quant_weight_absmean_pack_noalloc -- for callers that cannot allocate:
 * code under HIP graph capture, and serving or training loops (which
 * re-quantise the latent weights every step) that forbid allocation.
 * Same arguments (without ws), formats, bits and errors as
 * quant_weight_absmean_pack, whose kernels it runs; its fp64 block sums go to
 * a device array the library owns (512 KiB on each GPU it runs on, held until
 * the process ends) instead of a caller workspace.  Allocates nothing.
 *   N*K <= BL_NOALLOC_MAX_WEIGHTS (2^27), else BL_ERR_SHAPE.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (e.g. on two streams) race and must be serialised by the caller.  Each
 * call writes every block sum it reads before reading it.
 */
#define BL_NOALLOC_MAX_WEIGHTS (1LL << 27)

bl_status quant_weight_absmean_pack_noalloc(const float *W, int64_t N, int64_t K,
                                            uint8_t *Wp, float *gamma, void *stream);

/* ------------------------------------------------------------------------
 * quant_act_absmax_i8 -- per-token absmax int8 activation quantisation.
 * [NEWS] 权重映射为三元值; [CARD] 模型详情 (per-token absmax, 8-bit).
 *
 *   X      in   [M][K] row-major, element type `dtype` (BL_F32 or BL_BF16).
 *   M, K        M >= 0, K >= 0, K <= BL_MAX_K.
 *   Xq     out  int8 [M][K].
 *   d      out  fp32 [M], the per-token scale a / 127 (0 for a zero row).
 * Bit-exact with the formula in the header comment.
 */
bl_status quant_act_absmax_i8(const void *X, bl_dtype dtype, int64_t M, int64_t K,
                              int8_t *Xq, float *d, void *stream);

/* ------------------------------------------------------------------------
 * 4-bit activations (BitNet a4.8): "Microsoft BitNet 深度研究报告",
 * §3 论文演进时间线 (row 2024-11: activations at 4 bits, a further
 * compression) and §10 关键资源 (BitNet a4.8, activation quantisation).
 * The pages name the scheme only.  Readings: the per-token absmax rule above
 * with the signed 4-bit range,
 *     s = fp32(7 / a),  q = clamp(rne(fp32(x * s)), -7, 7),  d = fp32(a / 7),
 * an all-zero row giving q = 0, d = 0 (-8 is never produced); storage Xq4:
 * uint8 [M][K/2] row-major, byte b holding element 2b in bits 0..3 and
 * element 2b+1 in bits 4..7, each a 4-bit two's-complement number; the
 * product and rescale are those of the 8-bit codes:
 *     acc = sum_k q[m][k] * Wq[n][k] (exact int32),  Y = fp32(float(acc) * fp32(gamma * d[m])).
 *
 * quant_act_absmax_i4 -- X [M][K] fp32 or bf16 (16-byte aligned), K even,
 *   K <= BL_MAX_K -> Xq4 [M][K/2] (16-byte aligned) and d [M].  Bit-exact.
 */
bl_status quant_act_absmax_i4(const void *X, bl_dtype dtype, int64_t M, int64_t K,
                              uint8_t *Xq4, float *d, void *stream);

/* bitlinear_a4 -- the W1.58A4 product for any M >= 0: arguments, formats and
 * errors as bitlinear_gemm, with Xq4 [M][K/2] (16-byte aligned) in place of
 * Xq; K % 64 == 0.  The 4-bit codes are unpacked into the same int8 product
 * kernels (the decode kernel for M <= 8, the int8 MFMA tiles above), so acc
 * and Y are bit-exact. */
bl_status bitlinear_a4(const uint8_t *Xq4, const float *d, int64_t M,
                       const uint8_t *Wp, const float *gamma, int64_t N, int64_t K,
                       float *Y, int32_t *acc, void *stream);

/* ------------------------------------------------------------------------
 * bitlinear_gemv -- decode-sized W1.58A8 product, M = 1..64 tokens.
 * [RPT] §2 (3) 查找表优化 (add / subtract / skip); [TR] GPU端 (load the
 * packed weights, unpack, compute); [CARD] 模型详情 (W1.58A8).
 *
 *   Xq     in   int8 [M][K];  d  in  fp32 [M]  (from quant_act_absmax_i8).
 *   M           1 <= M <= 64 (M == 0 is a no-op returning BL_OK).
 *   Wp     in   uint8 [N][K/4];  gamma  in  fp32 [1]  (device).
 *   N, K        N >= 0; K % 64 == 0; K <= BL_MAX_K.
 *   Y      out  fp32 [M][N] = float(acc) * fp32(gamma * d[m]).
 *   acc    out  int32 [M][N], optional (NULL = not written): the exact
 *               accumulator sum_k Xq[m][k] * Wq[n][k].
 * Streams the packed weights once per launch; acc and Y are bit-exact.
 */
bl_status bitlinear_gemv(const int8_t *Xq, const float *d, int64_t M,
                         const uint8_t *Wp, const float *gamma, int64_t N, int64_t K,
                         float *Y, int32_t *acc, void *stream);

/* ------------------------------------------------------------------------
 * bitlinear_gemm -- prefill-sized W1.58A8 product, any M >= 0, on int8
 * matrix cores: the packed tiles are unpacked to int8 and multiplied with
 * int32 accumulation, with the rescale fused into the epilogue.
 * Same arguments, formats and results as bitlinear_gemv, except that M has
 * no upper bound (M <= 2^31 - 1).
 */
bl_status bitlinear_gemm(const int8_t *Xq, const float *d, int64_t M,
                         const uint8_t *Wp, const float *gamma, int64_t N, int64_t K,
                         float *Y, int32_t *acc, void *stream);

/* ------------------------------------------------------------------------
 * bitlinear_gemv_fused -- decode step: per-token absmax int8 quantisation
 * folded into the GEMV, for up to BL_MAX_JOBS independent BitLinears in one
 * launch.  Each job is Y = BitLinear(X) with its own activations, weights
 * and output, exactly as quant_act_absmax_i8 followed by bitlinear_gemv
 * (same int8 codes, scales, int32 sums and fp32 Y, bit for bit); the
 * quantisation is recomputed by every workgroup from X, so no intermediate
 * round trip through memory or second launch is needed.
 * [NEWS] 权重映射为三元值 (per-token absmax int8); [RPT] §2 (3) 查找表优化;
 * [TR] GPU端 (load packed weights, unpack, compute).
 *
 *   jobs   in   HOST array of `count` bl_gemv_job (read before return; the
 *               pointers inside are device pointers).
 *   count       1 <= count <= BL_MAX_JOBS.
 *   M           tokens, 1 <= M <= 8, shared by all jobs.
 * Per job: X is [M][K] of `dtype` (BL_F32 / BL_BF16, 16-byte aligned),
 * K % 64 == 0, 0 < K <= 16384, N >= 0, and T * K * (1 + element size) <=
 * 131072 bytes of LDS staging, T = M rounded up to 1, 2, 4 or 8 (e.g. M = 1:
 * K <= 16384; M = 8 bf16: K <= 5461); Wp [N][K/4] and gamma as for
 * bitlinear_gemv; Y [M][N] fp32; Xq [M][K] int8 and d [M] fp32 are optional
 * outputs (NULL = not written) holding the quantised activations.  Jobs
 * may share X; no output may overlap another job's input or output.
 */
#define BL_MAX_JOBS 8

typedef struct {
    const void *X;
    const uint8_t *Wp;
    const float *gamma;
    float *Y;
    int8_t *Xq;
    float *d;
    int64_t N;
    int64_t K;
    int32_t dtype;
    int32_t reserved;     /* must be 0 */
} bl_gemv_job;

bl_status bitlinear_gemv_fused(const bl_gemv_job *jobs, int count, int64_t M, void *stream);

/* ------------------------------------------------------------------------
 * bitlinear_ffn_relu2 -- the feed-forward tail of a BitNet b1.58 block:
 * ReLU² (gated) + subln RMSNorm + int8 requantisation + down projection.
 * [NEWS] 权重映射为三元值 (ReLU² in place of SwiGLU; subln);
 * [CARD] 模型详情 (ReLU², subln, no biases, W1.58A8 in every BitLinear).
 *
 * Readings (the pages print no formula for ReLU² gating or subln):
 *   G = Xq Wg^T and U = Xq Wu^T as W1.58A8 BitLinears (fp32, as Y above);
 *   H = fp32(fp32(r * r) * U) with r = max(G, 0)   (Wu == NULL: H = r * r);
 *   subln: Z = H / rms * g, rms = sqrt(sum_f H^2 / F + eps), g = norm_w
 *          (NULL = ones);
 *   Z is requantised per token (absmax int8) and Y = Zq Wd^T (W1.58A8).
 * Absmax codes do not change when a row is scaled by 1/rms > 0, so the int8
 * codes Hq are taken from fp32(H * g) and Z's scale is dh / rms, where dh is
 * the absmax scale of H * g.  Hq and dh are bit-exact; Y carries the rms sum,
 * whose summation order is the library's (fp32 relative error ~1e-6).
 *
 *   Xq, d       in   int8 [M][K], fp32 [M] (the block input, quantised).
 *   M, K, F, N       M >= 0; K % 64 == 0; F % 64 == 0; N >= 0; K, F <= BL_MAX_K.
 *   Wg, gamma_g in   uint8 [F][K/4], fp32 [1].
 *   Wu, gamma_u in   uint8 [F][K/4], fp32 [1]; Wu == NULL: ungated
 *                    (gamma_u ignored).
 *   norm_w      in   fp32 [F] or NULL.
 *   eps              RMSNorm epsilon (>= 0), e.g. 1e-5.
 *   Wd, gamma_d in   uint8 [N][F/4], fp32 [1].
 *   Y           out  fp32 [M][N].
 *   Hq          out  int8 [M][F], optional (NULL = not written).
 *   dh          out  fp32 [M], optional (NULL = not written).
 *   ws               >= bl_workspace_bytes(BL_OP_FFN_RELU2, M, N, K, F)
 *                    bytes of device memory, 16-byte aligned.
 */
bl_status bitlinear_ffn_relu2(const int8_t *Xq, const float *d,
                              int64_t M, int64_t K, int64_t F,
                              const uint8_t *Wg, const float *gamma_g,
                              const uint8_t *Wu, const float *gamma_u,
                              const float *norm_w, float eps,
                              const uint8_t *Wd, const float *gamma_d, int64_t N,
                              float *Y, int8_t *Hq, float *dh,
                              void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * bitlinear_decode_stack -- one decode token (M = 1) through a stack of
 * BitNet b1.58 layers, every projection a W1.58A8 BitLinear.
 * [CARD] 模型详情 (BitLinear without bias, W1.58A8, ReLU², subln);
 * [NEWS] 权重映射为三元值 (ReLU² FFN, subln, per-token absmax activations).
 *
 * Per layer (the parts that are not BitLinears are one-token stand-ins):
 *   q, k, v = BitLinear_q,k,v(x)        x: the fp32 residual stream [H]
 *   a[h D + i] = v[(h / g) D + i]       attention over one key returns v;
 *                                       g = (H / D) / (KV / D) query heads
 *                                       share a key/value head
 *   o = BitLinear_o(a);  x = x + o      (fp32 add)
 *   y = bitlinear_ffn_relu2(x) (gated, subln gain ffn_norm, eps);  x = x + y
 * Every BitLinear quantises its input per token as quant_act_absmax_i8.
 *
 *   layers   in   HOST array of n_layers bl_layer (device pointers inside):
 *                 Wq [H][H/4], Wk, Wv [KV][H/4], Wo [H][H/4], Wg, Wu
 *                 [F][H/4], Wd [H][F/4], their gammas, ffn_norm [F] or NULL.
 *   dims          H, KV, F multiples of 64 (<= 16384), D divides H and KV,
 *                 (KV / D) divides (H / D); eps >= 0; path (below).
 *   x        in/out  fp32 [H], updated in place.
 *   trace    out  NULL or fp32 [n_layers][5 H + 2 KV]: per layer x_in, q, k,
 *                 v, o, x_mid (= x_in + o), y (the FFN output).
 *   ws            >= bl_workspace_bytes(BL_OP_DECODE_STACK, 1, H, KV, F)
 *                 bytes, 16-byte aligned.
 */
typedef struct {
    const uint8_t *Wq, *Wk, *Wv, *Wo, *Wg, *Wu, *Wd;
    const float *gq, *gk, *gv, *go, *gg, *gu, *gd;
    const float *ffn_norm;
} bl_layer;

typedef struct {
    int64_t H, KV, F, D;
    float eps;
    int32_t path;         /* BL_STACK_AUTO, BL_STACK_LAUNCHES or BL_STACK_PERSISTENT */
    int32_t wait_us;      /* limit of each wait of the persistent path in microseconds;
                             0 = 1 s (the default); must be >= 0 */
    int32_t reserved;     /* must be 0 */
} bl_stack_dims;

/* How bitlinear_decode_stack runs (same results either way):
 *   BL_STACK_LAUNCHES    one launch per step (fused q/k/v, head expansion,
 *                        fused o, residual, fused gate/up, FFN tail, down,
 *                        residual): 8 launches per layer.
 *   BL_STACK_PERSISTENT  one launch per 16 layers with one workgroup per
 *                        compute unit; the steps are separated by grid-wide
 *                        barriers and each step's weights are fetched while
 *                        the previous barrier resolves.  BL_ERR_SHAPE if the
 *                        sizes exceed its per-workgroup limits on the device
 *                        (2B-class sizes fit).  If the grid is not resident
 *                        as a whole (the device shared with other work), a
 *                        wait gives up after dims->wait_us (1 s by default):
 *                        x is then filled with NaN and the call's status
 *                        word (bitlinear_decode_stack_status) is set.
 *   BL_STACK_AUTO        persistent where it fits, else launches. */
enum { BL_STACK_AUTO = 0, BL_STACK_LAUNCHES = 1, BL_STACK_PERSISTENT = 2 };

bl_status bitlinear_decode_stack(const bl_layer *layers, int n_layers, const bl_stack_dims *dims,
                                 float *x, float *trace, void *ws, size_t ws_bytes,
                                 void *stream);

/* bitlinear_decode_stack_status -- whether the last bitlinear_decode_stack
 * call with n_layers > 0 on this workspace finished every wait in time.
 *   ws, ws_bytes, dims   the workspace and the dims of that call.
 *   status  out  HOST int32: 0 = the call ran to the end (x is valid);
 *                1 = a wait of the persistent path gave up (x holds NaN).
 * Reads 4 bytes of the workspace with a blocking device-to-host copy: call it
 * only once the stack call's work has finished (e.g. after synchronising its
 * stream).  Allocates nothing; errors as for bitlinear_decode_stack, plus
 * BL_ERR_NULL for a NULL status and BL_ERR_HIP if the copy fails. */
bl_status bitlinear_decode_stack_status(const void *ws, size_t ws_bytes,
                                        const bl_stack_dims *dims, int32_t *status);

/* ------------------------------------------------------------------------
 * Five ternary weights per byte -- the denser storage the 1.58-bit figure
 * points to: [NEWS] "权重映射为三元值" (log2 3 = 1.58 bits per weight), the
 * 0.4 GB model of the aigc.izzi.cn news page "微软发布新型语言模型 BitNet
 * b1.58 2B4T，占用内存仅0.4GB", against the 2-bit codes of [RPT] 实际存储 and
 * the int2 I2_S kernel of [RPT] 内核类型.  3^5 = 243 <= 256: 1.6 bits per
 * weight, 20% fewer bytes than Wp.
 *
 * Format Wt5 (the pages give none): uint8 [N][bitlinear_t5_row_bytes(K)],
 * row-major.  Byte b of row n holds weights k = 5b .. 5b+4 as the base-3
 * digits d = w + 1 of v = sum_j d_j 3^(4-j) (weight 5b most significant),
 * stored as q = ceil(256 v / 243); v = floor(243 q / 256) recovers v.
 * Weights past K read as 0 (digit 1); rows are padded with such bytes to a
 * multiple of 16 bytes.
 */

/* Bytes per Wt5 row: ceil(K / 5) rounded up to a multiple of 16; 0 when K is
 * negative or above BL_MAX_K. */
size_t bitlinear_t5_row_bytes(int64_t K);

/* bitlinear_repack_t5 -- Wp (2-bit codes) -> Wt5, the same ternary weights.
 *   Wp     in   uint8 [N][K/4], 16-byte aligned.
 *   N, K        N >= 0, K >= 0, K % 4 == 0, K <= BL_MAX_K (N*K == 0: no-op).
 *   Wt5    out  uint8 [N][bitlinear_t5_row_bytes(K)], 16-byte aligned.
 * Bit-exact (integer arithmetic only).
 */
bl_status bitlinear_repack_t5(const uint8_t *Wp, int64_t N, int64_t K, uint8_t *Wt5,
                              void *stream);

/* bitlinear_gemv_t5 -- bitlinear_gemv on Wt5 rows, M = 1..8 tokens.
 *   Xq, d, gamma, Y, acc   as bitlinear_gemv (acc optional; Y and acc
 *                          bit-identical to bitlinear_gemv on the same
 *                          ternary weights).
 *   Wt5    in   uint8 [N][bitlinear_t5_row_bytes(K)], 16-byte aligned.
 *   M           0 <= M <= 8 (M == 0 or N == 0: no-op).
 *   K           K > 0, K % 4 == 0, K <= BL_MAX_K, and the staged codes of a
 *               token tile (1, 2, 4 or 8 tokens for M = 1, 2, 3..4, 5..8) at
 *               80 bytes per 16 Wt5 bytes of a row must fit 64 KiB
 *               (BL_ERR_SHAPE otherwise; e.g. M = 1 takes K <= 65520).
 */
bl_status bitlinear_gemv_t5(const int8_t *Xq, const float *d, int64_t M, const uint8_t *Wt5,
                            const float *gamma, int64_t N, int64_t K, float *Y, int32_t *acc,
                            void *stream);

/* ------------------------------------------------------------------------
 * bitlinear_backward_input / bitlinear_backward_weight -- the backward pass
 * of quantisation-aware training through one BitLinear.
 * [RPT] §2 (4) 量化感知训练: the forward uses the quantised weights, the
 * backward goes through the quantisers with the straight-through estimator,
 * and the optimiser updates the latent weights.  With the forward operands
 * X~ = Xq d (per token) and W~ = gamma Wq, the straight-through gradients of
 * the latent X and W are
 *     dX = dY . W~  = gamma (dY . Wq)          fp32 [M][K]
 *     dW = dY^T . X~ = (dY o d)^T . Xq         fp32 [N][K]
 * The integer operands are exact in bf16; each fp32 gradient value is split
 * into two bf16 halves (hi + lo, to about 2^-17 of the value) and both run on
 * bf16 MFMA with fp32 accumulation.  Each result element is within
 * 1e-3 * sum_c |term_c| of the exact sum (the terms being the products it
 * adds).  Gradients must be finite and below 2^127 in magnitude.  When the
 * last round of 128 x 256 output tiles would leave most of the GPU idle,
 * those tiles' contraction is split into up to 8 ranges whose fp32 partial
 * sums are added in a fixed order: results are deterministic for given
 * sizes.  Calls that share a workspace must not run concurrently.
 * An empty sum (N == 0 for dX, M == 0 for dW) writes zeros and reads no
 * operand (those pointers may then be NULL); an empty output is a no-op.
 * Both are asynchronous on `stream`; errors as for bitlinear_gemm.
 *
 * bitlinear_backward_input:
 *   dY     in   fp32 [M][N], 16-byte aligned; N % 4 == 0.
 *   Wp     in   uint8 [N][K/4], 16-byte aligned: the forward's packed weights.
 *   gamma  in   fp32 [1], the forward's weight scale.
 *   M, N, K     0 <= M, N < 2^31 - 63; K % 64 == 0; K <= BL_MAX_K; at most
 *               2^28 output tiles of 128 x 256 and 2^31 - 1 transpose tiles
 *               of 64 x 64 (else BL_ERR_HIP).
 *   dX     out  fp32 [M][K].
 *   ws          >= bl_workspace_bytes(BL_OP_BACKWARD_INPUT, M, N, K, 0) bytes,
 *               16-byte aligned (the weights unpacked to bf16, transposed;
 *               fp32 partial tiles when the product is split along N).
 * bitlinear_backward_weight:
 *   dY     in   fp32 [M][N], 16-byte aligned.
 *   Xq     in   int8 [M][K], 16-byte aligned;  d  in  fp32 [M]: the forward's
 *               quantised input (quant_act_absmax_i8).
 *   M, N, K     as above (N any).
 *   dW     out  fp32 [N][K].
 *   ws          >= bl_workspace_bytes(BL_OP_BACKWARD_WEIGHT, M, N, K, 0) bytes,
 *               16-byte aligned ((dY o d)^T as bf16 hi and lo planes, Xq^T in
 *               bf16; fp32 partial tiles when the product is split along M).
 * The forward of a training step is quant_weight_absmean_pack on the latent
 * weights, quant_act_absmax_i8 and bitlinear_gemm; the optimiser step is the
 * caller's.
 */
bl_status bitlinear_backward_input(const float *dY, int64_t M, int64_t N, const uint8_t *Wp,
                                   const float *gamma, int64_t K, float *dX, void *ws,
                                   size_t ws_bytes, void *stream);
bl_status bitlinear_backward_weight(const float *dY, int64_t M, int64_t N, const int8_t *Xq,
                                    const float *d, int64_t K, float *dW, void *ws,
                                    size_t ws_bytes, void *stream);

/* Workspace bytes a call needs for the given sizes (0 for calls that need
 * none; arguments a call does not use are ignored). */
size_t bl_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int64_t F);

/* Static, never NULL. */
const char *bl_status_string(bl_status status);

/* Detail of this thread's last non-OK return ("" if none).  Valid until the
 * thread's next call into the library. */
const char *bl_last_error(void);

/* BL_ABI_VERSION of the built library. */
int bl_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
