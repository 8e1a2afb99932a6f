/*
 * oracle.c -- plain CPU oracle for the BitLinear W1.58A8 layer.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  The
 * GPU library (libbitlinear) never calls it, and the two share no source,
 * header, table or helper.
 *
 * Every function below follows one definition from the pages, cited by page
 * title and section, in the pages' order and notation.  Nothing is blocked,
 * fused or reordered: the loops are the sums of the definitions.  Where the
 * pages leave a step open the reading taken is stated at the function.
 *
 * Pages cited:
 *   [RPT]  "Microsoft BitNet 深度研究报告" (conanxin.github.io), section 2
 *          "技术原理": (1) 三元量化, (2) AbsMean 量化 (quantisation function
 *          and the "实际存储" 2-bit storage map), (3) 查找表优化 (the
 *          add / subtract / skip rules).
 *   [CARD] "BitNet b1.58 2B4T - 原生1比特大语言模型规模化实践"
 *          (model.aibase.cn), "模型详情": W1.58A8, absmean weights,
 *          per-token absmax int8 activations, ReLU², subln, no biases.
 *   [NEWS] iaiol.com article on BitNet b1.58 2B4T, section
 *          "权重映射为三元值{-1, 0, +1}": per-token absmax 8-bit
 *          activations, subln, ReLU² in place of SwiGLU.
 *   [TR]   tanhuajipinx.com copy of the "BitNet b1.58 2B4T Technical Report",
 *          section "推理完满" / "GPU端": four ternary weights packed into one
 *          int8 for the W1.58A8 matmul.
 *
 * Floating point: built with -ffp-contract=off -fno-fast-math.  Results that
 * only feed a tolerance check are computed in fp64.  Where a float decides an
 * integer (an int8 activation code) the pages fix no precision, so the
 * decision is taken in fp32 with the op sequence stated at the function, the
 * same precision the GPU kernels use.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <stddef.h>
#include <string.h>

#define OB_EXPORT __attribute__((visibility("default")))

/* Threads the OpenMP loops below use (reported with CPU timings). */
OB_EXPORT int ob_num_threads(void) { return omp_get_max_threads(); }

/* Sets the threads of later parallel loops (for CPU timings at 1 thread). */
OB_EXPORT void ob_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ---------------------------------------------------------------------- */
/* [RPT] §2 (2) AbsMean 量化:  gamma = (1/n) * sum_i |w_i|.
 *
 * n runs over every element of the weight tensor, so gamma is one number per
 * BitLinear weight matrix W[N][K] (nn.Linear layout: N outputs, K inputs).
 * The pages give no precision or order for the sum.  Reading taken: the terms
 * |w_i| are taken in the tensor's own row-major order, i = n * K + k, and
 * summed in fp64 by pairwise summation: neighbours are added in pairs
 * (|w_0| + |w_1|, |w_2| + |w_3|, ...), then neighbouring pair sums, and so on
 * until one sum is left; a term or sum with no right neighbour at its level
 * is carried up unchanged (the same as adding a zero term).  The sum is
 * divided by n in fp64 and rounded once to fp32.  Every |w| is exact in
 * fp64, so only the pair additions round; pairwise summation keeps that error
 * below ~log2(n) * 2^-53 of the sum, so gamma is the fp32 nearest the exact
 * mean unless the mean lies that close to an fp32 rounding boundary.  An
 * empty tensor (n == 0) gets gamma = 0. */
OB_EXPORT float ob_absmean_gamma(const float *W, int64_t N, int64_t K)
{
    const int64_t n = N * K;
    if (N <= 0 || K <= 0)
        return 0.0f;
    double *v = (double *)malloc((size_t)n * sizeof(double));
    if (!v)
        return NAN;
    for (int64_t i = 0; i < n; ++i)
        v[i] = fabs((double)W[i]);
    /* level with stride h: v[i] (i a multiple of 2h) holds the sum of the
     * terms i .. i+h-1; it absorbs its right neighbour v[i + h] if there is
     * one. */
    for (int64_t h = 1; h < n; h *= 2) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n - h; i += 2 * h)
            v[i] += v[i + h];
    }
    const double total = v[0];
    free(v);
    return (float)(total / (double)n);
}

/* [RPT] §2 (2) AbsMean 量化:  Q(w) = round(clamp(w / gamma, -1, 1)).
 *
 * Written out literally in fp64.  round() is taken as IEEE round-half-to-even
 * (nearbyint in the default rounding mode), so w / gamma == +-0.5 maps to 0.
 * The pages print no epsilon: gamma == 0 means the tensor is all zeros (or so
 * small that its mean underflows), and then w == 0 maps to 0 and any nonzero
 * w to sign(w) (w / 0 is +-inf before the clamp). */
OB_EXPORT void ob_ternarize(const float *W, int64_t count, float gamma, int8_t *Wq)
{
    for (int64_t i = 0; i < count; ++i) {
        double w = (double)W[i];
        if (w == 0.0) {
            Wq[i] = 0;
            continue;
        }
        double t = w / (double)gamma;          /* +-inf when gamma == 0 */
        if (t > 1.0) t = 1.0;                   /* clamp(., -1, 1) */
        if (t < -1.0) t = -1.0;
        Wq[i] = (int8_t)nearbyint(t);          /* round, ties to even */
    }
}

/* [RPT] §2 (2) "实际存储": stored value {0: 0, +1: 1, -1: 2}, 2 bits each.
 * [TR] GPU端: four ternary weights per int8.
 *
 * Reading taken for the byte: row-major [N][K/4]; byte b of row n holds the
 * four consecutive weights k = 4b .. 4b+3, weight 4b+j in bits 2j..2j+1
 * (least significant pair first).  K must be a multiple of 4. */
static uint8_t ob_code_of(int8_t q)
{
    if (q == 1) return 1;
    if (q == -1) return 2;
    return 0;
}

OB_EXPORT void ob_pack(const int8_t *Wq, int64_t N, int64_t K, uint8_t *Wp)
{
    int64_t KB = K / 4;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < KB; ++b) {
            uint8_t byte = 0;
            for (int j = 0; j < 4; ++j)
                byte |= (uint8_t)(ob_code_of(Wq[n * K + 4 * b + j]) << (2 * j));
            Wp[n * KB + b] = byte;
        }
}

/* Inverse of the storage map.  Code 3 is never written; it reads as 0. */
static int8_t ob_value_of(unsigned code)
{
    if (code == 1) return 1;
    if (code == 2) return -1;
    return 0;
}

OB_EXPORT void ob_unpack(const uint8_t *Wp, int64_t N, int64_t K, int8_t *Wq)
{
    int64_t KB = K / 4;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            unsigned byte = Wp[n * KB + k / 4];
            Wq[n * K + k] = ob_value_of((byte >> (2 * (k % 4))) & 3u);
        }
}

/* Denser storage, five weights per byte.  The pages give ternary weights
 * about 1.58 bits each (log2 3; iaiol.com article, "权重映射为三元值"; the
 * 0.4 GB model of the aigc.izzi.cn news page) while the stored format is 2
 * bits ([RPT] 实际存储, the int2 I2_S kernel of its 内核类型 table).  Five
 * base-3 digits fit one byte (3^5 = 243 <= 256): 1.6 bits per weight.  The
 * pages give no layout; the one taken here:
 *   - digit d = w + 1 in {0, 1, 2} (linear in w);
 *   - byte b of a row holds weights 5b .. 5b + 4; with v = sum_j d_j 3^(4-j)
 *     (weight 5b first, as the most significant digit) the byte stores
 *     q = ceil(256 v / 243), so that q / 256 approximates v / 243 from above;
 *   - weights past K read as 0 (digit 1), and a row is padded to a multiple
 *     of 16 bytes with such bytes.
 * Decoding: v = floor(243 q / 256) recovers v exactly (243 q / 256 lies in
 * [v, v + 243/256)); its base-3 digits are the weights plus one. */
OB_EXPORT int64_t ob_t5_row_bytes(int64_t K) { return ((K + 4) / 5 + 15) / 16 * 16; }

OB_EXPORT void ob_pack_t5(const int8_t *Wq, int64_t N, int64_t K, uint8_t *Wt5)
{
    int64_t RB = ob_t5_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < RB; ++b) {
            int v = 0;
            for (int j = 0; j < 5; ++j) {
                int64_t k = 5 * b + j;
                int digit = k < K ? Wq[n * K + k] + 1 : 1;
                v = 3 * v + digit;
            }
            Wt5[n * RB + b] = (uint8_t)((256 * v + 242) / 243);
        }
}

OB_EXPORT void ob_unpack_t5(const uint8_t *Wt5, int64_t N, int64_t K, int8_t *Wq)
{
    static const int pow3[5] = {1, 3, 9, 27, 81};
    int64_t RB = ob_t5_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int q = Wt5[n * RB + k / 5];
            int v = (243 * q) / 256;
            int digit = (v / pow3[4 - (int)(k % 5)]) % 3;
            Wq[n * K + k] = (int8_t)(digit - 1);
        }
}

/* bf16 -> fp32 widening: the bf16 bits are the upper half of the fp32 bits,
 * so the conversion is exact. */
OB_EXPORT void ob_bf16_to_f32(const uint16_t *src, int64_t count, float *dst)
{
    for (int64_t i = 0; i < count; ++i) {
        uint32_t bits = (uint32_t)src[i] << 16;
        memcpy(&dst[i], &bits, sizeof bits);
    }
}

/* [NEWS] "权重映射为三元值", [CARD] 模型详情: activations are quantised to
 * 8-bit integers per token with absmax.
 *
 * The pages print neither the formula nor the constant.  Reading taken, the
 * symmetric absmax quantiser of the W1.58A8 scheme, for each token row m:
 *     a   = max_k |x[m][k]|                     (exact)
 *     s   = fl32(127 / a)
 *     Xq  = clamp(rne(fl32(x * s)), -127, 127)
 *     d   = fl32(a / 127)                        (x ~= Xq * d)
 * and an all-zero row gives Xq = 0, d = 0.  Each step is one fp32 operation
 * rounded to nearest; rne is round-half-to-even. */
OB_EXPORT void ob_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *d)
{
    for (int64_t m = 0; m < M; ++m) {
        const float *x = X + m * K;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float ax = fabsf(x[k]);
            if (ax > a) a = ax;
        }
        if (a == 0.0f) {
            for (int64_t k = 0; k < K; ++k) Xq[m * K + k] = 0;
            d[m] = 0.0f;
            continue;
        }
        float s = 127.0f / a;
        for (int64_t k = 0; k < K; ++k) {
            float p = x[k] * s;
            float r = nearbyintf(p);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            Xq[m * K + k] = (int8_t)r;
        }
        d[m] = a / 127.0f;
    }
}

/* "Microsoft BitNet 深度研究报告", §3 论文演进时间线 (the BitNet a4.8 row:
 * activations at 4 bits, a further compression) and §10 关键资源 (BitNet
 * a4.8, activation quantisation).  The pages name the 4-bit activations and
 * nothing else.  Reading taken: the absmax rule of ob_quant_act with the
 * signed 4-bit range, for each token row m:
 *     a   = max_k |x[m][k]|
 *     s   = fl32(7 / a)
 *     q   = clamp(rne(fl32(x * s)), -7, 7)
 *     d   = fl32(a / 7)                          (x ~= q * d)
 * an all-zero row giving q = 0, d = 0 (-8 is never produced).  The codes go
 * into the same ternary accumulation and rescale as the 8-bit ones. */
OB_EXPORT void ob_quant_act4(const float *X, int64_t M, int64_t K, int8_t *Xq, float *d)
{
    for (int64_t m = 0; m < M; ++m) {
        const float *x = X + m * K;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float ax = fabsf(x[k]);
            if (ax > a) a = ax;
        }
        if (a == 0.0f) {
            for (int64_t k = 0; k < K; ++k) Xq[m * K + k] = 0;
            d[m] = 0.0f;
            continue;
        }
        float s = 7.0f / a;
        for (int64_t k = 0; k < K; ++k) {
            float p = x[k] * s;
            float r = nearbyintf(p);
            if (r > 7.0f) r = 7.0f;
            if (r < -7.0f) r = -7.0f;
            Xq[m * K + k] = (int8_t)r;
        }
        d[m] = a / 7.0f;
    }
}

/* Storage of the 4-bit codes (the pages give none).  Reading taken: two
 * codes per byte, row-major [M][K/2]; byte b of a row holds element 2b in
 * bits 0..3 and element 2b+1 in bits 4..7, each as a 4-bit two's-complement
 * number.  K must be even. */
OB_EXPORT void ob_pack_act4(const int8_t *Xq, int64_t M, int64_t K, uint8_t *P)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < K / 2; ++b) {
            uint8_t lo = (uint8_t)Xq[m * K + 2 * b] & 0x0F;
            uint8_t hi = (uint8_t)Xq[m * K + 2 * b + 1] & 0x0F;
            P[m * (K / 2) + b] = (uint8_t)(lo | (hi << 4));
        }
}

static int8_t ob_nibble(uint8_t v)               /* 4-bit two's complement */
{
    return (int8_t)(v < 8 ? v : (int)v - 16);
}

OB_EXPORT void ob_unpack_act4(const uint8_t *P, int64_t M, int64_t K, int8_t *Xq)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < K / 2; ++b) {
            uint8_t v = P[m * (K / 2) + b];
            Xq[m * K + 2 * b] = ob_nibble(v & 0x0F);
            Xq[m * K + 2 * b + 1] = ob_nibble(v >> 4);
        }
}

/* [RPT] §2 (3) 查找表优化: with W in {-1, 0, +1}, C = A x Q(W) needs no
 * multiplication:  W = +1: C += A;  W = -1: C -= A;  W = 0: skip.
 *
 * acc[m][n] = sum_k Xq[m][k] * Wq[n][k], formed exactly that way from the
 * packed codes; the int32 result is exact while 127 * K < 2^31.  The rows
 * n are independent, so they are shared among OpenMP threads; each sum runs
 * in ascending k. */
OB_EXPORT void ob_ternary_acc(const int8_t *Xq, const uint8_t *Wp,
                              int64_t M, int64_t N, int64_t K, int32_t *acc)
{
    int64_t KB = K / 4;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t c = 0;
            for (int64_t k = 0; k < K; ++k) {
                unsigned code = (Wp[n * KB + k / 4] >> (2 * (k % 4))) & 3u;
                int8_t w = ob_value_of(code);
                if (w == 1)
                    c += Xq[m * K + k];
                else if (w == -1)
                    c -= Xq[m * K + k];
                /* w == 0: skip */
            }
            acc[m * N + n] = (int32_t)c;
        }
    }
}

/* W1.58A8 rescale ([CARD] 模型详情; [NEWS] section "微软在1 bit LLM上的探索"
 * names the mixed-precision W1.58A8 product).  The layer computes
 * Y = (Xq * d) (Wq * gamma)^T, so Y[m][n] = acc[m][n] * gamma * d[m].
 * Evaluated in fp64 (the result feeds a tolerance check only). */
OB_EXPORT void ob_dequant_f64(const int32_t *acc, const float *d, float gamma,
                              int64_t M, int64_t N, double *Y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = (double)acc[m * N + n] * (double)gamma * (double)d[m];
}

/* The same rescale as an fp32 value, for the points where it then decides an
 * integer (the FFN requantisation).  The pages give no order; reading taken:
 *     c_m = fl32(gamma * d[m]);  Y = fl32(float(acc) * c_m).
 * float(acc) is exact while |acc| <= 2^24. */
OB_EXPORT void ob_dequant_f32(const int32_t *acc, const float *d, float gamma,
                              int64_t M, int64_t N, float *Y)
{
    for (int64_t m = 0; m < M; ++m) {
        float c = gamma * d[m];
        for (int64_t n = 0; n < N; ++n) {
            float y = (float)acc[m * N + n] * c;
            Y[m * N + n] = y;
        }
    }
}

/* Feed-forward tail of a BitNet b1.58 block.
 * [NEWS] "权重映射为三元值" and [CARD] 模型详情: the FFN uses ReLU² in place
 * of SwiGLU, subln normalisation stabilises low-bit training, and every
 * linear layer is a BitLinear without bias.
 *
 * Readings taken (the pages print no formulas for these):
 *   - gated, like the SwiGLU it replaces:  H = relu(G)^2 * U, with
 *     G = Xq Wg^T and U = Xq Wu^T as W1.58A8 BitLinears (fp32 values);
 *     Wu == NULL gives the ungated H = relu(G)^2;
 *   - subln is an RMSNorm over the F features of H, with optional gain g
 *     (NULL = ones):  Z = H / rms * g,  rms = sqrt(sum_f H^2 / F + eps);
 *   - Z is requantised per token by the absmax rule of ob_quant_act and fed
 *     to the down projection Y = Zq Wd^T (W1.58A8, fp64 result).
 *
 * Absmax quantisation of a row does not change when the row is multiplied
 * by a positive number, and 1/rms is such a number for each row.  So the
 * int8 codes of Z equal the codes of H * g, and Z's scale is d_h / rms with
 * d_h the scale of H * g.  The int8 decision is therefore taken on the fp32
 * values H * g, independent of how rms is summed:
 *     G, U   = ob_dequant_f32(...)              (fp32)
 *     r      = max(G, 0)
 *     H      = fl32(fl32(r * r) * U)            (ungated: fl32(r * r))
 *     Z'     = fl32(H * g)                      (Z' = H when g is NULL)
 *     Hq, dh = ob_quant_act(Z')
 *     rms    = sqrt(sum_f H^2 / F + eps)        (fp64)
 *     Y      = acc_d * gamma_d * (dh / rms)     (fp64; 0 where dh == 0)
 * Outputs: Y [M][N] fp64, Hq [M][F] int8, dh [M] fp32, rms [M] fp64, and
 * optionally Y32 [M][N], the fp32 value of Y (see below). */
OB_EXPORT void ob_ffn_relu2(const int8_t *Xq, const float *d, int64_t M, int64_t K, int64_t F,
                            const uint8_t *Wg, float gamma_g,
                            const uint8_t *Wu, float gamma_u,
                            const float *norm_w, float eps,
                            const uint8_t *Wd, float gamma_d, int64_t N,
                            double *Y, int8_t *Hq, float *dh, double *rms,
                            int32_t *acc_scratch /* [M][max(F,N)] */,
                            float *G /* [M][F] */, float *U /* [M][F] */,
                            float *Zp /* [M][F] */, float *Y32 /* [M][N] or NULL */)
{
    ob_ternary_acc(Xq, Wg, M, F, K, acc_scratch);
    ob_dequant_f32(acc_scratch, d, gamma_g, M, F, G);
    if (Wu) {
        ob_ternary_acc(Xq, Wu, M, F, K, acc_scratch);
        ob_dequant_f32(acc_scratch, d, gamma_u, M, F, U);
    }
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t f = 0; f < F; ++f) {
            float r = G[m * F + f] > 0.0f ? G[m * F + f] : 0.0f;
            float r2 = r * r;
            float h = Wu ? r2 * U[m * F + f] : r2;
            float z = norm_w ? h * norm_w[f] : h;
            Zp[m * F + f] = z;
            ss += (double)h * (double)h;
        }
        rms[m] = sqrt(ss / (double)F + (double)eps);
    }
    ob_quant_act(Zp, M, F, Hq, dh);
    ob_ternary_acc(Hq, Wd, M, N, F, acc_scratch);
    for (int64_t m = 0; m < M; ++m) {
        /* Z's scale; a row whose H * g is all zero has Zq = 0 and scale 0. */
        double dz = dh[m] > 0.0f ? (double)dh[m] / rms[m] : 0.0;
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = (double)acc_scratch[m * N + n] * (double)gamma_d * dz;
        if (Y32) {
            /* The same output as an fp32 value, for when it feeds a later
             * quantisation: dz rounded once to fp32, then the BitLinear rescale
             * c = fl32(gamma_d * dz), Y = fl32(float(acc) * c). */
            float dz32 = (float)dz;
            float c = gamma_d * dz32;
            for (int64_t n = 0; n < N; ++n)
                Y32[m * N + n] = (float)acc_scratch[m * N + n] * c;
        }
    }
}
