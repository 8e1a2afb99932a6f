// device_common.h -- device helpers shared by the libbitlinear kernels.
//
// Packed weight format ("Microsoft BitNet 深度研究报告", §2 (2), 实际存储:
// codes {0: 0, +1: 1, -1: 2}; technical-report copy, GPU端: four weights per
// int8): byte b of a row holds weights 4b..4b+3, weight 4b+j in bits 2j..2j+1.
// A little-endian dword therefore holds 16 consecutive weights k = 16t + j,
// code j in bits 2j..2j+1.
//
// Unpacking.  (dw >> 2i) & 0x03030303 puts the codes of weights
// {i, 4+i, 8+i, 12+i} (one per byte) into a dword.  v_perm_b32 then maps each
// code byte to the int8 value {0, +1, -1} in one instruction, using the code
// as a byte selector into a constant table.  The four value dwords come out
// in "transposed" order: dword i holds weights i, 4+i, 8+i, 12+i.  The
// activations are put into the same order once (transpose16 below, a 4x4
// byte transpose of each 16-byte group), so that value dword i lines up with
// activation dword i and a v_dot4_i32_i8 (or an int8 MFMA) sums the right
// products.  A dot product does not depend on the order of its terms, so
// this reordering leaves every int32 sum exact and unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// v_perm_b32 semantics: the result byte i is selected by byte i of `sel`
// from the 8 bytes {hi:lo} (selector 0..3 -> bytes of lo, 4..7 -> bytes of
// hi, 8 -> bit 15 of lo replicated, 12 -> 0x00, >= 13 -> 0xFF).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Code selectors 0,1,2(,3) -> bytes of lo = {0x00, 0x01, 0xFF, 0x00}.
constexpr uint32_t kLutLo0 = 0x00FF0100u;
// Code selectors 0,4,8(,12) after masking with 0x0C: 0 -> lo byte 0 = 0x00,
// 4 -> hi byte 0 = 0x01, 8 -> sign of lo byte 1 (0x80) = 0xFF, 12 -> 0x00.
constexpr uint32_t kLutHi1 = 0x00000001u;
constexpr uint32_t kLutLo1 = 0x00008000u;

// 16 codes (one dword) -> four int8x4 value dwords, transposed order.
__device__ __forceinline__ void unpack16(uint32_t dw, uint32_t &v0, uint32_t &v1,
                                         uint32_t &v2, uint32_t &v3) {
    const uint32_t dw4 = dw >> 4;
    v0 = perm(0u, kLutLo0, dw & 0x03030303u);
    v1 = perm(kLutHi1, kLutLo1, dw & 0x0C0C0C0Cu);
    v2 = perm(0u, kLutLo0, dw4 & 0x03030303u);
    v3 = perm(kLutHi1, kLutLo1, dw4 & 0x0C0C0C0Cu);
}

// 4x4 byte transpose of a 16-byte group: out dword i = bytes i of in dwords
// 0..3, i.e. elements {i, 4+i, 8+i, 12+i}.
__device__ __forceinline__ uint4 transpose16(uint4 v) {
    const uint32_t lo01 = perm(v.y, v.x, 0x05010400u);  // x0 y0 x1 y1
    const uint32_t hi01 = perm(v.y, v.x, 0x07030602u);  // x2 y2 x3 y3
    const uint32_t lo23 = perm(v.w, v.z, 0x05010400u);  // z0 w0 z1 w1
    const uint32_t hi23 = perm(v.w, v.z, 0x07030602u);  // z2 w2 z3 w3
    uint4 o;
    o.x = perm(lo23, lo01, 0x05040100u);                 // x0 y0 z0 w0
    o.y = perm(lo23, lo01, 0x07060302u);                 // x1 y1 z1 w1
    o.z = perm(hi23, hi01, 0x05040100u);                 // x2 y2 z2 w2
    o.w = perm(hi23, hi01, 0x07060302u);                 // x3 y3 z3 w3
    return o;
}

// Sixteen 4-bit activation codes (8 bytes; element 2b in bits 0..3 of byte b,
// element 2b+1 in bits 4..7, 4-bit two's complement) -> their int8 values in
// the order transpose16 gives: dword i holds elements {i, 4+i, 8+i, 12+i}.
// The low and high nibbles are split into bytes, picked into place with
// v_perm, and each byte n is sign-extended as ((n ^ 8) + 0x78) ^ 0x80, which
// never carries into the next byte.
__device__ __forceinline__ uint32_t sext4_bytes(uint32_t v) {
    return ((v ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}
__device__ __forceinline__ uint4 a4_to_t16(uint2 p) {
    const uint32_t lx = p.x & 0x0F0F0F0Fu, hx = (p.x >> 4) & 0x0F0F0F0Fu;   // e0 e2 e4 e6 | e1 e3 e5 e7
    const uint32_t ly = p.y & 0x0F0F0F0Fu, hy = (p.y >> 4) & 0x0F0F0F0Fu;   // e8 .. e14  | e9 .. e15
    uint4 t;
    t.x = sext4_bytes(perm(ly, lx, 0x06040200u));                           // e0 e4 e8 e12
    t.y = sext4_bytes(perm(hy, hx, 0x06040200u));                           // e1 e5 e9 e13
    t.z = sext4_bytes(perm(ly, lx, 0x07050301u));                           // e2 e6 e10 e14
    t.w = sext4_bytes(perm(hy, hx, 0x07050301u));                           // e3 e7 e11 e15
    return t;
}

// Reductions across lanes.  Steps inside a row of 16 lanes go through DPP
// (no LDS round trip, unlike a ds_bpermute shuffle): xor 1 and xor 2 as quad
// permutes, then the mirrored lane of the 8-lane half-row and of the row.
// After the steps for a group of G lanes (G a power of two, groups aligned
// to G) every lane of the group holds the group's sum (or maximum); groups
// of 32 and 64 lanes add shuffle steps.  The combination order differs from
// a plain butterfly, so these serve order-free reductions only (integer
// sums, maxima).  Call them with every lane of the wave active.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int group_sum(int v, int G) {
    if (G >= 2) v += dpp_i32<kDppXor1>(v);
    if (G >= 4) v += dpp_i32<kDppXor2>(v);
    if (G >= 8) v += dpp_i32<kDppHalfMirror>(v);
    if (G >= 16) v += dpp_i32<kDppMirror>(v);
    if (G >= 32) v += __shfl_xor(v, 16);
    if (G >= 64) v += __shfl_xor(v, 32);
    return v;
}
__device__ __forceinline__ float group_max(float v, int G) {
    if (G >= 2) v = fmaxf(v, __int_as_float(dpp_i32<kDppXor1>(__float_as_int(v))));
    if (G >= 4) v = fmaxf(v, __int_as_float(dpp_i32<kDppXor2>(__float_as_int(v))));
    if (G >= 8) v = fmaxf(v, __int_as_float(dpp_i32<kDppHalfMirror>(__float_as_int(v))));
    if (G >= 16) v = fmaxf(v, __int_as_float(dpp_i32<kDppMirror>(__float_as_int(v))));
    if (G >= 32) v = fmaxf(v, __shfl_xor(v, 16));
    if (G >= 64) v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// fp32 rescale of an exact int32 sum: fl(float(acc) * c), c = fl(gamma * d).
__device__ __forceinline__ float rescale(int32_t acc, float c) {
    return __fmul_rn((float)acc, c);
}

// Per-token absmax int8 (iaiol.com article, 权重映射为三元值; model card,
// 模型详情): with a = max |x| over the token,
//   s = fl(127 / a),  q = clamp(rne(fl(x * s)), -127, 127),  d = fl(a / 127),
// and a == 0 gives s = 0, q = 0, d = 0.  Every kernel that quantises
// activations uses these three functions, so all paths give the same codes.
__device__ __forceinline__ float act_inv_scale(float a) {
    return a > 0.0f ? __fdiv_rn(127.0f, a) : 0.0f;
}
__device__ __forceinline__ float act_scale(float a) {
    return a > 0.0f ? __fdiv_rn(a, 127.0f) : 0.0f;
}
__device__ __forceinline__ int act_code(float x, float s) {
    float r = __builtin_rintf(__fmul_rn(x, s));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// The same rule at 4 bits ("Microsoft BitNet 深度研究报告", §3 论文演进时间线:
// BitNet a4.8): s = fl(7 / a), q = clamp(rne(fl(x * s)), -7, 7), d = fl(a / 7).
__device__ __forceinline__ float act4_inv_scale(float a) {
    return a > 0.0f ? __fdiv_rn(7.0f, a) : 0.0f;
}
__device__ __forceinline__ float act4_scale(float a) {
    return a > 0.0f ? __fdiv_rn(a, 7.0f) : 0.0f;
}
__device__ __forceinline__ int act4_code(float x, float s) {
    float r = __builtin_rintf(__fmul_rn(x, s));
    r = fminf(fmaxf(r, -7.0f), 7.0f);
    return (int)r;
}

// A read-only value every lane reads from the same address, through the
// constant address space: a scalar load.  It does not share the vector-memory
// counter with weight loads and output stores, so issuing it early and using
// it late never waits on those.
__device__ __forceinline__ float scalar_load(const float *p) {
    return *(const __attribute__((address_space(4))) float *)p;
}
__device__ __forceinline__ double scalar_load(const double *p) {
    return *(const __attribute__((address_space(4))) double *)p;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace bl
