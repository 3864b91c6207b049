// Device helpers of the CSA2 kernels for gfx950: bf16 moves, the fp32 exp of
// the pair gate, the FP4 (E2M1 + E8M0 per 32) and FP8 (E4M3FN + fp32 row
// scale) encoders, and the dequantisers used by the attention gather.
//
// Formats follow "Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV Cache"
// (sections "Deriving the 890 bytes per token", "FP4 is a storage choice") and
// "Inside DeepSeek V4.1", section "890 bytes": four-bit values with one byte
// scale per block of 32, an FP8 window.  Rounding is nearest-even, saturating;
// the block scale is 2^(floor(log2 max|x|) - 2) (the OCP MX rule for E2M1).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int D = 512;          // latent width
constexpr int ROPE_LO = 448;    // rotated channels of the latent: 448..511
constexpr int PAIRS = 32;       // rotated pairs per row
constexpr int WINDOW = 128;     // window rows
constexpr int HI = 32;          // indexer heads
constexpr int DI = 128;         // indexer width
constexpr int KI_ROPE_LO = 64;  // rotated channels of an index key: 64..127
constexpr int TOPK = 512;
constexpr int POOL_BLOCKS = 2048;  // blocks of 8 entries kept by the hierarchical pool
constexpr int IDX_CHUNK = 2048;  // index entries scanned by one wave of the score kernel
constexpr int ATT_THREADS = 768; // attention block: 4 QK waves + 8 PV waves

typedef __attribute__((ext_vector_type(2))) float f2;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(4))) int i4;
typedef __attribute__((ext_vector_type(8))) int i8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
typedef __attribute__((ext_vector_type(4))) unsigned int u4v;   // 16-byte loads with builtins

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Correctly rounded fp32 division / square root (IEEE), independent of compiler defaults.
__device__ __forceinline__ float div_rn(float a, float b) { return __fdiv_rn(a, b); }
__device__ __forceinline__ float sqrt_rn(float a) { return __fsqrt_rn(a); }

// exp(x) for x <= 0: Cody-Waite reduction by ln 2 (head with 16 significant
// bits, fp32 tail), degree-7 Taylor polynomial in Horner form, scaling by 2^k.
// Below -87 the result is 0 so every result is a normal number.
__device__ __forceinline__ float exp_neg(float x) {
    if (x < -87.0f) return 0.0f;
    const float kf = rintf(x * 1.44269502f);
    float r = __builtin_fmaf(-kf, 0.693145751953125f, x);
    r = __builtin_fmaf(-kf, 1.42860677e-06f, r);
    float p = 0.000198412701f;
    p = __builtin_fmaf(p, r, 0.00138888892f);
    p = __builtin_fmaf(p, r, 0.00833333377f);
    p = __builtin_fmaf(p, r, 0.0416666679f);
    p = __builtin_fmaf(p, r, 0.166666672f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return ldexpf(p, (int)kf);
}

// floor(log2 a) for a finite a > 0 (normal or subnormal)
__device__ __forceinline__ int floor_log2(float a) {
    uint32_t u = __float_as_uint(a);
    int e = (int)(u >> 23);
    if (e != 0) return e - 127;
    return (31 - __clz((int)(u & 0x7FFFFFu))) - 149;
}

// E8M0 block exponent of a block whose max magnitude is amax (0 for an empty block)
__device__ __forceinline__ int mx_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    int e = floor_log2(amax) - 2;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E2M1 code of y (already divided by the block scale): nearest of
// {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
    const float a = fabsf(y);
    uint32_t c;
    if (a <= 0.25f) c = 0;
    else if (a < 0.75f) c = 1;
    else if (a <= 1.25f) c = 2;
    else if (a < 1.75f) c = 3;
    else if (a <= 2.5f) c = 4;
    else if (a < 3.5f) c = 5;
    else if (a <= 5.0f) c = 6;
    else c = 7;
    return c | ((__float_as_uint(y) >> 28) & 8u);
}

// E4M3FN code of y: nearest even, saturating at 448 (NaN codes never produced).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const float a = fabsf(y);
    uint32_t c;
    if (!(a < 448.0f)) {
        c = 0x7E;
    } else if (a < 0.015625f) {              // below 2^-6: subnormal steps of 2^-9
        c = (uint32_t)rintf(a * 512.0f);     // 8 lands on the smallest normal code
    } else {
        int e = floor_log2(a);
        float m = ldexpf(a, -e);             // [1, 2), exact
        uint32_t q = (uint32_t)rintf((m - 1.0f) * 8.0f);
        if (q == 8) { q = 0; e += 1; }
        c = ((uint32_t)(e + 7) << 3) | q;
        if (c > 0x7E) c = 0x7E;
    }
    return c | ((__float_as_uint(y) >> 24) & 0x80u);
}

// E4M3FN codes of four values of magnitude below 464 (byte k = value k), by
// the hardware fp32 -> fp8 conversion, which rounds to nearest even as
// e4m3_code does and gives the same code for every such value (448 <= |v| <
// 464 included: 448).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// E4M3FN code of a non-negative finite value -> fp32 (exact)
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    return e ? ldexpf((float)(8u + m), (int)e - 10) : (float)m * 0.001953125f;
}

// ---- dequantisation to bf16 (exact) ----------------------------------------

// two E2M1 values (byte k of w) times an E4M3 scale value s, as packed bf16 (low =
// element 2i): the product has at most 6 significant bits, so the bf16 is exact
__device__ __forceinline__ uint32_t fp4x2_e4_to_bf16x2(uint32_t w, int k, float s) {
    const bf2 v = k == 0 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0)
                : k == 1 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1)
                : k == 2 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2)
                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
    return (uint32_t)f2bf((float)v[0] * s) | ((uint32_t)f2bf((float)v[1] * s) << 16);
}

// two E2M1 values of one byte, times 2^(sbyte-127), as packed bf16 (low = element 2i)
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t byte, float scale) {
    bf2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(byte, scale, 0);
    return __builtin_bit_cast(uint32_t, v);
}

// E8M0 byte -> fp32 power of two (byte 0 = 2^-127)
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// two E4M3FN codes (bytes 0,1 of w, or bytes 2,3 when HI_HALF) -> packed bf16, low = first
template <bool HI_HALF>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    bf2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI_HALF);
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace csa2
