// Compression of new positions into the FP4 caches, the FP8 window ring, and
// the plain row encoders/decoders.
//
// Steps of "DeepSeek V4.1 -- Pooled group -> Source layer, pairs pooled"
// (compressed sparse attention equations): pair pooling with a per-channel
// two-way softmax gate; RMSNorm of the pooled row (eps 1e-20, "Window layer ->
// Attention RMSNorm"); rotation of channels 448..511 at position 2j; FP4
// storage; the index-key projection 512->128, its RMSNorm, rotation of
// channels 64..127 at 2j and FP4 storage; the window rows rotated at their own
// position and stored FP8.  At compression ratio one ("Inside DeepSeek V4.1
// Flash: Deriving the 890-Byte KV Cache", CSA2 section) entry j is position j
// alone: the softmax over its single gate logit is 1, so the pooled key is its
// k^c, and both rotations are at j.
//
// Every value that decides a storage code is computed in fp32 with a fixed
// operation order (no contraction, explicit fma where one is meant,
// correctly rounded division and square root) so that the codes are
// reproducible bit for bit:
//   gate     m = max(a,b); ea = exp(a-m); eb = exp(b-m); s = ea+eb;
//            k^p = (ea/s)*ka + (eb/s)*kb        (two products, one sum)
//   RMSNorm  partial[g] = fma chain over channels 8g..8g+7 (ascending);
//            partial[g] += partial[g+s] for s = n/16 .. 1;
//            r = 1/sqrt(partial[0]*(1/n) + 1e-20); y = gamma*(x*r)
//   rotation (x0,x1) -> (x0*c - x1*s, x0*s + x1*c), products rounded first
//   K^I      k^i[n] = fma chain over k = 0..511 ascending of c[k]*W[k][n]
#include "csa2_device.h"

namespace csa2 {

// Entry j of request b from its two tokens' rows (pooled keys ka, kb and gate
// logits ga, gb; 512 bf16 each), or from the one row ka when kb_row is NULL
// (ratio one; no gate is read), on one wave: lane l owns channels 8l..8l+7 of
// the 512-wide row and channels 2l, 2l+1 of the 128-wide index key.  ki_row is
// the given index key (128 bf16) when w_ik is NULL.  c_lds and ki_lds are this
// wave's scratch rows in LDS (512 and 128 floats).
__device__ __forceinline__ void compress_entry(
    int b, int64_t j, int lane, const uint16_t* __restrict__ ka_row,
    const uint16_t* __restrict__ kb_row, const uint16_t* __restrict__ ga_row,
    const uint16_t* __restrict__ gb_row, const uint16_t* __restrict__ ki_row,
    const float* __restrict__ gamma_c, const uint16_t* __restrict__ w_ik,
    const float* __restrict__ gamma_ik, const float* __restrict__ cs,
    const float* __restrict__ sn, float* c_lds, float* ki_lds, uint8_t* __restrict__ z_codes,
    uint8_t* __restrict__ z_scales, uint8_t* __restrict__ ki_codes,
    uint8_t* __restrict__ ki_scales, int64_t entry_stride, int zfmt) {
    // ---- pair gate --------------------------------------------------------
    const uint4 ka = *(const uint4*)(ka_row + 8 * lane);
    const uint32_t kaw[4] = {ka.x, ka.y, ka.z, ka.w};
    float kp[8];
    if (!kb_row) {
#pragma unroll
        for (int i = 0; i < 8; ++i) kp[i] = bf2f((uint16_t)(kaw[i >> 1] >> ((i & 1) * 16)));
    } else {
        const uint4 kb = *(const uint4*)(kb_row + 8 * lane);
        const uint4 ga = *(const uint4*)(ga_row + 8 * lane), gb = *(const uint4*)(gb_row + 8 * lane);
        const uint32_t kbw[4] = {kb.x, kb.y, kb.z, kb.w};
        const uint32_t gaw[4] = {ga.x, ga.y, ga.z, ga.w}, gbw[4] = {gb.x, gb.y, gb.z, gb.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int w = i >> 1, sh = (i & 1) * 16;
            const float a = bf2f((uint16_t)(gaw[w] >> sh)), bb = bf2f((uint16_t)(gbw[w] >> sh));
            const float m = fmaxf(a, bb);
            const float ea = exp_neg(a - m), eb = exp_neg(bb - m);
            const float s = ea + eb;
            const float wa = div_rn(ea, s), wb = div_rn(eb, s);
            const float pa = wa * bf2f((uint16_t)(kaw[w] >> sh));
            const float pb = wb * bf2f((uint16_t)(kbw[w] >> sh));
            kp[i] = pa + pb;
        }
    }

    // ---- RMSNorm over 512: lane = group of 8 channels ----------------------
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) part = __builtin_fmaf(kp[i], kp[i], part);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        const float o = __shfl_down(part, s, 64);
        if (lane < s) part = part + o;
    }
    const float total = __shfl(part, 0, 64);
    const float rr = div_rn(1.0f, sqrt_rn(total * (1.0f / 512.0f) + 1e-20f));
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = gamma_c[8 * lane + i] * (kp[i] * rr);

    // ---- Z: rotate channels 448.. at the entry's position, FP4 -------------
    float z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = c[i];
    if (lane >= ROPE_LO / 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int pi = 4 * (lane - ROPE_LO / 8) + q;
            const float co = cs[pi], si = sn[pi];
            const float x0 = c[2 * q], x1 = c[2 * q + 1];
            const float a = x0 * co, bq = x1 * si, e = x0 * si, f = x1 * co;
            z[2 * q] = a - bq;
            z[2 * q + 1] = e + f;
        }
    }
    if (zfmt == 1) {
        // the pages' format: lanes 2k, 2k+1 share block k of 16 channels and its
        // E4M3 scale E4M3(max/6); elements E2M1(z / scale)
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(z[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        const uint32_t sc = e4m3_code(div_rn(amax, 6.0f));
        const float sv = e4m3_to_f32(sc);
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_code(div_rn(z[i], sv)) << (4 * i);
        if (!(sv > 0.0f)) word = 0;
        const int64_t ent = (int64_t)b * entry_stride + j;
        *(uint32_t*)(z_codes + ent * 256 + 4 * lane) = word;
        if ((lane & 1) == 0) z_scales[ent * 32 + (lane >> 1)] = (uint8_t)sc;
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(z[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        const int e = mx_exponent(amax);
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_code(ldexpf(z[i], -e)) << (4 * i);
        if (!(amax > 0.0f)) word = 0;
        const int64_t ent = (int64_t)b * entry_stride + j;
        *(uint32_t*)(z_codes + ent * 256 + 4 * lane) = word;
        if ((lane & 3) == 0) z_scales[ent * 16 + (lane >> 2)] = (uint8_t)(amax > 0.0f ? e + 127 : 0);
    }

    // ---- index key ---------------------------------------------------------
    float kn0, kn1;
    if (w_ik) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c_lds[8 * lane + i] = c[i];
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        float acc0 = 0.0f, acc1 = 0.0f;
        const uint32_t* W = (const uint32_t*)w_ik;   // [512][64] pairs of bf16
        for (int k = 0; k < D; ++k) {
            const uint32_t wv = W[k * (DI / 2) + lane];
            const float ck = c_lds[k];
            acc0 = __builtin_fmaf(ck, bf2f((uint16_t)wv), acc0);
            acc1 = __builtin_fmaf(ck, bf2f((uint16_t)(wv >> 16)), acc1);
        }
        ki_lds[2 * lane] = acc0;
        ki_lds[2 * lane + 1] = acc1;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        // RMSNorm over 128: group g = lane < 16 holds channels 8g..8g+7
        float p2 = 0.0f;
        if (lane < 16) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = ki_lds[8 * lane + i];
                p2 = __builtin_fmaf(x, x, p2);
            }
        }
#pragma unroll
        for (int s = 8; s >= 1; s >>= 1) {
            const float o = __shfl_down(p2, s, 64);
            if (lane < s) p2 = p2 + o;
        }
        const float tot = __shfl(p2, 0, 64);
        const float r2 = div_rn(1.0f, sqrt_rn(tot * (1.0f / 128.0f) + 1e-20f));
        kn0 = gamma_ik[2 * lane] * (acc0 * r2);
        kn1 = gamma_ik[2 * lane + 1] * (acc1 * r2);
        if (lane >= KI_ROPE_LO / 2) {
            const int pi = lane - KI_ROPE_LO / 2;
            const float co = cs[pi], si = sn[pi];
            const float a = kn0 * co, bq = kn1 * si, e = kn0 * si, f = kn1 * co;
            kn0 = a - bq;
            kn1 = e + f;
        }
    } else {
        const uint32_t v = *(const uint32_t*)(ki_row + 2 * lane);
        kn0 = bf2f((uint16_t)v);
        kn1 = bf2f((uint16_t)(v >> 16));
    }
    {
        float amax = fmaxf(fabsf(kn0), fabsf(kn1));
#pragma unroll
        for (int s = 1; s <= 8; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
        const int e = mx_exponent(amax);
        uint32_t byte = e2m1_code(ldexpf(kn0, -e)) | (e2m1_code(ldexpf(kn1, -e)) << 4);
        if (!(amax > 0.0f)) byte = 0;
        const int64_t ent = (int64_t)b * entry_stride + j;
        ki_codes[ent * 64 + lane] = (uint8_t)byte;
        if ((lane & 15) == 0) ki_scales[ent * 4 + (lane >> 4)] = (uint8_t)(amax > 0.0f ? e + 127 : 0);
    }
}

// One wave (64 lanes) per compressed entry of the call: a token pair (ratio
// 2, rsh = 1) or one token (ratio 1, rsh = 0).
__global__ void __launch_bounds__(256) k_compress(
    int B, int T, const int32_t* __restrict__ pos0, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ gc, const float* __restrict__ gamma_c,
    const uint16_t* __restrict__ w_ik, const float* __restrict__ gamma_ik,
    const uint16_t* __restrict__ ki_given, const float* __restrict__ rcos,
    const float* __restrict__ rsin, int64_t rope_rows, uint8_t* __restrict__ z_codes,
    uint8_t* __restrict__ z_scales, uint8_t* __restrict__ ki_codes,
    uint8_t* __restrict__ ki_scales, int64_t entry_stride, int rsh, int zfmt) {
    __shared__ float c_lds[4][D];
    __shared__ float ki_lds[4][DI];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nloc = T >> rsh;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    if (item >= (int64_t)B * nloc) return;
    const int b = (int)(item / nloc), jl = (int)(item % nloc);
    const int64_t j = (int64_t)(pos0[b] >> rsh) + jl;
    if (j < 0 || j >= entry_stride) return;
    int64_t prow = j << rsh;
    if (prow >= rope_rows) prow = rope_rows - 1;
    const int64_t r0 = ((int64_t)b * T + ((int64_t)jl << rsh)) * D;
    compress_entry(b, j, lane, kc + r0, rsh ? kc + r0 + D : nullptr, rsh ? gc + r0 : nullptr,
                   rsh ? gc + r0 + D : nullptr,
                   w_ik ? nullptr : ki_given + ((int64_t)b * nloc + jl) * DI, gamma_c, w_ik,
                   gamma_ik, rcos + prow * PAIRS, rsin + prow * PAIRS, c_lds[wave], ki_lds[wave],
                   z_codes, z_scales, ki_codes, ki_scales, entry_stride, zfmt);
}

// One window row on one wave: the 512 bf16 of wrow rotated at position p
// (rotary row prow) and written as E4M3FN codes plus one fp32 scale to ring
// slot `slot` (an index over [B][cap]).  Lane l owns channels 8l..8l+7.
__device__ __forceinline__ void window_row(int64_t slot, int64_t prow, int lane,
                                           const uint16_t* __restrict__ wrow,
                                           const float* __restrict__ rcos,
                                           const float* __restrict__ rsin,
                                           uint8_t* __restrict__ w_codes,
                                           float* __restrict__ w_scale) {
    const uint4 v = *(const uint4*)(wrow + 8 * lane);
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = bf2f((uint16_t)(vw[k >> 1] >> ((k & 1) * 16)));
    if (lane >= ROPE_LO / 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int pi = 4 * (lane - ROPE_LO / 8) + q;
            const float co = rcos[prow * PAIRS + pi], si = rsin[prow * PAIRS + pi];
            const float x0 = x[2 * q], x1 = x[2 * q + 1];
            const float a = x0 * co, bq = x1 * si, e = x0 * si, f = x1 * co;
            x[2 * q] = a - bq;
            x[2 * q + 1] = e + f;
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
    for (int s = 1; s <= 32; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
    const float scale = amax > 0.0f ? div_rn(amax, 448.0f) : 1.0f;
    uint32_t lo = 0, hi = 0;
    if (amax > 0.0f) {          // |x / scale| <= 448 (1 + 2^-23): inside e4m3_pack4's range
        float y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = div_rn(x[k], scale);
        lo = e4m3_pack4(y[0], y[1], y[2], y[3]);
        hi = e4m3_pack4(y[4], y[5], y[6], y[7]);
    }
    *(uint2*)(w_codes + slot * D + 8 * lane) = make_uint2(lo, hi);
    if (lane == 0) w_scale[slot] = scale;
}

// One wave per window row: rotate at its position, FP8 row encode into the ring.
__global__ void __launch_bounds__(256) k_window_encode(
    int B, int T, const int32_t* __restrict__ pos0, const uint16_t* __restrict__ wn,
    const float* __restrict__ rcos, const float* __restrict__ rsin, int64_t rope_rows,
    uint8_t* __restrict__ w_codes, float* __restrict__ w_scale, int cap) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    if (item >= (int64_t)B * T) return;
    const int b = (int)(item / T), i = (int)(item % T);
    const int64_t p = (int64_t)pos0[b] + i;
    if (p < 0) return;
    const int64_t prow = p < rope_rows ? p : rope_rows - 1;
    window_row((int64_t)b * cap + (p % cap), prow, lane, wn + item * D, rcos, rsin, w_codes,
               w_scale);
}

// Decode append: one new token per request at absolute position pos[b].  Its
// window row goes to ring slot pos mod cap.  A token at an even position opens
// a pair: its pooled key and gate logits wait in the pair buffer.  A token at
// an odd position closes the pair 2j, 2j+1 (j = pos / 2): entry j is computed
// from the buffered token and this one, exactly as the prefill path computes it.
// At ratio one (rsh = 0) every token writes its own entry j = pos and the pair
// buffer is not used.
// One block of two waves per request: wave 0 the window row, wave 1 the entry.
__global__ void __launch_bounds__(128) k_append(
    int B, const int32_t* __restrict__ pos, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ gc, const uint16_t* __restrict__ wn,
    uint16_t* __restrict__ pair_kc, uint16_t* __restrict__ pair_gc,
    const float* __restrict__ gamma_c, const uint16_t* __restrict__ w_ik,
    const float* __restrict__ gamma_ik, const uint16_t* __restrict__ ki_given,
    const float* __restrict__ rcos, const float* __restrict__ rsin, int64_t rope_rows,
    uint8_t* __restrict__ z_codes, uint8_t* __restrict__ z_scales,
    uint8_t* __restrict__ ki_codes, uint8_t* __restrict__ ki_scales, int64_t entry_stride,
    uint8_t* __restrict__ w_codes, float* __restrict__ w_scale, int cap, int rsh, int zfmt) {
    __shared__ float c_lds[D];
    __shared__ float ki_lds[DI];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int b = blockIdx.x;
    if (b >= B) return;
    const int64_t p = pos[b];
    if (p < 0) return;
    const int64_t row = (int64_t)b * D;
    if (wave == 0) {
        const int64_t prow = p < rope_rows ? p : rope_rows - 1;
        window_row((int64_t)b * cap + (p % cap), prow, lane, wn + row, rcos, rsin, w_codes,
                   w_scale);
    } else if (rsh == 0) {
        if (p >= entry_stride) return;
        const int64_t prow = p < rope_rows ? p : rope_rows - 1;
        compress_entry(b, p, lane, kc + row, nullptr, nullptr, nullptr,
                       w_ik ? nullptr : ki_given + (int64_t)b * DI, gamma_c, w_ik, gamma_ik,
                       rcos + prow * PAIRS, rsin + prow * PAIRS, c_lds, ki_lds, z_codes,
                       z_scales, ki_codes, ki_scales, entry_stride, zfmt);
    } else if ((p & 1) == 0) {
        *(uint4*)(pair_kc + row + 8 * lane) = *(const uint4*)(kc + row + 8 * lane);
        *(uint4*)(pair_gc + row + 8 * lane) = *(const uint4*)(gc + row + 8 * lane);
    } else {
        const int64_t j = p >> 1;
        if (j >= entry_stride) return;
        int64_t prow = 2 * j;
        if (prow >= rope_rows) prow = rope_rows - 1;
        compress_entry(b, j, lane, pair_kc + row, kc + row, pair_gc + row, gc + row,
                       w_ik ? nullptr : ki_given + (int64_t)b * DI, gamma_c, w_ik, gamma_ik,
                       rcos + prow * PAIRS, rsin + prow * PAIRS, c_lds, ki_lds, z_codes,
                       z_scales, ki_codes, ki_scales, entry_stride, zfmt);
    }
}

// FP4 rows: one thread per 32-element block.
__global__ void k_encode_fp4_rows(const uint16_t* __restrict__ x, int64_t rows, int cols,
                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int nb = cols / 32;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= rows * nb) return;
    const int64_t r = g / nb;
    const int blk = (int)(g % nb);
    const uint16_t* src = x + r * cols + 32 * blk;
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 u = *(const uint4*)(src + 8 * q);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) v[8 * q + k] = bf2f((uint16_t)(w[k >> 1] >> ((k & 1) * 16)));
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(v[k]));
    const int e = mx_exponent(amax);
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t wv = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) wv |= e2m1_code(ldexpf(v[8 * q + k], -e)) << (4 * k);
        out[q] = amax > 0.0f ? wv : 0u;
    }
    *(uint4*)(codes + r * (cols / 2) + 16 * blk) = make_uint4(out[0], out[1], out[2], out[3]);
    scales[r * nb + blk] = (uint8_t)(amax > 0.0f ? e + 127 : 0);
}

// Rows in the pages' format (E2M1, one E4M3 scale per 16): one thread per block.
__global__ void k_encode_fp4e4_rows(const uint16_t* __restrict__ x, int64_t rows, int cols,
                                    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int nb = cols / 16;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= rows * nb) return;
    const int64_t r = g / nb;
    const int blk = (int)(g % nb);
    const uint16_t* src = x + r * cols + 16 * blk;
    float v[16];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint4 u = *(const uint4*)(src + 8 * q);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) v[8 * q + k] = bf2f((uint16_t)(w[k >> 1] >> ((k & 1) * 16)));
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(v[k]));
    const uint32_t sc = e4m3_code(div_rn(amax, 6.0f));
    const float sv = e4m3_to_f32(sc);
    uint32_t out[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        uint32_t wv = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) wv |= e2m1_code(div_rn(v[8 * q + k], sv)) << (4 * k);
        out[q] = sv > 0.0f ? wv : 0u;
    }
    *(uint2*)(codes + r * (cols / 2) + 8 * blk) = make_uint2(out[0], out[1]);
    scales[r * nb + blk] = (uint8_t)sc;
}

__global__ void k_decode_fp4e4_rows(const uint8_t* __restrict__ codes,
                                    const uint8_t* __restrict__ scales, int64_t rows, int cols,
                                    uint16_t* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int per = cols / 8;
    if (g >= rows * per) return;
    const int64_t r = g / per;
    const int c8 = (int)(g % per);
    const uint32_t w = *(const uint32_t*)(codes + r * (cols / 2) + 4 * c8);
    const float sv = e4m3_to_f32(scales[r * (cols / 16) + (8 * c8) / 16]);
    const uint4 o = make_uint4(fp4x2_e4_to_bf16x2(w, 0, sv), fp4x2_e4_to_bf16x2(w, 1, sv),
                               fp4x2_e4_to_bf16x2(w, 2, sv), fp4x2_e4_to_bf16x2(w, 3, sv));
    *(uint4*)(out + r * cols + 8 * c8) = o;
}

// FP8 rows: one wave per row (cols <= 1024).
__global__ void __launch_bounds__(256) k_encode_fp8_rows(const uint16_t* __restrict__ x,
                                                         int64_t rows, int cols,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scale) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r >= rows) return;
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int k = lane + 64 * q;
        v[q] = k < cols ? bf2f(x[r * cols + k]) : 0.0f;
        amax = fmaxf(amax, fabsf(v[q]));
    }
#pragma unroll
    for (int s = 1; s <= 32; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
    const float sc = amax > 0.0f ? div_rn(amax, 448.0f) : 1.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int k = lane + 64 * q;
        if (k < cols) codes[r * cols + k] = (uint8_t)(amax > 0.0f ? e4m3_code(div_rn(v[q], sc)) : 0u);
    }
    if (lane == 0) scale[r] = sc;
}

// Decoders (the attention gather's own dequantisation), one thread per 8 elements.
__global__ void k_decode_fp4_rows(const uint8_t* __restrict__ codes,
                                  const uint8_t* __restrict__ scales, int64_t rows, int cols,
                                  uint16_t* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int per = cols / 8;
    if (g >= rows * per) return;
    const int64_t r = g / per;
    const int c8 = (int)(g % per);
    const uint32_t w = *(const uint32_t*)(codes + r * (cols / 2) + 4 * c8);
    const float sc = e8m0_to_f32(scales[r * (cols / 32) + (8 * c8) / 32]);
    uint4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
    *(uint4*)(out + r * cols + 8 * c8) = o;
}

__global__ void k_decode_fp8_rows(const uint8_t* __restrict__ codes, int64_t rows, int cols,
                                  uint16_t* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int per = cols / 8;
    if (g >= rows * per) return;
    const int64_t r = g / per;
    const int c8 = (int)(g % per);
    const uint2 w = *(const uint2*)(codes + r * cols + 8 * c8);
    uint4 o;
    o.x = fp8x2_to_bf16x2<false>(w.x);
    o.y = fp8x2_to_bf16x2<true>(w.x);
    o.z = fp8x2_to_bf16x2<false>(w.y);
    o.w = fp8x2_to_bf16x2<true>(w.y);
    *(uint4*)(out + r * cols + 8 * c8) = o;
}

// n_entries[b] = floor((pos0[b] + T) / ratio), clamped to the cache.
__global__ void k_prefill_entries(int B, int T, const int32_t* __restrict__ pos0,
                                  int64_t entry_stride, int32_t* __restrict__ n_entries, int rsh) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    int64_t n = ((int64_t)pos0[b] + T) >> rsh;
    if (n > entry_stride) n = entry_stride;
    if (n < 0) n = 0;
    n_entries[b] = (int32_t)n;
}

}  // namespace csa2
