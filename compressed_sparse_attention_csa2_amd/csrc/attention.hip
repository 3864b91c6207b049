// Sparse shared-latent attention with a per-head sink.
//
// "DeepSeek V4.1 -- Pooled group -> Source layer, pairs pooled", attention
// equations: J^w_t = {max(0,t-127)..t}; Y = [W; Z]; J = [J^w; I + |W|];
// G_t = Y[J_t]; S_{h,t,i} = Q_{h,t} . G_{t,i} / sqrt(512);
// A = exp S / (exp s_h + sum_j exp S_j); O = sum_i A_i G_i; then
// O_{448:} <- R_t^{-1} O_{448:}.  "Inside DeepSeek V4.1", section "Attention
// that looks at 640 places": 64 query heads share one key-value vector per
// place, and each head has a sink.
//
// One block per (query token, split of its rows); wave w owns heads
// 16w..16w+15.  Rows are processed 32 at a time: the block gathers the rows
// (FP8 window rows from the ring, FP4 entries picked by the indexer),
// dequantises them exactly to bf16 into LDS twice -- row-major for
// S^T = G Q^T (contraction over the 512 channels) and transposed for
// O^T = G^T P^T (contraction over rows) -- and runs bf16 MFMA 16x16x32.
// Window rows enter as their E4M3 codes; their fp32 row scale multiplies the
// logit and is folded into P before the PV product.  The softmax is online in
// fp32; the sink enters the denominator only.  Splits of the row range write
// (m, l, unnormalised O) partials that a combine kernel merges.
#include "csa2_device.h"

namespace csa2 {

constexpr int ATT_ROWS = 32;   // rows per chunk
constexpr int GRM_LD = D + 8;  // row-major LDS stride (bf16)
constexpr int GT_LD = ATT_ROWS + 8;  // transposed LDS stride (bf16)

__device__ __forceinline__ float fast_exp(float x) { return expf(x); }

template <int NW>
__global__ void __launch_bounds__(NW * 64) k_attn(
    int B, int Tq, int H, const int32_t* __restrict__ q_pos0, const uint16_t* __restrict__ Q,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scale, int cap,
    const uint8_t* __restrict__ z_codes, const uint8_t* __restrict__ z_scales,
    int64_t entry_stride, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    const float* __restrict__ sink, const float* __restrict__ rcos,
    const float* __restrict__ rsin, int64_t rope_rows, uint16_t* __restrict__ O,
    float* __restrict__ lse, int nsplit, int rows_per_split, float* __restrict__ part_O,
    float* __restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) uint16_t Grm[ATT_ROWS * GRM_LD];
    __shared__ __attribute__((aligned(16))) uint16_t Gt[D * GT_LD];
    __shared__ float rsc[ATT_ROWS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;
    const int row = blockIdx.x;                // b * Tq + t
    const int split = blockIdx.y;
    const int b = row / Tq, t = row % Tq;
    int64_t p = (int64_t)q_pos0[b] + t;
    if (p < 0) p = 0;
    const int64_t w0 = p - (WINDOW - 1) > 0 ? p - (WINDOW - 1) : 0;
    const int nwin = (int)(p - w0 + 1);
    int c = cnt[row];
    c = c < 0 ? 0 : (c > TOPK ? TOPK : c);
    const int nr = nwin + c;
    const int r_begin = split * rows_per_split;
    const int r_end = (r_begin + rows_per_split < nr) ? r_begin + rows_per_split : nr;

    const int h = wave * 16 + col;   // this lane's head (column of S^T and O^T)
    // Q^T operand: lane holds Q[h][32kk + 8grp .. +7]
    bf8 Qb[16];
    {
        const uint16_t* qrow = Q + (((int64_t)b * H + h) * Tq + t) * D + 8 * grp;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) Qb[kk] = *(const bf8*)(qrow + 32 * kk);
    }
    f4 oacc[32];
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) oacc[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;
    const float inv_sqrt_d = 0.044194173824159216f;   // 1/sqrt(512)
    const int32_t* irow = idx + (int64_t)row * TOPK;
    const int64_t wbase = (int64_t)b * cap;
    const int64_t zbase = (int64_t)b * entry_stride;

    for (int rb = r_begin; rb < r_end; rb += ATT_ROWS) {
        __syncthreads();
        // ---- gather + dequantise 32 rows into both LDS layouts -----------
        for (int item = tid; item < (ATT_ROWS / 2) * 64; item += NW * 64) {
            const int rp = item >> 6, g = item & 63;
            uint4 v[2];
            float scl[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int gr = rb + 2 * rp + q;
                v[q] = make_uint4(0, 0, 0, 0);
                scl[q] = 0.0f;
                if (gr < r_end) {
                    if (gr < nwin) {
                        const int64_t slot = wbase + (w0 + gr) % cap;
                        const uint2 w = *(const uint2*)(w_codes + slot * D + 8 * g);
                        v[q].x = fp8x2_to_bf16x2<false>(w.x);
                        v[q].y = fp8x2_to_bf16x2<true>(w.x);
                        v[q].z = fp8x2_to_bf16x2<false>(w.y);
                        v[q].w = fp8x2_to_bf16x2<true>(w.y);
                        scl[q] = w_scale[slot];
                    } else {
                        int64_t e = irow[gr - nwin];
                        e = e < 0 ? 0 : (e >= entry_stride ? entry_stride - 1 : e);
                        const uint32_t w = *(const uint32_t*)(z_codes + (zbase + e) * 256 + 4 * g);
                        const float sc = e8m0_to_f32(z_scales[(zbase + e) * 16 + (g >> 2)]);
                        v[q].x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
                        v[q].y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
                        v[q].z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
                        v[q].w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
                        scl[q] = 1.0f;
                    }
                }
                *(uint4*)(Grm + (2 * rp + q) * GRM_LD + 8 * g) = v[q];
            }
            const uint32_t a0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
            const uint32_t a1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t lo = (a0[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
                const uint32_t hi = (a1[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
                *(uint32_t*)(Gt + (8 * g + i) * GT_LD + 2 * rp) = lo | (hi << 16);
            }
            if (g == 0) {
                rsc[2 * rp] = scl[0];
                rsc[2 * rp + 1] = scl[1];
            }
        }
        __syncthreads();

        // ---- S^T[r][h] = G[r] . Q[h] ----------------------------------------
        f4 s[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f4 acc = f4{0.f, 0.f, 0.f, 0.f};
            const uint16_t* arow = Grm + (rt * 16 + col) * GRM_LD + 8 * grp;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const bf8 a = *(const bf8*)(arow + 32 * kk);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Qb[kk], acc, 0, 0, 0);
            }
            s[rt] = acc;
        }
        // logits; rows outside the range get -inf
        float pr[8], mx = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rt * 16 + 4 * grp + i;
                const float sc = rsc[r];
                const float x = (rb + r < r_end) ? s[rt][i] * sc * inv_sqrt_d : -INFINITY;
                pr[rt * 4 + i] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        float corr = 1.0f, lsum = 0.0f;
        if (m_new != -INFINITY) {
            corr = fast_exp(m_run - m_new);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                pr[k] = fast_exp(pr[k] - m_new);
                lsum += pr[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) pr[k] = 0.0f;
        }
        lsum += __shfl_xor(lsum, 16, 64);
        lsum += __shfl_xor(lsum, 32, 64);
        l_run = l_run * corr + lsum;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) oacc[dt] *= corr;
        // P^T operand: K slot 8grp+j <-> row (j<4 ? 4grp+j : 16+4grp+j-4); window scale folded in
        bf8 pb;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = (k < 4) ? 4 * grp + k : 16 + 4 * grp + (k - 4);
            pb[k] = (__bf16)(pr[k] * rsc[r]);
        }
        // ---- O^T[d][h] += G^T[d][r] P^T[r][h] ------------------------------
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
            const uint16_t* gt = Gt + (dt * 16 + col) * GT_LD + 4 * grp;
            const uint2 lo = *(const uint2*)gt;
            const uint2 hi = *(const uint2*)(gt + 16);
            const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, av), pb,
                                                             oacc[dt], 0, 0, 0);
        }
    }

    if (nsplit == 1) {
        const float sh = sink[h];
        const float M = fmaxf(m_run, sh);
        const float den = (m_run == -INFINITY ? 0.0f : l_run * fast_exp(m_run - M)) + fast_exp(sh - M);
        const float f = (m_run == -INFINITY ? 0.0f : fast_exp(m_run - M)) / den;
        int64_t prow = p < rope_rows ? p : rope_rows - 1;
        uint16_t* orow = O + (((int64_t)b * H + h) * Tq + t) * D;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
            float o[4] = {oacc[dt][0] * f, oacc[dt][1] * f, oacc[dt][2] * f, oacc[dt][3] * f};
            const int d0 = dt * 16 + 4 * grp;
            if (d0 >= ROPE_LO) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int pi = (d0 - ROPE_LO) / 2 + q;
                    const float co = rcos[prow * PAIRS + pi], si = rsin[prow * PAIRS + pi];
                    const float x0 = o[2 * q], x1 = o[2 * q + 1];
                    o[2 * q] = x0 * co + x1 * si;
                    o[2 * q + 1] = x1 * co - x0 * si;
                }
            }
            const uint32_t w0v = (uint32_t)f2bf(o[0]) | ((uint32_t)f2bf(o[1]) << 16);
            const uint32_t w1v = (uint32_t)f2bf(o[2]) | ((uint32_t)f2bf(o[3]) << 16);
            *(uint2*)(orow + d0) = make_uint2(w0v, w1v);
        }
        if (lse && grp == 0) lse[((int64_t)b * H + h) * Tq + t] = M + logf(den);
    } else {
        const int64_t pbase = ((int64_t)row * nsplit + split) * H + h;
        float* po = part_O + pbase * D;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) *(f4*)(po + dt * 16 + 4 * grp) = oacc[dt];
        if (grp == 0) {
            part_ml[pbase * 2] = m_run;
            part_ml[pbase * 2 + 1] = l_run;
        }
    }
}

// Merge split partials: one wave per (token, head), lane owns channels 8l..8l+7.
__global__ void __launch_bounds__(256) k_attn_combine(
    int B, int Tq, int H, const int32_t* __restrict__ q_pos0, const float* __restrict__ sink,
    const float* __restrict__ rcos, const float* __restrict__ rsin, int64_t rope_rows,
    int nsplit, const float* __restrict__ part_O, const float* __restrict__ part_ml,
    uint16_t* __restrict__ O, float* __restrict__ lse) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    if (item >= (int64_t)B * Tq * H) return;
    const int h = (int)(item % H);
    const int64_t row = item / H;
    const int b = (int)(row / Tq), t = (int)(row % Tq);
    const float sh = sink[h];
    float M = sh;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((row * nsplit + s) * H + h) * 2]);
    float den = fast_exp(sh - M);
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s = 0; s < nsplit; ++s) {
        const int64_t pb = (row * nsplit + s) * H + h;
        const float m = part_ml[pb * 2], l = part_ml[pb * 2 + 1];
        if (m == -INFINITY) continue;
        const float f = fast_exp(m - M);
        den += l * f;
        const float4 a = *(const float4*)(part_O + pb * D + 8 * lane);
        const float4 c = *(const float4*)(part_O + pb * D + 8 * lane + 4);
        o[0] += a.x * f; o[1] += a.y * f; o[2] += a.z * f; o[3] += a.w * f;
        o[4] += c.x * f; o[5] += c.y * f; o[6] += c.z * f; o[7] += c.w * f;
    }
    const float inv = 1.0f / den;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= inv;
    int64_t p = (int64_t)q_pos0[b] + t;
    if (p < 0) p = 0;
    const int64_t prow = p < rope_rows ? p : rope_rows - 1;
    if (8 * lane >= ROPE_LO) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int pi = (8 * lane - ROPE_LO) / 2 + q;
            const float co = rcos[prow * PAIRS + pi], si = rsin[prow * PAIRS + pi];
            const float x0 = o[2 * q], x1 = o[2 * q + 1];
            o[2 * q] = x0 * co + x1 * si;
            o[2 * q + 1] = x1 * co - x0 * si;
        }
    }
    uint4 w;
    w.x = (uint32_t)f2bf(o[0]) | ((uint32_t)f2bf(o[1]) << 16);
    w.y = (uint32_t)f2bf(o[2]) | ((uint32_t)f2bf(o[3]) << 16);
    w.z = (uint32_t)f2bf(o[4]) | ((uint32_t)f2bf(o[5]) << 16);
    w.w = (uint32_t)f2bf(o[6]) | ((uint32_t)f2bf(o[7]) << 16);
    *(uint4*)(O + (((int64_t)b * H + h) * Tq + t) * D + 8 * lane) = w;
    if (lse && lane == 0) lse[((int64_t)b * H + h) * Tq + t] = M + logf(den);
}

template __global__ void k_attn<1>(int, int, int, const int32_t*, const uint16_t*, const uint8_t*,
                                   const float*, int, const uint8_t*, const uint8_t*, int64_t,
                                   const int32_t*, const int32_t*, const float*, const float*,
                                   const float*, int64_t, uint16_t*, float*, int, int, float*,
                                   float*);
template __global__ void k_attn<2>(int, int, int, const int32_t*, const uint16_t*, const uint8_t*,
                                   const float*, int, const uint8_t*, const uint8_t*, int64_t,
                                   const int32_t*, const int32_t*, const float*, const float*,
                                   const float*, int64_t, uint16_t*, float*, int, int, float*,
                                   float*);
template __global__ void k_attn<3>(int, int, int, const int32_t*, const uint16_t*, const uint8_t*,
                                   const float*, int, const uint8_t*, const uint8_t*, int64_t,
                                   const int32_t*, const int32_t*, const float*, const float*,
                                   const float*, int64_t, uint16_t*, float*, int, int, float*,
                                   float*);
template __global__ void k_attn<4>(int, int, int, const int32_t*, const uint16_t*, const uint8_t*,
                                   const float*, int, const uint8_t*, const uint8_t*, int64_t,
                                   const int32_t*, const int32_t*, const float*, const float*,
                                   const float*, int64_t, uint16_t*, float*, int, int, float*,
                                   float*);

}  // namespace csa2
