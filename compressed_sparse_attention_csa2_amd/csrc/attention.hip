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

constexpr int ATT_ROWS = 32;          // rows per chunk

__device__ __forceinline__ float fast_exp(float x) { return expf(x); }
constexpr int GT_LD = ATT_ROWS + 4;   // transposed LDS stride (bf16): 18 dwords

// Row-major copy: row r holds its 64 chunks of 8 channels; chunk c is stored at
// position c ^ (r & 15).  The 64 lanes writing one row and the 16 lanes reading
// one chunk of 16 rows both touch distinct banks.
__device__ __forceinline__ int grm_index(int r, int chunk) {
    return r * D + ((chunk ^ (r & 15)) << 3);
}

// Transposed copy: channel d holds its 32 rows in 8 units of 4 rows (8 bytes);
// unit u is stored at position u ^ ((d >> 5) & 7).  Writers (64 lanes on 64
// consecutive 8-channel groups, one row pair) hit distinct banks, and readers
// (16 consecutive channels, one unit) still read 8 contiguous bytes.
__device__ __forceinline__ int gt_index(int d, int r) {
    return d * GT_LD + ((((r >> 2) ^ (d >> 5)) & 7) << 2) + (r & 3);
}

// Raw codes of one 8-channel segment of a row, in flight from global memory.
struct RowSeg {
    uint2 code;     // 8 FP8 codes, or 8 FP4 codes in .x
    float scale;    // FP4 block scale as an fp32 power of two (unused for FP8 rows)
};

constexpr float LOG2E = 1.4426950408889634f;

template <int HG>
__global__ void __launch_bounds__(HG * 128, 2) k_attn(
    int B, int Tq, int H, const int32_t* __restrict__ q_pos0, const uint16_t* __restrict__ Q,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scale, int cap,
    const uint8_t* __restrict__ z_codes, const uint8_t* __restrict__ z_scales,
    int64_t entry_stride, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    const float* __restrict__ sink, const float* __restrict__ rcos,
    const float* __restrict__ rsin, int64_t rope_rows, uint16_t* __restrict__ O,
    float* __restrict__ lse, int nsplit, int rows_per_split, float* __restrict__ part_O,
    float* __restrict__ part_ml) {
    constexpr int NT = HG * 128;                  // threads (2 waves per head group)
    constexpr int NWAVE = NT / 64;
    constexpr int RPW = ATT_ROWS / NWAVE;         // rows gathered per wave per chunk
    __shared__ __attribute__((aligned(16))) uint16_t Grm[ATT_ROWS * D];
    __shared__ __attribute__((aligned(16))) uint16_t Gt[D * GT_LD];
    __shared__ float Sx[HG * 2 * 4 * 64];
    __shared__ float rsc[ATT_ROWS];
    __shared__ int32_t sidx[TOPK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int hg = wave >> 1, half = wave & 1;
    const int row = blockIdx.x;                // b * Tq + t
    const int split = blockIdx.y;
    const int b = row / Tq, t = row - b * Tq;
    int64_t p = (int64_t)q_pos0[b] + t;
    if (p < 0) p = 0;
    const int64_t w0 = p - (WINDOW - 1) > 0 ? p - (WINDOW - 1) : 0;
    const int nwin = (int)(p - w0 + 1);
    const int slot0 = (int)(w0 % cap);         // ring slot of the first window row
    int c = cnt[row];
    c = c < 0 ? 0 : (c > TOPK ? TOPK : c);
    const int nr = nwin + c;
    const int r_begin = split * rows_per_split;
    const int r_end = (r_begin + rows_per_split < nr) ? r_begin + rows_per_split : nr;
    const uint8_t* wrow0 = w_codes + (int64_t)b * cap * D;
    const float* wsc = w_scale + (int64_t)b * cap;
    const uint8_t* zc0 = z_codes + (int64_t)b * entry_stride * 256;
    const uint8_t* zs0 = z_scales + (int64_t)b * entry_stride * 16;

    {   // the row's selected entries, clamped into the cache
        const int32_t* irow = idx + (int64_t)row * TOPK;
        const int emax = entry_stride < 0x7FFFFFFF ? (int)entry_stride - 1 : 0x7FFFFFFE;
        for (int i = tid; i < c; i += NT) {
            const int e = irow[i];
            sidx[i] = e < 0 ? 0 : (e > emax ? emax : e);
        }
    }

    const int h = hg * 16 + col;   // this lane's head (column of S^T and O^T)
    bf8 Qb[16];                    // Q^T operand: lane holds Q[h][32kk + 8grp .. +7]
    {
        const uint16_t* qrow = Q + (((int64_t)b * H + h) * Tq + t) * D + 8 * grp;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) Qb[kk] = *(const bf8*)(qrow + 32 * kk);
    }
    f4 oacc[16];                   // O^T for channels 256*half + 16*dt + 4*grp + i
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) oacc[dt] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;       // running max (log2 units) and sum
    const float lscale = 0.044194173824159216f * LOG2E;   // log2(e) / sqrt(512)
    __syncthreads();                              // sidx ready

    // Wave `wave` gathers rows wave + NWAVE*k of each chunk; lane owns channels 8*lane..+7.
    auto fetch = [&](int rb, RowSeg (&seg)[RPW], float (&wsr)[RPW]) {
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            const int gr = rb + wave + NWAVE * k;          // wave-uniform
            seg[k].code = make_uint2(0, 0);
            seg[k].scale = 0.0f;
            wsr[k] = 0.0f;
            if (gr < r_end) {
                if (gr < nwin) {
                    int slot = slot0 + gr;
                    if (slot >= cap) slot -= cap;
                    seg[k].code = *(const uint2*)(wrow0 + (int64_t)slot * D + 8 * lane);
                    wsr[k] = wsc[slot];
                } else {
                    const int e = __builtin_amdgcn_readfirstlane(sidx[gr - nwin]);
                    seg[k].code.x = *(const uint32_t*)(zc0 + (int64_t)e * 256 + 4 * lane);
                    seg[k].scale = e8m0_to_f32(zs0[(int64_t)e * 16 + (lane >> 2)]);
                    wsr[k] = 1.0f;
                }
            }
        }
    };

    RowSeg seg[RPW];
    float wsr[RPW];
    if (r_begin < r_end) fetch(r_begin, seg, wsr);

    for (int rb = r_begin; rb < r_end; rb += ATT_ROWS) {
        __syncthreads();   // previous chunk's readers are done with Grm, Gt, rsc, Sx
        // ---- dequantise this wave's rows into both LDS layouts -------------
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            const int r = wave + NWAVE * k;
            const int gr = rb + r;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (gr < r_end) {
                if (gr < nwin) {
                    v.x = fp8x2_to_bf16x2<false>(seg[k].code.x);
                    v.y = fp8x2_to_bf16x2<true>(seg[k].code.x);
                    v.z = fp8x2_to_bf16x2<false>(seg[k].code.y);
                    v.w = fp8x2_to_bf16x2<true>(seg[k].code.y);
                } else {
                    const uint32_t w = seg[k].code.x;
                    const float sc = seg[k].scale;
                    v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
                    v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
                    v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
                    v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
                }
            }
            *(uint4*)(Grm + grm_index(r, lane)) = v;
            // transposed copy: channel 8*lane + i, row r (16-bit stores)
            uint16_t* gt = Gt + gt_index(8 * lane, r);
            const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) gt[i * GT_LD] = (uint16_t)(vw[i >> 1] >> ((i & 1) * 16));
            if (lane == 0) rsc[r] = wsr[k];
        }
        __syncthreads();
        // ---- next chunk's codes are loaded while this one is computed ------
        if (rb + ATT_ROWS < r_end) fetch(rb + ATT_ROWS, seg, wsr);

        // ---- S^T for this wave's 16 rows: rows 16*half + 4*grp + i ----------
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
        {
            const int r = half * 16 + col;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const bf8 a = *(const bf8*)(Grm + grm_index(r, 4 * kk + grp));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Qb[kk], acc, 0, 0, 0);
            }
        }
        float* sx = Sx + ((hg * 2 + half) * 4) * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = half * 16 + 4 * grp + i;
            sx[i * 64 + lane] = (rb + r < r_end) ? acc[i] * (rsc[r] * lscale) : -INFINITY;
        }
        __syncthreads();
        // logits (log2 units) of all 32 rows, identical in both waves of the pair
        float pr[8];
        {
            const float* s0 = Sx + ((hg * 2 + 0) * 4) * 64;
            const float* s1 = Sx + ((hg * 2 + 1) * 4) * 64;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pr[i] = s0[i * 64 + lane];
                pr[4 + i] = s1[i * 64 + lane];
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(pr[0], pr[1]), fmaxf(pr[2], pr[3])),
                         fmaxf(fmaxf(pr[4], pr[5]), fmaxf(pr[6], pr[7])));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        float corr = 1.0f, lsum = 0.0f;
        if (m_new != -INFINITY) {
            corr = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                pr[k] = __builtin_amdgcn_exp2f(pr[k] - m_new);
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
        if (__any(corr != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) oacc[dt] *= corr;
        }
        // P^T operand: K slot 8grp+j <-> row (j<4 ? 4grp+j : 16+4grp+j-4); window scale folded in
        bf8 pb;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = (k < 4) ? 4 * grp + k : 16 + 4 * grp + (k - 4);
            pb[k] = (__bf16)(pr[k] * rsc[r]);
        }
        // ---- O^T[d][h] += G^T[d][r] P^T[r][h] for this wave's 256 channels ---
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
            const int d = (half * 16 + dt) * 16 + col;
            const uint2 lo = *(const uint2*)(Gt + gt_index(d, 4 * grp));
            const uint2 hi = *(const uint2*)(Gt + gt_index(d, 16 + 4 * grp));
            const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, av), pb,
                                                             oacc[dt], 0, 0, 0);
        }
    }

    if (nsplit == 1) {
        const float sh = sink[h] * LOG2E;
        const float M = fmaxf(m_run, sh);
        const float em = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
        const float den = l_run * em + __builtin_amdgcn_exp2f(sh - M);
        const float f = em / den;
        const int64_t prow = p < rope_rows ? p : rope_rows - 1;
        uint16_t* orow = O + (((int64_t)b * H + h) * Tq + t) * D;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
            float o[4] = {oacc[dt][0] * f, oacc[dt][1] * f, oacc[dt][2] * f, oacc[dt][3] * f};
            const int d0 = (half * 16 + dt) * 16 + 4 * grp;
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
        if (lse && half == 0 && grp == 0)
            lse[((int64_t)b * H + h) * Tq + t] = (M + log2f(den)) * 0.6931471805599453f;
    } else {
        const int64_t pbase = ((int64_t)row * nsplit + split) * H + h;
        float* po = part_O + pbase * D;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) *(f4*)(po + (half * 16 + dt) * 16 + 4 * grp) = oacc[dt];
        if (half == 0 && grp == 0) {
            part_ml[pbase * 2] = m_run;          // log2 units
            part_ml[pbase * 2 + 1] = l_run;
        }
    }
}

// Merge split partials: one wave per (token, head), lane owns channels 8l..8l+7.
// Partial maxima are in log2 units (logits scaled by log2 e).
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
    const float sh = sink[h] * LOG2E;
    float M = sh;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((row * nsplit + s) * H + h) * 2]);
    float den = __builtin_amdgcn_exp2f(sh - M);
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s = 0; s < nsplit; ++s) {
        const int64_t pb = (row * nsplit + s) * H + h;
        const float m = part_ml[pb * 2], l = part_ml[pb * 2 + 1];
        if (m == -INFINITY) continue;
        const float f = __builtin_amdgcn_exp2f(m - M);
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
    if (lse && lane == 0) lse[((int64_t)b * H + h) * Tq + t] = (M + log2f(den)) * 0.6931471805599453f;
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
