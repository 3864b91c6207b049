// Lightning indexer and causal top-512.
//
// "DeepSeek V4.1 -- Pooled group -> Source layer, pairs pooled", indexer
// equations: S^I_{t,j} = sum_h w^I_{t,h} ReLU(Q^I_{h,t} . K^I_j) over 32 heads
// of 128 channels, and I_t = top_512(S^I_{t,j} : j < floor((t+1)/2)).
// "Inside DeepSeek V4.1", section "Attention that looks at 640 places": the
// indexer scores every entry and keeps the top 512.
//
// Queries are quantised per (token, head) row to E4M3FN (scale max|x|/448);
// keys stay in their FP4 storage.  The dot products run on gfx950's block-
// scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4: A = FP8 queries with unit
// scale, B = FP4 keys with their E8M0 block scales), accumulating in fp32.
// The query scale is folded into the head weight (it is positive, so it
// commutes with the ReLU): S = sum_h (w_h * sq_h) * max(d_h, 0).
//
// Operand layout of the FP8 x FP4 form (measured on gfx950): B lane l holds
// entry l%16, channels 32(l/16)..32(l/16)+31 (16 bytes) and that block's scale;
// A lane l holds head l%16, channels 16(l/16)..+15 followed by 64+16(l/16)..+15.
// The result lane l holds entry l%16 for heads 4(l/16)..4(l/16)+3.
//
// Tile shapes: one MFMA covers 16 heads of one token x 16 entries x 128
// channels.  A wave holds TOK tokens (2 MFMA rows each) and walks a chunk of
// entries 16 at a time; lane l of the result holds entry l%16 and heads
// 4(l/16)..4(l/16)+3, so the head sum is 8 in-lane fmas and two cross-lane adds.
#include "csa2_device.h"

namespace csa2 {

// q^I [rows][128] bf16 -> E4M3FN codes [rows][128] and wq[row] = w[row] * scale.
// One wave per (token, head) row.
__global__ void __launch_bounds__(256) k_quant_index_query(const uint16_t* __restrict__ qI,
                                                           const float* __restrict__ wI,
                                                           int64_t rows,
                                                           uint8_t* __restrict__ q8,
                                                           float* __restrict__ wq) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r >= rows) return;
    const uint32_t v = *(const uint32_t*)(qI + r * DI + 2 * lane);
    const float x0 = bf2f((uint16_t)v), x1 = bf2f((uint16_t)(v >> 16));
    float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int s = 1; s <= 32; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
    const float sc = amax > 0.0f ? div_rn(amax, 448.0f) : 1.0f;
    uint32_t c = 0;
    if (amax > 0.0f) c = e4m3_code(div_rn(x0, sc)) | (e4m3_code(div_rn(x1, sc)) << 8);
    *(uint16_t*)(q8 + r * DI + 2 * lane) = (uint16_t)c;
    if (lane == 0) wq[r] = wI[r] * sc;
}

constexpr int IDX_CHUNK = 1024;   // entries per wave

__device__ __forceinline__ int64_t cand_count(int32_t qpos0, int t, int32_t n_ent,
                                              int64_t stride) {
    int64_t n = ((int64_t)qpos0 + t + 1) / 2;
    int64_t cap = n_ent < 0 ? 0 : (int64_t)n_ent;
    if (cap > stride) cap = stride;
    return n < cap ? (n < 0 ? 0 : n) : cap;
}

// Scores S[(b*Tq + t)][j] for j < n(t).  One wave per (request, TOK tokens,
// chunk of IDX_CHUNK entries); work items are ordered heaviest tokens first.
template <int TOK>
__global__ void __launch_bounds__(256) k_index_scores(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const uint8_t* __restrict__ q8, const float* __restrict__ wq,
    const uint8_t* __restrict__ ki_codes, const uint8_t* __restrict__ ki_scales,
    int64_t entry_stride, float* __restrict__ S, int n_tg, int n_ch) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    if (item >= (int64_t)B * n_tg * n_ch) return;
    const int ch = (int)(item % n_ch);
    const int tg = n_tg - 1 - (int)((item / n_ch) % n_tg);
    const int b = (int)(item / ((int64_t)n_ch * n_tg));
    const int t0 = tg * TOK;
    const int32_t qp = q_pos0[b], ne = n_entries[b];
    const int tlast = (t0 + TOK - 1 < Tq) ? t0 + TOK - 1 : Tq - 1;
    const int64_t n_max = cand_count(qp, tlast, ne, entry_stride);
    const int64_t j_begin = (int64_t)ch * IDX_CHUNK;
    if (j_begin >= n_max) return;
    const int64_t j_end = (j_begin + IDX_CHUNK < n_max) ? j_begin + IDX_CHUNK : n_max;

    const int col = lane & 15, grp = lane >> 4;
    i8 A[TOK][2];
    f4 W[TOK][2];
    int64_t ncand[TOK];
#pragma unroll
    for (int k = 0; k < TOK; ++k) {
        const int t = t0 + k;
        const bool ok = t < Tq;
        ncand[k] = ok ? cand_count(qp, t, ne, entry_stride) : 0;
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            const int64_t row = ((int64_t)b * Tq + (ok ? t : 0)) * HI + tile * 16;
            // FP8 A against an FP4 B operand: lane group g's 32 bytes meet the keys'
            // channels 16g..16g+15 and 64+16g..64+16g+15 (each B lane holds one
            // 32-channel block of its entry with that block's own E8M0 scale).
            const uint8_t* src = q8 + (row + col) * DI + 16 * grp;
            const uint4 u0 = *(const uint4*)src, u1 = *(const uint4*)(src + 64);
            A[k][tile] = ok ? i8{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                                 (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w}
                            : i8{0, 0, 0, 0, 0, 0, 0, 0};
            const float4 w4 = *(const float4*)(wq + row + 4 * grp);
            W[k][tile] = ok ? f4{w4.x, w4.y, w4.z, w4.w} : f4{0.f, 0.f, 0.f, 0.f};
        }
    }
    const int64_t ebase = (int64_t)b * entry_stride;
    for (int64_t jt = j_begin; jt < j_end; jt += 16) {
        int64_t j = jt + col;
        const bool jok = j < j_end;
        if (!jok) j = j_end - 1;
        const uint4 kc = *(const uint4*)(ki_codes + (ebase + j) * 64 + 16 * grp);
        const uint32_t sw = *(const uint32_t*)(ki_scales + (ebase + j) * 4);
        const int sc = (int)((sw >> (8 * grp)) & 0xFFu);
        const i8 Bv = i8{(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
        float s[TOK];
#pragma unroll
        for (int k = 0; k < TOK; ++k) {
            f4 d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A[k][0], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
            f4 d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A[k][1], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[k][0][i], fmaxf(d0[i], 0.0f), acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[k][1][i], fmaxf(d1[i], 0.0f), acc);
            s[k] = acc;
        }
#pragma unroll
        for (int k = 0; k < TOK; ++k) {
            s[k] += __shfl_xor(s[k], 16, 64);
            s[k] += __shfl_xor(s[k], 32, 64);
        }
        // lane group g writes tokens g, g+4, ...
#pragma unroll
        for (int k = 0; k < TOK; ++k) {
            if ((k & 3) == grp && jok && j < ncand[k])
                S[((int64_t)b * Tq + t0 + k) * entry_stride + j] = s[k];
        }
    }
}

// ---------------------------------------------------------------------------
// Top-512 by radix select over order-preserving 32-bit keys, one block of 256
// threads per query token.  Ties: larger score, then smaller entry index.
// Output: selected entries in ascending order, padded with -1; count.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float f) {
    f = f + 0.0f;   // -0 -> +0 so equal scores compare equal
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive block scan of one value per thread (256 threads); returns prefix, total in *tot
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* lds4, uint32_t* tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = v;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const uint32_t o = __shfl_up(inc, s, 64);
        if (lane >= s) inc += o;
    }
    if (lane == 63) lds4[wave] = inc;
    __syncthreads();
    uint32_t base = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t x = lds4[w];
        if (w < wave) base += x;
        all += x;
    }
    __syncthreads();
    *tot = all;
    return base + inc - v;
}

__global__ void __launch_bounds__(256) k_topk(int B, int Tq, const int32_t* __restrict__ q_pos0,
                                              const int32_t* __restrict__ n_entries,
                                              const float* __restrict__ S, int64_t entry_stride,
                                              int32_t* __restrict__ idx,
                                              int32_t* __restrict__ cnt) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sel_digit, sel_above, lds4[4];
    const int row = blockIdx.x;
    const int b = row / Tq, t = row % Tq;
    const int tid = threadIdx.x;
    const int64_t n = cand_count(q_pos0[b], t, n_entries[b], entry_stride);
    int32_t* out = idx + (int64_t)row * TOPK;
    if (n <= TOPK) {
        for (int i = tid; i < TOPK; i += 256) out[i] = i < n ? i : -1;
        if (tid == 0) cnt[row] = (int32_t)n;
        return;
    }
    const float* s = S + (int64_t)row * entry_stride;
    uint32_t prefix = 0, pmask = 0, krem = TOPK;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        for (int64_t j = tid; j < n; j += 256) {
            const uint32_t key = score_key(s[j]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l owns digits 255-4l .. 252-4l (descending)
            uint32_t h[4], loc = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) { h[q] = hist[255 - 4 * tid - q]; loc += h[q]; }
            uint32_t inc = loc;
#pragma unroll
            for (int sft = 1; sft < 64; sft <<= 1) {
                const uint32_t o = __shfl_up(inc, sft, 64);
                if (tid >= sft) inc += o;
            }
            uint32_t above = inc - loc;   // count in strictly higher digits
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (above < krem && krem <= above + h[q]) {
                    sel_digit = 255 - 4 * tid - q;
                    sel_above = above;
                }
                above += h[q];
            }
        }
        __syncthreads();
        prefix |= sel_digit << shift;
        pmask |= 255u << shift;
        krem -= sel_above;
        __syncthreads();
    }
    // prefix is the key of the 512th element; take all larger keys and the
    // first krem equal keys in index order, writing in index order.
    const uint32_t kth = prefix;
    uint32_t eq_base = 0, sel_base = 0;
    for (int64_t j0 = 0; j0 < n; j0 += 256 * 4) {
        uint32_t keys[4];
        uint32_t neq = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t j = j0 + 4 * tid + q;
            keys[q] = j < n ? score_key(s[j]) : 0u;
            neq += (j < n && keys[q] == kth) ? 1u : 0u;
        }
        uint32_t eq_tot;
        uint32_t eq_rank = eq_base + block_excl_scan(neq, lds4, &eq_tot);
        uint32_t sel[4], nsel = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t j = j0 + 4 * tid + q;
            bool take = false;
            if (j < n) {
                if (keys[q] > kth) take = true;
                else if (keys[q] == kth) { take = eq_rank < krem; ++eq_rank; }
            }
            sel[q] = take;
            nsel += take;
        }
        uint32_t sel_tot;
        uint32_t pos = sel_base + block_excl_scan(nsel, lds4, &sel_tot);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (sel[q] && pos < TOPK) out[pos] = (int32_t)(j0 + 4 * tid + q);
            pos += sel[q];
        }
        eq_base += eq_tot;
        sel_base += sel_tot;
    }
    if (tid == 0) cnt[row] = TOPK;
}

template __global__ void k_index_scores<1>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                           const float*, const uint8_t*, const uint8_t*, int64_t,
                                           float*, int, int);
template __global__ void k_index_scores<4>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                           const float*, const uint8_t*, const uint8_t*, int64_t,
                                           float*, int, int);
template __global__ void k_index_scores<8>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                           const float*, const uint8_t*, const uint8_t*, int64_t,
                                           float*, int, int);

}  // namespace csa2
