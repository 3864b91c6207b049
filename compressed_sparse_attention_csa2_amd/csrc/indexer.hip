// Lightning indexer and causal top-512.
//
// "DeepSeek V4.1 -- Pooled group -> Source layer, pairs pooled", indexer
// equations: S^I_{t,j} = sum_h w^I_{t,h} ReLU(Q^I_{h,t} . K^I_j) over 32 heads
// of 128 channels, and I_t = top_512(S^I_{t,j} : j < floor((t+1)/2)).
// "Inside DeepSeek V4.1", section "Attention that looks at 640 places": all
// compressed entries are scored; 512 of them go on to the main attention.
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


__device__ __forceinline__ int64_t cand_count(int32_t qpos0, int t, int32_t n_ent,
                                              int64_t stride) {
    int64_t n = ((int64_t)qpos0 + t + 1) / 2;
    int64_t cap = n_ent < 0 ? 0 : (int64_t)n_ent;
    if (cap > stride) cap = stride;
    return n < cap ? (n < 0 ? 0 : n) : cap;
}

// max(x, 0) as one integer max on the bit pattern: every negative float
// (including -0) is a negative integer.
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// Sum over the four 16-lane rows, scattered: after the call lane row g holds
// the total of token slot g (slots: a, b, c, d).  Built from the gfx950 lane
// swaps: permlane32 exchanges the upper half of its first operand with the
// lower half of its second, permlane16 the odd rows of the first with the even
// rows of the second.
__device__ __forceinline__ float rowsum_scatter4(float a, float b, float c, float d) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(c), false, false);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(b), __float_as_uint(d), false, false);
    const float u0 = __uint_as_float(p[0]) + __uint_as_float(p[1]);   // rows: a(0+2), a(1+3) | c ...
    const float u1 = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(u0), __float_as_uint(u1), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scores S[(b*Tq + t)][j] for j < n(t).  One wave per (request, TOK tokens,
// chunk of IDX_CHUNK entries); work items are ordered heaviest tokens first.
// The next 16 entries' codes and scales are loaded while the current ones are
// multiplied.
template <int TOK>
__global__ void __launch_bounds__(256) k_index_scores(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const uint8_t* __restrict__ q8, const float* __restrict__ wq,
    const uint8_t* __restrict__ ki_codes, const uint8_t* __restrict__ ki_scales,
    int64_t entry_stride, float* __restrict__ S, int n_tg, int n_ch) {
    static_assert(TOK == 1 || TOK % 4 == 0, "token slots per wave");
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
    const int j_len = (int)((j_begin + IDX_CHUNK < n_max) ? IDX_CHUNK : n_max - j_begin);

    const int col = lane & 15, grp = lane >> 4;
    i8 A[TOK][2];
    f4 W[TOK][2];
    int ncand[TOK];                 // candidates of each token within this chunk
#pragma unroll
    for (int k = 0; k < TOK; ++k) {
        const int t = t0 + k;
        const bool ok = t < Tq;
        const int64_t nk = ok ? cand_count(qp, t, ne, entry_stride) - j_begin : 0;
        ncand[k] = nk < 0 ? 0 : (int)nk;
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
    const uint8_t* kbase = ki_codes + ((int64_t)b * entry_stride + j_begin) * 64 + 16 * grp;
    const uint8_t* sbase = ki_scales + ((int64_t)b * entry_stride + j_begin) * 4;
    float* Sbase = S + ((int64_t)b * Tq + t0) * entry_stride + j_begin;

    auto load = [&](int jt, uint4& kc, uint32_t& sw) {
        int j = jt + col;
        j = j < j_len ? j : j_len - 1;
        kc = *(const uint4*)(kbase + (int64_t)j * 64);
        sw = *(const uint32_t*)(sbase + (int64_t)j * 4);
    };
    uint4 kc_n;
    uint32_t sw_n;
    load(0, kc_n, sw_n);
#pragma unroll 2
    for (int jt = 0; jt < j_len; jt += 16) {
        const uint4 kc = kc_n;
        const uint32_t sw = sw_n;
        if (jt + 16 < j_len) load(jt + 16, kc_n, sw_n);
        const int sc = (int)((sw >> (8 * grp)) & 0xFFu);
        const i8 Bv = i8{(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
        float s[TOK];
#pragma unroll
        for (int k = 0; k < TOK; ++k) {
            const f4 d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A[k][0], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
            const f4 d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A[k][1], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[k][0][i], relu(d0[i]), acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[k][1][i], relu(d1[i]), acc);
            s[k] = acc;
        }
        const int j = jt + col;
        if (TOK == 1) {
            const float tot = rowsum_scatter4(s[0], s[0], s[0], s[0]);
            if (grp == 0 && j < ncand[0]) Sbase[j] = tot;
        } else {
#pragma unroll
            for (int k4 = 0; k4 < TOK; k4 += 4) {
                const float tot = rowsum_scatter4(s[k4], s[k4 + 1 < TOK ? k4 + 1 : k4],
                                                  s[k4 + 2 < TOK ? k4 + 2 : k4],
                                                  s[k4 + 3 < TOK ? k4 + 3 : k4]);
                // lane row g holds token k4 + g
                int nc = ncand[k4];
#pragma unroll
                for (int g = 1; g < 4; ++g)
                    if (grp == g) nc = ncand[k4 + g < TOK ? k4 + g : k4];
                if (j < nc) Sbase[(int64_t)(k4 + grp) * entry_stride + j] = tot;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Top-512 selection.  Keys are the scores mapped to order-preserving u32 (-0
// first turned into +0 so equal scores compare equal).  Ties: larger score,
// then smaller entry index; output in ascending entry order, padded with -1.
//
// One block of 256 threads per list (a query row, or the merged candidates of
// a long row's segments):
//  1. theta = the 512th largest key of a strided sample (at most SAMPLE keys)
//     of the list -- a lower bound of the list's 512th largest key;
//  2. one pass compacts every element with key >= theta, in list order, into
//     LDS (at most CAND);
//  3. radix select of the 512th largest key among those, then an ordered
//     compaction of the winners.
// When more than CAND elements reach theta (large exact ties) the block falls
// back to radix passes over the list in global memory.  Lists longer than
// TOPK_SEG are cut into segments whose top-512 are merged by a second launch.
// ---------------------------------------------------------------------------
constexpr int TK_THREADS = 256;
constexpr int TK_SAMPLE = 8192;
constexpr int TK_CAND = 4096;
constexpr int TOPK_SEG = 32768;

__device__ __forceinline__ uint32_t score_key(float f) {
    f = f + 0.0f;   // -0 -> +0 so equal scores compare equal
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive block scan of one value per thread; returns prefix, total in *tot
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
    for (int w = 0; w < TK_THREADS / 64; ++w) {
        const uint32_t x = lds4[w];
        if (w < wave) base += x;
        all += x;
    }
    __syncthreads();
    *tot = all;
    return base + inc - v;
}

struct TopkShared {
    uint32_t hist[256];
    uint32_t lds4[TK_THREADS / 64];
    uint32_t sel_digit, sel_above;
    uint32_t keys[TK_SAMPLE];       // sample keys, then candidate keys
    int32_t cj[TK_CAND];            // candidate list positions
};

// After histogramming the current digit, pick the digit holding the k-th largest.
__device__ __forceinline__ void pick_digit(TopkShared& sh, uint32_t krem) {
    const int tid = threadIdx.x;
    if (tid < 64) {
        uint32_t h[4], loc = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { h[q] = sh.hist[255 - 4 * tid - q]; loc += h[q]; }
        uint32_t inc = loc;
#pragma unroll
        for (int sft = 1; sft < 64; sft <<= 1) {
            const uint32_t o = __shfl_up(inc, sft, 64);
            if (tid >= sft) inc += o;
        }
        uint32_t above = inc - loc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (above < krem && krem <= above + h[q]) {
                sh.sel_digit = 255 - 4 * tid - q;
                sh.sel_above = above;
            }
            above += h[q];
        }
    }
}

// k-th largest key (1-based k <= n) of n keys given by get(i); returns the key,
// *krem = how many elements equal to it belong to the top k.
template <typename Get>
__device__ uint32_t radix_kth(TopkShared& sh, int n, uint32_t k, Get get, uint32_t* krem_out) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0, krem = k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        sh.hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += TK_THREADS) {
            const uint32_t key = get(i);
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        pick_digit(sh, krem);
        __syncthreads();
        prefix |= sh.sel_digit << shift;
        pmask |= 255u << shift;
        krem -= sh.sel_above;
        __syncthreads();
    }
    *krem_out = krem;
    return prefix;
}

// Winners among n elements in list order: keys above kth, and the first krem equal
// to it.  pos_of(i) gives the output value for element i.
template <typename Get, typename Pos>
__device__ void ordered_winners(TopkShared& sh, int n, uint32_t kth, uint32_t krem, Get get,
                                Pos pos_of, int32_t* out) {
    const int tid = threadIdx.x;
    uint32_t eq_base = 0, sel_base = 0;
    for (int i0 = 0; i0 < n; i0 += TK_THREADS * 4) {
        uint32_t keys[4], neq = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = i0 + 4 * tid + q;
            keys[q] = i < n ? get(i) : 0u;
            neq += (i < n && keys[q] == kth) ? 1u : 0u;
        }
        uint32_t eq_tot;
        uint32_t eq_rank = eq_base + block_excl_scan(neq, sh.lds4, &eq_tot);
        uint32_t take[4], nsel = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = i0 + 4 * tid + q;
            bool tk = false;
            if (i < n) {
                if (keys[q] > kth) tk = true;
                else if (keys[q] == kth) { tk = eq_rank < krem; ++eq_rank; }
            }
            take[q] = tk;
            nsel += tk;
        }
        uint32_t sel_tot;
        uint32_t pos = sel_base + block_excl_scan(nsel, sh.lds4, &sel_tot);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (take[q] && pos < TOPK) out[pos] = pos_of(i0 + 4 * tid + q);
            pos += take[q];
        }
        eq_base += eq_tot;
        sel_base += sel_tot;
    }
}

// Top-512 of a list of n scores (list element i: score sc(i), entry index jj(i));
// writes TOPK entry indices (ascending, -1 padded) and returns the count.
template <typename Sc, typename Jj>
__device__ int select_list(TopkShared& sh, int n, Sc sc, Jj jj, int32_t* out) {
    const int tid = threadIdx.x;
    if (n <= TOPK) {
        for (int i = tid; i < TOPK; i += TK_THREADS) out[i] = i < n ? jj(i) : -1;
        return n;
    }
    // 1. sampled lower bound of the 512th largest key
    const int stride = (n + TK_SAMPLE - 1) / TK_SAMPLE;
    const int m = (n + stride - 1) / stride;
    for (int i = tid; i < m; i += TK_THREADS) sh.keys[i] = score_key(sc(i * stride));
    __syncthreads();
    uint32_t krem;
    const uint32_t theta = radix_kth(sh, m, TOPK, [&](int i) { return sh.keys[i]; }, &krem);
    if (stride == 1) {   // the sample is the whole list: theta is the exact 512th key
        ordered_winners(sh, n, theta, krem, [&](int i) { return sh.keys[i]; },
                        [&](int i) { return jj(i); }, out);
        return TOPK;
    }
    // 2. ordered compaction of keys >= theta
    uint32_t base = 0;
    for (int i0 = 0; i0 < n; i0 += TK_THREADS * 4) {
        uint32_t keys[4], nge = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = i0 + 4 * tid + q;
            keys[q] = i < n ? score_key(sc(i)) : 0u;
            nge += (i < n && keys[q] >= theta) ? 1u : 0u;
        }
        uint32_t tot;
        uint32_t pos = base + block_excl_scan(nge, sh.lds4, &tot);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = i0 + 4 * tid + q;
            if (i < n && keys[q] >= theta) {
                if (pos < TK_CAND) { sh.keys[pos] = keys[q]; sh.cj[pos] = jj(i); }
                ++pos;
            }
        }
        base += tot;
    }
    __syncthreads();
    if (base <= (uint32_t)TK_CAND) {
        // 3. exact selection among the candidates (held in list order)
        const int nc = (int)base;
        const uint32_t kth = radix_kth(sh, nc, TOPK, [&](int i) { return sh.keys[i]; }, &krem);
        ordered_winners(sh, nc, kth, krem, [&](int i) { return sh.keys[i]; },
                        [&](int i) { return sh.cj[i]; }, out);
    } else {
        // many exact ties at theta: radix passes over the whole list
        const uint32_t kth = radix_kth(sh, n, TOPK, [&](int i) { return score_key(sc(i)); }, &krem);
        ordered_winners(sh, n, kth, krem, [&](int i) { return score_key(sc(i)); },
                        [&](int i) { return jj(i); }, out);
    }
    return TOPK;
}

// One block per query row of length n(t) <= TOPK_SEG, or per (row, segment)
// when the cache is longer (then writes the segment's winners as candidates).
__global__ void __launch_bounds__(TK_THREADS) k_topk(int B, int Tq,
                                                     const int32_t* __restrict__ q_pos0,
                                                     const int32_t* __restrict__ n_entries,
                                                     const float* __restrict__ S,
                                                     int64_t entry_stride, int nseg,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ seg_j,
                                                     float* __restrict__ seg_s,
                                                     int32_t* __restrict__ seg_n) {
    __shared__ TopkShared sh;
    const int row = blockIdx.x;
    const int seg = blockIdx.y;
    const int b = row / Tq, t = row - b * Tq;
    const int64_t n = cand_count(q_pos0[b], t, n_entries[b], entry_stride);
    const float* srow = S + (int64_t)row * entry_stride;
    if (nseg == 1) {
        const int c = select_list(sh, (int)n, [&](int i) { return srow[i]; },
                                  [&](int i) { return i; }, idx + (int64_t)row * TOPK);
        if (threadIdx.x == 0) cnt[row] = c;
        return;
    }
    const int64_t j0 = (int64_t)seg * TOPK_SEG;
    int len = (int)(n - j0 < TOPK_SEG ? n - j0 : TOPK_SEG);
    len = len < 0 ? 0 : len;
    int32_t* oj = seg_j + ((int64_t)row * nseg + seg) * TOPK;
    const int c = select_list(sh, len, [&](int i) { return srow[j0 + i]; },
                              [&](int i) { return (int)(j0 + i); }, oj);
    __syncthreads();
    // scores of this segment's winners for the merge
    float* os = seg_s + ((int64_t)row * nseg + seg) * TOPK;
    for (int i = threadIdx.x; i < c; i += TK_THREADS) os[i] = srow[oj[i]];
    if (threadIdx.x == 0) seg_n[(int64_t)row * nseg + seg] = c;
}

// Merge of the segments' candidates of one row (in segment order, i.e. entry order).
__global__ void __launch_bounds__(TK_THREADS) k_topk_merge(int B, int Tq, int nseg,
                                                           const int32_t* __restrict__ seg_j,
                                                           const float* __restrict__ seg_s,
                                                           const int32_t* __restrict__ seg_n,
                                                           int32_t* __restrict__ idx,
                                                           int32_t* __restrict__ cnt) {
    __shared__ TopkShared sh;
    __shared__ int32_t off[65];
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    // prefix of the segments' counts (nseg <= 64)
    if (tid == 0) {
        int acc = 0;
        for (int s = 0; s < nseg; ++s) {
            off[s] = acc;
            acc += seg_n[(int64_t)row * nseg + s];
        }
        off[nseg] = acc;
    }
    __syncthreads();
    const int total = off[nseg];
    const int32_t* sj = seg_j + (int64_t)row * nseg * TOPK;
    const float* ss = seg_s + (int64_t)row * nseg * TOPK;
    auto where = [&](int i) {
        int s = 0;
        while (s + 1 < nseg && off[s + 1] <= i) ++s;   // nseg is small
        return s * TOPK + (i - off[s]);
    };
    const int c = select_list(sh, total, [&](int i) { return ss[where(i)]; },
                              [&](int i) { return sj[where(i)]; }, idx + (int64_t)row * TOPK);
    if (tid == 0) cnt[row] = c;
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
