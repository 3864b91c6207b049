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
#include "index_device.h"

namespace csa2 {

// q^I [rows][128] bf16 -> E4M3FN codes [rows][128] and wq[row] = w[row] * scale.
// Sixteen lanes (one DPP row) per (token, head) row (quant_index_row).
__global__ void __launch_bounds__(256) k_quant_index_query(const uint16_t* __restrict__ qI,
                                                           const float* __restrict__ wI,
                                                           int64_t rows,
                                                           uint8_t* __restrict__ q8,
                                                           float* __restrict__ wq) {
    const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
    if (r >= rows) return;          // whole 16-lane rows leave together
    quant_index_row(qI + r * DI, wI[r], q8 + r * DI, wq + r, threadIdx.x & 15);
}

// Scores S[(b*Tq + t)][j] for j < n(t).  One wave per (request, TOK tokens,
// chunk of IDX_CHUNK entries); work items are ordered heaviest tokens first.
// The codes and scales of the next tiles of 16 entries are in flight while the
// current tile is multiplied; all products of a tile are issued before the
// first is read.
template <int TOK>
__global__ void __launch_bounds__(256) k_index_scores(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const uint8_t* __restrict__ q8, const float* __restrict__ wq,
    const uint8_t* __restrict__ ki_codes, const uint8_t* __restrict__ ki_scales,
    int64_t entry_stride, float* __restrict__ S, int64_t s_stride, int n_tg, int n_ch, int rsh) {
    static_assert(TOK == 1 || TOK % 4 == 0, "token slots per wave");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    int b, tg, ch;
    if (TOK == 4) {
        // A block takes four consecutive token groups (one per wave) at one chunk,
        // so its waves share the chunk's keys in L1.  Blocks walk the groups of four
        // heaviest first; within them the chunk index is rotated by the group, so
        // the blocks that land on one XCD (every eighth) see all chunk indices alike
        // instead of always the same ones (which would give the XCDs holding the
        // first chunks several times the work of the others).
        const int nq = (n_tg + 3) >> 2;
        const int64_t per_b = (int64_t)nq * n_ch;
        const int64_t bb = blockIdx.x;
        if (bb >= (int64_t)B * per_b) return;
        b = (int)(bb / per_b);
        const int64_t r = bb % per_b;
        const int q = nq - 1 - (int)(r / n_ch);
        ch = (int)((r % n_ch + q) % n_ch);
        tg = 4 * q + wave;
        if (tg >= n_tg) return;
    } else {
        const int64_t item = (int64_t)blockIdx.x * 4 + wave;
        if (item >= (int64_t)B * n_tg * n_ch) return;
        ch = (int)(item % n_ch);
        tg = n_tg - 1 - (int)((item / n_ch) % n_tg);
        b = (int)(item / ((int64_t)n_ch * n_tg));
    }
    const int t0 = tg * TOK;
    const int32_t qp = q_pos0[b], ne = n_entries[b];
    const int tlast = (t0 + TOK - 1 < Tq) ? t0 + TOK - 1 : Tq - 1;
    const int64_t n_max = cand_count(qp, tlast, ne, entry_stride, rsh);
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
        const int64_t nk = ok ? cand_count(qp, t, ne, entry_stride, rsh) - j_begin : 0;
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
    float* Sbase = S + ((int64_t)b * Tq + t0) * s_stride + j_begin;
    // Stores go through a buffer resource: lanes past their token's candidates
    // get an out-of-range offset and are dropped by the hardware, so the loop has
    // no branch around memory operations and every wait is exact.
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        Sbase, (short)0, (int)((int64_t)TOK * s_stride * 4), 0x00020000);

    if constexpr (TOK == 4) {
        // Software-pipelined form: the products of one token pair run on the matrix
        // unit while the vector unit reduces the other pair, so one wave keeps both
        // busy.  Per tile p:  [products of tokens 0,1 on p | head sums of tokens 2,3
        // of p - 1, then the scatter-sum and store of p - 1]  [products of tokens
        // 2,3 on p | head sums of tokens 0,1 of p].  Codes and scales come through
        // buffer resources bounded to the chunk, so the tiles past its end read
        // zeros (their stores are masked) and the tile count rounds up to groups of
        // four, the depth of the load rotation.
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(ki_codes + ((int64_t)b * entry_stride + j_begin) * 64), (short)0, j_len * 64,
            0x00020000);
        const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(ki_scales + ((int64_t)b * entry_stride + j_begin) * 4), (short)0, j_len * 4,
            0x00020000);
        int nc = ncand[0];
#pragma unroll
        for (int g = 1; g < 4; ++g)
            if (grp == g) nc = ncand[g];
        const int lim = nc - col > 0 ? nc - col : 0;    // tile jt is stored iff jt < lim
        int kld = col * 64 + 16 * grp;                  // code bytes of the next tile to load
        int sld = col * 4;                              // and its entry's four block scales
        int stv = 4 * (grp * (int)s_stride + col) - 64; // store offset of the tile before jt
        uint4 kb[4];
        int sb[4];
        auto ld = [&](int p, uint4& kc, int& sc) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(krs, kld + 1024 * p, 0, 0);
            kc = uint4{v[0], v[1], v[2], v[3]};
            sc = (int)__builtin_amdgcn_raw_buffer_load_b32(ksr, sld + 16 * 4 * p, 0, 0);
        };
        auto mm2 = [&](int k0, const uint4 kc, const int sw, f4 (&d)[2][2]) {
            const int sc = (int)(((uint32_t)sw >> (8 * grp)) & 0xFFu);   // block grp's scale
            const i8 Bv = i8{(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int tile = 0; tile < 2; ++tile)
                    d[k][tile] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A[k0 + k][tile], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
        };
        auto epi2 = [&](int k0, const f4 (&d)[2][2], float& sa, float& sb2) {
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int tile = 0; tile < 2; ++tile)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a0 = __builtin_fmaf(W[k0][tile][i], relu(d[0][tile][i]), a0);
                    a1 = __builtin_fmaf(W[k0 + 1][tile][i], relu(d[1][tile][i]), a1);
                }
            sa = a0;
            sb2 = a1;
        };
        // lane row g holds token g's sum for entry jt + col
        auto put = [&](int jt, int p, float s0, float s1, float s2, float s3) {
            const float tot = rowsum_scatter4(s0, s1, s2, s3);
            const int off = (unsigned)jt < (unsigned)lim ? stv + 64 * p : 0x7FFFFFFF;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), srs, off, 0, 0);
        };
        f4 dA[2][2], dB[2][2];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int tile = 0; tile < 2; ++tile) dB[k][tile] = f4{0.f, 0.f, 0.f, 0.f};
        float s0 = 0.0f, s1 = 0.0f, s2, s3;
#pragma unroll
        for (int p = 0; p < 3; ++p) ld(p, kb[p], sb[p]);
        kld += 3 * 1024;
        sld += 3 * 64;
        auto group = [&](int g) {      // tiles 4g .. 4g + 3
            const int jt = g * 64;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                ld(p, kb[(p + 3) & 3], sb[(p + 3) & 3]);
                mm2(0, kb[p], sb[p], dA);
                epi2(2, dB, s2, s3);
                put(jt + 16 * p - 16, p, s0, s1, s2, s3);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                mm2(2, kb[p], sb[p], dB);
                epi2(0, dA, s0, s1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            kld += 4096;
            sld += 256;
            stv += 256;
        };
        const int ngroups = (j_len + 63) >> 6;
        for (int g = 0; g < ngroups; ++g) group(g);
        epi2(2, dB, s2, s3);
        put(ngroups * 64 - 16, 0, s0, s1, s2, s3);
        return;
    }
    // Few query rows per request (decode, verify): each key is read by one wave
    // only, so the loads are non-temporal (they stream past the caches).
    // Each lane loads the one scale byte its 32-channel block needs (no byte
    // extraction, which the compiler would hoist ahead of the loop's waits).
    auto load = [&](int jt, uint4& kc, uint32_t& sw) {
        int j = jt + col;
        j = j < j_len ? j : j_len - 1;
        const u4v k4 = __builtin_nontemporal_load((const u4v*)(kbase + (int64_t)j * 64));
        kc = uint4{k4[0], k4[1], k4[2], k4[3]};
        sw = __builtin_nontemporal_load(sbase + (int64_t)j * 4 + grp);
    };
    // loads are clamped to the chunk, so always issued
    auto step = [&](int jt, const uint4 kc, const uint32_t sw) {
        const int sc = (int)sw;
        const i8 Bv = i8{(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
        float s[TOK];
        constexpr int KG = TOK < 4 ? TOK : 4;     // tokens whose products are issued together
#pragma unroll
        for (int k0 = 0; k0 < TOK; k0 += KG) {
            f4 d[KG][2];
#pragma unroll
            for (int k = 0; k < KG; ++k)
#pragma unroll
                for (int tile = 0; tile < 2; ++tile)
                    d[k][tile] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A[k0 + k][tile], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
            __builtin_amdgcn_sched_barrier(0);   // all products issued before the first is read
#pragma unroll
            for (int k = 0; k < KG; ++k) {
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[k0 + k][0][i], relu(d[k][0][i]), acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[k0 + k][1][i], relu(d[k][1][i]), acc);
                s[k0 + k] = acc;
            }
        }
        const int j = jt + col;
        if (TOK == 1) {
            const float tot = rowsum_scatter4(s[0], s[0], s[0], s[0]);
            const int off = (grp == 0 && j < ncand[0]) ? 4 * j : 0x7FFFFFFF;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), srs, off, 0, 0);
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
                const int off = j < nc ? 4 * ((k4 + grp) * (int)s_stride + j) : 0x7FFFFFFF;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), srs, off, 0, 0);
            }
        }
    };
    if constexpr (TOK == 1) {
        // One query row: the head sums of four tiles go through one row-sum
        // scatter, which leaves tile g's sums on lane row g, so lane l holds the
        // score of entry jt + l and the four tiles leave in one coalesced store.
        // Eight tile buffers rotate: tile jt + 16p lives in buffer p and is loaded
        // seven tiles ahead.
        const __amdgpu_buffer_rsrc_t srs1 = __builtin_amdgcn_make_buffer_rsrc(
            Sbase, (short)0, ncand[0] * 4, 0x00020000);
        auto partial = [&](const uint4 kc, const uint32_t sw) {
            const int sc = (int)sw;
            const i8 Bv = i8{(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
            const f4 d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A[0][0], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
            const f4 d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A[0][1], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[0][0][i], relu(d0[i]), acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[0][1][i], relu(d1[i]), acc);
            return acc;
        };
        // the query and weights complete before the key stream starts, so the
        // loop's waits only ever count key loads (otherwise the loop head waits
        // for every load in flight on each pass)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        uint4 kb[8];
        uint32_t sb[8];
        // issued in tile order (the loop's waits count on it)
#pragma unroll
        for (int p = 0; p < 7; ++p) {
            load(16 * p, kb[p], sb[p]);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int jt = 0; jt < j_len; jt += 128) {
            float sp[4];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                // tile p + 7 goes into the buffer tile p - 1 used (a fixed rotation,
                // so every wait is on the oldest loads)
                load(jt + 16 * (p + 7), kb[(p + 7) & 7], sb[(p + 7) & 7]);
                sp[p & 3] = partial(kb[p], sb[p]);
                if ((p & 3) == 3) {
                    const float tot = rowsum_scatter4(sp[0], sp[1], sp[2], sp[3]);
                    // entries past the row's candidates fall outside the resource: dropped
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), srs1,
                                                          4 * (jt + 16 * (p - 3) + lane), 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        return;
    }
    // NB tile buffers rotate: tile jt + 16p lives in buffer p % NB and is loaded
    // NB - 1 tiles ahead; no buffer is copied, so no wait lands on a load just
    // issued.
    constexpr int NB = 4;
    uint4 kb[NB];
    uint32_t sb[NB];
#pragma unroll
    for (int p = 0; p < NB - 1; ++p) load(16 * p, kb[p], sb[p]);
    int jt = 0;
    for (; jt + 16 * NB <= j_len; jt += 16 * NB) {
#pragma unroll
        for (int p = 0; p < NB; ++p) {
            load(jt + 16 * (p + NB - 1), kb[(p + NB - 1) % NB], sb[(p + NB - 1) % NB]);
            step(jt + 16 * p, kb[p], sb[p]);
        }
    }
    // up to NB tiles left: the first NB - 1 already in kb[0..NB-2]
    if (jt + 16 * (NB - 1) < j_len) load(jt + 16 * (NB - 1), kb[NB - 1], sb[NB - 1]);
#pragma unroll
    for (int p = 0; p < NB; ++p)
        if (jt + 16 * p < j_len) step(jt + 16 * p, kb[p], sb[p]);
}

// One wave per (query row, segment).  Row scores are spad floats apart (spad a
// multiple of 64); segment s covers entries [s*seg_len, (s+1)*seg_len).  With one
// segment the result goes to idx/cnt, otherwise to the segment buffers.
__global__ void __launch_bounds__(64 * WS_WAVES) k_topk(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const float* __restrict__ S, int64_t spad, int64_t entry_stride, int nseg, int seg_len,
    int32_t* __restrict__ idx, int32_t* __restrict__ cnt, uint32_t* __restrict__ seg_key,
    int32_t* __restrict__ seg_j, int32_t* __restrict__ seg_n, uint32_t* __restrict__ seg_kth,
    const int32_t* __restrict__ row_len, int rsh) {
    __shared__ WaveSel sel[WS_WAVES];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * WS_WAVES + wave;
    if (item >= (int64_t)B * Tq * nseg) return;
    const int64_t row = item / nseg;
    const int seg = (int)(item - row * nseg);
    const int b = (int)(row / Tq), t = (int)(row - (int64_t)b * Tq);
    // the list is the row's causal candidates, or (row_len given) its first
    // row_len[row] scores, e.g. the candidates of a hierarchical pool
    int64_t n = row_len ? (int64_t)row_len[row] : cand_count(q_pos0[b], t, n_entries[b], entry_stride, rsh);
    if (n > (int64_t)nseg * seg_len) n = (int64_t)nseg * seg_len;
    const int64_t j0 = (int64_t)seg * seg_len;
    int len = (int)(n - j0 < seg_len ? n - j0 : seg_len);
    len = len < 0 ? 0 : len;
    const float* src = S + row * spad + j0;       // 16-byte aligned
    WaveTopk st{sel[wave], 0, 0u};
    // 1024 elements per step: four 256-element groups, the next step's loads in
    // flight.  The list comes through a buffer resource bounded to its len scores
    // rounded up to a whole 16-byte group (inside the row's padded storage), so a
    // group is either wholly in range or reads zeros, and no load sits behind a
    // branch; the keys past len are masked below.
    const __amdgpu_buffer_rsrc_t srb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)src, (short)0, 4 * ((len + 3) & ~3), 0x00020000);
    auto fetch = [&](int base, float4 (&v)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i0 = base + 256 * u + 4 * lane;
            const auto w = __builtin_amdgcn_raw_buffer_load_b128(srb, 4 * i0, 0, 0);
            v[u] = make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                               __uint_as_float(w[3]));
        }
    };
    // Long lists start from a threshold taken on a sample (16 runs of 64 elements
    // spread over the list): the key th with about 1.5 * 512 * len / 1024 sample
    // keys at or above it, so that roughly 768 list elements pass.  Elements below
    // th are skipped.  If fewer than 512 pass, some of the top 512 were skipped and
    // the list is streamed again from threshold 0; otherwise every skipped key is
    // below the 512th largest, and all copies of that key were kept.
    bool sampled = false;
    if (len >= 4096) {
        const int gap = (len / 16) & ~63;
        uint32_t kr[16];
#pragma unroll
        for (int g = 0; g < 16; ++g) kr[g] = score_key(src[g * gap + lane]);
        const uint32_t r = (uint32_t)((768 * 1024 + len - 1) / len);
        uint32_t th = wave_threshold_bisect(kr, r, r + r / 2);
        if (th == 0u) {          // repeated keys: the sample's r-th largest
            uint32_t krem;
            th = wave_kth_bisect(kr, r, &krem);
        }
        st.thr = th - 1u;        // keys of finite scores are >= 1
        sampled = true;
    }
    float4 nxt[4];
    if (len > 0) fetch(0, nxt);
    for (int base = 0; base < len; base += 1024) {
        float4 cur[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) cur[u] = nxt[u];
        if (base + 1024 < len) fetch(base + 1024, nxt);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i0 = base + 256 * u + 4 * lane;
            if (base + 256 * u >= len) break;
            const uint32_t k[4] = {i0 < len ? score_key(cur[u].x) : 0u, i0 + 1 < len ? score_key(cur[u].y) : 0u,
                                   i0 + 2 < len ? score_key(cur[u].z) : 0u, i0 + 3 < len ? score_key(cur[u].w) : 0u};
            const int32_t jj[4] = {(int32_t)(j0 + i0), (int32_t)(j0 + i0 + 1), (int32_t)(j0 + i0 + 2),
                                   (int32_t)(j0 + i0 + 3)};
            st.push(k, jj);
        }
    }
    if (sampled && st.nc < TOPK) {
        // rare: the sample threshold was too high; a plain pass from threshold 0
        st.nc = 0;
        st.thr = 0u;
        for (int base = 0; base < len; base += 256) {
            const int i0 = base + 4 * lane;
            const uint32_t k[4] = {i0 < len ? score_key(src[i0]) : 0u, i0 + 1 < len ? score_key(src[i0 + 1]) : 0u,
                                   i0 + 2 < len ? score_key(src[i0 + 2]) : 0u, i0 + 3 < len ? score_key(src[i0 + 3]) : 0u};
            const int32_t jj[4] = {(int32_t)(j0 + i0), (int32_t)(j0 + i0 + 1), (int32_t)(j0 + i0 + 2),
                                   (int32_t)(j0 + i0 + 3)};
            st.push(k, jj);
        }
    }
    if (nseg == 1) {
        const int c = st.finish(idx + row * TOPK, nullptr, nullptr);
        if (lane == 0) cnt[row] = c;
    } else {
        // the segment's 512th and ceil(512 / nseg)-th largest keys bound the merge
        uint32_t kth, kqv;
        const int c = st.finish(seg_j + item * TOPK, seg_key + item * TOPK, &kth,
                                (uint32_t)((TOPK + nseg - 1) / nseg), &kqv);
        if (lane == 0) {
            seg_n[item] = c;
            seg_kth[2 * item] = kth;
            seg_kth[2 * item + 1] = kqv;
        }
    }
}

// Merge of a row's segment winners (segments in entry order): one wave per row.
__global__ void __launch_bounds__(64 * WS_WAVES) k_topk_merge(
    int rows, int nseg, const uint32_t* __restrict__ seg_key, const int32_t* __restrict__ seg_j,
    const int32_t* __restrict__ seg_n, const uint32_t* __restrict__ seg_kth,
    int32_t* __restrict__ idx, int32_t* __restrict__ cnt) {
    __shared__ WaveSel sel[WS_WAVES];
    const int wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * WS_WAVES + wave;
    if (row >= rows) return;
    merge_segments(sel[wave], row, nseg, seg_key, seg_j, seg_n, seg_kth, idx, cnt);
}

// Exclusive prefix sum over a block of NW waves (DPP scans in the waves, the
// wave totals through LDS); *tot = the block total.
template <int NW>
__device__ __forceinline__ uint32_t block_scan_nw(uint32_t v, uint32_t* wsum, uint32_t* tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_scan_add(v);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0u, all = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t x = wsum[w];
        before += w < wave ? x : 0u;
        all += x;
    }
    __syncthreads();
    *tot = all;
    return before + inc - v;
}

// The selection for few query rows of moderate length (one block of eight waves
// per row instead of segments and a merge): a threshold from 1,024 sampled
// scores (2,048 to 2,560 of the row's scores above it, by the sample; each wave
// has room for 768, so a wave's eighth may hold half again its share) filters
// the row, each wave
// compacting its contiguous eighth in order into LDS; a block-wide search
// halving the candidates' key range finds the 512th largest key K and how many
// copies of it are kept (the first, as in every selection here), and a block
// scan writes the kept entries in ascending order.  When the sample misjudges (fewer than 512
// candidates, or more than the buffer holds) wave 0 selects the row exactly
// with the one-segment streaming selection.
constexpr int TR_WAVES = 8, TR_WCAP = 768;
__global__ void __launch_bounds__(64 * TR_WAVES) k_topk_row(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const float* __restrict__ S, int64_t spad, int64_t entry_stride, int32_t* __restrict__ idx,
    int32_t* __restrict__ cnt, int rsh, const int32_t* __restrict__ row_len) {
    constexpr int NSLOT = TR_WAVES * TR_WCAP;
    __shared__ uint32_t ck[NSLOT];
    __shared__ int32_t cj[NSLOT];
    __shared__ WaveSel wsel;
    __shared__ uint32_t wcnt[TR_WAVES];
    __shared__ uint32_t wsum[TR_WAVES];
    __shared__ uint32_t wcount[2][TR_WAVES];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t bc[4];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t row = blockIdx.x;
    if (row >= (int64_t)B * Tq) return;
    const int b = (int)(row / Tq), t = (int)(row - (int64_t)b * Tq);
    // the row's causal candidates, or (row_len given) its first row_len[row]
    // scores, the list of a hierarchical pool
    int n = row_len ? row_len[row] : (int)cand_count(q_pos0[b], t, n_entries[b], entry_stride, rsh);
    n = n < 0 ? 0 : (n > (int)entry_stride ? (int)entry_stride : n);
    int32_t* out = idx + row * TOPK;
    if (n <= TOPK) {
        for (int i = tid; i < TOPK; i += 64 * TR_WAVES) out[i] = i < n ? i : -1;
        if (tid == 0) cnt[row] = n;
        return;
    }
    const float* src = S + row * spad;              // spad: a multiple of 64 floats
    const __amdgpu_buffer_rsrc_t srb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)src, (short)0, 4 * ((n + 3) & ~3), 0x00020000);
    // wave w filters its run [r0, r1) of the row, 8,192 scores a step held in
    // registers; the first step's loads are issued before the threshold is
    // known, so they overlap the sample
    const int per = (n + TR_WAVES * 256 - 1) / (TR_WAVES * 256) * 256;
    const int r0 = wave * per, r1 = min(n, r0 + per);
    constexpr int FU = 32;                         // 16-byte loads a lane a step
    float4 v[FU];
    auto ldc = [&](int base) {
#pragma unroll
        for (int u = 0; u < FU; ++u) {
            const auto w = __builtin_amdgcn_raw_buffer_load_b128(srb, 4 * (base + 256 * u + 4 * lane), 0, 0);
            v[u] = make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                               __uint_as_float(w[3]));
        }
    };
    if (r0 < r1) ldc(r0);
    if (n <= NSLOT) {                               // every score fits: no sample
        if (tid == 0) bc[0] = 1u;
    } else if (wave == 0) {
        uint32_t kr[16];
#pragma unroll
        for (int g = 0; g < 16; ++g) kr[g] = score_key(src[((int64_t)(64 * g + lane) * n) >> 10]);
        const uint32_t ks = (uint32_t)((2048ll * 1024 + n - 1) / n);   // < 512
        uint32_t th = wave_threshold_bisect(kr, ks, ks + ks / 4);
        if (th == 0u) {                 // repeated keys: the sample's ks-th largest
            uint32_t krem;
            th = wave_kth_bisect(kr, ks, &krem);
        }
        if (lane == 0) bc[0] = th;
    }
    __syncthreads();
    const uint32_t th = bc[0];
    // the keys >= th of the run, compacted in order into the wave's region
    const uint64_t below = (1ull << lane) - 1ull;
    uint32_t nc = 0u;
    bool over = false;
    auto compact = [&](int base) {
#pragma unroll
        for (int u = 0; u < FU; ++u) {
            const int i0 = base + 256 * u + 4 * lane;
            const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            uint32_t k[4];
            uint64_t m[4];
            uint32_t c = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                k[q] = i0 + q < r1 ? score_key(f[q]) : 0u;
                m[q] = __ballot(k[q] >= th && k[q] != 0u);
                c += (uint32_t)__popcll(m[q]);
            }
            if (nc + c > (uint32_t)TR_WCAP) {
                over = true;
            } else {
                uint32_t pos = (uint32_t)(wave * TR_WCAP) + nc;
#pragma unroll
                for (int q = 0; q < 4; ++q) pos += (uint32_t)__popcll(m[q] & below);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (k[q] >= th && k[q] != 0u) {
                        ck[pos] = k[q];
                        cj[pos] = i0 + q;
                        ++pos;
                    }
                }
                nc += c;
            }
        }
    };
    for (int base = r0; base < r1; base += 256 * FU) {
        if (base != r0) ldc(base);
        compact(base);
        if (over) break;
    }
    if (lane == 0) wcnt[wave] = over ? 0xFFFFFFFFu : nc;
    __syncthreads();
    uint32_t total = 0u;
    bool fallback = false;
#pragma unroll
    for (int w = 0; w < TR_WAVES; ++w) {
        fallback |= wcnt[w] == 0xFFFFFFFFu;
        total += wcnt[w] == 0xFFFFFFFFu ? 0u : wcnt[w];
    }
    if (fallback || total < (uint32_t)TOPK) {
        if (wave == 0) {
            WaveTopk st{wsel, 0, 0u};
            for (int base = 0; base < n; base += 256) {
                const int i0 = base + 4 * lane;
                const auto w = __builtin_amdgcn_raw_buffer_load_b128(srb, 4 * i0, 0, 0);
                const uint32_t k[4] = {i0 < n ? score_key(__uint_as_float(w[0])) : 0u,
                                       i0 + 1 < n ? score_key(__uint_as_float(w[1])) : 0u,
                                       i0 + 2 < n ? score_key(__uint_as_float(w[2])) : 0u,
                                       i0 + 3 < n ? score_key(__uint_as_float(w[3])) : 0u};
                const int32_t jj[4] = {i0, i0 + 1, i0 + 2, i0 + 3};
                st.push(k, jj);
            }
            const int c = st.finish(out, nullptr, nullptr);
            if (lane == 0) cnt[row] = c;
        }
        return;
    }
    // slots in order: wave region w, positions below wcnt[w] (ascending entries)
    auto slot_key = [&](int s) -> uint32_t {
        return (uint32_t)(s % TR_WCAP) < wcnt[s / TR_WCAP] ? ck[s] : 0u;
    };
    constexpr int SPT = NSLOT / (64 * TR_WAVES);    // slots per thread: 12, consecutive
    uint32_t kv[SPT];
#pragma unroll
    for (int e = 0; e < SPT; ++e) kv[e] = slot_key(SPT * tid + e);
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
        if (kv[e] != 0u) lo = min(lo, kv[e]);
        hi = max(hi, kv[e]);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) { hist[wave] = lo; hist[TR_WAVES + wave] = hi; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < TR_WAVES; ++w) { lo = min(lo, hist[w]); hi = max(hi, hist[TR_WAVES + w]); }
    __syncthreads();
    // the 512th largest key K by halving [lo, hi] (block-wide counts), stopping
    // early when exactly 512 keys reach the middle (K is then their minimum);
    // krem = how many copies of K are kept, eq_total = how many there are
    // keys >= th2 (th2 >= 1) over the block; one barrier a call: the wave totals
    // alternate between two slot sets, and a set is rewritten only after the
    // next call's barrier, which every reader of it has passed
    int par = 0;
    auto block_count = [&](uint32_t th2) -> uint32_t {
        uint32_t c = 0u;
#pragma unroll
        for (int e = 0; e < SPT; ++e) c += kv[e] >= th2 ? 1u : 0u;
        c = wave_sum(c);
        if (lane == 0) wcount[par][wave] = c;
        __syncthreads();
        uint32_t t2 = 0u;
#pragma unroll
        for (int w = 0; w < TR_WAVES; ++w) t2 += wcount[par][w];
        par ^= 1;
        return t2;
    };
    uint32_t a = lo;
    uint64_t bnd = (uint64_t)hi + 1u;
    while (bnd - a > 1u) {
        const uint32_t mid = (uint32_t)(a + ((bnd - a) >> 1));
        const uint32_t c = block_count(mid);
        if (c >= (uint32_t)TOPK) {
            a = mid;
            if (c == (uint32_t)TOPK) break;
        } else {
            bnd = mid;
        }
    }
    uint32_t mk = 0xFFFFFFFFu;                 // K: the smallest key >= a
#pragma unroll
    for (int e = 0; e < SPT; ++e)
        if (kv[e] >= a) mk = min(mk, kv[e]);
    mk = wave_min(mk);
    if (lane == 0) wsum[wave] = mk;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < TR_WAVES; ++w) mk = min(mk, wsum[w]);
    __syncthreads();
    const uint32_t K = mk;
    const uint32_t above = block_count(K + 1u);
    const uint32_t krem = (uint32_t)TOPK - above;
    const uint32_t eq_total = block_count(K) - above;
    // ordered write: keys > K and the first krem keys == K
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
        gt += kv[e] > K;
        eq += kv[e] == K;
    }
    uint32_t take = eq;
    if (krem < eq_total) {
        uint32_t eq_tot;
        const uint32_t rank0 = block_scan_nw<TR_WAVES>(eq, wsum, &eq_tot);
        take = krem > rank0 ? min(krem - rank0, eq) : 0u;
    }
    uint32_t sel_tot;
    uint32_t off = block_scan_nw<TR_WAVES>(gt + take, wsum, &sel_tot);
    uint32_t taken = 0u;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
        const bool keep = kv[e] > K || (kv[e] == K && taken < take);
        if (keep) {
            out[off++] = cj[SPT * tid + e];
            taken += kv[e] == K;
        }
    }
    if (tid == 0) cnt[row] = TOPK;
}

// ---------------------------------------------------------------------------
// Hierarchical candidate pool and Reindex selection.  "Inside DeepSeek V4.1"
// (the Hierarchical Sparse Indexer paragraph) and "Inside DeepSeek V4.1 Flash:
// Deriving the 890-Byte KV Cache" (section "Hierarchical indexing bounds the
// later searches"): the Full layer's scores are grouped into blocks of 8
// entries ranked by their best score; 2,048 blocks (16,384 candidates) are
// kept, the block holding the newest entry always; Reindex layers score only
// the pool with their own index query and take their own top 512.
// ---------------------------------------------------------------------------

// key[row][k] = largest order-preserving key of the scores of entries
// 8k..8k+7 below n(row); one thread per (row, block).
__global__ void __launch_bounds__(256) k_block_keys(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    int64_t entry_stride, const float* __restrict__ S, int64_t spad,
    uint32_t* __restrict__ keys, int64_t kpad, int rsh) {
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (item >= (int64_t)B * Tq * kpad) return;
    const int64_t row = item / kpad;
    const int64_t k = item - row * kpad;
    const int b = (int)(row / Tq), t = (int)(row - (int64_t)b * Tq);
    const int64_t n = cand_count(q_pos0[b], t, n_entries[b], entry_stride, rsh);
    if (8 * k >= n) return;
    const float* src = S + row * spad + 8 * k;        // 32-byte aligned (spad % 64 == 0)
    const float4 a = *(const float4*)src, c = *(const float4*)(src + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    const int m = n - 8 * k < 8 ? (int)(n - 8 * k) : 8;
    uint32_t best = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < m) best = max(best, score_key(v[i]));
    keys[row * kpad + k] = best;
}

// Block-wide (256 threads) exclusive prefix sum: DPP scans within the waves,
// the four wave totals through LDS.  Returns the block total in *tot.
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, uint32_t* wsum, uint32_t* tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_scan_add(v);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0u, all = 0u;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t x = wsum[w];
        before += w < wave ? x : 0u;
        all += x;
    }
    __syncthreads();
    *tot = all;
    return before + inc - v;
}

// The pool of each query row, one block of 256 threads per row: every block
// when there are at most POOL_BLOCKS, else the newest block plus the
// POOL_BLOCKS - 1 others with the largest keys (ties: the smaller block).  A
// radix select (8 bits per pass, the bits common to all keys skipped) finds
// the threshold key K and how many copies of it are kept; a pass over the keys
// in tiles of 1024 (4 consecutive keys per thread, block scans for the output
// offsets) writes the kept blocks in ascending order.  Key rows are padded to
// a multiple of 4 for the 16-byte loads.
__global__ void __launch_bounds__(256) k_pool_select(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    int64_t entry_stride, const uint32_t* __restrict__ keys, int64_t kpad,
    int32_t* __restrict__ pool, int32_t* __restrict__ pool_cnt, int rsh) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wsum[4];
    __shared__ uint32_t bc[4];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    if (row >= (int64_t)B * Tq) return;
    const int b = (int)(row / Tq), t = (int)(row - (int64_t)b * Tq);
    const int64_t n = cand_count(q_pos0[b], t, n_entries[b], entry_stride, rsh);
    const int nb = (int)((n + 7) / 8);
    int32_t* out = pool + row * POOL_BLOCKS;
    if (nb <= POOL_BLOCKS) {
        for (int i = tid; i < POOL_BLOCKS; i += 256) out[i] = i < nb ? i : -1;
        if (tid == 0) pool_cnt[row] = nb;
        return;
    }
    const int m = nb - 1;                          // blocks other than the newest
    const uint4* kr4 = (const uint4*)(keys + row * kpad);
    const int ntile = (m + 1023) / 1024;
    const uint32_t r = POOL_BLOCKS - 1;            // how many of them are kept
    // the row's keys through a buffer resource bounded to the m keys rounded up
    // to a whole 16-byte group (rows are padded to that): a group is either in
    // range or reads zeros, so the passes have no branch around their loads and
    // keep many in flight (keys past m are masked)
    const __amdgpu_buffer_rsrc_t krb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(keys + row * kpad), (short)0, 4 * ((m + 3) & ~3), 0x00020000);
    auto load4 = [&](int c, uint32_t (&k)[4]) {   // keys 1024c + 4 tid .. +3; 0 past m
        const int i = 1024 * c + 4 * tid;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(krb, 4 * i, 0, 0);
        k[0] = v[0]; k[1] = i + 1 < m ? v[1] : 0u; k[2] = i + 2 < m ? v[2] : 0u; k[3] = i + 3 < m ? v[3] : 0u;
    };
    // keys are >= 1 for every real block, so 0 marks "none"
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll 16
    for (int c = 0; c < ntile; ++c) {
        uint32_t k[4];
        load4(c, k);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (k[q] != 0u) lo = min(lo, k[q]);
            hi = max(hi, k[q]);
        }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if ((tid & 63) == 0) { hist[tid >> 6] = lo; hist[4 + (tid >> 6)] = hi; }
    __syncthreads();
    lo = min(min(hist[0], hist[1]), min(hist[2], hist[3]));
    hi = max(max(hist[4], hist[5]), max(hist[6], hist[7]));
    __syncthreads();
    uint32_t K = hi, krem = r, eq_total = (uint32_t)m;   // all keys equal
    if (lo < hi) {
        int hib = 31 - __clz((int)(lo ^ hi));
        uint32_t pmask = hib == 31 ? 0u : ~((2u << hib) - 1u);
        uint32_t prefix = lo & pmask;
        while (hib >= 0) {
            const int lob = hib - 7 > 0 ? hib - 7 : 0;
            const uint32_t dmask = (2u << (hib - lob)) - 1u;
            hist[tid] = 0u;
            __syncthreads();
            // sixteen tiles' loads issued together, then their atomics (tiles
            // past the keys read zeros, which are never counted)
            for (int c0 = 0; c0 < ntile; c0 += 16) {
                uint32_t kk[16][4];
#pragma unroll
                for (int u = 0; u < 16; ++u) load4(c0 + u, kk[u]);
#pragma unroll
                for (int u = 0; u < 16; ++u)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (kk[u][q] != 0u && (kk[u][q] & pmask) == prefix)
                            atomicAdd(&hist[(kk[u][q] >> lob) & dmask], 1u);
            }
            __syncthreads();
            // digit holding the krem-th largest: bins in descending order, one per thread
            const int nbins = (int)dmask + 1;
            const uint32_t h = tid < nbins ? hist[nbins - 1 - tid] : 0u;
            uint32_t tot;
            const uint32_t ex = block_excl_sum(h, wsum, &tot);
            if (tid < nbins && ex < krem && krem <= ex + h) {
                bc[0] = (uint32_t)(nbins - 1 - tid);
                bc[1] = ex;
                bc[2] = h;
            }
            __syncthreads();
            prefix |= bc[0] << lob;
            pmask |= dmask << lob;
            krem -= bc[1];
            eq_total = bc[2];
            hib = lob - 1;
            __syncthreads();
        }
        K = prefix;
    }
    // kept: every key > K and the first krem keys == K in block order.  Each
    // wave owns a contiguous run of the keys: a first pass counts its keys
    // above and equal to K, the four counts give each wave its output offset and
    // the equal keys before it, and a second pass writes its kept blocks in
    // order with in-wave ballot ranks (no block barrier per tile).
    const bool all_eq = krem >= eq_total;
    const int wave = tid >> 6, lane = tid & 63;
    const int per = (m + 1023) / 1024 * 256;      // keys per wave, a multiple of 256
    const int wbeg = wave * per, wend = min(m, wbeg + per);
    auto ldw = [&](int i, uint32_t (&k)[4]) {      // keys i..i+3 of this wave's run, 0 past it
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(krb, 4 * i, 0, 0);
        k[0] = i < wend ? v[0] : 0u; k[1] = i + 1 < wend ? v[1] : 0u;
        k[2] = i + 2 < wend ? v[2] : 0u; k[3] = i + 3 < wend ? v[3] : 0u;
    };
    uint32_t cg = 0u, ce = 0u;
#pragma unroll 16
    for (int i = wbeg + 4 * lane; i < wend; i += 256) {
        uint32_t k[4];
        ldw(i, k);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            cg += k[q] > K;
            ce += k[q] == K;
        }
    }
    cg = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_add(cg), 63);
    ce = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_add(ce), 63);
    if (lane == 0) { hist[2 * wave] = cg; hist[2 * wave + 1] = ce; }
    __syncthreads();
    uint32_t off = 0u, eq_seen = 0u;               // output offset, equal keys before this wave
    for (int w = 0; w < wave; ++w) {
        const uint32_t e = hist[2 * w + 1];
        off += hist[2 * w] + (all_eq ? e : (krem > eq_seen ? min(krem - eq_seen, e) : 0u));
        eq_seen += e;
    }
    uint32_t kq[4][4];                             // four groups' loads in flight
#pragma unroll
    for (int d = 0; d < 4; ++d) ldw(wbeg + 256 * d + 4 * lane, kq[d]);
    for (int base0 = wbeg; base0 < wend; base0 += 1024) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int base = base0 + 256 * d;
            if (base >= wend) break;
            uint32_t k[4] = {kq[d][0], kq[d][1], kq[d][2], kq[d][3]};
            ldw(base + 1024 + 4 * lane, kq[d]);
            uint32_t gt = 0u, eq = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                gt += k[q] > K;
                eq += k[q] == K;
            }
            // this lane's equal keys rank after those of the lanes before it
            const uint32_t eq_inc = wave_scan_add(eq);
            const uint32_t eq_tot = (uint32_t)__builtin_amdgcn_readlane((int)eq_inc, 63);
            const uint32_t rank0 = eq_seen + eq_inc - eq;
            const uint32_t take = all_eq ? eq : (krem > rank0 ? min(krem - rank0, eq) : 0u);
            const uint32_t sel_inc = wave_scan_add(gt + take);
            const uint32_t sel_tot = (uint32_t)__builtin_amdgcn_readlane((int)sel_inc, 63);
            uint32_t o = off + sel_inc - (gt + take), taken = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool keep = k[q] > K || (k[q] == K && taken < take);
                if (keep) {
                    out[o++] = base + 4 * lane + q;
                    taken += k[q] == K;
                }
            }
            off += sel_tot;
            eq_seen += eq_tot;
        }
    }
    if (tid == 0) {
        out[POOL_BLOCKS - 1] = m;                  // the newest block, largest index
        pool_cnt[row] = POOL_BLOCKS;
    }
}

// Reindex scores: the row's own index query against the pool's candidates,
// written as a list in pool order (entry 8 pool[s] + e at position 8 s + e).
// One wave per (row, 128 pool slots); a 16-entry tile is two pool blocks.
// row_len[row] = the list's length: every pool block is full except the
// newest, the last one.
__global__ void __launch_bounds__(256) k_pool_scores(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const uint8_t* __restrict__ q8, const float* __restrict__ wq,
    const uint8_t* __restrict__ ki_codes, const uint8_t* __restrict__ ki_scales,
    int64_t entry_stride, const int32_t* __restrict__ pool, const int32_t* __restrict__ pool_cnt,
    float* __restrict__ Sc, int64_t scpad, int32_t* __restrict__ row_len, int rsh) {
    constexpr int SLOTS = 128;
    constexpr int NPC = POOL_BLOCKS / SLOTS;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    if (item >= (int64_t)B * Tq * NPC) return;
    const int64_t row = item / NPC;
    const int pc = (int)(item - row * NPC);
    const int b = (int)(row / Tq), t = (int)(row - (int64_t)b * Tq);
    const int64_t n = cand_count(q_pos0[b], t, n_entries[b], entry_stride, rsh);
    const int cntp = pool_cnt[row];
    const int64_t nb = (n + 7) / 8;
    if (pc == 0 && lane == 0) row_len[row] = cntp > 0 ? (int32_t)(n - 8 * (nb - cntp)) : 0;
    const int s_begin = pc * SLOTS;
    if (s_begin >= cntp) return;
    const int s_end = min(s_begin + SLOTS, cntp);
    const int col = lane & 15, grp = lane >> 4;
    i8 A[2];
    f4 W[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
        const int64_t qrow = ((int64_t)b * Tq + t) * HI + tile * 16;
        const uint8_t* src = q8 + (qrow + col) * DI + 16 * grp;
        const uint4 u0 = *(const uint4*)src, u1 = *(const uint4*)(src + 64);
        A[tile] = i8{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
        const float4 w4 = *(const float4*)(wq + qrow + 4 * grp);
        W[tile] = f4{w4.x, w4.y, w4.z, w4.w};
    }
    const int32_t* prow = pool + row * POOL_BLOCKS;
    const int64_t ebase = (int64_t)b * entry_stride;
    auto load = [&](int s0, uint4& kc, uint32_t& sw) {
        const int s = s0 + (col >> 3);
        const int blk = s < s_end ? prow[s] : 0;
        int64_t e = 8 * (int64_t)blk + (col & 7);
        e = e < n ? e : n - 1;                     // past the list: any valid entry, not stored
        kc = *(const uint4*)(ki_codes + (ebase + e) * 64 + 16 * grp);
        sw = *(const uint32_t*)(ki_scales + (ebase + e) * 4);
    };
    uint4 kc_n;
    uint32_t sw_n;
    load(s_begin, kc_n, sw_n);
    for (int s0 = s_begin; s0 < s_end; s0 += 2) {
        const uint4 kc = kc_n;
        const uint32_t sw = sw_n;
        if (s0 + 2 < s_end) load(s0 + 2, kc_n, sw_n);
        const int sc = (int)((sw >> (8 * grp)) & 0xFFu);
        const i8 Bv = i8{(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
        const f4 d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[0], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
        const f4 d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[1], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[0][i], relu(d0[i]), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[1][i], relu(d1[i]), acc);
        const float tot = rowsum_scatter4(acc, acc, acc, acc);
        const int pos = 8 * s0 + col;
        if (grp == 0 && s0 + (col >> 3) < s_end) Sc[row * scpad + pos] = tot;
    }
}

// list positions -> entries: position 8 s + e is entry 8 pool[s] + e.
__global__ void __launch_bounds__(256) k_pool_map(int64_t rows, const int32_t* __restrict__ pool,
                                                  int32_t* __restrict__ idx) {
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (item >= rows * TOPK) return;
    const int64_t row = item / TOPK;
    const int32_t v = idx[item];
    if (v >= 0) idx[item] = 8 * pool[row * POOL_BLOCKS + (v >> 3)] + (v & 7);
}

template __global__ void k_index_scores<1>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                           const float*, const uint8_t*, const uint8_t*, int64_t,
                                           float*, int64_t, int, int, int);
template __global__ void k_index_scores<4>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                           const float*, const uint8_t*, const uint8_t*, int64_t,
                                           float*, int64_t, int, int, int);
template __global__ void k_index_scores<8>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                           const float*, const uint8_t*, const uint8_t*, int64_t,
                                           float*, int64_t, int, int, int);

}  // namespace csa2
