// Lightning indexer with the causal top-512 fused in: no score row ever
// reaches memory.
//
// "DeepSeek V4.1 -- Pooled group -> Source layer, pairs pooled", indexer and
// top-k equations: S^I_{t,j} = sum_h w^I_{t,h} ReLU(Q^I_{h,t} . K^I_j) and
// I_t = top_512(S^I_{t,j} : j < floor((t+1)/2)) (the entries' ratio in place
// of 2).  "Inside DeepSeek V4.1", section "Attention that looks at 640
// places": every compressed entry is scored, 512 go on to attention.
//
// One wave per (group of TOK query tokens of one request, segment of entries).
// The wave loads its tokens' E4M3 query rows once and walks the segment's
// entries in order, 16 per tile, with the same block-scaled FP8 x FP4 MFMA and
// the same epilogue (integer-max ReLU, head weights folded with the query
// scales, lane-swap head sums) as the score-only kernel, so every score is the
// same fp32 value.  After a tile, lane row g holds token g's 16 scores; each
// is compared with that token's running threshold and the passing ones are
// appended, in entry order, to the token's candidate buffer in LDS (a DPP
// prefix count over the lane row gives the slots; no branch: lanes that do not
// pass write a spare slot).  Long lists start from a threshold scored on a
// sample of 16 tiles spread over the entries (a token left with too few
// candidates is scanned again from minus infinity); without it the threshold
// starts at minus infinity and the buffers fill many more times.  When a
// buffer is nearly full, a wave-wide search over it (halving the key range,
// counting with compares and a DPP sum) finds a key theta with at least 512
// candidates at or above it and at most `keep`, keeps those in order and makes
// theta the token's new (strict) threshold: a later entry equal to theta ranks
// below every kept one, which has a smaller j.
// At the end an exact select keeps the 512 largest (ties: smaller j).
//
// Segments: when the token groups are many, each wave takes all of its
// tokens' entries (one segment).  When they are too few to fill the GPU, a row
// is cut into segments; each segment's wave writes its winners (at most 512
// keys and entries, its 512th and ceil(512/nseg)-th keys), and the last
// segment wave of a row to finish -- counted with a device-scope atomic per
// row -- merges them while other rows are still being scanned.
#include "index_device.h"

namespace csa2 {

// Per-token candidate buffers: the scores' bit patterns and the entries as
// 16-bit offsets from the segment's first entry (segments are at most 65,536
// entries).  cap slots per token (plus one spare slot per lane column), sized
// so that the four-token form fits two waves per SIMD in LDS.  tiles: tiles
// between two checks of the fill; a buffer past `cap - 16 * (tiles + 1)` is
// refilled, so the admissions before the next check always fit.  keep: a refill
// keeps at most about this many.  waves: the occupancy the registers are
// budgeted for.
template <int TOK> struct SelCfg {
    static constexpr int cap = TOK == 1 ? 1024 : 768;
    static constexpr int pad = cap + 16;
    static constexpr int tiles = TOK == 1 ? 8 : 4;
    static constexpr int keep = cap - 192;
    static constexpr int waves = TOK == 1 ? 3 : (TOK == 4 ? 2 : 1);
};
// Lists at least this long start from a sampled threshold.  Four-token groups:
// from 1,024 candidates (a shorter list is trimmed only once or twice).
// Single-token rows: from 4,096 up to 65,536 entries.
constexpr int SAMPLE_MIN = 1024;
constexpr int ROW_SAMPLE_MIN = 4096;

template <int TOK>
struct SelBuf {
    uint32_t key[TOK][SelCfg<TOK>::pad];     // bit patterns of the candidates' scores
    uint16_t j[TOK][SelCfg<TOK>::pad];       // their entries (offsets), ascending
};
// the wave's LDS: the candidate buffers while scanning, a merge buffer after
template <int TOK>
union SelLds {
    SelBuf<TOK> b;
    WaveSel ws;
};

template <int TOK>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(SelCfg<TOK>::waves))) k_index_select(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const uint8_t* __restrict__ q8, const float* __restrict__ wq,
    const uint8_t* __restrict__ ki_codes, const uint8_t* __restrict__ ki_scales,
    int64_t entry_stride, int n_tg, int nseg, int seg_len, int rsh, int32_t* __restrict__ idx,
    int32_t* __restrict__ cnt, uint32_t* __restrict__ seg_key, int32_t* __restrict__ seg_j,
    int32_t* __restrict__ seg_n, uint32_t* __restrict__ seg_kth, uint32_t* __restrict__ row_done) {
    static_assert(TOK == 1 || TOK == 4 || TOK == 8, "token slots per wave");
    constexpr int NR = TOK == 8 ? 2 : 1;          // lane-row sets: tokens 4r .. 4r+3
    constexpr int CAP = SelCfg<TOK>::cap;
    constexpr int CHK = SelCfg<TOK>::tiles;
    constexpr int TRIGGER = CAP - 16 * (CHK + 1);
    constexpr int KR = CAP / 64;                  // register rows of a buffer's keys
    __shared__ SelLds<TOK> L;
    const int lane = threadIdx.x;
    const int col = lane & 15, grp = lane >> 4;

    // ---- work item: heaviest token groups first, a row's segments together
    const int64_t item = blockIdx.x;
    const int seg = (int)(item % nseg);
    const int64_t rest = item / nseg;
    const int b = (int)(rest % B);
    const int tg = n_tg - 1 - (int)(rest / B);
    if (tg < 0) return;
    const int t0 = tg * TOK;
    const int32_t qp = q_pos0[b], ne = n_entries[b];
    const int64_t j0 = (int64_t)seg * seg_len;

    // this lane row's tokens: candidates inside the segment, threshold, fill
    int lim[NR];                 // tile jt of this lane is a candidate iff jt < lim (unsigned)
    int ncnd[NR];                // the row's token's candidates in the segment
    float thr[NR];
    int fill[NR];
    int jlen = 0;                // entries the segment scans: the largest ncnd
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int k = TOK == 1 ? 0 : 4 * r + grp;
        const int t = t0 + k;
        int64_t n = (t < Tq && (TOK > 1 || grp == 0)) ? cand_count(qp, t, ne, entry_stride, rsh) - j0 : 0;
        n = n < 0 ? 0 : (n > seg_len ? seg_len : n);
        ncnd[r] = (int)n;
        lim[r] = (int)n - col > 0 ? (int)n - col : 0;
        thr[r] = -INFINITY;
        fill[r] = 0;
        jlen = max(jlen, (int)n);
    }
    jlen = (int)wave_max((uint32_t)jlen);

    // the whole row of a single-token item (its segments' union), for the sampled start
    const int n_row = TOK == 1 ? (int)min(cand_count(qp, t0, ne, entry_stride, rsh), (int64_t)0x7FFFFFFF) : 0;
    const bool row_sampled = TOK == 1 && n_row >= ROW_SAMPLE_MIN && n_row <= 65536;   // offsets fit 16 bits
    const __amdgpu_buffer_rsrc_t krow = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ki_codes + (int64_t)b * entry_stride * 64), (short)0, row_sampled ? n_row * 64 : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t srow = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ki_scales + (int64_t)b * entry_stride * 4), (short)0, row_sampled ? n_row * 4 : 0, 0x00020000);

    // ---- query operands (as the score-only kernel loads them)
    i8 A[TOK][2];
    f4 W[TOK][2];
#pragma unroll
    for (int k = 0; k < TOK; ++k) {
        const int t = t0 + k;
        const bool ok = t < Tq;
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            const int64_t row = ((int64_t)b * Tq + (ok ? t : 0)) * HI + tile * 16;
            const uint8_t* src = q8 + (row + col) * DI + 16 * grp;
            const uint4 u0 = *(const uint4*)src, u1 = *(const uint4*)(src + 64);
            A[k][tile] = ok ? i8{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                                 (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w}
                            : i8{0, 0, 0, 0, 0, 0, 0, 0};
            const float4 w4 = *(const float4*)(wq + row + 4 * grp);
            W[k][tile] = ok ? f4{w4.x, w4.y, w4.z, w4.w} : f4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // ---- admission of one tile's scores: lane row g holds token 4r + g's score
    // of entry jt + col (TOK = 1: row 0 holds token 0's, the other rows copies).
    // The passing lanes of a row take consecutive slots in lane (entry) order:
    // an inclusive prefix count over the row's 16 lanes (DPP row shifts) and the
    // row's total from its last lane (DPP row broadcast).
    auto admit = [&](int r, int jt, float tot) {
        const bool pass = (TOK > 1 || grp == 0) && (unsigned)jt < (unsigned)lim[r] && tot > thr[r];
        const int b = pass ? 1 : 0;
        int sc = b;
        sc += __builtin_amdgcn_update_dpp(0, sc, 0x111, 0xf, 0xf, true);   // row_shr:1
        sc += __builtin_amdgcn_update_dpp(0, sc, 0x112, 0xf, 0xf, true);   // row_shr:2
        sc += __builtin_amdgcn_update_dpp(0, sc, 0x114, 0xf, 0xf, true);   // row_shr:4
        sc += __builtin_amdgcn_update_dpp(0, sc, 0x118, 0xf, 0xf, true);   // row_shr:8
        const int total = __builtin_amdgcn_update_dpp(0, sc, 0x15F, 0xf, 0xf, false);  // row_newbcast:15
        const int slot = pass ? fill[r] + sc - 1 : CAP + col;
        const int tk = TOK == 1 ? 0 : 4 * r + grp;
        L.b.key[tk][slot] = __float_as_uint(tot);
        L.b.j[tk][slot] = (uint16_t)(jt + col);
        fill[r] += total;
    };

    // ---- refill of token tk's buffer (whole wave): keep the candidates at or
    // above a key theta that at least 512 of them reach, theta becomes strict
    auto refill = [&](int r, int g) {      // r: a compile-time row set, g: the lane row
        const int tk = TOK == 1 ? 0 : 4 * r + g;
        const int nc = __builtin_amdgcn_readlane(fill[r], 16 * g);
        uint32_t kr[KR];
#pragma unroll
        for (int q = 0; q < KR; ++q) {
            const int i = 64 * q + lane;
            kr[q] = i < nc ? score_key(__uint_as_float(L.b.key[tk][i])) : 0u;
        }
        uint32_t theta = wave_threshold_bisect(kr, TOPK, SelCfg<TOK>::keep);
        int kept;
        if (theta != 0u) {
            kept = wave_keep_buf<true>(L.b.key[tk], L.b.j[tk], nc, kr, theta, 0xFFFFFFFFu);
        } else {
            // so many equal keys that no threshold keeps between 512 and `keep`:
            // the exact 512th key and its copies among the first 512
            uint32_t krem;
            theta = wave_kth_bisect(kr, TOPK, &krem);
            kept = wave_keep_buf<true>(L.b.key[tk], L.b.j[tk], nc, kr, theta, krem);
        }
        if (grp == g) {
            fill[r] = kept;
            thr[r] = key_score(theta);
        }
    };
    auto check = [&]() {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            uint64_t over = __ballot(fill[r] > TRIGGER) & (TOK == 1 ? 0xFFFFull : ~0ull);
            while (over) {
                const int g = (__ffsll((long long)over) - 1) >> 4;
                refill(r, g);
                over = __ballot(fill[r] > TRIGGER) & (TOK == 1 ? 0xFFFFull : ~0ull);
            }
        }
    };

    const uint8_t* kbase = ki_codes + ((int64_t)b * entry_stride + j0) * 64;
    const uint8_t* sbase = ki_scales + ((int64_t)b * entry_stride + j0) * 4;
    // codes and scales through buffer resources bounded to the scanned entries:
    // tiles past them read zeros (their scores are never admitted), so no load
    // sits behind a branch and every wait is exact
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)kbase, (short)0, jlen * 64, 0x00020000);
    const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)sbase, (short)0, jlen * 4, 0x00020000);

    auto load = [&](const __amdgpu_buffer_rsrc_t kr_, const __amdgpu_buffer_rsrc_t sr_, int jt,
                    uint4& kc, uint32_t& sw) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(kr_, (jt + col) * 64 + 16 * grp, 0, 0);
        kc = uint4{v[0], v[1], v[2], v[3]};
        sw = __builtin_amdgcn_raw_buffer_load_b32(sr_, (jt + col) * 4, 0, 0);
    };
    // one tile's head sums per token (lane row g: heads 4g..4g+3 of each 16)
    auto sums = [&](const uint4 kc, const uint32_t sw, float (&s)[TOK]) {
        const int sc = (int)((sw >> (8 * grp)) & 0xFFu);
        const i8 Bv = i8{(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
        constexpr int KG = TOK < 4 ? TOK : 4;
#pragma unroll
        for (int k0 = 0; k0 < TOK; k0 += KG) {
            f4 d[KG][2];
#pragma unroll
            for (int k = 0; k < KG; ++k)
#pragma unroll
                for (int tile = 0; tile < 2; ++tile)
                    d[k][tile] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A[k0 + k][tile], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
            __builtin_amdgcn_sched_barrier(0);
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
    };
    auto step = [&](int jt, const uint4 kc, const uint32_t sw) {
        float s[TOK];
        sums(kc, sw, s);
        if (TOK == 1) {
            admit(0, jt, rowsum_scatter4(s[0], s[0], s[0], s[0]));
        } else {
#pragma unroll
            for (int r = 0; r < NR; ++r)
                admit(r, jt, rowsum_scatter4(s[4 * r], s[4 * r + 1], s[4 * r + 2], s[4 * r + 3]));
        }
    };
    // the entries [0, len) of the resources, NB tile buffers rotating: tile
    // jt + 16p lives in buffer p % NB and is loaded NB - 1 tiles ahead
    // (buffer loads past the entries read zeros)
    constexpr int NB = CHK;
    auto scan = [&](const __amdgpu_buffer_rsrc_t kr_, const __amdgpu_buffer_rsrc_t sr_, int len) {
        uint4 kb[NB];
        uint32_t sb[NB];
#pragma unroll
        for (int p = 0; p < NB - 1; ++p) load(kr_, sr_, 16 * p, kb[p], sb[p]);
        for (int jt = 0; jt < len; jt += 16 * NB) {
#pragma unroll
            for (int p = 0; p < NB; ++p) {
                load(kr_, sr_, jt + 16 * (p + NB - 1), kb[(p + NB - 1) % NB], sb[(p + NB - 1) % NB]);
                step(jt + 16 * p, kb[p], sb[p]);
            }
            check();
        }
    };
    // a single-token row scanned whole from minus infinity (the sampled start
    // was too high), then cut to its exact top 512, written in entry order
    auto rescan_row = [&](int64_t row) {
        thr[0] = -INFINITY;
        fill[0] = 0;
        lim[0] = grp == 0 ? max(n_row - col, 0) : 0;
        scan(krow, srow, n_row);
        int nc = __builtin_amdgcn_readfirstlane(fill[0]);
        if (nc > TOPK) {
            uint32_t kr[KR];
#pragma unroll
            for (int q = 0; q < KR; ++q) {
                const int i = 64 * q + lane;
                kr[q] = i < nc ? score_key(__uint_as_float(L.b.key[0][i])) : 0u;
            }
            uint32_t krem;
            const uint32_t kth = wave_kth_bisect(kr, TOPK, &krem);
            nc = wave_keep_buf<true>(L.b.key[0], L.b.j[0], nc, kr, kth, krem);
        }
        int32_t* out = idx + row * TOPK;
        for (int i = lane; i < TOPK; i += 64) out[i] = i < nc ? (int)L.b.j[0][i] : -1;
        if (lane == 0) cnt[row] = nc;
    };

    if constexpr (TOK == 4) {
        const int kld0 = col * 64 + 16 * grp;
        const int sld0 = col * 4;
        auto ld = [&](int off, uint4& kc, int& sc) {     // off: the tile's first entry
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(krs, kld0 + 64 * off, 0, 0);
            kc = uint4{v[0], v[1], v[2], v[3]};
            sc = (int)__builtin_amdgcn_raw_buffer_load_b32(ksr, sld0 + 4 * off, 0, 0);
        };
        auto mm2 = [&](int k0, const uint4 kc, const int sw, f4 (&d)[2][2]) {
            const int sc = (int)(((uint32_t)sw >> (8 * grp)) & 0xFFu);
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

        // Starting thresholds from a sample: 16 tiles spread evenly over the
        // entries every token of the group may select.  With p = 512 / n the
        // fraction of a token's n candidates in its top 512, about 256 p of the
        // sample's scores fall there; a threshold reached by r = 256 p + 3
        // sqrt(256 p) + 1 of them (up to 1.5 r, within the 256 scores for
        // n >= 1,024) leaves fewer than 512 scores above it only rarely, and
        // then the token is scanned again from
        // minus infinity.  Without it a token's threshold starts at minus
        // infinity and rises only as its buffer fills, so a long list is
        // trimmed many more times.
        const int nmin = (int)wave_min((uint32_t)ncnd[0]);
        bool sampled = false;
        if (nmin >= SAMPLE_MIN) {
            constexpr int NS = 16;
            uint4 skc[NS];
            int ssc[NS];
#pragma unroll
            for (int q = 0; q < NS; ++q) ld((((2 * q + 1) * nmin) / (2 * NS)) & ~15, skc[q], ssc[q]);
            uint32_t kv[NS];
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                f4 d0[2][2], d1[2][2];
                mm2(0, skc[q], ssc[q], d0);
                mm2(2, skc[q], ssc[q], d1);
                float a0, a1, a2, a3;
                epi2(0, d0, a0, a1);
                epi2(2, d1, a2, a3);
                kv[q] = score_key(rowsum_scatter4(a0, a1, a2, a3));
            }
            const float mean = 256.0f * (float)TOPK / (float)nmin;
            const uint32_t r = (uint32_t)ceilf(mean + 3.0f * sqrtf(mean) + 1.0f);
            const uint32_t a = row_threshold_bisect<NS>(kv, r, r + (r >> 1));
            // admission is strict: the threshold is the score just below key a
            // (below +0 when a is the key of +0, which -0 shares)
            const uint32_t kb = a == 0x80000000u ? 0x7FFFFFFEu : a - 1u;
            thr[0] = key_score(kb);
            sampled = true;
        }

        for (int pass = 0; pass < 2; ++pass) {
            // Software-pipelined by token pairs, as in the score-only kernel: the
            // products of one pair run on the matrix unit while the vector unit
            // reduces the other pair.  Per tile p: [products of tokens 0,1 on p |
            // head sums of tokens 2,3 of p - 1, then the admission of p - 1]
            // [products of tokens 2,3 on p | head sums of tokens 0,1 of p].
            uint4 kb[4];
            int sb[4];
            f4 dA[2][2], dB[2][2];
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int tile = 0; tile < 2; ++tile) dB[k][tile] = f4{0.f, 0.f, 0.f, 0.f};
            float s0 = 0.0f, s1 = 0.0f, s2, s3;
#pragma unroll
            for (int p = 0; p < 3; ++p) ld(16 * p, kb[p], sb[p]);
            const int ngroups = (jlen + 63) >> 6;
            for (int gi = 0; gi < ngroups; ++gi) {      // tiles 4 gi .. 4 gi + 3
                const int jt = gi * 64;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    ld(jt + 16 * (p + 3), kb[(p + 3) & 3], sb[(p + 3) & 3]);
                    mm2(0, kb[p], sb[p], dA);
                    epi2(2, dB, s2, s3);
                    admit(0, jt + 16 * p - 16, rowsum_scatter4(s0, s1, s2, s3));
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
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
                check();
            }
            epi2(2, dB, s2, s3);
            admit(0, ngroups * 64 - 16, rowsum_scatter4(s0, s1, s2, s3));
            if (!sampled) break;
            // a refill keeps at least 512, so a short buffer never had one: its
            // sampled threshold let too few through; rescan those tokens alone
            const bool short_ = fill[0] < min(TOPK, ncnd[0]);
            if (__ballot(short_) == 0ull) break;
            lim[0] = short_ ? max(ncnd[0] - col, 0) : 0;
            thr[0] = short_ ? -INFINITY : thr[0];
            fill[0] = short_ ? 0 : fill[0];
            sampled = false;
        }
    } else {
        if constexpr (TOK == 1) {
            // A row of 4,096 to 65,536 entries starts every one of its segments
            // from one threshold taken on 16 tiles spread evenly over the row (all
            // of them score the same sample, so all agree): with p = 512 / n,
            // about 256 p sampled scores fall in the row's top 512, and a
            // threshold reached by r = 256 p + 4 sqrt(256 p) + 2 of them (up to
            // 1.5 r) leaves fewer than 512 of the row's scores above it only
            // rarely.  Each segment then admits a small share of its entries
            // instead of selecting its own 512.  If the row ends up short, it is
            // scanned again from minus infinity: here when it is one segment, by
            // the wave that merges it otherwise.
            if (row_sampled) {
                uint4 skc[16];
                uint32_t ssc[16];
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    load(krow, srow, (((2 * q + 1) * n_row) / 32) & ~15, skc[q], ssc[q]);
                uint32_t kv[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    float s1[TOK];
                    sums(skc[q], ssc[q], s1);
                    kv[q] = score_key(rowsum_scatter4(s1[0], s1[0], s1[0], s1[0]));
                }
                const float mean = 256.0f * (float)TOPK / (float)n_row;
                const uint32_t r = (uint32_t)ceilf(mean + 4.0f * sqrtf(mean) + 2.0f);
                const uint32_t a = row_threshold_bisect<16>(kv, r, r + (r >> 1));
                thr[0] = key_score(a == 0x80000000u ? 0x7FFFFFFEu : a - 1u);
            }
            scan(krs, ksr, jlen);
            if (row_sampled && nseg == 1 &&
                __builtin_amdgcn_readfirstlane(fill[0]) < min(TOPK, __builtin_amdgcn_readfirstlane(ncnd[0]))) {
                thr[0] = -INFINITY;
                fill[0] = 0;
                scan(krs, ksr, jlen);
            }
        } else {
            scan(krs, ksr, jlen);
        }
    }

    // ---- results per token: the exact top 512 of its candidates, in entry order
#pragma unroll
    for (int tk = 0; tk < TOK; ++tk) {
        const int r = TOK == 1 ? 0 : tk >> 2, g = TOK == 1 ? 0 : tk & 3;
        const int t = t0 + tk;
        if (t >= Tq) break;
        const int64_t row = (int64_t)b * Tq + t;
        int nc = __builtin_amdgcn_readlane(fill[r], 16 * g);
        uint32_t kr[KR];
        if (nc > TOPK || nseg > 1) {
#pragma unroll
            for (int q = 0; q < KR; ++q) {
                const int i = 64 * q + lane;
                kr[q] = i < nc ? score_key(__uint_as_float(L.b.key[tk][i])) : 0u;
            }
        }
        if (nc > TOPK) {
            uint32_t krem;
            const uint32_t kth = wave_kth_bisect(kr, TOPK, &krem);
            nc = wave_keep_buf<true>(L.b.key[tk], L.b.j[tk], nc, kr, kth, krem);
            if (nseg > 1) {          // the segment's keys again, for its winners' bound
#pragma unroll
                for (int q = 0; q < KR; ++q) {
                    const int i = 64 * q + lane;
                    kr[q] = i < nc ? score_key(__uint_as_float(L.b.key[tk][i])) : 0u;
                }
            }
        }
        if (nseg == 1) {
            int32_t* out = idx + row * TOPK;
            for (int i = lane; i < TOPK; i += 64) out[i] = i < nc ? (int)j0 + L.b.j[tk][i] : -1;
            if (lane == 0) cnt[row] = nc;
        } else {
            // the segment's winners, its 512th key (0 when it has fewer) and its
            // ceil(512 / nseg)-th key (0 when it has fewer), for the merge's bound
            const int64_t it = row * nseg + seg;
            uint32_t mn = 0xFFFFFFFFu;
            for (int i = lane; i < TOPK; i += 64) {
                const bool v = i < nc;
                const uint32_t kv = v ? score_key(__uint_as_float(L.b.key[tk][i])) : 0u;
                seg_key[it * TOPK + i] = kv;
                seg_j[it * TOPK + i] = v ? (int)j0 + L.b.j[tk][i] : -1;
                if (v) mn = min(mn, kv);
            }
            const uint32_t kq = (uint32_t)((TOPK + nseg - 1) / nseg);
            uint32_t kqv = 0u;
            if (nc >= (int)kq) {
                uint32_t krem;
                kqv = wave_kth_bisect(kr, kq, &krem);
            }
            const uint32_t kth = nc == TOPK ? wave_min(mn) : 0u;
            if (lane == 0) {
                seg_n[it] = nc;
                seg_kth[2 * it] = kth;
                seg_kth[2 * it + 1] = kqv;
            }
        }
    }
    if (nseg == 1) return;

    // ---- the last segment wave of a row merges the row's winners
    WaveSel& ws = L.ws;
#pragma unroll
    for (int tk = 0; tk < TOK; ++tk) {
        const int t = t0 + tk;
        if (t >= Tq) break;
        const int64_t row = (int64_t)b * Tq + t;
        __threadfence();                   // this wave's winners are visible device-wide
        uint32_t prev = 0u;
        if (lane == 0) prev = atomicAdd(&row_done[row], 1u);
        prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
        if (prev == (uint32_t)(nseg - 1)) {
            __threadfence();               // and the other segments' winners are visible here
            if (TOK == 1 && row_sampled) {
                // the segments' candidates together: at least min(512, n) of them
                // means the row's top 512 are among them
                const int m = lane < nseg ? seg_n[row * nseg + lane] : 0;
                const int total = (int)wave_sum((uint32_t)max(m, 0));
                if (total < min(TOPK, n_row)) {
                    rescan_row(row);
                    continue;
                }
            }
            merge_segments(ws, row, nseg, seg_key, seg_j, seg_n, seg_kth, idx, cnt);
        }
    }
}

// rows of a u32 array set to zero (the per-row arrival counters of the merge)
__global__ void __launch_bounds__(256) k_zero_u32(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

#define CSA2_SEL_INST(T)                                                                       \
    template __global__ void k_index_select<T>(                                                \
        int, int, const int32_t*, const int32_t*, const uint8_t*, const float*, const uint8_t*, \
        const uint8_t*, int64_t, int, int, int, int, int32_t*, int32_t*, uint32_t*, int32_t*,  \
        int32_t*, uint32_t*, uint32_t*);
CSA2_SEL_INST(1)
CSA2_SEL_INST(4)
CSA2_SEL_INST(8)
#undef CSA2_SEL_INST

}  // namespace csa2
