// Top-512 of the query rows of decode steps (one to eight tokens a request)
// over long caches, without writing the rows' scores.
//
// "DeepSeek V4.1 -- Pooled group -> Source layer, pairs pooled", indexer and
// top-k equations: S^I_{t,j} = sum_h w^I_{t,h} ReLU(Q^I_{h,t} . K^I_j) and
// I_t = top_512(S^I_{t,j} : j < floor((t+1)/2)) (the entries' ratio in place
// of 2).  "Inside DeepSeek V4.1", section "Attention that looks at 640
// places": every compressed entry is scored, 512 go on to attention.
//
// A decode step reads each request's index keys once, so its time is the key
// stream; writing every fp32 score and reading it back for the selection cost
// as much as a third of that stream again.  Three passes instead:
//   k_fs_threshold  one block per row quantises the row's index query, scores
//                   S = 1,024 .. 4,096 entries (runs of four spread evenly over
//                   the row) and takes a threshold th that ks .. 1.25 ks of the
//                   sample keys reach, ks = max(24, ceil(2,048 S / n)) (about
//                   2,048 of the row's n scores by the sample);
//   k_fs_scan       one wave per (row, chunk of IDX_CHUNK entries) scores the
//                   chunk and keeps the keys >= th with their entries, in entry
//                   order, in the chunk's own slots (no atomics, so the order
//                   survives); k_fs_scan_nt does it for two to eight tokens of a
//                   request in one stream of the chunk's keys;
//   k_fs_select     one block per row gathers the chunks' candidates in order
//                   and cuts the exact top 512 (ties: smaller entry) by halving
//                   the key range.
// When at least 512 keys reach th, the 512th largest key is >= th, so every
// key of the top 512 -- and every copy of the 512th -- is a candidate, and the
// cut equals the full selection.  When the sample misjudges (fewer than 512
// candidates, a chunk's slots overflow, or more candidates than the cut holds)
// and for rows of 513..FS_MIN-1 entries, one wave of k_fs_select scores the
// whole row again and selects it exactly with the streaming selection.
// Scores are the same fp32 values the other indexer kernels produce (the same
// products, head-sum order and lane sums).
#include "index_device.h"

namespace csa2 {

constexpr int FS_MIN = 16384;                      // shorter rows: the fallback
constexpr int FS_WAVES = 8;                        // waves of a select block
constexpr int FS_NSLOT = FS_WAVES * 1536;          // candidates a select block cuts
constexpr uint32_t FS_ALL = 0xFFFFFFFFu;           // threshold word: at most 512 entries, take all
constexpr uint32_t FS_SLOW = 0u;                   // threshold word: select by the fallback

// The row's index query as FP8 MFMA operands and its folded head weights.
// Lane (col, grp): head col of each 16-head tile, channel bytes 16grp..+15 and
// 64+16grp..+15 (the A layout against an FP4 B operand), weights of heads
// 4grp..4grp+3 of each tile.
struct RowQuery {
    i8 A[2];
    f4 W[2];
    __device__ __forceinline__ void load(const uint8_t* q8, const float* wq, int64_t row, int col,
                                         int grp) {
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            const int64_t hr = row * HI + tile * 16;
            const uint8_t* src = q8 + (hr + col) * DI + 16 * grp;
            const uint4 u0 = *(const uint4*)src, u1 = *(const uint4*)(src + 64);
            A[tile] = i8{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                         (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
            const float4 w4 = *(const float4*)(wq + hr + 4 * grp);
            W[tile] = f4{w4.x, w4.y, w4.z, w4.w};
        }
    }
    // this lane's part of the head sum for its entry of a 16-entry tile: the
    // tile's FP4 codes (16 bytes, block grp) and that block's E8M0 scale sc
    __device__ __forceinline__ float partial(const uint4 kc, int sc) const {
        const i8 Bv = i8{(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
        const f4 d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            A[0], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
        const f4 d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            A[1], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[0][i], relu(d0[i]), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[1][i], relu(d1[i]), acc);
        return acc;
    }
};

// entries of query row (request b, token t at position q_pos0[b] + t)
__device__ __forceinline__ int fs_row_len(const int32_t* q_pos0, const int32_t* n_entries, int b,
                                          int t, int64_t entry_stride, int rsh) {
    int64_t n = cand_count(q_pos0[b], t, n_entries[b], entry_stride, rsh);
    return (int)(n < 0 ? 0 : (n > entry_stride ? entry_stride : n));
}

// Keys >= piv among keys[0, nr) (LDS, 16-byte aligned, nr a multiple of
// 1,024; unused slots hold 0, which no point (>= 1) counts), counted by one
// wave with ballots: one vector compare and two scalar operations a key.
__device__ __forceinline__ uint32_t fs_wave_count(const uint32_t* keys, int nr, uint32_t piv) {
    const int lane = threadIdx.x & 63;
    uint32_t c = 0u;
    for (int i = 4 * lane; i < nr; i += 4 * 256) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *(const uint4*)(keys + i + 256 * u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            c += (uint32_t)__builtin_popcountll(__ballot(v[u].x >= piv));
            c += (uint32_t)__builtin_popcountll(__ballot(v[u].y >= piv));
            c += (uint32_t)__builtin_popcountll(__ballot(v[u].z >= piv));
            c += (uint32_t)__builtin_popcountll(__ballot(v[u].w >= piv));
        }
    }
    return c;
}

// Search of the key interval [a, bnd) for a key th with k <= #(keys >= th) <=
// lim, given ca = #(keys >= a) >= k > cb = #(keys >= bnd): each step the
// block's eight waves count the keys at eight evenly spaced points of the
// interval (one point a wave, one barrier a step; the counts alternate
// between two slot sets), so the interval shrinks ninefold per step.  The
// counts fall as the points rise, so the points that k keys reach come first
// and, among them, those that at most lim keys reach come last.  Ends at the
// first point whose count is in [k, lim] (hit), else when bnd = a + 1: then a
// is the k-th largest key, ca keys reach it and cb pass it.
struct FsSearch {
    uint32_t a, ca, cb;
    bool hit;
};
__device__ __forceinline__ FsSearch fs_pivot_search(const uint32_t* keys, int nr, uint32_t a,
                                                    uint64_t bnd, uint32_t ca, uint32_t cb,
                                                    uint32_t k, uint32_t lim,
                                                    uint32_t (*cbuf)[FS_WAVES]) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    constexpr uint32_t NP = FS_WAVES + 1;
    int par = 0;
    while (bnd - a > 1u) {
        // point i = a + floor(w (i + 1) / 9) in 32-bit arithmetic (w < 2^32: a >= 1)
        const uint32_t w = (uint32_t)(bnd - a), wq = w / NP, wr = w - wq * NP;
        auto point = [&](int i) { return a + wq * (uint32_t)(i + 1) + wr * (uint32_t)(i + 1) / NP; };
        const uint32_t c = fs_wave_count(keys, nr, point(wave));
        if (lane == 0) cbuf[par][wave] = c;
        __syncthreads();
        const uint32_t cl = cbuf[par][lane & (FS_WAVES - 1)];
        par ^= 1;
        const bool mine = lane < FS_WAVES;
        const int nk = __builtin_popcountll(__ballot(mine && cl >= k));    // points 0 .. nk-1 reach k
        const int nl = __builtin_popcountll(__ballot(mine && cl > lim));   // points 0 .. nl-1 pass lim
        if (nl < nk) return FsSearch{point(nl), (uint32_t)__shfl((int)cl, nl), 0u, true};
        const uint32_t a2 = nk > 0 ? point(nk - 1) : a;
        if (nk > 0) ca = (uint32_t)__shfl((int)cl, nk - 1);
        if (nk < FS_WAVES) {
            bnd = point(nk);
            cb = (uint32_t)__shfl((int)cl, nk);
        }
        a = a2;
    }
    return FsSearch{a, ca, cb, false};
}

// ---- threshold: one block of eight waves per row ---------------------------
// Also quantises the row's index query (the 32 head rows as k_quant_index_query
// does) into q8 / wq for the scan and the cut; the sample's key loads are
// issued first, so they are in flight while the query is quantised.
__global__ void __launch_bounds__(64 * FS_WAVES) k_fs_threshold(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const uint16_t* __restrict__ qI, const float* __restrict__ wI, uint8_t* __restrict__ q8,
    float* __restrict__ wq, const uint8_t* __restrict__ ki_codes,
    const uint8_t* __restrict__ ki_scales, int64_t entry_stride, int rsh,
    uint32_t* __restrict__ th_out) {
    __shared__ __attribute__((aligned(16))) uint32_t skey[4096];
    __shared__ uint32_t cbuf[2][FS_WAVES];
    __shared__ uint32_t smm[2][FS_WAVES];
    __shared__ __attribute__((aligned(16))) uint8_t sq8[HI * DI];
    __shared__ __attribute__((aligned(16))) float swq[HI];
    const int row = blockIdx.x;                     // query row: request b, token t
    if (row >= B * Tq) return;
    const int b = row / Tq, t = row - b * Tq;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;
    const int n = fs_row_len(q_pos0, n_entries, b, t, entry_stride, rsh);
    if (n <= TOPK) {                    // every entry is taken: no scan, no query needed
        if (tid == 0) th_out[row] = FS_ALL;
        return;
    }
    const bool sample = n >= FS_MIN;
    // S = 1024 m samples (m = 1, 2 or 4 as the row passes 65,536 and 131,072
    // entries) in S/4 runs of four consecutive entries (two whole 128-byte
    // lines of codes and one line of scales per run, a quarter of the lines
    // single entries would touch): sample i is entry 4 floor(r n / (4 R)) +
    // (i mod 4), r = floor(i / 4), R = S / 4; wave w scores samples
    // 128 m w .. 128 m (w + 1) - 1 in m rounds of eight tiles of sixteen, the
    // next round's loads in flight during the current one's products
    const int lm = n <= 65536 ? 0 : (n <= 131072 ? 1 : 2), m = 1 << lm;
    const int S = 1024 << lm;
    const uint8_t* kb = ki_codes + (int64_t)b * entry_stride * 64 + 16 * grp;
    const uint8_t* sb = ki_scales + (int64_t)b * entry_stride * 4 + grp;
    uint4 kc[2][8];
    int sc[2][8];
    auto issue = [&](int rnd, int buf) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = 128 * (m * wave + rnd) + 16 * u + col;
            const int64_t e = ((((int64_t)(i >> 2) * n) >> (8 + lm)) & ~(int64_t)3) + (i & 3);
            kc[buf][u] = *(const uint4*)(kb + e * 64);
            sc[buf][u] = (int)sb[e * 4];
        }
    };
    if (sample) issue(0, 0);
    // the query: head row tid >> 4, sixteen lanes each, into LDS, then to q8 / wq
    {
        const int r = tid >> 4, l16 = tid & 15;
        const int64_t gr = (int64_t)row * HI + r;
        quant_index_row(qI + gr * DI, wI[gr], &sq8[r * DI], &swq[r], l16);
        __syncthreads();
        *(uint2*)(q8 + gr * DI + 8 * l16) = *(const uint2*)&sq8[r * DI + 8 * l16];
        if (l16 == 0) wq[gr] = swq[r];
    }
    if (!sample) {                      // 513 .. FS_MIN - 1 entries: the cut's fallback
        if (tid == 0) th_out[row] = FS_SLOW;
        return;
    }
    RowQuery q;
    q.load(sq8, swq, 0, col, grp);
#pragma unroll
    for (int rnd = 0; rnd < 4; ++rnd) {        // unrolled: the buffers stay in registers
        if (rnd >= m) break;
            if (rnd + 1 < m) issue(rnd + 1, (rnd + 1) & 1);
#pragma unroll
        for (int u0 = 0; u0 < 8; u0 += 4) {
            float p[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) p[g] = q.partial(kc[rnd & 1][u0 + g], sc[rnd & 1][u0 + g]);
            // lane 16g + col now holds sample 128(m w + rnd) + 16(u0 + g) + col
            skey[128 * (m * wave + rnd) + 16 * u0 + lane] =
                score_key(rowsum_scatter4(p[0], p[1], p[2], p[3]));
        }
    }
    __syncthreads();
    const uint32_t ks = (uint32_t)max((int64_t)24, ((int64_t)S * 2048 + n - 1) / n);
    // A key th that ks .. ks + ks/4 of the S sample keys reach (about 2,048 of the
    // row's scores by the sample, at least 24 sample keys above th); with
    // repeated keys and no such key, the ks-th largest sample key.
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int i = tid + 64 * FS_WAVES * e;
        if (i < S) {
            lo = min(lo, skey[i]);
            hi = max(hi, skey[i]);
        }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) { smm[0][wave] = lo; smm[1][wave] = hi; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < FS_WAVES; ++w) { lo = min(lo, smm[0][w]); hi = max(hi, smm[1][w]); }
    const uint32_t a =
        fs_pivot_search(skey, S, lo, (uint64_t)hi + 1u, (uint32_t)S, 0u, ks, ks + ks / 4, cbuf).a;
    if (tid == 0) th_out[row] = a;      // >= the smallest finite key: never 0 or FS_ALL
}

// ---- filter, single-token rows: one wave per (row, chunk) --------------------
// ck/cj [rows][n_ch][wcap]: the chunk's keys >= th and their entries, in entry
// order; ccnt [rows][n_ch]: how many passed (more than wcap: the slots overflowed).
__global__ void __launch_bounds__(256) k_fs_scan(
    int B, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const uint8_t* __restrict__ q8, const float* __restrict__ wq,
    const uint8_t* __restrict__ ki_codes, const uint8_t* __restrict__ ki_scales,
    int64_t entry_stride, int n_ch, int rsh, int wcap, const uint32_t* __restrict__ th_in,
    uint32_t* __restrict__ ck, int32_t* __restrict__ cj, int32_t* __restrict__ ccnt) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    if (item >= (int64_t)B * n_ch) return;
    const int b = (int)(item / n_ch), ch = (int)(item - (int64_t)b * n_ch);
    const uint32_t th = th_in[b];
    if (th == FS_ALL || th == FS_SLOW) return;            // the select pass handles the row
    const int n = fs_row_len(q_pos0, n_entries, b, 0, entry_stride, rsh);
    const int j_begin = ch * IDX_CHUNK;
    const int64_t slot0 = item * wcap;
    if (j_begin >= n) {
        if (lane == 0) ccnt[item] = 0;
        return;
    }
    const int j_len = min(IDX_CHUNK, n - j_begin);
    const int col = lane & 15, grp = lane >> 4;
    RowQuery q;
    q.load(q8, wq, b, col, grp);
    // the query and weights complete before the key stream starts, so the
    // loop's waits only ever count key loads
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint8_t* kbase = ki_codes + ((int64_t)b * entry_stride + j_begin) * 64 + 16 * grp;
    const uint8_t* sbase = ki_scales + ((int64_t)b * entry_stride + j_begin) * 4 + grp;
    // each key is read by this wave only: non-temporal loads; each lane loads the
    // one scale byte its block needs
    auto load = [&](int jt, uint4& kc, uint32_t& sw) {
        int j = jt + col;
        j = j < j_len ? j : j_len - 1;
        const u4v k4 = __builtin_nontemporal_load((const u4v*)(kbase + (int64_t)j * 64));
        kc = uint4{k4[0], k4[1], k4[2], k4[3]};
        sw = __builtin_nontemporal_load(sbase + (int64_t)j * 4);
    };
    const uint64_t below = (1ull << lane) - 1ull;
    int nc = 0;
    uint4 kb[8];
    uint32_t sb[8];
#pragma unroll
    for (int p = 0; p < 7; ++p) {           // issued in tile order (the waits count on it)
        load(16 * p, kb[p], sb[p]);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int jt = 0; jt < j_len; jt += 128) {
        float sp[4];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            load(jt + 16 * (p + 7), kb[(p + 7) & 7], sb[(p + 7) & 7]);
            sp[p & 3] = q.partial(kb[p], (int)sb[p]);
            if ((p & 3) == 3) {
                // lane l: entry jt + 16(p - 3) + l of the chunk
                const int jl = jt + 16 * (p - 3) + lane;
                const float tot = rowsum_scatter4(sp[0], sp[1], sp[2], sp[3]);
                const uint32_t key = jl < j_len ? score_key(tot) : 0u;
                const bool adm = key != 0u && key >= th;
                const uint64_t m = __ballot(adm);
                const int pos = nc + (int)__popcll(m & below);
                if (adm && pos < wcap) {
                    ck[slot0 + pos] = key;
                    cj[slot0 + pos] = j_begin + jl;
                }
                nc += (int)__popcll(m);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (lane == 0) ccnt[item] = nc;
}

// ---- filter, NT = 2..8 tokens of a request: one wave per (request, chunk) ----
// The wave streams the chunk's keys once for all its tokens (as the score pass
// does for few query rows): per tile, up to four tokens' products and head sums
// at a time, lane row g then holding token 4r + g's scores of the tile's 16
// entries; each token keeps its own keys >= its threshold in its own slots.
// Exactly NT token slots (no padding to eight: the products and head sums of
// absent tokens would cost as much as real ones).
template <int NT>
__global__ void __launch_bounds__(256) k_fs_scan_nt(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const uint8_t* __restrict__ q8, const float* __restrict__ wq,
    const uint8_t* __restrict__ ki_codes, const uint8_t* __restrict__ ki_scales,
    int64_t entry_stride, int n_ch, int rsh, int wcap, const uint32_t* __restrict__ th_in,
    uint32_t* __restrict__ ck, int32_t* __restrict__ cj, int32_t* __restrict__ ccnt) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    if (item >= (int64_t)B * n_ch) return;
    const int b = (int)(item / n_ch), ch = (int)(item - (int64_t)b * n_ch);
    const int col = lane & 15, grp = lane >> 4;
    const int j_begin = ch * IDX_CHUNK;
    // this lane row's tokens 4r + grp: threshold, candidates in the chunk, slots
    uint32_t thr[2];
    int ncand[2];
    bool act[2];
    int64_t slot0[2], crow[2];
    int n_max = 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int t = 4 * r + grp;
        const bool valid = t < Tq;
        const int64_t row = (int64_t)b * Tq + (valid ? t : 0);
        const uint32_t th = valid ? th_in[row] : FS_SLOW;
        act[r] = valid && th != FS_ALL && th != FS_SLOW;
        thr[r] = th;
        const int n = act[r] ? fs_row_len(q_pos0, n_entries, b, t, entry_stride, rsh) : 0;
        ncand[r] = min(max(n - j_begin, 0), IDX_CHUNK);
        n_max = max(n_max, n);
        crow[r] = row * n_ch + ch;
        slot0[r] = crow[r] * wcap;
    }
    if (__ballot(act[0] || act[1]) == 0ull) return;      // every token is the cut's alone
    n_max = (int)wave_max((uint32_t)n_max);
    const int j_len = min(IDX_CHUNK, n_max - j_begin);
    if (j_len <= 0) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
            if (act[r] && col == 0) ccnt[crow[r]] = 0;
        return;
    }
    // query operands of the NT tokens
    i8 A[NT][2];
    f4 W[NT][2];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const bool ok = k < Tq;
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            const int64_t hr = ((int64_t)b * Tq + (ok ? k : 0)) * HI + tile * 16;
            const uint8_t* src = q8 + (hr + col) * DI + 16 * grp;
            const uint4 u0 = *(const uint4*)src, u1 = *(const uint4*)(src + 64);
            A[k][tile] = ok ? i8{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                                 (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w}
                            : i8{0, 0, 0, 0, 0, 0, 0, 0};
            const float4 w4 = *(const float4*)(wq + hr + 4 * grp);
            W[k][tile] = ok ? f4{w4.x, w4.y, w4.z, w4.w} : f4{0.f, 0.f, 0.f, 0.f};
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint8_t* kbase = ki_codes + ((int64_t)b * entry_stride + j_begin) * 64 + 16 * grp;
    const uint8_t* sbase = ki_scales + ((int64_t)b * entry_stride + j_begin) * 4 + grp;
    auto load = [&](int jt, uint4& kc, uint32_t& sw) {
        int j = jt + col;
        j = j < j_len ? j : j_len - 1;
        const u4v k4 = __builtin_nontemporal_load((const u4v*)(kbase + (int64_t)j * 64));
        kc = uint4{k4[0], k4[1], k4[2], k4[3]};
        sw = __builtin_nontemporal_load(sbase + (int64_t)j * 4);
    };
    const uint32_t below = (1u << col) - 1u;
    int nc[2] = {0, 0};
    auto tile = [&](int jt, const uint4 kc, const int sc) {
        const i8 Bv = i8{(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < (NT + 3) / 4; ++r) {
            constexpr int NG0 = NT < 4 ? NT : 4;
            const int ng = r == 0 ? NG0 : NT - 4;          // tokens of this group
            f4 d[4][2];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2)
                    if (k < ng)
                        d[k][t2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            A[4 * r + k][t2], Bv, f4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sc);
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (k >= ng) continue;
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[4 * r + k][0][i], relu(d[k][0][i]), acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(W[4 * r + k][1][i], relu(d[k][1][i]), acc);
                s4[k] = acc;
            }
            const float tot = rowsum_scatter4(s4[0], s4[1], s4[2], s4[3]);
            const int jl = jt + col;
            const uint32_t key = act[r] && jl < ncand[r] ? score_key(tot) : 0u;
            const bool adm = key != 0u && key >= thr[r];
            const uint32_t mr = (uint32_t)(__ballot(adm) >> (16 * grp)) & 0xFFFFu;
            const int pos = nc[r] + (int)__popc(mr & below);
            if (adm && pos < wcap) {
                ck[slot0[r] + pos] = key;
                cj[slot0[r] + pos] = j_begin + jl;
            }
            nc[r] += (int)__popc(mr);
        }
    };
    uint4 kb[4];
    uint32_t sb[4];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        load(16 * p, kb[p], sb[p]);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int jt = 0; jt < j_len; jt += 64) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            load(jt + 16 * (p + 3), kb[(p + 3) & 3], sb[(p + 3) & 3]);
            tile(jt + 16 * p, kb[p], (int)sb[p]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
        if (act[r] && col == 0) ccnt[crow[r]] = nc[r];
}

template __global__ void k_fs_scan_nt<2>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                        const float*, const uint8_t*, const uint8_t*, int64_t, int,
                                        int, int, const uint32_t*, uint32_t*, int32_t*, int32_t*);
template __global__ void k_fs_scan_nt<3>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                        const float*, const uint8_t*, const uint8_t*, int64_t, int,
                                        int, int, const uint32_t*, uint32_t*, int32_t*, int32_t*);
template __global__ void k_fs_scan_nt<4>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                        const float*, const uint8_t*, const uint8_t*, int64_t, int,
                                        int, int, const uint32_t*, uint32_t*, int32_t*, int32_t*);
template __global__ void k_fs_scan_nt<5>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                        const float*, const uint8_t*, const uint8_t*, int64_t, int,
                                        int, int, const uint32_t*, uint32_t*, int32_t*, int32_t*);
template __global__ void k_fs_scan_nt<6>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                        const float*, const uint8_t*, const uint8_t*, int64_t, int,
                                        int, int, const uint32_t*, uint32_t*, int32_t*, int32_t*);
template __global__ void k_fs_scan_nt<7>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                        const float*, const uint8_t*, const uint8_t*, int64_t, int,
                                        int, int, const uint32_t*, uint32_t*, int32_t*, int32_t*);
template __global__ void k_fs_scan_nt<8>(int, int, const int32_t*, const int32_t*, const uint8_t*,
                                        const float*, const uint8_t*, const uint8_t*, int64_t, int,
                                        int, int, const uint32_t*, uint32_t*, int32_t*, int32_t*);


// Exclusive prefix sum over the block (FS_WAVES waves); *tot = the block total.
__device__ __forceinline__ uint32_t fs_block_scan(uint32_t v, uint32_t* wsum, uint32_t* tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_scan_add(v);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0u, all = 0u;
#pragma unroll
    for (int w = 0; w < FS_WAVES; ++w) {
        const uint32_t x = wsum[w];
        before += w < wave ? x : 0u;
        all += x;
    }
    __syncthreads();
    *tot = all;
    return before + inc - v;
}

// The cut of a block's candidates sk/sj[0, total) (entry order): the 512th
// largest key K by halving the key range (block-wide counts of the keys the
// threads hold), ending early at a point p that exactly 512 keys reach (then
// the keys >= p are the top 512); else the keys > K and the first
// (512 - #(> K)) copies of K, written to out in ascending entry order.  SPT:
// consecutive slots per thread (total <= 512 SPT).
template <int SPT>
__device__ __forceinline__ void fs_cut(const uint32_t* sk, const int32_t* sj, int total,
                                       uint32_t* bc, uint32_t (*wcount)[FS_WAVES], uint32_t* wsum,
                                       int32_t* out, int32_t* cnt_out) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint32_t kv[SPT];
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
        const int s = SPT * tid + e;
        kv[e] = s < (int)total ? sk[s] : 0u;
    }
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
        if (kv[e] != 0u) lo = min(lo, kv[e]);
        hi = max(hi, kv[e]);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) { bc[wave] = lo; bc[FS_WAVES + wave] = hi; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < FS_WAVES; ++w) { lo = min(lo, bc[w]); hi = max(hi, bc[FS_WAVES + w]); }
    int par = 0;
    // keys >= th2 (th2 >= 1) over the block; one barrier a call (the wave totals
    // alternate between two slot sets)
    auto block_count = [&](uint32_t th2) -> uint32_t {
        uint32_t c = 0u;
#pragma unroll
        for (int e = 0; e < SPT; ++e) c += kv[e] >= th2 ? 1u : 0u;
        c = wave_sum(c);
        if (lane == 0) wcount[par][wave] = c;
        __syncthreads();
        uint32_t t2 = 0u;
#pragma unroll
        for (int w = 0; w < FS_WAVES; ++w) t2 += wcount[par][w];
        par ^= 1;
        return t2;
    };
    // #(keys >= a) = ca >= 512 > cb = #(keys >= bnd)
    FsSearch r{lo, (uint32_t)total, 0u, false};
    for (uint64_t bnd = (uint64_t)hi + 1u; bnd - r.a > 1u;) {
        const uint32_t mid = (uint32_t)(r.a + ((bnd - r.a) >> 1));
        const uint32_t c = block_count(mid);
        if (c >= (uint32_t)TOPK) {
            r.a = mid;
            r.ca = c;
            if (c == (uint32_t)TOPK) {
                r.hit = true;
                break;
            }
        } else {
            bnd = mid;
            r.cb = c;
        }
    }
    // taken: the keys > K and the first `take` copies of K of this thread's slots
    uint32_t K, take = 0u;
    uint32_t gt = 0u, eq = 0u;
    if (r.hit) {
        K = r.a - 1u;                           // the keys >= p: exactly 512
#pragma unroll
        for (int e = 0; e < SPT; ++e) gt += kv[e] > K;
    } else {
        K = r.a;                                // r.ca keys reach K, r.cb pass it
        const uint32_t krem = (uint32_t)TOPK - r.cb;
#pragma unroll
        for (int e = 0; e < SPT; ++e) {
            gt += kv[e] > K;
            eq += kv[e] == K;
        }
        take = eq;
        if (krem < r.ca - r.cb) {
            uint32_t eq_tot;
            const uint32_t rank0 = fs_block_scan(eq, wsum, &eq_tot);
            take = krem > rank0 ? min(krem - rank0, eq) : 0u;
        }
    }
    uint32_t sel_tot;
    uint32_t off = fs_block_scan(gt + take, wsum, &sel_tot);
    uint32_t taken = 0u;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
        const bool keep = kv[e] > K || (kv[e] == K && taken < take);
        if (keep) {
            out[off++] = sj[SPT * tid + e];
            taken += kv[e] == K;
        }
    }
    if (tid == 0) *cnt_out = TOPK;
}

// ---- cut: one block of FS_WAVES waves per row --------------------------------
__global__ void __launch_bounds__(64 * FS_WAVES) k_fs_select(
    int B, int Tq, const int32_t* __restrict__ q_pos0, const int32_t* __restrict__ n_entries,
    const uint8_t* __restrict__ q8, const float* __restrict__ wq,
    const uint8_t* __restrict__ ki_codes, const uint8_t* __restrict__ ki_scales,
    int64_t entry_stride, int n_ch, int rsh, int wcap, const uint32_t* __restrict__ th_in,
    const uint32_t* __restrict__ ck, const int32_t* __restrict__ cj,
    const int32_t* __restrict__ ccnt, int32_t* __restrict__ idx, int32_t* __restrict__ cnt) {
    __shared__ uint32_t sk[FS_NSLOT];
    __shared__ int32_t sj[FS_NSLOT];
    __shared__ WaveSel wsel;
    __shared__ uint32_t wsum[FS_WAVES];
    __shared__ uint32_t wcount[2][FS_WAVES];
    __shared__ uint32_t bc[2 * FS_WAVES + 2];
    __shared__ uint32_t spre[2 * 64 * FS_WAVES];     // a gather pass's chunk offsets and counts
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row = blockIdx.x;                     // query row: request b, token t
    if (row >= B * Tq) return;
    const int b = row / Tq, t = row - b * Tq;
    const int n = fs_row_len(q_pos0, n_entries, b, t, entry_stride, rsh);
    int32_t* out = idx + (int64_t)row * TOPK;
    // chunk tid's count is loaded beside the threshold word (the slots of a row
    // that the scan skipped hold stale values, which are then not used)
    const int k_tid = tid < n_ch ? ccnt[(int64_t)row * n_ch + tid] : 0;
    const uint32_t th = th_in[row];
    if (th == FS_ALL) {
        for (int i = tid; i < TOPK; i += 64 * FS_WAVES) out[i] = i < n ? i : -1;
        if (tid == 0) cnt[row] = n;
        return;
    }
    // the chunks' counts: total, and whether any chunk overflowed its slots
    uint32_t total = 0u;
    uint32_t k_first = 0u;                          // chunk tid's count (the first pass's)
    bool bad = th == FS_SLOW;
    if (!bad) {
        uint32_t tc = 0u, over = 0u;
        for (int c = tid; c < n_ch; c += 64 * FS_WAVES) {
            const int k = c == tid ? k_tid : ccnt[(int64_t)row * n_ch + c];
            over |= (uint32_t)(k < 0 || k > wcap);
            const uint32_t kc = (uint32_t)(k < 0 ? 0 : (k > wcap ? wcap : k));
            if (c == tid) k_first = kc;
            tc += kc;
        }
        tc = wave_sum(tc);
        over = wave_max(over);
        if (lane == 0) { bc[wave] = tc; bc[FS_WAVES + wave] = over; }
        __syncthreads();
        uint32_t ov = 0u;
#pragma unroll
        for (int w = 0; w < FS_WAVES; ++w) { total += bc[w]; ov |= bc[FS_WAVES + w]; }
        __syncthreads();
        bad = ov != 0u || total < (uint32_t)TOPK || total > (uint32_t)FS_NSLOT;
    }
    if (bad) {
        // the exact selection of the whole row: wave 0 scores it again, 64
        // entries a step (one per lane, in entry order), into the streaming selection
        if (wave != 0) return;
        const int col = lane & 15, grp = lane >> 4;
        RowQuery q;
        q.load(q8, wq, row, col, grp);
        const uint8_t* kb = ki_codes + (int64_t)b * entry_stride * 64 + 16 * grp;
        const uint8_t* sb = ki_scales + (int64_t)b * entry_stride * 4 + grp;
        WaveTopk st{wsel, 0, 0u};
        for (int jt = 0; jt < n; jt += 64) {
            float p[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                int e = jt + 16 * g + col;
                e = e < n ? e : n - 1;
                const uint4 kc = *(const uint4*)(kb + (int64_t)e * 64);
                p[g] = q.partial(kc, (int)sb[(int64_t)e * 4]);
            }
            const float tot = rowsum_scatter4(p[0], p[1], p[2], p[3]);
            const uint32_t k[4] = {jt + lane < n ? score_key(tot) : 0u, 0u, 0u, 0u};
            const int32_t jj[4] = {jt + lane, 0, 0, 0};
            st.push(k, jj);
        }
        const int c = st.finish(out, nullptr, nullptr);
        if (lane == 0) cnt[row] = c;
        return;
    }
    // gather the candidates in entry order: chunk c's to slots pre[c] .., the
    // chunks' offsets by a block scan, 512 chunks a pass; wave w copies chunks
    // w, w + 8, .., four chunks' first 128 candidates in flight at a time (a
    // chunk holds about 64 at the usual threshold), a lane per candidate
    {
        constexpr int NT = 64 * FS_WAVES;
        uint32_t run = 0u;                 // slots before this pass's chunks
        for (int c0 = 0; c0 < n_ch; c0 += NT) {
            const int c = c0 + tid;
            uint32_t k = 0u;
            if (n_ch <= NT) {
                k = k_first;
            } else if (c < n_ch) {
                const int kk = ccnt[(int64_t)row * n_ch + c];
                k = (uint32_t)(kk < 0 ? 0 : kk);
            }
            uint32_t tot;
            spre[tid] = run + fs_block_scan(k, wsum, &tot);
            spre[NT + tid] = k;
            __syncthreads();
            const int nc = min(n_ch - c0, NT);
            for (int cc0 = wave; cc0 < nc; cc0 += 4 * FS_WAVES) {
                uint32_t kq[4][2];
                int32_t jq[4][2];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int cc = cc0 + u * FS_WAVES;
                    const uint32_t kc = cc < nc ? spre[NT + cc] : 0u;
                    const int64_t s0 = ((int64_t)row * n_ch + c0 + cc) * wcap;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t i = (uint32_t)(lane + 64 * h);
                        if (i < kc) {
                            kq[u][h] = ck[s0 + i];
                            jq[u][h] = cj[s0 + i];
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int cc = cc0 + u * FS_WAVES;
                    if (cc >= nc) break;
                    const uint32_t p0 = spre[cc], kc = spre[NT + cc];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t i = (uint32_t)(lane + 64 * h);
                        if (i < kc) {
                            sk[p0 + i] = kq[u][h];
                            sj[p0 + i] = jq[u][h];
                        }
                    }
                    const int64_t s0 = ((int64_t)row * n_ch + c0 + cc) * wcap;
                    for (uint32_t i = (uint32_t)lane + 128u; i < kc; i += 64u) {
                        sk[p0 + i] = ck[s0 + i];
                        sj[p0 + i] = cj[s0 + i];
                    }
                }
            }
            __syncthreads();
            run += tot;
        }
    }
    if (total <= 12 * 64 * FS_WAVES) fs_cut<12>(sk, sj, (int)total, bc, wcount, wsum, out, cnt + row);
    else fs_cut<24>(sk, sj, (int)total, bc, wcount, wsum, out, cnt + row);
}

}  // namespace csa2
