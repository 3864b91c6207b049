// Device helpers shared by the indexer kernels: the causal candidate count,
// the ReLU, the head sums across lane rows, order-preserving score keys, wave
// scans and reductions, and the wave-wide radix threshold and ordered keep used
// by every top-512 selection.
//
// Selections follow the top-k equation of "DeepSeek V4.1 -- Pooled group ->
// Source layer, pairs pooled" with ties broken by the smaller entry: the
// larger score first, then the smaller j.
#pragma once
#include "csa2_device.h"

namespace csa2 {

// Causal candidates of the query at p = qpos0 + t: entries j < floor((p+1)/ratio)
// (ratio = 1 << rsh: 2 for pooled pairs, 1 for one entry per position), at
// most the request's n_ent valid rows and the cache's stride.
__device__ __forceinline__ int64_t cand_count(int32_t qpos0, int t, int32_t n_ent,
                                              int64_t stride, int rsh) {
    int64_t n = ((int64_t)qpos0 + t + 1) >> rsh;
    int64_t cap = n_ent < 0 ? 0 : (int64_t)n_ent;
    if (cap > stride) cap = stride;
    return n < cap ? (n < 0 ? 0 : n) : cap;
}

// max(x, 0) as one integer max on the bit pattern: every negative float
// (including -0) is a negative integer.
// One (token, head) row of the index query: 128 bf16 values -> E4M3FN codes
// with scale s = max|x| / 448 (1 for an all-zero row), and the head weight
// folded with it, wq = w * s.  Sixteen lanes (one DPP row) per row, eight
// channels per lane (lane l16 of the row): a 16-byte load, an 8-byte store,
// the row maximum in four in-row steps.
__device__ __forceinline__ void quant_index_row(const uint16_t* qrow, float w, uint8_t* q8row,
                                                float* wq_out, int l16) {
    const uint4 v = *(const uint4*)(qrow + 8 * l16);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    float x[8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf2f((uint16_t)w4[i]);
        x[2 * i + 1] = bf2f((uint16_t)(w4[i] >> 16));
        amax = fmaxf(amax, fmaxf(fabsf(x[2 * i]), fabsf(x[2 * i + 1])));
    }
#pragma unroll
    for (int s = 1; s <= 8; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 16));
    const float sc = amax > 0.0f ? div_rn(amax, 448.0f) : 1.0f;
    uint32_t c[2] = {0u, 0u};
    if (amax > 0.0f) {          // |x / sc| <= 448 (1 + 2^-23): inside e4m3_pack4's range
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = div_rn(x[i], sc);
        c[0] = e4m3_pack4(y[0], y[1], y[2], y[3]);
        c[1] = e4m3_pack4(y[4], y[5], y[6], y[7]);
    }
    *(uint2*)(q8row + 8 * l16) = uint2{c[0], c[1]};
    if (l16 == 0) *wq_out = w * sc;
}

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

// Selection keys: a score mapped to an order-preserving u32 (-0 first turned
// into +0 so equal scores compare equal; 0 never occurs for a finite score and
// marks "no element").  A wave's candidate buffer holds keys and entries in
// entry order, so ties (equal keys) are broken by position.
constexpr int WS_CAP = 1024;          // per-wave candidate buffer
constexpr int WS_WAVES = 4;           // lists per block

__device__ __forceinline__ uint32_t score_key(float f) {
    f = f + 0.0f;   // -0 -> +0 so equal scores compare equal
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inverse of score_key for keys of finite scores
__device__ __forceinline__ float key_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

struct WaveSel {
    uint32_t key[WS_CAP];
    int32_t j[WS_CAP];
};

// Wave-wide inclusive prefix sum with DPP row shifts and row broadcasts (no LDS).
__device__ __forceinline__ uint32_t wave_scan_add(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}
// Wave-wide min / max of u32 values (DPP; lanes outside a row keep the identity),
// returned in every lane.
template <int CTRL, int RMASK>
__device__ __forceinline__ uint32_t dpp_min(uint32_t v) {
    return min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)0xFFFFFFFFu, (int)v, CTRL, RMASK, 0xf, false));
}
template <int CTRL, int RMASK>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, RMASK, 0xf, false));
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
    v = dpp_min<0x111, 0xf>(v);
    v = dpp_min<0x112, 0xf>(v);
    v = dpp_min<0x114, 0xf>(v);
    v = dpp_min<0x118, 0xf>(v);
    v = dpp_min<0x142, 0xa>(v);
    v = dpp_min<0x143, 0xc>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = dpp_max<0x111, 0xf>(v);
    v = dpp_max<0x112, 0xf>(v);
    v = dpp_max<0x114, 0xf>(v);
    v = dpp_max<0x118, 0xf>(v);
    v = dpp_max<0x142, 0xa>(v);
    v = dpp_max<0x143, 0xc>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Reductions over a 16-lane row (DPP row rotations by 1, 2, 4 and 8): every
// lane of the row gets the row's result.
__device__ __forceinline__ uint32_t row_sum(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false);   // row_ror:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false);   // row_ror:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false);   // row_ror:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);   // row_ror:8
    return v;
}
__device__ __forceinline__ uint32_t row_min(uint32_t v) {
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));
    return v;
}
__device__ __forceinline__ uint32_t row_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));
    return v;
}

// Per 16-lane row: a key theta that at least r and at most rhi of the row's
// 16 x NS keys reach (halving the row's key range), or, when repeated keys
// leave none, the largest key that at least r reach.  Needs r <= 16 * NS.
template <int NS>
__device__ __forceinline__ uint32_t row_threshold_bisect(const uint32_t (&kv)[NS], uint32_t r, uint32_t rhi) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        lo = min(lo, kv[s]);
        hi = max(hi, kv[s]);
    }
    uint32_t a = row_min(lo);                       // at least r keys >= a
    uint64_t b = (uint64_t)row_max(hi) + 1u;        // fewer than r keys >= b
    bool done = false;
    for (int it = 0; it < 33; ++it) {               // the interval halves every step
        done = done || b - a <= 1u;
        if (__ballot(!done) == 0ull) break;
        const uint32_t mid = (uint32_t)(a + ((b - a) >> 1));
        uint32_t c = 0u;
#pragma unroll
        for (int s = 0; s < NS; ++s) c += kv[s] >= mid ? 1u : 0u;
        c = row_sum(c);
        if (!done) {
            if (c >= r) {
                a = mid;
                done = c <= rhi;
            } else {
                b = mid;
            }
        }
    }
    return a;
}

// Wave-wide sum of u32 values, returned in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_add(v), 63);
}

// How many of the buffered keys (R register rows of 64, 0 = no element) reach
// x: a ballot and a scalar bit count per row, the same in every lane.
template <int R>
__device__ __forceinline__ uint32_t wave_count_ge(const uint32_t (&kr)[R], uint32_t x) {
    uint32_t c = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) c += (uint32_t)__popcll(__ballot(kr[r] >= x));
    return c;
}

// A key theta that at least k and at most `limit` of the buffered keys (held in
// registers as below, 0 = no element) reach, found by halving the interval
// [smallest key, largest key]: each step counts the keys >= its middle.
// Returns 0 when no such theta exists (so many keys equal one value that every
// threshold leaves either fewer than k or more than `limit`; all keys equal
// included).  The caller's buffer holds more than `limit` keys.
template <int R>
__device__ __forceinline__ uint32_t wave_threshold_bisect(const uint32_t (&kr)[R], uint32_t k, uint32_t limit) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (kr[r] != 0u) lo = min(lo, kr[r]);
        hi = max(hi, kr[r]);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    uint32_t a = lo;                        // at least k keys >= a
    uint64_t b = (uint64_t)hi + 1u;         // fewer than k keys >= b
    while (b - a > 1u) {
        const uint32_t mid = (uint32_t)(a + ((b - a) >> 1));
        const uint32_t c = wave_count_ge(kr, mid);
        if (c >= k) {
            a = mid;
            if (c <= limit) return a;
        } else {
            b = mid;
        }
    }
    return 0u;
}

// The k-th largest of the buffered keys (registers as below, 0 = no element;
// at least k keys present) and in *krem_out how many of its copies belong to
// the k largest (0xFFFFFFFF: all of them), by halving [smallest, largest key]:
// each step counts the keys >= its middle.  Stops early when exactly k keys
// reach the middle (the k-th largest is then their minimum).
template <int R>
__device__ __forceinline__ uint32_t wave_kth_bisect(const uint32_t (&kr)[R], uint32_t k, uint32_t* krem_out) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (kr[r] != 0u) lo = min(lo, kr[r]);
        hi = max(hi, kr[r]);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    uint32_t a = lo;                        // at least k keys >= a
    uint64_t b = (uint64_t)hi + 1u;         // fewer than k keys >= b: cb of them
    uint32_t cb = 0u;
    while (b - a > 1u) {
        const uint32_t mid = (uint32_t)(a + ((b - a) >> 1));
        const uint32_t c = wave_count_ge(kr, mid);
        if (c == k) {
            uint32_t m = 0xFFFFFFFFu;
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (kr[r] >= mid) m = min(m, kr[r]);
            *krem_out = 0xFFFFFFFFu;
            return wave_min(m);
        }
        if (c > k) {
            a = mid;
        } else {
            b = mid;
            cb = c;
        }
    }
    *krem_out = k - cb;
    return a;
}

// Keep, in order, the buffered elements above theta and the first krem equal to
// it; the buffer (key, jb) holds keys, or with AS_SCORE the scores' bit patterns.
template <bool AS_SCORE, typename JT, int R>
__device__ __forceinline__ int wave_keep_buf(uint32_t* key, JT* jb, int nc, const uint32_t (&kr)[R],
                             uint32_t theta, uint32_t krem) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    int32_t jr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) jr[r] = 64 * r + lane < nc ? (int32_t)jb[64 * r + lane] : 0;
    uint32_t kept = 0, eq = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (64 * r >= nc) break;
        const bool valid = 64 * r + lane < nc;
        const uint64_t meq = __ballot(valid && kr[r] == theta);
        const bool keep = valid && (kr[r] > theta ||
                                    (kr[r] == theta && eq + (uint32_t)__popcll(meq & below) < krem));
        const uint64_t mk = __ballot(keep);
        if (keep) {
            const uint32_t pos = kept + (uint32_t)__popcll(mk & below);
            key[pos] = AS_SCORE ? __float_as_uint(key_score(kr[r])) : kr[r];
            jb[pos] = (JT)jr[r];
        }
        kept += (uint32_t)__popcll(mk);
        eq += (uint32_t)__popcll(meq);
    }
    return (int)kept;
}

__device__ __forceinline__ int wave_keep(WaveSel& ws, int nc, const uint32_t (&kr)[16],
                                         uint32_t theta, uint32_t krem) {
    return wave_keep_buf<false, int32_t>(ws.key, ws.j, nc, kr, theta, krem);
}

__device__ __forceinline__ void load_keys(const WaveSel& ws, int nc, uint32_t (&kr)[16]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < 16; ++r) kr[r] = 64 * r + lane < nc ? ws.key[64 * r + lane] : 0u;
}

// ---------------------------------------------------------------------------
// Top-512 selection.  Keys are the scores mapped to order-preserving u32 (-0
// first turned into +0 so equal scores compare equal; 0 never occurs for a
// finite score and marks "no element").  Ties: larger score, then smaller
// entry index; output in ascending entry order, padded with -1.
//
// One wave per list (a query row, a segment of a long row, or the merged
// candidates of a row's segments), no block barriers.  The list is streamed
// once, in order, 256 elements per step (lane l holds elements 4l..4l+3), and
// every element whose key exceeds the wave's threshold is appended to a
// per-wave LDS buffer (ballot compaction keeps list order).  When the buffer
// would overflow, a wave-wide search halving the key range finds a key K that
// between 512 and 768 of the buffered keys reach (or, when repeated keys leave
// none, the exact 512th key and how many of its copies belong to the top 512);
// the buffer is compacted to those and the threshold becomes K, now strict: a
// later element equal to K ranks below every kept one (all earlier in the
// list).  At the end an exact search of the same kind trims the buffer to 512.
// ---------------------------------------------------------------------------
struct WaveTopk {
    WaveSel& ws;
    int nc;
    uint32_t thr;     // elements with key > thr are appended (0: every element)

    // four elements per lane, in list order (lane, then q); key 0 = no element
    __device__ __forceinline__ void push(const uint32_t (&k)[4], const int32_t (&jj)[4]) {
        const int lane = threadIdx.x & 63;
        const uint64_t below = (1ull << lane) - 1ull;
        uint64_t m[4];
        uint32_t cnt = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { m[q] = __ballot(k[q] > thr); cnt += (uint32_t)__popcll(m[q]); }
        if (nc + (int)cnt > WS_CAP) {
            // keep every key >= theta, where at least 512 are >= theta: a later key
            // equal to theta ranks below all of them
            // (more than WS_CAP - 256 >= 512 are buffered: a theta between the
            // bounds, found by halving the key range, or the exact 512th key)
            uint32_t kr[16], krem = 0xFFFFFFFFu;
            load_keys(ws, nc, kr);
            uint32_t theta = wave_threshold_bisect(kr, TOPK, WS_CAP - 256);
            if (theta == 0u) theta = wave_kth_bisect(kr, TOPK, &krem);
            nc = wave_keep(ws, nc, kr, theta, krem);
            thr = theta;
            cnt = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) { m[q] = __ballot(k[q] > thr); cnt += (uint32_t)__popcll(m[q]); }
        }
        uint32_t pos = (uint32_t)nc;
#pragma unroll
        for (int q = 0; q < 4; ++q) pos += (uint32_t)__popcll(m[q] & below);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (k[q] > thr) {
                ws.key[pos] = k[q];
                ws.j[pos] = jj[q];
                ++pos;
            }
        }
        nc += (int)cnt;
    }

    // the top 512 in list order to out_j (padded with -1) and, if given, their keys;
    // *kth_out = the 512th largest key (0 when fewer than 512 elements); if kq_out
    // is given, *kq_out = the kq-th largest key (0 when fewer than kq elements)
    __device__ __forceinline__ int finish(int32_t* out_j, uint32_t* out_key, uint32_t* kth_out,
                          uint32_t kq = 0, uint32_t* kq_out = nullptr) {
        const int lane = threadIdx.x & 63;
        if (nc > TOPK) {
            uint32_t kr[16], krem;
            load_keys(ws, nc, kr);
            const uint32_t kth = wave_kth_bisect(kr, TOPK, &krem);
            nc = wave_keep(ws, nc, kr, kth, krem);
        }
        uint32_t mn = 0xFFFFFFFFu;
        for (int i = lane; i < TOPK; i += 64) {
            out_j[i] = i < nc ? ws.j[i] : -1;
            if (i < nc) {
                mn = min(mn, ws.key[i]);
                if (out_key) out_key[i] = ws.key[i];
            }
        }
        if (kth_out) *kth_out = nc == TOPK ? wave_min(mn) : 0u;
        if (kq_out) {
            uint32_t v = 0u;
            if (kq > 0 && nc >= (int)kq) {
                uint32_t kr[16], krem;
                load_keys(ws, nc, kr);
                v = wave_kth_bisect(kr, kq, &krem);
            }
            *kq_out = v;
        }
        return nc;
    }
};


// The top 512 of a row's segment winners (each segment: up to 512 keys and
// entries in entry order, its count, its 512th and ceil(512/nseg)-th keys),
// written to idx / cnt by one wave.  The largest of the segments' 512th keys
// bounds the row's 512th key from below (that segment alone holds 512 keys at
// or above it), so only keys at or above it are streamed.
__device__ __forceinline__ void merge_segments(WaveSel& ws, int64_t row, int nseg, const uint32_t* seg_key,
                               const int32_t* seg_j, const int32_t* seg_n,
                               const uint32_t* seg_kth, int32_t* idx, int32_t* cnt) {
    const int lane = threadIdx.x & 63;
    // Lower bounds of the row's 512th largest key: the largest of the segments'
    // 512th keys (that segment alone holds 512 keys at or above it), and, when
    // every segment holds at least q = ceil(512 / nseg) keys, the smallest of
    // their q-th keys (together the segments hold nseg * q >= 512 keys at or
    // above it).  Keys below the larger bound cannot be selected.
    const uint32_t kth_s = lane < nseg ? seg_kth[2 * (row * nseg + lane)] : 0u;
    const uint32_t kq_s = lane < nseg ? seg_kth[2 * (row * nseg + lane) + 1] : 0xFFFFFFFFu;
    const uint32_t kq_min = wave_min(kq_s);
    const uint32_t bound = max(wave_max(kth_s), kq_min);
    WaveTopk st{ws, 0, bound > 0u ? bound - 1u : 0u};
    // each segment's 512 slots in one step: two 256-element groups, vector loads
    auto fetch = [&](int s, uint4 (&kv)[2], int4 (&jv)[2]) {
        const int64_t it = row * nseg + s;
        int m = seg_n[it];
        m = m < 0 ? 0 : (m > TOPK ? TOPK : m);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i0 = 256 * u + 4 * lane;
            kv[u] = *(const uint4*)(seg_key + it * TOPK + i0);
            jv[u] = *(const int4*)(seg_j + it * TOPK + i0);
            if (i0 >= m) kv[u].x = 0u;
            if (i0 + 1 >= m) kv[u].y = 0u;
            if (i0 + 2 >= m) kv[u].z = 0u;
            if (i0 + 3 >= m) kv[u].w = 0u;
        }
    };
    uint4 nk[2];
    int4 nj[2];
    fetch(0, nk, nj);
    for (int s = 0; s < nseg; ++s) {
        const uint4 ck[2] = {nk[0], nk[1]};
        const int4 cj[2] = {nj[0], nj[1]};
        if (s + 1 < nseg) fetch(s + 1, nk, nj);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t k[4] = {ck[u].x, ck[u].y, ck[u].z, ck[u].w};
            const int32_t jj[4] = {cj[u].x, cj[u].y, cj[u].z, cj[u].w};
            st.push(k, jj);
        }
    }
    const int c = st.finish(idx + row * TOPK, nullptr, nullptr);
    if (lane == 0) cnt[row] = c;
}

}  // namespace csa2
