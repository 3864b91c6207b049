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
// Persistent blocks of 12 waves, one per compute unit, walk the (query token,
// split of its rows) units.  The rows of a unit are taken 32 at a time
// ("chunks"; window rows and compressed rows never share a chunk, and each
// kind has its own compiled QK body).  Waves 0..3 ("QK waves", head group q)
// and waves 4..11 ("PV waves", channel eighth p) share the SIMDs (one QK wave
// and two PV waves each) and work one chunk apart; one block barrier B(k) per
// chunk:
//   QK wave  computes S for its 16 heads x 32 rows of chunk k with the
//            block-scaled MFMA 16x16x128 (A = the raw row codes, FP4 with their
//            own block scales or FP8; B = the query as two E4M3 terms hi + lo
//            with an E8M0 scale per 128 channels, which together reproduce the
//            bf16 query up to the smallest elements of a block); then the
//            online softmax in log2 units with a wave-local running maximum
//            that only moves when a chunk exceeds it by more than 2^32; P (bf16,
//            [head][row]), the row corrections and a "some maximum moved" flag
//            go to LDS.
//   PV wave  copies rows four chunks ahead (direct-to-LDS into five raw
//            buffers, swizzled by 16-byte unit); PV(k-1): O^T[64p.., heads] +=
//            G^T P^T with bf16 MFMA 16x16x32 on the operand converted in phase
//            k-1 (rescaled first only when a flag is set); then converts chunk
//            k: a 4-bit (FP4 rows) or 8-bit (FP8 rows) transposing LDS load hands
//            each lane one channel's values of 8 rows (the MFMA's A operand
//            layout) straight from the staged bytes, and the lane converts them
//            to bf16 -- FP4 with each row's own E8M0 block scale (exact, from a
//            per-wave fp32 scale table), FP8 unscaled (the row's fp32 scale is
//            already in P).  No bf16 copy of the rows is made.
// A unit's entries, rotary row, first window chunks and query are fetched
// while the previous unit is finished; its scalars come from LDS, copied 64
// units at a time.  At the end of a unit the QK waves normalise (sink
// included) and write the row's log-sum-exp; the PV waves write the unit's
// output during the next unit's first chunk (staged in LDS one head tile at a
// time, written as contiguous 128-byte head segments).  Window rows enter as
// E4M3 codes; their fp32 row scale multiplies the logit and is folded into P.
// Splits of a token's chunk range write (m, l, unnormalised O) partials that
// k_attn_combine merges.
#include <type_traits>

#include "csa2_device.h"

namespace csa2 {

constexpr int CH = 32;                 // rows per chunk
constexpr float LAZY_TAU = 32.0f;      // log2 headroom before the running max is moved
constexpr float LOG2E = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(4))) short s4;
typedef __attribute__((address_space(3))) s4 lds_s4;
typedef __attribute__((ext_vector_type(2))) short s2v;

// raw staging buffers: chunk k is copied four chunks ahead and read in phase
// k by the QK waves (products) and the PV waves (conversion), so five are in use
constexpr int NRAW = 5;

// Direct-to-LDS copies: every active lane copies 16 (4) bytes from a
// wave-uniform base plus its own 32-bit byte offset to lds + 16 (4) * lane;
// lds is wave-uniform and goes to M0.  The kernel uses M0 for nothing else.
// Completion is tracked by vmcnt.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4s(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(off), "s"(base), "s"(lds) : "memory");
}
// Workgroup barrier after this wave's LDS operations and all but its N most
// recent direct-to-LDS copies have completed.
template <int N>
__device__ __forceinline__ void barrier_vm() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(__attribute__((address_space(3))) const void*)p;
}
// max / sum over the four lanes l, l^16, l^32, l^48 (the 16-lane rows)
__device__ __forceinline__ float rows_max(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// max of three floats in one instruction (the logits are never NaN; no quieting)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// the two E2M1 codes of byte SEL of w, times sc, as packed bf16 (low nibble first)
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_bf16(uint32_t w, float sc) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, SEL));
}
typedef __attribute__((ext_vector_type(2))) int v2i;
typedef __attribute__((address_space(3))) v2i lds_v2i;
// P [head][32 rows] bf16, 64 bytes per head: unit u at u ^ ((h >> 2) & 3)
__device__ __forceinline__ int pb_off(int h, int u) { return h * 64 + ((u ^ ((h >> 2) & 3)) << 4); }

template <int HT, bool ZF8>
__global__ void __launch_bounds__(ATT_THREADS, 1) k_attn(
    int B, int Tq, int H, const int32_t* __restrict__ q_pos0, const uint16_t* __restrict__ Q,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scale, int cap,
    const uint8_t* __restrict__ z_codes, const uint8_t* __restrict__ z_scales,
    int64_t entry_stride, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    const float* __restrict__ sink, const float* __restrict__ rcos,
    const float* __restrict__ rsin, int64_t rope_rows, uint16_t* __restrict__ O,
    float* __restrict__ lse, int nsplit, float* __restrict__ part_O,
    float* __restrict__ part_ml, const int32_t* __restrict__ win_floor, int hsplit) {
    __shared__ __attribute__((aligned(16))) uint8_t rawc[NRAW][CH * 512];
    __shared__ __attribute__((aligned(16))) uint32_t zsc[NRAW][CH][4];
    __shared__ __attribute__((aligned(16))) float rscl[NRAW][CH];
    __shared__ __attribute__((aligned(16))) uint16_t Pb[2][64 * CH];
    __shared__ __attribute__((aligned(16))) float corb[2][16][4];   // [n16][head tile]
    __shared__ __attribute__((aligned(16))) uint32_t cflag[2][4];   // QK wave q moved a maximum
    __shared__ __attribute__((aligned(16))) float sfw[8][2][CH];    // PV wave's block scales [block][row]
    __shared__ float mfin[2][64], lfin[2][64], finf[2][64];   // [unit parity][head]
    __shared__ __attribute__((aligned(16))) uint8_t Ost[8][16 * 128];   // PV wave's output staging
    __shared__ int32_t sidx[TOPK];
    __shared__ float sinkl[64];               // sink of head h
    __shared__ float ropel[2][2][PAIRS];      // [unit parity][cos, sin] of the token's position
    __shared__ int32_t uinfo[2][3][64];       // [batch parity][cnt, q_pos0, win_floor][unit]

    const int tid = threadIdx.x;
    int lane = tid & 63;            // re-derived opaquely per QK chunk (see there)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    // roles: waves 0..3 stage the rows and take QK and the softmax for heads
    // 16q..16q+15 (q = wave); waves 4..11 take the conversion and PV for channels
    // 64p..64p+63 (p = wave - 4).  Each SIMD holds one QK wave and two PV waves.
    const bool qk_wave = wave < 4;
    const int q4 = wave & 3;
    const bool qk_on = HT == 4 || q4 < HT;
    const float lscale = 0.044194173824159216f * LOG2E;   // log2(e) / sqrt(512)
    const int nunits = B * Tq * nsplit * hsplit;

    if (wave == 0 && lane < H) dma4s(sink, 4u * (uint32_t)lane, lds_addr(&sinkl[0]));

    // The block walks its units (query row, split) in the order unit_at gives.
    // Per unit both roles pass the same barriers: start, one per chunk, final.
    // Between final(u) and start(u + 1) the PV waves write unit u's output while
    // the QK waves convert the query of unit u + 1 (its rows, entries and
    // query were fetched during unit u).  A unit's three scalars from global
    // memory (its entry count, its request's first position and window floor)
    // come from LDS, copied 64 units at a time, so that no barrier waits on a
    // scalar load.
    struct Unit {
        int row, split, h0, b, t, nwin, slot0, ncmp, nwch, k_begin, k_end;
        int64_t p, prow;
    };
    // u = unit_at(i): the block's i-th unit
    auto unit_of = [&](int u, int i) {
        const int32_t* inf = &uinfo[(i >> 6) & 1][0][i & 63];
        Unit U;
        // a unit is (query row, split, head group): a head group's 16 HT heads
        // start at h0; the groups of a row are adjacent units
        const int uh = u / hsplit;
        U.h0 = (u - uh * hsplit) * 16 * HT;
        U.row = uh / nsplit;
        U.split = uh - U.row * nsplit;
        U.b = U.row / Tq;
        U.t = U.row - U.b * Tq;
        int64_t p = (int64_t)inf[64] + U.t;
        if (p < 0) p = 0;
        U.p = p;
        U.prow = p < rope_rows ? p : rope_rows - 1;
        int64_t w0 = p - (WINDOW - 1) > 0 ? p - (WINDOW - 1) : 0;
        if (win_floor) {     // bounded replay: the window starts no earlier than s (s <= p)
            int64_t fl = inf[128];
            fl = fl > p ? p : fl;
            w0 = w0 > fl ? w0 : fl;
        }
        U.nwin = (int)(p - w0 + 1);
        U.slot0 = (int)(w0 % cap);
        int nc = inf[0];
        U.ncmp = nc < 0 ? 0 : (nc > TOPK ? TOPK : nc);
        U.nwch = (U.nwin + CH - 1) / CH;
        const int nch = U.nwch + (U.ncmp + CH - 1) / CH;
        const int cps = (nch + nsplit - 1) / nsplit;
        U.k_begin = U.split * cps;
        U.k_end = (U.k_begin + cps < nch) ? U.k_begin + cps : nch;
        return U;
    };
    const int emax = (int)entry_stride - 1;        // entries are clamped into the cache on use
    // Unit order: block b runs on XCD b % 8 (round-robin dispatch), so the
    // G/8 blocks of one XCD take G/8 consecutive units at a time and tokens
    // that share window and selected rows meet in that XCD's L2.
    const int G = gridDim.x;
    const bool xcd_order = (G & 7) == 0;
    const int G8 = G >> 3, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    auto unit_at = [&](int i) -> int {
        return xcd_order ? ((i * 8 + xcd) * G8 + slot) : (int)blockIdx.x + i * G;
    };
    // wave 0: the scalars of the block's units i0 .. i0 + 63 (past the end: row 0's)
    auto info_issue = [&](int i0) {
        const int par = (i0 >> 6) & 1;
        const int uu = unit_at(i0 + lane);
        const int row = uu < nunits ? uu / hsplit / nsplit : 0;
        const int b = row / Tq;
        dma4s(cnt, 4u * (uint32_t)row, lds_addr(&uinfo[par][0][0]));
        dma4s(q_pos0, 4u * (uint32_t)b, lds_addr(&uinfo[par][1][0]));
        if (win_floor) dma4s(win_floor, 4u * (uint32_t)b, lds_addr(&uinfo[par][2][0]));
    };
    if (wave == 0) {
        info_issue(0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    barrier_lds();

    if (qk_wave) {
        // ======================= QK waves ==================================
        const int h = 16 * q4 + n16;
        const uint32_t sel_g = 0x0c0c0400u + 0x00000101u * (uint32_t)g;
        // bf16 query of head h for a unit: lane group g's 16-channel pieces of
        // every 64 channels (block m, half s2), all sixteen loads in flight at once
        // (a wave with no heads reads head H - 1 and discards it).  Issued
        // unconditionally, so the registers hold nothing across the chunk loop.
        uint4 qraw[4][4];
        auto q_issue = [&](int b, int t, int h0) {
            const int hq = h0 + h < H ? h0 + h : H - 1;
            const uint16_t* qrow = Q + (((int64_t)b * H + hq) * Tq + t) * D;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const uint16_t* src = qrow + 128 * m + 64 * s2 + 16 * g;
                    qraw[m][2 * s2] = *(const uint4*)src;
                    qraw[m][2 * s2 + 1] = *(const uint4*)(src + 8);
                }
        };
        // ---- staging: direct-to-LDS copies of a chunk into a raw buffer.
        // QK wave q copies rows 8q..8q+7.  Rows past the chunk's end copy the
        // chunk's first row (finite values; their logits are masked).
        // Compressed rows are 256 bytes apart, window rows 512; lane j of a
        // row copies 16-byte unit j ^ (row & 15) of it to unit j, so the
        // row's unit u sits at u ^ (row & 15).  Source offsets are 32-bit,
        // relative to the request's cache base (sizes are checked for that).
        auto stage_win = [&](const Unit& V, int k, int buf) {
            const uint8_t* wrow0 = w_codes + (int64_t)V.b * cap * D;
            const float* wsc = w_scale + (int64_t)V.b * cap;
            const int base = k * CH;
            const int nv = min(V.nwin - base, CH);
#pragma unroll
            for (int h2 = 0; h2 < 4; ++h2) {
                const int rr = 8 * q4 + 2 * h2 + (lane >> 5), j = lane & 31;
                int slot = V.slot0 + base + (rr < nv ? rr : 0);
                slot = slot >= cap ? slot - cap : slot;
                dma16s(wrow0, (uint32_t)slot * D + 16u * (uint32_t)(j ^ (rr & 15)),
                       lds_addr(&rawc[buf][(8 * q4 + 2 * h2) * 512]));
            }
            if (wave == 0 && lane < CH) {
                int slot = V.slot0 + base + (lane < nv ? lane : 0);
                slot = slot >= cap ? slot - cap : slot;
                dma4s(wsc, 4u * (uint32_t)slot, lds_addr(&rscl[buf][0]));
            }
        };
        // Everything unit V needs before its first chunk, issued while the
        // previous unit is still being finished: its 512 selected entries (every
        // QK wave copies all of them: the same values, and each wave waits only
        // for its own copy), its rotary row, the window chunks among its first
        // four (raw buffers rb, rb + 1, ..); then its query, whose loads are
        // the youngest, so waiting for them (the compiler does, before
        // converting) also completes the copies.
        auto prefetch = [&](const Unit& V, int rb, int vp) {
            const int32_t* irow = idx + (int64_t)V.row * TOPK;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                dma4s(irow, 4u * (uint32_t)(64 * j + lane), lds_addr(&sidx[64 * j]));
            if (wave == 1 && lane < PAIRS) dma4s(rcos + V.prow * PAIRS, 4u * (uint32_t)lane, lds_addr(&ropel[vp][0][0]));
            if (wave == 2 && lane < PAIRS) dma4s(rsin + V.prow * PAIRS, 4u * (uint32_t)lane, lds_addr(&ropel[vp][1][0]));
            const int kw4 = min(min(V.k_begin + 4, V.nwch), V.k_end);
            for (int k = V.k_begin; k < kw4; ++k) stage_win(V, k, (rb + k - V.k_begin) % NRAW);
        };
        int rb0 = 0;                    // raw buffer of the unit's first chunk
        if (unit_at(0) < nunits) {
            const Unit U0 = unit_of(unit_at(0), 0);
            prefetch(U0, 0, 0);
            q_issue(U0.b, U0.t, U0.h0);
        }
        for (int i = 0, u = unit_at(0), up = 0; u < nunits; u = unit_at(++i), up ^= 1) {
            const Unit U = unit_of(u, i);
            const int k_begin = U.k_begin, k_end = U.k_end, nwch = U.nwch, nwin = U.nwin;
            const int ncmp = U.ncmp;
            // the next 64 units' scalars (the other half of uinfo, last read for
            // units i - 64 .. i - 1), complete before start(u)
            const bool info = wave == 0 && (i & 63) == 0 && unit_at(i + 64) < nunits;
            if (info) info_issue(i + 64);
            const int nch = k_end > k_begin ? k_end - k_begin : 0;
            const uint8_t* zc0 = z_codes + (int64_t)U.b * entry_stride * (ZF8 ? 512 : 256);
            const uint8_t* zs0 = z_scales + (int64_t)U.b * entry_stride * (ZF8 ? 4 : 16);
            auto bufi = [&](int k) { return (rb0 + k - k_begin) % NRAW; };
            // compressed chunk k (k < k_end) of this unit
            auto stage_cmp = [&](int k) {
                const int buf = bufi(k);
                const int base = (k - nwch) * CH;
                const int nv = min(ncmp - base, CH);
                if constexpr (ZF8) {
                    // FP8 rows of 512 bytes, as the window's; QK wave q copies rows 8q..8q+7
#pragma unroll
                    for (int h2 = 0; h2 < 4; ++h2) {
                        const int rr = 8 * q4 + 2 * h2 + (lane >> 5), j = lane & 31;
                        const int e = min(max(sidx[base + (rr < nv ? rr : 0)], 0), emax);
                        dma16s(zc0, (uint32_t)e * 512u + 16u * (uint32_t)(j ^ (rr & 15)),
                               lds_addr(&rawc[buf][(8 * q4 + 2 * h2) * 512]));
                    }
                    if (wave == 0 && lane < CH) {
                        const int e2 = min(max(sidx[base + (lane < nv ? lane : 0)], 0), emax);
                        dma4s(zs0, 4u * (uint32_t)e2, lds_addr(&rscl[buf][0]));
                    }
                    return;
                }
                const int ra = 8 * q4 + (lane >> 4), rb = ra + 4;
                const int e0 = min(max(sidx[base + (ra < nv ? ra : 0)], 0), emax);
                const int e1 = min(max(sidx[base + (rb < nv ? rb : 0)], 0), emax);
                const int e2 = min(max(sidx[base + ((lane & 31) < nv ? (lane & 31) : 0)], 0), emax);
                const int j = lane & 15;
                dma16s(zc0, (uint32_t)e0 * 256u + 16u * (uint32_t)(j ^ (ra & 15)),
                       lds_addr(&rawc[buf][8 * q4 * 256]));
                dma16s(zc0, (uint32_t)e1 * 256u + 16u * (uint32_t)(j ^ (rb & 15)),
                       lds_addr(&rawc[buf][(8 * q4 + 4) * 256]));
                if (wave == 0 && lane < CH) dma16s(zs0, (uint32_t)e2 * 16u, lds_addr(&zsc[buf][0][0]));
            };

            // ---- query of heads 16q..16q+15 as two E4M3 terms ----------------
            // Lane (head 16q + n16, group g) holds, for channel block M,
            // channels 128M + 16g..+15 and 128M + 64 + 16g..+15 (the FP8
            // operand layout).  One exponent s per (head, 128 channels): an FP8
            // operand's scale bytes attach to K blocks, not to the lane holding
            // the bytes, so the four lane groups of a head share it.
            // hi = E4M3(q / 2^s) (|q| / 2^s < 256), lo = E4M3((q - hi 2^s) /
            // 2^(s-4)); hi + lo reproduces the bf16 query up to the block's
            // smallest elements.
            i8 qh[4], ql[4];
            uint32_t qsh = 0x7F7F7F7Fu, qsl = 0x7F7F7F7Fu;
            if (qk_on) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    uint32_t w[16];
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const uint4 u0 = qraw[m][2 * s2], u1 = qraw[m][2 * s2 + 1];
                        w[8 * s2 + 0] = u0.x; w[8 * s2 + 1] = u0.y; w[8 * s2 + 2] = u0.z; w[8 * s2 + 3] = u0.w;
                        w[8 * s2 + 4] = u1.x; w[8 * s2 + 5] = u1.y; w[8 * s2 + 6] = u1.z; w[8 * s2 + 7] = u1.w;
                    }
                    uint32_t mx = 0;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const uint32_t a = w[j] & 0x7FFF7FFFu;
                        mx = max(mx, max(a & 0xFFFFu, a >> 16));
                    }
                    const float amax = rows_max(__uint_as_float(mx << 16));
                    int sh = amax > 0.0f ? floor_log2(amax) - 7 : 0;
                    sh = sh < -120 ? -120 : sh;
                    const float sc_hi = __uint_as_float((uint32_t)(sh + 127) << 23);
                    const float sc_lo = __uint_as_float((uint32_t)(sh - 4 + 127) << 23);
                    uint32_t hw[8], lw[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        s2v hc = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s2v{0, 0}, __builtin_bit_cast(bf2, w[2 * j]), sc_hi, false);
                        hc = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hc, __builtin_bit_cast(bf2, w[2 * j + 1]), sc_hi, true);
                        const uint32_t hcu = __builtin_bit_cast(uint32_t, hc);
                        const f2 h01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hcu, sc_hi, false);
                        const f2 h23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hcu, sc_hi, true);
                        const float x0 = __uint_as_float(w[2 * j] << 16), x1 = __uint_as_float(w[2 * j] & 0xFFFF0000u);
                        const float x2 = __uint_as_float(w[2 * j + 1] << 16), x3 = __uint_as_float(w[2 * j + 1] & 0xFFFF0000u);
                        s2v lc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s2v{0, 0}, x0 - h01[0], x1 - h01[1], sc_lo, false);
                        lc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lc, x2 - h23[0], x3 - h23[1], sc_lo, true);
                        hw[j] = hcu;
                        lw[j] = __builtin_bit_cast(uint32_t, lc);
                    }
                    qh[m] = i8{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
                    ql[m] = i8{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
                    const uint32_t bh = (uint32_t)(sh + 127), bl = (uint32_t)(sh - 4 + 127);
                    qsh = (qsh & ~(0xFFu << (8 * m))) | (bh << (8 * m));
                    qsl = (qsl & ~(0xFFu << (8 * m))) | (bl << (8 * m));
                }
            }
            // compressed chunks among the first four (after the window ones, so
            // copies stay in chunk order), once this wave's copy of the entries
            // is in LDS
            const int kc0 = k_begin > nwch ? k_begin : nwch, kc1 = min(k_begin + 4, k_end);
            if (kc0 < kc1) {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                for (int k = kc0; k < kc1; ++k) stage_cmp(k);
            }
            if (info) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // start(u): chunk k_begin staged (n later chunks in flight: n copies)
            if (k_begin + 3 < k_end) barrier_vm<3>();
            else if (k_begin + 2 < k_end) barrier_vm<2>();
            else if (k_begin + 1 < k_end) barrier_vm<1>();
            else barrier_vm<0>();

            // running maximum (log2 units) of head h and this lane's share of
            // its denominator (rows 4g..4g+3 and 16+4g..16+4g+3 of every chunk)
            float m_used = -INFINITY, l_lane = 0.0f;
            // the raw logit (Q.G, before the 1/sqrt(512) and log2 e factors) above
            // which a chunk moves the running maximum: (m_used + TAU) / lscale
            float m_thr = -INFINITY;
            auto chunk = [&](int k, auto win_c) {
                constexpr bool WIN = decltype(win_c)::value;
                constexpr bool F8 = WIN || ZF8;          // rows of E4M3 codes with a row scale
                constexpr int RB = F8 ? 512 : 256;       // row bytes
                // lane coordinates re-derived per chunk: keeps the per-lane
                // offsets below (and in the copies) from being held across the loop
                asm volatile("" : "+v"(lane));
                const int n16 = lane & 15, g = lane >> 4;
                const int buf = k & 1, rbuf = bufi(k);
                const int base = WIN ? k * CH : (k - nwch) * CH;
                const int nv = min((WIN ? nwin : ncmp) - base, CH);
                f4 acc0 = f4{0.f, 0.f, 0.f, 0.f}, acc1 = f4{0.f, 0.f, 0.f, 0.f};
                float4 r0 = make_float4(1.f, 1.f, 1.f, 1.f), r1 = r0;
                // the products go first on the SIMD: the softmax waits on them
                __builtin_amdgcn_s_setprio(2);
                if (qk_on) {
                    if constexpr (F8) {
                        // Lane (row n16 of tile 0 and 16 + n16 of tile 1, group g)
                        // takes 16-byte units (8m + g) ^ n16 and (8m + 4 + g) ^ n16
                        // of its rows for channel block m.  With X = g ^ n16 (< 16)
                        // those are X ^ 8(m & 1) + 16(m >> 1) and the same ^ 4, so
                        // the byte addresses are A, A ^ 64, A ^ 128, A ^ 192 (m = 0,
                        // 1) and the same + 256 (m = 2, 3); tile 1 is 16 rows on.
                        const uint32_t A = lds_addr(&rawc[rbuf][0]) + (uint32_t)(n16 * 512 + 16 * (g ^ n16));
                        const uint32_t Ad[4] = {A, A ^ 64u, A ^ 128u, A ^ 192u};
                        auto rd = [&](uint32_t a) {
                            const i4 v = *(const __attribute__((address_space(3))) i4*)(size_t)a;
                            return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
                        };
                        // row scales: the window's fp32 scales multiply the products
                        // below; the re-encoded compressed rows' scales are powers of
                        // two and enter the product as the rows' E8M0 block scale
                        int sa0 = 127, sa1 = 127;
                        if constexpr (!WIN) {
                            sa0 = (int)((__float_as_uint(rscl[rbuf][n16]) >> 23) & 0xFFu);
                            sa1 = (int)((__float_as_uint(rscl[rbuf][16 + n16]) >> 23) & 0xFFu);
                        }
                        auto ld = [&](int m, i8& a0, i8& a1) {
                            const uint32_t o = 256u * (uint32_t)(m >> 1);
                            const uint4 x0 = rd(Ad[2 * (m & 1)] + o), x1 = rd(Ad[2 * (m & 1) + 1] + o);
                            const uint4 y0 = rd(Ad[2 * (m & 1)] + o + 8192u), y1 = rd(Ad[2 * (m & 1) + 1] + o + 8192u);
                            a0 = i8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                            a1 = i8{(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w, (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
                        };
                        i8 a0, a1;
                        ld(0, a0, a1);
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            i8 b0, b1;
                            if (m < 3) ld(m + 1, b0, b1);
                            const int sh = (int)((qsh >> (8 * m)) & 0xFFu), sl = (int)((qsl >> (8 * m)) & 0xFFu);
                            acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, qh[m], acc0, 0, 0, 0, sa0, 0, sh);
                            acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, qh[m], acc1, 0, 0, 0, sa1, 0, sh);
                            acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, ql[m], acc0, 0, 0, 0, sa0, 0, sl);
                            acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, ql[m], acc1, 0, 0, 0, sa1, 0, sl);
                            __builtin_amdgcn_sched_barrier(0);
                            if (m < 3) { a0 = b0; a1 = b1; }
                        }
                        r0 = *(const float4*)&rscl[rbuf][4 * g];
                        r1 = *(const float4*)&rscl[rbuf][16 + 4 * g];
                    } else {
                        const uint8_t* rrow0 = &rawc[rbuf][n16 * RB];
                        const uint8_t* rrow1 = &rawc[rbuf][(16 + n16) * RB];
                        // the rows' scale bytes regrouped for lane group g: byte m = block 4m + g
                        const uint4 z0 = *(const uint4*)&zsc[rbuf][n16][0];
                        const uint4 z1 = *(const uint4*)&zsc[rbuf][16 + n16][0];
                        const uint32_t zs0v = __builtin_amdgcn_perm(__builtin_amdgcn_perm(z0.w, z0.z, sel_g),
                                                                    __builtin_amdgcn_perm(z0.y, z0.x, sel_g), 0x05040100u);
                        const uint32_t zs1v = __builtin_amdgcn_perm(__builtin_amdgcn_perm(z1.w, z1.z, sel_g),
                                                                    __builtin_amdgcn_perm(z1.y, z1.x, sel_g), 0x05040100u);
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const int uu = 16 * ((4 * m + g) ^ n16);
                            const uint4 x = *(const uint4*)(rrow0 + uu), y = *(const uint4*)(rrow1 + uu);
                            const i8 a0 = i8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
                            const i8 a1 = i8{(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
                            if (m == 1) __builtin_amdgcn_sched_barrier(0);
                            const int sh = (int)((qsh >> (8 * m)) & 0xFFu), sl = (int)((qsl >> (8 * m)) & 0xFFu);
                            const int sa0 = (int)((zs0v >> (8 * m)) & 0xFFu), sa1 = (int)((zs1v >> (8 * m)) & 0xFFu);
                            acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, qh[m], acc0, 4, 0, 0, sa0, 0, sh);
                            acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, qh[m], acc1, 4, 0, 0, sa1, 0, sh);
                            acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, ql[m], acc0, 4, 0, 0, sa0, 0, sl);
                            acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, ql[m], acc1, 4, 0, 0, sa1, 0, sl);
                        }
                    }
                }
                // the products are consumed here, so they cannot sink below the
                // priority drop (the compiler may move arithmetic across it)
                asm volatile("" : "+v"(acc0), "+v"(acc1));
                __builtin_amdgcn_s_setprio(0);
                // ---- softmax: wave-local running maximum with headroom --------
                // x: this lane's raw logits (rows 4g..4g+3 and 16+4g..16+4g+3 of the
                // chunk, head h).  The running maximum m_used (log2 units) moves
                // only when some logit passes it by TAU: the lane compares its own
                // largest logit with m_thr, and only when a lane of the wave passes
                // does the wave take the head's maximum over its four lanes.
                uint32_t moved = 0;
                if (qk_on) {
                    const float rs[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
                    float x[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[i] = WIN ? acc0[i] * rs[i] : acc0[i];
                        x[4 + i] = WIN ? acc1[i] * rs[4 + i] : acc1[i];
                    }
                    if (nv < CH) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            x[i] = 4 * g + i < nv ? x[i] : -INFINITY;
                            x[4 + i] = 16 + 4 * g + i < nv ? x[4 + i] : -INFINITY;
                        }
                    }
                    const float lmax = max3f(max3f(x[0], x[1], x[2]), max3f(x[3], x[4], x[5]), max3f(x[6], x[7], x[7]));
                    float corr = 1.0f;
                    if (__builtin_amdgcn_ballot_w64(lmax > m_thr) != 0) {
                        const float lm = rows_max(lmax) * lscale;
                        if (lm > m_used + LAZY_TAU) {
                            corr = (m_used == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_used - lm);
                            m_used = lm;
                            m_thr = (lm + LAZY_TAU) * (1.0f / lscale);
                        }
                        if (g == 0) corb[buf][n16][q4] = corr;
                        moved = __builtin_amdgcn_ballot_w64(corr != 1.0f) != 0;
                    }
                    float ps = 0.0f, pv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], lscale, -m_used));
                        ps += e;
                        pv[i] = e * rs[i];
                    }
                    l_lane = l_lane * corr + ps;
                    uint8_t* pb0 = (uint8_t*)&Pb[buf][0] + pb_off(h, (4 * g) >> 3) + 2 * ((4 * g) & 7);
                    uint8_t* pb1 = (uint8_t*)&Pb[buf][0] + pb_off(h, (16 + 4 * g) >> 3) + 2 * ((16 + 4 * g) & 7);
                    *(uint2*)pb0 = make_uint2(__builtin_bit_cast(uint32_t, bf2{(__bf16)pv[0], (__bf16)pv[1]}),
                                              __builtin_bit_cast(uint32_t, bf2{(__bf16)pv[2], (__bf16)pv[3]}));
                    *(uint2*)pb1 = make_uint2(__builtin_bit_cast(uint32_t, bf2{(__bf16)pv[4], (__bf16)pv[5]}),
                                              __builtin_bit_cast(uint32_t, bf2{(__bf16)pv[6], (__bf16)pv[7]}));
                }
                if (lane == 0) cflag[buf][q4] = moved;
                // B(k): P, corrections and flags of chunk k visible; this wave's
                // copies (the unit's first four chunks) complete
                barrier_vm<0>();
            };
            const int kw = nwch < k_end ? nwch : k_end;
            for (int k = k_begin; k < kw; ++k) chunk(k, std::true_type{});
            for (int k = (k_begin > nwch ? k_begin : nwch); k < k_end; ++k) chunk(k, std::false_type{});

            // the next unit's entries, rotary row, first window chunks and query
            // are fetched while the PV waves finish this one: its chunks take the
            // raw buffers after this unit's (the PV waves still read the last)
            {
                const int un = unit_at(i + 1);
                const bool more = un < nunits;
                const Unit N = more ? unit_of(un, i + 1) : U;
                if (more) prefetch(N, (rb0 + nch) % NRAW, up ^ 1);
                q_issue(N.b, N.t, N.h0);      // the last unit re-reads its own query
            }
            // final(u): this unit's per-head state for the PV waves: running
            // maximum and denominator (log2 units), and, for a whole row, the
            // normalisation with the sink and the row's log-sum-exp
            const float l_tot = rows_sum(l_lane);
            if (qk_on && g == 0) {
                mfin[up][h] = m_used;
                lfin[up][h] = l_tot;
                if (nsplit == 1) {
                    const float shv = sinkl[U.h0 + h] * LOG2E;
                    const float M = fmaxf(m_used, shv);
                    const float em = (m_used == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_used - M);
                    const float den = l_tot * em + __builtin_amdgcn_exp2f(shv - M);
                    finf[up][h] = em / den;
                    if (lse) lse[((int64_t)U.b * H + U.h0 + h) * Tq + U.t] = (M + log2f(den)) * 0.6931471805599453f;
                }
            }
            barrier_lds();
            rb0 = (rb0 + nch) % NRAW;
        }
    } else {
        // ======================= PV waves ==================================
        const int p8 = wave - 4;
        f4 oacc[4][HT];                 // O^T tiles: [channel tile][head tile]
        // ---- output of unit P (parity pp) -----------------------------------
        // A unit's output is written after start of the next unit, while the QK
        // waves take its first chunk.  Lane (head 16ht + n16, group g) holds
        // channels 64p + 16ct + 4g..+3.  A whole row is normalised (sink
        // included), rotated back where rotary, converted to bf16 and staged in
        // this wave's LDS, one head tile at a time, to leave as contiguous
        // 128-byte head segments (8 lanes per head; the 16-byte unit u of head
        // h's segment sits at u ^ (h & 7)).  A split writes its unnormalised
        // partial and (m, l).
        struct Done { int b, t, row, split, h0; };  // a unit whose output is pending
        auto output = [&](const Done& P, int pp) {
            uint8_t* const stage = &Ost[p8][0];
            float rco[4][2], rsi[4][2];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2) {
                    const int d0 = 64 * p8 + 16 * ct + 4 * g;
                    const int pi = d0 >= ROPE_LO ? (d0 - ROPE_LO) / 2 + q2 : 0;
                    rco[ct][q2] = ropel[pp][0][pi];
                    rsi[ct][q2] = ropel[pp][1][pi];
                }
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const int hh = 16 * ht + n16;
                if (nsplit == 1) {
                    const float f = finf[pp][hh];
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) {
                        const int d0 = 64 * p8 + 16 * ct + 4 * g;
                        float o[4] = {oacc[ct][ht][0] * f, oacc[ct][ht][1] * f, oacc[ct][ht][2] * f,
                                      oacc[ct][ht][3] * f};
                        if (d0 >= ROPE_LO) {
#pragma unroll
                            for (int q2 = 0; q2 < 2; ++q2) {
                                const float co = rco[ct][q2], si = rsi[ct][q2];
                                const float x0 = o[2 * q2], x1 = o[2 * q2 + 1];
                                o[2 * q2] = x0 * co + x1 * si;
                                o[2 * q2 + 1] = x1 * co - x0 * si;
                            }
                        }
                        const uint32_t w0v = __builtin_bit_cast(uint32_t, bf2{(__bf16)o[0], (__bf16)o[1]});
                        const uint32_t w1v = __builtin_bit_cast(uint32_t, bf2{(__bf16)o[2], (__bf16)o[3]});
                        *(uint2*)(stage + n16 * 128 + (((2 * ct + (g >> 1)) ^ (n16 & 7)) << 4) + 8 * (g & 1)) =
                            make_uint2(w0v, w1v);
                    }
                    // heads 16ht + hl + 8i, channels 64p + 8c8 .. + 7
                    const int hl = lane >> 3, c8 = lane & 7;
#pragma unroll
                    for (int i2 = 0; i2 < 2; ++i2) {
                        const int hr = hl + 8 * i2;
                        const uint4 v = *(const uint4*)(stage + hr * 128 + ((c8 ^ (hr & 7)) << 4));
                        *(uint4*)(O + (((int64_t)P.b * H + P.h0 + 16 * ht + hr) * Tq + P.t) * D + 64 * p8 + 8 * c8) = v;
                    }
                } else {
                    const int64_t pbase = ((int64_t)P.row * nsplit + P.split) * H + P.h0 + hh;
                    float* po = part_O + pbase * D;
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) *(f4*)(po + 64 * p8 + 16 * ct + 4 * g) = oacc[ct][ht];
                    if (p8 == 0 && g == 0) {
                        part_ml[pbase * 2] = mfin[pp][hh];          // log2 units
                        part_ml[pbase * 2 + 1] = lfin[pp][hh];
                    }
                }
            }
        };
        int rb0 = 0;                    // raw buffer of the unit's first chunk
        Done Uprev{0, 0, 0, 0, 0};
        int nmine = 0;                  // units taken so far
        for (int i = 0, u = unit_at(0), up = 0; u < nunits; u = unit_at(++i), up ^= 1) {
            nmine = i + 1;
            const Unit U = unit_of(u, i);
            const int k_begin = U.k_begin, k_end = U.k_end, nwch = U.nwch;
            const int nch = k_end > k_begin ? k_end - k_begin : 0;
            auto bufi = [&](int k) { return (rb0 + k - k_begin) % NRAW; };
            barrier_lds();      // start(u)
            // the previous unit's output goes out first (its stores are older
            // than this unit's copies)
            if (i > 0) output(Uprev, up ^ 1);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) oacc[ct][ht] = f4{0.f, 0.f, 0.f, 0.f};

            // A operand of chunk k for channel tile ct (channel 64p + 16ct + n16,
            // rows 8g..8g+7), converted to bf16 from the raw chunk through the
            // transposing loads: in each 16-lane group, destination lane j
            // receives element j of every source lane's 8 bytes.  FP4 rows (256
            // bytes): source lanes 2m and 2m+1 read row 8g+m, channels 32b +
            // 0..15 and 32b + 16..31 of block b, so byte m of the result holds two
            // channels of row m -- one block scale, applied exactly in the
            // conversion.  FP8 rows (512 bytes): source lanes 2m, 2m+1 read row
            // 8g+m, channels c0..c0+7 and c0+8..c0+15, so byte m is channel c0 + j
            // of row m (its fp32 row scale is in P).  Units of a staged row are
            // swizzled: unit u of row r at u ^ (r & 15).
            const int sr = 8 * g + (n16 >> 1), sh = n16 & 1;   // source row and half of this lane
            auto convert = [&](int k, bf8 (&a)[4]) {
                const int rb = bufi(k);
                if (ZF8 || k < nwch) {
                    const uint8_t* rrow = &rawc[rb][sr * 512];
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) {
                        const int u = 4 * p8 + ct;                  // channels 16u .. 16u + 15
                        const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (lds_v2i*)(rrow + 16 * (u ^ (sr & 15)) + 8 * sh));
                        const uint32_t w0 = (uint32_t)v[0], w1 = (uint32_t)v[1];
                        a[ct] = __builtin_bit_cast(bf8, make_uint4(
                            fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                            fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1)));
                    }
                } else {
                    // this wave's 64 block scales (rows 0..31 of blocks 2p, 2p+1),
                    // one per lane, as fp32 in its own table [block][row]
                    {
                        const int zr = lane & 31, zb = lane >> 5;
                        const uint8_t e = ((const uint8_t*)&zsc[rb][zr][0])[2 * p8 + zb];
                        sfw[p8][zb][zr] = e8m0_to_f32(e);
                    }
                    const uint8_t* rrow = &rawc[rb][sr * 256];
#pragma unroll
                    for (int bl = 0; bl < 2; ++bl) {
                        const int u = 2 * p8 + bl;                  // block: channels 32u .. 32u + 31
                        const v2i v = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                            (lds_v2i*)(rrow + 16 * (u ^ (sr & 15)) + 8 * sh));
                        const float4 s0 = *(const float4*)&sfw[p8][bl][8 * g];
                        const float4 s1 = *(const float4*)&sfw[p8][bl][8 * g + 4];
                        const uint32_t v0 = (uint32_t)v[0], v1 = (uint32_t)v[1];
                        const uint32_t res[8] = {fp4x2_bf16<0>(v0, s0.x), fp4x2_bf16<1>(v0, s0.y),
                                                 fp4x2_bf16<2>(v0, s0.z), fp4x2_bf16<3>(v0, s0.w),
                                                 fp4x2_bf16<0>(v1, s1.x), fp4x2_bf16<1>(v1, s1.y),
                                                 fp4x2_bf16<2>(v1, s1.z), fp4x2_bf16<3>(v1, s1.w)};
                        uint32_t lo[4], hi[4];
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            lo[d] = __builtin_amdgcn_perm(res[2 * d + 1], res[2 * d], 0x05040100u);
                            hi[d] = __builtin_amdgcn_perm(res[2 * d + 1], res[2 * d], 0x07060302u);
                        }
                        a[2 * bl] = __builtin_bit_cast(bf8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
                        a[2 * bl + 1] = __builtin_bit_cast(bf8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
                    }
                }
            };
            // PV of chunk kp: O^T[64p + 16ct + .., heads] += G^T P^T over its 32
            // rows (A converted in the previous phase), after scaling by the
            // chunk's row corrections where a QK wave moved its maximum
            auto pv = [&](int kp, const bf8 (&a)[4]) {
                const int bp = kp & 1;
                const uint4 fl = *(const uint4*)&cflag[bp][0];
                bf8 pb[HT];
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
                    pb[ht] = *(const bf8*)((const uint8_t*)&Pb[bp][0] + pb_off(16 * ht + n16, g));
                if ((fl.x | fl.y | fl.z | fl.w) != 0) {
                    // a QK wave writes its corrections only in a chunk where it moved
                    // a maximum: the head tiles of the others keep theirs
                    const float4 c4 = *(const float4*)&corb[bp][n16][0];
                    const float cr[4] = {fl.x ? c4.x : 1.0f, fl.y ? c4.y : 1.0f, fl.z ? c4.z : 1.0f,
                                         fl.w ? c4.w : 1.0f};
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                        for (int ht = 0; ht < HT; ++ht) oacc[ct][ht] *= cr[ht];
                }
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht)
                        oacc[ct][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ct], pb[ht], oacc[ct][ht], 0, 0, 0);
            };
            // copies of chunk k (k >= k_begin + 4) into its raw buffer: PV wave
            // p copies rows 4p..4p+3 (the QK waves stage the first four chunks)
            const int nwin = U.nwin, ncmp = U.ncmp, slot0 = U.slot0;
            const uint8_t* wrow0 = w_codes + (int64_t)U.b * cap * D;
            const float* wsc = w_scale + (int64_t)U.b * cap;
            const uint8_t* zc0 = z_codes + (int64_t)U.b * entry_stride * (ZF8 ? 512 : 256);
            const uint8_t* zs0 = z_scales + (int64_t)U.b * entry_stride * (ZF8 ? 4 : 16);
            // the entries of the two rows this wave copies in compressed chunk kk
            // (re-encoded rows), read one phase ahead of their copies
            auto cmp_entries = [&](int kk, int& e0, int& e1) {
                const int base = min(max(kk - nwch, 0), TOPK / CH - 1) * CH;
                const int r = 4 * p8 + (lane >> 5);
                e0 = sidx[base + r];
                e1 = sidx[base + r + 2];
            };
            int ce0 = 0, ce1 = 0;
            auto copy_chunk = [&](int k) {
                if (k >= k_end) return;
                const int buf = bufi(k);
                if (k < nwch) {
                    const int base = k * CH;
                    const int nv = min(nwin - base, CH);
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int rr = 4 * p8 + 2 * h2 + (lane >> 5), j = lane & 31;
                        int slot = slot0 + base + (rr < nv ? rr : 0);
                        slot = slot >= cap ? slot - cap : slot;
                        dma16s(wrow0, (uint32_t)slot * D + 16u * (uint32_t)(j ^ (rr & 15)),
                               lds_addr(&rawc[buf][(4 * p8 + 2 * h2) * 512]));
                    }
                    if (p8 == 0 && lane < CH) {
                        int slot = slot0 + base + (lane < nv ? lane : 0);
                        slot = slot >= cap ? slot - cap : slot;
                        dma4s(wsc, 4u * (uint32_t)slot, lds_addr(&rscl[buf][0]));
                    }
                } else if constexpr (ZF8) {
                    // rows past the chunk's end copy whatever entry their slot names,
                    // clamped into the cache: every re-encoded row is finite, and
                    // their logits are masked
                    const int base = (k - nwch) * CH;
                    const int nv = min(ncmp - base, CH);
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int rr = 4 * p8 + 2 * h2 + (lane >> 5), j = lane & 31;
                        const int e = min(max(h2 ? ce1 : ce0, 0), emax);
                        dma16s(zc0, (uint32_t)e * 512u + 16u * (uint32_t)(j ^ (rr & 15)),
                               lds_addr(&rawc[buf][(4 * p8 + 2 * h2) * 512]));
                    }
                    if (p8 == 0 && lane < CH) {
                        const int e2 = min(max(sidx[base + (lane < nv ? lane : 0)], 0), emax);
                        dma4s(zs0, 4u * (uint32_t)e2, lds_addr(&rscl[buf][0]));
                    }
                } else {
                    const int base = (k - nwch) * CH;
                    const int nv = min(ncmp - base, CH);
                    const int rr = 4 * p8 + (lane >> 4), j = lane & 15;
                    const int e = min(max(sidx[base + (rr < nv ? rr : 0)], 0), emax);
                    dma16s(zc0, (uint32_t)e * 256u + 16u * (uint32_t)(j ^ (rr & 15)),
                           lds_addr(&rawc[buf][4 * p8 * 256]));
                    if (p8 == 0 && lane < CH) {
                        const int e2 = min(max(sidx[base + (lane < nv ? lane : 0)], 0), emax);
                        dma16s(zs0, (uint32_t)e2 * 16u, lds_addr(&zsc[buf][0][0]));
                    }
                }
            };
            // phase k: copies of chunk k+4 (raw buffer (k+4) % NRAW held chunk
            // k-1, converted before B(k-1)), PV(k-1) on the operand converted in
            // phase k-1, conversion of chunk k, B(k).  B(k) needs chunk k+1
            // staged: the QK waves staged the first four; of this wave's copies
            // those of k+2, k+3, k+4 may be in flight (at least one copy each),
            // and the previous unit's output stores may be in flight until
            // B(k_begin + 3)
            auto phase = [&](int k, const bf8 (&ap)[4], bf8 (&an)[4]) {
                copy_chunk(k + 4);
                if constexpr (ZF8) cmp_entries(k + 5, ce0, ce1);
                if (k > k_begin) pv(k - 1, ap);
                // the products go out first; the conversion runs while they (and
                // the other waves of the SIMD) use the matrix core
                __builtin_amdgcn_sched_barrier(0);
                convert(k, an);
                if (k + 1 < k_begin + 4) barrier_vm<63>();   // the QK waves staged chunk k+1
                else if (k + 4 < k_end) barrier_vm<3>();
                else if (k + 3 < k_end) barrier_vm<2>();
                else if (k + 2 < k_end) barrier_vm<1>();
                else barrier_vm<0>();
            };
            bf8 a0[4], a1[4];
            if constexpr (ZF8) cmp_entries(k_begin + 4, ce0, ce1);
            for (int k = k_begin; k < k_end; ++k) {
                phase(k, a1, a0);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) a1[ct] = a0[ct];
            }
            if (k_end > k_begin) pv(k_end - 1, a1);
            barrier_lds();      // final(u): the QK waves' m, l and normalisation
            Uprev = Done{U.b, U.t, U.row, U.split, U.h0};
            rb0 = (rb0 + nch) % NRAW;
        }
        // the last unit's output
        if (nmine > 0) output(Uprev, (nmine - 1) & 1);
    }
}

// FP4 rows (E2M1 codes, one E8M0 scale per 32 channels) rewritten as E4M3
// rows with one fp32 scale per row, for attention calls that gather each
// entry many times (a prefill): the attention kernel then reads every row in
// the window's format.  Row scale S = 2^(Emax - 127 - 6), Emax the larger of
// the row's largest block exponent byte and 7 (S is a normal number, and a
// power of two, so the kernel passes it to the matrix unit as the row's E8M0
// scale); element x * 2^(E_b - 127) becomes the E4M3 code of
// x * 2^(E_b - Emax + 6), at most 6 * 2^6 = 384.  That is exact whenever every
// block exponent is within 14 of Emax (E4M3 keeps two significant bits down to
// 2^-8); a smaller block rounds to nearest even.  32 lanes per entry, 16
// elements each.
__global__ void __launch_bounds__(256) k_z_fp8_rows(int64_t n, const uint8_t* __restrict__ zc,
                                                    const uint8_t* __restrict__ zs,
                                                    uint8_t* __restrict__ oc,
                                                    float* __restrict__ os) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 5;
    const int l = threadIdx.x & 31;
    if (e >= n) return;
    const uint4 sv = *(const uint4*)(zs + e * 16);
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
    uint32_t emx = 7;       // at least 7: the row scale stays a normal fp32 number
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int b = 0; b < 4; ++b) emx = max(emx, (sw[w] >> (8 * b)) & 0xFFu);
    const int eb = (int)((sw[l >> 3] >> (8 * ((l >> 1) & 3))) & 0xFFu);
    const float f = ldexpf(1.0f, eb - (int)emx + 6);
    const uint2 c = *(const uint2*)(zc + e * 256 + 8 * l);
    const uint32_t cw[2] = {c.x, c.y};
    uint32_t out[4];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        float q[8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f2 v = b == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[w], 1.0f, 0)
                       : b == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[w], 1.0f, 1)
                       : b == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[w], 1.0f, 2)
                                : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[w], 1.0f, 3);
            q[2 * b] = v[0] * f;                // exact: f is a power of two, |v f| <= 384
            q[2 * b + 1] = v[1] * f;
        }
        out[2 * w] = e4m3_pack4(q[0], q[1], q[2], q[3]);
        out[2 * w + 1] = e4m3_pack4(q[4], q[5], q[6], q[7]);
    }
    *(uint4*)(oc + e * 512 + 16 * l) = make_uint4(out[0], out[1], out[2], out[3]);
    if (l == 0) os[e] = ldexpf(1.0f, (int)emx - 133);
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

#define CSA2_ATTN_INST(HTV, ZF)                                                                \
    template __global__ void k_attn<HTV, ZF>(int, int, int, const int32_t*, const uint16_t*,   \
                                         const uint8_t*, const float*, int, const uint8_t*,    \
                                         const uint8_t*, int64_t, const int32_t*,              \
                                         const int32_t*, const float*, const float*,           \
                                         const float*, int64_t, uint16_t*, float*, int, float*, \
                                         float*, const int32_t*, int);
CSA2_ATTN_INST(1, false)
CSA2_ATTN_INST(2, false)
CSA2_ATTN_INST(3, false)
CSA2_ATTN_INST(4, false)
CSA2_ATTN_INST(1, true)
CSA2_ATTN_INST(2, true)
CSA2_ATTN_INST(3, true)
CSA2_ATTN_INST(4, true)
#undef CSA2_ATTN_INST

}  // namespace csa2
