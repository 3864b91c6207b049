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
// One block of 8 waves per (query token, split of its rows).  The rows are
// taken 32 at a time ("chunks"; window rows and compressed rows never share a
// chunk, and each kind has its own compiled chunk body).  Per chunk:
//   staging  the chunk's raw codes (FP8 window rows or FP4 entries with their
//            E8M0 block scales) are copied straight into LDS three chunks
//            ahead (four raw buffers), swizzled by 16-byte unit;
//   QK       wave (g4 = w/2, half = w%2) computes S for 16 heads x 16 rows
//            with the block-scaled MFMA 16x16x128: A = the raw row codes (FP4
//            with their own block scales, or FP8), B = the query split into
//            two E4M3 terms hi + lo (each with an E8M0 scale per 128 channels),
//            which together reproduce the bf16 query exactly up to the
//            smallest elements of a block.  The same wave dequantises one
//            quarter of its rows' channels to bf16 for the PV product;
//   softmax  online, in log2 units, against a running maximum per head that
//            only moves when a chunk exceeds it by more than 2^32: each wave
//            writes P for its 16 rows with the current maximum, and a chunk
//            that passes the headroom (always the first) raises a flag after
//            which the whole block exchanges row-half maxima, rescales and
//            redoes P.  P (bf16) goes to LDS as [head][row], double-buffered;
//   PV       wave w owns channels 64w..64w+63 for every head: O^T += G^T P^T
//            with bf16 MFMA 16x16x32; G^T is read with the transposing LDS
//            load (ds_read_b64_tr_b16), so each bf16 row is stored once.
// One block barrier per chunk (after P), plus one on flagged chunks.
// Window rows enter as E4M3 codes; their fp32 row scale multiplies the logit
// and is folded into P.  Splits of the chunk range write (m, l, unnormalised
// O) partials that k_attn_combine merges.
#include <type_traits>

#include "csa2_device.h"

namespace csa2 {

constexpr int CH = 32;                 // rows per chunk
constexpr int ATT_THREADS = 512;       // 8 waves
constexpr float LAZY_TAU = 32.0f;      // log2 headroom before the running max is moved
constexpr float LOG2E = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(4))) short s4;
typedef __attribute__((address_space(3))) s4 lds_s4;
typedef __attribute__((ext_vector_type(2))) short s2v;

constexpr int NRAW = 4;                // raw staging buffers (chunks in flight)

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

// bf16 copy of a chunk, [row][512]: 16-byte unit u of row r sits at u ^ gb_swz(r).
// Conflict-free for the transposing reads (16 rows x 32 bytes per read, two
// half-waves of 8 rows) and for the dequantising writes (16 rows, one unit).
__device__ __forceinline__ int gb_swz(int r) {
    return (((r & 3) | ((r >> 1) & 4)) << 1) | ((r >> 2) & 1);
}
// P [head][32 rows] bf16, 64 bytes per head: unit u at u ^ ((h >> 2) & 3)
__device__ __forceinline__ int pb_off(int h, int u) { return h * 64 + ((u ^ ((h >> 2) & 3)) << 4); }

template <int HT>
__global__ void __launch_bounds__(ATT_THREADS, 1) k_attn(
    int B, int Tq, int H, const int32_t* __restrict__ q_pos0, const uint16_t* __restrict__ Q,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scale, int cap,
    const uint8_t* __restrict__ z_codes, const uint8_t* __restrict__ z_scales,
    int64_t entry_stride, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    const float* __restrict__ sink, const float* __restrict__ rcos,
    const float* __restrict__ rsin, int64_t rope_rows, uint16_t* __restrict__ O,
    float* __restrict__ lse, int nsplit, float* __restrict__ part_O,
    float* __restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) uint8_t rawc[NRAW][CH * 512];
    __shared__ __attribute__((aligned(16))) uint32_t zsc[NRAW][CH][4];
    __shared__ __attribute__((aligned(16))) float rscl[NRAW][CH];
    __shared__ __attribute__((aligned(16))) uint16_t Gb[2][CH * D];
    __shared__ __attribute__((aligned(16))) uint16_t Pb[2][64 * CH];
    __shared__ float mxb[2][2][64];
    __shared__ float cor[64];
    __shared__ int flag[2];
    __shared__ float mfin[64], lfin[2][64];
    __shared__ int32_t sidx[TOPK];
    __shared__ float sinkl[64];               // sink of head h
    __shared__ float ropel[2][PAIRS];         // cos, sin of the token's position

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    const int g4 = wave >> 1, half = wave & 1;     // QK role: head group, row half
    const bool qk = HT == 4 || g4 < HT;
    const int row = blockIdx.x;                    // b * Tq + t
    const int split = blockIdx.y;
    const int b = row / Tq, t = row - b * Tq;
    int64_t p = (int64_t)q_pos0[b] + t;
    if (p < 0) p = 0;
    const int64_t w0 = p - (WINDOW - 1) > 0 ? p - (WINDOW - 1) : 0;
    const int nwin = (int)(p - w0 + 1);
    const int slot0 = (int)(w0 % cap);
    int ncmp = cnt[row];
    ncmp = ncmp < 0 ? 0 : (ncmp > TOPK ? TOPK : ncmp);
    const int nwch = (nwin + CH - 1) / CH;
    const int nch = nwch + (ncmp + CH - 1) / CH;
    const int cps = (nch + nsplit - 1) / nsplit;
    const int k_begin = split * cps;
    const int k_end = (k_begin + cps < nch) ? k_begin + cps : nch;
    const uint8_t* wrow0 = w_codes + (int64_t)b * cap * D;
    const float* wsc = w_scale + (int64_t)b * cap;
    const uint8_t* zc0 = z_codes + (int64_t)b * entry_stride * 256;
    const uint8_t* zs0 = z_scales + (int64_t)b * entry_stride * 16;
    const int emax = (int)entry_stride - 1;        // entries are clamped into the cache on use
    const int64_t prow = p < rope_rows ? p : rope_rows - 1;

    // ---- direct copies that nothing waits for until later --------------------
    // the row's 512 selected entries (64 per wave), the sinks, the rotary row
    dma4s(idx + (int64_t)row * TOPK, 4u * (uint32_t)(64 * wave + lane), lds_addr(&sidx[64 * wave]));
    if (wave == 0 && lane < H) dma4s(sink, 4u * (uint32_t)lane, lds_addr(&sinkl[0]));
    if (wave == 1 && lane < PAIRS) dma4s(rcos + prow * PAIRS, 4u * (uint32_t)lane, lds_addr(&ropel[0][0]));
    if (wave == 2 && lane < PAIRS) dma4s(rsin + prow * PAIRS, 4u * (uint32_t)lane, lds_addr(&ropel[1][0]));

    // ---- staging: direct-to-LDS copies of chunk k into raw buffer k % NRAW ----
    // Rows past the chunk's end copy the chunk's first row (finite values; their
    // logits are masked).  Compressed rows are 256 bytes apart, window rows 512;
    // lane q of a row copies 16-byte unit q ^ (row & 15) of it to unit q, so the
    // row's unit u sits at u ^ (row & 15).  Source offsets are 32-bit, relative
    // to the request's cache base (the caller's sizes are checked for that).
    auto chunk_entries = [&](int k, int& e, int& e2) {
        if (k >= k_end || k < nwch) return;
        const int base = (k - nwch) * CH;
        const int nv = min(ncmp - base, CH);
        const int rr = 4 * wave + (lane >> 4);
        e = min(max(sidx[base + (rr < nv ? rr : 0)], 0), emax);
        e2 = min(max(sidx[base + ((lane & 31) < nv ? (lane & 31) : 0)], 0), emax);
    };
    auto dma_chunk = [&](int k, bool have_entries, int pe, int pe2) {
        if (k >= k_end) return;
        const int buf = k % NRAW;
        if (k < nwch) {
            const int base = k * CH;
            const int nv = min(nwin - base, CH);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int rr = 4 * wave + 2 * h2 + (lane >> 5), q = lane & 31;
                int slot = slot0 + base + (rr < nv ? rr : 0);
                slot = slot >= cap ? slot - cap : slot;
                dma16s(wrow0, (uint32_t)slot * D + 16u * (uint32_t)(q ^ (rr & 15)),
                       lds_addr(&rawc[buf][(4 * wave + 2 * h2) * 512]));
            }
            if (wave == 0 && lane < CH) {
                int slot = slot0 + base + (lane < nv ? lane : 0);
                slot = slot >= cap ? slot - cap : slot;
                dma4s(wsc, 4u * (uint32_t)slot, lds_addr(&rscl[buf][0]));
            }
        } else {
            if (!have_entries) chunk_entries(k, pe, pe2);
            const int rr = 4 * wave + (lane >> 4), q = lane & 15;
            dma16s(zc0, (uint32_t)pe * 256u + 16u * (uint32_t)(q ^ (rr & 15)),
                   lds_addr(&rawc[buf][4 * wave * 256]));
            if (wave == 0 && lane < CH) dma16s(zs0, (uint32_t)pe2 * 16u, lds_addr(&zsc[buf][0][0]));
        }
    };

    // window chunks among the first three need nothing else: start them now
    for (int k = k_begin; k < k_begin + 3 && k < nwch; ++k) dma_chunk(k, false, 0, 0);

    // ---- query of this wave's 16 heads as two E4M3 terms (QK waves) ---------
    // Lane (head 16*g4 + n16, group g) holds, for channel block M, channels
    // 128M + 16g..+15 and 128M + 64 + 16g..+15 (the FP8 operand layout).  One
    // exponent s per (head, 128 channels): an FP8 operand's scale bytes attach
    // to K blocks, not to the lane holding the bytes, so the four lane groups of
    // a head share it.  hi = E4M3(q / 2^s) (|q| / 2^s < 256), lo = E4M3((q - hi
    // 2^s) / 2^(s-4)); hi + lo reproduces the bf16 query up to the block's
    // smallest elements.  Wave (g4, half) converts blocks 2 half and 2 half + 1
    // and swaps them with its partner through LDS (the bf16 row buffers and P,
    // unused until the first chunk).
    i8 qh[4], ql[4];
    uint32_t qsh = 0x7F7F7F7Fu, qsl = 0x7F7F7F7Fu;
    uint4* qx = (uint4*)&Gb[0][0];                 // [g4][m][4 quads][64 lanes]
    uint32_t* qxs = (uint32_t*)&Pb[0][0];               // [g4][m][64 lanes] exponents (4 KB)
    if (qk) {
        const uint16_t* qrow = Q + (((int64_t)b * H + 16 * g4 + n16) * Tq + t) * D;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            const int m = 2 * half + mm;
            uint32_t w[16];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const uint16_t* src = qrow + 128 * m + 64 * s2 + 16 * g;
                const uint4 u0 = *(const uint4*)src, u1 = *(const uint4*)(src + 8);
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
            uint4* dst = qx + ((g4 * 4 + m) * 4) * 64 + lane;
            dst[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            dst[64] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
            dst[128] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
            dst[192] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
            qxs[(g4 * 4 + m) * 64 + lane] = (uint32_t)sh;
        }
    }
    if (tid < 2) flag[tid] = -1;
    // every copy issued so far (entries, sinks, rotary row, window chunks) is
    // older than the query loads just consumed; make the entries visible
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // sidx ready, both halves of the query converted
    if (qk) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint4* srcq = qx + ((g4 * 4 + m) * 4) * 64 + lane;
            const uint4 a0 = srcq[0], a1 = srcq[64], c0 = srcq[128], c1 = srcq[192];
            qh[m] = i8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            ql[m] = i8{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, (int)c1.x, (int)c1.y, (int)c1.z, (int)c1.w};
            const int sh = (int)qxs[(g4 * 4 + m) * 64 + lane];
            const uint32_t bh = (uint32_t)(sh + 127), bl = (uint32_t)(sh - 4 + 127);
            qsh = (qsh & ~(0xFFu << (8 * m))) | (bh << (8 * m));
            qsl = (qsl & ~(0xFFu << (8 * m))) | (bl << (8 * m));
        }
    }

    f4 oacc[4][HT];                       // O^T tiles: [channel tile][head tile]
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) oacc[ct][ht] = f4{0.f, 0.f, 0.f, 0.f};
    // QK waves, head 16*g4 + n16: running maximum (log2 units) and this lane's
    // share of the denominator (its four rows of every chunk)
    float m_used = -INFINITY, l_lane = 0.0f;
    const float lscale = 0.044194173824159216f * LOG2E;   // log2(e) / sqrt(512)

    // compressed chunks among the first three (issued after the window ones, so
    // copies stay in chunk order)
    for (int k = (k_begin > nwch ? k_begin : nwch); k < k_begin + 3; ++k) dma_chunk(k, false, 0, 0);
    // chunk k_begin staged: every staged chunk is at least one copy per wave, so
    // n later chunks in flight allow n outstanding copies
    if (k_begin + 2 < k_end) barrier_vm<2>();
    else if (k_begin + 1 < k_end) barrier_vm<1>();
    else barrier_vm<0>();

    // Per-lane constants: the QK operand lane (row 16*half + n16, group g)
    // reads unit (4m + g) ^ r15 of a compressed row and units (8m + g) ^ r15,
    // (8m + 4 + g) ^ r15 of a window row; bf16 row r's unit u is at u ^ gb_swz(r).
    const int r = 16 * half + n16, r15 = r & 15;
    const int gsw = gb_swz(r);
    const int h = 16 * g4 + n16;
    const int rr0 = 16 * half + 4 * g;             // first of this lane's four logit rows
    const uint32_t sel_g = 0x0c0c0400u + 0x00000101u * (uint32_t)g;

    // PV of chunk kp: O^T[64w + 16ct + .., heads] += G^T P^T over its 32 rows
    auto pv = [&](int kp) {
        const int bp = kp & 1;
        bf8 pb[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
            pb[ht] = *(const bf8*)((const uint8_t*)&Pb[bp][0] + pb_off(16 * ht + n16, g));
        const int sr = n16 >> 2, sq = n16 & 3;        // transposing-read source: row, 4-channel group
        const int ra_ = 8 * g + sr, rb2 = ra_ + 4;
        const uint16_t* gba = &Gb[bp][ra_ * D];
        const uint16_t* gbb = &Gb[bp][rb2 * D];
        const int swa = gb_swz(ra_), swb = gb_swz(rb2);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int c0 = 64 * wave + 16 * ct;
            const int u = (c0 >> 3) + (sq >> 1);
            const int off = 4 * (sq & 1);
            const s4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(gba + 8 * (u ^ swa) + off));
            const s4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(gbb + 8 * (u ^ swb) + off));
            const bf8 a = __builtin_bit_cast(bf8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
                oacc[ct][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[ht], oacc[ct][ht], 0, 0, 0);
        }
    };

    // One chunk; WIN selects window rows (E4M3 codes, fp32 row scales) or
    // compressed rows (E2M1 codes, E8M0 block scales) at compile time.
    auto chunk = [&](int k, auto win_c) {
        constexpr bool WIN = decltype(win_c)::value;
        const int buf = k & 1, rbuf = k % NRAW;
        const int base = WIN ? k * CH : (k - nwch) * CH;
        const int nv = min((WIN ? nwin : ncmp) - base, CH);
        const uint8_t* rrow = &rawc[rbuf][r * (WIN ? 512 : 256)];
        uint16_t* grow = &Gb[buf][r * D];

        // ---- QK: S (16 heads x 16 rows) = rows . (q_hi + q_lo), one chain ----
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
        uint32_t zs = 0;
        float rs[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (WIN) {
            if (qk) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint4 x0 = *(const uint4*)(rrow + 16 * ((8 * m + g) ^ r15));
                    const uint4 x1 = *(const uint4*)(rrow + 16 * ((8 * m + 4 + g) ^ r15));
                    const i8 a = i8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                    (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                    const int sh = (int)((qsh >> (8 * m)) & 0xFFu), sl = (int)((qsl >> (8 * m)) & 0xFFu);
                    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qh[m], acc, 0, 0, 0, 127, 0, sh);
                    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, ql[m], acc, 0, 0, 0, 127, 0, sl);
                }
            }
            const float4 q4 = *(const float4*)&rscl[rbuf][rr0];
            rs[0] = q4.x; rs[1] = q4.y; rs[2] = q4.z; rs[3] = q4.w;
        } else {
            // the row's scale bytes regrouped for lane group g: byte m = block 4m + g
            const uint4 z4 = *(const uint4*)&zsc[rbuf][r][0];
            zs = __builtin_amdgcn_perm(__builtin_amdgcn_perm(z4.w, z4.z, sel_g),
                                       __builtin_amdgcn_perm(z4.y, z4.x, sel_g), 0x05040100u);
            if (qk) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint4 x = *(const uint4*)(rrow + 16 * ((4 * m + g) ^ r15));
                    const i8 a = i8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
                    const int sh = (int)((qsh >> (8 * m)) & 0xFFu), sl = (int)((qsl >> (8 * m)) & 0xFFu);
                    const int sa = (int)((zs >> (8 * m)) & 0xFFu);
                    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qh[m], acc, 4, 0, 0, sa, 0, sh);
                    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, ql[m], acc, 4, 0, 0, sa, 0, sl);
                }
            }
        }
        // PV of the previous chunk shares this phase with the QK products
        if (k > k_begin) pv(k - 1);
        // ---- bf16 copy of channel block g4 of rows 16*half.. (for PV) ----------
        int pe = 0, pe2 = 0;
        chunk_entries(k + NRAW - 1, pe, pe2);
        if constexpr (WIN) {
            // channels 128*g4 + 16g..+15 (units 16g4 + 2g, +1) and +64 (units +8)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const uint4 x = *(const uint4*)(rrow + 16 * ((8 * g4 + 4 * s2 + g) ^ r15));
                const uint4 lo = make_uint4(fp8x2_to_bf16x2<false>(x.x), fp8x2_to_bf16x2<true>(x.x),
                                            fp8x2_to_bf16x2<false>(x.y), fp8x2_to_bf16x2<true>(x.y));
                const uint4 hi = make_uint4(fp8x2_to_bf16x2<false>(x.z), fp8x2_to_bf16x2<true>(x.z),
                                            fp8x2_to_bf16x2<false>(x.w), fp8x2_to_bf16x2<true>(x.w));
                const int u = 16 * g4 + 8 * s2 + 2 * g;
                *(uint4*)(grow + 8 * (u ^ gsw)) = lo;
                *(uint4*)(grow + 8 * ((u + 1) ^ gsw)) = hi;
            }
        } else {
            // channels 128*g4 + 32g..+31 (units 16g4 + 4g .. +3)
            const uint4 x = *(const uint4*)(rrow + 16 * ((4 * g4 + g) ^ r15));
            const float sc = e8m0_to_f32((zs >> (8 * g4)) & 0xFFu);
            const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) {
                const uint32_t w = w4[k2];
                const uint4 v = make_uint4(
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3)));
                *(uint4*)(grow + 8 * ((16 * g4 + 4 * g + k2) ^ gsw)) = v;
            }
        }
        // raw buffer (k + NRAW - 1) % NRAW held chunk k - 1, read by every wave before B(k-1)
        dma_chunk(k + NRAW - 1, true, pe, pe2);

        // ---- logits of rows rr0 + i (log2 units) and P against the running max -
        float s[4], lm;
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = acc[i] * (WIN ? lscale * rs[i] : lscale);
        if (nv < CH) {
#pragma unroll
            for (int i = 0; i < 4; ++i) s[i] = rr0 + i < nv ? s[i] : -INFINITY;
        }
        lm = rows_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        uint8_t* pbk = (uint8_t*)&Pb[buf][0] + pb_off(h, rr0 >> 3) + 2 * (rr0 & 7);
        float ps = 0.0f;
        if (qk) {
            if (g == 0) mxb[buf][half][h] = lm;
            // past the headroom (and always on the first chunk, m_used = -inf):
            // the block redoes P below with both halves' maxima
            if (lm > m_used + LAZY_TAU) flag[buf] = k;
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = __builtin_amdgcn_exp2f(s[i] - m_used);
                ps += e;
                pv[i] = WIN ? e * rs[i] : e;
            }
            const uint32_t p01 = __builtin_bit_cast(uint32_t, bf2{(__bf16)pv[0], (__bf16)pv[1]});
            const uint32_t p23 = __builtin_bit_cast(uint32_t, bf2{(__bf16)pv[2], (__bf16)pv[3]});
            *(uint2*)pbk = make_uint2(p01, p23);
        }
        // B: P, maxima, flag and bf16 rows visible; chunk k+1 staged (k+2, k+3 may be in flight)
        if (k + 3 < k_end) barrier_vm<2>();
        else if (k + 2 < k_end) barrier_vm<1>();
        else barrier_vm<0>();

        // a flagged chunk redoes P with both halves' maxima before its PV
        if (flag[buf] == k) {
            // block-uniform: move the maximum of every head whose chunk maximum
            // (both row halves) is past the headroom, rescale, redo P
            if (qk) {
                const float cm = fmaxf(lm, mxb[buf][half ^ 1][h]);
                float corr = 1.0f;
                if (cm > m_used + LAZY_TAU) {
                    corr = (m_used == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_used - cm);
                    m_used = cm;
                }
                float ps2 = 0.0f, pv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = (s[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s[i] - m_used);
                    ps2 += e;
                    pv[i] = WIN ? e * rs[i] : e;
                }
                l_lane = l_lane * corr + ps2;
                const uint32_t p01 = __builtin_bit_cast(uint32_t, bf2{(__bf16)pv[0], (__bf16)pv[1]});
                const uint32_t p23 = __builtin_bit_cast(uint32_t, bf2{(__bf16)pv[2], (__bf16)pv[3]});
                *(uint2*)pbk = make_uint2(p01, p23);
                if (half == 0 && g == 0) cor[h] = corr;
            }
            barrier_lds();
            // PV(k-1) is already in oacc; PV(k) comes with the next chunk
            float cr[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) cr[ht] = cor[16 * ht + n16];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) oacc[ct][ht] *= cr[ht];
        } else if (qk) {
            l_lane += ps;
        }
    };

    {
        const int kw = nwch < k_end ? nwch : k_end;
        for (int k = k_begin; k < kw; ++k) chunk(k, std::true_type{});
        for (int k = (k_begin > nwch ? k_begin : nwch); k < k_end; ++k) chunk(k, std::false_type{});
        if (k_end > k_begin) pv(k_end - 1);
    }

    // ---- final per-head state ----------------------------------------------
    {
        const float l_half = rows_sum(l_lane);
        if (qk && g == 0) {
            if (half == 0) mfin[h] = m_used;
            lfin[half][h] = l_half;
        }
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = 16 * ht + n16;
        const float m = mfin[h], l = lfin[0][h] + lfin[1][h];
        if (nsplit == 1) {
            const float shv = sinkl[h] * LOG2E;
            const float M = fmaxf(m, shv);
            const float em = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
            const float den = l * em + __builtin_amdgcn_exp2f(shv - M);
            const float f = em / den;
            uint16_t* orow = O + (((int64_t)b * H + h) * Tq + t) * D;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int d0 = 64 * wave + 16 * ct + 4 * g;
                float o[4] = {oacc[ct][ht][0] * f, oacc[ct][ht][1] * f, oacc[ct][ht][2] * f,
                              oacc[ct][ht][3] * f};
                if (d0 >= ROPE_LO) {
#pragma unroll
                    for (int q2 = 0; q2 < 2; ++q2) {
                        const int pi = (d0 - ROPE_LO) / 2 + q2;
                        const float co = ropel[0][pi], si = ropel[1][pi];
                        const float x0 = o[2 * q2], x1 = o[2 * q2 + 1];
                        o[2 * q2] = x0 * co + x1 * si;
                        o[2 * q2 + 1] = x1 * co - x0 * si;
                    }
                }
                const uint32_t w0v = __builtin_bit_cast(uint32_t, bf2{(__bf16)o[0], (__bf16)o[1]});
                const uint32_t w1v = __builtin_bit_cast(uint32_t, bf2{(__bf16)o[2], (__bf16)o[3]});
                *(uint2*)(orow + d0) = make_uint2(w0v, w1v);
            }
            if (lse && wave == 0 && g == 0)
                lse[((int64_t)b * H + h) * Tq + t] = (M + log2f(den)) * 0.6931471805599453f;
        } else {
            const int64_t pbase = ((int64_t)row * nsplit + split) * H + h;
            float* po = part_O + pbase * D;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) *(f4*)(po + 64 * wave + 16 * ct + 4 * g) = oacc[ct][ht];
            if (wave == 0 && g == 0) {
                part_ml[pbase * 2] = m;          // log2 units
                part_ml[pbase * 2 + 1] = l;
            }
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

#define CSA2_ATTN_INST(HTV)                                                                    \
    template __global__ void k_attn<HTV>(int, int, int, const int32_t*, const uint16_t*,       \
                                         const uint8_t*, const float*, int, const uint8_t*,    \
                                         const uint8_t*, int64_t, const int32_t*,              \
                                         const int32_t*, const float*, const float*,           \
                                         const float*, int64_t, uint16_t*, float*, int, float*, \
                                         float*);
CSA2_ATTN_INST(1)
CSA2_ATTN_INST(2)
CSA2_ATTN_INST(3)
CSA2_ATTN_INST(4)
#undef CSA2_ATTN_INST

}  // namespace csa2
