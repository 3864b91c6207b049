// Sparse shared-latent attention over compressed rows stored in the pages' own
// main-entry format: E2M1 values with one E4M3 scale per 16 channels
// ("Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV Cache", sections
// "Deriving the 890 bytes per token" and "FP4 is a storage choice", which also
// says the cache is dequantised for attention rather than multiplied in its
// storage format).  The scaled FP4 matrix instructions take one power-of-two
// scale per 32 elements, which cannot carry a 16-channel E4M3 scale, so this
// kernel dequantises every row to bf16 in LDS first (exact: a code times a scale
// has at most 6 significant bits) and runs both products as bf16 MFMA.
//
// The computation is the one of the pages' attention equations, as in the
// per-32 kernel: window rows J^w = max(0, s, p-127)..p from the FP8 ring, then
// the selected rows; S = Q G / sqrt(512); a per-head sink in the softmax
// denominator; O = A G; channels 448.. turned back by R_p^{-1}.
//
// One block of four waves per (query token, split of its rows); with several
// splits the blocks leave unnormalised partials (O, running max in log2 units,
// denominator) for the merge kernel shared with the per-32 path.  Per chunk of
// 32 rows: all waves
// copy the rows into LDS twice, row-major (the operand of Q G^T) and
// channel-major (the operand of G^T P^T); wave w then owns heads 16w..16w+15
// (its Q in registers as the MFMA A operand) and keeps its O^T in 32 tiles of
// 16 channels x 16 heads.  Window rows are copied as their E4M3 values; their
// fp32 row scale multiplies the logit and the probability instead.
#include "csa2_device.h"

namespace csa2 {

namespace {
constexpr int DQ_ROWS = 32;              // rows per chunk
constexpr int GS_PITCH = D + 8;          // row-major copy: 1040 bytes per row
constexpr int GT_PITCH = DQ_ROWS + 8;    // channel-major copy: 80 bytes per channel, and
constexpr int GT_SKEW = 32;              // 64 more bytes per block of 32 channels (banks)
constexpr int PT_PITCH = DQ_ROWS + 8;    // P^T staging: 80 bytes per head
constexpr float DQ_LOG2E = 1.4426950408889634f;
}  // namespace

__global__ void __launch_bounds__(256) k_attn_dq(
    int B, int Tq, int H, const int32_t* __restrict__ q_pos0, const uint16_t* __restrict__ Q,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scale, int cap,
    const uint8_t* __restrict__ z_codes, const uint8_t* __restrict__ z_scales,
    int64_t entry_stride, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    const float* __restrict__ sink, const float* __restrict__ rcos,
    const float* __restrict__ rsin, int64_t rope_rows, uint16_t* __restrict__ O,
    float* __restrict__ lse, const int32_t* __restrict__ win_floor, int nsplit,
    float* __restrict__ part_O, float* __restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) uint16_t Gs[DQ_ROWS * GS_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t Gt[D * GT_PITCH + (D / 32) * GT_SKEW];
    __shared__ __attribute__((aligned(16))) uint16_t Pt[4][16 * PT_PITCH];
    __shared__ float rsc[DQ_ROWS];
    __shared__ int32_t sidx[TOPK];
    __shared__ float corr_s[4][16];
    __shared__ float ml_s[4][2][16];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n16 = lane & 15, g = lane >> 4;
    const int64_t qrow = blockIdx.x / nsplit;
    const int split = (int)(blockIdx.x - qrow * nsplit);
    if (qrow >= (int64_t)B * Tq) return;
    const int b = (int)(qrow / Tq), t = (int)(qrow - (int64_t)b * Tq);
    int64_t p = (int64_t)q_pos0[b] + t;
    if (p < 0) p = 0;
    const int64_t prow = p < rope_rows ? p : rope_rows - 1;
    int64_t w0 = p - (WINDOW - 1) > 0 ? p - (WINDOW - 1) : 0;
    if (win_floor) {
        int64_t fl = win_floor[b];
        fl = fl > p ? p : fl;
        w0 = w0 > fl ? w0 : fl;
    }
    const int nwin = (int)(p - w0 + 1);
    int nc = cnt[qrow];
    nc = nc < 0 ? 0 : (nc > TOPK ? TOPK : nc);
    const int nrows = nwin + nc;
    const int64_t emax = entry_stride - 1;
    const int32_t* sel = idx + qrow * TOPK;
    const uint8_t* wrow0 = w_codes + (int64_t)b * cap * D;
    const float* wsc0 = w_scale + (int64_t)b * cap;
    const uint8_t* zc0 = z_codes + (int64_t)b * entry_stride * 256;
    const uint8_t* zs0 = z_scales + (int64_t)b * entry_stride * 32;

    const bool heads = 16 * wave < H;
    const int hq = 16 * wave + n16;          // this lane's head as an MFMA row / column
    // Q tile of heads 16w..: A operand of k-step kk holds channels 32kk + 8g..+7
    bf8 qa[16];
    if (heads) {
        const uint16_t* qsrc = Q + (((int64_t)b * H + hq) * Tq + t) * D + 8 * g;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) qa[kk] = *(const bf8*)(qsrc + 32 * kk);
    }
    f4 oacc[32];
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) oacc[ct] = f4{0.f, 0.f, 0.f, 0.f};
    // running max (log2 units) and denominator of heads 16w + 4g + i
    float m_run[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float l_run[4] = {0.f, 0.f, 0.f, 0.f};
    const float lscale = DQ_LOG2E / sqrtf((float)D);

    // copy role: rows 2rp, 2rp+1 of the chunk, channels 32cq..32cq+31 (a wave's
    // lanes take 16 row pairs of 4 channel blocks: its channel-major writes fall
    // in distinct banks)
    const int rp = tid & 15, cq = tid >> 4;
    uint16_t* const gtw = &Gt[32 * cq * GT_PITCH + cq * GT_SKEW + 2 * rp];
    const int nchunks = (nrows + DQ_ROWS - 1) / DQ_ROWS;
    const int cps = (nchunks + nsplit - 1) / nsplit;
    const int ck0 = split * cps, ck1 = ck0 + cps < nchunks ? ck0 + cps : nchunks;
    // the selected entries, clamped into the cache
    for (int k = tid; k < nc; k += 256) {
        const int32_t e = sel[k];
        sidx[k] = e < 0 ? 0 : (e > emax ? (int32_t)emax : e);
    }
    __syncthreads();
    // raw bytes of this thread's two rows of chunk ck: loaded one chunk ahead
    uint4 ra[2], rb[2];
    uint32_t rw[2];                          // window: fp32 scale bits; compressed: scale bytes
    int kind[2];                             // 0 no row, 1 window row, 2 compressed row
    auto load = [&](int ck) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int i = ck * DQ_ROWS + 2 * rp + h2;
            if (i < nwin) {
                const int64_t slot = (w0 + i) % cap;
                const uint8_t* src = wrow0 + slot * D + 32 * cq;
                ra[h2] = *(const uint4*)src;
                rb[h2] = *(const uint4*)(src + 16);
                rw[h2] = __float_as_uint(wsc0[slot]);
                kind[h2] = 1;
            } else if (i < nrows) {
                const int64_t e = sidx[i - nwin];
                ra[h2] = *(const uint4*)(zc0 + e * 256 + 16 * cq);
                rw[h2] = *(const uint16_t*)(zs0 + e * 32 + 2 * cq);
                kind[h2] = 2;
            } else {
                kind[h2] = 0;
            }
        }
    };
    if (ck0 < ck1) load(ck0);
    for (int ck = ck0; ck < ck1; ++ck) {
        // ---- copy: two rows, 32 channels each, into both LDS layouts -------
        uint32_t v[2][16];                   // packed bf16 pairs: channels 32cq + 2k, +1
        float scale[2] = {0.0f, 0.0f};       // row scale: window rows' fp32 scale, else 1 (0: no row)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            if (kind[h2] == 1) {
                const uint4 a = ra[h2], c = rb[h2];
                const uint32_t wv[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    v[h2][2 * k] = fp8x2_to_bf16x2<false>(wv[k]);
                    v[h2][2 * k + 1] = fp8x2_to_bf16x2<true>(wv[k]);
                }
                scale[h2] = __uint_as_float(rw[h2]);
            } else if (kind[h2] == 2) {
                const uint4 a = ra[h2];
                const float s0 = e4m3_to_f32(rw[h2] & 0xFFu), s1 = e4m3_to_f32(rw[h2] >> 8);
                const uint32_t wv[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float sv = k < 2 ? s0 : s1;       // words 0,1: channels 0..15
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[h2][4 * k + q] = fp4x2_e4_to_bf16x2(wv[k], q, sv);
                }
                scale[h2] = 1.0f;
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) v[h2][k] = 0u;
            }
        }
        // the previous chunk's products are done before its copies are replaced
        __syncthreads();
        if (cq == 0) {
            rsc[2 * rp] = scale[0];
            rsc[2 * rp + 1] = scale[1];
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            uint16_t* dst = &Gs[(2 * rp + h2) * GS_PITCH + 32 * cq];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                *(uint4*)(dst + 8 * u) = make_uint4(v[h2][4 * u], v[h2][4 * u + 1],
                                                    v[h2][4 * u + 2], v[h2][4 * u + 3]);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            // channels 32cq + 2k and +1: rows 2rp, 2rp+1 side by side
            const uint32_t a = v[0][k], c = v[1][k];
            *(uint32_t*)(gtw + (2 * k) * GT_PITCH) = (a & 0xFFFFu) | (c << 16);
            *(uint32_t*)(gtw + (2 * k + 1) * GT_PITCH) = (a >> 16) | (c & 0xFFFF0000u);
        }
        __syncthreads();
        if (ck + 1 < ck1) load(ck + 1);      // in flight during this chunk's products
        if (!heads) continue;

        // ---- S = Q G^T over the chunk's two tiles of 16 rows -------------------
        f4 sacc[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            sacc[rt] = f4{0.f, 0.f, 0.f, 0.f};
            const uint16_t* gsrc = &Gs[(16 * rt + n16) * GS_PITCH + 8 * g];
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
                sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], *(const bf8*)(gsrc + 32 * kk),
                                                                   sacc[rt], 0, 0, 0);
        }
        // lane holds heads 16w + 4g + i at rows 16rt + n16 of the chunk
        float z[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int r = 16 * rt + n16;
            const bool ok = ck * DQ_ROWS + r < nrows;
            const float f = rsc[r] * lscale;
#pragma unroll
            for (int i = 0; i < 4; ++i) z[rt][i] = ok ? sacc[rt][i] * f : -INFINITY;
        }
        float corr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mx = fmaxf(z[0][i], z[1][i]);
#pragma unroll
            for (int s = 1; s < 16; s <<= 1) mx = fmaxf(mx, __shfl_xor(mx, s, 64));
            const float mn = fmaxf(m_run[i], mx);
            corr[i] = m_run[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[i] - mn);
            m_run[i] = mn;
            float ps = 0.0f;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const float e = __builtin_amdgcn_exp2f(z[rt][i] - mn);
                ps += e;
                z[rt][i] = e * rsc[16 * rt + n16];      // the window row's scale goes to P
            }
#pragma unroll
            for (int s = 1; s < 16; s <<= 1) ps += __shfl_xor(ps, s, 64);
            l_run[i] = l_run[i] * corr[i] + ps;
        }
        // P^T and the corrections to the PV layout (head = column n16)
        uint16_t* pt = &Pt[wave][0];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) pt[(4 * g + i) * PT_PITCH + 16 * rt + n16] = f2bf(z[rt][i]);
        if (n16 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) corr_s[wave][4 * g + i] = corr[i];
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const float cr = corr_s[wave][n16];
        const bf8 pb = *(const bf8*)&pt[n16 * PT_PITCH + 8 * g];
        if (__any(cr != 1.0f)) {
#pragma unroll
            for (int ct = 0; ct < 32; ++ct) oacc[ct] *= cr;
        }
        // ---- O^T += G^T P^T: channel tiles of 16 --------------------------------
        const uint16_t* gt = &Gt[n16 * GT_PITCH + 8 * g];
#pragma unroll
        for (int ct = 0; ct < 32; ++ct)
            oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                *(const bf8*)(gt + 16 * ct * GT_PITCH + (ct >> 1) * GT_SKEW), pb, oacc[ct], 0, 0, 0);
        // Pt and corr_s are rewritten next chunk only after the block barrier
    }
    if (!heads) return;

    // ---- output: sink, normalisation, inverse rotation ------------------------
    if (n16 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ml_s[wave][0][4 * g + i] = m_run[i];
            ml_s[wave][1][4 * g + i] = l_run[i];
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const float m = ml_s[wave][0][n16], l = ml_s[wave][1][n16];
    if (nsplit > 1) {
        // partials of this split: O^T tiles as they are, (m, l) per head
        const int64_t pbase = (qrow * nsplit + split) * H + hq;
        float* po = part_O + pbase * D;
#pragma unroll
        for (int ct = 0; ct < 32; ++ct) *(f4*)(po + 16 * ct + 4 * g) = oacc[ct];
        if (g == 0) {
            part_ml[pbase * 2] = m;
            part_ml[pbase * 2 + 1] = l;
        }
        return;
    }
    const float shv = sink[hq] * DQ_LOG2E;
    const float M = fmaxf(m, shv);
    const float em = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    const float den = l * em + __builtin_amdgcn_exp2f(shv - M);
    const float f = em / den;
    uint16_t* orow = O + (((int64_t)b * H + hq) * Tq + t) * D;
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
        const int c0 = 16 * ct + 4 * g;
        float o[4] = {oacc[ct][0] * f, oacc[ct][1] * f, oacc[ct][2] * f, oacc[ct][3] * f};
        if (c0 >= ROPE_LO) {
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int pi = (c0 - ROPE_LO) / 2 + q2;
                const float co = rcos[prow * PAIRS + pi], si = rsin[prow * PAIRS + pi];
                const float x0 = o[2 * q2], x1 = o[2 * q2 + 1];
                o[2 * q2] = x0 * co + x1 * si;
                o[2 * q2 + 1] = x1 * co - x0 * si;
            }
        }
        *(uint2*)(orow + c0) = make_uint2((uint32_t)f2bf(o[0]) | ((uint32_t)f2bf(o[1]) << 16),
                                          (uint32_t)f2bf(o[2]) | ((uint32_t)f2bf(o[3]) << 16));
    }
    if (lse && g == 0) lse[((int64_t)b * H + hq) * Tq + t] = (M + log2f(den)) * 0.6931471805599453f;
}

}  // namespace csa2
