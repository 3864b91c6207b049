/*
 * CSA2 CPU ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, single-threaded, slow and (meant to be) obviously correct CPU
 * implementation of one Compressed Sparse Attention 2 layer as the pages
 * state it.  Only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no source with the HIP
 * library: every format, rounding rule and formula below is written out here
 * from the pages' definitions.
 *
 * Sources (cited by page title and equation/section):
 *  [P2] "DeepSeek V4.1 -- Pooled group -> Source layer, pairs pooled" (atlas,
 *       prefill view): the compressed-sparse-attention equations -- window
 *       rotation and FP8 storage, pair pooling with a softmax gate, the
 *       compressed RMSNorm, rotation at position 2j and FP4 storage, index-key
 *       projection/normalisation/rotation/FP4, the lightning-indexer score,
 *       the causal top-512, the window index set, the concatenated index
 *       space, the scaled scores, the sink softmax, the weighted sum and the
 *       inverse rotation; plus the "between forward calls" cache note.
 *  [P3] "DeepSeek V4.1 -- Window layer -> Attention RMSNorm": RMSNorm formula
 *       (mean of squares, epsilon 1e-20, gain applied after the rsqrt).
 *  [P1] "Inside DeepSeek V4.1" (blog), sections "Attention that looks at 640
 *       places" (128-token FP8 window, 512 selected entries, 32x128 FP4
 *       indexer, 64 heads sharing one latent, per-head sink) and "890 bytes"
 *       (FP4 entries with 8-bit block scales, the 22.6 value bound).
 *  [P4] "Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV Cache",
 *       sections "Deriving the 890 bytes per token" (entry byte layouts),
 *       "FP4 is a storage choice" (quantisation after RoPE, keep block size,
 *       scale type and rounding), the CSA2 section (compression ratio one is
 *       a supported case; the decoder layers use it) and "Bounded replay
 *       trades exact state for cheaper resumption".
 *
 * Precision.  Steps whose result is an integer code (the FP4/FP8 encodings
 * and everything feeding them: pair gate, RMSNorm, rotation, index-key
 * projection) are evaluated in fp32 with a fixed operation order, because a
 * code must be decided in the same precision on both sides.  Scores and
 * attention are evaluated in double.  Readings where the pages are silent:
 *   - rotation: adjacent pairs (lo+2i, lo+2i+1), angle table given as input;
 *   - pair gate: per-channel softmax over the two positions;
 *   - exp in the gate: Cody-Waite reduction (Cody & Waite, "Software Manual
 *     for the Elementary Functions", 1980) + degree-7 Taylor polynomial;
 *   - RMSNorm sum of squares: groups of 8 consecutive channels, each an
 *     ascending fma chain, then a pairwise tree (halving strides);
 *   - FP4: OCP MX E2M1 elements, one E8M0 scale per 32 (2^(floor(log2 amax)-2)),
 *     round to nearest, ties to the even code, saturating at 6;
 *   - FP8: OCP E4M3FN with one fp32 scale per row, scale = amax/448, round to
 *     nearest even, saturating at 448;
 *   - index queries: FP8 E4M3FN per (token, head) row of 128;
 *   - top-k ties: larger score first, then smaller entry index; output sorted
 *     by ascending entry index, padded with -1.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_D 512
#define ORC_ROPE_LO 448
#define ORC_PAIRS 32
#define ORC_WINDOW 128
#define ORC_HI 32
#define ORC_DI 128
#define ORC_KI_ROPE_LO 64
#define ORC_EPS 1e-20f

/* ------------------------------------------------------------------ */
/* bf16 / format helpers                                                */
/* ------------------------------------------------------------------ */

static float bf16f(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t f64_to_bf16(double v) {
    /* round a double to bf16, nearest-even, through exact comparison */
    float f = (float)v;                /* nearest fp32 (may double-round; tolerance covers it) */
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0x7FFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* E2M1 magnitudes of codes 0..7 (OCP MX v1.0: 1 sign, 2 exponent, 1 mantissa bit) */
static const float E2M1_MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float orc_e2m1_value(int code) {
    float m = E2M1_MAG[code & 7];
    return (code & 8) ? -m : m;
}

/* nearest E2M1 code to y (magnitudes above 6 saturate); ties to the even code */
int orc_e2m1_encode(float y) {
    float a = fabsf(y);
    int best = 7;
    if (!(a >= 6.0f)) {
        /* first magnitude >= a, then compare with its lower neighbour */
        int hi = 0;
        while (E2M1_MAG[hi] < a) ++hi;
        if (hi == 0) {
            best = 0;
        } else {
            float dlo = a - E2M1_MAG[hi - 1], dhi = E2M1_MAG[hi] - a;
            if (dlo < dhi) best = hi - 1;
            else if (dhi < dlo) best = hi;
            else best = ((hi - 1) % 2 == 0) ? hi - 1 : hi;
        }
    }
    return best | (signbit(y) ? 8 : 0);
}

/* E4M3FN value of code (bias 7; exponent field 0 = subnormal m*2^-9; 0x7F/0xFF are NaN) */
float orc_e4m3_value(int code) {
    int e = (code >> 3) & 15, m = code & 7;
    float v;
    if ((code & 0x7F) == 0x7F) return NAN;
    if (e == 0) v = ldexpf((float)m, -9);
    else v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return (code & 0x80) ? -v : v;
}

/* nearest finite E4M3FN code (0..126 magnitudes, saturating at 448); ties to even code */
int orc_e4m3_encode(float y) {
    float a = fabsf(y);
    int best;
    if (a >= 448.0f) {
        best = 126;
    } else {
        /* binary search for the first code with value >= a (values rise with the code) */
        int lo = 0, hi = 126;
        while (lo < hi) {
            int mid = (lo + hi) / 2;
            if (orc_e4m3_value(mid) >= a) hi = mid;
            else lo = mid + 1;
        }
        if (lo == 0) {
            best = 0;
        } else {
            float dlo = a - orc_e4m3_value(lo - 1), dhi = orc_e4m3_value(lo) - a;
            if (dlo < dhi) best = lo - 1;
            else if (dhi < dlo) best = lo;
            else best = ((lo - 1) % 2 == 0) ? lo - 1 : lo;
        }
    }
    return best | (signbit(y) ? 0x80 : 0);
}

/*
 * FP4 (MX) encoding of n values, n a multiple of 32: per block of 32, the
 * shared scale is 2^(floor(log2(max|x|)) - 2) stored as the biased byte
 * e + 127 (E8M0); every element is x / 2^e rounded to E2M1.  Codes are packed
 * two per byte, element 2i in the low nibble of byte i.  [P1 "890 bytes";
 * P4 "Deriving the 890 bytes per token": 4-bit values, one byte scale per 32.]
 */
void orc_fp4_encode(const float* x, int n, uint8_t* codes, uint8_t* scales) {
    for (int b = 0; b < n / 32; ++b) {
        const float* xb = x + 32 * b;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(xb[i]));
        int e = 0;
        if (amax > 0.0f) {
            int ex;
            frexpf(amax, &ex);   /* amax = f * 2^ex, f in [0.5, 1) */
            e = (ex - 1) - 2;    /* floor(log2 amax) - emax(E2M1) */
            if (e < -127) e = -127;
            if (e > 127) e = 127;
        }
        scales[b] = (uint8_t)(amax > 0.0f ? e + 127 : 0);
        for (int i = 0; i < 32; i += 2) {
            int c0 = 0, c1 = 0;
            if (amax > 0.0f) {
                c0 = orc_e2m1_encode(ldexpf(xb[i], -e));
                c1 = orc_e2m1_encode(ldexpf(xb[i + 1], -e));
            }
            codes[16 * b + i / 2] = (uint8_t)(c0 | (c1 << 4));
        }
    }
}

/* exact value of element k of an FP4 row */
double orc_fp4_value(const uint8_t* codes, const uint8_t* scales, int k) {
    int c = (codes[k / 2] >> ((k & 1) * 4)) & 15;
    return ldexp((double)orc_e2m1_value(c), (int)scales[k / 32] - 127);
}

/*
 * The pages' main-entry format [P4 "Deriving the 890 bytes per token": E2M1
 * values, one one-byte E4M3 scale per 16 channels, 288 bytes per entry; P4
 * "FP4 is a storage choice": E4M3 block scales in the manner of NVFP4's local
 * scaling, without its second, global scale].  Per block of 16 the scale is
 * E4M3FN(max|x| / 6) (6 = the largest E2M1 magnitude; division in fp32,
 * correctly rounded; nearest code, ties to even), and every element is
 * E2M1(x / s) with s the scale code's value (fp32 division; nearest, ties to
 * even, saturating at 6).  A scale that rounds to 0 gives an all-zero block.
 * Codes packed as in orc_fp4_encode; scales one byte per 16 elements.
 */
void orc_fp4e4_encode(const float* x, int n, uint8_t* codes, uint8_t* scales) {
    for (int b = 0; b < n / 16; ++b) {
        const float* xb = x + 16 * b;
        float amax = 0.0f;
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xb[i]));
        int sc = orc_e4m3_encode(amax / 6.0f);
        float s = orc_e4m3_value(sc);
        scales[b] = (uint8_t)sc;
        for (int i = 0; i < 16; i += 2) {
            int c0 = 0, c1 = 0;
            if (s > 0.0f) {
                c0 = orc_e2m1_encode(xb[i] / s);
                c1 = orc_e2m1_encode(xb[i + 1] / s);
            }
            codes[8 * b + i / 2] = (uint8_t)(c0 | (c1 << 4));
        }
    }
}

/* exact value of element k of a row in the pages' format */
double orc_fp4e4_value(const uint8_t* codes, const uint8_t* scales, int k) {
    int c = (codes[k / 2] >> ((k & 1) * 4)) & 15;
    return (double)orc_e2m1_value(c) * (double)orc_e4m3_value(scales[k / 16]);
}

/*
 * FP8 row encoding: scale = max|x| / 448 (fp32, correctly rounded), element
 * code = E4M3FN(x / scale).  An all-zero row gets scale 1.  [P2 "W <- FP8(W)";
 * P1 "the window cache stays FP8".]
 */
void orc_fp8_encode_row(const float* x, int n, uint8_t* codes, float* scale) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) amax = fmaxf(amax, fabsf(x[i]));
    if (amax == 0.0f) {
        *scale = 1.0f;
        memset(codes, 0, (size_t)n);
        return;
    }
    float s = amax / 448.0f;
    *scale = s;
    for (int i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e4m3_encode(x[i] / s);
}

/* ------------------------------------------------------------------ */
/* fp32 building blocks of the compression step                          */
/* ------------------------------------------------------------------ */

/*
 * exp(x) for x <= 0 in fp32: k = nearest-even integer of x*log2(e);
 * r = x - k*ln2 in two fma steps (ln2 split in a 16-bit head and its fp32
 * tail); exp(r) by the degree-7 Taylor polynomial in Horner form; result
 * 2^k * p.  Below -87 the result is 0 (keeps every output a normal number).
 */
float orc_exp(float x) {
    const float LOG2E = 1.44269502f;          /* 0x3fb8aa3b */
    const float LN2_HI = 0.693145751953125f;  /* 0x3f317200 */
    const float LN2_LO = 1.42860677e-06f;     /* 0x35bfbe8e */
    const float C[8] = {1.0f, 1.0f, 0.5f, 0.166666672f, 0.0416666679f, 0.00833333377f,
                        0.00138888892f, 0.000198412701f};
    if (x < -87.0f) return 0.0f;
    float kf = rintf(x * LOG2E);
    float r = fmaf(-kf, LN2_HI, x);
    r = fmaf(-kf, LN2_LO, r);
    float p = C[7];
    for (int i = 6; i >= 0; --i) p = fmaf(p, r, C[i]);
    return ldexpf(p, (int)kf);
}

/*
 * RMSNorm y = gamma * (x * (1/sqrt(mean(x^2) + eps))) over n in {128, 512}
 * [P2 compressed RMSNorm and index-key norm; P3 formula, eps 1e-20].
 * Sum of squares: partial g = fma chain over x[8g..8g+7] ascending from 0,
 * then partial[g] += partial[g+s] for s = n/16, ..., 1.
 */
void orc_rmsnorm(const float* x, const float* gamma, int n, float* y) {
    float part[64];
    int G = n / 8;
    for (int g = 0; g < G; ++g) {
        float acc = 0.0f;
        for (int i = 0; i < 8; ++i) acc = fmaf(x[8 * g + i], x[8 * g + i], acc);
        part[g] = acc;
    }
    for (int s = G / 2; s >= 1; s /= 2)
        for (int g = 0; g < s; ++g) part[g] = part[g] + part[g + s];
    float mean = part[0] * (1.0f / (float)n);
    float v = mean + ORC_EPS;
    float r = 1.0f / sqrtf(v);
    for (int i = 0; i < n; ++i) y[i] = gamma[i] * (x[i] * r);
}

/* R_p on the 64 channels starting at lo: pairs (lo+2i, lo+2i+1) turned by angle (p, i) */
static void rope_fwd(float* x, int lo, const float* cs, const float* sn) {
    for (int i = 0; i < ORC_PAIRS; ++i) {
        float x0 = x[lo + 2 * i], x1 = x[lo + 2 * i + 1];
        float c = cs[i], s = sn[i];
        float a = x0 * c;
        float b = x1 * s;
        float e = x0 * s;
        float f = x1 * c;
        x[lo + 2 * i] = a - b;
        x[lo + 2 * i + 1] = e + f;
    }
}

/*
 * One compressed entry j from positions 2j, 2j+1 [P2 pooling equations]:
 *   k^p = sum_i softmax_i(g^c_i) (.) k^c_i          (per channel, i in {2j, 2j+1})
 * or, at compression ratio one [zharf, CSA2 section: ratio one is a supported
 * case; blog: decoder layers keep one entry per token], from the one position
 * j alone (kc1 == NULL): the softmax over a single logit is 1, so k^p = k^c_j
 * and the gate logits are not read.
 *   c   = RMSNorm_{gamma_C}(k^p)
 *   Z_j = FP4(c with channels 448.. rotated by R_{2j})
 *   K^I_j = FP4(RMSNorm_{gamma_IK}(c W_IK) with channels 64.. rotated by R_{2j})
 * In given mode (w_ik == NULL) the index key's pre-quantisation values are
 * ki_given (already normalised and rotated) and are only encoded.
 * z_pre / ki_pre (optional) receive the fp32 values before quantisation.
 * z_fmt selects Z's storage: 0 = one E8M0 scale per 32 (16 scale bytes),
 * 1 = the pages' one E4M3 scale per 16 (32 scale bytes); K^I is always the
 * former.
 */
void orc_compress_entry(const uint16_t* kc0, const uint16_t* kc1, const uint16_t* gc0,
                        const uint16_t* gc1, const float* gamma_c, const uint16_t* w_ik,
                        const float* gamma_ik, const uint16_t* ki_given, const float* cs,
                        const float* sn, uint8_t* z_codes, uint8_t* z_scales, uint8_t* ki_codes,
                        uint8_t* ki_scales, float* z_pre, float* ki_pre, int z_fmt) {
    float kp[ORC_D], c[ORC_D], z[ORC_D], ki[ORC_DI], kn[ORC_DI];
    for (int ch = 0; ch < ORC_D && !kc1; ++ch) kp[ch] = bf16f(kc0[ch]);
    for (int ch = 0; ch < ORC_D && kc1; ++ch) {
        float a = bf16f(gc0[ch]), b = bf16f(gc1[ch]);
        float m = fmaxf(a, b);
        float ea = orc_exp(a - m), eb = orc_exp(b - m);
        float s = ea + eb;
        float wa = ea / s, wb = eb / s;
        float pa = wa * bf16f(kc0[ch]);
        float pb = wb * bf16f(kc1[ch]);
        kp[ch] = pa + pb;
    }
    orc_rmsnorm(kp, gamma_c, ORC_D, c);
    memcpy(z, c, sizeof z);
    rope_fwd(z, ORC_ROPE_LO, cs, sn);
    if (z_pre) memcpy(z_pre, z, sizeof z);
    if (z_fmt == 1)
        orc_fp4e4_encode(z, ORC_D, z_codes, z_scales);
    else
        orc_fp4_encode(z, ORC_D, z_codes, z_scales);

    if (w_ik) {
        for (int n = 0; n < ORC_DI; ++n) {
            float acc = 0.0f;
            for (int k = 0; k < ORC_D; ++k) acc = fmaf(c[k], bf16f(w_ik[k * ORC_DI + n]), acc);
            ki[n] = acc;
        }
        orc_rmsnorm(ki, gamma_ik, ORC_DI, kn);
        rope_fwd(kn, ORC_KI_ROPE_LO, cs, sn);
    } else {
        for (int n = 0; n < ORC_DI; ++n) kn[n] = bf16f(ki_given[n]);
    }
    if (ki_pre) memcpy(ki_pre, kn, sizeof kn);
    orc_fp4_encode(kn, ORC_DI, ki_codes, ki_scales);
}

/*
 * Compression of B requests x T new positions starting at absolute position
 * pos0.  ratio 2: pos0 even; entry j (absolute) pools positions 2j, 2j+1 and
 * is rotated at 2j; T odd leaves the last position pending (floor(T/2)
 * entries).  ratio 1: entry j is position j alone, rotated at j (T entries).
 * Layouts: kc, gc [B][T][512] bf16; ki_given [B][T/2][128] bf16 or NULL;
 * caches [B][entry_stride][...]; cos/sin [rows][32] indexed by absolute position.
 */
void orc_compress(int B, int T, int pos0, const uint16_t* kc, const uint16_t* gc,
                  const float* gamma_c, const uint16_t* w_ik, const float* gamma_ik,
                  const uint16_t* ki_given, const float* cos_t, const float* sin_t,
                  uint8_t* z_codes, uint8_t* z_scales, uint8_t* ki_codes, uint8_t* ki_scales,
                  int64_t entry_stride, int ratio, int z_fmt) {
    const int zsb = z_fmt == 1 ? 32 : 16;   /* scale bytes per Z entry */
    int nloc = T / ratio;
    for (int b = 0; b < B; ++b) {
        for (int jl = 0; jl < nloc; ++jl) {
            int64_t j = pos0 / ratio + jl;
            const uint16_t* k0 = kc + ((int64_t)b * T + ratio * jl) * ORC_D;
            const uint16_t* g0 = gc ? gc + ((int64_t)b * T + ratio * jl) * ORC_D : NULL;
            const uint16_t* kg = ki_given ? ki_given + ((int64_t)b * nloc + jl) * ORC_DI : NULL;
            int64_t e = (int64_t)b * entry_stride + j;
            orc_compress_entry(k0, ratio == 2 ? k0 + ORC_D : NULL, g0,
                               ratio == 2 ? g0 + ORC_D : NULL, gamma_c, w_ik, gamma_ik, kg,
                               cos_t + ratio * j * ORC_PAIRS, sin_t + ratio * j * ORC_PAIRS,
                               z_codes + e * 256, z_scales + e * zsb, ki_codes + e * 64,
                               ki_scales + e * 4, NULL, NULL, z_fmt);
        }
    }
}

/*
 * Window rows [P2: W_{t,448:} <- R_t w^n_{t,448:}; W <- FP8(W)]: rows
 * wn[b][i] are the window vectors of absolute positions pos0 + i; each is
 * rotated at its position and FP8-encoded into ring slot (position mod cap).
 */
void orc_window_encode(int B, int T, int pos0, const uint16_t* wn, const float* cos_t,
                       const float* sin_t, int cap, uint8_t* w_codes, float* w_scale) {
    float x[ORC_D];
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < T; ++i) {
            int64_t p = (int64_t)pos0 + i;
            const uint16_t* src = wn + ((int64_t)b * T + i) * ORC_D;
            for (int ch = 0; ch < ORC_D; ++ch) x[ch] = bf16f(src[ch]);
            rope_fwd(x, ORC_ROPE_LO, cos_t + p * ORC_PAIRS, sin_t + p * ORC_PAIRS);
            int64_t slot = (int64_t)b * cap + (p % cap);
            orc_fp8_encode_row(x, ORC_D, w_codes + slot * ORC_D, w_scale + slot);
        }
    }
}

/* encode arbitrary bf16 rows to FP4 / FP8 (cache fill for decode workloads) */
void orc_fp4_encode_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes, uint8_t* scales) {
    float* tmp = (float*)malloc(sizeof(float) * (size_t)cols);
    for (int64_t r = 0; r < rows; ++r) {
        for (int k = 0; k < cols; ++k) tmp[k] = bf16f(x[r * cols + k]);
        orc_fp4_encode(tmp, cols, codes + r * (cols / 2), scales + r * (cols / 32));
    }
    free(tmp);
}

void orc_fp4e4_encode_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes,
                           uint8_t* scales) {
    float* tmp = (float*)malloc(sizeof(float) * (size_t)cols);
    for (int64_t r = 0; r < rows; ++r) {
        for (int k = 0; k < cols; ++k) tmp[k] = bf16f(x[r * cols + k]);
        orc_fp4e4_encode(tmp, cols, codes + r * (cols / 2), scales + r * (cols / 16));
    }
    free(tmp);
}

void orc_fp8_encode_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes, float* scale) {
    float* tmp = (float*)malloc(sizeof(float) * (size_t)cols);
    for (int64_t r = 0; r < rows; ++r) {
        for (int k = 0; k < cols; ++k) tmp[k] = bf16f(x[r * cols + k]);
        orc_fp8_encode_row(tmp, cols, codes + r * cols, scale + r);
    }
    free(tmp);
}

/* ------------------------------------------------------------------ */
/* lightning indexer and selection                                      */
/* ------------------------------------------------------------------ */

/*
 * Scores of one query token against entries 0..n-1 [P2 indexer score]:
 *   S[j] = sum_h w[h] * ReLU(Q^I_h . K^I_j)
 * with Q^I_h = sq[h] * dec(q8[h]) (FP8 row) and K^I_j the exact FP4 values.
 * Each dot product is accumulated in double (exact for these formats), the
 * head sum in double, and the result rounded once to fp32.
 */
void orc_index_scores(const uint8_t* q8, const float* sq, const float* w, const uint8_t* ki_codes,
                      const uint8_t* ki_scales, int64_t n, float* S) {
    double qv[ORC_HI][ORC_DI];
    for (int h = 0; h < ORC_HI; ++h)
        for (int k = 0; k < ORC_DI; ++k) qv[h][k] = (double)orc_e4m3_value(q8[h * ORC_DI + k]);
    double kv[ORC_DI];
    for (int64_t j = 0; j < n; ++j) {
        for (int k = 0; k < ORC_DI; ++k) kv[k] = orc_fp4_value(ki_codes + j * 64, ki_scales + j * 4, k);
        double s = 0.0;
        for (int h = 0; h < ORC_HI; ++h) {
            double d = 0.0;
            for (int k = 0; k < ORC_DI; ++k) d += qv[h][k] * kv[k];
            double dq = (double)sq[h] * d;
            s += (double)w[h] * (dq > 0.0 ? dq : 0.0);
        }
        S[j] = (float)s;
    }
}

typedef struct {
    float s;
    int32_t j;
} orc_cand;

static int cand_cmp(const void* a, const void* b) {
    const orc_cand* x = (const orc_cand*)a;
    const orc_cand* y = (const orc_cand*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int int_cmp(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/*
 * I = top_k(S[j] : j < n) [P2 causal top-512].  n <= k takes every entry.
 * Ties: larger score first, then smaller j.  idx holds the chosen j in
 * ascending order, padded with -1 to k; returns the count.
 */
int orc_topk(const float* S, int64_t n, int k, int32_t* idx) {
    int cnt;
    if (n <= k) {
        for (int64_t j = 0; j < n; ++j) idx[j] = (int32_t)j;
        cnt = (int)n;
    } else {
        orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)n);
        for (int64_t j = 0; j < n; ++j) {
            c[j].s = S[j];
            c[j].j = (int32_t)j;
        }
        qsort(c, (size_t)n, sizeof(orc_cand), cand_cmp);
        for (int i = 0; i < k; ++i) idx[i] = c[i].j;
        free(c);
        qsort(idx, (size_t)k, sizeof(int32_t), int_cmp);
        cnt = k;
    }
    for (int i = cnt; i < k; ++i) idx[i] = -1;
    return cnt;
}

/* FP8 per-(token, head) quantisation of index queries: q [32][128] bf16 -> codes, scales */
void orc_quant_index_query(const uint16_t* q, uint8_t* q8, float* sq) {
    float tmp[ORC_DI];
    for (int h = 0; h < ORC_HI; ++h) {
        for (int k = 0; k < ORC_DI; ++k) tmp[k] = bf16f(q[h * ORC_DI + k]);
        orc_fp8_encode_row(tmp, ORC_DI, q8 + h * ORC_DI, sq + h);
    }
}

/* ------------------------------------------------------------------ */
/* sparse attention over window + selected entries                       */
/* ------------------------------------------------------------------ */

/*
 * One query token at absolute position p, H heads [P2 attention equations]:
 *   J^w = {max(0, s, p-127) .. p} (window rows, ring slot = position mod cap;
 *         s = w_floor, the start of a bounded replay, 0 when none),
 *   G   = [W[J^w]; Z[I]]                     (no de-duplication),
 *   S_i = Q_h . G_i / sqrt(512),
 *   A_i = exp S_i / (exp s_h + sum_j exp S_j),
 *   O_h = sum_i A_i G_i,  then channels 448.. turned back by R_p^{-1}.
 * G rows are the exact dequantised values (Z in format z_fmt, as for
 * orc_compress_entry); everything is in double.
 * Q: [H][512] bf16.  Out: O [H][512] double, lse [H] (log of the full
 * denominator, sink included), O_bf16 [H][512] (nearest bf16).
 */
void orc_attend(const uint16_t* Q, int H, int64_t p, const uint8_t* w_codes, const float* w_scale,
                int cap, const uint8_t* z_codes, const uint8_t* z_scales, const int32_t* idx,
                int cnt, const float* sink, const float* cos_t, const float* sin_t, double* O,
                double* lse, uint16_t* O_bf16, int64_t w_floor, int z_fmt) {
    int64_t w0 = p - (ORC_WINDOW - 1);
    if (w0 < 0) w0 = 0;
    /* bounded replay from s = w_floor: the window is max(s, p-127) .. p (s > p read as p) */
    if (w_floor > p) w_floor = p;
    if (w0 < w_floor) w0 = w_floor;
    int nw = (int)(p - w0 + 1);
    int nr = nw + cnt;
    double* G = (double*)malloc(sizeof(double) * (size_t)nr * ORC_D);
    for (int r = 0; r < nw; ++r) {
        int64_t slot = (w0 + r) % cap;
        double sc = (double)w_scale[slot];
        for (int k = 0; k < ORC_D; ++k)
            G[(size_t)r * ORC_D + k] = (double)orc_e4m3_value(w_codes[slot * ORC_D + k]) * sc;
    }
    for (int r = 0; r < cnt; ++r) {
        int64_t j = idx[r];
        for (int k = 0; k < ORC_D; ++k)
            G[(size_t)(nw + r) * ORC_D + k] =
                z_fmt == 1 ? orc_fp4e4_value(z_codes + j * 256, z_scales + j * 32, k)
                           : orc_fp4_value(z_codes + j * 256, z_scales + j * 16, k);
    }
    double* s = (double*)malloc(sizeof(double) * (size_t)nr);
    double qd[ORC_D], o[ORC_D];
    const double inv = 1.0 / sqrt((double)ORC_D);
    for (int h = 0; h < H; ++h) {
        for (int k = 0; k < ORC_D; ++k) qd[k] = (double)bf16f(Q[h * ORC_D + k]);
        double m = (double)sink[h];
        for (int r = 0; r < nr; ++r) {
            double acc = 0.0;
            for (int k = 0; k < ORC_D; ++k) acc += qd[k] * G[(size_t)r * ORC_D + k];
            s[r] = acc * inv;
            if (s[r] > m) m = s[r];
        }
        double den = exp((double)sink[h] - m);
        for (int k = 0; k < ORC_D; ++k) o[k] = 0.0;
        for (int r = 0; r < nr; ++r) {
            double e = exp(s[r] - m);
            den += e;
            for (int k = 0; k < ORC_D; ++k) o[k] += e * G[(size_t)r * ORC_D + k];
        }
        for (int k = 0; k < ORC_D; ++k) o[k] /= den;
        /* inverse rotation R_p^{-1} on channels 448.. */
        for (int i = 0; i < ORC_PAIRS; ++i) {
            double c = (double)cos_t[p * ORC_PAIRS + i], sn = (double)sin_t[p * ORC_PAIRS + i];
            double o0 = o[ORC_ROPE_LO + 2 * i], o1 = o[ORC_ROPE_LO + 2 * i + 1];
            o[ORC_ROPE_LO + 2 * i] = o0 * c + o1 * sn;
            o[ORC_ROPE_LO + 2 * i + 1] = -o0 * sn + o1 * c;
        }
        for (int k = 0; k < ORC_D; ++k) {
            if (O) O[(size_t)h * ORC_D + k] = o[k];
            if (O_bf16) O_bf16[(size_t)h * ORC_D + k] = f64_to_bf16(o[k]);
        }
        if (lse) lse[h] = m + log(den);
    }
    free(s);
    free(G);
}

/*
 * Selection + attention for a list of query tokens of one request.
 * For query i at absolute position pos[i]: n = min(floor((pos+1)/ratio), n_entries)
 * candidates; q^I row quantised to FP8; scores; top-k; attention.
 * qI: [nq][32][128] bf16, wI: [nq][32], Q: [nq][H][512] bf16.
 * Outputs: idx [nq][k], cnt [nq], O [nq][H][512] double (optional),
 * O_bf16 [nq][H][512], lse [nq][H] (optional), S_out (optional) receives each
 * query's scores in a buffer of n_entries floats per query.
 */
void orc_query_rows(int nq, const int64_t* pos, int64_t n_entries, const uint16_t* qI,
                    const float* wI, const uint16_t* Q, int H, const uint8_t* ki_codes,
                    const uint8_t* ki_scales, const uint8_t* z_codes, const uint8_t* z_scales,
                    const uint8_t* w_codes, const float* w_scale, int cap, const float* sink,
                    const float* cos_t, const float* sin_t, int k, int32_t* idx, int32_t* cnt,
                    double* O, uint16_t* O_bf16, double* lse, float* S_out, int ratio,
                    int z_fmt) {
    uint8_t q8[ORC_HI * ORC_DI];
    float sq[ORC_HI];
    float* S = (float*)malloc(sizeof(float) * (size_t)(n_entries > 0 ? n_entries : 1));
    for (int i = 0; i < nq; ++i) {
        int64_t p = pos[i];
        int64_t n = (p + 1) / ratio;
        if (n > n_entries) n = n_entries;
        orc_quant_index_query(qI + (size_t)i * ORC_HI * ORC_DI, q8, sq);
        orc_index_scores(q8, sq, wI + (size_t)i * ORC_HI, ki_codes, ki_scales, n, S);
        if (S_out) memcpy(S_out + (size_t)i * n_entries, S, sizeof(float) * (size_t)n);
        cnt[i] = orc_topk(S, n, k, idx + (size_t)i * k);
        if (Q)
            orc_attend(Q + (size_t)i * H * ORC_D, H, p, w_codes, w_scale, cap, z_codes, z_scales,
                       idx + (size_t)i * k, cnt[i], sink, cos_t, sin_t,
                       O ? O + (size_t)i * H * ORC_D : NULL, lse ? lse + (size_t)i * H : NULL,
                       O_bf16 ? O_bf16 + (size_t)i * H * ORC_D : NULL, 0, z_fmt);
    }
    free(S);
}
