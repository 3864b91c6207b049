/*
 * Seeded synthetic inputs for the CSA2 attention layer.
 *
 * This file only draws random numbers and shapes them into the input
 * distributions of the workloads (Gaussian activations, clustered or
 * log-normal index keys, duplicated keys) plus the rotary-embedding angle
 * table that the layer takes as an input.  It holds none of the attention
 * method's arithmetic: no pooling, normalisation, quantisation, scoring,
 * selection or softmax.  Both the HIP library's tests and the CPU oracle read
 * the buffers written here, so the two sides see byte-identical inputs.
 *
 * Generator: element e of tensor id k under seed s is driven by the
 * counter-based SplitMix64 output of (s XOR k<<56 XOR counter) (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014).
 * Uniforms take the top 53 bits; normals use the Box-Muller transform in
 * double on element pairs (2p, 2p+1).  Every value is computed in double and
 * rounded once to fp32, then (for bf16 tensors) once more to bf16 with
 * round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static inline uint64_t smix(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t seed, uint32_t id, uint64_t ctr) {
    return smix(seed ^ ((uint64_t)id << 56) ^ ctr);
}

/* uniform in [0, 1) */
static inline double uni(uint64_t seed, uint32_t id, uint64_t ctr) {
    return (double)(draw(seed, id, ctr) >> 11) * 0x1.0p-53;
}

/* standard normal for element e (Box-Muller on the pair containing e) */
static inline double gauss(uint64_t seed, uint32_t id, uint64_t e) {
    uint64_t p = e >> 1;
    double u1 = ((double)(draw(seed, id, 2 * p) >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
    double u2 = (double)(draw(seed, id, 2 * p + 1) >> 11) * 0x1.0p-53;     /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925286766559 * u2;
    return (e & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) /* inf / nan: keep, quiet nan */
        return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x40u : 0u));
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static inline void put(void* out, int kind, int64_t i, double v) {
    float f = (float)v;
    if (kind == 0)
        ((float*)out)[i] = f;
    else
        ((uint16_t*)out)[i] = to_bf16(f);
}

/* out[i] = add + mul * N(0,1)[start + i], i < n.  kind 0 = fp32, 1 = bf16. */
void synth_normal(uint64_t seed, uint32_t id, int64_t start, int64_t n, double mul, double add,
                  int kind, void* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        put(out, kind, i, add + mul * gauss(seed, id, (uint64_t)(start + i)));
}

/* out[i] = U[0,1)[start + i] as double */
void synth_uniform(uint64_t seed, uint32_t id, int64_t start, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = uni(seed, id, (uint64_t)(start + i));
}

/*
 * Rotary angle table for absolute positions p0 .. p0+rows-1 and `pairs`
 * frequency pairs: angle(p, i) = p * theta^(-2i / (2*pairs)), evaluated in
 * double and rounded once to fp32.  Row-major [rows][pairs].
 */
void synth_rope_table(double theta, int64_t p0, int64_t rows, int pairs, float* cos_out,
                      float* sin_out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int i = 0; i < pairs; ++i) {
            double freq = pow(theta, -2.0 * (double)i / (double)(2 * pairs));
            double ang = (double)(p0 + r) * freq;
            cos_out[r * pairs + i] = (float)cos(ang);
            sin_out[r * pairs + i] = (float)sin(ang);
        }
    }
}

/*
 * Clustered keys: row j (j0 <= j < j0+n) of width dim is
 *   mu[c(j)] + noise * N(0, I),  c(j) = floor(U_j * n_centres),
 * with centres mu[c] ~ N(0, I_dim) drawn from tensor id_centre.
 * Written as bf16, row-major [n][dim].
 */
void synth_clustered_rows(uint64_t seed, uint32_t id_centre, uint32_t id_assign, uint32_t id_noise,
                          int n_centres, double noise, int64_t j0, int64_t n, int dim,
                          uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        int64_t j = j0 + r;
        int64_t c = (int64_t)(uni(seed, id_assign, (uint64_t)j) * n_centres);
        if (c >= n_centres) c = n_centres - 1;
        for (int k = 0; k < dim; ++k) {
            double mu = gauss(seed, id_centre, (uint64_t)(c * dim + k));
            double z = gauss(seed, id_noise, (uint64_t)(j * dim + k));
            out[r * dim + k] = to_bf16((float)(mu + noise * z));
        }
    }
}

/*
 * Heavy-tailed keys with exact duplicates.  Row j is exp(xi_j) * g_j with
 * xi_j ~ N(0, sigma^2) and g_j ~ N(0, I_dim), unless j >= 1 is drawn as a
 * duplicate (probability dup_p), in which case it is a copy of row src(j),
 * src uniform over 0..j-1 (followed until a non-duplicate row is reached).
 * Copies are exact, so their encodings and scores tie exactly.
 * Written as bf16, row-major [n][dim].
 */
static int64_t dup_root(uint64_t seed, uint32_t id_flag, uint32_t id_src, double dup_p, int64_t j) {
    while (j >= 1 && uni(seed, id_flag, (uint64_t)j) < dup_p) {
        int64_t s = (int64_t)(uni(seed, id_src, (uint64_t)j) * (double)j);
        if (s >= j) s = j - 1;
        j = s;
    }
    return j;
}

void synth_lognormal_rows(uint64_t seed, uint32_t id_xi, uint32_t id_g, uint32_t id_flag,
                          uint32_t id_src, double sigma, double dup_p, int64_t j0, int64_t n,
                          int dim, uint16_t* out, int64_t* root_out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        int64_t j = dup_root(seed, id_flag, id_src, dup_p, j0 + r);
        if (root_out) root_out[r] = j;
        double amp = exp(sigma * gauss(seed, id_xi, (uint64_t)j));
        for (int k = 0; k < dim; ++k)
            out[r * dim + k] = to_bf16((float)(amp * gauss(seed, id_g, (uint64_t)(j * dim + k))));
    }
}

/* Gather rows of a Gaussian tensor: rows[i] of width dim from tensor id, bf16 or fp32. */
void synth_normal_rows(uint64_t seed, uint32_t id, const int64_t* rows, int64_t n, int dim,
                       double mul, double add, int kind, void* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int k = 0; k < dim; ++k)
            put(out, kind, r * dim + k,
                add + mul * gauss(seed, id, (uint64_t)(rows[r] * (int64_t)dim + k)));
}

int synth_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
