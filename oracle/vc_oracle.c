/*
 * vc_oracle.c -- CPU oracle for VC-Attention (V-Smooth + ExpCast-FP8).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header or constant table with the HIP library.
 *
 * Sources (web pages on VC-Attention, cited by page title and section):
 *  [AGI]  "VC-Attention: Training-Free Low-Bit Attention Speeds Video
 *         Diffusion Up to 3.6x" (agihunt summary): the V-Smooth and
 *         ExpCast-FP8 bullet points.
 *  [MTP]  "Nunchux AI Introduces VC-Attention ..." (yifor blog; the embedded
 *         MarkTechPost English abstract and the section headed by the puzzle
 *         emoji, "V-Smooth and ExpCast-FP8, two targeted designs").
 *  [AIK]  aikraft.ru news item, section "Reshenie" (Solution).
 *  [TRT]  TensorRT-LLM tech blog "Accelerating Video Generation with GEMM
 *         Quantization, Attention Quantization and Skip Softmax Attention",
 *         sections "Quantized Attention" and "Sparse Attention with Skip
 *         Softmax".
 *
 * What is computed (all free choices are fixed here; each is a reading of the
 * pages where they leave a step open):
 *  - E4M3 is the OCP E4M3FN format (bias 7, max 448, no infinities): [MTP]
 *    states that an E4M3 byte read as an integer is about 8*log2(v)+56, which
 *    holds only with exponent bias 7.
 *  - V-Smooth: tokens of one (batch, head) are grouped by a lightweight,
 *    seeded k-means over the value rows ([AGI] V-Smooth bullet; [AIK]
 *    "Reshenie"), sorted by cluster into 128-token blocks; each block keeps
 *    its exact mean and only the residual is quantised ([AGI], [MTP]).
 *  - ExpCast-FP8: the E4M3 byte of a probability is written directly from the
 *    log2-domain score with one fused multiply-add, byte = round(8 z + 56 +
 *    beta), beta = -0.35, clamped at zero ([MTP] abstract; [AIK]).
 *  - Mean restore: the block mean is added back weighted by the row sum that
 *    the online softmax keeps anyway ([AGI] V-Smooth bullet).
 *  - Online (flash) softmax over 128-key blocks ([TRT] "Quantized Attention"
 *    and "Sparse Attention with Skip Softmax" notation m~, m).
 *
 * Floating point: reductions are done in double and rounded once; the
 * values this oracle promises to reproduce bit-for-bit (codes, scales,
 * means, ExpCast bytes) are produced by IEEE single-precision operations
 * written out one at a time.  Build with -O2 -fno-fast-math
 * -ffp-contract=off so that no operation is fused or reordered.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define VCO_BLK 128

/* ------------------------------------------------------------------------ */
/* E4M3FN codec, written from the format definition: sign bit, 4 exponent    */
/* bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal          */
/* (value = m * 2^-9); 0x7F / 0xFF are NaN; the largest finite is 0x7E = 448. */
/* ------------------------------------------------------------------------ */

double vco_e4m3_decode(uint8_t b)
{
    int s = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if ((b & 0x7F) == 0x7F) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round-to-nearest, ties-to-even, of a non-negative double that is an exact
 * multiple of 1/2 away from any tie it may sit on. */
static double vco_rne(double x)
{
    double f = floor(x);
    double r = x - f;
    if (r > 0.5) return f + 1.0;
    if (r < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* Saturating round-to-nearest-even encoder (finite inputs only). */
uint8_t vco_e4m3_encode(float xf)
{
    double x = (double)xf; /* exact */
    uint8_t s = (x < 0.0 || (x == 0.0 && signbit(xf))) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a >= 448.0) return s | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: value = m * 2^-9, m in 0..7; m = 8 is the
         * smallest normal 0x08, so the code is simply the rounded m. */
        double m = vco_rne(a * 512.0); /* exact scaling */
        return s | (uint8_t)m;
    }
    int e = (int)floor(log2(a));
    /* guard log2 rounding near powers of two */
    while (ldexp(1.0, e) > a) e--;
    while (ldexp(1.0, e + 1) <= a) e++;
    double frac = (a / ldexp(1.0, e) - 1.0) * 8.0; /* exact: in [0, 8) */
    double q = vco_rne(frac);
    if (q >= 8.0) { q = 0.0; e += 1; }
    int code = ((e + 7) << 3) | (int)q;
    if (code > 0x7E) code = 0x7E; /* saturate (cannot exceed for a < 448) */
    return s | (uint8_t)code;
}

void vco_e4m3_encode_array(const float* x, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = vco_e4m3_encode(x[i]);
}

void vco_e4m3_decode_array(const uint8_t* b, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = vco_e4m3_decode(b[i]);
}

/* ------------------------------------------------------------------------ */
/* E2M1 (the 4-bit element format of the OCP MX formats, FP4), written from   */
/* the format: sign bit, 2 exponent bits with bias 1, 1 mantissa bit;        */
/* exponent field 0 is subnormal (value = m / 2).  Magnitudes 0, 0.5, 1,     */
/* 1.5, 2, 3, 4, 6; no infinities, no NaN.                                  */
/* ------------------------------------------------------------------------ */

double vco_e2m1_decode(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* Saturating round-to-nearest-even: the nearest of the eight magnitudes,
 * a tie going to the code whose mantissa bit is 0; |x| >= 6 gives 6. */
uint8_t vco_e2m1_encode(double x)
{
    uint8_t s = (x < 0.0 || (x == 0.0 && signbit(x))) ? 8 : 0;
    double a = fabs(x);
    if (a >= 6.0) return s | 7;
    int best = 0;
    for (int c = 1; c < 8; c++) {
        double dc = fabs(a - vco_e2m1_decode((uint8_t)c)), db = fabs(a - vco_e2m1_decode((uint8_t)best));
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return s | (uint8_t)best;
}

void vco_e2m1_encode_array(const double* x, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = vco_e2m1_encode(x[i]);
}

/* Power-of-two (E8M0) scale of an FP4 group with amax A: the least e with
 * A <= 6 * 2^e, so no element clips; A < 2^-100 gives e = -127 and the
 * group's codes are all 0. */
int vco_e8m0_exp(double A)
{
    if (!(A >= ldexp(1.0, -100))) return -127;
    int e = (int)floor(log2(A)) - 4;
    while (!(A <= 6.0 * ldexp(1.0, e))) e++;
    while (e > -127 && A <= 6.0 * ldexp(1.0, e - 1)) e--;
    return e;
}

/* ------------------------------------------------------------------------ */
/* SplitMix64 (Steele, Lea & Flood, OOPSLA 2014; finaliser "Mix13" of        */
/* D. Stafford as in Vigna's public-domain reference).  Output i (0-based)    */
/* of the stream started at `seed` is mix(seed + (i+1)*gamma): a counter-     */
/* based generator, so any output can be computed independently.             */
/* ------------------------------------------------------------------------ */

#define VCO_GAMMA 0x9E3779B97F4A7C15ULL

uint64_t vco_splitmix64(uint64_t seed, uint64_t i)
{
    uint64_t z = seed + (i + 1) * VCO_GAMMA;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Seed of head (b, h): output number b*H+h of the stream seeded by `seed`. */
uint64_t vco_head_seed(uint64_t seed, int b, int h, int H)
{
    return vco_splitmix64(seed, (uint64_t)b * (uint64_t)H + (uint64_t)h);
}

/* k distinct seeded token indices: token range [0, L) is cut into k
 * contiguous strata [floor(c L / k), floor((c+1) L / k)); centroid c starts
 * at a uniformly drawn token of stratum c.  Requires 1 <= k <= L. */
void vco_kmeans_init_indices(int L, int k, uint64_t seed_bh, int32_t* idx)
{
    for (int c = 0; c < k; c++) {
        int64_t lo = ((int64_t)c * L) / k;
        int64_t hi = ((int64_t)(c + 1) * L) / k;
        uint64_t r = vco_splitmix64(seed_bh, (uint64_t)c);
        idx[c] = (int32_t)(lo + (int64_t)(r % (uint64_t)(hi - lo)));
    }
}

static inline float vco_bf16(uint16_t u)
{
    uint32_t w = ((uint32_t)u) << 16;
    float f;
    memcpy(&f, &w, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* QK smoothing, K side: per-channel mean of K over all L tokens.           */
/* The pages measure with QK smoothing applied; subtracting one vector from  */
/* every key adds a per-query constant to each score row, which softmax     */
/* ignores.                                                                  */
/* ------------------------------------------------------------------------ */

void vco_k_mean(const uint16_t* k, int L, int d, float* kbar)
{
    for (int c = 0; c < d; c++) {
        double s = 0.0;
        for (int j = 0; j < L; j++) s += (double)vco_bf16(k[(int64_t)j * d + c]);
        kbar[c] = (float)(s / (double)L);
    }
}

/* ------------------------------------------------------------------------ */
/* Lloyd k-means on x_j = fp32(V_j) of one head.                            */
/*  assign: argmin_c sum_ch (x - C_c)^2 in double, ties -> lowest c;          */
/*  update: C_c = fp32(double sum / n_c); an empty cluster keeps C_c.         */
/* J_hist (iters+1 entries, may be NULL): J_hist[0] is the objective of the   */
/* initial centroids under their own best assignment; J_hist[t] is the       */
/* objective after t full (assign, update) rounds, measured with the t-th    */
/* assignment and the t-th updated centroids.  Returns J_hist[iters].        */
/* ------------------------------------------------------------------------ */

static double vco_dist2(const float* x, const float* c, int d)
{
    double s = 0.0;
    for (int i = 0; i < d; i++) {
        double t = (double)x[i] - (double)c[i];
        s += t * t;
    }
    return s;
}

static void vco_assign(const float* x, int L, int d, const float* C, int k, int32_t* a)
{
    for (int j = 0; j < L; j++) {
        double best = INFINITY;
        int bi = 0;
        for (int c = 0; c < k; c++) {
            double t = vco_dist2(x + (int64_t)j * d, C + (int64_t)c * d, d);
            if (t < best) { best = t; bi = c; }
        }
        a[j] = bi;
    }
}

static double vco_objective(const float* x, int L, int d, const float* C, const int32_t* a)
{
    double J = 0.0;
    for (int j = 0; j < L; j++) J += vco_dist2(x + (int64_t)j * d, C + (int64_t)a[j] * d, d);
    return J;
}

/* Lloyd rounds from the given centroids (updated in place): each round
 * assigns every row to its nearest centroid, then moves each non-empty
 * cluster's centroid to the fp32-rounded fp64 mean of its members.  Returns
 * J of the last assignment with the updated centroids (iters = 0: one
 * assignment, centroids unchanged). */
static double vco_lloyd(const float* x, int L, int d, int k, int iters, float* centroids, int32_t* assign,
                        double* J_hist)
{
    double* sum = (double*)malloc(sizeof(double) * (size_t)k * d);
    int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * (size_t)k);
    if (J_hist) {
        vco_assign(x, L, d, centroids, k, assign);
        J_hist[0] = vco_objective(x, L, d, centroids, assign);
    }
    double J = 0.0;
    for (int it = 0; it < iters; it++) {
        vco_assign(x, L, d, centroids, k, assign);
        memset(sum, 0, sizeof(double) * (size_t)k * d);
        memset(cnt, 0, sizeof(int64_t) * (size_t)k);
        for (int j = 0; j < L; j++) {
            int c = assign[j];
            cnt[c]++;
            for (int i = 0; i < d; i++) sum[(int64_t)c * d + i] += (double)x[(int64_t)j * d + i];
        }
        for (int c = 0; c < k; c++)
            if (cnt[c] > 0)
                for (int i = 0; i < d; i++)
                    centroids[(int64_t)c * d + i] = (float)(sum[(int64_t)c * d + i] / (double)cnt[c]);
        J = vco_objective(x, L, d, centroids, assign);
        if (J_hist) J_hist[it + 1] = J;
    }
    if (iters == 0) {
        vco_assign(x, L, d, centroids, k, assign);
        J = vco_objective(x, L, d, centroids, assign);
    }
    free(sum); free(cnt);
    return J;
}

double vco_kmeans(const uint16_t* v, int L, int d, int k, int iters, uint64_t seed_bh,
                  int32_t* assign, float* centroids, double* J_hist)
{
    float* x = (float*)malloc(sizeof(float) * (size_t)L * d);
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    for (int64_t i = 0; i < (int64_t)L * d; i++) x[i] = vco_bf16(v[i]);
    vco_kmeans_init_indices(L, k, seed_bh, idx);
    for (int c = 0; c < k; c++) memcpy(centroids + (int64_t)c * d, x + (int64_t)idx[c] * d, sizeof(float) * d);
    double J = vco_lloyd(x, L, d, k, iters, centroids, assign, J_hist);
    free(x); free(idx);
    return J;
}

/* k-means warm-started from caller centroids (a reading of the MarkTechPost
 * abstract's grouping amortised across denoising steps: the clusters of one
 * step seed the next): init [k, d] fp32, then the same Lloyd rounds. */
double vco_kmeans_warm(const uint16_t* v, int L, int d, int k, int iters, const float* init,
                       int32_t* assign, float* centroids, double* J_hist)
{
    float* x = (float*)malloc(sizeof(float) * (size_t)L * d);
    for (int64_t i = 0; i < (int64_t)L * d; i++) x[i] = vco_bf16(v[i]);
    memcpy(centroids, init, sizeof(float) * (size_t)k * d);
    double J = vco_lloyd(x, L, d, k, iters, centroids, assign, J_hist);
    free(x);
    return J;
}

/* The permutation: stable argsort of the assignment.  perm[i] = original token that
 * lands in permuted slot i; slots are ordered by cluster id, then token id. */
void vco_stable_perm(const int32_t* a, int L, int k, int32_t* perm)
{
    int64_t* start = (int64_t*)calloc((size_t)k + 1, sizeof(int64_t));
    for (int j = 0; j < L; j++) start[a[j] + 1]++;
    for (int c = 0; c < k; c++) start[c + 1] += start[c];
    for (int j = 0; j < L; j++) perm[start[a[j]]++] = j;
    free(start);
}

/* ------------------------------------------------------------------------ */
/* Scales.  A = amax of what the scale covers.                                */
/*  mode 0: s = fp32(A/448), inv = fp32(448/A)  (IEEE single division)       */
/*  mode 1: s = 2^e with e the least integer such that A <= 448 * 2^e;       */
/*          inv = 2^-e exactly.                                              */
/*  A < 2^-100 (in particular A == 0): s = inv = 0 and all codes are 0.      */
/* ------------------------------------------------------------------------ */

static void vco_scale(float A, int mode, float* s, float* inv)
{
    /* amax below 2^-100 (zero included) makes the whole group quantise to 0 */
    if (!((double)A >= ldexp(1.0, -100))) { *s = 0.0f; *inv = 0.0f; return; }
    if (mode == 0) {
        volatile float num = 448.0f;
        *s = A / num;
        *inv = num / A;
        return;
    }
    int e = -120;
    while (!((double)A <= 448.0 * ldexp(1.0, e))) e++;
    *s = (float)ldexp(1.0, e);
    *inv = (float)ldexp(1.0, -e);
}

static inline uint8_t vco_quant(float x, float inv)
{
    volatile float y = x * inv; /* one IEEE single multiply */
    return vco_e4m3_encode(y);
}

/* ------------------------------------------------------------------------ */
/* Q/K codes, block means, residual scales and codes for one head, given the */
/* permutation.                                                             */
/*  q,k,v : bf16 bits [L, d] of this head                                     */
/*  perm  : [L]                                                               */
/*  q8,k8 : [Lp, d] codes (Q in original order, K' = K - kbar in perm order)  */
/*  v8    : [nb, d, 128] residual codes, natural slot order inside a block    */
/*  q_scale,k_scale : [nb]; v_scale,v_mean : [nb, d]                          */
/* Padded slots (>= L) get code 0 and take no part in any mean or amax.       */
/* ------------------------------------------------------------------------ */

void vco_prepare_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int L, int d,
                      int smooth_k, int v_mode, const int32_t* perm,
                      uint8_t* q8, uint8_t* k8, uint8_t* v8, float* q_scale, float* k_scale,
                      float* v_scale, float* v_mean, float* kbar_out)
{
    int nb = (L + VCO_BLK - 1) / VCO_BLK;
    float* kbar = (float*)calloc((size_t)d, sizeof(float));
    if (smooth_k) vco_k_mean(k, L, d, kbar);
    if (kbar_out) memcpy(kbar_out, kbar, sizeof(float) * d);
    float* buf = (float*)malloc(sizeof(float) * VCO_BLK * d);

    for (int b = 0; b < nb; b++) {
        int i0 = b * VCO_BLK;
        int n = (L - i0 < VCO_BLK) ? L - i0 : VCO_BLK;

        /* Q: original order, one scalar scale per block */
        float A = 0.0f;
        for (int i = 0; i < n; i++)
            for (int c = 0; c < d; c++) {
                float t = fabsf(vco_bf16(q[(int64_t)(i0 + i) * d + c]));
                if (t > A) A = t;
            }
        float s, inv;
        vco_scale(A, 0, &s, &inv);
        q_scale[b] = s;
        for (int i = 0; i < VCO_BLK; i++)
            for (int c = 0; c < d; c++)
                q8[(int64_t)(i0 + i) * d + c] =
                    (i < n) ? vco_quant(vco_bf16(q[(int64_t)(i0 + i) * d + c]), inv) : 0;

        /* K: permuted order, K' = fp32(K - kbar) */
        A = 0.0f;
        for (int i = 0; i < n; i++)
            for (int c = 0; c < d; c++) {
                volatile float t = vco_bf16(k[(int64_t)perm[i0 + i] * d + c]) - kbar[c];
                buf[i * d + c] = t;
                if (fabsf(t) > A) A = fabsf(t);
            }
        vco_scale(A, 0, &s, &inv);
        k_scale[b] = s;
        for (int i = 0; i < VCO_BLK; i++)
            for (int c = 0; c < d; c++)
                k8[(int64_t)(i0 + i) * d + c] = (i < n) ? vco_quant(buf[i * d + c], inv) : 0;

        /* V: permuted order, exact block mean, residual, per-channel scale */
        for (int c = 0; c < d; c++) {
            double sum = 0.0;
            for (int i = 0; i < n; i++) sum += (double)vco_bf16(v[(int64_t)perm[i0 + i] * d + c]);
            float mu = (float)(sum / (double)n);
            float Ac = 0.0f;
            for (int i = 0; i < n; i++) {
                volatile float r = vco_bf16(v[(int64_t)perm[i0 + i] * d + c]) - mu;
                buf[i * d + c] = r;
                if (fabsf(r) > Ac) Ac = fabsf(r);
            }
            float sv, iv;
            vco_scale(Ac, v_mode, &sv, &iv);
            v_mean[(int64_t)b * d + c] = mu;
            v_scale[(int64_t)b * d + c] = sv;
            for (int i = 0; i < VCO_BLK; i++)
                v8[((int64_t)b * d + c) * VCO_BLK + i] = (i < n) ? vco_quant(buf[i * d + c], iv) : 0;
        }
    }
    free(buf);
    free(kbar);
}

/* ------------------------------------------------------------------------ */
/* 4-bit V-Smooth ([MTP] abstract: 4-bit V-Smooth on workstation cards;     */
/* ExpCast has no 4-bit form).  Readings: Q and K as the 8-bit path (per-    */
/* block FP8); the same exact block mean; the residual r = fp32(v - mean)   */
/* quantised to E2M1 with one power-of-two scale per (block, channel, key   */
/* group), the group of key kk in its block being kk div 32: 32 consecutive */
/* slots of the permuted block (the pages do not define the groups; this is */
/* the plain reading, and the slots of a block hold same-cluster tokens).   */
/* Outputs as vco_prepare_head, except v4 [nb, d, 128] (one E2M1 code per    */
/* byte, natural key order, 0 for padded keys) and v_exp [nb, d, 4] (e +     */
/* 127 of each group's scale 2^e) in place of v8 / v_scale.                 */
/* ------------------------------------------------------------------------ */

/* the 4-bit key group of in-block slot j: 32 consecutive slots */
static int vco_fp4_group(int j) { return j / 32; }

void vco_prepare_head_fp4v(const uint16_t* q, const uint16_t* k, const uint16_t* v, int L, int d,
                           int smooth_k, const int32_t* perm, uint8_t* q8, uint8_t* k8, uint8_t* v4,
                           uint8_t* v_exp, float* q_scale, float* k_scale, float* v_mean)
{
    int nb = (L + VCO_BLK - 1) / VCO_BLK;
    uint8_t* v8 = (uint8_t*)malloc((size_t)nb * d * VCO_BLK);
    float* vs = (float*)malloc(sizeof(float) * (size_t)nb * d);
    vco_prepare_head(q, k, v, L, d, smooth_k, 0, perm, q8, k8, v8, q_scale, k_scale, vs, v_mean, NULL);
    free(v8);
    free(vs);
    float r[VCO_BLK];
    for (int b = 0; b < nb; b++) {
        int i0 = b * VCO_BLK;
        int n = (L - i0 < VCO_BLK) ? L - i0 : VCO_BLK;
        for (int c = 0; c < d; c++) {
            float mu = v_mean[(int64_t)b * d + c];
            for (int j = 0; j < VCO_BLK; j++) {
                volatile float t = (j < n) ? vco_bf16(v[(int64_t)perm[i0 + j] * d + c]) - mu : 0.0f;
                r[j] = t;
            }
            for (int g = 0; g < 4; g++) {
                double A = 0.0;
                for (int j = 0; j < n; j++)
                    if (vco_fp4_group(j) == g && fabs((double)r[j]) > A) A = fabs((double)r[j]);
                int e = vco_e8m0_exp(A);
                v_exp[((int64_t)b * d + c) * 4 + g] = (uint8_t)(e + 127);
                for (int j = 0; j < VCO_BLK; j++)
                    if (vco_fp4_group(j) == g)
                        v4[((int64_t)b * d + c) * VCO_BLK + j] =
                            (j < n && e > -127) ? vco_e2m1_encode(ldexp((double)r[j], -e)) : 0;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* ExpCast-FP8 ([MTP] abstract, [AIK]): y = fma(S, c8, krow) with            */
/* c8 = 8 c_b and krow = KB - 8 m; byte = min(max(rne(y), 0), 126).          */
/* ------------------------------------------------------------------------ */

static inline uint8_t vco_expcast1(float S, float c8, float krow)
{
    float y = fmaf(S, c8, krow);
    double r = (y > 0.0f) ? vco_rne((double)y) : 0.0;
    if (r > 126.0) r = 126.0;
    return (uint8_t)r;
}

void vco_expcast(const float* S, int64_t n, float c8, float krow, uint8_t* out)
{
    for (int64_t i = 0; i < n; i++) out[i] = vco_expcast1(S[i], c8, krow);
}

/* Per-row arrays of (c8, krow), as a kernel would use them. */
void vco_expcast_rows(const float* S, const float* c8, const float* krow, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; i++) out[i] = vco_expcast1(S[i], c8[i], krow[i]);
}

/* KB = fp32(56 + beta + 8 z_off), beta = -0.35; C0 = fp32(log2(e)/sqrt(d)). */
float vco_kb(int z_off) { return (float)(56.0 - 0.35 + 8.0 * (double)z_off); }
float vco_c0(int d) { return (float)(1.4426950408889634074 / sqrt((double)d)); }

/* ------------------------------------------------------------------------ */
/* Blockwise attention for query rows [r0, r1) of one head.                 */
/*                                                                          */
/* mode 0 (quantised, the method):                                          */
/*   S_j   = fp32(exact sum_c qhat_c khat_jc)                                */
/*   c_b   = fp32(fp32(s_q s_k,b) C0)                                        */
/*   t     = fp32(max_valid S * c_b);  m' = max(m, t)                        */
/*   krow  = fp32(KB - 8 m');  byte_j = ExpCast(S_j, 8 c_b, krow)            */
/*   p_j   = decode(byte_j);  l_b = sum_j p_j                                */
/*   acc_c = fp32(exact sum_j p_j rhat_jc)                                   */
/*   alpha = 2^(m - m')   (0 on the first block)                             */
/*   O     = alpha O + s_v,b (.) acc + l_b mu_b;  l = alpha l + l_b          */
/* mode 2 (exp-then-cast, the FP8 path ExpCast replaces): as mode 0 but    */
/*   byte_j = E4M3(fp32(2^z_j)), z_j = fmaf(S_j, c_b, fp32(z_off - m')),      */
/*   2^z correctly rounded to fp32, E4M3 round to nearest even ([MTP]       */
/*   abstract: ExpCast is compared with computing the FP32 exponential and  */
/*   casting it to FP8).                                                    */
/* mode 3 (4-bit P V, with vco_prepare_head_fp4v inputs): p_j as mode 2     */
/*   before the cast, fp32(2^z_j); per key group G of the block (key j in   */
/*   group j div 32), e_G = the E8M0 rule on max_{j in G} p_j and           */
/*   phat_j = 2^e_G E2M1(p_j / 2^e_G); l_b = sum phat_j; acc_c = fp32(sum_j  */
/*   phat_j rhat_jc), rhat_jc = 2^(v_exp - 127) E2M1 code value; O = alpha O */
/*   + acc + l_b mu_b (no separate V scale).  bytes_out holds the E2M1 codes */
/*   and y_out the values phat.                                             */
/* mode 4 (probabilities alone quantised, for the error decomposition):     */
/*   qf, kf, rf real as in mode 1, S the double sum rounded once to fp32,   */
/*   c_b = C0 (scales 1), ExpCast bytes and the running maximum as mode 0;  */
/*   values exact as in mode 1.                                             */
/* mode 1 (exact algebra, for checking the blockwise bookkeeping):          */
/*   qhat, khat, rhat are the real values (scales 1), S is a double sum,      */
/*   p_j = 2^(S_j C0 - m') in double; the rest as in mode 0.  With mode 1 the */
/*   result equals softmax(Q K^T / sqrt(d)) V up to double rounding.         */
/*                                                                          */
/* Inputs for mode 0: q8,k8 [Lp,d], v8 [nb,d,128], scales and means as      */
/* produced by vco_prepare_head.  For mode 1 pass qf [L,d], kf [Lp,d]         */
/* (keys already in permuted order), rf [nb,d,128], v_mean; scales ignored.  */
/* out: [r1-r0, d] fp32.  bytes_out (may be NULL): [r1-r0, Lp] ExpCast bytes */
/* of the final pass, for byte-level checks.  S_out and y_out (the fp32 FMA  */
/* result before rounding) likewise (may be NULL).                           */
/* S_in (mode 0, may be NULL): fp32 scores [r1-r0, Lp] to use in place of    */
/* the exactly rounded sums -- the pages fix the score only as the product  */
/* of the quantised Q and K, so any fp32 value a matrix core returns for it */
/* is a valid score, and every later step is then unique given S.           */
/*                                                                          */
/* Skip Softmax ([TRT] "Sparse Attention with Skip Softmax"): row i rejects */
/* block b when exp(mtilde - m) < lambda, mtilde the block's maximum score  */
/* and m the running maximum, both in natural-log units.  In the log2 units */
/* used here that is 2^(t - m) < lambda, tested as fp32(t - m) < skip_thr   */
/* with skip_thr = fp32(log2(lambda)) (-infinity: nothing is rejected).     */
/* A rejected block leaves m, l and O as they are and its bytes are 0; it   */
/* never moves the running maximum, since t < m there.                      */
/* ------------------------------------------------------------------------ */

void vco_attention_rows(int mode, int L, int d, int z_off,
                        const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                        const float* q_scale, const float* k_scale,
                        const float* v_scale, const float* v_mean,
                        const double* qf, const double* kf, const double* rf,
                        int r0, int r1, float* out, uint8_t* bytes_out, float* S_out,
                        float* y_out, const float* S_in, float skip_thr, const uint8_t* v_exp)
{
    int nb = (L + VCO_BLK - 1) / VCO_BLK;
    int64_t Lp = (int64_t)nb * VCO_BLK;
    double dec[256]; /* decode table, filled from vco_e4m3_decode */
    for (int t = 0; t < 256; t++) dec[t] = vco_e4m3_decode((uint8_t)t);
    float C0 = vco_c0(d);
    double C0d = 1.4426950408889634074 / sqrt((double)d);
    float KB = vco_kb(z_off);

#pragma omp parallel for schedule(dynamic, 1)
    for (int i = r0; i < r1; i++) {
        double* qrow = (double*)malloc(sizeof(double) * d);
        double* O = (double*)calloc((size_t)d, sizeof(double));
        double* Sd = (double*)malloc(sizeof(double) * VCO_BLK);
        float* S = (float*)malloc(sizeof(float) * VCO_BLK);
        double* p = (double*)malloc(sizeof(double) * VCO_BLK);
        const int real_qk = (mode == 1 || mode == 4); /* real-valued q, k and residual */
        for (int c = 0; c < d; c++)
            qrow[c] = real_qk ? qf[(int64_t)i * d + c] : dec[q8[(int64_t)i * d + c]];
        double* p4 = (double*)malloc(sizeof(double) * VCO_BLK);
        double m = -INFINITY, l = 0.0;
        for (int b = 0; b < nb; b++) {
            int n = (L - b * VCO_BLK < VCO_BLK) ? L - b * VCO_BLK : VCO_BLK;
            double m_new, ell = 0.0;
            /* scores */
            for (int j = 0; j < n; j++) {
                if (!real_qk && S_in) {
                    S[j] = S_in[(int64_t)(i - r0) * Lp + b * VCO_BLK + j];
                    Sd[j] = S[j];
                    continue;
                }
                int64_t kr = (int64_t)(b * VCO_BLK + j) * d;
                double acc = 0.0;
                for (int c = 0; c < d; c++)
                    acc += qrow[c] * (real_qk ? kf[kr + c] : dec[k8[kr + c]]);
                Sd[j] = acc;
                S[j] = (float)acc;
            }
            if (mode == 0 || mode == 2 || mode == 3 || mode == 4) {
                volatile float sqk = (mode == 4) ? 1.0f : q_scale[i / VCO_BLK] * k_scale[b];
                volatile float cb = sqk * C0;
                float mx = -INFINITY;
                for (int j = 0; j < n; j++) if (S[j] > mx) mx = S[j];
                volatile float t = mx * cb;
                volatile float gap = t - (float)m; /* +inf on the first block */
                if (gap < skip_thr) {
                    for (int j = 0; j < VCO_BLK; j++) {
                        int64_t o = (int64_t)(i - r0) * Lp + b * VCO_BLK + j;
                        if (bytes_out) bytes_out[o] = 0;
                        if (S_out) S_out[o] = (j < n) ? S[j] : 0.0f;
                        if (y_out) y_out[o] = -INFINITY;
                    }
                    continue;
                }
                float mnf = ((float)m > t) ? (float)m : t;
                if (m == -INFINITY) mnf = t;
                m_new = mnf;
                volatile float e8 = 8.0f * mnf;
                volatile float krow = KB - e8;
                volatile float c8 = 8.0f * cb;
                volatile float zrow = (float)z_off - mnf;
                if (mode == 3) {
                    /* fp32 probabilities, then one E8M0 scale and E2M1 codes per key group */
                    for (int j = 0; j < VCO_BLK; j++) p4[j] = (j < n) ? (double)(float)exp2((double)fmaf(S[j], cb, zrow)) : 0.0;
                    for (int g = 0; g < 4; g++) {
                        double A = 0.0;
                        for (int j = 0; j < n; j++)
                            if (vco_fp4_group(j) == g && p4[j] > A) A = p4[j];
                        int e = vco_e8m0_exp(A);
                        for (int j = 0; j < VCO_BLK; j++) {
                            if (vco_fp4_group(j) != g) continue;
                            uint8_t code = (j < n && e > -127) ? vco_e2m1_encode(ldexp(p4[j], -e)) : 0;
                            double ph = vco_e2m1_decode(code) * ldexp(1.0, e);
                            int64_t o = (int64_t)(i - r0) * Lp + b * VCO_BLK + j;
                            if (bytes_out) bytes_out[o] = code;
                            if (S_out) S_out[o] = (j < n) ? S[j] : 0.0f;
                            if (y_out) y_out[o] = (float)ph;
                            p[j] = ph;
                            if (j < n) ell += ph;
                        }
                    }
                }
                for (int j = 0; j < VCO_BLK && mode != 3; j++) {
                    uint8_t by = 0;
                    if (j < n)
                        by = (mode == 0 || mode == 4) ? vco_expcast1(S[j], c8, krow)
                                                      : vco_e4m3_encode((float)exp2((double)fmaf(S[j], cb, zrow)));
                    if (bytes_out) bytes_out[(int64_t)(i - r0) * Lp + b * VCO_BLK + j] = by;
                    if (S_out) S_out[(int64_t)(i - r0) * Lp + b * VCO_BLK + j] = (j < n) ? S[j] : 0.0f;
                    if (y_out)
                        y_out[(int64_t)(i - r0) * Lp + b * VCO_BLK + j] =
                            (j >= n) ? -INFINITY : (mode == 0 || mode == 4) ? fmaf(S[j], c8, krow) : fmaf(S[j], cb, zrow);
                    p[j] = dec[by];
                    if (j < n) ell += p[j];
                }
            } else {
                double mx = -INFINITY;
                for (int j = 0; j < n; j++) if (Sd[j] * C0d > mx) mx = Sd[j] * C0d;
                if (mx - m < (double)skip_thr) continue;
                m_new = (m > mx) ? m : mx;
                for (int j = 0; j < n; j++) { p[j] = exp2(Sd[j] * C0d - m_new); ell += p[j]; }
            }
            double alpha = (m == -INFINITY) ? 0.0 : exp2(m - m_new);
            for (int c = 0; c < d; c++) {
                int64_t vr = ((int64_t)b * d + c) * VCO_BLK;
                double acc = 0.0;
                for (int j = 0; j < n; j++) {
                    double rv;
                    if (mode == 3)
                        rv = vco_e2m1_decode(v8[vr + j]) * ldexp(1.0, (int)v_exp[((int64_t)b * d + c) * 4 + vco_fp4_group(j)] - 127);
                    else
                        rv = real_qk ? rf[vr + j] : dec[v8[vr + j]];
                    acc += p[j] * rv;
                }
                double sv = (real_qk || mode == 3) ? 1.0 : (double)v_scale[(int64_t)b * d + c];
                double accr = real_qk ? acc : (double)(float)acc;
                O[c] = alpha * O[c] + sv * accr + ell * (double)v_mean[(int64_t)b * d + c];
            }
            l = alpha * l + ell;
            m = m_new;
        }
        for (int c = 0; c < d; c++) out[(int64_t)(i - r0) * d + c] = (float)(O[c] / l);
        free(qrow); free(O); free(Sd); free(S); free(p); free(p4);
    }
}

/* ------------------------------------------------------------------------ */
/* SAGE-style quantised attention, the baseline of [TRT] "Quantized          */
/* Attention": five settings fix it -- QK^T in INT8 (the blog's choice) or   */
/* FP8, PV in FP8 E4M3, one Q scale per query token (q block size 1), one K  */
/* scale per 16 consecutive keys (k block size 16), and one V scale per      */
/* channel of a head, taken over all of its tokens (v block size 1).         */
/* Readings where the blog is silent:                                       */
/*  - a scale is amax / qmax with qmax = 127 (INT8) or 448 (E4M3), and the   */
/*    same zero rule as above (amax < 2^-100: scale 0, codes 0);            */
/*  - INT8 codes: round to nearest, ties to even, of fp32(x * inv), clamped  */
/*    to [-127, 127], stored as two's-complement bytes;                     */
/*  - K is smoothed by its per-channel mean when smooth_k is set (the       */
/*    SageAttention line smooths K; the softmax does not change);           */
/*  - tokens stay in sequence order and there are no block means;           */
/*  - the score coefficient of query i and key j is                         */
/*    c_ij = fp32(fp32(s_q,i C0) s_k,j/16);                                  */
/*  - P bytes come from the exp-then-cast path (prob_cast 1, the FP8 path    */
/*    of the SageAttention line) or from ExpCast (prob_cast 0), with the     */
/*    same running maximum and z_off as the V-Smooth path.                  */
/* ------------------------------------------------------------------------ */

static void vco_sage_scale(float A, float qmax, float* s, float* inv)
{
    if (!((double)A >= ldexp(1.0, -100))) { *s = 0.0f; *inv = 0.0f; return; }
    volatile float num = qmax;
    *s = A / num;
    *inv = num / A;
}

static inline uint8_t vco_i8_code(float x, float inv)
{
    volatile float y = x * inv; /* one IEEE single multiply */
    double a = vco_rne(fabs((double)y));
    if (a > 127.0) a = 127.0;
    int v = (y < 0.0f) ? -(int)a : (int)a;
    return (uint8_t)(int8_t)v;
}

static inline double vco_i8_value(uint8_t b) { return (double)(int8_t)b; }

/* One head.  q,k,v: bf16 bits [L, d].  Outputs: q8 [Lp, d] and k8 [Lp, d]   */
/* (INT8 or E4M3 codes, sequence order), v8 [nb, d, 128] E4M3 codes in       */
/* natural slot order, q_scale [Lp], k_scale [Lp / 16], v_scale [d].  Padded  */
/* tokens (>= L) get code 0 and scale 0 and take no part in any amax.       */
void vco_sage_prepare_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int L, int d,
                           int qk_int8, int smooth_k, uint8_t* q8, uint8_t* k8, uint8_t* v8,
                           float* q_scale, float* k_scale, float* v_scale)
{
    int nb = (L + VCO_BLK - 1) / VCO_BLK;
    int Lp = nb * VCO_BLK;
    float qmax = qk_int8 ? 127.0f : 448.0f;
    float* kbar = (float*)calloc((size_t)d, sizeof(float));
    if (smooth_k) vco_k_mean(k, L, d, kbar);
    float* buf = (float*)malloc(sizeof(float) * 16 * d);

    /* Q: one scale per token */
    for (int i = 0; i < Lp; i++) {
        float A = 0.0f, s, inv;
        for (int c = 0; c < d && i < L; c++) {
            float t = fabsf(vco_bf16(q[(int64_t)i * d + c]));
            if (t > A) A = t;
        }
        vco_sage_scale(A, qmax, &s, &inv);
        q_scale[i] = (i < L) ? s : 0.0f;
        for (int c = 0; c < d; c++) {
            uint8_t code = 0;
            if (i < L) {
                float x = vco_bf16(q[(int64_t)i * d + c]);
                code = qk_int8 ? vco_i8_code(x, inv) : vco_quant(x, inv);
            }
            q8[(int64_t)i * d + c] = code;
        }
    }

    /* K: K' = fp32(K - kbar), one scale per 16 consecutive tokens */
    for (int g = 0; g < Lp / 16; g++) {
        float A = 0.0f, s, inv;
        for (int r = 0; r < 16; r++) {
            int i = 16 * g + r;
            for (int c = 0; c < d; c++) {
                volatile float t = (i < L) ? vco_bf16(k[(int64_t)i * d + c]) - kbar[c] : 0.0f;
                buf[r * d + c] = t;
                if (fabsf(t) > A) A = fabsf(t);
            }
        }
        vco_sage_scale(A, qmax, &s, &inv);
        k_scale[g] = s;
        for (int r = 0; r < 16; r++) {
            int i = 16 * g + r;
            for (int c = 0; c < d; c++) {
                uint8_t code = 0;
                if (i < L) code = qk_int8 ? vco_i8_code(buf[r * d + c], inv) : vco_quant(buf[r * d + c], inv);
                k8[(int64_t)i * d + c] = code;
            }
        }
    }

    /* V: one E4M3 scale per channel over the head's tokens */
    for (int c = 0; c < d; c++) {
        float A = 0.0f, s, inv;
        for (int i = 0; i < L; i++) {
            float t = fabsf(vco_bf16(v[(int64_t)i * d + c]));
            if (t > A) A = t;
        }
        vco_sage_scale(A, 448.0f, &s, &inv);
        v_scale[c] = s;
        for (int b = 0; b < nb; b++)
            for (int j = 0; j < VCO_BLK; j++) {
                int i = b * VCO_BLK + j;
                v8[((int64_t)b * d + c) * VCO_BLK + j] = (i < L) ? vco_quant(vco_bf16(v[(int64_t)i * d + c]), inv) : 0;
            }
    }
    free(buf);
    free(kbar);
}

/* Blockwise SAGE attention for query rows [r0, r1) of one head, from the    */
/* output of vco_sage_prepare_head.  Per row i, for each 128-key block b in  */
/* ascending order:                                                          */
/*   S_j   = fp32(exact sum_c qhat_ic khat_jc)   (or S_in, as above)         */
/*   c_j   = fp32(fp32(s_q,i C0) s_k,j/16)                                   */
/*   t     = max over valid j of fp32(S_j c_j);  m' = max(m, t)             */
/*   bytes = ExpCast(S_j, fp32(8 c_j), fp32(KB - 8 m'))       (prob_cast 0)  */
/*         | E4M3(fp32(2^fmaf(S_j, c_j, fp32(z_off - m'))))   (prob_cast 1)  */
/*   l_b   = sum_j decode(byte_j);  acc_c = fp32(exact sum_j p_j vhat_jc)    */
/*   alpha = 2^(m - m') (0 on the first block)                              */
/*   O     = alpha O + acc;  l = alpha l + l_b       (double)                */
/* and the output is O_c s_v,c / l.  bytes_out / S_out as in                */
/* vco_attention_rows (may be NULL).                                         */
void vco_sage_rows(int prob_cast, int qk_int8, int L, int d, int z_off,
                   const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                   const float* q_scale, const float* k_scale, const float* v_scale,
                   int r0, int r1, float* out, uint8_t* bytes_out, float* S_out, const float* S_in)
{
    int nb = (L + VCO_BLK - 1) / VCO_BLK;
    int64_t Lp = (int64_t)nb * VCO_BLK;
    double dec[256];
    for (int t = 0; t < 256; t++) dec[t] = vco_e4m3_decode((uint8_t)t);
    float C0 = vco_c0(d);
    float KB = vco_kb(z_off);

#pragma omp parallel for schedule(dynamic, 1)
    for (int i = r0; i < r1; i++) {
        double* qrow = (double*)malloc(sizeof(double) * d);
        double* O = (double*)calloc((size_t)d, sizeof(double));
        float* S = (float*)malloc(sizeof(float) * VCO_BLK);
        float* cj = (float*)malloc(sizeof(float) * VCO_BLK);
        double* p = (double*)malloc(sizeof(double) * VCO_BLK);
        for (int c = 0; c < d; c++) {
            uint8_t b = q8[(int64_t)i * d + c];
            qrow[c] = qk_int8 ? vco_i8_value(b) : dec[b];
        }
        volatile float sqc = q_scale[i] * C0;
        double m = -INFINITY, l = 0.0;
        for (int b = 0; b < nb; b++) {
            int n = (L - b * VCO_BLK < VCO_BLK) ? L - b * VCO_BLK : VCO_BLK;
            float t = -INFINITY;
            for (int j = 0; j < n; j++) {
                int64_t kr = (int64_t)(b * VCO_BLK + j) * d;
                if (S_in) {
                    S[j] = S_in[(int64_t)(i - r0) * Lp + b * VCO_BLK + j];
                } else {
                    double acc = 0.0;
                    for (int c = 0; c < d; c++)
                        acc += qrow[c] * (qk_int8 ? vco_i8_value(k8[kr + c]) : dec[k8[kr + c]]);
                    S[j] = (float)acc;
                }
                volatile float cc = sqc * k_scale[(b * VCO_BLK + j) / 16];
                cj[j] = cc;
                volatile float x = S[j] * cc;
                if (x > t) t = x;
            }
            float mnf = (m == -INFINITY || t > (float)m) ? t : (float)m;
            double m_new = mnf;
            volatile float e8 = 8.0f * mnf;
            volatile float krow = KB - e8;
            volatile float zrow = (float)z_off - mnf;
            double ell = 0.0;
            for (int j = 0; j < VCO_BLK; j++) {
                uint8_t by = 0;
                if (j < n) {
                    if (prob_cast == 0) {
                        volatile float c8 = 8.0f * cj[j];
                        by = vco_expcast1(S[j], c8, krow);
                    } else {
                        by = vco_e4m3_encode((float)exp2((double)fmaf(S[j], cj[j], zrow)));
                    }
                }
                int64_t o = (int64_t)(i - r0) * Lp + b * VCO_BLK + j;
                if (bytes_out) bytes_out[o] = by;
                if (S_out) S_out[o] = (j < n) ? S[j] : 0.0f;
                p[j] = dec[by];
                if (j < n) ell += p[j];
            }
            double alpha = (m == -INFINITY) ? 0.0 : exp2(m - m_new);
            for (int c = 0; c < d; c++) {
                int64_t vr = ((int64_t)b * d + c) * VCO_BLK;
                double acc = 0.0;
                for (int j = 0; j < n; j++) acc += p[j] * dec[v8[vr + j]];
                O[c] = alpha * O[c] + (double)(float)acc;
            }
            l = alpha * l + ell;
            m = m_new;
        }
        for (int c = 0; c < d; c++) out[(int64_t)(i - r0) * d + c] = (float)((double)v_scale[c] * O[c] / l);
        free(qrow); free(O); free(S); free(cj); free(p);
    }
}

/* ------------------------------------------------------------------------ */
/* Whole-tensor drivers over B*H heads (OpenMP over heads).                  */
/* ------------------------------------------------------------------------ */

int vco_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Full prepare.  perm_in may be NULL (k-means); perm_out receives the used
 * permutation.  kmeans_obj may be NULL.  kmeans_k <= 0 means nb. */
void vco_prepare(int B, int H, int L, int d, int kmeans_k, int kmeans_iters, uint64_t seed,
                 int smooth_k, int v_mode, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                 const int32_t* perm_in, uint8_t* q8, uint8_t* k8, uint8_t* v8, float* q_scale,
                 float* k_scale, float* v_scale, float* v_mean, int32_t* perm_out,
                 double* kmeans_obj)
{
    int nb = (L + VCO_BLK - 1) / VCO_BLK;
    int64_t Lp = (int64_t)nb * VCO_BLK;
    int kk = (kmeans_k > 0) ? kmeans_k : nb;
    int nh = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < nh; bh++) {
        int b = bh / H, h = bh % H;
        int64_t off = (int64_t)bh * L * d;
        int32_t* perm = perm_out + (int64_t)bh * L;
        if (perm_in) {
            memcpy(perm, perm_in + (int64_t)bh * L, sizeof(int32_t) * L);
            if (kmeans_obj) kmeans_obj[bh] = NAN;
        } else {
            int32_t* a = (int32_t*)malloc(sizeof(int32_t) * L);
            float* C = (float*)malloc(sizeof(float) * (size_t)kk * d);
            double J = vco_kmeans(v + off, L, d, kk, kmeans_iters, vco_head_seed(seed, b, h, H), a, C, NULL);
            vco_stable_perm(a, L, kk, perm);
            if (kmeans_obj) kmeans_obj[bh] = J;
            free(a); free(C);
        }
        vco_prepare_head(q + off, k + off, v + off, L, d, smooth_k, v_mode, perm,
                         q8 + (int64_t)bh * Lp * d, k8 + (int64_t)bh * Lp * d,
                         v8 + (int64_t)bh * nb * d * VCO_BLK, q_scale + (int64_t)bh * nb,
                         k_scale + (int64_t)bh * nb, v_scale + (int64_t)bh * nb * d,
                         v_mean + (int64_t)bh * nb * d, NULL);
    }
}
