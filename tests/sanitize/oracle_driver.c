/* Runs every entry point of the CPU oracle on small ragged problems, for an
 * AddressSanitizer / UndefinedBehaviorSanitizer build (test support; built
 * and run by tests/test_sanitizers_cpu.py).  Exits 0 when every call
 * returns finite outputs; the sanitizers abort on any memory or UB error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double vco_e4m3_decode(uint8_t b);
uint8_t vco_e4m3_encode(float xf);
void vco_e4m3_encode_array(const float* x, uint8_t* out, int64_t n);
void vco_e4m3_decode_array(const uint8_t* b, double* out, int64_t n);
void vco_e2m1_encode_array(const double* x, uint8_t* out, int64_t n);
int vco_e8m0_exp(double A);
uint64_t vco_head_seed(uint64_t seed, int b, int h, int H);
double vco_kmeans(const uint16_t* v, int L, int d, int k, int iters, uint64_t seed_bh, int32_t* assign,
                  float* centroids, double* J_hist);
double vco_kmeans_warm(const uint16_t* v, int L, int d, int k, int iters, const float* init, int32_t* assign,
                       float* centroids, double* J_hist);
void vco_stable_perm(const int32_t* a, int L, int k, int32_t* perm);
void vco_prepare_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int L, int d, int smooth_k,
                      int v_mode, const int32_t* perm, uint8_t* q8, uint8_t* k8, uint8_t* v8, float* q_scale,
                      float* k_scale, float* v_scale, float* v_mean, float* kbar_out);
void vco_prepare_head_fp4v(const uint16_t* q, const uint16_t* k, const uint16_t* v, int L, int d, int smooth_k,
                           const int32_t* perm, uint8_t* q8, uint8_t* k8, uint8_t* v4, uint8_t* v_exp,
                           float* q_scale, float* k_scale, float* v_mean);
void vco_expcast(const float* S, int64_t n, float c8, float krow, uint8_t* out);
void vco_attention_rows(int mode, int L, int d, int z_off, const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                        const float* q_scale, const float* k_scale, const float* v_scale, const float* v_mean,
                        const double* qf, const double* kf, const double* rf, int r0, int r1, float* out,
                        uint8_t* bytes_out, float* S_out, float* y_out, const float* S_in, float skip_thr,
                        const uint8_t* v_exp);
void vco_sage_prepare_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int L, int d, int qk_int8,
                           int smooth_k, uint8_t* q8, uint8_t* k8, uint8_t* v8, float* q_scale, float* k_scale,
                           float* v_scale);
void vco_sage_rows(int prob_cast, int qk_int8, int L, int d, int z_off, const uint8_t* q8, const uint8_t* k8,
                   const uint8_t* v8, const float* q_scale, const float* k_scale, const float* v_scale, int r0,
                   int r1, float* out, uint8_t* bytes_out, float* S_out, const float* S_in);
void vco_prepare(int B, int H, int L, int d, int kmeans_k, int kmeans_iters, uint64_t seed, int smooth_k,
                 int v_mode, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* perm_in,
                 uint8_t* q8, uint8_t* k8, uint8_t* v8, float* q_scale, float* k_scale, float* v_scale,
                 float* v_mean, int32_t* perm_out, double* kmeans_obj);

static uint64_t st = 12345;
static double unif(void) { st = st * 6364136223846793005ULL + 1442695040888963407ULL; return ((st >> 11) + 0.5) / 9007199254740992.0; }
static double gauss(void) { return sqrt(-2.0 * log(unif())) * cos(6.283185307179586 * unif()); }
static uint16_t bf16(float x) { uint32_t u; memcpy(&u, &x, 4); return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16); }

static int finite_f(const float* x, int64_t n) { for (int64_t i = 0; i < n; i++) if (!isfinite(x[i])) return 0; return 1; }

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); exit(1); } } while (0)

static void head_case(int L, int d)
{
    int nb = (L + 127) / 128, Lp = nb * 128;
    uint16_t *q = malloc(2 * (size_t)L * d), *k = malloc(2 * (size_t)L * d), *v = malloc(2 * (size_t)L * d);
    for (int64_t i = 0; i < (int64_t)L * d; i++) { q[i] = bf16((float)gauss()); k[i] = bf16((float)(gauss() + 0.5)); v[i] = bf16((float)gauss()); }
    int32_t *a = malloc(4 * (size_t)L), *perm = malloc(4 * (size_t)L);
    float* C = malloc(4 * (size_t)nb * d);
    double hist[4];
    double J = vco_kmeans(v, L, d, nb, 3, vco_head_seed(1, 0, 0, 1), a, C, hist);
    CHECK(isfinite(J) && J >= 0);
    J = vco_kmeans_warm(v, L, d, nb, 2, C, a, C, NULL);
    CHECK(isfinite(J));
    vco_stable_perm(a, L, nb, perm);
    uint8_t *q8 = malloc((size_t)Lp * d), *k8 = malloc((size_t)Lp * d), *v8 = malloc((size_t)nb * d * 128);
    float *qs = malloc(4 * (size_t)nb), *ks = malloc(4 * (size_t)nb), *vs = malloc(4 * (size_t)nb * d), *vm = malloc(4 * (size_t)nb * d);
    float* kbar = malloc(4 * (size_t)d);
    float* out = malloc(4 * (size_t)L * d);
    uint8_t* by = malloc((size_t)L * Lp);
    float *S = malloc(4 * (size_t)L * Lp), *y = malloc(4 * (size_t)L * Lp);
    for (int vmode = 0; vmode < 2; vmode++) {
        vco_prepare_head(q, k, v, L, d, 1, vmode, perm, q8, k8, v8, qs, ks, vs, vm, kbar);
        for (int mode = 0; mode <= 2; mode += 2) {
            vco_attention_rows(mode, L, d, 8, q8, k8, v8, qs, ks, vs, vm, NULL, NULL, NULL, 0, L, out, by, S, y, NULL,
                               -INFINITY, NULL);
            CHECK(finite_f(out, (int64_t)L * d));
            vco_attention_rows(mode, L, d, 0, q8, k8, v8, qs, ks, vs, vm, NULL, NULL, NULL, 0, L, out, by, NULL, NULL,
                               S, (float)log2(0.3), NULL);  /* given scores, Skip Softmax */
            CHECK(finite_f(out, (int64_t)L * d));
        }
    }
    /* real-valued modes 1 and 4 */
    double *qf = malloc(8 * (size_t)L * d), *kf = calloc((size_t)Lp * d, 8), *rf = calloc((size_t)nb * d * 128, 8);
    for (int64_t i = 0; i < (int64_t)L * d; i++) { qf[i] = gauss(); kf[i] = gauss(); }
    for (int64_t i = 0; i < (int64_t)nb * d * 128; i++) rf[i] = gauss();
    for (int mode = 1; mode <= 4; mode += 3) {
        vco_attention_rows(mode, L, d, 8, NULL, NULL, NULL, NULL, NULL, NULL, vm, qf, kf, rf, 0, L, out, NULL, NULL,
                           NULL, NULL, -INFINITY, NULL);
        CHECK(finite_f(out, (int64_t)L * d));
    }
    /* 4-bit */
    uint8_t *v4 = malloc((size_t)nb * d * 128), *ve = malloc((size_t)nb * d * 4);
    vco_prepare_head_fp4v(q, k, v, L, d, 1, perm, q8, k8, v4, ve, qs, ks, vm);
    vco_attention_rows(3, L, d, 8, q8, k8, v4, qs, ks, NULL, vm, NULL, NULL, NULL, 0, L, out, by, S, y, NULL,
                       -INFINITY, ve);
    CHECK(finite_f(out, (int64_t)L * d));
    /* SAGE */
    float* qss = malloc(4 * (size_t)Lp);
    float* kss = malloc(4 * (size_t)(Lp / 16));
    float* vss = malloc(4 * (size_t)d);
    for (int i8 = 0; i8 < 2; i8++)
        for (int pc = 0; pc < 2; pc++) {
            vco_sage_prepare_head(q, k, v, L, d, i8, 1, q8, k8, v8, qss, kss, vss);
            vco_sage_rows(pc, i8, L, d, 8, q8, k8, v8, qss, kss, vss, 0, L, out, by, S, NULL);
            CHECK(finite_f(out, (int64_t)L * d));
        }
    free(q); free(k); free(v); free(a); free(perm); free(C); free(q8); free(k8); free(v8); free(qs); free(ks);
    free(vs); free(vm); free(kbar); free(out); free(by); free(S); free(y); free(qf); free(kf); free(rf); free(v4);
    free(ve); free(qss); free(kss); free(vss);
}

int main(void)
{
    for (int c = 0; c < 256; c++) {
        if ((c & 0x7F) == 0x7F) continue; /* NaN codes: the encoder takes finite inputs only */
        CHECK(vco_e4m3_encode((float)vco_e4m3_decode((uint8_t)c)) == (uint8_t)c);
    }
    float xs[5] = {0.0f, -0.0f, 448.0f, 1e30f, -3.5f};
    uint8_t cs[5];
    double ds[5];
    vco_e4m3_encode_array(xs, cs, 5);
    vco_e4m3_decode_array(cs, ds, 5);
    double e2[3] = {0.3, 5.9, -7.0};
    uint8_t c2[3];
    vco_e2m1_encode_array(e2, c2, 3);
    CHECK(vco_e8m0_exp(0.0) == -127);
    float Sx[3] = {1.0f, -200.0f, 3.0f};
    uint8_t bx[3];
    vco_expcast(Sx, 3, 8.0f, 119.65f, bx);
    head_case(300, 64);
    head_case(129, 128);
    head_case(1, 128);
    /* whole-tensor prepare with k-means, B = 1, H = 2 */
    int B = 1, H = 2, L = 200, d = 64, nb = 2, Lp = 256;
    uint16_t* qkv = malloc(2 * 3 * (size_t)B * H * L * d);
    for (int64_t i = 0; i < 3LL * B * H * L * d; i++) qkv[i] = bf16((float)gauss());
    uint8_t *q8 = malloc((size_t)B * H * Lp * d), *k8 = malloc((size_t)B * H * Lp * d), *v8 = malloc((size_t)B * H * nb * d * 128);
    float *qs = malloc(4 * (size_t)B * H * nb), *ks = malloc(4 * (size_t)B * H * nb);
    float *vs = malloc(4 * (size_t)B * H * nb * d), *vm = malloc(4 * (size_t)B * H * nb * d);
    int32_t* po = malloc(4 * (size_t)B * H * L);
    double obj[2];
    vco_prepare(B, H, L, d, 0, 4, 7, 1, 0, qkv, qkv + (size_t)B * H * L * d, qkv + 2 * (size_t)B * H * L * d, NULL, q8, k8,
                v8, qs, ks, vs, vm, po, obj);
    CHECK(isfinite(obj[0]) && isfinite(obj[1]));
    free(qkv); free(q8); free(k8); free(v8); free(qs); free(ks); free(vs); free(vm); free(po);
    printf("oracle driver ok\n");
    return 0;
}
