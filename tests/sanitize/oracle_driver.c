/*
 * Exercise every entry point of the CPU oracle (oracle/attn_oracle.c) on small shapes, every mask, grouped
 * K/V heads, empty and degenerate sizes, so that a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * sees each loop and index. Checks a few invariants on the way (rows of weights sum to 1, masked weights are
 * 0); exits non-zero on a failed check. Test infrastructure, built and run by tests/test_sanitizers.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attn(const double *Q, const double *K, const double *V, int64_t B, int64_t H, int64_t Hkv, int64_t Nq,
                int64_t Nk, int64_t d, int64_t dv, int mask_kind, const int32_t *valid_lens, double scale, double *O,
                double *A, double *LSE, int nthreads);
int oracle_attn_rows(const double *Q, const double *K, const double *V, int64_t B, int64_t H, int64_t Hkv,
                     int64_t Nq, int64_t Nk, int64_t d, int64_t dv, int mask_kind, const int32_t *valid_lens,
                     double scale, const int64_t *rows, int64_t nrows, double *O_rows, double *LSE_rows, int nthreads);
int oracle_attn_bwd(const double *Q, const double *K, const double *V, const double *dO, int64_t B, int64_t H,
                    int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, int mask_kind,
                    const int32_t *valid_lens, double scale, double *dQ, double *dK, double *dV, int nthreads);
int oracle_mha(const double *X, const double *Wqkv, const double *Wo, int64_t B, int64_t N, int64_t d_model,
               int64_t h, double *Y, int nthreads);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uni(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0 - 0.5;
}

static double *rnd(int64_t n)
{
    double *p = malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) p[i] = uni();
    return p;
}

static int fails = 0;
#define CHECK(c)                                                                                               \
    do {                                                                                                       \
        if (!(c)) {                                                                                            \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);                                    \
            ++fails;                                                                                           \
        }                                                                                                      \
    } while (0)

int main(void)
{
    const int64_t shapes[][7] = {/* B, H, Hkv, Nq, Nk, d, dv */
                                 {1, 1, 1, 1, 1, 1, 1}, {2, 2, 1, 5, 5, 16, 16}, {2, 4, 2, 7, 9, 8, 3},
                                 {1, 3, 3, 6, 6, 4, 4}, {2, 2, 2, 0, 4, 8, 8},   {1, 2, 1, 4, 0, 8, 8}};
    for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; ++si) {
        const int64_t B = shapes[si][0], H = shapes[si][1], Hkv = shapes[si][2], Nq = shapes[si][3],
                      Nk = shapes[si][4], d = shapes[si][5], dv = shapes[si][6];
        double *Q = rnd(B * H * Nq * d), *K = rnd(B * Hkv * Nk * d), *V = rnd(B * Hkv * Nk * dv);
        double *dO = rnd(B * H * Nq * dv);
        double *O = rnd(B * H * Nq * dv), *A = rnd(B * H * Nq * Nk), *L = rnd(B * H * Nq);
        double *dQ = rnd(B * H * Nq * d), *dK = rnd(B * Hkv * Nk * d), *dV = rnd(B * Hkv * Nk * dv);
        int32_t *vl = malloc((size_t)(B > 0 ? B : 1) * sizeof(int32_t));
        for (int64_t b = 0; b < B; ++b) vl[b] = (int32_t)(b % 2 ? Nk : Nk / 2);
        for (int mask = 0; mask < 4; ++mask) {
            CHECK(oracle_attn(Q, K, V, B, H, Hkv, Nq, Nk, d, dv, mask, vl, 0.3, O, A, L, 2) > 0);
            for (int64_t r = 0; r < B * H * Nq; ++r) {
                double z = 0.0;
                for (int64_t j = 0; j < Nk; ++j) z += A[r * Nk + j];
                CHECK(z == 0.0 || fabs(z - 1.0) < 1e-12);
            }
            int64_t rows[3] = {0, B * H * Nq / 2, B * H * Nq - 1};
            double *Or = rnd(3 * dv), *Lr = rnd(3);
            if (B * H * Nq > 0)
                CHECK(oracle_attn_rows(Q, K, V, B, H, Hkv, Nq, Nk, d, dv, mask, vl, 0.3, rows, 3, Or, Lr, 1) > 0);
            free(Or), free(Lr);
            CHECK(oracle_attn_bwd(Q, K, V, dO, B, H, Hkv, Nq, Nk, d, dv, mask, vl, 0.3, dQ, dK, dV, 2) > 0);
        }
        CHECK(oracle_attn(Q, K, V, B, H, Hkv, Nq, Nk, d, dv, 7, vl, 0.3, O, A, L, 1) == -1);
        CHECK(oracle_attn(Q, K, V, B, H, Hkv, Nq, Nk, d, dv, 2, NULL, 0.3, O, A, L, 1) == -1);
        free(Q), free(K), free(V), free(dO), free(O), free(A), free(L), free(dQ), free(dK), free(dV), free(vl);
    }
    const int64_t mshapes[][3] = {{1, 3, 2}, {2, 5, 1}, {2, 4, 4}, {0, 3, 2}};
    for (size_t si = 0; si < sizeof mshapes / sizeof mshapes[0]; ++si) {
        const int64_t B = mshapes[si][0], N = mshapes[si][1], h = mshapes[si][2], dm = 4 * h;
        double *X = rnd(B * N * dm), *W = rnd(dm * 3 * dm), *Wo = rnd(dm * dm), *Y = rnd(B * N * dm);
        CHECK(oracle_mha(X, W, Wo, B, N, dm, h, Y, 2) > 0);
        CHECK(oracle_mha(X, W, Wo, B, N, dm, h + 1 + (dm % (h + 1) == 0), Y, 1) == -1 || dm % (h + 1) == 0);
        free(X), free(W), free(Wo), free(Y);
    }
    if (fails) return 1;
    printf("oracle driver: all checks passed\n");
    return 0;
}
