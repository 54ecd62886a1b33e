/* Driver for the address/undefined-behaviour sanitizer build of the oracle:
 * every exported function on small seeded inputs, ragged sizes included.
 * The values are checked elsewhere (the oracle's pins); here only memory and
 * arithmetic safety are at stake.  Exits non-zero on an inconsistency. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t oracle_u16(uint64_t seed, uint64_t c);
uint32_t oracle_threshold(float p);
void oracle_keep(uint64_t seed, uint64_t offset, const int64_t *rows, int64_t nrows, int64_t k, uint32_t T,
                 uint8_t *keep);
void oracle_pack_bits(const uint8_t *keep, int64_t nrows, int64_t k, uint32_t *bits);
void oracle_lora_s(const double *X, const uint8_t *keep, const double *A, int64_t nrows, int64_t k, int64_t r,
                   float p, double *S);
void oracle_lora_y(const double *X, const double *W, const double *S, const double *B, int64_t nrows, int64_t k,
                   int64_t n, int64_t r, double alpha, double *Y);
void oracle_lora_ds(const double *dY, const double *B, int64_t nrows, int64_t n, int64_t r, double alpha,
                    double *dS);
void oracle_lora_dx(const double *dY, const double *W, const double *dS, const double *A, const uint8_t *keep,
                    int64_t nrows, int64_t k, int64_t n, int64_t r, float p, double *dX);
void oracle_lora_db_acc(const double *S, const double *dY, int64_t nrows, int64_t n, int64_t r, double alpha,
                        double *dB);
void oracle_lora_da_acc(const double *X, const uint8_t *keep, const double *dS, int64_t nrows, int64_t k,
                        int64_t r, float p, double *dA);
void oracle_dora_norm(const double *W, const double *A, const double *B, int64_t k, int64_t n, int64_t r,
                      double alpha, const int64_t *cols, int64_t ncols, double *out);
int oracle_num_threads(void);

static double *rnd(int64_t n, unsigned *st) {
    double *v = (double *)malloc((size_t)n * sizeof(double));
    for (int64_t i = 0; i < n; ++i) v[i] = (double)(rand_r(st) % 2001 - 1000) / 1000.0;
    return v;
}

int main(void) {
    unsigned st = 11;
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
    oracle_philox4x32_10(ctr, key, out);
    const float ps[] = {0.0f, 0.1f, 0.5f, 0.9999f};
    for (int q = 0; q < 4; ++q)
        if (oracle_threshold(ps[q]) > 65536u) return 1;
    const int64_t shapes[][4] = {{5, 40, 24, 3}, {1, 8, 8, 1}, {7, 33, 16, 17}, {3, 64, 40, 8}};
    for (int sh = 0; sh < 4; ++sh) {
        const int64_t m = shapes[sh][0], k = shapes[sh][1], n = shapes[sh][2], r = shapes[sh][3];
        int64_t *rows = (int64_t *)malloc((size_t)m * sizeof(int64_t));
        for (int64_t i = 0; i < m; ++i) rows[i] = 3 * i + 1;
        uint8_t *keep = (uint8_t *)malloc((size_t)(m * k));
        const uint32_t T = oracle_threshold(0.25f);
        oracle_keep(99, 8 * (uint64_t)sh, rows, m, k, T, keep);
        uint32_t *bits = (uint32_t *)malloc((size_t)(m * ((k + 31) / 32)) * sizeof(uint32_t));
        oracle_pack_bits(keep, m, k, bits);
        double *X = rnd(m * k, &st), *W = rnd(k * n, &st), *A = rnd(k * r, &st), *B = rnd(r * n, &st);
        double *dY = rnd(m * n, &st), *S = rnd(m * r, &st), *Y = rnd(m * n, &st), *dS = rnd(m * r, &st);
        double *dX = rnd(m * k, &st), *dA = (double *)calloc((size_t)(k * r), sizeof(double));
        double *dB = (double *)calloc((size_t)(r * n), sizeof(double));
        oracle_lora_s(X, keep, A, m, k, r, 0.25f, S);
        oracle_lora_y(X, W, S, B, m, k, n, r, 2.0, Y);
        oracle_lora_ds(dY, B, m, n, r, 2.0, dS);
        oracle_lora_dx(dY, W, dS, A, keep, m, k, n, r, 0.25f, dX);
        oracle_lora_db_acc(S, dY, m, n, r, 2.0, dB);
        oracle_lora_da_acc(X, keep, dS, m, k, r, 0.25f, dA);
        int64_t cols[3] = {0, n / 2, n - 1};
        double norms[3];
        oracle_dora_norm(W, A, B, k, n, r, 2.0, cols, 3, norms);
        for (int q = 0; q < 3; ++q)
            if (!(norms[q] >= 0.0)) return 2;
        free(rows); free(keep); free(bits); free(X); free(W); free(A); free(B); free(dY); free(S);
        free(Y); free(dS); free(dX); free(dA); free(dB);
    }
    if (oracle_num_threads() < 1) return 3;
    printf("oracle driver: all calls completed\n");
    return 0;
}
