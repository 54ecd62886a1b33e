/*
 * CPU oracle for the LoRA linear layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, double-precision C.  Only tests/, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library; the product path
 * (the HIP library) never does, and the two share no code.
 *
 * What is computed (page "LoRAFusion: Efficient LoRA Fine-Tuning for LLMs",
 * juhe.plus blog, section 2 "LoRA parameter structure": Y = XW + alpha*(XA)B
 * with S = XA; papers.chlience.com notes, section 3, where the intermediate is
 * written S = X^ A, i.e. dropout is applied to X before A only):
 *
 *   keep[i][j] = u16(seed, offset + i*k + j) >= T          (dropout mask)
 *   X^         = s * keep (.) X,   s = 1/(1-p)             (inverted dropout)
 *   S          = X^ A                                      (m x r)
 *   Y          = X W + alpha * S B                         (m x n)
 *
 * Backward (the pages give no formulas; chain rule on the four lines above,
 * W frozen so there is no dW -- juhe.plus blog section 2, "W is frozen, only
 * A and B are updated"):
 *
 *   dB = alpha * S^T dY        dS = alpha * dY B^T
 *   dA = X^^T dS               dX = dY W^T + s * keep (.) (dS A^T)
 *
 * Dropout mask generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), keyed by the 64-bit
 * seed, evaluated at block index c >> 3 of the element counter c; the eight
 * 16-bit halves of its 128-bit output are the uniforms of elements 8b..8b+7,
 * lowest half of the lowest word first.  T = floor(p * 65536 + 0.5) computed
 * in double.  Element (i, j) of an m x k mask lives in 32-bit word
 * i*ceil(k/32) + j/32, bit j % 32.
 *
 * Every matrix is row-major.  Inputs arrive as double arrays holding the
 * exact values of the bf16 tensors.  OpenMP parallelises the outer loop of
 * each function; the arithmetic inside is a direct transcription of the
 * definition above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------------
 * Philox4x32-10, written from the SC'11 definition: a round multiplies the
 * even words by two fixed odd constants, keeps both halves of each 64-bit
 * product, and mixes the high halves with the odd words and the round key;
 * the key advances by two Weyl constants between rounds.
 * ------------------------------------------------------------------------- */
#define PHILOX_MUL0 0xD2511F53u
#define PHILOX_MUL1 0xCD9E8D57u
#define PHILOX_WEYL0 0x9E3779B9u
#define PHILOX_WEYL1 0xBB67AE85u

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_WEYL0;
            k1 += PHILOX_WEYL1;
        }
        uint64_t prod0 = (uint64_t)PHILOX_MUL0 * (uint64_t)x0;
        uint64_t prod1 = (uint64_t)PHILOX_MUL1 * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t y0 = hi1 ^ x1 ^ k0;
        uint32_t y1 = lo1;
        uint32_t y2 = hi0 ^ x3 ^ k1;
        uint32_t y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* The 16-bit uniform of element counter c. */
uint32_t oracle_u16(uint64_t seed, uint64_t c)
{
    uint64_t block = c >> 3;
    uint32_t ctr[4] = {(uint32_t)block, (uint32_t)(block >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    uint32_t lane = (uint32_t)(c & 7u);
    uint32_t word = out[lane >> 1];
    return (lane & 1u) ? (word >> 16) : (word & 0xFFFFu);
}

/* Drop threshold: an element is kept iff its uniform is >= T. */
uint32_t oracle_threshold(float p)
{
    double t = (double)p * 65536.0 + 0.5;
    return (uint32_t)t; /* t >= 0.5, so truncation is floor */
}

/* keep[ii*k + j] (0/1 bytes) for the rows listed in `rows` (global indices). */
void oracle_keep(uint64_t seed, uint64_t offset, const int64_t *rows, int64_t nrows, int64_t k,
                 uint32_t T, uint8_t *keep)
{
    #pragma omp parallel for schedule(static)
    for (int64_t ii = 0; ii < nrows; ++ii) {
        for (int64_t j = 0; j < k; ++j) {
            uint64_t c = offset + (uint64_t)rows[ii] * (uint64_t)k + (uint64_t)j;
            keep[ii * k + j] = (uint8_t)(oracle_u16(seed, c) >= T);
        }
    }
}

/* Pack a 0/1 byte mask into the documented bit layout. */
void oracle_pack_bits(const uint8_t *keep, int64_t nrows, int64_t k, uint32_t *bits)
{
    int64_t words = (k + 31) / 32;
    memset(bits, 0, (size_t)(nrows * words) * sizeof(uint32_t));
    for (int64_t i = 0; i < nrows; ++i)
        for (int64_t j = 0; j < k; ++j)
            if (keep[i * k + j])
                bits[i * words + j / 32] |= (1u << (j % 32));
}

/* Inverted-dropout scale s = 1/(1-p). */
static double dropout_scale(float p) { return 1.0 / (1.0 - (double)p); }

/* S = (s * keep (.) X) A for nrows rows: X nrows x k, A k x r, S nrows x r. */
void oracle_lora_s(const double *X, const uint8_t *keep, const double *A, int64_t nrows, int64_t k,
                   int64_t r, float p, double *S)
{
    double s = dropout_scale(p);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        for (int64_t c = 0; c < r; ++c) S[i * r + c] = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            double xhat = keep[i * k + j] ? s * X[i * k + j] : 0.0;
            if (xhat == 0.0) continue;
            for (int64_t c = 0; c < r; ++c) S[i * r + c] += xhat * A[j * r + c];
        }
    }
}

/* Y = X W + alpha * S B for nrows rows: W k x n, B r x n. */
void oracle_lora_y(const double *X, const double *W, const double *S, const double *B, int64_t nrows,
                   int64_t k, int64_t n, int64_t r, double alpha, double *Y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        double *y = Y + i * n;
        for (int64_t j = 0; j < n; ++j) y[j] = 0.0;
        for (int64_t t = 0; t < k; ++t) {
            double x = X[i * k + t];
            const double *w = W + t * n;
            for (int64_t j = 0; j < n; ++j) y[j] += x * w[j];
        }
        for (int64_t c = 0; c < r; ++c) {
            double as = alpha * S[i * r + c];
            const double *b = B + c * n;
            for (int64_t j = 0; j < n; ++j) y[j] += as * b[j];
        }
    }
}

/* dS = alpha * dY B^T for nrows rows: dY nrows x n, B r x n, dS nrows x r. */
void oracle_lora_ds(const double *dY, const double *B, int64_t nrows, int64_t n, int64_t r,
                    double alpha, double *dS)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        for (int64_t c = 0; c < r; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < n; ++j) acc += dY[i * n + j] * B[c * n + j];
            dS[i * r + c] = alpha * acc;
        }
    }
}

/* dX = dY W^T + s * keep (.) (dS A^T) for nrows rows: dX nrows x k. */
void oracle_lora_dx(const double *dY, const double *W, const double *dS, const double *A,
                    const uint8_t *keep, int64_t nrows, int64_t k, int64_t n, int64_t r, float p,
                    double *dX)
{
    double s = dropout_scale(p);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        for (int64_t t = 0; t < k; ++t) {
            double base = 0.0;
            const double *w = W + t * n;
            for (int64_t j = 0; j < n; ++j) base += dY[i * n + j] * w[j];
            double lora = 0.0;
            for (int64_t c = 0; c < r; ++c) lora += dS[i * r + c] * A[t * r + c];
            dX[i * k + t] = base + (keep[i * k + t] ? s * lora : 0.0);
        }
    }
}

/* dB += alpha * S^T dY over nrows rows (dB r x n is accumulated into). */
void oracle_lora_db_acc(const double *S, const double *dY, int64_t nrows, int64_t n, int64_t r,
                        double alpha, double *dB)
{
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t c = 0; c < r; ++c) {
            double acc = 0.0;
            for (int64_t i = 0; i < nrows; ++i) acc += S[i * r + c] * dY[i * n + j];
            dB[c * n + j] += alpha * acc;
        }
    }
}

/* dA += (s * keep (.) X)^T dS over nrows rows (dA k x r is accumulated into). */
void oracle_lora_da_acc(const double *X, const uint8_t *keep, const double *dS, int64_t nrows,
                        int64_t k, int64_t r, float p, double *dA)
{
    double s = dropout_scale(p);
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < k; ++t) {
        for (int64_t c = 0; c < r; ++c) {
            double acc = 0.0;
            for (int64_t i = 0; i < nrows; ++i) {
                double xhat = keep[i * k + t] ? s * X[i * k + t] : 0.0;
                acc += xhat * dS[i * r + c];
            }
            dA[t * r + c] += acc;
        }
    }
}

/* DoRA norm of the adapted weight per output feature (page on the factored
 * DoRA norm, "core method": the norm of W + sBA per output feature, with s the
 * LoRA scale; with X W and W k x n an output feature is a column):
 *   out[q] = sqrt( sum_i ( W[i][j] + alpha * sum_t A[i][t] B[t][j] )^2 ),
 * j = cols[q].  The definition itself, dense, in double. */
void oracle_dora_norm(const double *W, const double *A, const double *B, int64_t k, int64_t n, int64_t r,
                      double alpha, const int64_t *cols, int64_t ncols, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < ncols; ++q) {
        int64_t j = cols[q];
        double acc = 0.0;
        for (int64_t i = 0; i < k; ++i) {
            double ab = 0.0;
            for (int64_t t = 0; t < r; ++t) ab += A[i * r + t] * B[t * n + j];
            double v = W[i * n + j] + alpha * ab;
            acc += v * v;
        }
        out[q] = sqrt(acc);
    }
}

/* Number of OpenMP threads the oracle runs with (for the CPU baseline). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
