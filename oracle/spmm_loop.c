/* Plain C oracle of the Load-as-Sparse, Compute-as-Dense product: Tiled-CSL decode and the
 * fp64 triple loop.
 *
 * TEST INFRASTRUCTURE ONLY.  It is loaded by the test suite and by the CPU-baseline leg of
 * bench.py; nothing on the product path links or calls it, and it shares no code, header or
 * table with the HIP library.
 *
 * Sources (Flash-LLM paper review, xllm-io):
 *   - section 3, "Tiled-CSL sparse encoding format": A is cut into tiles laid out one after
 *     another; each nonzero is a 32-bit word of a 16-bit value and a 16-bit position inside
 *     its tile; a per-tile offset array locates each tile's words;
 *   - section 2, "solution", and section 3, "core formulas": the product is C = A x B over the
 *     decoded (dense) A, so the oracle is the definition C[n][i] = sum_k A[i][k] * B[n][k].
 *
 * Readings where the pages are silent (the same as the Python oracle's):
 *   - a word holds the fp16 bits of the value in bits [15:0] and the row-major in-tile
 *     position r * tile_k + c in bits [31:16];
 *   - tiles are row-block-major; offsets[] has T + 1 entries counted in words, starting at 0,
 *     non-decreasing, each tile a multiple of 4 words; a position written twice must carry the
 *     same bits both times (padding repeats a real word);
 *   - B is [N][K] row-major, C is [N][rows] row-major; the sum runs over k in ascending order
 *     and accumulates in fp64.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16 -> binary64, from the format's definition: 1 sign bit, 5 exponent bits
 * (bias 15), 10 fraction bits; exponent 0 is zero / subnormal (fraction * 2^-24), exponent 31
 * is infinity (fraction 0) or NaN.  Every binary16 value is exact in binary64. */
static double half_to_double(uint16_t h) {
    const int sign = h >> 15;
    const int e = (h >> 10) & 0x1F;
    const int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = (double)f / 16777216.0; /* f * 2^-24 */
    } else if (e == 31) {
        if (f == 0) {
            v = 1.0 / 0.0;
        } else {
            v = 0.0 / 0.0;
        }
    } else {
        v = (double)(1024 + f);
        int s = e - 25; /* (1 + f / 1024) * 2^(e - 15) = (1024 + f) * 2^(e - 25) */
        while (s > 0) {
            v *= 2.0;
            --s;
        }
        while (s < 0) {
            v *= 0.5;
            ++s;
        }
    }
    return sign ? -v : v;
}

/* Decode a Tiled-CSL encoding into dense[M][K] (fp16 bits), which starts all +0.0.
 * `seen` is caller scratch of M * K bytes.  Returns 0, or a positive code naming the first
 * violated rule: 1 offsets[0] != 0, 2 decreasing offsets, 3 a tile not a multiple of 4 words,
 * 4 offsets[T] != nwords, 5 position outside the tile, 6 position outside A, 7 a position
 * written twice with different bits. */
int oracle_decode_tiled_csl(const uint32_t* words, int64_t nwords, const uint32_t* offs, int64_t M, int64_t K,
                            int32_t tile_m, int32_t tile_k, uint16_t* dense, uint8_t* seen) {
    const int64_t MB = (M + tile_m - 1) / tile_m;
    const int64_t KT = (K + tile_k - 1) / tile_k;
    const int64_t T = MB * KT;
    if (offs[0] != 0) return 1;
    for (int64_t t = 0; t < T; ++t) {
        if (offs[t + 1] < offs[t]) return 2;
        if ((offs[t + 1] - offs[t]) % 4 != 0) return 3;
    }
    if ((int64_t)offs[T] != nwords) return 4;
    memset(dense, 0, (size_t)(M * K) * sizeof(uint16_t));
    memset(seen, 0, (size_t)(M * K));
    for (int64_t t = 0; t < T; ++t) {
        const int64_t bm = t / KT, bk = t % KT;
        for (uint32_t w = offs[t]; w < offs[t + 1]; ++w) {
            const uint32_t word = words[w];
            const uint16_t value = (uint16_t)(word & 0xFFFFu);
            const uint32_t pos = word >> 16;
            if (pos >= (uint32_t)tile_m * (uint32_t)tile_k) return 5;
            const int64_t r = pos / (uint32_t)tile_k, c = pos % (uint32_t)tile_k;
            const int64_t i = bm * tile_m + r, j = bk * tile_k + c;
            if (i >= M || j >= K) return 6;
            if (seen[i * K + j] && dense[i * K + j] != value) return 7;
            seen[i * K + j] = 1;
            dense[i * K + j] = value;
        }
    }
    return 0;
}

/* out[n][r] = sum over k = 0 .. K-1 of A[rows[r]][k] * B[n][k], in fp64, k ascending.
 * A is the dense [M][K] matrix (fp16 bits, dropped positions +0.0), B is [N][K] (fp16 bits).
 * B is converted to fp64 once, each row of A when its turn comes.  The rows are shared out
 * over `threads` OpenMP threads (0: the runtime's default).  Returns 0, or 1 when memory for
 * the converted operands cannot be had. */
int oracle_spmm_loop(const uint16_t* A, const uint16_t* B, int64_t M, int64_t K, int64_t N, const int64_t* rows,
                     int64_t nrows, double* out, int threads) {
    (void)M;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
    double* b = (double*)malloc((size_t)(N * K) * sizeof(double));
    if (!b) return 1;
    for (int64_t x = 0; x < N * K; ++x) b[x] = half_to_double(B[x]);
    int failed = 0;
#pragma omp parallel
    {
        double* a = (double*)malloc((size_t)K * sizeof(double));
        if (!a) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!a) continue;
            const uint16_t* arow = A + rows[r] * K;
            for (int64_t k = 0; k < K; ++k) a[k] = half_to_double(arow[k]);
            for (int64_t n = 0; n < N; ++n) {
                const double* bn = b + n * K;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) acc += a[k] * bn[k];
                out[n * nrows + r] = acc;
            }
        }
        free(a);
    }
    free(b);
    return failed;
}

/* Threads the OpenMP runtime would use for a parallel region right now. */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
