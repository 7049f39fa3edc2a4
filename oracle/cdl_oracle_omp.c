/*
 * cdl_oracle_omp.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT; TIMING
 * ONLY.
 *
 * The oracle's dispatch and combine loops (cdl_oracle.c) run over tokens on
 * every host core with OpenMP, so that the benchmark can report the CPU
 * baseline on all cores next to the single-threaded oracle.  The arithmetic
 * of each token is the oracle's, token by token: the same bf16 decode, the
 * same fmaf chain over the valid slots in ascending order from +0, the same
 * single bf16 rounding, so the results are bit-identical to oracle_dispatch
 * and oracle_combine (a CPU test checks this).  Parity tests never use this
 * file; only the benchmark's cpu_baseline leg times it.  The layout (a stable
 * counting sort, well under 0.1% of a step) is not parallelised: the
 * all-core timing calls the single-threaded oracle_layout.
 *
 * Build (with cdl_oracle.c, which supplies the number formats):
 *   gcc -O2 -std=c99 -fPIC -shared -fopenmp -ffp-contract=off -fno-fast-math
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

float oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_bf16_rne(float v);

/* oracle_dispatch over tokens on `threads` threads: P[src2dst[t*k+j]] = x[t]
 * for every valid slot (each destination row is written by one token). */
void oracle_omp_dispatch(const uint16_t *x, int64_t T, int64_t H, int32_t k,
                         const int32_t *src2dst, uint16_t *P, int32_t threads)
{
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t d = src2dst[t * k + j];
            if (d >= 0)
                memcpy(P + (int64_t)d * H, x + t * H, (size_t)H * sizeof(uint16_t));
        }
    }
}

/* oracle_combine over tokens on `threads` threads (each thread keeps its own
 * fp32 accumulator row).  Returns the number of map entries at or beyond
 * y_rows (skipped, as in oracle_combine), or -1 if a buffer could not be
 * allocated. */
int64_t oracle_omp_combine(const uint16_t *Y, int64_t y_rows, int64_t H,
                           const int32_t *map, const float *w, int64_t T,
                           int32_t k, uint16_t *out, int32_t threads)
{
    int64_t bad = 0;
    int failed = 0;
#pragma omp parallel num_threads(threads) reduction(+ : bad) reduction(| : failed)
    {
        float *acc = (float *)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
        if (!acc)
            failed = 1;
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            if (!acc)
                continue;
            for (int64_t h = 0; h < H; ++h)
                acc[h] = 0.0f;
            for (int32_t j = 0; j < k; ++j) {
                int32_t r = map[t * k + j];
                if (r < 0)
                    continue;
                if ((int64_t)r >= y_rows) {
                    ++bad;
                    continue;
                }
                float wj = w[t * k + j];
                const uint16_t *yr = Y + (int64_t)r * H;
                for (int64_t h = 0; h < H; ++h)
                    acc[h] = fmaf(wj, oracle_bf16_to_f32(yr[h]), acc[h]);
            }
            for (int64_t h = 0; h < H; ++h)
                out[t * H + h] = oracle_bf16_rne(acc[h]);
        }
        free(acc);
    }
    return failed ? -1 : bad;
}
