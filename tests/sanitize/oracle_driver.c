/* Drives the C oracle under AddressSanitizer/UBSan or ThreadSanitizer (host
 * builds only): rotary code, append and attention with a multi-threaded
 * row pool over a small chunk-causal case, including a row subset.  Exits
 * non-zero if a call fails or a result is not finite; the sanitizers abort
 * on their own findings. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_rope(const double *x, double *y, int B, int64_t n, int H, int D, int64_t t0,
                int64_t tok_off, int64_t gh, int64_t gw, double theta);
int oracle_append(const double *x, double *cache, int B, int64_t n, int H, int D, int64_t cap,
                  int64_t cache_pos);
int oracle_attn(const double *q, const double *k, const double *v, int64_t cap, int64_t kv_len,
                int64_t q_pos0, int64_t chunk_tokens, double *o, double *lse, int B, int H,
                int D, int64_t Lq, double scale, const int64_t *rows, int64_t nrows,
                int nthreads);

static double rnd(unsigned *s) {
    *s = *s * 1103515245u + 12345u;
    return ((double)((*s >> 8) & 0xffff) / 32768.0) - 1.0;
}

int main(void) {
    const int B = 2, H = 3, D = 64, L = 48;
    const int64_t cap = 4 * L, n = L;
    unsigned seed = 7;
    double *x = malloc(sizeof(double) * B * n * H * D);
    double *y = malloc(sizeof(double) * B * n * H * D);
    double *k = calloc((size_t)B * H * cap * D, sizeof(double));
    double *v = calloc((size_t)B * H * cap * D, sizeof(double));
    double *o = malloc(sizeof(double) * B * n * H * D);
    double *lse = malloc(sizeof(double) * B * H * n);
    if (!x || !y || !k || !v || !o || !lse) return 2;
    for (int64_t i = 0; i < (int64_t)B * H * cap * D; ++i) k[i] = rnd(&seed), v[i] = rnd(&seed);
    for (int64_t i = 0; i < (int64_t)B * n * H * D; ++i) x[i] = rnd(&seed);
    /* rotate the chunk at t0 = 9 (6x8 frames), append it to slot 3 */
    if (oracle_rope(x, y, B, n, H, D, 9, 0, 6, 8, 10000.0)) return 3;
    if (oracle_append(y, k, B, n, H, D, cap, 3 * L)) return 4;
    /* every row, then a subset, with 4 worker threads */
    if (oracle_attn(y, k, v, cap, cap, 3 * L, L, o, lse, B, H, D, n, 0.125, NULL, 0, 4)) return 5;
    const int64_t rows[5] = {0, 7, 23, 24, 47};
    if (oracle_attn(y, k, v, cap, cap, 3 * L, L, o, lse, B, H, D, n, 0.125, rows, 5, 3)) return 6;
    for (int64_t i = 0; i < (int64_t)B * 5 * H * D; ++i)
        if (!isfinite(o[i])) return 7;
    /* an invalid call is rejected */
    if (oracle_attn(y, k, v, cap, cap + 1, 3 * L, L, o, lse, B, H, D, n, 0.125, NULL, 0, 2) == 0)
        return 8;
    free(x), free(y), free(k), free(v), free(o), free(lse);
    puts("oracle driver: ok");
    return 0;
}
