/*
 * oracle.c -- plain, slow, fp64 CPU reference for the Causal-RoPE
 * chunk-causal attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header or table with the HIP library.
 *
 * Sources (web pages, cited by title and section):
 *  [CRSP]  "Accelerating Video Generation Inference with Sequential-Parallel
 *          3D Positional Encoding Using a Global Time Index" (technical
 *          summary): §1 Het Probleem (KV cache, rolling windows), §2.B
 *          Causal-RoPE SP (global time index t_global = t + s, local rotation
 *          without a gather), §2.C (cos/sin precomputed into contiguous
 *          tensors).
 *  [WF]    "Wave Forcing" abstract: chunk-causal attention over earlier
 *          chunks; the cache update is a second forward pass.
 *  [SVG2]  "Sparse VideoGen2", §2.A: attention is invariant under a
 *          permutation of the key/value pairs.
 *
 * The pages print no RoPE formula.  The definition below is the standard
 * rotary code applied per axis, with the readings stated beside each
 * function.  Everything is computed in double precision with plain loops:
 * no SIMD, no BLAS, no fast-math, no blocking and no online softmax.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <pthread.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_EEMPTY 2

/* ---------------------------------------------------------------------- */
/* head_dim split into (t, h, w) groups.                                   */
/* Reading: h and w each get 2*floor(D/6) dims, t gets the rest, in the     */
/* order t, h, w (24/20/20 at D = 64, 44/42/42 at D = 128).                 */
/* ---------------------------------------------------------------------- */
int oracle_split(int D, int *Dt, int *Dh, int *Dw)
{
    if (D <= 0 || (D % 2) != 0)
        return ORACLE_EINVAL;
    int dhw = 2 * (D / 6);
    *Dh = dhw;
    *Dw = dhw;
    *Dt = D - 2 * dhw;
    return ORACLE_OK;
}

/* Frequency of pair j on an axis with Da dims: theta^(-2j/Da).            */
/* Reading: each axis is its own 1-D rotary code over its own Da dims.      */
static double axis_freq(double theta, int j, int Da)
{
    return pow(theta, -2.0 * (double)j / (double)Da);
}

/* ---------------------------------------------------------------------- */
/* cos/sin table [CRSP §2.C]: for axis a in (t, h, w), position p < max_a   */
/* and pair j < Da/2, angle p * freq(j).  Output order: axis t entries      */
/* (p-major, then j), then axis h, then axis w; cos and sin in two arrays.  */
/* Entry count = sum_a max_a * Da / 2.                                       */
/* ---------------------------------------------------------------------- */
int oracle_rope_table(double *cos_out, double *sin_out, int D, int max_t,
                      int max_h, int max_w, double theta)
{
    int dims[3];
    if (oracle_split(D, &dims[0], &dims[1], &dims[2]) != ORACLE_OK)
        return ORACLE_EINVAL;
    if (max_t < 0 || max_h < 0 || max_w < 0 || !(theta > 0.0))
        return ORACLE_EINVAL;
    int maxes[3] = {max_t, max_h, max_w};
    int64_t e = 0;
    for (int a = 0; a < 3; ++a) {
        for (int p = 0; p < maxes[a]; ++p) {
            for (int j = 0; j < dims[a] / 2; ++j) {
                double phi = (double)p * axis_freq(theta, j, dims[a]);
                cos_out[e] = cos(phi);
                sin_out[e] = sin(phi);
                ++e;
            }
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* Position decode with the global time index [CRSP §2.B].                  */
/* Token i of the call has chunk-local raster index g = tok_off + i        */
/* (frame-major, then row, then column).  Its frame is f = g / (gh*gw); its */
/* temporal position is t0 + f (t_global = t + s with s = t0); its spatial  */
/* positions are the row and column inside the frame.                       */
/* pos is [n][3] = (p_t, p_h, p_w).                                          */
/* ---------------------------------------------------------------------- */
int oracle_positions(int64_t n, int64_t t0, int64_t tok_off, int64_t gh,
                     int64_t gw, int64_t *pos)
{
    if (n < 0 || gh <= 0 || gw <= 0 || tok_off < 0)
        return ORACLE_EINVAL;
    int64_t per_frame = gh * gw;
    for (int64_t i = 0; i < n; ++i) {
        int64_t g = tok_off + i;
        int64_t f = g / per_frame;
        int64_t in_frame = g - f * per_frame;
        pos[3 * i + 0] = t0 + f;
        pos[3 * i + 1] = in_frame / gw;
        pos[3 * i + 2] = in_frame % gw;
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* Rotation from explicit positions.  x, y: [B][n][H][D].  pos: [n][3].      */
/* Pair j of axis a occupies dims (o_a + 2j, o_a + 2j + 1) (reading: adjacent */
/* pairs); it is rotated by phi = p_a * freq(j):                              */
/*     x' = x cos(phi) - y sin(phi),   y' = x sin(phi) + y cos(phi).          */
/* y may alias x.                                                            */
/* ---------------------------------------------------------------------- */
int oracle_rope_pos(const double *x, double *y, int B, int64_t n, int H, int D,
                    const int64_t *pos, double theta)
{
    int dims[3];
    if (oracle_split(D, &dims[0], &dims[1], &dims[2]) != ORACLE_OK)
        return ORACLE_EINVAL;
    if (B < 0 || n < 0 || H < 0 || !(theta > 0.0))
        return ORACLE_EINVAL;
    int offs[3] = {0, dims[0], dims[0] + dims[1]};
    for (int b = 0; b < B; ++b) {
        for (int64_t i = 0; i < n; ++i) {
            for (int h = 0; h < H; ++h) {
                int64_t row = (((int64_t)b * n + i) * H + h) * D;
                for (int a = 0; a < 3; ++a) {
                    double p = (double)pos[3 * i + a];
                    for (int j = 0; j < dims[a] / 2; ++j) {
                        double phi = p * axis_freq(theta, j, dims[a]);
                        double c = cos(phi), s = sin(phi);
                        int64_t d0 = row + offs[a] + 2 * j;
                        double u = x[d0], v = x[d0 + 1];
                        y[d0] = u * c - v * s;
                        y[d0 + 1] = u * s + v * c;
                    }
                }
            }
        }
    }
    return ORACLE_OK;
}

/* Rotation of n tokens of a chunk that starts at frame t0, the first token */
/* being chunk-local raster index tok_off [CRSP §2.B: each rank rotates its  */
/* own tokens from the start offset and its local index, with no gather].   */
int oracle_rope(const double *x, double *y, int B, int64_t n, int H, int D,
                int64_t t0, int64_t tok_off, int64_t gh, int64_t gw,
                double theta)
{
    int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * 3 * (size_t)(n > 0 ? n : 1));
    if (!pos)
        return ORACLE_EINVAL;
    int st = oracle_positions(n, t0, tok_off, gh, gw, pos);
    if (st == ORACLE_OK)
        st = oracle_rope_pos(x, y, B, n, H, D, pos, theta);
    free(pos);
    return st;
}

/* ---------------------------------------------------------------------- */
/* KV-cache append [CRSP §1: KV cache; WF: cache update pass].               */
/* cache[b][h][cache_pos + i][:] = x[b][i][h][:].  Cache is [B][H][cap][D].   */
/* ---------------------------------------------------------------------- */
int oracle_append(const double *x, double *cache, int B, int64_t n, int H,
                  int D, int64_t cap, int64_t cache_pos)
{
    if (cache_pos < 0 || n < 0 || cache_pos + n > cap)
        return ORACLE_EINVAL;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int64_t i = 0; i < n; ++i)
                for (int d = 0; d < D; ++d)
                    cache[(((int64_t)b * H + h) * cap + cache_pos + i) * D + d] =
                        x[(((int64_t)b * n + i) * H + h) * D + d];
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* Chunk-causal attention, textbook two-pass softmax.                        */
/*                                                                           */
/* q:   [B][Lq][H][D]           query row i has global token index q_pos0+i  */
/* k,v: [B][H][cap][D]          keys 0 .. kv_len-1 exist                     */
/* Key j is visible to row i iff j < kv_len and                              */
/*     floor(j / chunk_tokens) <= floor((q_pos0 + i) / chunk_tokens)         */
/* (bidirectional inside a chunk, causal across chunks [WF abstract]).       */
/*                                                                           */
/* For each (b, h, i):  s_j = scale * sum_d q_d k_jd over visible j;         */
/* m = max s_j;  l = sum exp(s_j - m);  o = sum exp(s_j - m) v_j / l;        */
/* lse = m + ln l.                                                           */
/*                                                                           */
/* rows: optional list of nrows query-row indices; when given, o is          */
/* [B][nrows][H][D] and lse is [B][H][nrows].  When rows is NULL, all Lq     */
/* rows are computed (nrows is ignored).  lse may be NULL.                    */
/* Work is split over nthreads threads by (b, h, row); each row is computed  */
/* by one thread in a fixed order, so results do not depend on nthreads.    */
/* ---------------------------------------------------------------------- */
typedef struct {
    const double *q, *k, *v;
    double *o, *lse;
    int64_t cap, kv_len, q_pos0, chunk_tokens;
    int B, H, D;
    int64_t Lq, nrows;
    const int64_t *rows;
    double scale;
    int64_t items;
    int64_t next; /* work counter, taken atomically */
    int status;
} attn_job;

static void attn_row(attn_job *J, int64_t item, double *s)
{
    int64_t nr = J->nrows;
    int b = (int)(item / ((int64_t)J->H * nr));
    int h = (int)((item / nr) % J->H);
    int64_t r = item % nr;
    int64_t i = J->rows ? J->rows[r] : r;
    int D = J->D;
    const double *qrow = J->q + (((int64_t)b * J->Lq + i) * J->H + h) * D;
    const double *kh = J->k + ((int64_t)b * J->H + h) * J->cap * D;
    const double *vh = J->v + ((int64_t)b * J->H + h) * J->cap * D;
    double *orow = J->o + (((int64_t)b * nr + r) * J->H + h) * D;
    int64_t q_chunk = (J->q_pos0 + i) / J->chunk_tokens;

    /* pass 1: scores of the visible keys and their maximum */
    int any = 0;
    double m = -INFINITY;
    for (int64_t j = 0; j < J->kv_len; ++j) {
        if (j / J->chunk_tokens > q_chunk)
            continue;
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += qrow[d] * kh[j * D + d];
        s[j] = J->scale * acc;
        if (!any || s[j] > m)
            m = s[j];
        any = 1;
    }
    if (!any) {
        __atomic_store_n(&J->status, ORACLE_EEMPTY, __ATOMIC_RELAXED);
        for (int d = 0; d < D; ++d)
            orow[d] = NAN;
        if (J->lse)
            J->lse[((int64_t)b * J->H + h) * nr + r] = NAN;
        return;
    }
    /* pass 2: normaliser and weighted sum of values */
    double l = 0.0;
    for (int d = 0; d < D; ++d)
        orow[d] = 0.0;
    for (int64_t j = 0; j < J->kv_len; ++j) {
        if (j / J->chunk_tokens > q_chunk)
            continue;
        double p = exp(s[j] - m);
        l += p;
        for (int d = 0; d < D; ++d)
            orow[d] += p * vh[j * D + d];
    }
    for (int d = 0; d < D; ++d)
        orow[d] /= l;
    if (J->lse)
        J->lse[((int64_t)b * J->H + h) * nr + r] = m + log(l);
}

static void *attn_worker(void *arg)
{
    attn_job *J = (attn_job *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)(J->kv_len > 0 ? J->kv_len : 1));
    if (!s) {
        __atomic_store_n(&J->status, ORACLE_EINVAL, __ATOMIC_RELAXED);
        return NULL;
    }
    for (;;) {
        int64_t item = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (item >= J->items)
            break;
        attn_row(J, item, s);
    }
    free(s);
    return NULL;
}

int oracle_attn(const double *q, const double *k, const double *v, int64_t cap,
                int64_t kv_len, int64_t q_pos0, int64_t chunk_tokens,
                double *o, double *lse, int B, int H, int D, int64_t Lq,
                double scale, const int64_t *rows, int64_t nrows, int nthreads)
{
    if (B < 0 || H < 0 || D <= 0 || Lq < 0 || kv_len < 0 || kv_len > cap ||
        chunk_tokens <= 0 || q_pos0 < 0)
        return ORACLE_EINVAL;
    attn_job J;
    J.q = q; J.k = k; J.v = v; J.o = o; J.lse = lse;
    J.cap = cap; J.kv_len = kv_len; J.q_pos0 = q_pos0;
    J.chunk_tokens = chunk_tokens;
    J.B = B; J.H = H; J.D = D; J.Lq = Lq;
    J.rows = rows;
    J.nrows = rows ? nrows : Lq;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= Lq)
                return ORACLE_EINVAL;
    J.scale = scale;
    J.items = (int64_t)B * H * J.nrows;
    J.next = 0;
    J.status = ORACLE_OK;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t tid[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[started], NULL, attn_worker, &J) != 0)
            break;
        ++started;
    }
    attn_worker(&J);
    for (int t = 0; t < started; ++t)
        pthread_join(tid[t], NULL);
    return J.status;
}
