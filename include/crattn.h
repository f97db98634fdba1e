/*
 * crattn.h -- C ABI of the chunk-causal Causal-RoPE attention library
 * (libcrattn.so, HIP for AMD CDNA4 / gfx950).
 *
 * The library implements the attention step of a chunk-causal autoregressive
 * video diffusion transformer (Self-Forcing style):
 *
 *   1. rope_precompute    -- cos/sin tables of the 3D rotary code, computed
 *                            once on the device.
 *   2. rope_apply_append  -- rotate the current chunk's Q and K with the 3D
 *                            rotary code from a global time index, write the
 *                            rotated Q, and append the rotated K and the V
 *                            to the KV cache, in one pass.
 *   3. chunk_causal_attn  -- flash attention of the chunk's queries against
 *                            the cache: bidirectional inside a chunk, causal
 *                            across chunks.
 *
 * Sources (web pages, by title and section):
 *   [CRSP] "Accelerating Video Generation Inference with Sequential-Parallel
 *          3D Positional Encoding Using a Global Time Index", technical
 *          summary: §1 (KV cache, rolling windows), §2.A (sequence
 *          parallelism: each rank holds a slice of the tokens), §2.B
 *          (Causal-RoPE SP: t_global = t + s; each rank rotates its own
 *          tokens from the start offset and its local index, no gather),
 *          §2.C (cos/sin precomputed into contiguous device tensors instead of
 *          dynamic caching; RoPE fused into one kernel).
 *   [WF]   "Wave Forcing" abstract: chunk-based causal attention over earlier
 *          chunks; the cache update is a separate forward pass.
 *   [SVG2] "Sparse VideoGen2" §2.A: attention output does not depend on the
 *          order of the key/value pairs (so a ring-buffer window is legal).
 *
 * Conventions shared by every entry point
 *   - All tensors are caller-owned device memory (any allocator).  The library
 *     allocates nothing, frees nothing, keeps no state between calls except a
 *     thread-local error message, and never synchronises: every call is
 *     enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *     stream).
 *   - Every argument is validated on the host before anything is launched; a
 *     call that returns non-zero has written nothing.  Faults inside a kernel
 *     (for example a pointer to too small a buffer) surface as a HIP error at
 *     the caller's next synchronisation.
 *   - Device pointers must be 16-byte aligned.
 *   - Token order inside a chunk is raster order: frame, then row, then
 *     column.  A chunk of F frames on a gh x gw grid has F*gh*gw tokens.
 *   - The rotary code splits head_dim D into three groups of adjacent feature
 *     pairs, in the order t, h, w: D_h = D_w = 2*floor(D/6), D_t = D - 2*D_h
 *     (44/42/42 at D = 128, 24/20/20 at D = 64).  Pair j of an axis group with
 *     D_a dims has frequency theta^(-2j/D_a); at position p it is rotated by
 *     the angle p * theta^(-2j/D_a):  x' = x cos - y sin,  y' = x sin + y cos.
 */
#ifndef CRATTN_H
#define CRATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define CRATTN_OK 0
#define CRATTN_EINVAL 1   /* invalid argument; nothing was launched            */
#define CRATTN_ENOTSUP 2  /* valid but unsupported (head_dim, dtype); nothing launched */
#define CRATTN_EHIP 3     /* the HIP runtime reported an error at launch        */

/* Element types of rope_apply_append's tensors. */
#define CRATTN_F32 0
#define CRATTN_BF16 1

/* Largest head_dim any entry point accepts. */
#define CRATTN_MAX_HEAD_DIM 256

/* Hierarchical block-sparse attention: key blocks of 64 tokens inside a
 * frame, query blocks of 256 rows of a call, at most 512 selected blocks
 * and 64 selected frames per query block, at most 4096 block candidates. */
#define CRATTN_HSA_KBLOCK 64
#define CRATTN_HSA_QBLOCK 256
#define CRATTN_HSA_MAX_KB 512
#define CRATTN_HSA_MAX_KF 64
#define CRATTN_HSA_MAX_CAND 4096

/* Semantic-permutation sparse attention: at most 256 clusters and 16384
 * tokens per k-means call, 64 Lloyd iterations, 1024 key-cluster candidates
 * per selection; query tiles of 256 rows. */
#define CRATTN_SVG2_MAX_C 256
#define CRATTN_SVG2_MAX_N 16384
#define CRATTN_SVG2_MAX_ITERS 64
#define CRATTN_SVG2_MAX_CAND 1024
#define CRATTN_SVG2_QTILE 256

/*
 * Size in bytes of the cos/sin table for head_dim D and position extents
 * (max_t, max_h, max_w): 8 * (max_t*D_t/2 + max_h*D_h/2 + max_w*D_w/2).
 * Returns 0 for invalid arguments (D not a positive even number, negative
 * extent).  Pure host function.
 */
size_t rope_table_bytes(int head_dim, int max_t, int max_h, int max_w);

/*
 * Build the cos/sin table on the device [CRSP §2.C].
 *
 *   table  device, rope_table_bytes(...) bytes, written.  Layout: float pairs
 *          (cos, sin); axis t entries first ([max_t][D_t/2]), then axis h
 *          ([max_h][D_h/2]), then axis w ([max_w][D_w/2]).  Entry (a, p, j)
 *          holds cos and sin of p * theta^(-2j/D_a), evaluated in double
 *          precision and rounded to float.
 *   max_t  temporal positions covered: global time indices 0 .. max_t-1.
 *          Positions past the model's training length are allowed.
 *   max_h, max_w  rows / columns covered.
 *   theta  frequency base (10000 for Wan2.1-class models); must be > 1.
 *
 * Errors: EINVAL for a NULL table, a misaligned table, D not even in
 * [2, CRATTN_MAX_HEAD_DIM], an extent < 1 or > 1<<20, theta <= 1; EHIP.
 */
int rope_precompute(float *table, int head_dim, int max_t, int max_h, int max_w,
                    double theta, void *stream);

/*
 * Rotate the chunk's Q and K and append K' and V to the KV cache, in one pass
 * [CRSP §2.B, §2.C; WF].
 *
 *   q, k, v   device, [B][n][H][D] of `dtype` (token-major, as a QKV projection
 *             emits them).  q may be NULL (a cache-update call: only K and V).
 *   q_out     device, [B][n][H][D] of `dtype`: the rotated Q.  May equal q
 *             (in place); must be NULL exactly when q is NULL.
 *   k_cache, v_cache  device, [B][H][cap][D] of `dtype` (head-major).  Rows
 *             cache_pos .. cache_pos+n-1 of every (b, h) are overwritten with
 *             the rotated K and the unrotated V; no other byte is touched.
 *   cap       rows per (b, h) in the cache; cache_pos + n <= cap.
 *   table     the rope_precompute table for (D, max_t, max_h, max_w).
 *   n         tokens in this call (>= 1).
 *   t0        global time index of the first frame of the chunk (the
 *             chunk's start-frame offset s of [CRSP §2.B]).
 *   tok_off   chunk-local raster index of the call's first token: 0 for a
 *             whole chunk, r*n for rank r's slice under sequence parallelism.
 *             Token i sits at g = tok_off + i; its positions are
 *             p_t = t0 + g / (grid_h*grid_w), p_h = (g mod grid_h*grid_w) / grid_w,
 *             p_w = g mod grid_w.  They are decoded from these scalars alone,
 *             so a slice rotates exactly as the same rows of the whole chunk.
 *   dtype     CRATTN_BF16 (fp32 arithmetic, round-to-nearest-even stores) or
 *             CRATTN_F32.  V is copied bit for bit.
 *
 * Errors: EINVAL for NULL k/v/caches/table, q and q_out not both NULL or both
 * set, a misaligned pointer, n < 1, B < 1, H < 1, D not a multiple of 8 in
 * [8, CRATTN_MAX_HEAD_DIM], cap < 1, cache_pos < 0, cache_pos + n > cap,
 * t0 < 0, tok_off < 0, grid_h < 1, grid_w < 1, a position outside the table
 * (t0 + last frame >= max_t, grid_h > max_h, grid_w > max_w), a frame of
 * grid_h * grid_w >= 2^31 tokens, an unknown dtype, or sizes whose element
 * counts overflow 2^40; EHIP.
 */
int rope_apply_append(const void *q, void *q_out, const void *k, const void *v,
                      void *k_cache, void *v_cache, int64_t cap, int64_t cache_pos,
                      const float *table, int max_t, int max_h, int max_w,
                      int B, int H, int D, int64_t n, int64_t t0, int64_t tok_off,
                      int grid_h, int grid_w, int dtype, void *stream);

/*
 * The QKV projection of the chunk with the rotary code and the cache append
 * fused into its epilogue [CRSP §2.C; §2.B; §1]: y = x W^T, then Q' = rot(Q),
 * K' = rot(K) appended with V to the cache, exactly as rope_apply_append does
 * with the projected Q, K, V (rotated in fp32 from the fp32 accumulators,
 * before any bf16 rounding).
 *
 *   x         device bf16 [B][n][C]: the chunk's hidden states.
 *   w         device bf16 [3*H*D][C] (linear-layer layout, out x in): rows
 *             [0, HD) project Q, [HD, 2HD) K, [2HD, 3HD) V, head h owning
 *             rows [h*D, (h+1)*D) of each part.  No bias.
 *   q_out     device bf16 [B][n][H][D] or NULL (a cache-update call: the Q
 *             rows of w are not computed).
 *   k_cache, v_cache, cap, cache_pos, table, max_t, max_h, max_w, n, t0,
 *   tok_off, grid_h, grid_w   as for rope_apply_append.
 *   C         hidden size: a multiple of 64, at most 65536.
 *
 * Arithmetic: bf16 products with fp32 accumulation (matrix cores), rotation in
 * fp32 with the table's fp32 cos/sin, round-to-nearest-even bf16 stores.
 *
 * Errors: EINVAL for NULL x/w/caches/table, a misaligned pointer, B, H, n or
 * C < 1, the cache-range, position and grid errors of rope_apply_append, B*n or
 * 3*H*D >= 2^31, or a cache over 2^40 elements; ENOTSUP for D other than 64
 * or 128, or C not a multiple of 64 or above 65536; EHIP.
 */
int qkv_rope_append(const void *x, const void *w, void *q_out, void *k_cache, void *v_cache,
                    int64_t cap, int64_t cache_pos, const float *table, int max_t, int max_h,
                    int max_w, int B, int H, int D, int C, int64_t n, int64_t t0,
                    int64_t tok_off, int grid_h, int grid_w, void *stream);

/*
 * Workspace bytes chunk_causal_attn needs to split the key range of a call
 * of this shape across workgroups (0 when it does not split).  Depends on the
 * shape only.  Pure host function; returns 0 for invalid shapes.
 */
size_t chunk_causal_attn_workspace_bytes(int B, int H, int64_t Lq, int64_t kv_len,
                                         int64_t q_pos0, int64_t chunk_tokens, int D);

/*
 * Chunk-causal flash attention [WF; CRSP §1].
 *
 *   q        device bf16 [B][Lq][H][D]: the rotated queries of this call.
 *   k_cache, v_cache  device bf16 [B][H][cap][D]: rotated keys and values.
 *            Only rows 0 .. kv_len-1 are ever read; rows past the visible
 *            range of a query may hold anything (NaN included) and do not
 *            affect it.
 *   kv_len   keys present (1 <= kv_len <= cap).
 *   q_pos0   global token index of query row 0 (row i sits at q_pos0 + i).
 *   chunk_tokens  tokens per chunk, L_c.  Key j is visible to row i iff
 *            j < kv_len and floor(j / L_c) <= floor((q_pos0 + i) / L_c):
 *            bidirectional inside the chunk, causal across chunks.  The whole
 *            chunk of the last query row must be present:
 *            kv_len >= (floor((q_pos0 + Lq - 1) / L_c) + 1) * L_c.
 *            A ring window of W chunk slots is addressed by passing
 *            kv_len = cap = W * L_c and q_pos0 = (W-1) * L_c (+ slice offset):
 *            every slot is then visible, which is correct because attention
 *            does not depend on key order [SVG2 §2.A].
 *   out      device bf16 [B][Lq][H][D]: softmax(scale * q k^T) v over the
 *            visible keys, rounded to nearest even.  Must not overlap q.
 *   lse      device float [B][H][Lq] or NULL: natural-log log-sum-exp of the
 *            scaled scores of each row.
 *   workspace, ws_bytes  device scratch of at least
 *            chunk_causal_attn_workspace_bytes(...) bytes, or NULL/0: the
 *            call then runs without splitting the key range (same result up
 *            to floating-point summation order, possibly slower).
 *   scale    score scale; 0 means 1/sqrt(D).
 *
 * Arithmetic: q.k products in bf16 with fp32 accumulation, softmax in fp32
 * (base-2 exponent with log2(e) folded into the scale), probabilities
 * rounded to bf16 for the P.V product, fp32 accumulation, one final division.
 *
 * Errors: EINVAL for NULL q/k_cache/v_cache/out, misaligned pointers, B, H or
 * Lq < 1, kv_len < 1 or > cap, q_pos0 < 0, chunk_tokens < 1, an incomplete
 * last chunk (see above), a non-finite or negative scale, cap * D >= 2^31
 * (the keys of one head are indexed in 32 bits), a workspace that is
 * non-NULL but too small; ENOTSUP for D other than 64 or 128; EHIP.
 */
int chunk_causal_attn(const void *q, const void *k_cache, const void *v_cache,
                      int64_t cap, int64_t kv_len, int64_t q_pos0, int64_t chunk_tokens,
                      void *out, float *lse, void *workspace, size_t ws_bytes,
                      int B, int H, int D, int64_t Lq, float scale, void *stream);

/*
 * chunk_causal_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation with the same arguments minus the
 * workspace.  When the call's shape splits the key range, the split partials
 * go to a scratch array the library holds on each device it runs on:
 * 32 MiB (CRATTN_NOALLOC_SCRATCH_BYTES), kept until the process ends, its
 * address looked up once per device.  The call allocates nothing.
 *
 * Every call on one device shares that device's scratch, which keeps the
 * last call's contents (nothing in it has to start at zero): calls that
 * overlap on one device (two streams, or two threads) race and must be
 * ordered by the caller.
 *
 * Errors: those of chunk_causal_attn, and EINVAL when the shape needs more
 * than CRATTN_NOALLOC_SCRATCH_BYTES of partials
 * (chunk_causal_attn_workspace_bytes of the same shape tells how much).
 */
#define CRATTN_NOALLOC_SCRATCH_BYTES (72u << 20)
int chunk_causal_attn_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              int64_t cap, int64_t kv_len, int64_t q_pos0, int64_t chunk_tokens,
                              void *out, float *lse, int B, int H, int D, int64_t Lq, float scale,
                              void *stream);

/*
 * Chunk-causal flash attention with the queries' Causal-RoPE applied on
 * load [CRSP §2.B-§2.C; WF]: the same computation as rope_apply_append
 * followed by chunk_causal_attn on the rotated queries, without writing Q'
 * to memory.
 *
 *   q        device bf16 [B][Lq][H][D]: the queries of this call, NOT
 *            rotated.  Row i is token (q_pos0 mod chunk_tokens) + i of its
 *            chunk, in raster order over grid_h x grid_w frames; its time
 *            index is t0 + that token's frame.  All Lq rows must lie in one
 *            chunk: (q_pos0 mod chunk_tokens) + Lq <= chunk_tokens.
 *   table, max_t, max_h, max_w  the cos/sin table of rope_precompute for
 *            head_dim D, and the extents it was built with.
 *   t0       global time index of the chunk's first frame.
 *   grid_h, grid_w  latent grid of one frame; chunk_tokens must be a whole
 *            number of frames.
 *   all other arguments as for chunk_causal_attn.
 *
 * Arithmetic: each query pair is rotated in fp32 and rounded to bf16 once,
 * exactly as rope_apply_append does, so the result equals that two-call
 * sequence bit for bit; the attention arithmetic is chunk_causal_attn's.
 *
 * Errors: those of chunk_causal_attn, and EINVAL for a NULL or misaligned
 * table, table extents outside [1, 2^20], t0 < 0, a grid below 1, beyond
 * the table or of grid_h * grid_w >= 2^31 tokens, chunk_tokens not a whole
 * number of frames, query rows that leave their chunk, or a time index
 * t0 + last frame >= max_t.
 */
int chunk_causal_attn_rope(const void *q, const float *table, int max_t, int max_h, int max_w,
                           int64_t t0, int grid_h, int grid_w, const void *k_cache,
                           const void *v_cache, int64_t cap, int64_t kv_len, int64_t q_pos0,
                           int64_t chunk_tokens, void *out, float *lse, void *workspace,
                           size_t ws_bytes, int B, int H, int D, int64_t Lq, float scale,
                           void *stream);

/*
 * Hierarchical block-sparse attention (HSA) ["LIGHT FORCING" §2.2]: queries
 * and keys are compressed by mean pooling at block and frame level; each
 * query block picks a few history frames with the frame-level keys, then
 * the best blocks inside those frames with the block-level keys; attention
 * runs over the query's own chunk plus the selected blocks, so its cost
 * stays constant as the history grows.
 *
 * Geometry.  The cache holds whole frames of per_frame tokens in raster
 * order (row r is in frame r / per_frame).  Key block j of frame f covers
 * rows f*per_frame + 64 j .. min(+64, (f+1)*per_frame); its global id is
 * f * nbf + j with nbf = ceil(per_frame / 64).  Query block i of a call is
 * rows 256 i .. min(256 i + 256, Lq).  The own chunk is chunk
 * c = q_pos0 / chunk_tokens (rows c*chunk_tokens .. (c+1)*chunk_tokens) and
 * is always attended in full.  History = every frame of the visible rows
 * [0, kv_len) outside the own chunk.  While a ring of chunk slots fills,
 * kv_len = (c+1)*chunk_tokens and the history is the chunks before the own
 * one; in a full ring, kv_len = cap and the own chunk is the current slot,
 * wherever it sits, so every other slot is history (attention does not
 * depend on key order ["Sparse VideoGen2" §2.A]).
 *
 * Pooled keys ("pool"): device float [B][H][nf][D] frame means followed by
 * [B][H][nf * nbf][D] block means, nf = cap / per_frame;
 * hsa_pool_bytes(...) bytes (0 for invalid arguments).
 */
size_t hsa_pool_bytes(int B, int H, int64_t cap, int D, int per_frame);

/*
 * Mean-pool the keys of cache rows [row0, row0 + nrows) (whole frames: both
 * multiples of per_frame) into the frame and block means of `pool`; call
 * once per chunk after its keys are appended.  Sums in fp32 in a fixed order.
 *
 * Errors: EINVAL for NULL or misaligned pointers, B, H, per_frame < 1,
 * cap not a whole number of frames, a row range that is not whole frames or
 * leaves [0, cap); ENOTSUP for D other than 64 or 128; EHIP.
 */
int hsa_pool_keys(const void *k_cache, int64_t cap, int64_t row0, int64_t nrows,
                  int per_frame, void *pool, int B, int H, int D, void *stream);

/*
 * Two-level selection for each (b, h, query block).
 *
 *   q        device bf16 [B][Lq][H][D]: the rotated queries of the call (all
 *            rows in one chunk: (q_pos0 mod chunk_tokens) + Lq <= chunk_tokens).
 *   pool     pooled keys of the history (hsa_pool_keys).
 *   kv_len   visible rows: whole frames, past the own chunk's end, <= cap.
 *   kf, kb   frames and blocks kept (1 <= kf <= 64, 1 <= kb <= 512; at most
 *            4096 history frames and 4096 block candidates:
 *            min(kf, history frames) * nbf).
 *   sel      device int32 [B][H][ceil(Lq/256)][kb]: the kept block ids in
 *            ascending order, then -1 for the places left when the kept
 *            frames hold fewer than kb blocks (all -1 with no history).
 *
 * Arithmetic: the query block's mean and the dot products with the pooled
 * keys in fp32; the k largest scores are kept, equal scores by the lower
 * frame / block id first.  A NaN score (from non-finite queries or keys)
 * ranks below every number; sel then still holds at most kb valid ids.
 *
 * Errors: EINVAL for NULL or misaligned pointers, B, H, Lq < 1, q_pos0 < 0,
 * chunk_tokens or per_frame < 1, chunk_tokens or cap not whole frames, query
 * rows that leave their chunk, kv_len not whole frames, above cap or before
 * the query chunk's end, kf or kb outside the limits, too many candidates;
 * ENOTSUP for D not 64 or 128; EHIP.
 */
int hsa_select(const void *q, const void *pool, int64_t cap, int64_t kv_len, int per_frame,
               int64_t q_pos0, int64_t chunk_tokens, int kf, int kb, int32_t *sel, int B, int H,
               int D, int64_t Lq, void *stream);

/*
 * Attention over the own chunk plus the selected blocks.
 *
 *   q, k_cache, v_cache, out, lse, scale  as for chunk_causal_attn (q
 *            rotated; all rows in one chunk).  The own chunk is rows
 *            [c*chunk_tokens, (c+1)*chunk_tokens) with c = q_pos0 / chunk_tokens.
 *   kv_len   visible rows, as for hsa_select.
 *   sel, kb  the selection (hsa_select's layout).  The ids of a row are used
 *            up to the end of the row; ids that are not history blocks
 *            (negative, in frames at or past kv_len, or in the own chunk) are
 *            skipped.  Each id should appear once: a repeated id attends its
 *            block's keys once per appearance (hsa_select never repeats one).
 *
 * Arithmetic: chunk_causal_attn's, over the visible rows in list order (own
 * chunk first).  Selecting every history block gives the dense result up to
 * summation order.
 *
 * Errors: those of chunk_causal_attn, and EINVAL for a NULL or misaligned
 * sel, kb outside [1, 512], per_frame < 1, chunk_tokens, cap or kv_len not
 * whole frames, query rows that leave their chunk.
 */
int hsa_attn(const void *q, const void *k_cache, const void *v_cache, int64_t cap, int64_t kv_len,
             int64_t q_pos0, int64_t chunk_tokens, int per_frame, const int32_t *sel, int kb,
             void *out, float *lse, int B, int H, int D, int64_t Lq, float scale, void *stream);

/*
 * Semantic-aware permutation with centroid top-p sparse attention
 * ["Sparse VideoGen2" §2.A-§2.C]: the queries and the keys of every head are
 * clustered by k-means, tokens are reordered so that each cluster is
 * contiguous, each query cluster keeps the key clusters of highest
 * estimated attention share (centroid scores) until their cumulative share
 * reaches p, and attention runs densely over the query tiles of a cluster,
 * loading the kept keys through a list of their rows.  The keys of a cache
 * are clustered chunk slot by chunk slot (a stored chunk's keys are
 * clustered once, when stored), the queries of a call as one set.
 *
 * Bytes of workspace svg2_kmeans needs (0 for invalid arguments).
 */
size_t svg2_kmeans_workspace_bytes(int B, int H, int n, int C);

/*
 * k-means (Lloyd) on the n tokens of every (b, h), then their stable
 * reordering by cluster.
 *
 *   x           device bf16; token t of (b, h) at x + b*stride_b + h*stride_h
 *               + t*stride_row elements (strides multiples of 8, x 16-byte
 *               aligned).  Q [B][Lq][H][D]: (Lq*H*D, D, H*D); one chunk slot
 *               of a cache [B][H][cap][D]: x = slot's first row, (H*cap*D,
 *               cap*D, D).
 *   C, iters    clusters (1..256) and Lloyd iterations (1..64).
 *   from_tokens 1: centroid c starts at token floor(c n / C); 0: the
 *               centroids already in `centroids` start (the previous step's).
 *   centroids   device float, head (b, h) at centroids + (b*H + h)*cent_stride:
 *               [C][D], in/out.  After the call: the means of the final
 *               assignment's clusters (an empty cluster keeps its centroid).
 *   perm        device int32, head at perm + (b*H + h)*perm_stride: [n], the
 *               token at each reordered position (clusters in id order, tokens
 *               ascending inside a cluster).
 *   offsets     device int32, head at offsets + (b*H + h)*off_stride: [C + 1],
 *               cluster c = positions offsets[c] .. offsets[c+1].
 *   workspace   device, svg2_kmeans_workspace_bytes(B, H, n, C) bytes.
 *
 * Arithmetic: the distance to centroid c is |c|^2 - 2 x.c in fp32 (the
 * nearest centroid, the lower index on a tie); means are fp32 sums in
 * reordered order divided by the count.
 *
 * Errors: EINVAL for NULL or misaligned pointers, B, H < 1, n outside
 * [1, 16384], C or iters outside their range, strides not multiples of 8 or
 * negative, output strides smaller than a head's extent (cent_stride >= C*D
 * and a multiple of 4, perm_stride >= n, off_stride >= C + 1), a short
 * workspace; ENOTSUP for D not 64 or 128; EHIP.
 */
int svg2_kmeans(const void *x, int64_t stride_b, int64_t stride_h, int64_t stride_row, int B,
                int H, int n, int D, int C, int iters, int from_tokens, float *centroids,
                int64_t cent_stride, int32_t *perm, int64_t perm_stride, int32_t *offsets,
                int64_t off_stride, void *workspace, size_t ws_bytes, void *stream);

/*
 * One k-means problem of svg2_kmeans2: the arguments of svg2_kmeans that
 * differ between the two problems, with the same meaning and limits.
 */
typedef struct svg2_kmeans_problem {
  const void *x;
  int64_t stride_b, stride_h, stride_row;
  int B, H, n, C;
  float *centroids;
  int64_t cent_stride;
  int32_t *perm;
  int64_t perm_stride;
  int32_t *offsets;
  int64_t off_stride;
  void *workspace;
  size_t ws_bytes;
} svg2_kmeans_problem;

/*
 * svg2_kmeans of two problems at once ("Sparse VideoGen2" §2.A: a denoising
 * call clusters its queries and the new keys), p[0] and p[1], with the same
 * D, iters and from_tokens: every kernel of the sequence is launched once
 * for both, so the two share no stream synchronisation.  Each result equals
 * that of svg2_kmeans on the problem alone, bit for bit.
 *
 *   p   host pointer to two problems (read during the call only).
 *
 * Errors: those of svg2_kmeans for either problem (the message names it);
 * EINVAL if p is NULL or if an output, or the workspace bytes it needs, of
 * one problem overlaps any range (x included) of the other.
 */
int svg2_kmeans2(const svg2_kmeans_problem *p, int D, int iters, int from_tokens, void *stream);

/* Query tiles of a call with Lq queries in Cq clusters: ceil(Lq / 256) + Cq
 * (an upper bound of sum over clusters of ceil(size / 256)); 0 if invalid. */
int svg2_n_slots(int64_t Lq, int Cq);

/*
 * Centroid top-p selection and the sparse attention's work lists.
 *
 *   q_cent, q_off  the queries' clusters (svg2_kmeans on Q, cent_stride
 *               Cq*D, off_stride Cq + 1): float [B][H][Cq][D], int32
 *               [B][H][Cq + 1].
 *   k_cent, k_off, k_perm  the keys' clusters of S chunk slots of L rows
 *               each: float [B][H][S][Ck][D], int32 [B][H][S][Ck + 1] and
 *               [B][H][S][L] (svg2_kmeans per slot).  Slots 0 .. n_vis-1 are
 *               visible; candidate j = slot j / Ck, cluster j mod Ck; its
 *               keys are cache rows slot*L + k_perm[..].
 *   p, scale    top-p threshold (0 < p; p >= 1 keeps every non-empty cluster)
 *               and the score scale (0: 1/sqrt(D)).
 *   sel         device int32 [B][H][Cq][n_vis*Ck]: kept candidates in
 *               ascending id order, then -1.
 *   lists       device int32 [B][H][Cq][list_cap]: the key rows of every query
 *               cluster, kept clusters in id order, each in its reordered
 *               order; list_len int32 [B][H][Cq] their counts (0 for an empty
 *               query cluster).  list_cap: a multiple of 64, at least n_vis*L.
 *   slots       device int32 [B][H][n_slots][4]: query tiles (first reordered
 *               position, rows <= 256, query cluster, 0), cluster by cluster;
 *               unused slots have 0 rows.  n_slots >= svg2_n_slots(Lq, Cq).
 *
 * Arithmetic: scores s_j = scale qc.kc_j in fp32; share w_j = n_j
 * exp(s_j - max s) (0 for an empty cluster); candidates ranked by decreasing
 * share (lower id first on a tie); a candidate is kept while the shares
 * ranked before it add up to less than p times the total (fp32, fixed
 * order).
 *
 * Errors: EINVAL for NULL or misaligned pointers, B, H, Lq < 1, Cq or Ck
 * outside [1, 256], n_vis outside [1, S], more than 1024 candidates, L
 * outside [1, 16384], p not positive, scale negative or not finite, list_cap
 * or n_slots too small; ENOTSUP for D not 64 or 128; EHIP.
 */
int svg2_plan(const float *q_cent, const int32_t *q_off, const float *k_cent,
              const int32_t *k_off, const int32_t *k_perm, int B, int H, int D, int Cq, int Ck,
              int S, int n_vis, int64_t L, int64_t Lq, float p, float scale, int32_t *sel,
              int32_t *lists, int64_t list_cap, int32_t *list_len, int32_t *slots, int n_slots,
              void *stream);

/* Workspace bytes of svg2_attn with n_slots query tiles per head and
 * `splits` key-range splits: 256 (the work counter of its persistent
 * launch), the work order (a 16-byte record per slot, rounded up to 256)
 * and the split partials; 0 for invalid arguments. */
size_t svg2_attn_workspace_bytes(int B, int H, int64_t Lq, int D, int n_slots, int splits);

/*
 * Attention of every query tile over its cluster's key list.
 *
 *   q           device bf16 [B][Lq][H][D] (rotated); out the same layout.
 *   k_cache, v_cache  device bf16 [B][H][cap][D].
 *   q_perm      device int32 [B][H][Lq]: the query row of each reordered
 *               position (svg2_kmeans perm of Q).
 *   slots, n_slots, lists, list_cap, list_len, Cq  svg2_plan's outputs.
 *   splits      key-range splits per query tile (1..16); with splits > 1 the
 *               partial results are merged by log-sum-exp.
 *   workspace   device, svg2_attn_workspace_bytes(B, H, Lq, D, n_slots, splits)
 *               bytes, 16-byte aligned (a work counter, the work order, the
 *               partials).  Calls that overlap on one workspace race.
 *
 * Launch: one workgroup per compute unit takes the non-empty query tiles,
 * longest key list first, from a counter in the workspace (reset by the
 * call) until none are left.  A slot with rows outside [1, 256] or past Lq,
 * or a cluster outside [0, Cq), is skipped (its rows are not written).
 *   lse         NULL or device float [B][H][Lq] (natural log).
 *
 * Arithmetic: chunk_causal_attn's (bf16 products, fp32 online softmax) over
 * the listed keys in list order.  Key rows past cap - 1 and query rows past
 * Lq - 1 are clamped, so no access leaves the buffers; a query row in no
 * tile is not written.
 *
 * Errors: EINVAL for NULL or misaligned pointers, B, H, Lq, cap, n_slots < 1,
 * Cq outside [1, 256], list_cap not a positive multiple of 64, splits outside
 * [1, 16], a missing or short workspace, cap * D >= 2^31; ENOTSUP for D not
 * 64 or 128; EHIP.
 */
int svg2_attn(const void *q, const void *k_cache, const void *v_cache, int64_t cap,
              const int32_t *q_perm, const int32_t *slots, int n_slots, const int32_t *lists,
              int64_t list_cap, const int32_t *list_len, int Cq, int splits, void *out,
              float *lse, void *workspace, size_t ws_bytes, int B, int H, int D, int64_t Lq,
              float scale, void *stream);

/* Message describing the last non-zero return on this thread ("" if none). */
const char *crattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CRATTN_H */
