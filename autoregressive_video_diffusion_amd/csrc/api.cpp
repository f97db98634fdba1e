// C-ABI front end of libcrattn.so: argument validation, launch planning and
// error reporting.  The entry points and their contracts are declared and
// documented in include/crattn.h.  Every check runs on the host before any
// HIP call, so an invalid call launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/crattn.h"
#include "crattn_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return CRATTN_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(CRATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int64_t kMaxElems = int64_t(1) << 40;
static_assert(crattn::kAttnScratchBytes == CRATTN_NOALLOC_SCRATCH_BYTES, "scratch size");
constexpr int kMaxExtent = 1 << 20;

}  // namespace

extern "C" {

size_t rope_table_bytes(int head_dim, int max_t, int max_h, int max_w) {
  if (head_dim < 2 || head_dim > CRATTN_MAX_HEAD_DIM || (head_dim % 2) != 0) return 0;
  if (max_t < 0 || max_h < 0 || max_w < 0) return 0;
  if (max_t > kMaxExtent || max_h > kMaxExtent || max_w > kMaxExtent) return 0;
  const crattn::RopeSplit sp = crattn::rope_split(head_dim);
  return 8u * ((size_t)max_t * (sp.dt / 2) + (size_t)max_h * (sp.dh / 2) +
               (size_t)max_w * (sp.dw / 2));
}

int rope_precompute(float *table, int head_dim, int max_t, int max_h, int max_w, double theta,
                    void *stream) {
  if (table == nullptr) return fail(CRATTN_EINVAL, "rope_precompute: table is NULL");
  if (!aligned16(table)) return fail(CRATTN_EINVAL, "rope_precompute: table not 16-byte aligned");
  if (head_dim < 2 || head_dim > CRATTN_MAX_HEAD_DIM || (head_dim % 2) != 0)
    return fail(CRATTN_EINVAL, "rope_precompute: head_dim %d not even in [2, %d]", head_dim,
                CRATTN_MAX_HEAD_DIM);
  if (max_t < 1 || max_h < 1 || max_w < 1 || max_t > kMaxExtent || max_h > kMaxExtent ||
      max_w > kMaxExtent)
    return fail(CRATTN_EINVAL, "rope_precompute: extents (%d, %d, %d) outside [1, %d]", max_t,
                max_h, max_w, kMaxExtent);
  if (!(theta > 1.0) || !isfinite(theta))
    return fail(CRATTN_EINVAL, "rope_precompute: theta must be finite and > 1");
  const crattn::RopeSplit sp = crattn::rope_split(head_dim);
  crattn::RopeTableArgs a;
  a.table = reinterpret_cast<float2 *>(table);
  a.dt = sp.dt;
  a.dh = sp.dh;
  a.dw = sp.dw;
  a.max_t = max_t;
  a.max_h = max_h;
  a.max_w = max_w;
  a.theta = theta;
  return hip_status(crattn::launch_rope_table(a, static_cast<hipStream_t>(stream)),
                    "rope_precompute launch");
}

int rope_apply_append(const void *q, void *q_out, const void *k, const void *v, void *k_cache,
                      void *v_cache, int64_t cap, int64_t cache_pos, const float *table,
                      int max_t, int max_h, int max_w, int B, int H, int D, int64_t n, int64_t t0,
                      int64_t tok_off, int grid_h, int grid_w, int dtype, void *stream) {
  if (k == nullptr || v == nullptr || k_cache == nullptr || v_cache == nullptr ||
      table == nullptr)
    return fail(CRATTN_EINVAL, "rope_apply_append: k, v, k_cache, v_cache and table are required");
  if ((q == nullptr) != (q_out == nullptr))
    return fail(CRATTN_EINVAL, "rope_apply_append: q and q_out must both be set or both be NULL");
  if (!aligned16(q) || !aligned16(q_out) || !aligned16(k) || !aligned16(v) ||
      !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(table))
    return fail(CRATTN_EINVAL, "rope_apply_append: pointers must be 16-byte aligned");
  if (dtype != CRATTN_BF16 && dtype != CRATTN_F32)
    return fail(CRATTN_EINVAL, "rope_apply_append: unknown dtype %d", dtype);
  if (D < 8 || D > CRATTN_MAX_HEAD_DIM || (D % 8) != 0)
    return fail(CRATTN_EINVAL, "rope_apply_append: head_dim %d not a multiple of 8 in [8, %d]", D,
                CRATTN_MAX_HEAD_DIM);
  if (B < 1 || H < 1 || n < 1)
    return fail(CRATTN_EINVAL, "rope_apply_append: B=%d H=%d n=%lld must be >= 1", B, H,
                (long long)n);
  if (cap < 1 || cache_pos < 0 || cache_pos > cap || n > cap - cache_pos)
    return fail(CRATTN_EINVAL, "rope_apply_append: %lld rows from row %lld leave the cache (cap %lld)",
                (long long)n, (long long)cache_pos, (long long)cap);
  if (t0 < 0 || tok_off < 0 || grid_h < 1 || grid_w < 1)
    return fail(CRATTN_EINVAL, "rope_apply_append: t0, tok_off >= 0 and grid >= 1 required");
  if (max_t < 1 || max_h < 1 || max_w < 1 || max_t > kMaxExtent || max_h > kMaxExtent ||
      max_w > kMaxExtent)
    return fail(CRATTN_EINVAL, "rope_apply_append: table extents outside [1, %d]", kMaxExtent);
  if (grid_h > max_h || grid_w > max_w)
    return fail(CRATTN_EINVAL, "rope_apply_append: grid %dx%d exceeds the table (%dx%d)", grid_h,
                grid_w, max_h, max_w);
  // the kernels decode positions with a 32-bit frame size
  if ((int64_t)grid_h * grid_w >= (int64_t(1) << 31))
    return fail(CRATTN_EINVAL, "rope_apply_append: grid_h * grid_w must be below 2^31");
  const int64_t per_frame = (int64_t)grid_h * grid_w;
  if (tok_off > kMaxElems || n > kMaxElems)
    return fail(CRATTN_EINVAL, "rope_apply_append: token range too large");
  const int64_t last_t = t0 + (tok_off + n - 1) / per_frame;
  if (last_t >= max_t)
    return fail(CRATTN_EINVAL,
                "rope_apply_append: time index %lld outside the table (max_t %d)",
                (long long)last_t, max_t);
  if (tok_off + n > (int64_t(1) << 31))
    return fail(CRATTN_EINVAL, "rope_apply_append: token index exceeds 2^31");
  const int esize = dtype == CRATTN_BF16 ? 2 : 4;
  const int64_t vec_per_row = (int64_t)D * esize / 16;
  const double threads = (double)B * (double)n * (double)H * (double)vec_per_row;
  if (threads >= 2147483648.0)
    return fail(CRATTN_EINVAL, "rope_apply_append: B*n*H*D too large for one launch");
  if ((double)B * H * (double)cap * D > (double)kMaxElems)
    return fail(CRATTN_EINVAL, "rope_apply_append: cache element count exceeds 2^40");
  crattn::RopeAppendArgs a;
  a.q = q;
  a.q_out = q_out;
  a.k = k;
  a.v = v;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cap = cap;
  a.cache_pos = cache_pos;
  a.table = reinterpret_cast<const float2 *>(table);
  a.max_t = max_t;
  a.max_h = max_h;
  a.max_w = max_w;
  a.B = B;
  a.H = H;
  a.D = D;
  a.n = n;
  a.t0 = t0;
  a.tok_off = tok_off;
  a.grid_h = grid_h;
  a.grid_w = grid_w;
  a.dtype = dtype;
  return hip_status(crattn::launch_rope_append(a, static_cast<hipStream_t>(stream)),
                    "rope_apply_append launch");
}

int qkv_rope_append(const void *x, const void *w, void *q_out, void *k_cache, void *v_cache,
                    int64_t cap, int64_t cache_pos, const float *table, int max_t, int max_h,
                    int max_w, int B, int H, int D, int C, int64_t n, int64_t t0, int64_t tok_off,
                    int grid_h, int grid_w, void *stream) {
  if (x == nullptr || w == nullptr || k_cache == nullptr || v_cache == nullptr ||
      table == nullptr)
    return fail(CRATTN_EINVAL, "qkv_rope_append: x, w, k_cache, v_cache and table are required");
  if (!aligned16(x) || !aligned16(w) || !aligned16(q_out) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(table))
    return fail(CRATTN_EINVAL, "qkv_rope_append: pointers must be 16-byte aligned");
  if (B < 1 || H < 1 || n < 1 || C < 1)
    return fail(CRATTN_EINVAL, "qkv_rope_append: B=%d H=%d n=%lld C=%d must be >= 1", B, H,
                (long long)n, C);
  if (D != 64 && D != 128)
    return fail(CRATTN_ENOTSUP, "qkv_rope_append: head_dim %d not supported (64 or 128)", D);
  if (C % 64 != 0 || C > 65536)
    return fail(CRATTN_ENOTSUP, "qkv_rope_append: C=%d must be a multiple of 64, at most 65536",
                C);
  if (cap < 1 || cache_pos < 0 || cache_pos > cap || n > cap - cache_pos)
    return fail(CRATTN_EINVAL, "qkv_rope_append: %lld rows from row %lld leave the cache (cap %lld)",
                (long long)n, (long long)cache_pos, (long long)cap);
  if (t0 < 0 || tok_off < 0 || grid_h < 1 || grid_w < 1)
    return fail(CRATTN_EINVAL, "qkv_rope_append: t0, tok_off >= 0 and grid >= 1 required");
  if (max_t < 1 || max_h < 1 || max_w < 1 || max_t > kMaxExtent || max_h > kMaxExtent ||
      max_w > kMaxExtent)
    return fail(CRATTN_EINVAL, "qkv_rope_append: table extents outside [1, %d]", kMaxExtent);
  if (grid_h > max_h || grid_w > max_w)
    return fail(CRATTN_EINVAL, "qkv_rope_append: grid %dx%d exceeds the table (%dx%d)", grid_h,
                grid_w, max_h, max_w);
  // the kernels decode positions with a 32-bit frame size
  if ((int64_t)grid_h * grid_w >= (int64_t(1) << 31))
    return fail(CRATTN_EINVAL, "qkv_rope_append: grid_h * grid_w must be below 2^31");
  if (tok_off > kMaxElems || n > kMaxElems)
    return fail(CRATTN_EINVAL, "qkv_rope_append: token range too large");
  const int64_t last_t = t0 + (tok_off + n - 1) / ((int64_t)grid_h * grid_w);
  if (last_t >= max_t)
    return fail(CRATTN_EINVAL, "qkv_rope_append: time index %lld outside the table (max_t %d)",
                (long long)last_t, max_t);
  if (tok_off + n > (int64_t(1) << 31) || (double)B * (double)n >= 2147483648.0 ||
      3.0 * H * D >= 2147483648.0)
    return fail(CRATTN_EINVAL, "qkv_rope_append: B*n, tok_off + n or 3*H*D exceeds 2^31");
  if ((double)B * H * (double)cap * D > (double)kMaxElems)
    return fail(CRATTN_EINVAL, "qkv_rope_append: cache element count exceeds 2^40");
  crattn::QkvArgs a;
  a.x = x;
  a.w = w;
  a.q_out = q_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cap = cap;
  a.cache_pos = cache_pos;
  a.table = table;
  a.max_t = max_t;
  a.max_h = max_h;
  a.max_w = max_w;
  a.B = B;
  a.H = H;
  a.D = D;
  a.C = C;
  a.n = n;
  a.t0 = t0;
  a.tok_off = tok_off;
  a.grid_h = grid_h;
  a.grid_w = grid_w;
  return hip_status(crattn::launch_qkv_rope(a, static_cast<hipStream_t>(stream)),
                    "qkv_rope_append launch");
}

static int attn_shape_check(int B, int H, int64_t Lq, int64_t kv_len, int64_t q_pos0,
                            int64_t chunk_tokens, int D, int64_t cap, const char *who) {
  if (B < 1 || H < 1 || Lq < 1)
    return fail(CRATTN_EINVAL, "%s: B=%d H=%d Lq=%lld must be >= 1", who, B, H, (long long)Lq);
  if (chunk_tokens < 1 || q_pos0 < 0)
    return fail(CRATTN_EINVAL, "%s: chunk_tokens >= 1 and q_pos0 >= 0 required", who);
  if (kv_len < 1 || (cap >= 0 && kv_len > cap))
    return fail(CRATTN_EINVAL, "%s: kv_len %lld outside [1, cap=%lld]", who, (long long)kv_len,
                (long long)cap);
  if (Lq > kMaxElems || q_pos0 > kMaxElems || kv_len > kMaxElems || chunk_tokens > kMaxElems)
    return fail(CRATTN_EINVAL, "%s: sizes exceed 2^40", who);
  const int64_t last_chunk = (q_pos0 + Lq - 1) / chunk_tokens;
  if (kv_len < (last_chunk + 1) * chunk_tokens)
    return fail(CRATTN_EINVAL,
                "%s: kv_len %lld leaves the chunk of the last query incomplete (needs %lld)", who,
                (long long)kv_len, (long long)((last_chunk + 1) * chunk_tokens));
  if (D != 64 && D != 128)
    return fail(CRATTN_ENOTSUP, "%s: head_dim %d not supported (64 or 128)", who, D);
  if ((double)B * H * (double)Lq * (D / 4) >= 4294967296.0)
    return fail(CRATTN_EINVAL, "%s: B*H*Lq*D too large for one launch", who);
  return CRATTN_OK;
}

size_t chunk_causal_attn_workspace_bytes(int B, int H, int64_t Lq, int64_t kv_len,
                                         int64_t q_pos0, int64_t chunk_tokens, int D) {
  if (attn_shape_check(B, H, Lq, kv_len, q_pos0, chunk_tokens, D, -1, "workspace") != CRATTN_OK)
    return 0;
  return crattn::attn_plan(B, H, Lq, kv_len, q_pos0, chunk_tokens, D, true).ws_bytes;
}

}  // extern "C"

namespace {

// Table and chunk geometry for rotating the queries on load.
struct QRope {
  const float *table;
  int max_t, max_h, max_w;
  int64_t t0;
  int grid_h, grid_w;
};

// Selected key blocks for the block-sparse instance.
struct Sparse {
  const int32_t *sel;
  int kb, per_frame;
};

int attn_call(const char *who, const QRope *rq, const Sparse *sp, const void *q,
              const void *k_cache,
              const void *v_cache, int64_t cap, int64_t kv_len, int64_t q_pos0,
              int64_t chunk_tokens, void *out, float *lse, void *workspace, size_t ws_bytes, int B,
              int H, int D, int64_t Lq, float scale, void *stream) {
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || out == nullptr)
    return fail(CRATTN_EINVAL, "%s: q, k_cache, v_cache and out are required", who);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(lse) || !aligned16(workspace))
    return fail(CRATTN_EINVAL, "%s: pointers must be 16-byte aligned", who);
  if (cap < 1) return fail(CRATTN_EINVAL, "%s: cap must be >= 1", who);
  const int st = attn_shape_check(B, H, Lq, kv_len, q_pos0, chunk_tokens, D, cap, who);
  if (st != CRATTN_OK) return st;
  if (!(scale >= 0.f) || !isfinite(scale))
    return fail(CRATTN_EINVAL, "%s: scale must be finite and >= 0", who);
  if ((double)B * H * (double)cap * D > (double)kMaxElems)
    return fail(CRATTN_EINVAL, "%s: cache element count exceeds 2^40", who);
  // the kernel indexes the keys of one head (cap rows of D elements) in 32 bits
  if ((double)cap * D >= 2147483648.0)
    return fail(CRATTN_EINVAL, "%s: cap * head_dim = %.0f must be below 2^31", who,
                (double)cap * D);
  crattn::AttnArgs a{};
  a.rope = rq != nullptr;
  if (sp != nullptr) {
    if (sp->sel == nullptr || !aligned16(sp->sel))
      return fail(CRATTN_EINVAL, "%s: sel is required, 16-byte aligned", who);
    if (sp->kb < 1 || sp->kb > CRATTN_HSA_MAX_KB)
      return fail(CRATTN_EINVAL, "%s: kb %d outside [1, %d]", who, sp->kb, CRATTN_HSA_MAX_KB);
    if (sp->per_frame < 1 || chunk_tokens % sp->per_frame != 0 || cap % sp->per_frame != 0)
      return fail(CRATTN_EINVAL, "%s: chunk_tokens and cap must be whole frames of %d tokens",
                  who, sp->per_frame);
    if (q_pos0 % chunk_tokens + Lq > chunk_tokens)
      return fail(CRATTN_EINVAL, "%s: the query rows must lie in one chunk", who);
    if (kv_len % sp->per_frame != 0)
      return fail(CRATTN_EINVAL, "%s: kv_len must be whole frames of %d tokens", who,
                  sp->per_frame);
    const int nbf = (sp->per_frame + CRATTN_HSA_KBLOCK - 1) / CRATTN_HSA_KBLOCK;
    const int64_t vis_blocks = kv_len / sp->per_frame * nbf;
    const int64_t own_b0 = q_pos0 / chunk_tokens * (chunk_tokens / sp->per_frame) * nbf;
    const int64_t own_b1 = own_b0 + chunk_tokens / sp->per_frame * nbf;
    if (vis_blocks >= (int64_t(1) << 31) || cap >= (int64_t(1) << 31))
      return fail(CRATTN_EINVAL, "%s: history too long for 32-bit block ids", who);
    a.sel = sp->sel;
    a.sel_kb = sp->kb;
    a.sel_nbf = nbf;
    a.sel_per_frame = sp->per_frame;
    a.sel_vis_blocks = (int)vis_blocks;
    a.sel_own_b0 = (int)own_b0;
    a.sel_own_b1 = (int)own_b1;
  }
  if (rq != nullptr) {
    if (rq->table == nullptr || !aligned16(rq->table))
      return fail(CRATTN_EINVAL, "%s: table is required, 16-byte aligned", who);
    if (rq->max_t < 1 || rq->max_h < 1 || rq->max_w < 1 || rq->max_t > kMaxExtent ||
        rq->max_h > kMaxExtent || rq->max_w > kMaxExtent)
      return fail(CRATTN_EINVAL, "%s: table extents outside [1, %d]", who, kMaxExtent);
    if (rq->t0 < 0 || rq->grid_h < 1 || rq->grid_w < 1)
      return fail(CRATTN_EINVAL, "%s: t0 >= 0 and grid >= 1 required", who);
    if (rq->grid_h > rq->max_h || rq->grid_w > rq->max_w)
      return fail(CRATTN_EINVAL, "%s: grid %dx%d exceeds the table (%dx%d)", who, rq->grid_h,
                  rq->grid_w, rq->max_h, rq->max_w);
    if ((int64_t)rq->grid_h * rq->grid_w >= (int64_t(1) << 31))
      return fail(CRATTN_EINVAL, "%s: grid_h * grid_w must be below 2^31", who);
    const int64_t per_frame = (int64_t)rq->grid_h * rq->grid_w;
    if (chunk_tokens % per_frame != 0)
      return fail(CRATTN_EINVAL, "%s: chunk_tokens %lld is not a whole number of %dx%d frames",
                  who, (long long)chunk_tokens, rq->grid_h, rq->grid_w);
    const int64_t tok_off = q_pos0 % chunk_tokens;
    if (tok_off + Lq > chunk_tokens)
      return fail(CRATTN_EINVAL, "%s: the query rows must lie in one chunk", who);
    const int64_t last_t = rq->t0 + (tok_off + Lq - 1) / per_frame;
    if (last_t >= rq->max_t || rq->t0 > kMaxElems)
      return fail(CRATTN_EINVAL, "%s: time index %lld outside the table (max_t %d)", who,
                  (long long)last_t, rq->max_t);
    if (tok_off + Lq > (int64_t(1) << 31))
      return fail(CRATTN_EINVAL, "%s: token index exceeds 2^31", who);
    a.table = rq->table;
    a.max_t = rq->max_t;
    a.max_h = rq->max_h;
    a.max_w = rq->max_w;
    a.t0 = rq->t0;
    a.tok_off = tok_off;
    a.grid_h = rq->grid_h;
    a.grid_w = rq->grid_w;
  }
  const bool split_ok = workspace != nullptr && sp == nullptr;
  const crattn::AttnPlan plan =
      crattn::attn_plan(B, H, Lq, kv_len, q_pos0, chunk_tokens, D, split_ok);
  if (split_ok && ws_bytes < plan.ws_bytes)
    return fail(CRATTN_EINVAL, "%s: workspace of %zu bytes, %zu needed", who, ws_bytes,
                plan.ws_bytes);
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.cap = cap;
  a.kv_len = kv_len;
  a.q_pos0 = q_pos0;
  a.chunk_tokens = chunk_tokens;
  a.out = out;
  a.lse = lse;
  a.workspace = workspace;
  a.ws_bytes = ws_bytes;
  a.B = B;
  a.H = H;
  a.D = D;
  a.Lq = Lq;
  a.scale = scale;
  char what[64];
  snprintf(what, sizeof what, "%s launch", who);
  return hip_status(crattn::launch_attn(a, plan, static_cast<hipStream_t>(stream)), what);
}

}  // namespace

extern "C" {

int chunk_causal_attn(const void *q, const void *k_cache, const void *v_cache, int64_t cap,
                      int64_t kv_len, int64_t q_pos0, int64_t chunk_tokens, void *out, float *lse,
                      void *workspace, size_t ws_bytes, int B, int H, int D, int64_t Lq,
                      float scale, void *stream) {
  return attn_call("chunk_causal_attn", nullptr, nullptr, q, k_cache, v_cache, cap, kv_len, q_pos0,
                   chunk_tokens, out, lse, workspace, ws_bytes, B, H, D, Lq, scale, stream);
}

int chunk_causal_attn_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              int64_t cap, int64_t kv_len, int64_t q_pos0, int64_t chunk_tokens,
                              void *out, float *lse, int B, int H, int D, int64_t Lq, float scale,
                              void *stream) {
  const char *who = "chunk_causal_attn_noalloc";
  // the workspace this shape needs (0 when the key range is not split); the
  // rest of the validation is chunk_causal_attn's, run below before any launch
  const int st = attn_shape_check(B, H, Lq, kv_len, q_pos0, chunk_tokens, D, cap, who);
  if (st != CRATTN_OK) return st;
  const size_t need = crattn::attn_plan(B, H, Lq, kv_len, q_pos0, chunk_tokens, D, true).ws_bytes;
  if (need > crattn::kAttnScratchBytes)
    return fail(CRATTN_EINVAL, "%s: the call needs %zu bytes of scratch, the library holds %zu",
                who, need, crattn::kAttnScratchBytes);
  void *ws = nullptr;
  if (need > 0) {
    hipError_t e = hipSuccess;
    ws = crattn::attn_scratch(&e);
    if (ws == nullptr) return hip_status(e, "chunk_causal_attn_noalloc scratch");
  }
  return attn_call(who, nullptr, nullptr, q, k_cache, v_cache, cap, kv_len, q_pos0, chunk_tokens,
                   out, lse, ws, need, B, H, D, Lq, scale, stream);
}

int chunk_causal_attn_rope(const void *q, const float *table, int max_t, int max_h, int max_w,
                           int64_t t0, int grid_h, int grid_w, const void *k_cache,
                           const void *v_cache, int64_t cap, int64_t kv_len, int64_t q_pos0,
                           int64_t chunk_tokens, void *out, float *lse, void *workspace,
                           size_t ws_bytes, int B, int H, int D, int64_t Lq, float scale,
                           void *stream) {
  const QRope rq{table, max_t, max_h, max_w, t0, grid_h, grid_w};
  return attn_call("chunk_causal_attn_rope", &rq, nullptr, q, k_cache, v_cache, cap, kv_len, q_pos0,
                   chunk_tokens, out, lse, workspace, ws_bytes, B, H, D, Lq, scale, stream);
}

size_t hsa_pool_bytes(int B, int H, int64_t cap, int D, int per_frame) {
  if (B < 1 || H < 1 || per_frame < 1 || cap < 1 || cap % per_frame != 0) return 0;
  if (D != 64 && D != 128) return 0;
  const int64_t nf = cap / per_frame;
  const int64_t nbf = (per_frame + CRATTN_HSA_KBLOCK - 1) / CRATTN_HSA_KBLOCK;
  const double bytes = (double)B * H * (double)(nf + nf * nbf) * D * 4.0;
  if (bytes > (double)kMaxElems) return 0;
  return (size_t)B * H * (size_t)(nf + nf * nbf) * D * 4u;
}

int hsa_pool_keys(const void *k_cache, int64_t cap, int64_t row0, int64_t nrows, int per_frame,
                  void *pool, int B, int H, int D, void *stream) {
  if (k_cache == nullptr || pool == nullptr)
    return fail(CRATTN_EINVAL, "hsa_pool_keys: k_cache and pool are required");
  if (!aligned16(k_cache) || !aligned16(pool))
    return fail(CRATTN_EINVAL, "hsa_pool_keys: pointers must be 16-byte aligned");
  if (D != 64 && D != 128)
    return fail(CRATTN_ENOTSUP, "hsa_pool_keys: head_dim %d not supported (64 or 128)", D);
  if (B < 1 || H < 1 || per_frame < 1 || cap < 1 || cap % per_frame != 0)
    return fail(CRATTN_EINVAL, "hsa_pool_keys: B, H, per_frame >= 1 and cap a whole number of "
                               "frames required");
  if (row0 < 0 || nrows < 1 || row0 % per_frame != 0 || nrows % per_frame != 0 ||
      nrows > cap - row0)
    return fail(CRATTN_EINVAL, "hsa_pool_keys: %lld rows from row %lld must be whole frames "
                               "inside [0, %lld)", (long long)nrows, (long long)row0,
                (long long)cap);
  if (hsa_pool_bytes(B, H, cap, D, per_frame) == 0 || (double)B * H * (double)cap * D > (double)kMaxElems)
    return fail(CRATTN_EINVAL, "hsa_pool_keys: sizes too large");
  if ((double)B * H * (double)(nrows / per_frame) *
              (double)((per_frame + CRATTN_HSA_KBLOCK - 1) / CRATTN_HSA_KBLOCK) >=
          2147483648.0 ||
      cap / per_frame >= (1 << 30))
    return fail(CRATTN_EINVAL, "hsa_pool_keys: too many frames for one launch");
  crattn::HsaPoolArgs a;
  a.k = static_cast<const uint16_t *>(k_cache);
  a.cap = cap;
  a.per_frame = per_frame;
  a.nbf = (per_frame + CRATTN_HSA_KBLOCK - 1) / CRATTN_HSA_KBLOCK;
  a.nf = (int)(cap / per_frame);
  a.frames = static_cast<float *>(pool);
  a.blocks = a.frames + (size_t)B * H * a.nf * D;
  a.frame0 = (int)(row0 / per_frame);
  a.n_frames = (int)(nrows / per_frame);
  a.B = B;
  a.H = H;
  return hip_status(crattn::launch_hsa_pool(a, D, static_cast<hipStream_t>(stream)),
                    "hsa_pool_keys launch");
}

int hsa_select(const void *q, const void *pool, int64_t cap, int64_t kv_len, int per_frame,
               int64_t q_pos0, int64_t chunk_tokens, int kf, int kb, int32_t *sel, int B, int H,
               int D, int64_t Lq, void *stream) {
  if (q == nullptr || pool == nullptr || sel == nullptr)
    return fail(CRATTN_EINVAL, "hsa_select: q, pool and sel are required");
  if (!aligned16(q) || !aligned16(pool) || !aligned16(sel))
    return fail(CRATTN_EINVAL, "hsa_select: pointers must be 16-byte aligned");
  if (D != 64 && D != 128)
    return fail(CRATTN_ENOTSUP, "hsa_select: head_dim %d not supported (64 or 128)", D);
  if (B < 1 || H < 1 || Lq < 1 || q_pos0 < 0 || chunk_tokens < 1 || per_frame < 1 || cap < 1)
    return fail(CRATTN_EINVAL, "hsa_select: B, H, Lq, chunk_tokens, per_frame, cap >= 1 and "
                               "q_pos0 >= 0 required");
  if (chunk_tokens % per_frame != 0 || cap % per_frame != 0)
    return fail(CRATTN_EINVAL, "hsa_select: chunk_tokens and cap must be whole frames");
  if (q_pos0 > kMaxElems || Lq > kMaxElems || q_pos0 % chunk_tokens + Lq > chunk_tokens)
    return fail(CRATTN_EINVAL, "hsa_select: the query rows must lie in one chunk");
  const int64_t q_chunk = q_pos0 / chunk_tokens;
  if (kv_len > cap || kv_len % per_frame != 0 || (q_chunk + 1) * chunk_tokens > kv_len)
    return fail(CRATTN_EINVAL, "hsa_select: kv_len %lld must be whole frames, at most cap and "
                               "past the query chunk's end", (long long)kv_len);
  if (kf < 1 || kf > CRATTN_HSA_MAX_KF || kb < 1 || kb > CRATTN_HSA_MAX_KB)
    return fail(CRATTN_EINVAL, "hsa_select: kf in [1, %d] and kb in [1, %d] required",
                CRATTN_HSA_MAX_KF, CRATTN_HSA_MAX_KB);
  const int64_t nbf = (per_frame + CRATTN_HSA_KBLOCK - 1) / CRATTN_HSA_KBLOCK;
  const int64_t fc = chunk_tokens / per_frame;
  const int64_t n_hist = kv_len / per_frame - fc;
  if (n_hist > CRATTN_HSA_MAX_CAND || std::min<int64_t>(kf, n_hist) * nbf > CRATTN_HSA_MAX_CAND)
    return fail(CRATTN_EINVAL, "hsa_select: %lld history frames, %lld block candidates: at most "
                               "%d each", (long long)n_hist,
                (long long)(std::min<int64_t>(kf, n_hist) * nbf), CRATTN_HSA_MAX_CAND);
  if (hsa_pool_bytes(B, H, cap, D, per_frame) == 0)
    return fail(CRATTN_EINVAL, "hsa_select: sizes too large");
  const int64_t n_qblocks = (Lq + CRATTN_HSA_QBLOCK - 1) / CRATTN_HSA_QBLOCK;
  if ((double)B * H * (double)n_qblocks >= 2147483648.0)
    return fail(CRATTN_EINVAL, "hsa_select: too many query blocks for one launch");
  crattn::HsaSelectArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.nf = (int)(cap / per_frame);
  a.nbf = (int)nbf;
  a.frames = static_cast<const float *>(pool);
  a.blocks = a.frames + (size_t)B * H * a.nf * D;
  a.sel = sel;
  a.Lq = Lq;
  a.n_hist = (int)n_hist;
  a.own_f0 = (int)(q_chunk * fc);
  a.fc = (int)fc;
  a.kf = kf;
  a.kb = kb;
  a.n_qblocks = (int)n_qblocks;
  a.B = B;
  a.H = H;
  return hip_status(crattn::launch_hsa_select(a, D, static_cast<hipStream_t>(stream)),
                    "hsa_select launch");
}

int hsa_attn(const void *q, const void *k_cache, const void *v_cache, int64_t cap, int64_t kv_len,
             int64_t q_pos0, int64_t chunk_tokens, int per_frame, const int32_t *sel, int kb,
             void *out, float *lse, int B, int H, int D, int64_t Lq, float scale, void *stream) {
  const Sparse sp{sel, kb, per_frame};
  return attn_call("hsa_attn", nullptr, &sp, q, k_cache, v_cache, cap, kv_len, q_pos0,
                   chunk_tokens, out, lse, nullptr, 0, B, H, D, Lq, scale, stream);
}

size_t svg2_kmeans_workspace_bytes(int B, int H, int n, int C) {
  if (B < 1 || H < 1 || n < 1 || n > CRATTN_SVG2_MAX_N || C < 1 || C > CRATTN_SVG2_MAX_C)
    return 0;
  if ((double)B * H * CRATTN_SVG2_MAX_N >= 2147483648.0) return 0;
  // every token's cluster and rank, then every 128-token block's counts
  const size_t assign = ((size_t)B * H * n * 4u + 255u) & ~size_t(255);
  return assign + (size_t)B * H * ((n + 127) / 128) * C * 4u;
}

namespace {

// Checks one k-means problem as svg2_kmeans documents and fills its kernel
// arguments; `fn` names the call in the error message.
int km_setup(const char *fn, const svg2_kmeans_problem &p, int D, int iters,
             crattn::KmArgs *a) {
  const int B = p.B, H = p.H, n = p.n, C = p.C;
  if (p.x == nullptr || p.centroids == nullptr || p.perm == nullptr || p.offsets == nullptr ||
      p.workspace == nullptr)
    return fail(CRATTN_EINVAL, "%s: x, centroids, perm, offsets, workspace required", fn);
  if (!aligned16(p.x) || !aligned16(p.centroids) || !aligned16(p.workspace) ||
      (reinterpret_cast<uintptr_t>(p.perm) & 3u) || (reinterpret_cast<uintptr_t>(p.offsets) & 3u))
    return fail(CRATTN_EINVAL, "%s: x, centroids, workspace 16-byte aligned required", fn);
  if (D != 64 && D != 128)
    return fail(CRATTN_ENOTSUP, "%s: head_dim %d not supported (64 or 128)", fn, D);
  if (B < 1 || H < 1 || n < 1 || n > CRATTN_SVG2_MAX_N)
    return fail(CRATTN_EINVAL, "%s: B, H >= 1 and n in [1, %d] required", fn,
                CRATTN_SVG2_MAX_N);
  if (C < 1 || C > CRATTN_SVG2_MAX_C || iters < 1 || iters > CRATTN_SVG2_MAX_ITERS)
    return fail(CRATTN_EINVAL, "%s: C in [1, %d] and iters in [1, %d] required", fn,
                CRATTN_SVG2_MAX_C, CRATTN_SVG2_MAX_ITERS);
  if (p.stride_b < 0 || p.stride_h < 0 || p.stride_row < 0 || p.stride_b % 8 ||
      p.stride_h % 8 || p.stride_row % 8 || p.stride_b > kMaxElems || p.stride_h > kMaxElems ||
      p.stride_row > kMaxElems)
    return fail(CRATTN_EINVAL, "%s: strides must be non-negative multiples of 8", fn);
  if (p.cent_stride < (int64_t)C * D || p.cent_stride % 4 || p.perm_stride < n ||
      p.off_stride < C + 1 || p.cent_stride > kMaxElems || p.perm_stride > kMaxElems ||
      p.off_stride > kMaxElems)
    return fail(CRATTN_EINVAL, "%s: output strides smaller than one head's extent", fn);
  const size_t need = svg2_kmeans_workspace_bytes(B, H, n, C);
  if (need == 0 || p.ws_bytes < need)
    return fail(CRATTN_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn, p.ws_bytes, need);
  a->x = static_cast<const uint16_t *>(p.x);
  a->sb = p.stride_b;
  a->sh = p.stride_h;
  a->sr = p.stride_row;
  a->B = B;
  a->H = H;
  a->n = n;
  a->C = C;
  a->cent = p.centroids;
  a->cent_s = p.cent_stride;
  a->perm = p.perm;
  a->perm_s = p.perm_stride;
  a->off = p.offsets;
  a->off_s = p.off_stride;
  a->assign = static_cast<int32_t *>(p.workspace);
  a->bcnt = reinterpret_cast<int32_t *>(static_cast<char *>(p.workspace) +
                                        (((size_t)B * H * n * 4u + 255u) & ~size_t(255)));
  return CRATTN_OK;
}

struct ByteRange {
  uintptr_t lo, hi;  // [lo, hi)
};

// The bytes a problem writes (centroids, perm, offsets, the workspace bytes
// it needs) and, last, the bytes of x it reads, from its (already checked)
// arguments.
void km_ranges(const svg2_kmeans_problem &p, int D, ByteRange r[5]) {
  const int64_t heads = (int64_t)p.B * p.H;
  auto span = [](const void *ptr, int64_t last_elem_end, size_t elem) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
    return ByteRange{lo, lo + (uintptr_t)last_elem_end * elem};
  };
  r[0] = span(p.centroids, (heads - 1) * p.cent_stride + (int64_t)p.C * D, 4);
  r[1] = span(p.perm, (heads - 1) * p.perm_stride + p.n, 4);
  r[2] = span(p.offsets, (heads - 1) * p.off_stride + p.C + 1, 4);
  r[3] = span(p.workspace, (int64_t)svg2_kmeans_workspace_bytes(p.B, p.H, p.n, p.C), 1);
  r[4] = span(p.x, (int64_t)(p.B - 1) * p.stride_b + (int64_t)(p.H - 1) * p.stride_h +
                       (int64_t)(p.n - 1) * p.stride_row + D, 2);
}

}  // namespace

int svg2_kmeans(const void *x, int64_t stride_b, int64_t stride_h, int64_t stride_row, int B,
                int H, int n, int D, int C, int iters, int from_tokens, float *centroids,
                int64_t cent_stride, int32_t *perm, int64_t perm_stride, int32_t *offsets,
                int64_t off_stride, void *workspace, size_t ws_bytes, void *stream) {
  const svg2_kmeans_problem p{x,         stride_b,    stride_h, stride_row, B,          H,
                              n,         C,           centroids, cent_stride, perm,     perm_stride,
                              offsets,   off_stride,  workspace, ws_bytes};
  crattn::KmArgs a;
  const int rc = km_setup("svg2_kmeans", p, D, iters, &a);
  if (rc != CRATTN_OK) return rc;
  return hip_status(crattn::launch_svg2_kmeans(a, D, iters, from_tokens != 0,
                                               static_cast<hipStream_t>(stream)),
                    "svg2_kmeans launch");
}

int svg2_kmeans2(const svg2_kmeans_problem *p, int D, int iters, int from_tokens, void *stream) {
  if (p == nullptr) return fail(CRATTN_EINVAL, "svg2_kmeans2: problems required");
  crattn::KmArgs a[2];
  for (int k = 0; k < 2; ++k) {
    const int rc = km_setup(k == 0 ? "svg2_kmeans2 (problem 0)" : "svg2_kmeans2 (problem 1)",
                            p[k], D, iters, &a[k]);
    if (rc != CRATTN_OK) return rc;
  }
  ByteRange r0[5], r1[5];
  km_ranges(p[0], D, r0);
  km_ranges(p[1], D, r1);
  // every written range of one problem against every range of the other
  for (int i = 0; i < 5; ++i)
    for (int j = 0; j < 5; ++j)
      if ((i < 4 || j < 4) && r0[i].lo < r1[j].hi && r1[j].lo < r0[i].hi)
        return fail(CRATTN_EINVAL, "svg2_kmeans2: the two problems' buffers overlap");
  return hip_status(crattn::launch_svg2_kmeans2(a[0], a[1], D, iters, from_tokens != 0,
                                                static_cast<hipStream_t>(stream)),
                    "svg2_kmeans2 launch");
}

int svg2_n_slots(int64_t Lq, int Cq) {
  if (Lq < 1 || Lq > kMaxElems || Cq < 1 || Cq > CRATTN_SVG2_MAX_C) return 0;
  const int64_t v = (Lq + CRATTN_SVG2_QTILE - 1) / CRATTN_SVG2_QTILE + Cq;
  return v >= (int64_t(1) << 30) ? 0 : (int)v;
}

int svg2_plan(const float *q_cent, const int32_t *q_off, const float *k_cent,
              const int32_t *k_off, const int32_t *k_perm, int B, int H, int D, int Cq, int Ck,
              int S, int n_vis, int64_t L, int64_t Lq, float p, float scale, int32_t *sel,
              int32_t *lists, int64_t list_cap, int32_t *list_len, int32_t *slots, int n_slots,
              void *stream) {
  if (q_cent == nullptr || q_off == nullptr || k_cent == nullptr || k_off == nullptr ||
      k_perm == nullptr || sel == nullptr || lists == nullptr || list_len == nullptr ||
      slots == nullptr)
    return fail(CRATTN_EINVAL, "svg2_plan: every pointer is required");
  if (!aligned16(q_cent) || !aligned16(k_cent) || !aligned16(slots) || !aligned16(sel) ||
      !aligned16(lists) || !aligned16(list_len) || !aligned16(q_off) || !aligned16(k_off) ||
      !aligned16(k_perm))
    return fail(CRATTN_EINVAL, "svg2_plan: pointers must be 16-byte aligned");
  if (D != 64 && D != 128)
    return fail(CRATTN_ENOTSUP, "svg2_plan: head_dim %d not supported (64 or 128)", D);
  if (B < 1 || H < 1 || Lq < 1 || Lq > kMaxElems)
    return fail(CRATTN_EINVAL, "svg2_plan: B, H, Lq >= 1 required");
  if (Cq < 1 || Cq > CRATTN_SVG2_MAX_C || Ck < 1 || Ck > CRATTN_SVG2_MAX_C)
    return fail(CRATTN_EINVAL, "svg2_plan: Cq and Ck in [1, %d] required", CRATTN_SVG2_MAX_C);
  if (S < 1 || n_vis < 1 || n_vis > S || (int64_t)n_vis * Ck > CRATTN_SVG2_MAX_CAND)
    return fail(CRATTN_EINVAL, "svg2_plan: 1 <= n_vis <= S and n_vis*Ck <= %d required",
                CRATTN_SVG2_MAX_CAND);
  if (L < 1 || L > CRATTN_SVG2_MAX_N)
    return fail(CRATTN_EINVAL, "svg2_plan: L in [1, %d] required", CRATTN_SVG2_MAX_N);
  if (!(p > 0.f) || !isfinite(p) || !(scale >= 0.f) || !isfinite(scale))
    return fail(CRATTN_EINVAL, "svg2_plan: p > 0 and a finite scale >= 0 required");
  if (list_cap % 64 != 0 || list_cap < (int64_t)n_vis * L || list_cap > kMaxElems)
    return fail(CRATTN_EINVAL, "svg2_plan: list_cap must be a multiple of 64, >= %lld",
                (long long)((int64_t)n_vis * L));
  if (n_slots < svg2_n_slots(Lq, Cq) || svg2_n_slots(Lq, Cq) == 0)
    return fail(CRATTN_EINVAL, "svg2_plan: n_slots %d below %d", n_slots, svg2_n_slots(Lq, Cq));
  if ((double)B * H * Cq >= 2147483648.0 || (double)S * L * B * H > (double)kMaxElems)
    return fail(CRATTN_EINVAL, "svg2_plan: sizes too large");
  crattn::SvgPlanArgs a;
  a.q_cent = q_cent;
  a.q_off = q_off;
  a.k_cent = k_cent;
  a.k_off = k_off;
  a.k_perm = k_perm;
  a.B = B;
  a.H = H;
  a.Cq = Cq;
  a.Ck = Ck;
  a.S = S;
  a.n_vis = n_vis;
  a.L = L;
  a.p = p;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)D);
  a.sel = sel;
  a.lists = lists;
  a.list_cap = list_cap;
  a.list_len = list_len;
  a.slots = slots;
  a.n_slots = n_slots;
  a.qtile = CRATTN_SVG2_QTILE;
  return hip_status(crattn::launch_svg2_plan(a, D, static_cast<hipStream_t>(stream)),
                    "svg2_plan launch");
}

size_t svg2_attn_workspace_bytes(int B, int H, int64_t Lq, int D, int n_slots, int splits) {
  if (B < 1 || H < 1 || Lq < 1 || Lq > kMaxElems || (D != 64 && D != 128) || splits < 1 ||
      splits > 16 || n_slots < 1 || (double)B * H * n_slots >= 1073741824.0)
    return 0;
  // the work counter and slot count, the work order (16-byte records), then
  // the split partials
  const size_t order = ((size_t)B * H * n_slots * 16u + 255u) & ~size_t(255);
  return 256u + order +
         (splits > 1 ? (size_t)splits * (size_t)B * H * Lq * (size_t)(D + 1) * 4u : 0);
}

int svg2_attn(const void *q, const void *k_cache, const void *v_cache, int64_t cap,
              const int32_t *q_perm, const int32_t *slots, int n_slots, const int32_t *lists,
              int64_t list_cap, const int32_t *list_len, int Cq, int splits, void *out,
              float *lse, void *workspace, size_t ws_bytes, int B, int H, int D, int64_t Lq,
              float scale, void *stream) {
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || out == nullptr ||
      q_perm == nullptr || slots == nullptr || lists == nullptr || list_len == nullptr)
    return fail(CRATTN_EINVAL, "svg2_attn: q, caches, q_perm, slots, lists, list_len and out "
                               "are required");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(lse) || !aligned16(workspace) || !aligned16(slots) || !aligned16(lists) ||
      !aligned16(q_perm) || !aligned16(list_len))
    return fail(CRATTN_EINVAL, "svg2_attn: pointers must be 16-byte aligned");
  if (D != 64 && D != 128)
    return fail(CRATTN_ENOTSUP, "svg2_attn: head_dim %d not supported (64 or 128)", D);
  if (B < 1 || H < 1 || Lq < 1 || Lq > kMaxElems || cap < 1 || n_slots < 1)
    return fail(CRATTN_EINVAL, "svg2_attn: B, H, Lq, cap, n_slots >= 1 required");
  if (Cq < 1 || Cq > CRATTN_SVG2_MAX_C)
    return fail(CRATTN_EINVAL, "svg2_attn: Cq in [1, %d] required", CRATTN_SVG2_MAX_C);
  if (list_cap < 64 || list_cap % 64 != 0 || list_cap >= (int64_t(1) << 31))
    return fail(CRATTN_EINVAL, "svg2_attn: list_cap must be a positive multiple of 64");
  if (splits < 1 || splits > 16)
    return fail(CRATTN_EINVAL, "svg2_attn: splits in [1, 16] required");
  if (!(scale >= 0.f) || !isfinite(scale))
    return fail(CRATTN_EINVAL, "svg2_attn: scale must be finite and >= 0");
  if ((double)cap * D >= 2147483648.0 || (double)B * H * (double)cap * D > (double)kMaxElems)
    return fail(CRATTN_EINVAL, "svg2_attn: cap * head_dim must be below 2^31");
  if ((double)B * H * (double)Lq * (D / 4) >= 4294967296.0 ||
      (double)B * H * (double)n_slots * splits >= 2147483648.0 || Lq >= (int64_t(1) << 31))
    return fail(CRATTN_EINVAL, "svg2_attn: too large for one launch");
  const size_t need = svg2_attn_workspace_bytes(B, H, Lq, D, n_slots, splits);
  if (workspace == nullptr || ws_bytes < need)
    return fail(CRATTN_EINVAL, "svg2_attn: workspace of %zu bytes, %zu needed", ws_bytes, need);
  crattn::AttnPlan plan{};
  plan.d = D;
  plan.bm = CRATTN_SVG2_QTILE;
  plan.bn = 64;
  plan.n_tiles = n_slots;
  plan.splits = splits;
  plan.grid = (int64_t)B * H * n_slots * splits;
  plan.ws_bytes = need;
  crattn::AttnArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.cap = cap;
  a.kv_len = cap;
  a.q_pos0 = 0;
  a.chunk_tokens = 1;
  a.out = out;
  a.lse = lse;
  a.workspace = workspace;
  a.ws_bytes = ws_bytes;
  a.B = B;
  a.H = H;
  a.D = D;
  a.Lq = Lq;
  a.scale = scale;
  a.q_perm = q_perm;
  a.gslots = slots;
  a.lists = lists;
  a.list_len = list_len;
  a.list_cap = list_cap;
  a.cq = Cq;
  return hip_status(crattn::launch_attn(a, plan, static_cast<hipStream_t>(stream)),
                    "svg2_attn launch");
}

const char *crattn_last_error(void) { return g_err; }

}  // extern "C"
