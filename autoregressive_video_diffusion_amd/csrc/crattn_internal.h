// Internal declarations shared by the C-ABI front end (api.cpp) and the HIP
// kernel files.  Not installed; the public interface is include/crattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace crattn {

// head_dim split of the 3D rotary code: h and w get 2*floor(D/6) dims each,
// t the rest, in the order t, h, w.
struct RopeSplit {
  int dt, dh, dw;
};
inline RopeSplit rope_split(int D) {
  const int hw = 2 * (D / 6);
  return RopeSplit{D - 2 * hw, hw, hw};
}

// Compute units of the current device, asked at each call: the library
// keeps no state between calls (a cache would also go stale on another
// device).  256 if the runtime cannot tell.
inline int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  return n;
}

struct RopeTableArgs {
  float2 *table;
  int dt, dh, dw;
  int max_t, max_h, max_w;
  double theta;
};

struct RopeAppendArgs {
  const void *q;
  void *q_out;
  const void *k;
  const void *v;
  void *k_cache;
  void *v_cache;
  int64_t cap, cache_pos;
  const float2 *table;
  int max_t, max_h, max_w;
  int B, H, D;
  int64_t n;
  int64_t t0, tok_off;
  int grid_h, grid_w;
  int dtype;  // CRATTN_F32 / CRATTN_BF16
};

struct QkvArgs {
  const void *x;      // [B][n][C] bf16
  const void *w;      // [3*H*D][C] bf16
  void *q_out;        // [B][n][H][D] bf16 or null
  void *k_cache;      // [B][H][cap][D] bf16
  void *v_cache;
  int64_t cap, cache_pos;
  const float *table;
  int max_t, max_h, max_w;
  int B, H, D, C;
  int64_t n;
  int64_t t0, tok_off;
  int grid_h, grid_w;
};

struct AttnArgs {
  const void *q;
  const void *k;
  const void *v;
  int64_t cap, kv_len, q_pos0, chunk_tokens;
  void *out;
  float *lse;
  void *workspace;
  size_t ws_bytes;
  int B, H, D;
  int64_t Lq;
  float scale;
  // Causal-RoPE of the queries on load (chunk_causal_attn_rope)
  bool rope;
  const float *table;
  int max_t, max_h, max_w;
  int64_t t0, tok_off;
  int grid_h, grid_w;
  // block-sparse attention (hsa_attn): selected block ids per query tile;
  // ids in [0, sel_vis_blocks) outside the own chunk's [sel_own_b0,
  // sel_own_b1) are history blocks, any other id is skipped
  const int32_t *sel;
  int sel_kb, sel_nbf, sel_per_frame, sel_vis_blocks, sel_own_b0, sel_own_b1;
  // cluster-sparse attention (svg2_attn): query tiles of query clusters,
  // each with an explicit list of key rows
  const int32_t *q_perm;    // [B][H][Lq] query row of each reordered position
  const int32_t *gslots;    // [B][H][n_slots][4] (first position, rows, cluster, 0)
  const int32_t *lists;     // [B][H][Cq][list_cap] key rows
  const int32_t *list_len;  // [B][H][Cq]
  int64_t list_cap;
  int n_slots, cq, splits;
};

// Key pooling of whole frames [frame0, frame0 + n_frames) of the cache.
struct HsaPoolArgs {
  const uint16_t *k;  // [B][H][cap][D] bf16
  float *frames;      // [B][H][nf][D]
  float *blocks;      // [B][H][nf * nbf][D]
  int64_t cap;
  int per_frame, nbf, nf;
  int frame0, n_frames;
  int B, H;
};

// Two-level selection of each (b, h, query block).
struct HsaSelectArgs {
  const uint16_t *q;     // [B][Lq][H][D] bf16, rotated
  const float *frames;   // pooled keys (HsaPoolArgs layout)
  const float *blocks;
  int32_t *sel;          // [B][H][n_qblocks][kb]
  int64_t Lq;
  // history = the visible frames [0, n_vis) except the own chunk's
  // [own_f0, own_f0 + fc): candidate c is frame c, or c + fc from own_f0 on
  int nf, nbf, n_hist, own_f0, fc;
  int kf, kb, n_qblocks;
  int B, H;
};

// k-means of one token set per (b, h) and its stable reordering by cluster.
// Token t of (b, h) is x + b*sb + h*sh + t*sr (bf16).  Per-head outputs sit
// at stride cent_s / perm_s / off_s elements from one head to the next.
struct KmArgs {
  const uint16_t *x;
  int64_t sb, sh, sr;
  int B, H, n, C;
  float *cent;     // [.., C, D]
  int64_t cent_s;
  int32_t *perm;   // [.., n]
  int64_t perm_s;
  int32_t *off;    // [.., C + 1]
  int64_t off_s;
  int32_t *assign;  // workspace [B*H][n]: cluster | rank in its block << 16
  int32_t *bcnt;    // workspace [B*H][ceil(n/128)][C]: cluster counts per block
};

// Centroid top-p selection and key lists of every (b, h, query cluster).
struct SvgPlanArgs {
  const float *q_cent;     // [B][H][Cq][D]
  const int32_t *q_off;    // [B][H][Cq + 1]
  const float *k_cent;     // [B][H][S][Ck][D]
  const int32_t *k_off;    // [B][H][S][Ck + 1]
  const int32_t *k_perm;   // [B][H][S][L]
  int B, H, Cq, Ck, S, n_vis;
  int64_t L;
  float p, scale;
  int32_t *sel;            // [B][H][Cq][n_vis * Ck]
  int32_t *lists;          // [B][H][Cq][list_cap]
  int64_t list_cap;
  int32_t *list_len;       // [B][H][Cq]
  int32_t *slots;          // [B][H][n_slots][4]
  int n_slots, qtile;
};

// Launch plan of one attention call: how query rows are tiled and how the
// key range of each tile is split.  A pure function of the shape.
struct AttnPlan {
  int d;             // head_dim (64 or 128)
  int bm;            // query rows per workgroup
  int bn;            // keys per LDS tile
  int64_t n_tiles;   // query tiles over all chunk segments (per b, h)
  int splits;        // key-range splits per query tile (1 = no workspace)
  int64_t grid;      // workgroups launched by the main kernel
  size_t ws_bytes;   // workspace the split needs (0 when splits == 1)
  // segments: query rows grouped by chunk; tiles never straddle a chunk
  int64_t seg0_rows;  // rows in the first (possibly partial) chunk segment
  int64_t tiles0;     // tiles of the first segment
  int64_t tiles_full; // tiles of every full middle segment
  int64_t n_full;     // number of full middle segments
  int64_t last_rows;  // rows of the trailing partial segment (0 if none)
  // balanced split (dense head_dim-128 kernel with a workspace): the key
  // steps of all query tiles, in (batch, head, tile, key tile) order, cut
  // into `grid` equal ranges, one per workgroup; a tile cut between ranges
  // is merged by the last of its parts to finish
  bool stream;
  int64_t steps_bh;     // key steps of one (batch, head): sum over tiles
  int64_t total_steps;  // B * H * steps_bh
};

// Workspace of the balanced split: per-range completion counters, then two
// partial slots per workgroup (normalised O, fp32, then base-2 log-sum-exp)
// of one 256-row query tile each.
constexpr int kStreamRows = 256;
constexpr size_t kStreamCounterBytes = 1024;  // 256 counters
inline size_t stream_slot_floats(int D) { return (size_t)kStreamRows * (size_t)(D + 1); }

AttnPlan attn_plan(int B, int H, int64_t Lq, int64_t kv_len, int64_t q_pos0,
                   int64_t chunk_tokens, int D, bool allow_split);

hipError_t launch_rope_table(const RopeTableArgs &a, hipStream_t s);
hipError_t launch_rope_append(const RopeAppendArgs &a, hipStream_t s);
hipError_t launch_attn(const AttnArgs &a, const AttnPlan &p, hipStream_t s);

// The library's fixed device scratch for callers that cannot allocate
// (chunk_causal_attn_noalloc): kAttnScratchBytes on every device the library
// runs on, held until the process ends.  attn_scratch returns its address on
// the current device (looked up once per device), or null with *err set.
constexpr size_t kAttnScratchBytes = size_t(72) << 20;
void *attn_scratch(hipError_t *err);
hipError_t launch_qkv_rope(const QkvArgs &a, hipStream_t s);
hipError_t launch_hsa_pool(const HsaPoolArgs &a, int D, hipStream_t s);
hipError_t launch_hsa_select(const HsaSelectArgs &a, int D, hipStream_t s);
hipError_t launch_svg2_kmeans(const KmArgs &a, int D, int iters, bool from_tokens, hipStream_t s);
// two problems (same D, iters and start) in one launch sequence
hipError_t launch_svg2_kmeans2(const KmArgs &a0, const KmArgs &a1, int D, int iters,
                               bool from_tokens, hipStream_t s);
hipError_t launch_svg2_plan(const SvgPlanArgs &a, int D, hipStream_t s);

}  // namespace crattn
