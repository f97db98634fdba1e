// Device helpers shared by the RoPE/append pass and the fused QKV projection:
// token position decode (global time index) and the cos/sin table gather.
//
// Source: "Accelerating Video Generation Inference with Sequential-Parallel
// 3D Positional Encoding Using a Global Time Index", technical summary §2.B
// (temporal position = start offset + local frame; no gather across ranks)
// and §2.C (cos/sin precomputed into contiguous device tensors).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace crattn {

struct Pos {
  uint32_t t, h, w;
};

// Token g of the chunk (raster order) -> (t0 + frame, row, column).
__device__ inline Pos decode_pos(uint32_t g, uint32_t per_frame, uint32_t gw, uint32_t t0) {
  const uint32_t f = g / per_frame;
  const uint32_t in_frame = g - f * per_frame;
  const uint32_t r = in_frame / gw;
  return Pos{t0 + f, r, in_frame - r * gw};
}

// Geometry of the cos/sin table: [t: max_t x ht | h: max_h x hh | w: max_w x hh]
// float2 (cos, sin) entries.
struct TabGeom {
  uint32_t ht, hh;      // pairs in the t group and in the h (= w) group
  uint32_t base_h;      // first entry of axis h  = max_t * ht
  uint32_t base_w;      // first entry of axis w  = base_h + max_h * hh
};

// (cos, sin) of feature pair `pair` of head_dim at position p.
__device__ inline float2 pair_cs(const float2 *__restrict__ tab, const TabGeom &g,
                                 uint32_t pair, const Pos &p) {
  uint32_t idx;
  if (pair < g.ht)
    idx = p.t * g.ht + pair;
  else if (pair < g.ht + g.hh)
    idx = g.base_h + p.h * g.hh + (pair - g.ht);
  else
    idx = g.base_w + p.w * g.hh + (pair - g.ht - g.hh);
  return tab[idx];
}

// Rotation of the pair (x, y) by the angle whose (cos, sin) is cs, in fp32
// with one fixed rounding order (the two products of each output fused as
// written), so every kernel that rotates produces the same bits.
__device__ inline float2 rotate_pair(float x, float y, float2 cs) {
  return make_float2(__builtin_fmaf(x, cs.x, -(y * cs.y)), __builtin_fmaf(x, cs.y, y * cs.x));
}

}  // namespace crattn
