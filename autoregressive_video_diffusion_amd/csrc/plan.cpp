// Launch planning of the attention kernels: how the query rows of a call
// are tiled and how the key range of each tile is split.  Host code only (no
// device code), shared by the C-ABI front end; a pure function of the shape.
#include <algorithm>

#include "crattn_internal.h"

namespace crattn {

namespace {
// Every attention kernel works on 256 query rows per workgroup (4
// wavefronts x 64 rows, or 8 x 32) and walks the keys in tiles of 64.
constexpr int kQueryTile = 256;
constexpr int kKeyTile = 64;
}  // namespace

AttnPlan attn_plan(int B, int H, int64_t Lq, int64_t kv_len, int64_t q_pos0,
                   int64_t chunk_tokens, int D, bool allow_split) {
  AttnPlan p{};
  p.d = D;
  p.bm = kQueryTile;
  p.bn = kKeyTile;
  const int64_t L = chunk_tokens;
  const int64_t c0 = q_pos0 / L;
  p.seg0_rows = std::min(Lq, (c0 + 1) * L - q_pos0);
  p.tiles0 = (p.seg0_rows + p.bm - 1) / p.bm;
  const int64_t rest = Lq - p.seg0_rows;
  p.n_full = rest / L;
  p.last_rows = rest - p.n_full * L;
  p.tiles_full = (L + p.bm - 1) / p.bm;
  p.n_tiles = p.tiles0 + p.n_full * p.tiles_full + (p.last_rows + p.bm - 1) / p.bm;
  const int64_t units = (int64_t)B * H * p.n_tiles;
  // Fewest key tiles any query tile has (the first segment sees the least).
  const int64_t min_keys = std::min(kv_len, (c0 + 1) * L);
  const int64_t min_ktiles = (min_keys + p.bn - 1) / p.bn;
  constexpr int64_t kSlots = 256;  // one workgroup per compute unit of an MI355X
  p.splits = 1;
  // Split the key range only when the query tiles alone leave most of the
  // chip idle: partials cost (D + 1) * 4 bytes per row and split of traffic.
  if (allow_split && units * 2 <= kSlots) {
    double best = (double)units / (double)(((units + kSlots - 1) / kSlots) * kSlots);
    for (int s = 2; s <= 16; ++s) {
      if (min_ktiles / s < 8) break;
      const int64_t u = units * s;
      const double eff = (double)u / (double)(((u + kSlots - 1) / kSlots) * kSlots);
      if (eff > best + 0.05) {
        best = eff;
        p.splits = s;
      }
    }
  }
  p.grid = units * p.splits;
  p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)B * H * Lq * (size_t)(D + 1) * 4u : 0;
  return p;
}

}  // namespace crattn
