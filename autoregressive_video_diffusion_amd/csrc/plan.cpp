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
  // Split the key range uniformly only when the query tiles alone leave most
  // of the chip idle (partials cost (D + 1) * 4 bytes per row and split of
  // traffic, merged by a second kernel).
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
  p.stream = false;
  p.steps_bh = p.total_steps = 0;
  // Balanced split of the dense head_dim-128 kernel, for launches whose
  // query tiles number between half and all of the compute units and whose
  // tiles are long (at least 192 key tiles): one workgroup per compute unit,
  // each taking an equal share of all key steps (whole tiles where the
  // shares line up, parts of a tile where they do not), so no unit idles
  // while the last tiles finish.  With fewer tiles the uniform split above
  // (partials merged by a second kernel) serves better, with more tiles or
  // short ones one workgroup per tile.  Segment s (query rows of chunk
  // c0 + s) sees min(kv_len, (c0 + s + 1) L) keys.
  if (D == 128 && allow_split && units * 2 > kSlots && units <= kSlots && min_ktiles >= 192) {
    const int64_t n_seg = 1 + p.n_full + (p.last_rows > 0 ? 1 : 0);
    int64_t steps = 0;
    for (int64_t s = 0; s < n_seg; ++s) {
      const int64_t tiles = s == 0 ? p.tiles0
                            : s <= p.n_full ? p.tiles_full
                                            : (p.last_rows + p.bm - 1) / p.bm;
      const int64_t limit = std::min(kv_len, (c0 + s + 1) * L);
      steps += tiles * ((limit + p.bn - 1) / p.bn);
    }
    const int64_t total = (int64_t)B * H * steps;
    // At least 8 key steps per workgroup (unless whole tiles are smaller),
    // and at least 1/8 of the longest tile's: the part that finishes a tile
    // last reads the others' partials alone, so a tile is cut into at most
    // about 9 parts.
    const int64_t nkt_max = (std::min(kv_len, (c0 + n_seg) * L) + p.bn - 1) / p.bn;
    const int64_t min_steps = std::max<int64_t>(8, (nkt_max + 7) / 8);
    int64_t g = std::min<int64_t>(kSlots, std::max<int64_t>(units, total / min_steps));
    g = std::max<int64_t>(1, std::min(g, total));
    // one workgroup per tile already gives all the parallelism there is:
    // no split (and a row's result then does not depend on the call's other
    // rows)
    if (units <= kSlots && total / min_steps <= units) return p;
    p.stream = true;
    p.splits = 1;
    p.steps_bh = steps;
    p.total_steps = total;
    p.grid = g;
    p.ws_bytes = kStreamCounterBytes + 2u * (size_t)g * stream_slot_floats(D) * 4u;
  }
  return p;
}

}  // namespace crattn
