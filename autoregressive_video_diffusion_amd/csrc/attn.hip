// Chunk-causal flash attention for AMD CDNA4 (gfx950), bf16 MFMA.
//
// Sources: "Wave Forcing" abstract (chunk-based causal attention over the
// earlier chunks); "Accelerating Video Generation Inference with
// Sequential-Parallel 3D Positional Encoding Using a Global Time Index" §1
// (attention against a KV cache).  Key j is visible to query row i iff
// j < kv_len and floor(j/L) <= floor((q_pos0+i)/L): bidirectional inside a
// chunk, causal across chunks.  The design below is this file's own.
//
// Work decomposition
//   * A workgroup (4 wavefronts) owns BM query rows of one (batch, head) and
//     walks the visible keys in tiles of BN = 64.  Query tiles never straddle
//     a chunk boundary, so every row of a workgroup has the same visible key
//     range [0, limit): masking is needed on the last key tile only, and keys
//     beyond `limit` are never loaded (NaN/Inf in future chunks cannot leak
//     through 0 * NaN).
//   * Each wavefront owns QB blocks of 32 query rows.
//   * Optionally the key range of a tile is split over several workgroups
//     (split-KV); partial (O, lse) go to a workspace and a combine kernel
//     merges them with the log-sum-exp identity.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, 64-wide wavefronts)
//   * S^T = K Q^T: A = 32 keys x 16 dims from LDS, B = 16 dims x 32 queries
//     held in registers for the whole key loop.  In the accumulator each lane
//     owns one query column and 16 keys, so the softmax row reductions over
//     keys are in-lane plus one exchange between the two half-wavefronts.
//   * K rows are fed to the A operand in a permuted order chosen so that the
//     accumulator registers of S^T are, unchanged, the B operand (P^T) of the
//     next product: lane half hf, register r holds key 16*(r/8) + 8*hf + r%8.
//   * O^T = V^T P^T: A = 32 dims x 16 keys from LDS, where V is stored in
//     "key octets" (for each group of 8 keys and each dim, the 8 values are
//     contiguous), written by an in-register 4x8 transpose during staging.
//   * Softmax in fp32 with base-2 exponent, log2(e) folded into the scale;
//     P rounded to bf16 for the second product; O kept in fp32.
#include "crattn_internal.h"
#include "rope_common.h"
#include "../../include/crattn.h"
#include "attn_loop.inc"

#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace crattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X
constexpr int kMaxSelBlocks = CRATTN_HSA_MAX_KB;  // selected blocks per query tile

struct AttnKArgs {
  const uint16_t *q;
  const uint16_t *k;
  const uint16_t *v;
  uint16_t *out;
  float *lse;
  float *ws_o;    // [splits][B][H][Lq][D]   (split > 1 only)
  float *ws_lse;  // [splits][B][H][Lq]      base-2 log-sum-exp
  int B, H;
  int64_t Lq, cap, kv_len, q_pos0, L;
  float scale_log2, inv_scale_log2;
  int64_t seg0_rows, tiles0, tiles_full, n_full, last_rows, n_tiles;
  int splits;
  // Causal-RoPE of the queries on load (the rotating instance only)
  const float2 *table;
  TabGeom tg;
  uint32_t per_frame, gw, t0, tok_off;
  // block-sparse instance: per (b, h, query tile) kb selected key blocks;
  // history blocks are ids in [0, vis_blocks) outside [own_b0, own_b1)
  const int32_t *sel;
  int kb, nbf, blk_frame, vis_blocks, own_b0, own_b1;
  // gather instance: query tiles of query clusters and their key lists
  const int32_t *q_perm;    // [B][H][Lq]
  const int32_t *gslots;    // [B][H][n_tiles][4]
  const int32_t *lists;     // [B][H][cq][list_cap]
  const int32_t *list_len;  // [B][H][cq]
  int64_t list_cap;
  int cq;
  unsigned long long *work;  // next work item (set to the grid size before launch)
  // balanced split of the dense head_dim-128 kernel: the workgroups' equal
  // ranges of all key steps; ws_o / ws_lse hold two partial slots each
  int stream;
  int64_t steps_bh, total_steps;
  unsigned *counters;  // per workgroup: parts of the tile it ends in that are done
  const int4 *order;         // work records (list, first row, rows, keys), costliest first
  const int32_t *n_real;     // their number
};

__device__ inline uint32_t pack_bf16(float lo, float hi) {
  f32x2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

// Row of the 32-key block that lane (l32) feeds into the A operand, chosen so
// that accumulator register r of lane half hf holds key 16*(r/8) + 8*hf + r%8.
// Accumulator layout of the 32x32 product: lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32.
__device__ inline int k_row_perm(int m) {
  const int r = (m >> 3) * 4 + (m & 3);
  const int hf = (m >> 2) & 1;
  return (r >> 3) * 16 + hf * 8 + (r & 7);
}

// Key (within a 32-key block) held by accumulator register r of lane half hf.
__device__ inline int acc_key(int r, int hf) { return (r >> 3) * 16 + hf * 8 + (r & 7); }


// The two lane halves of a wavefront hold the same query column (different
// keys): fold a value with its partner in the other half.
__device__ inline float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Running maximum is only raised when a new score exceeds it by more than
// 2^kRescaleLog2 (in base-2 units): until then p = 2^(s - m) stays <= 2^8,
// harmless in bf16 P and fp32 accumulators, and O is not rescaled.  The
// final division uses the same m for numerator and denominator, so the
// result is unchanged.
constexpr float kRescaleLog2 = 8.0f;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Wait until at most N vector-memory loads of this wavefront are outstanding.
// An asm with a memory clobber, so the compiler keeps LDS reads after it.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// LDS row pitches, in 16-byte cells.  Rows are padded instead of swizzled
// so that every fragment read is a per-lane base plus an immediate offset.
//  * K: CPR + 1 cells.  The QK A-operand read has 16 lanes fetch the same
//    chunk of 16 different rows; a 16-byte shift per row puts them on 16
//    distinct bank groups.
//  * V: CPR + 4 cells.  A transposed V read has 32 lanes fetch 4 consecutive
//    rows x 64 bytes; a row pitch of 64 mod 256 bytes keeps them disjoint.
// Global -> LDS copy with a wave-uniform global base and a per-lane 32-bit
// byte offset (the scalar-base form of global_load_lds_dwordx4): lane i's 16
// bytes land at LDS byte address lds_addr + 16 * i; lds_addr is wave-uniform.
// Issued through asm so the compiler does not treat the LDS write as a
// pending access to every LDS buffer (which makes it wait for the copy
// before unrelated LDS reads); completion is tracked explicitly with
// wait_vmcnt and made visible to the workgroup with a barrier.  The asm has
// no register outputs; its operands are consumed at issue.  M0 (the LDS
// base) is set inside the asm; nothing else in these kernels uses M0, so
// listing it as clobbered only tells the compiler not to assume its value
// afterwards.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_dma16_sv(const void *gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
// The same with 4 bytes per lane (lane i fills LDS bytes 4i .. 4i + 3).
__device__ inline void lds_dma4_sv(const void *gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int D>
struct Pitch {
  static constexpr int CPR = D / 8;
  static constexpr int K = CPR + 1;
  static constexpr int V = CPR + 4;
};

template <int D, int NW, int QB, int MINB, bool ROPE, bool SPARSE, bool GATHER>
__global__ void __launch_bounds__(NW * 64, MINB) attn_fwd_kernel(AttnKArgs a) {
  constexpr int kBN = 64;
  constexpr int DK = D / 16;    // k-steps of the QK product
  constexpr int DB = D / 32;    // 32-dim blocks of O
  constexpr int KB = kBN / 32;  // 32-key blocks per tile
  constexpr int CPR = D / 8;    // 16-byte chunks per key row
  constexpr int BM = NW * QB * 32;
  constexpr int NS = 4;                          // LDS ring stages
  constexpr int KP = Pitch<D>::K, VP = Pitch<D>::V;
  constexpr int K_CELLS = kBN * KP;              // 16-byte cells of one K tile (padded)
  constexpr int V_CELLS = kBN * VP;
  constexpr int K_INSTR = K_CELLS / 64;          // DMA instructions per K tile (= KP)
  constexpr int V_INSTR = V_CELLS / 64;
  constexpr int K_SLOTS = (K_INSTR + NW - 1) / NW;  // per wavefront
  constexpr int V_SLOTS = (V_INSTR + NW - 1) / NW;

  // K and V tiles of the four ring stages, row-major with padded rows,
  // 16-byte cells.  Tile t lives in stage t % 4: its K is read while tile
  // t-1 is finished, its V one tile later, and its copy is issued three
  // tiles ahead.  The copies are asm the compiler does not track, so the
  // ordering against LDS reads is explicit: wait_vmcnt + barrier.
  constexpr int STAGE_CELLS = K_CELLS + V_CELLS;
  __shared__ uint4 lds_ring[NS * STAGE_CELLS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int l32 = lane & 31;

  // ---- which (b, h, query tile, key split) this workgroup computes ----
  // Workgroups are dealt to the 8 XCDs round-robin (XCD = blockIdx % 8).
  // Renumber so that consecutive work items -- the query tiles of one head,
  // which stream the same K/V -- land on the same XCD and share its L2.
  // The gather instance is persistent instead: one workgroup per compute
  // unit takes work items in order from a device counter until none are
  // left, since its tiles differ widely in cost (list lengths, rows).
  int64_t item;
  if constexpr (GATHER) {
    item = blockIdx.x;
  } else {
    const int64_t G = gridDim.x;
    const int64_t xcd = blockIdx.x % kXcds, idx = blockIdx.x / kXcds;
    const int64_t q = G / kXcds, r = G % kXcds;
    item = xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  }
  [[maybe_unused]] __shared__ int64_t next_item;
  [[maybe_unused]] int64_t n_items = 0;
  if constexpr (GATHER)  // uniform, so the loop below has a uniform exit
    n_items = (int64_t)__builtin_amdgcn_readfirstlane(*a.n_real) * a.splits;
  for (;;) {
  if constexpr (GATHER)
    if (item >= n_items) break;
  int64_t bid = item;
  const int split = (int)(bid % a.splits);
  bid /= a.splits;
  [[maybe_unused]] int4 rec = make_int4(0, 0, 0, 0);
  if constexpr (GATHER) {  // the work record: (b, h, query cluster), rows, keys
    const int4 rv = a.order[bid];
    rec = make_int4(__builtin_amdgcn_readfirstlane(rv.x), __builtin_amdgcn_readfirstlane(rv.y),
                    __builtin_amdgcn_readfirstlane(rv.z), __builtin_amdgcn_readfirstlane(rv.w));
    bid = (rec.x / a.cq) * a.n_tiles;
  }
  const int64_t tile = bid % a.n_tiles;
  bid /= a.n_tiles;
  const int h = (int)(bid % a.H);
  const int b = (int)(bid / a.H);

  // Gather instance: the work item is query tile `tile` of the head's
  // slot table: reordered query positions [first, first + rows) of one
  // query cluster, attending to the key rows listed for that cluster.  A
  // slot with no rows (or out of range) has nothing to do.
  int64_t row0, nrows, q_chunk = 0;
  int limit;
  [[maybe_unused]] const int32_t *g_list = nullptr;
  [[maybe_unused]] const int32_t *g_qperm = nullptr;
  if constexpr (GATHER) {
    static_assert(BM == CRATTN_SVG2_QTILE, "a query tile of the plan is one workgroup's rows");
    // (gather_order_kernel checked the slot and clamped the list length)
    const int64_t bhi = (int64_t)b * a.H + h;
    row0 = rec.y;
    nrows = rec.z;
    limit = rec.w;
    g_list = a.lists + (int64_t)rec.x * a.list_cap;
    g_qperm = a.q_perm + bhi * a.Lq;
  } else {
  int64_t seg, t_in, seg_row0, seg_rows;
  if (tile < a.tiles0) {
    seg = 0;
    t_in = tile;
    seg_row0 = 0;
    seg_rows = a.seg0_rows;
  } else {
    const int64_t u = tile - a.tiles0;
    if (u < a.n_full * a.tiles_full) {
      const int64_t s = u / a.tiles_full;
      t_in = u - s * a.tiles_full;
      seg = 1 + s;
      seg_row0 = a.seg0_rows + s * a.L;
      seg_rows = a.L;
    } else {
      t_in = u - a.n_full * a.tiles_full;
      seg = 1 + a.n_full;
      seg_row0 = a.seg0_rows + a.n_full * a.L;
      seg_rows = a.last_rows;
    }
  }
  row0 = seg_row0 + t_in * BM;
  nrows = min((int64_t)BM, seg_rows - t_in * BM);
  q_chunk = a.q_pos0 / a.L + seg;
  // keys of one head fit 32-bit indices (the front end bounds cap * D)
  limit = (int)min(a.kv_len, (q_chunk + 1) * a.L);
  }
  int nkt = (limit + kBN - 1) / kBN;

  // ---- block-sparse key list: the tiles of the own chunk, then the
  // selected history blocks as (first row, end row), compacted in list
  // order.  Ids that are not history blocks (negative, past the visible
  // frames, or in the own chunk) are dropped, so nothing outside the own
  // chunk and the history is ever read and no tile is empty.  The ids are
  // taken a workgroup's width at a time. ----
  [[maybe_unused]] int own0 = 0, n_own = 0;
  [[maybe_unused]] int2 *sp_tiles = nullptr;
  if constexpr (SPARSE) {
    static_assert(BM == CRATTN_HSA_QBLOCK, "one selection row per query tile");
    static_assert(kBN == CRATTN_HSA_KBLOCK, "a selected block is one key tile");
    __shared__ int2 sp_buf[kMaxSelBlocks];
    __shared__ int sp_count[NW];
    sp_tiles = sp_buf;
    own0 = (int)(q_chunk * a.L);
    n_own = (limit - own0 + kBN - 1) / kBN;
    const int32_t *sl = a.sel + (((int64_t)b * a.H + h) * a.n_tiles + tile) * a.kb;
    int base = 0;
    for (int i0 = 0; i0 < a.kb; i0 += NW * 64) {
      const int i = i0 + tid;
      const int id = i < a.kb ? sl[i] : -1;
      const bool v = id >= 0 && id < a.vis_blocks && (id < a.own_b0 || id >= a.own_b1);
      const uint64_t bal = __builtin_amdgcn_ballot_w64(v);
      const int before = __builtin_popcountll(bal & ((uint64_t(1) << lane) - 1));
      if (lane == 0) sp_count[wave] = __builtin_popcountll(bal);
      __syncthreads();
      int off = base, tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        off += w < wave ? sp_count[w] : 0;
        tot += sp_count[w];
      }
      if (v) {
        const int f = id / a.nbf, j = id - f * a.nbf;
        const int start = f * a.blk_frame + j * kBN;
        sp_buf[off + before] = make_int2(start, start + min(kBN, a.blk_frame - j * kBN));
      }
      base += tot;
      __syncthreads();
    }
    nkt = n_own + base;
  }
  // first key row and end of the visible range of tile kt (the visible
  // rows of a tile are [key0, min(key0 + kBN, lim)))
  auto tile_key0 = [&](int kt) -> int {
    if constexpr (SPARSE)
      return kt < n_own ? own0 + kt * kBN
                        : __builtin_amdgcn_readfirstlane(sp_tiles[kt - n_own].x);
    else
      return kt * kBN;
  };
  auto tile_lim = [&](int kt) -> int {
    if constexpr (SPARSE)
      return kt < n_own ? limit : __builtin_amdgcn_readfirstlane(sp_tiles[kt - n_own].y);
    else
      return limit;
  };
  const int kt_begin = split * nkt / a.splits;
  const int kt_end = (split + 1) * nkt / a.splits;

  const int64_t head_off = ((int64_t)b * a.H + h) * a.cap * D;
  const uint16_t *__restrict__ kh = a.k + head_off;
  const uint16_t *__restrict__ vh = a.v + head_off;

  // ---- this wavefront's queries, as B operands (16 dims x 32 queries) ----
  const int64_t wrow0 = row0 + (int64_t)wave * QB * 32;
  const bool active = (int64_t)wave * QB * 32 < nrows;
  bf16x8_t qf[QB][DK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t row = wrow0 + qb * 32 + l32;
    const bool ok = row < row0 + nrows;
    int64_t mrow = row;  // the query's row in memory
    if constexpr (GATHER) mrow = ok ? min((uint32_t)g_qperm[row], (uint32_t)(a.Lq - 1)) : 0;
    const uint16_t *qp = a.q + (((int64_t)b * a.Lq + mrow) * a.H + h) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (ok) x = *reinterpret_cast<const uint4 *>(qp + ks * 16);
      qf[qb][ks] = __builtin_bit_cast(bf16x8_t, x);
    }
    if constexpr (ROPE) {
      // Causal-RoPE of the query on load.  Row `row` of the call is token
      // tok_off + row of its chunk (the rows of a rotating call lie in one
      // chunk).  The lane's 8 features of sub-step ks are pairs
      // 8 ks + 4 hf + e.  Their (cos, sin) are gathered in one batch from
      // per-lane pointers into the three axis sections of the table (pair q
      // of axis a is entry base_a + q), then each pair is rotated with the
      // same fp32 arithmetic and single bf16 rounding as the RoPE/append pass.
      constexpr int HT = (D - 4 * (D / 6)) / 2;  // pairs of the t group
      constexpr int HH = D / 6;                  // pairs of the h (= w) group
      const Pos p = decode_pos(a.tok_off + (uint32_t)min(row, a.Lq - 1), a.per_frame, a.gw, a.t0);
      const float2 *ax[3] = {a.table + p.t * HT + 4 * hf,
                             a.table + a.tg.base_h + p.h * HH - HT + 4 * hf,
                             a.table + a.tg.base_w + p.w * HH - HT - HH + 4 * hf};
      auto axis = [](int q) { return q < HT ? 0 : q < HT + HH ? 1 : 2; };
      float2 cs[DK][4];
#pragma unroll
      for (int ks = 0; ks < DK; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q0 = ks * 8 + e;  // pair of the low half-wave; the high one is q0 + 4
          const int a0 = axis(q0), a1 = axis(q0 + 4);
          const float2 *ptr = a0 == a1 ? ax[a0] : (hf ? ax[a1] : ax[a0]);
          cs[ks][e] = ptr[q0];
        }
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const uint4 x = __builtin_bit_cast(uint4, qf[qb][ks]);
        uint32_t wv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 r = rotate_pair(__uint_as_float(wv[e] << 16),
                                       __uint_as_float(wv[e] & 0xffff0000u), cs[ks][e]);
          wv[e] = pack_bf16(r.x, r.y);
        }
        qf[qb][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(wv[0], wv[1], wv[2], wv[3]));
      }
    }
  }
  // Settle the Q loads here (vmcnt 0; expcnt and lgkmcnt not waited on), in
  // a form the compiler tracks, so it does not re-wait inside the key loop
  // where the LDS copies of later tiles are in flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  f32x16_t o[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][qb][r] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  const int kperm = k_row_perm(l32);

  // ---- global -> LDS DMA of one K/V tile into a ring stage ----
  // DMA instruction j of a tile fills padded cells [64j, 64j + 64); lane i
  // writes cell 64j + i, so each lane fetches the global 16-byte chunk of its
  // cell's (row, column); a lane on a pad cell fetches its row's first chunk
  // (a line the same instruction reads anyway) into that never-read cell, so
  // no lane is masked off.  Instruction j is issued by wavefront j % NW.  The
  // per-lane byte offsets within a tile are fixed; only the scalar tile base
  // and the LDS address move.  In the tile holding `limit`, keys at or past
  // it fetch the last visible key instead: their scores are masked to -inf
  // (p = 0) and the copied values are finite whenever the visible ones are,
  // so nothing past the visible range is ever read.
  auto cell_off = [&](int cell, int pitch) -> uint32_t {
    const int row = cell / pitch;
    const int c = cell - row * pitch;
    return (uint32_t)(row * D + (c < CPR ? c * 8 : 0)) * 2u;
  };
  constexpr uint32_t kRowBytes = D * 2;
  uint32_t dma_k_off[K_SLOTS], dma_v_off[V_SLOTS];
#pragma unroll
  for (int n = 0; n < K_SLOTS; ++n) dma_k_off[n] = cell_off((wave + n * NW) * 64 + lane, KP);
#pragma unroll
  for (int n = 0; n < V_SLOTS; ++n) dma_v_off[n] = cell_off((wave + n * NW) * 64 + lane, VP);
  // In the edge tile, rows past the last visible key re-read that key.
  auto clamp_off = [&](uint32_t off, int last) -> uint32_t {
    const int r = (int)(off / kRowBytes);
    return off - (uint32_t)(r - min(r, last)) * kRowBytes;
  };
  // LDS byte address of the ring (one generic-to-LDS conversion)
  typedef __attribute__((address_space(3))) char lds_char_t;
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(lds_char_t *)reinterpret_cast<char *>(lds_ring));
  // (slots n with (n + 1) * NW <= instructions exist for every wavefront:
  // the test is decided at compile time)
  // Gather instance: the rows of tile kt are list entries 64 kt .. 64 kt + 63,
  // whose key rows sit in LDS ring entry kt mod 8 (copied there earlier,
  // see the key loop).  A lane's cell keeps its row-in-tile and column; the
  // key row comes from the ring, clamped to the head's rows.  Entries past
  // the list's end re-read its last key (masked, as in the edge tile).
  [[maybe_unused]] int *g_idx = nullptr;
  [[maybe_unused]] uint32_t g_idx_lds = 0;
  if constexpr (GATHER) {
    __shared__ int idx_ring[8 * kBN];
    g_idx = idx_ring;
    g_idx_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_char_t *)reinterpret_cast<char *>(idx_ring));
  }
  // The byte offsets of one gathered tile are read from the ring a step
  // before its copy is issued (gather_offsets), so the LDS reads do not sit
  // between the barrier and the copy.
  [[maybe_unused]] uint32_t g_off[K_SLOTS + V_SLOTS];
#pragma unroll
  for (int n = 0; n < K_SLOTS + V_SLOTS; ++n) g_off[n] = 0;
  [[maybe_unused]] auto gather_offsets = [&](int kt) {
    const int last = min(kBN, limit - kt * kBN) - 1;
    const int *ir = g_idx + (kt & 7) * kBN;
    const uint32_t rows_max = (uint32_t)a.cap - 1u;
#pragma unroll
    for (int n = 0; n < K_SLOTS; ++n) {
      const int r = min((int)(dma_k_off[n] / kRowBytes), last);
      g_off[n] = min((uint32_t)ir[r], rows_max) * kRowBytes + dma_k_off[n] % kRowBytes;
    }
#pragma unroll
    for (int n = 0; n < V_SLOTS; ++n) {
      const int r = min((int)(dma_v_off[n] / kRowBytes), last);
      g_off[K_SLOTS + n] = min((uint32_t)ir[r], rows_max) * kRowBytes + dma_v_off[n] % kRowBytes;
    }
  };
  auto dma = [&](int kt, int stage) {
    const uint32_t kdst = ring_lds + (uint32_t)stage * (STAGE_CELLS * 16);
    const uint32_t vdst = kdst + K_CELLS * 16;
    if constexpr (GATHER) {
      // the offsets of tile kt are in g_off
#pragma unroll
      for (int n = 0; n < K_SLOTS; ++n) {
        const int j = wave + n * NW;
        if ((n + 1) * NW <= K_INSTR || j < K_INSTR) lds_dma16_sv(kh, g_off[n], kdst + j * 1024);
      }
#pragma unroll
      for (int n = 0; n < V_SLOTS; ++n) {
        const int j = wave + n * NW;
        if ((n + 1) * NW <= V_INSTR || j < V_INSTR)
          lds_dma16_sv(vh, g_off[K_SLOTS + n], vdst + j * 1024);
      }
      return;
    }
    const int key0 = tile_key0(kt);
    const int lim = tile_lim(kt);
    const uint16_t *kb = kh + key0 * D;
    const uint16_t *vb = vh + key0 * D;
    if (key0 + kBN <= lim) {
#pragma unroll
      for (int n = 0; n < K_SLOTS; ++n) {
        const int j = wave + n * NW;
        if ((n + 1) * NW <= K_INSTR || j < K_INSTR) lds_dma16_sv(kb, dma_k_off[n], kdst + j * 1024);
      }
#pragma unroll
      for (int n = 0; n < V_SLOTS; ++n) {
        const int j = wave + n * NW;
        if ((n + 1) * NW <= V_INSTR || j < V_INSTR) lds_dma16_sv(vb, dma_v_off[n], vdst + j * 1024);
      }
    } else {
      const int last = lim - 1 - key0;
#pragma unroll
      for (int n = 0; n < K_SLOTS; ++n) {
        const int j = wave + n * NW;
        if ((n + 1) * NW <= K_INSTR || j < K_INSTR) lds_dma16_sv(kb, clamp_off(dma_k_off[n], last), kdst + j * 1024);
      }
#pragma unroll
      for (int n = 0; n < V_SLOTS; ++n) {
        const int j = wave + n * NW;
        if ((n + 1) * NW <= V_INSTR || j < V_INSTR) lds_dma16_sv(vb, clamp_off(dma_v_off[n], last), vdst + j * 1024);
      }
    }
  };
  // Fewest LDS-DMA instructions any wavefront issues per tile.  Loads retire
  // in order, so "at most kDmaMin outstanding" after a later tile was issued
  // implies every earlier tile's copies are complete.
  constexpr int kDmaMin = K_INSTR / NW + V_INSTR / NW;
  static_assert(kDmaMin >= 1 && 2 * kDmaMin < 16, "vmcnt wait range");

  // V^T A-operand lane geometry for the transposed reads: a 16-lane block
  // reads 4 key rows x 16 dims; lane j of the block points at 4 dims of row
  // j/4, and receives 4 keys of dim (block's first dim) + j.
  const int vblk = l32 >> 4;         // which 16-dim half of the 32-dim block
  const int vj = lane & 15;
  const int v_row_in = vj >> 2;      // key row within the 4-row group
  const int v_dim = vblk * 16 + 4 * (vj & 3);

  // ---- operand fragments from a ring stage ----
  // K (A operand of S^T = K Q^T) for QK MFMA i of a tile: k-step i / KB,
  // 32-key block i % KB (consecutive MFMAs alternate accumulators).
  auto k_frag = [&](int stage, int i) -> bf16x8_t {
    const uint4 *__restrict__ kt_lds = lds_ring + stage * STAGE_CELLS;
    const int ks = i / KB, kb = i % KB;
    return __builtin_bit_cast(bf16x8_t, kt_lds[(kb * 32 + kperm) * KP + 2 * ks + hf]);
  };
  // V^T (A operand of O^T += V^T P^T) for PV MFMA i of 32-key block kb:
  // key half h2 = i / DB, dims db = i % DB; keys kb*32 + h2*16 + 8*hf + 0..7
  // arrive as two transposed 4-key reads.
  auto v_frag = [&](int stage, int kb, int i) -> bf16x8_t {
    const char *__restrict__ vt_lds =
        reinterpret_cast<const char *>(lds_ring + stage * STAGE_CELLS + K_CELLS);
    const int h2 = i / DB, db = i % DB;
    const int vr0 = kb * 32 + h2 * 16 + 8 * hf + v_row_in;
    const int dbyte = (db * 32 + v_dim) * 2;  // byte offset of 4 dims within a row
    const i16x4_t lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vt_lds + vr0 * (VP * 16) + dbyte));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t *)(vt_lds + (vr0 + 4) * (VP * 16) + dbyte));
    const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8_t, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
  };
  // ---- S^T = K Q^T of one whole tile (prologue) ----
  auto qk = [&](int stage, f32x16_t (&sc)[KB][QB]) {
#pragma unroll
    for (int i = 0; i < KB * DK; ++i) {
      const bf16x8_t kf = k_frag(stage, i);
      const int ks = i / KB, kb = i % KB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (ks == 0) {
          f32x16_t z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          sc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], z, 0, 0, 0);
        } else {
          sc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], sc[kb][qb], 0, 0, 0);
        }
      }
    }
  };
  // ---- softmax, part 1: row maximum of a tile (no mask) ----
  auto row_max = [&](const f32x16_t (&sc)[KB][QB], float (&mx)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, sc[kb][qb][r]);
      mx[qb] = half_swap_max(m);
    }
  };
  // ---- softmax, part 2 (branchy, after the tile's products): edge mask,
  // running max, lazy rescale of the row sums and of O ----
  auto softmax_fix = [&](f32x16_t (&sc)[KB][QB], int kt, float (&mx)[QB]) {
    const int key0 = tile_key0(kt);
    const int lim = tile_lim(kt);
    if (key0 + kBN > lim) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool dead = key0 + kb * 32 + acc_key(r, hf) >= lim;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if (dead) sc[kb][qb][r] = -INFINITY;
        }
      row_max(sc, mx);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_cand = mx[qb] * a.scale_log2;
      const bool need = m_cand > m_run[qb] + kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = need ? m_cand : m_run[qb];
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
      }
    }
  };
  // ---- softmax, part 3: p = 2^(s*c - m) for the two keys of packed pair j
  // (0..15) of a tile, rounded to bf16 for the P.V product; the row sums add
  // the fp32 p in two chains.
  auto exp_pair = [&](const f32x16_t (&sc)[KB][QB], uint32_t (&pk)[QB][16],
                      float (&rs)[QB][2], int j) {
    const int kb = j >> 3, r = ((j >> 2) & 1) * 8 + 2 * (j & 3);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kb][qb][r], a.scale_log2, -m_run[qb]));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kb][qb][r + 1], a.scale_log2, -m_run[qb]));
      pk[qb][j] = pack_bf16(p0, p1);
      rs[qb][j & 1] += p0 + p1;
    }
  };
  // P^T B operand of 16 keys (chunk c = 2 * kb + h2) from the packed pairs
  auto p_frag = [&](const uint32_t (&pk)[QB][16], int qb, int c) -> bf16x8_t {
    return __builtin_bit_cast(bf16x8_t,
                              make_uint4(pk[qb][4 * c], pk[qb][4 * c + 1], pk[qb][4 * c + 2],
                                         pk[qb][4 * c + 3]));
  };

  // ---- the key loop, software-pipelined across tiles ----
  // Step for tile kt: wait for tile kt+1's copy, barrier, issue the copy of
  // tile kt+3, then three MFMA streams, each interleaved one MFMA at a time
  // with a share of the vector work:
  //   S(kt+1) = K Q^T        (16 MFMAs) with p of S(kt), pairs 0..11
  //   O += P V, keys 0..31   ( 8 MFMAs) with p of S(kt), pairs 12..15
  //   O += P V, keys 32..63  ( 8 MFMAs) with the row maximum of S(kt+1)
  // and finally, outside the MFMA streams, the edge mask and the (rare)
  // rescale for tile kt+1.  Operand fragments are read from LDS two MFMAs
  // ahead.  A scheduling barrier after each slot keeps MFMAs and vector
  // instructions in this order while letting LDS reads and scalar work move.
  constexpr int kSlotMask = 0x0100 | 0x0004;  // DS reads, SALU may cross
  f32x16_t sbuf[2][KB][QB];
  if constexpr (GATHER) {
    // key rows of the first five tiles; later ones are copied five tiles
    // ahead inside the loop
    for (int e = tid; e < 5 * kBN; e += NW * 64) {
      const int t = kt_begin + e / kBN;
      if (t < kt_end) g_idx[(t & 7) * kBN + e % kBN] = g_list[(int64_t)t * kBN + e % kBN];
    }
    __syncthreads();
  }
  if constexpr (GATHER) {
    for (int t = 0; t < 3 && kt_begin + t < kt_end; ++t) {
      gather_offsets(kt_begin + t);
      dma(kt_begin + t, t);
    }
    if (kt_begin + 3 < kt_end) gather_offsets(kt_begin + 3);
  } else {
    if (kt_begin < kt_end) dma(kt_begin, 0);
    if (kt_begin + 1 < kt_end) dma(kt_begin + 1, 1);
    if (kt_begin + 2 < kt_end) dma(kt_begin + 2, 2);
  }
  if (kt_begin + 2 < kt_end)
    wait_vmcnt<2 * kDmaMin>();
  else if (kt_begin + 1 < kt_end)
    wait_vmcnt<kDmaMin>();
  else
    wait_vmcnt<0>();
  __syncthreads();
  if (active && kt_begin < kt_end) {
    qk(0, sbuf[0]);
    float mx[QB];
    row_max(sbuf[0], mx);
    softmax_fix(sbuf[0], kt_begin, mx);
  }

  auto step = [&](int kt, auto P) {
    constexpr int par = decltype(P)::value;
    constexpr int NQK = KB * DK;  // 16 (D = 128) or 8 (D = 64)
    constexpr int NPV = 2 * DB;   // per 32-key block: 8 or 4
    constexpr int NPAIR = 16;     // packed p pairs per tile
    constexpr int NA = NPAIR * 3 / 4;  // pairs done during S(kt+1)
    const int stage = (kt - kt_begin) & (NS - 1);
    const int st1 = (stage + 1) & (NS - 1);
    const bool more = kt + 1 < kt_end;
    if (more) {
      // tile kt+1 has landed once at most tile kt+2's copies are pending
      if (kt + 2 < kt_end)
        wait_vmcnt<kDmaMin>();
      else
        wait_vmcnt<0>();
      // every wavefront now sees tile kt+1 and has finished tile kt-1, whose
      // stage the copy of tile kt+3 refills
      __syncthreads();
      if constexpr (GATHER) {
        // Key rows of tile kt+5, issued before tile kt+3's copies: the wait
        // for tile kt+3 (two steps on) then covers them too, so they are in
        // LDS, behind a barrier, when tile kt+5's copy reads them.  Ring
        // entry (kt+5) mod 8 last served tile kt-3, copied three steps ago.
        if (wave == NW - 1 && kt + 5 < kt_end)
          lds_dma4_sv(g_list + (int64_t)(kt + 5) * kBN, (uint32_t)lane * 4u,
                      __builtin_amdgcn_readfirstlane(g_idx_lds +
                                                     (uint32_t)((kt + 5) & 7) * (kBN * 4)));
      }
      if (kt + 3 < kt_end) dma(kt + 3, (stage + 3) & (NS - 1));
      // (gather) tile kt+4's key rows arrived with the copies of tile kt+2
      // or earlier and are behind this barrier
      if constexpr (GATHER)
        if (kt + 4 < kt_end) gather_offsets(kt + 4);
    }
    if (!active) return;
    f32x16_t (&cur)[KB][QB] = sbuf[par];
    f32x16_t (&nxt)[KB][QB] = sbuf[par ^ 1];
    uint32_t pk[QB][16];
    float rs[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) rs[qb][0] = rs[qb][1] = 0.f;

    // S(kt+1), unconditionally so that the stream keeps its shape; on the
    // last tile it reads a stage no copy is writing (stale, in bounds) and
    // the result is never used.
    bf16x8_t kf[NQK];
    kf[0] = k_frag(st1, 0);
    kf[1] = k_frag(st1, 1);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      if (i + 2 < NQK) kf[i + 2] = k_frag(st1, i + 2);
      const int ks = i / KB, kb = i % KB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (ks == 0) {
          f32x16_t z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          nxt[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[qb][ks], z, 0, 0, 0);
        } else {
          nxt[kb][qb] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[qb][ks], nxt[kb][qb], 0, 0, 0);
        }
      }
      // NA pairs spread over NQK slots
      if (i * NA / NQK != (i + 1) * NA / NQK) exp_pair(cur, pk, rs, i * NA / NQK);
      if ((i + 1) * NA / NQK - i * NA / NQK == 2) exp_pair(cur, pk, rs, i * NA / NQK + 1);
      __builtin_amdgcn_sched_barrier(kSlotMask);
    }

    // O += P V for keys 0..31 with the last quarter of p, then for keys
    // 32..63 with the row maximum of S(kt+1)
    float mp[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mp[qb] = -INFINITY;
    bf16x8_t vf[2 * NPV];
    vf[0] = v_frag(stage, 0, 0);
    vf[1] = v_frag(stage, 0, 1);
#pragma unroll
    for (int i = 0; i < 2 * NPV; ++i) {
      if (i + 2 < 2 * NPV) vf[i + 2] = v_frag(stage, (i + 2) / NPV, (i + 2) % NPV);
      const int kb = i / NPV, h2 = (i % NPV) / DB, db = i % DB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], p_frag(pk, qb, 2 * kb + h2),
                                                            o[db][qb], 0, 0, 0);
      if (kb == 0) {
        // pairs NA..15 over the first block's slots
        const int j0 = NA + i * (NPAIR - NA) / NPV, j1 = NA + (i + 1) * (NPAIR - NA) / NPV;
#pragma unroll
        for (int j = j0; j < j1; ++j) exp_pair(cur, pk, rs, j);
      } else {
        // a share of the scores of S(kt+1) into the running row maximum
        constexpr int per = KB * 16 / NPV;
#pragma unroll
        for (int v = 0; v < per; ++v) {
          const int idx = (i - NPV) * per + v;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) mp[qb] = fmaxf(mp[qb], nxt[idx / 16][qb][idx % 16]);
        }
      }
      __builtin_amdgcn_sched_barrier(kSlotMask);
    }
    float mx[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      mx[qb] = half_swap_max(mp[qb]);
      l_run[qb] += rs[qb][0] + rs[qb][1];
    }
    if (more) softmax_fix(nxt, kt + 1, mx);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  for (int kt = kt_begin; kt < kt_end;) {
    step(kt++, P0{});
    if (kt >= kt_end) break;
    step(kt++, P1{});
  }

  // ---- epilogue: normalise and store ----
#pragma unroll
  for (int qb = 0; qb < QB && active; ++qb) {
    const float lt = half_swap_sum(l_run[qb]);
    const int64_t row = wrow0 + qb * 32 + l32;
    if (row >= row0 + nrows) continue;
    int64_t mrow = row;
    if constexpr (GATHER) mrow = min((uint32_t)g_qperm[row], (uint32_t)(a.Lq - 1));
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const float lse2 = lt > 0.f ? m_run[qb] + __log2f(lt) : -INFINITY;
    if (a.splits == 1) {
      uint16_t *op = a.out + (((int64_t)b * a.Lq + mrow) * a.H + h) * D + hf * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x16_t &acc = o[db][qb];
          uint2 w;
          w.x = pack_bf16(acc[i4 * 4 + 0] * inv, acc[i4 * 4 + 1] * inv);
          w.y = pack_bf16(acc[i4 * 4 + 2] * inv, acc[i4 * 4 + 3] * inv);
          *reinterpret_cast<uint2 *>(op + db * 32 + i4 * 8) = w;
        }
      if (hf == 0 && a.lse != nullptr) a.lse[((int64_t)b * a.H + h) * a.Lq + mrow] = lse2 * kLn2;
    } else {
      const int64_t prow = (((int64_t)split * a.B + b) * a.H + h) * a.Lq + mrow;
      float *op = a.ws_o + prow * D + hf * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x16_t &acc = o[db][qb];
          *reinterpret_cast<float4 *>(op + db * 32 + i4 * 8) =
              make_float4(acc[i4 * 4 + 0] * inv, acc[i4 * 4 + 1] * inv, acc[i4 * 4 + 2] * inv,
                          acc[i4 * 4 + 3] * inv);
        }
      if (hf == 0) a.ws_lse[prow] = lse2;
    }
  }
  if constexpr (!GATHER) break;
  // every wavefront is done with this item's LDS before the next one's
  // copies start
  __syncthreads();
  if (tid == 0) next_item = (int64_t)atomicAdd(a.work, 1ull);
  __syncthreads();
  // (item < 2^31: the front end bounds the work count)
  item = (int64_t)__builtin_amdgcn_readfirstlane((int)min(next_item, (int64_t)0x7fffffff));
  }
}


// ---------------------------------------------------------------------------
// Dense chunk-causal attention, head_dim 128, with the key loop written in
// CDNA4 assembly (attn_loop.inc, generated by gen_attn_loop.py).
//
// A workgroup of 4 wavefronts (one per SIMD) owns 256 query rows of one
// (batch, head), each wavefront 64 rows as two 32-query blocks, so each K or
// V fragment read from LDS feeds two matrix products.  With 64 query rows a
// wavefront needs O (128 fp32 registers) and Q (64) beside the scores: O and
// Q stay in the accumulation registers, where the matrix cores read and
// write them directly, and the loop's registers are fixed by hand (the
// compiler's own allocation of this shape spills).  The loop follows the
// same arithmetic as attn_fwd_kernel (online softmax in base 2 with a lazily
// raised maximum, P rounded to bf16, O in fp32) except that the row sums
// add the bf16-rounded probabilities, the values the P.V product uses.
//
// This function does what the compiler is good at: it decodes the work
// item, loads (and for ROPE rotates) the queries, computes the lane's copy
// offsets and LDS fragment addresses, runs the loop, then normalises and
// stores.
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
typedef float f32x32_t __attribute__((ext_vector_type(32)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#define CRT_D(p, t) \
  p #t "0", p #t "1", p #t "2", p #t "3", p #t "4", p #t "5", p #t "6", p #t "7", p #t "8", p #t "9"

// One query tile of the dense kernel: its rows and key range, and (balanced
// split) where its key steps sit in the (batch, head, tile, key tile) order.
struct FwdTile {
  int b, h;
  int64_t row0, nrows;  // query rows [row0, row0 + nrows) of (b, h)
  int limit, nkt;       // visible keys and 64-key tiles
  int64_t pos0;         // linear index of the tile's first key step
};

// Query rows of segment s (chunk q_pos0 / L + s) start at seg_row0 and
// number seg_rows; its tiles see min(kv_len, (chunk + 1) L) keys.
__device__ inline int64_t fwd_seg_tiles(const AttnKArgs &a, int64_t s) {
  return s == 0 ? a.tiles0
       : s <= a.n_full ? a.tiles_full
                       : a.n_tiles - a.tiles0 - a.n_full * a.tiles_full;
}
__device__ inline int fwd_seg_nkt(const AttnKArgs &a, int64_t s) {
  const int64_t limit = min(a.kv_len, (a.q_pos0 / a.L + s + 1) * a.L);
  return (int)((limit + 63) / 64);
}

__device__ inline FwdTile fwd_tile_in(const AttnKArgs &a, int64_t bh, int64_t s, int64_t t_in) {
  FwdTile t;
  t.b = (int)(bh / a.H);
  t.h = (int)(bh % a.H);
  const int64_t seg_row0 = s == 0 ? 0 : a.seg0_rows + (s - 1) * a.L;
  const int64_t seg_rows = s == 0 ? a.seg0_rows : s <= a.n_full ? a.L : a.last_rows;
  t.row0 = seg_row0 + t_in * 256;
  t.nrows = min((int64_t)256, seg_rows - t_in * 256);
  t.limit = (int)min(a.kv_len, (a.q_pos0 / a.L + s + 1) * a.L);
  t.nkt = (t.limit + 63) / 64;
  t.pos0 = 0;
  return t;
}

// Tile g (of B * H * n_tiles): the unsplit launch, one tile per workgroup.
__device__ inline FwdTile fwd_tile(const AttnKArgs &a, int64_t g) {
  const int64_t bh = g / a.n_tiles, tile = g % a.n_tiles;
  int64_t s, t_in;
  if (tile < a.tiles0) {
    s = 0;
    t_in = tile;
  } else {
    const int64_t u = tile - a.tiles0;
    s = 1 + min(u / a.tiles_full, a.n_full);
    t_in = u - (s - 1) * a.tiles_full;
  }
  return fwd_tile_in(a, bh, s, t_in);
}

// The tile holding linear key step x (balanced split).
__device__ inline FwdTile fwd_locate(const AttnKArgs &a, int64_t x) {
  const int64_t bh = x / a.steps_bh;
  int64_t r = x - bh * a.steps_bh, base = bh * a.steps_bh;
  const int64_t n_seg = 1 + a.n_full + (a.last_rows > 0 ? 1 : 0);
  int64_t s = 0;
  for (;; ++s) {
    const int64_t cnt = fwd_seg_tiles(a, s) * fwd_seg_nkt(a, s);
    if (r < cnt || s == n_seg - 1) break;
    r -= cnt;
    base += cnt;
  }
  const int nkt = fwd_seg_nkt(a, s);
  const int64_t t_in = r / nkt;
  FwdTile t = fwd_tile_in(a, bh, s, t_in);
  t.pos0 = base + t_in * nkt;
  return t;
}

// Largest key-tile table of the block-sparse instance (own chunk tiles,
// selected blocks, four padding entries): its LDS beside the ring.
constexpr int kListMax = 1500;

template <bool ROPE, bool LIST, bool GATHER = false>
__global__ void __launch_bounds__(256, 1) attn_fwd64_kernel(AttnKArgs a) {
  static_assert(!(GATHER && (ROPE || LIST)), "one instance kind at a time");
  constexpr int D = 128, kBN = 64;
  constexpr int DK = D / 16, DB = D / 32;
  constexpr int KP = Pitch<D>::K, VP = Pitch<D>::V;
  constexpr int K_CELLS = kBN * KP, V_CELLS = kBN * VP;
  constexpr int STAGE_CELLS = K_CELLS + V_CELLS;
  constexpr int STAGE_BYTES = STAGE_CELLS * 16;
  static_assert(STAGE_BYTES == 37888 && K_CELLS * 16 == 17408, "layout the loop assumes");
  __shared__ uint4 lds_ring[4 * STAGE_CELLS];
  __shared__ int sh_count;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int l32 = lane & 31;

  // ---- work: consecutive work indices on one XCD (they share K/V in its L2)
  int64_t w;
  {
    const int64_t G = gridDim.x;
    const int64_t xcd = blockIdx.x % kXcds, idx = blockIdx.x / kXcds;
    const int64_t q = G / kXcds, r = G % kXcds;
    w = xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  }
  // Balanced split: key steps [s_lo, s_hi) of the linear order.  Its tiles
  // are taken last to first: the last one starts at key tile 0, as do the
  // other workgroups' first tiles, so the workgroups of one head walk the
  // keys nearly in step.
  const int64_t G = gridDim.x, T = a.total_steps;
  const int64_t s_lo = a.stream ? w * T / G : 0, s_hi = a.stream ? (w + 1) * T / G : 0;
  auto part_of = [&](int64_t x) { return ((x + 1) * G - 1) / T; };  // workgroup holding step x

  // ---- LDS addresses: ring base, per-lane fragment bases per stage ----
  typedef __attribute__((address_space(3))) char lds_char_t;
  const uint32_t ring = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(lds_char_t *)reinterpret_cast<char *>(lds_ring));
  // LDS: a ring of 4 K stages, then a ring of 4 V stages
  u32x8_t bases;
  {
    const uint32_t kb0 = ring + (uint32_t)((k_row_perm(l32) * KP + hf) * 16);
    const int vj = lane & 15;
    const int v_dim = (l32 >> 4) * 16 + 4 * (vj & 3);
    const uint32_t vb0 =
        ring + 4 * K_CELLS * 16 + (uint32_t)((8 * hf + (vj >> 2)) * VP * 16 + v_dim * 2);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bases[s] = kb0 + s * K_CELLS * 16;
      bases[4 + s] = vb0 + s * V_CELLS * 16;
    }
  }
  const uint32_t kh8 = 8u * (uint32_t)hf;
  const uint32_t wb = ring + (uint32_t)wave * 1024u;
  const uint32_t k5 = (uint32_t)((wave == 0 ? 16 : wave + 12) - wave) * 1024u;
  const float sc = a.scale_log2;

  int64_t x_end = s_hi;
  // Gather instance: persistent, one workgroup per compute unit taking work
  // items (a query tile of one query cluster, one key split of its list) in
  // the cost order of gather_order_kernel from a device counter.
  [[maybe_unused]] __shared__ int64_t next_item;
  [[maybe_unused]] int64_t n_items = 0, item = blockIdx.x;
  [[maybe_unused]] const int32_t *g_list = nullptr;
  [[maybe_unused]] const int32_t *g_qperm = nullptr;
  [[maybe_unused]] int g_split = 0;
  if constexpr (GATHER)
    n_items = (int64_t)__builtin_amdgcn_readfirstlane(*a.n_real) * a.splits;
  for (bool first = true;; first = false) {
    FwdTile ti;
    int k0, k1;
    if constexpr (GATHER) {
      if (!first) {
        // every wavefront is done with this item's LDS (and with next_item)
        // before the next item is taken (taking it earlier, to hide the
        // counter's latency, holds cheap items back from idle workgroups at
        // the end: measured slower)
        __syncthreads();
        if (tid == 0) next_item = (int64_t)atomicAdd(a.work, 1ull);
        __syncthreads();
        item = (int64_t)__builtin_amdgcn_readfirstlane((int)min(next_item, (int64_t)0x7fffffff));
      }
      if (item >= n_items) break;
      g_split = (int)(item % a.splits);
      // the work record (gather_order_kernel checked the slot and clamped
      // the list length): list (b, h, query cluster), first row, rows, keys
      const int4 rv = a.order[item / a.splits];
      const int li = __builtin_amdgcn_readfirstlane(rv.x);
      const int64_t bh = li / a.cq;
      ti.b = (int)(bh / a.H);
      ti.h = (int)(bh % a.H);
      ti.row0 = __builtin_amdgcn_readfirstlane(rv.y);
      ti.nrows = __builtin_amdgcn_readfirstlane(rv.z);
      ti.limit = __builtin_amdgcn_readfirstlane(rv.w);
      ti.nkt = (ti.limit + kBN - 1) / kBN;
      ti.pos0 = 0;
      g_list = a.lists + (int64_t)li * a.list_cap;
      g_qperm = a.q_perm + bh * a.Lq;
      k0 = g_split * ti.nkt / a.splits;
      k1 = (g_split + 1) * ti.nkt / a.splits;
    } else if (!a.stream) {
      // one tile per workgroup, or one of its uniform key splits
      if (!first) break;
      ti = fwd_tile(a, w / a.splits);
      k0 = (int)(w % a.splits) * ti.nkt / a.splits;
      k1 = (int)(w % a.splits + 1) * ti.nkt / a.splits;
    } else {
      if (x_end <= s_lo) break;
      ti = fwd_locate(a, x_end - 1);
      k0 = (int)(max(s_lo, ti.pos0) - ti.pos0);
      k1 = (int)(x_end - ti.pos0);
      x_end = ti.pos0 + k0;
    }
    k0 = __builtin_amdgcn_readfirstlane(k0);
    k1 = __builtin_amdgcn_readfirstlane(k1);
    // every wavefront is done with the previous tile's LDS before this
    // tile's copies start
    if (!GATHER && !first) __syncthreads();
    const int b = ti.b, h = ti.h;
    const int64_t row0 = ti.row0, nrows = ti.nrows;

    // ---- block-sparse instance: the key tiles as a table of (first row,
    // rows) in LDS: the own chunk's 64-key tiles, then the selected history
    // blocks in selection order, then four copies of the last entry.  Ids
    // that are not history blocks (negative, past the visible frames, or in
    // the own chunk) are dropped, so nothing outside the own chunk and the
    // history is ever read and no tile is empty.  (One tile per workgroup:
    // the loop runs once.) ----
    [[maybe_unused]] uint32_t tab_addr = 0;
    if constexpr (LIST) {
      static_assert(CRATTN_HSA_QBLOCK == 256, "one selection row per query tile");
      static_assert(CRATTN_HSA_KBLOCK == kBN, "a selected block is one key tile");
      __shared__ int2 tab[kListMax];
      __shared__ int tab_count[4];
      const int own_first = (int)((a.q_pos0 / a.L) * a.L);
      const int n_own = (ti.limit - own_first + kBN - 1) / kBN;
      for (int i = tid; i < n_own; i += 256)
        tab[i] = make_int2(own_first + i * kBN, min(kBN, ti.limit - (own_first + i * kBN)));
      const int32_t *sl = a.sel + (((int64_t)b * a.H + h) * a.n_tiles + w % a.n_tiles) * a.kb;
      int nsel = 0;
      for (int i0 = 0; i0 < a.kb; i0 += 256) {
        const int i = i0 + tid;
        const int id = i < a.kb ? sl[i] : -1;
        const bool v = id >= 0 && id < a.vis_blocks && (id < a.own_b0 || id >= a.own_b1);
        const uint64_t bal = __builtin_amdgcn_ballot_w64(v);
        const int before = __builtin_popcountll(bal & ((uint64_t(1) << lane) - 1));
        if (lane == 0) tab_count[wave] = __builtin_popcountll(bal);
        __syncthreads();
        int off = n_own + nsel, tot = 0;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          off += w2 < wave ? tab_count[w2] : 0;
          tot += tab_count[w2];
        }
        if (v) {
          const int f = id / a.nbf, j = id - f * a.nbf;
          const int start = f * a.blk_frame + j * kBN;
          tab[off + before] = make_int2(start, min(kBN, a.blk_frame - j * kBN));
        }
        nsel += tot;
        __syncthreads();
      }
      const int n = n_own + nsel;
      if (tid < 4) tab[n + tid] = tab[n - 1];
      __syncthreads();
      k0 = 0;
      k1 = __builtin_amdgcn_readfirstlane(n);
      tab_addr = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(lds_char_t *)reinterpret_cast<char *>(tab));
    }
    const int last = k1 - 1;
    const int rem = __builtin_amdgcn_readfirstlane(min(kBN, ti.limit - last * kBN));

    // ---- this wavefront's 64 queries as B operands (Q in registers) ----
    const int64_t wrow0 = row0 + (int64_t)wave * 64;
    bf16x8_t qf[2][DK];
    // (gather instance) the queries' rows in memory, kept for the stores
    [[maybe_unused]] int32_t g_mrow[2] = {0, 0};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int64_t row = wrow0 + qb * 32 + l32;
      const bool ok = row < row0 + nrows;
      int64_t mrow = row;
      if constexpr (GATHER) {
        mrow = ok ? min((uint32_t)g_qperm[row], (uint32_t)(a.Lq - 1)) : 0;
        g_mrow[qb] = (int32_t)mrow;
      }
      const uint16_t *qp = a.q + (((int64_t)b * a.Lq + mrow) * a.H + h) * D + hf * 8;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (ok) x = *reinterpret_cast<const uint4 *>(qp + ks * 16);
        qf[qb][ks] = __builtin_bit_cast(bf16x8_t, x);
      }
      if constexpr (ROPE) {
        constexpr int HT = (D - 4 * (D / 6)) / 2;
        constexpr int HH = D / 6;
        const Pos p =
            decode_pos(a.tok_off + (uint32_t)min(row, a.Lq - 1), a.per_frame, a.gw, a.t0);
        const float2 *ax[3] = {a.table + p.t * HT + 4 * hf,
                               a.table + a.tg.base_h + p.h * HH - HT + 4 * hf,
                               a.table + a.tg.base_w + p.w * HH - HT - HH + 4 * hf};
        auto axis = [](int q) { return q < HT ? 0 : q < HT + HH ? 1 : 2; };
        float2 cs[DK][4];
#pragma unroll
        for (int ks = 0; ks < DK; ++ks)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int q0 = ks * 8 + e;
            const int a0 = axis(q0), a1 = axis(q0 + 4);
            const float2 *ptr = a0 == a1 ? ax[a0] : (hf ? ax[a1] : ax[a0]);
            cs[ks][e] = ptr[q0];
          }
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
          const uint4 x = __builtin_bit_cast(uint4, qf[qb][ks]);
          uint32_t wv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float2 r = rotate_pair(__uint_as_float(wv[e] << 16),
                                         __uint_as_float(wv[e] & 0xffff0000u), cs[ks][e]);
            wv[e] = pack_bf16(r.x, r.y);
          }
          qf[qb][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(wv[0], wv[1], wv[2], wv[3]));
        }
      }
    }
    f32x32_t qa[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const uint4 x = __builtin_bit_cast(uint4, qf[qb][ks]);
        qa[qb][4 * ks + 0] = __uint_as_float(x.x);
        qa[qb][4 * ks + 1] = __uint_as_float(x.y);
        qa[qb][4 * ks + 2] = __uint_as_float(x.z);
        qa[qb][4 * ks + 3] = __uint_as_float(x.w);
      }

    // ---- the lane's copy offsets: slot n of the tile (K: instructions
    // wave + 4n, and for n = 4 instruction 16 on wave 0, a repeat of slot 3
    // elsewhere; V: wave + 4n), full rows and rows clamped to the last valid
    // key of the final tile ----
    u32x8_t dma_a, dmal_a;
    u32x2_t dma_b, dmal_b;
    [[maybe_unused]] u32x3_t gcol = {0u, 0u, 0u};
    {
      uint32_t off[10], offl[10];
#pragma unroll
      for (int n = 0; n < 10; ++n) {
        const bool kside = n < 5;
        const int j =
            kside ? (n < 4 ? wave + 4 * n : (wave == 0 ? 16 : wave + 12)) : wave + 4 * (n - 5);
        const int pitch = kside ? KP : VP;
        const int cell = j * 64 + lane;
        const int row = cell / pitch, c = cell - row * pitch;
        const uint32_t col = (uint32_t)(c < D / 8 ? c * 16 : 0);
        off[n] = (uint32_t)row * (D * 2) + col;
        // (the block-sparse instance clamps each ragged tile from the full
        // offsets; the gather instance takes the lane's row index with
        // ds_bpermute from lane `row` and or-s the column bytes in)
        offl[n] = LIST ? off[n] : GATHER ? (uint32_t)row * 4u
                                         : (uint32_t)min(row, rem - 1) * (D * 2) + col;
        if constexpr (GATHER) gcol[n / 4] |= col << (8 * (n % 4));
      }
      for (int n = 0; n < 8; ++n) {
        dma_a[n] = off[n];
        dmal_a[n] = offl[n];
      }
      dma_b[0] = off[8];
      dma_b[1] = off[9];
      dmal_b[0] = offl[8];
      dmal_b[1] = offl[9];
    }
    const int64_t head_off = ((int64_t)b * a.H + h) * a.cap * D;
    const uint16_t *kh = a.k + head_off;
    const uint16_t *vh = a.v + head_off;

    f32x32_t o[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 32; ++r) o[g][r] = 0.f;
    f32x2_t m2 = {-INFINITY, -INFINITY};
    f32x4_t l4 = {0.f, 0.f, 0.f, 0.f};
    int t = k0;
    if (k0 < k1) {
      if constexpr (GATHER) {
        const uint32_t lane4 = (uint32_t)lane * 4u;
        const uint32_t capm1 = (uint32_t)(a.cap - 1);
        // row indices of tiles k0 .. k0+3 (clamped to the last tile; lanes
        // past its rows read its last row), loaded here so that their
        // latency passes beside the query loads
        int32_t gi[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tj = min(k0 + j, last);
          const int rl = tj == last ? rem - 1 : kBN - 1;
          gi[j] = g_list[(int64_t)tj * kBN + min(lane, rl)];
        }
    #pragma clang diagnostic push
    #pragma clang diagnostic ignored "-Winline-asm"
          asm volatile(CRATTN_ATTN_LOOP_GATHER_ASM
                       : "+{a[0:31]}"(o[0]), "+{a[32:63]}"(o[1]), "+{a[64:95]}"(o[2]),
                         "+{a[96:127]}"(o[3]), "={v[192:193]}"(m2), "={v[194:197]}"(l4),
                         "+{v[208:215]}"(dma_a), "+{v[216:217]}"(dma_b), "+{s68}"(t),
                         "+{v242}"(gi[0]), "+{v243}"(gi[1]), "+{v244}"(gi[2]), "+{v245}"(gi[3])
                       : "{a[128:159]}"(qa[0]), "{a[160:191]}"(qa[1]), "{v[218:225]}"(dmal_a),
                         "{v[226:227]}"(dmal_b), "{v[228:235]}"(bases), "{v207}"(kh8),
                         "{s[64:65]}"(kh), "{s[66:67]}"(vh), "{s69}"(last), "{s70}"(rem),
                         "{s71}"(sc), "{s72}"(wb), "{s73}"(k5), "{s[88:89]}"(g_list),
                         "{s95}"(capm1), "{v246}"(lane4), "{v[248:250]}"(gcol)
                       : "v0", "v1", "v2", "v3", "v4", "v5", "v6", "v7", "v8", "v9", CRT_D("v", 1),
                         CRT_D("v", 2), CRT_D("v", 3), CRT_D("v", 4), CRT_D("v", 5),
                         CRT_D("v", 6), CRT_D("v", 7), CRT_D("v", 8), CRT_D("v", 9),
                         CRT_D("v", 10), CRT_D("v", 11), CRT_D("v", 12), CRT_D("v", 13),
                         CRT_D("v", 14), CRT_D("v", 15), CRT_D("v", 16), CRT_D("v", 17),
                         CRT_D("v", 18), "v190", "v191", "v198", "v199", "v200", "v201", "v202",
                         "v203", "v204", "v205", "v206", "v236", "v237", "v238", "v239", "v240", "v241",
                         "s74", "s75", "s76", "s77",
                         "s78", "s79", "s80", "s81", "s82", "s83", "s84", "s85", "s86", "s87",
                         "s90", "s91", "s92", "s93", "s94", "v247",
                         "m0", "vcc", "scc", "memory");
    #pragma clang diagnostic pop
      } else if constexpr (LIST) {
    #pragma clang diagnostic push
    #pragma clang diagnostic ignored "-Winline-asm"
          asm volatile(CRATTN_ATTN_LOOP_LIST_ASM
                       : "+{a[0:31]}"(o[0]), "+{a[32:63]}"(o[1]), "+{a[64:95]}"(o[2]),
                         "+{a[96:127]}"(o[3]), "={v[192:193]}"(m2), "={v[194:197]}"(l4),
                         "+{v[208:215]}"(dma_a), "+{v[216:217]}"(dma_b), "+{s68}"(t)
                       : "{a[128:159]}"(qa[0]), "{a[160:191]}"(qa[1]), "{v[218:225]}"(dmal_a),
                         "{v[226:227]}"(dmal_b), "{v[228:235]}"(bases), "{v207}"(kh8),
                         "{s[64:65]}"(kh), "{s[66:67]}"(vh), "{s69}"(last),
                         "{s71}"(sc), "{s72}"(wb), "{s73}"(k5), "{s88}"(tab_addr)
                       : "v0", "v1", "v2", "v3", "v4", "v5", "v6", "v7", "v8", "v9", CRT_D("v", 1),
                         CRT_D("v", 2), CRT_D("v", 3), CRT_D("v", 4), CRT_D("v", 5),
                         CRT_D("v", 6), CRT_D("v", 7), CRT_D("v", 8), CRT_D("v", 9),
                         CRT_D("v", 10), CRT_D("v", 11), CRT_D("v", 12), CRT_D("v", 13),
                         CRT_D("v", 14), CRT_D("v", 15), CRT_D("v", 16), CRT_D("v", 17),
                         CRT_D("v", 18), "v190", "v191", "v198", "v199", "v200", "v201", "v202",
                         "v203", "v204", "v205", "v206", "v236", "v237", "v238", "v239", "v240", "v241",
                         "s74", "s75", "s76", "s77",
                         "s78", "s79", "s80", "s81", "s82", "s83", "s84", "s85", "s86", "s87", "s89",
                         "s90", "s91", "s92", "s93", "s94", "s95", "s96", "s97", "v242", "v243",
                         "v244", "m0",
                         "vcc", "scc", "memory");
    #pragma clang diagnostic pop
      } else {
    #pragma clang diagnostic push
    #pragma clang diagnostic ignored "-Winline-asm"
          asm volatile(CRATTN_ATTN_LOOP_ASM
                       : "+{a[0:31]}"(o[0]), "+{a[32:63]}"(o[1]), "+{a[64:95]}"(o[2]),
                         "+{a[96:127]}"(o[3]), "={v[192:193]}"(m2), "={v[194:197]}"(l4),
                         "+{v[208:215]}"(dma_a), "+{v[216:217]}"(dma_b), "+{s68}"(t)
                       : "{a[128:159]}"(qa[0]), "{a[160:191]}"(qa[1]), "{v[218:225]}"(dmal_a),
                         "{v[226:227]}"(dmal_b), "{v[228:235]}"(bases), "{v207}"(kh8),
                         "{s[64:65]}"(kh), "{s[66:67]}"(vh), "{s69}"(last), "{s70}"(rem),
                         "{s71}"(sc), "{s72}"(wb), "{s73}"(k5)
                       : "v0", "v1", "v2", "v3", "v4", "v5", "v6", "v7", "v8", "v9", CRT_D("v", 1),
                         CRT_D("v", 2), CRT_D("v", 3), CRT_D("v", 4), CRT_D("v", 5),
                         CRT_D("v", 6), CRT_D("v", 7), CRT_D("v", 8), CRT_D("v", 9),
                         CRT_D("v", 10), CRT_D("v", 11), CRT_D("v", 12), CRT_D("v", 13),
                         CRT_D("v", 14), CRT_D("v", 15), CRT_D("v", 16), CRT_D("v", 17),
                         CRT_D("v", 18), "v190", "v191", "v198", "v199", "v200", "v201", "v202",
                         "v203", "v204", "v205", "v206", "v236", "v237", "v238", "v239", "v240", "v241",
                         "s74", "s75", "s76", "s77",
                         "s78", "s79", "s80", "s81", "s82", "s83", "s84", "s85", "s86", "s87", "m0",
                         "vcc", "scc", "memory");
    #pragma clang diagnostic pop
      }
    }

    // ---- this tile's rows: base-2 log-sum-exp and the normalised O ----
    float lse2[2], inv[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float lt = half_swap_sum(l4[2 * qb] + l4[2 * qb + 1]);
      inv[qb] = lt > 0.f ? 1.0f / lt : 0.f;
      lse2[qb] = lt > 0.f ? m2[qb] + __log2f(lt) : -INFINITY;
    }
    const int trow0 = wave * 64 + l32;  // tile row of (qb = 0); qb adds 32

    if (a.splits > 1) {
      // uniform split: the partial (normalised O, base-2 log-sum-exp) of
      // this key range, merged by attn_combine_kernel (gather instance: at
      // the query's own row)
      const int64_t split = GATHER ? g_split : w % a.splits;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int r = trow0 + qb * 32;
        if (r >= nrows) continue;
        int64_t orow = row0 + r;
        if constexpr (GATHER) orow = g_mrow[qb];
        const int64_t prow = ((split * a.B + b) * a.H + h) * a.Lq + orow;
        float *op = a.ws_o + prow * D + hf * 4;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int base = qb * 16 + i4 * 4;
            *reinterpret_cast<float4 *>(op + db * 32 + i4 * 8) =
                make_float4(o[db][base + 0] * inv[qb], o[db][base + 1] * inv[qb],
                            o[db][base + 2] * inv[qb], o[db][base + 3] * inv[qb]);
          }
        if (hf == 0) a.ws_lse[prow] = lse2[qb];
      }
      continue;
    }

    bool merge = false;
    int64_t part0 = 0, part1 = 0, a0 = 0;
    if (!LIST && !GATHER && (k0 != 0 || k1 != ti.nkt)) {
      // A part of a tile cut between workgroups (balanced split only): the
      // parts are those of workgroups part0 .. part1; a part writes its
      // normalised O and log-sum-exp to its slot (slot 0 of a workgroup for
      // the tile its range starts in, slot 1 for the tile it ends in) and
      // counts itself done; the part that finds all others done merges them.
      a0 = ti.pos0;
      part0 = part_of(a0);
      part1 = part_of(a0 + ti.nkt - 1);
      const int n_parts = (int)(part1 - part0 + 1);
      // Only wavefront 0 fences at device scope: the workgroup barriers order
      // the other wavefronts' slot stores before its release and its acquire
      // before their slot loads.  Slot writers release (L2 write-back) once;
      // only the merging part acquires (L2 invalidate).
      // A workgroup's first part (the head of its last tile) is never the
      // tile's last part in practice: it writes its slot without first
      // asking whether the others are done (one counter round trip less).
      unsigned *cnt = a.counters + part0;
      if (!first) {
        if (tid == 0)
          sh_count = (int)__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        merge = sh_count == n_parts - 1;
        __syncthreads();
      }
      if (!merge) {
        const int64_t slot = 2 * w + (s_lo >= a0 ? 0 : 1);
        float *so = a.ws_o + slot * (256 * D);
        float *sl = a.ws_lse + slot * 256;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int r = trow0 + qb * 32;
          if (r >= nrows) continue;
          float *op = so + (int64_t)r * D + hf * 4;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int base = qb * 16 + i4 * 4;
              *reinterpret_cast<float4 *>(op + db * 32 + i4 * 8) =
                  make_float4(o[db][base + 0] * inv[qb], o[db][base + 1] * inv[qb],
                              o[db][base + 2] * inv[qb], o[db][base + 3] * inv[qb]);
            }
          if (hf == 0) sl[r] = lse2[qb];
        }
        __syncthreads();
        if (tid == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          sh_count = (int)__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        merge = sh_count == n_parts - 1;
      }
      if (!merge) continue;
      if (tid == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __syncthreads();
    }

    // ---- final rows: this part alone, or merged with the tile's other
    // parts (O = sum_p 2^(lse_p - lse) O_p, lse = log2 sum_p 2^lse_p).  The
    // merge takes the parts in workgroup order with this part's normalised
    // O rounded as its slot would hold it, so the result does not depend on
    // which part finished last. ----
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int r = trow0 + qb * 32;
      if (r >= nrows) continue;
      float scl = inv[qb], lse_f = lse2[qb];
      if (merge && part1 == part0 + 1) {
        // two parts, the usual cut: the other part's log-sum-exp and O are
        // loaded together, then combined in workgroup order with the same
        // operations, in the same order, as the general merge below
        const int64_t vo = part0 == w ? part1 : part0;
        const int64_t so = 2 * vo + (vo * T / G >= a0 ? 0 : 1);
        const float lo = a.ws_lse[so * 256 + r];
        const float *opo = a.ws_o + so * (256 * D) + (int64_t)r * D + hf * 4;
        float4 xo[DB][4];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            xo[db][i4] = *reinterpret_cast<const float4 *>(opo + db * 32 + i4 * 8);
        const bool own0 = part0 == w;
        const float l0 = own0 ? lse2[qb] : lo, l1 = own0 ? lo : lse2[qb];
        float mx = -INFINITY;
        mx = fmaxf(mx, l0);
        mx = fmaxf(mx, l1);
        const float w0 = l0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(l0 - mx);
        const float w1 = l1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(l1 - mx);
        float wsum = 0.f;
        wsum += w0;
        wsum += w1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int base = qb * 16 + i4 * 4;
            const float4 own = make_float4(o[db][base + 0] * inv[qb], o[db][base + 1] * inv[qb],
                                           o[db][base + 2] * inv[qb], o[db][base + 3] * inv[qb]);
            const float4 x0 = own0 ? own : xo[db][i4], x1 = own0 ? xo[db][i4] : own;
            o[db][base + 0] = fmaf(w1, x1.x, fmaf(w0, x0.x, 0.f));
            o[db][base + 1] = fmaf(w1, x1.y, fmaf(w0, x0.y, 0.f));
            o[db][base + 2] = fmaf(w1, x1.z, fmaf(w0, x0.z, 0.f));
            o[db][base + 3] = fmaf(w1, x1.w, fmaf(w0, x0.w, 0.f));
          }
        scl = wsum > 0.f ? 1.0f / wsum : 0.f;
        lse_f = wsum > 0.f ? mx + __log2f(wsum) : -INFINITY;
      } else if (merge) {
        float mx = -INFINITY;
        for (int64_t v = part0; v <= part1; ++v) {
          const int64_t slot = 2 * v + (v * T / G >= a0 ? 0 : 1);
          mx = fmaxf(mx, v == w ? lse2[qb] : a.ws_lse[slot * 256 + r]);
        }
        float acc[DB][16];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
        float wsum = 0.f;
        for (int64_t v = part0; v <= part1; ++v) {
          const int64_t slot = 2 * v + (v * T / G >= a0 ? 0 : 1);
          const float lv = v == w ? lse2[qb] : a.ws_lse[slot * 256 + r];
          const float wv = lv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lv - mx);
          wsum += wv;
          const float *op = a.ws_o + slot * (256 * D) + (int64_t)r * D + hf * 4;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int base = qb * 16 + i4 * 4;
              float4 x;
              if (v == w)
                x = make_float4(o[db][base + 0] * inv[qb], o[db][base + 1] * inv[qb],
                                o[db][base + 2] * inv[qb], o[db][base + 3] * inv[qb]);
              else
                x = *reinterpret_cast<const float4 *>(op + db * 32 + i4 * 8);
              acc[db][i4 * 4 + 0] = fmaf(wv, x.x, acc[db][i4 * 4 + 0]);
              acc[db][i4 * 4 + 1] = fmaf(wv, x.y, acc[db][i4 * 4 + 1]);
              acc[db][i4 * 4 + 2] = fmaf(wv, x.z, acc[db][i4 * 4 + 2]);
              acc[db][i4 * 4 + 3] = fmaf(wv, x.w, acc[db][i4 * 4 + 3]);
            }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][qb * 16 + i] = acc[db][i];
        scl = wsum > 0.f ? 1.0f / wsum : 0.f;
        lse_f = wsum > 0.f ? mx + __log2f(wsum) : -INFINITY;
      }
      int64_t row = row0 + r;
      if constexpr (GATHER) row = g_mrow[qb];
      uint16_t *op = a.out + (((int64_t)b * a.Lq + row) * a.H + h) * D + hf * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int base = qb * 16 + i4 * 4;
          uint2 u;
          u.x = pack_bf16(o[db][base + 0] * scl, o[db][base + 1] * scl);
          u.y = pack_bf16(o[db][base + 2] * scl, o[db][base + 3] * scl);
          *reinterpret_cast<uint2 *>(op + db * 32 + i4 * 8) = u;
        }
      if (hf == 0 && a.lse != nullptr) a.lse[((int64_t)b * a.H + h) * a.Lq + row] = lse_f * kLn2;
    }
  }
}

// Clear the balanced split's completion counters before a launch.
__global__ void attn_clear_counters_kernel(unsigned *c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = 0u;
}
#undef CRT_D

struct CombineArgs {
  const float *ws_o;
  const float *ws_lse;
  uint16_t *out;
  float *lse;
  int B, H, D, splits;
  int64_t Lq;
  uint32_t total;  // B * H * Lq * (D / 4)
};

// Merge split-KV partials: lse = log2 sum_s 2^lse_s; O = sum_s 2^(lse_s - lse) O_s.
__global__ void __launch_bounds__(256) attn_combine_kernel(CombineArgs a) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  if (t >= a.total) return;
  const uint32_t nc = (uint32_t)a.D / 4;
  const uint32_t c4 = t % nc;
  const uint64_t r = t / nc;  // (b * H + h) * Lq + row
  const int64_t row = (int64_t)(r % (uint64_t)a.Lq);
  const uint64_t bh = r / (uint64_t)a.Lq;
  const int h = (int)(bh % (uint64_t)a.H);
  const int b = (int)(bh / (uint64_t)a.H);
  const uint64_t plane = (uint64_t)a.B * a.H * a.Lq;
  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.ws_lse[s * plane + r]);
  float wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < a.splits; ++s) {
    const float ls = a.ws_lse[s * plane + r];
    const float w = ls == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ls - mx);
    wsum += w;
    const float4 x = *reinterpret_cast<const float4 *>(a.ws_o + (s * plane + r) * a.D + c4 * 4);
    acc.x += w * x.x;
    acc.y += w * x.y;
    acc.z += w * x.z;
    acc.w += w * x.w;
  }
  const float inv = 1.0f / wsum;
  uint2 wv;
  wv.x = pack_bf16(acc.x * inv, acc.y * inv);
  wv.y = pack_bf16(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2 *>(a.out + (((int64_t)b * a.Lq + row) * a.H + h) * a.D + c4 * 4) = wv;
  if (c4 == 0 && a.lse != nullptr) a.lse[r] = (mx + __log2f(wsum)) * kLn2;
}

// Work order of the gather instance: a record per (b, h, slot) entry with
// rows -- its key list, first row, rows and key count, so a workgroup finds
// its work in one load -- by decreasing key-tile count (a counting sort over
// 2048 cost bins; the order inside a bin is whatever the atomics give, which
// changes no result), so the persistent workgroups take the longest tiles
// first.
constexpr int kCostBins = 2048;

// It also starts the work counter at the persistent grid's size.
__global__ void __launch_bounds__(1024) gather_order_kernel(AttnKArgs a, int n_entries,
                                                            unsigned long long grid) {
  __shared__ int hist[kCostBins];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) *a.work = grid;
  for (int c = tid; c < kCostBins; c += 1024) hist[c] = 0;
  __syncthreads();
  // the work record of entry e -- list (b, h, query cluster), first row,
  // rows, keys (the list length clamped to the capacity) -- or one with no
  // rows for a slot that is empty or out of range
  auto rec_of = [&](int e) {
    const int4 sl = reinterpret_cast<const int4 *>(a.gslots)[e];
    if (sl.y <= 0 || sl.y > CRATTN_SVG2_QTILE || sl.x < 0 || (int64_t)sl.x + sl.y > a.Lq ||
        sl.z < 0 || sl.z >= a.cq)
      return make_int4(0, 0, 0, 0);
    const int64_t li = e / a.n_tiles * a.cq + sl.z;
    const int len = min(max(a.list_len[li], 0), (int)a.list_cap);
    return make_int4((int)li, sl.x, sl.y, len);
  };
  // bin (kCostBins - 1 - tiles) of a record, or -1 without rows
  auto bin_of = [&](int4 r) {
    return r.z <= 0 ? -1 : kCostBins - 1 - min((r.w + 63) / 64, kCostBins - 1);
  };
  for (int e = tid; e < n_entries; e += 1024) {
    const int b = bin_of(rec_of(e));
    if (b >= 0) atomicAdd(&hist[b], 1);
  }
  __syncthreads();
  // exclusive scan of the bins: two per thread, then over the 16 waves
  const int h0 = hist[2 * tid], h1 = hist[2 * tid + 1];
  int inc = h0 + h1;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int base = inc - h0 - h1;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  __syncthreads();
  hist[2 * tid] = base;
  hist[2 * tid + 1] = base + h0;
  if (tid == 1023) *const_cast<int32_t *>(a.n_real) = base + h0 + h1;
  __syncthreads();
  int4 *order = const_cast<int4 *>(a.order);
  for (int e = tid; e < n_entries; e += 1024) {
    const int4 r = rec_of(e);
    const int b = bin_of(r);
    if (b >= 0) order[atomicAdd(&hist[b], 1)] = r;
  }
}


template <int D, int NW, int QB, int MINB, bool ROPE, bool SPARSE, bool GATHER = false>
hipError_t launch_fwd(const AttnKArgs &k, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW, QB, MINB, ROPE, SPARSE, GATHER>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, s, k);
  return hipGetLastError();
}

}  // namespace

// Fixed scratch for the split-KV partials of chunk_causal_attn_noalloc.  In
// host code `scratch` is only a stand-in for the device array: its device
// address comes from hipGetSymbolAddress, once per device (each device holds
// its own copy), and only that address is handed to kernels.
static __device__ __align__(256) char scratch[kAttnScratchBytes];

void *attn_scratch(hipError_t *err) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> ptr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  void *p = ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    ptr[dev].store(p, std::memory_order_release);  // the same address in every thread
  }
  *err = hipSuccess;
  return p;
}

hipError_t launch_attn(const AttnArgs &a, const AttnPlan &p, hipStream_t s) {
  AttnKArgs k;
  k.q = static_cast<const uint16_t *>(a.q);
  k.k = static_cast<const uint16_t *>(a.k);
  k.v = static_cast<const uint16_t *>(a.v);
  k.out = static_cast<uint16_t *>(a.out);
  k.lse = a.lse;
  k.B = a.B;
  k.H = a.H;
  k.Lq = a.Lq;
  k.cap = a.cap;
  k.kv_len = a.kv_len;
  k.q_pos0 = a.q_pos0;
  k.L = a.chunk_tokens;
  const float scale = a.scale > 0.f ? a.scale : 1.0f / sqrtf((float)a.D);
  k.scale_log2 = scale * 1.44269504088896340736f;
  k.inv_scale_log2 = 1.0f / k.scale_log2;
  k.seg0_rows = p.seg0_rows;
  k.tiles0 = p.tiles0;
  k.tiles_full = p.tiles_full;
  k.n_full = p.n_full;
  k.last_rows = p.last_rows;
  k.n_tiles = p.n_tiles;
  k.splits = p.splits;
  const size_t o_bytes = (size_t)p.splits * a.B * a.H * a.Lq * (size_t)a.D * 4u;
  k.ws_o = p.splits > 1 ? static_cast<float *>(a.workspace) : nullptr;
  k.ws_lse = p.splits > 1 ? reinterpret_cast<float *>(static_cast<char *>(a.workspace) + o_bytes)
                          : nullptr;
  k.table = nullptr;
  k.tg = TabGeom{};
  k.per_frame = k.gw = k.t0 = k.tok_off = 0;
  if (a.rope) {
    const RopeSplit sp = rope_split(a.D);
    k.table = reinterpret_cast<const float2 *>(a.table);
    k.tg.ht = (uint32_t)(sp.dt / 2);
    k.tg.hh = (uint32_t)(sp.dh / 2);
    k.tg.base_h = (uint32_t)a.max_t * k.tg.ht;
    k.tg.base_w = k.tg.base_h + (uint32_t)a.max_h * k.tg.hh;
    k.per_frame = (uint32_t)a.grid_h * (uint32_t)a.grid_w;
    k.gw = (uint32_t)a.grid_w;
    k.t0 = (uint32_t)a.t0;
    k.tok_off = (uint32_t)a.tok_off;
  }
  k.sel = a.sel;
  k.kb = a.sel_kb;
  k.nbf = a.sel_nbf;
  k.blk_frame = a.sel_per_frame;
  k.vis_blocks = a.sel_vis_blocks;
  k.own_b0 = a.sel_own_b0;
  k.own_b1 = a.sel_own_b1;
  k.q_perm = a.q_perm;
  k.gslots = a.gslots;
  k.lists = a.lists;
  k.list_len = a.list_len;
  k.list_cap = a.list_cap;
  k.cq = a.cq;
  k.work = nullptr;
  k.order = nullptr;
  k.n_real = nullptr;
  k.stream = 0;
  k.steps_bh = k.total_steps = 0;
  k.counters = nullptr;
  hipError_t e;
  if (a.gslots != nullptr) {
    // persistent: the workspace holds the work counter and the number of
    // non-empty slots (first 256 bytes), their order, then the split
    // partials
    char *ws = static_cast<char *>(a.workspace);
    const int64_t n_entries = (int64_t)a.B * a.H * p.n_tiles;
    const size_t order_bytes = ((size_t)n_entries * 16u + 255u) & ~size_t(255);
    k.work = reinterpret_cast<unsigned long long *>(ws);
    k.n_real = reinterpret_cast<const int32_t *>(ws + 8);
    k.order = reinterpret_cast<const int4 *>(ws + 256);
    if (p.splits > 1) {
      k.ws_o = reinterpret_cast<float *>(ws + 256 + order_bytes);
      k.ws_lse = reinterpret_cast<float *>(ws + 256 + order_bytes + o_bytes);
    }
    const int64_t grid = std::min<int64_t>(p.grid, device_cu_count());
    hipLaunchKernelGGL(gather_order_kernel, dim3(1), dim3(1024), 0, s, k, (int)n_entries,
                       (unsigned long long)grid);
    if (a.D == 128) {
      // the kernel with the hand-scheduled key loop, in its gather form
      hipLaunchKernelGGL((attn_fwd64_kernel<false, false, true>), dim3((unsigned)grid), dim3(256),
                         0, s, k);
      e = hipGetLastError();
    } else {
      e = launch_fwd<64, 8, 1, 1, false, false, true>(k, grid, s);
    }
  } else if (a.D == 128) {
    if (a.sel != nullptr) {
      // block-sparse: the hand-scheduled loop over a table of key tiles when
      // the own chunk's tiles and the selection fit it
      const int64_t own_tiles = (a.chunk_tokens + 63) / 64;
      if (p.splits == 1 && own_tiles + a.sel_kb + 4 <= kListMax) {
        hipLaunchKernelGGL((attn_fwd64_kernel<false, true>), dim3((unsigned)p.grid), dim3(256), 0,
                           s, k);
        e = hipGetLastError();
      } else {
        e = launch_fwd<128, 8, 1, 1, false, true>(k, p.grid, s);
      }
    } else {
      // dense: the kernel with the hand-scheduled key loop
      if (p.stream) {
        // workspace: counters, then the partial slots' O, then their lse
        char *ws = static_cast<char *>(a.workspace);
        const size_t n_slots = 2u * (size_t)p.grid;
        k.stream = 1;
        k.steps_bh = p.steps_bh;
        k.total_steps = p.total_steps;
        k.counters = reinterpret_cast<unsigned *>(ws);
        k.ws_o = reinterpret_cast<float *>(ws + kStreamCounterBytes);
        k.ws_lse = k.ws_o + n_slots * (size_t)kStreamRows * 128u;
        hipLaunchKernelGGL(attn_clear_counters_kernel, dim3(1), dim3(256), 0, s, k.counters,
                           (int)p.grid);
      }
      if (a.rope)
        hipLaunchKernelGGL((attn_fwd64_kernel<true, false>), dim3((unsigned)p.grid), dim3(256), 0, s, k);
      else
        hipLaunchKernelGGL((attn_fwd64_kernel<false, false>), dim3((unsigned)p.grid), dim3(256), 0, s, k);
      e = hipGetLastError();
    }
  } else {
    e = a.sel != nullptr ? launch_fwd<64, 8, 1, 1, false, true>(k, p.grid, s)
        : a.rope         ? launch_fwd<64, 8, 1, 1, true, false>(k, p.grid, s)
                         : launch_fwd<64, 8, 1, 1, false, false>(k, p.grid, s);
  }
  if (e != hipSuccess || p.splits == 1) return e;
  CombineArgs c;
  c.ws_o = k.ws_o;
  c.ws_lse = k.ws_lse;
  c.out = k.out;
  c.lse = a.lse;
  c.B = a.B;
  c.H = a.H;
  c.D = a.D;
  c.splits = p.splits;
  c.Lq = a.Lq;
  c.total = (uint32_t)((uint64_t)a.B * a.H * a.Lq * (a.D / 4));
  hipLaunchKernelGGL(attn_combine_kernel, dim3((c.total + 255u) / 256u), dim3(256), 0, s, c);
  return hipGetLastError();
}

}  // namespace crattn
