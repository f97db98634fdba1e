// Fused QKV projection + 3D Causal-RoPE + KV-cache append for AMD CDNA4
// (gfx950), bf16 MFMA with fp32 accumulation.
//
// Sources: "Accelerating Video Generation Inference with Sequential-Parallel
// 3D Positional Encoding Using a Global Time Index", technical summary §2.C
// (the rotary embedding fused into the QKV projection, cos/sin precomputed
// into device tensors), §2.B (global time index) and §1 (KV cache).  The
// projection is the plain linear map y = x W^T, W in [3*H*D, C] (the usual
// linear-layer layout), columns Q, K, V with heads contiguous, no bias.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, 64-wide wavefronts)
//   * Y^T = W X^T: A = 32 features x 16 of C (rows of W), B = 16 of C x 32
//     tokens (rows of X).  Both operands are read along C, 16 bytes a lane.
//   * In the 32x32 accumulator, lane l owns token l%32 and register r the
//     feature 8*(r/4) + 4*(l/32) + r%4: the two features of a rotation pair
//     (2j, 2j+1) are registers r, r+1 of one lane.  After the rotation,
//     lanes l and l+32 trade halves (v_permlane32_swap) so that each lane
//     holds 8 consecutive features of its token and writes 16 bytes.
//   * A 32-feature block lies inside one of Q, K, V and one head (D is 64
//     or 128), so the epilogue decides per block where it goes: Q' to
//     [B, n, H, D], K' and V to the cache rows cache_pos + i.
//
// Work decomposition: a workgroup of 4 wavefronts (one per SIMD) computes
// 256 features x 64*TN tokens; wavefront w owns 128 features (w%2) and
// 32*TN tokens (w/2), 4 x TN accumulator blocks held in the accumulation
// registers.  C is walked in stages of 64 (128-byte row segments: the
// global -> LDS copy path sustains about 20% more than with 64-byte
// segments when LDS reads run beside it) through a 2- or 3-stage LDS ring;
// each stage is consumed in two halves whose fragments are read from LDS
// while the matrix cores work on the previous half's.  The token tile
// width TN (2, 3 or 4 blocks) is picked per call so that the tiles fill
// the chip's CUs in as few weighted rounds as possible.
#include "crattn_internal.h"
#include "rope_common.h"
#include "../../include/crattn.h"

#include <type_traits>

namespace crattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kNW = 4;        // wavefronts per workgroup (one per SIMD)
constexpr int kBK = 64;       // C per ring stage (8 cells of 16 bytes per row)

struct QkvKArgs {
  const uint16_t *x;   // [M = B * n][C]
  const uint16_t *w;   // [F = 3 * H * D][C]
  uint16_t *q_out;     // [B][n][H][D] or null (then features start at H*D)
  uint16_t *k_cache;   // [B][H][cap][D]
  uint16_t *v_cache;
  const float2 *table;
  int64_t cap, cache_pos, n;
  int M, F, f_begin, C, H, D;
  int fg;  // feature tiles per group of the tile order
  uint32_t per_frame, gw, t0, tok_off;
  TabGeom tg;
};

__device__ inline uint32_t pack_bf16(float lo, float hi) {
  f32x2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (an asm with a memory clobber: LDS reads stay after it).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Global -> LDS copy, scalar-base form of global_load_lds_dwordx4: lane i's
// 16 bytes at gbase + voff land at LDS byte address lds_addr + 16 * i
// (lds_addr wave-uniform).  Issued through asm so the compiler does not
// order unrelated LDS reads after it; completion is tracked with
// wait_vmcnt and published to the workgroup with a barrier.  M0 is set in
// the asm and used by nothing else in this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_dma16(const void *gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
// The same with 4 bytes a lane: 256 bytes per instruction.
__device__ inline void lds_dma4(const void *gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Tile of workgroup blockIdx.x: first feature f0 and first token m0 of a
// kBM x kBN output tile.
__device__ inline void tile_origin(const QkvKArgs &a, int kBM, int kBN, int &f0, int &m0) {
  // workgroups go round-robin over the 8 XCDs; renumber them so that each
  // XCD gets a contiguous range of tiles.  Tiles are ordered in groups of
  // fg feature tiles, token tile slowest inside a group, so the tiles an XCD
  // runs at once form a block of about fg feature tiles by a few token
  // tiles, and its L2 serves their shared rows of W and X
  const int G = (int)gridDim.x, q8 = G >> 3, r8 = G & 7;
  const int xcd = (int)blockIdx.x & 7;
  const int tile = xcd * q8 + min(xcd, r8) + ((int)blockIdx.x >> 3);
  const int n_ft = (a.F - a.f_begin + kBM - 1) / kBM;
  const int n_tt = (a.M + kBN - 1) / kBN;
  const int grp = tile / (a.fg * n_tt), in_grp = tile - grp * a.fg * n_tt;
  const int fg = min(a.fg, n_ft - grp * a.fg);
  f0 = a.f_begin + (grp * a.fg + in_grp % fg) * kBM;
  m0 = (in_grp / fg) * kBN;
}

typedef __attribute__((address_space(3))) f32x2_t lds_f2;

// Where the epilogue finds the (cos, sin) rows of a position: entry q of
// axis t at row t is base + (t - t_lo) HT + q, of axis h at base + base_h +
// h HH + q, of axis w at base + base_w + w HH + q.
struct TabView {
  int t_lo, base_h, base_w;
};

// LDS the wide tile sets aside for the rows of the (cos, sin) table.
constexpr int kQkvTabBytes = 40 * 1024;

// Rows of the (cos, sin) table that the call's tokens use: the chunk's
// frames of axis t, every row of axes h and w of the grid (float2 entries).
template <int D>
__host__ __device__ inline int staged_rows(uint32_t t0, uint32_t tok_off, int64_t n,
                                           uint32_t per_frame, uint32_t gw, int &t_lo) {
  constexpr int HT = (D - 4 * (D / 6)) / 2, HH = D / 6;
  t_lo = (int)(t0 + tok_off / per_frame);
  const int t_hi = (int)(t0 + (uint32_t)((tok_off + n - 1) / per_frame));
  return (t_hi - t_lo + 1) * HT + (int)(per_frame / gw) * HH + (int)gw * HH;
}

// Copy those rows into LDS at byte address dst, in that order, and return
// the view of the copy.  The epilogue's per-lane reads then go to LDS: each
// lane reads the rows of its own token, which in global memory are a gather
// over many cache lines per instruction (the w rows differ from lane to
// lane).  The rows go global -> LDS with 4-byte copies (no registers held,
// in flight beside the ring's first stages; entries are 8 bytes and the
// ranges start anywhere), wavefront w taking copies w, w + kNW, ...  The
// caller waits for them (vmcnt) and passes a barrier before the rows are
// read; the launcher checks that the rows fit.
template <int D>
__device__ inline TabView dma_table(const QkvKArgs &a, uint32_t dst, int wave, int lane) {
  constexpr int HT = (D - 4 * (D / 6)) / 2, HH = D / 6;
  int t_lo;
  const int total = staged_rows<D>(a.t0, a.tok_off, a.n, a.per_frame, a.gw, t_lo);
  const int nh = (int)(a.per_frame / a.gw) * HH;
  const int nt = total - nh - (int)a.gw * HH;
  const int ndw = 2 * total;
  const int n_copies = (ndw + 63) / 64;
  for (int k = wave; k < n_copies; k += kNW) {
    const int q = min(k * 64 + lane, ndw - 1);  // dword of the copy (lanes past the end repeat the last)
    const int e = q >> 1;
    const int src = e < nt        ? t_lo * HT + e
                    : e < nt + nh ? (int)a.tg.base_h + (e - nt)
                                  : (int)a.tg.base_w + (e - nt - nh);
    lds_dma4(a.table, (uint32_t)src * 8u + (uint32_t)(q & 1) * 4u,
             __builtin_amdgcn_readfirstlane(dst + (uint32_t)k * 256u));
  }
  return TabView{t_lo, nt, nt + nh};
}

// Epilogue of a wavefront's TM x TN accumulator blocks (features f0 +
// 32 TM fw.., tokens m0 + 32 TN tw..): rotate Q/K pairs, store Q', K', V.
// One 32-feature block of one token block: rotate its pairs (ROT) with the
// lane's (cos, sin), pack to bf16, trade halves with the lane 32 apart and
// store 16 bytes a lane at dst (null for tokens past the end).
template <bool ROT>
__device__ __forceinline__ void store_block(const f32x16_t &acc, const float2 (&cs)[4][2],
                                            uint16_t *dst) {
  uint32_t wv[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = acc[4 * g + e];
    if constexpr (ROT) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float2 r = rotate_pair(y[2 * e], y[2 * e + 1], cs[g][e]);
        y[2 * e] = r.x;
        y[2 * e + 1] = r.y;
      }
    }
    wv[g][0] = pack_bf16(y[0], y[1]);
    wv[g][1] = pack_bf16(y[2], y[3]);
  }
  // lane l < 32 holds features 8g..8g+3 of its token, lane l+32 the
  // features 8g+4..8g+7: swapping group 2u+1 of the low lane with group 2u
  // of the high lane leaves 16u..16u+7 in the low lane, 16u+8..16u+15 in
  // the high one
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const auto r = __builtin_amdgcn_permlane32_swap(wv[2 * u][c], wv[2 * u + 1][c], false, false);
      wv[2 * u][c] = r[0];
      wv[2 * u + 1][c] = r[1];
    }
  if (dst == nullptr) return;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    uint4 o;
    o.x = wv[2 * u][0];
    o.y = wv[2 * u][1];
    o.z = wv[2 * u + 1][0];
    o.w = wv[2 * u + 1][1];
    *reinterpret_cast<uint4 *>(dst + 16 * u) = o;
  }
}

template <int TM, int TN, int JG, int D, bool LDS_TAB>
__device__ __forceinline__ void rope_store_tile(const QkvKArgs &a, const f32x16_t (&acc)[TM][TN],
                                                int f0, int m0, int fw, int tw, int l32, int hf,
                                                const lds_f2 *tl, TabView tv) {
  static_assert(TN % JG == 0, "gather batches");
  // The wavefront's TM blocks cover 32 TM consecutive features starting on
  // a head boundary, so each block's head, part (Q, K, V) and offset in the
  // head follow from one division.  Per token block: the (cos, sin) of the
  // lane's pairs are gathered in one batch (tokens past the end use the
  // last token's position), rotated, then lanes l and l+32 trade halves so
  // that each lane holds 8 consecutive features and writes 16 bytes.
  constexpr int HT = (D - 4 * (D / 6)) / 2;  // pairs of the t group
  constexpr int HH = D / 6;                  // pairs of the h group (= w group)
  const int fw0 = f0 + fw * 32 * TM;
  const int hg0 = fw0 / D;                   // global head index (over Q, K, V)
  const int part0 = hg0 / a.H, h0 = hg0 - part0 * a.H;
  int part[TM], head[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int h = h0 + (32 * i) / D;
    part[i] = h >= a.H ? part0 + 1 : part0;
    head[i] = h >= a.H ? h - a.H : h;
  }
  const int n32 = (int)a.n;
  // token blocks go in batches of JG: the (cos, sin) gathers of a batch are
  // all issued before any of them is used, so their latencies overlap
#pragma unroll
  for (int j0 = 0; j0 < TN; j0 += JG) {
  float2 cs[JG][TM][4][2];
  int mrow[JG], bidx[JG], itok[JG];
#pragma unroll
  for (int jj = 0; jj < JG; ++jj) {
    const int j = j0 + jj;
    const int m = m0 + tw * 32 * TN + j * 32 + l32;
    const int mc = min(m, a.M - 1);
    const int b = mc / n32, i_tok = mc - b * n32;
    mrow[jj] = m;
    bidx[jj] = b;
    itok[jj] = i_tok;
    const Pos p = decode_pos(a.tok_off + (uint32_t)i_tok, a.per_frame, a.gw, a.t0);
    // per-lane table pointers of the three axes (into the table, or its
    // copy in LDS), offset so that entry q of the lane's pair set is
    // ptr[axis][q] (the high half-wave's pairs are 2 further on)
    auto fetch = [&](auto base) {
      decltype(base) ax[3] = {base + (p.t - tv.t_lo) * HT + 2 * hf,
                              base + tv.base_h + p.h * HH - HT + 2 * hf,
                              base + tv.base_w + p.w * HH - HT - HH + 2 * hf};
      auto axis = [](int q) { return q < HT ? 0 : q < HT + HH ? 1 : 2; };
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (fw0 + 32 * i >= a.F || part[i] >= 2) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int q0 = ((32 * i) % D) / 2 + 4 * g + e;  // pair of the low half-wave
            const int a0 = axis(q0), a1 = axis(q0 + 2);
            const auto ptr = a0 == a1 ? ax[a0] : (hf ? ax[a1] : ax[a0]);
            const auto v = ptr[q0];
            cs[jj][i][g][e] = make_float2(v.x, v.y);
          }
      }
    };
    if constexpr (LDS_TAB)
      fetch(tl);
    else
      fetch(a.table);
  }
#pragma unroll
  for (int jj = 0; jj < JG; ++jj) {
    const int j = j0 + jj;
    const int m = mrow[jj], b = bidx[jj], i_tok = itok[jj];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (fw0 + 32 * i >= a.F) continue;
      const int d_blk = (32 * i) % D;
      uint32_t wv[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * g + e];
        if (part[i] < 2) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float2 r = rotate_pair(y[2 * e], y[2 * e + 1], cs[jj][i][g][e]);
            y[2 * e] = r.x;
            y[2 * e + 1] = r.y;
          }
        }
        wv[g][0] = pack_bf16(y[0], y[1]);
        wv[g][1] = pack_bf16(y[2], y[3]);
      }
      // lane l < 32 holds features 8g..8g+3 of its token, lane l+32 the
      // features 8g+4..8g+7: swapping group 2u+1 of the low lane with group 2u
      // of the high lane leaves 16u..16u+7 in the low lane, 16u+8..16u+15 in
      // the high one
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const auto r = __builtin_amdgcn_permlane32_swap(wv[2 * u][c], wv[2 * u + 1][c], false, false);
          wv[2 * u][c] = r[0];
          wv[2 * u + 1][c] = r[1];
        }
      if (m >= a.M) continue;
      uint16_t *dst;
      if (part[i] == 0)
        dst = a.q_out + ((int64_t)m * a.H + head[i]) * D;
      else
        dst = (part[i] == 1 ? a.k_cache : a.v_cache) +
              (((int64_t)b * a.H + head[i]) * a.cap + a.cache_pos + i_tok) * D;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint4 o;
        o.x = wv[2 * u][0];
        o.y = wv[2 * u][1];
        o.z = wv[2 * u + 1][0];
        o.w = wv[2 * u + 1][1];
        *reinterpret_cast<uint4 *>(dst + d_blk + 16 * u + 8 * hf) = o;
      }
    }
  }
  }
}

template <int TM, int TN, int D>
__device__ __forceinline__ void rope_store_tile_wide(const QkvKArgs &a, const f32x16_t (&acc)[TM][TN],
                                                     int f0, int m0, int fw, int tw, int l32,
                                                     int hf, const lds_f2 *tl, TabView tv) {
  constexpr int JG = 1;
  // The wide tile's epilogue (the narrow tile's is rope_store_tile, which
  // gathers from the table in global memory).  The wavefront's TM blocks
  // cover 32 TM consecutive features starting on a head boundary, so each
  // block's head, part (Q, K, V) and offset in the head follow from one
  // division, made once per wavefront in scalar registers: the choice
  // between rotating and not is a uniform branch per block.  Per token block: the (cos, sin) of the lane's pairs are
  // gathered in one batch (tokens past the end use the last token's
  // position), rotated, then lanes l and l+32 trade halves so that each
  // lane holds 8 consecutive features and writes 16 bytes.
  constexpr int HT = (D - 4 * (D / 6)) / 2;  // pairs of the t group
  constexpr int HH = D / 6;                  // pairs of the h group (= w group)
  const int fw0 = __builtin_amdgcn_readfirstlane(f0 + fw * 32 * TM);
  const int hg0 = fw0 / D;                   // global head index (over Q, K, V)
  const int part0 = __builtin_amdgcn_readfirstlane(hg0 / a.H);
  const int h0 = hg0 - part0 * a.H;
  int part[TM], head[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int h = h0 + (32 * i) / D;
    part[i] = __builtin_amdgcn_readfirstlane(h >= a.H ? part0 + 1 : part0);
    head[i] = __builtin_amdgcn_readfirstlane(h >= a.H ? h - a.H : h);
  }
  const int n32 = (int)a.n;
  // one token block at a time (the table rows are in LDS)
#pragma unroll
  for (int j0 = 0; j0 < TN; j0 += JG) {
    float2 cs[JG][TM][4][2];
    // the lane's token row in Q' and in the caches (elements), -1 past the end
    int64_t rowq[JG], rowc[JG];
#pragma unroll
    for (int jj = 0; jj < JG; ++jj) {
      const int j = j0 + jj;
      const int m = m0 + tw * 32 * TN + j * 32 + l32;
      const int mc = min(m, a.M - 1);
      const int b = mc / n32, i_tok = mc - b * n32;
      rowq[jj] = m < a.M ? (int64_t)m * a.H * D : -1;
      rowc[jj] = ((int64_t)b * a.H * a.cap + a.cache_pos + i_tok) * D;
      const Pos p = decode_pos(a.tok_off + (uint32_t)i_tok, a.per_frame, a.gw, a.t0);
      // per-lane table pointers of the three axes (into the table, or its
      // copy in LDS), offset so that entry q of the lane's pair set is
      // ptr[axis][q] (the high half-wave's pairs are 2 further on)
      auto fetch = [&](auto base) {
        decltype(base) ax[3] = {base + (p.t - tv.t_lo) * HT + 2 * hf,
                                base + tv.base_h + p.h * HH - HT + 2 * hf,
                                base + tv.base_w + p.w * HH - HT - HH + 2 * hf};
        auto axis = [](int q) { return q < HT ? 0 : q < HT + HH ? 1 : 2; };
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (fw0 + 32 * i >= a.F || part[i] >= 2) continue;
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int q0 = ((32 * i) % D) / 2 + 4 * g + e;  // pair of the low half-wave
              const int a0 = axis(q0), a1 = axis(q0 + 2);
              const auto ptr = a0 == a1 ? ax[a0] : (hf ? ax[a1] : ax[a0]);
              const auto v = ptr[q0];
              cs[jj][i][g][e] = make_float2(v.x, v.y);
            }
        }
      };
      fetch(tl);
    }
#pragma unroll
    for (int jj = 0; jj < JG; ++jj) {
      const int j = j0 + jj;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (fw0 + 32 * i >= a.F) continue;
        // the block's base (scalar) plus the lane's token row
        uint16_t *base = part[i] == 0 ? a.q_out : part[i] == 1 ? a.k_cache : a.v_cache;
        base += (int64_t)head[i] * (part[i] == 0 ? D : a.cap * D) + (32 * i) % D;
        uint16_t *dst = rowq[jj] < 0 ? nullptr
                        : base + (part[i] == 0 ? rowq[jj] : rowc[jj]) + 8 * hf;
        if (part[i] < 2)
          store_block<true>(acc[i][j], cs[jj][i], dst);
        else
          store_block<false>(acc[i][j], cs[jj][i], dst);
      }
    }
  }
}

// TM x TN accumulator blocks (32 x 32) per wavefront; the 4 wavefronts
// tile the workgroup 2 x 2, so a workgroup covers 64 TM features x 64 TN
// tokens.  NS ring stages of 64 C-values each; D is head_dim.
template <int TM, int TN, int NS, int D>
__global__ void __launch_bounds__(kNW * 64, 1) qkv_rope_kernel(QkvKArgs a) {
  constexpr int kBM = 64 * TM, kBN = 64 * TN;
  constexpr int kACells = kBM * 8, kBCells = kBN * 8;  // 8 cells of 16 bytes per row
  constexpr int kStageCells = kACells + kBCells;
  constexpr int kAInstr = kACells / 64, kBInstr = kBCells / 64;
  // each wavefront issues 2 TM copies of A and 2 TN of B per stage (the
  // same count for all), so "at most k stages' copies pending" is an exact
  // vmcnt count
  constexpr int kDma = 2 * (TM + TN);
  static_assert(kAInstr == kNW * 2 * TM && kBInstr == kNW * 2 * TN, "copies split evenly");
  static_assert((NS - 1) * kDma < 64, "vmcnt wait range");
  static_assert(NS * kStageCells * 16 <= 160 * 1024, "LDS");
  __shared__ uint4 ring[NS * kStageCells];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int l32 = lane & 31;
  const int fw = wave & 1, tw = wave >> 1;

  int f0, m0;
  tile_origin(a, kBM, kBN, f0, m0);

  // ---- per-lane DMA offsets (bytes from the tile's first row, column 0).
  // LDS row r holds its 8 chunks of 8 C-values (128 bytes) in swizzled
  // order: physical cell p has chunk p ^ ((r >> 1) & 7), so the 16 rows a
  // quarter-wavefront reads fall on distinct bank groups.  Rows past the
  // matrix re-read its last row. ----
  auto cell_off = [&](int cell, int rows_valid) -> uint32_t {
    int row = cell >> 3;
    const int c = (cell & 7) ^ ((row >> 1) & 7);
    row = min(row, rows_valid - 1);
    return (uint32_t)row * (uint32_t)a.C * 2u + (uint32_t)(c * 16);
  };
  // copy slot s of this wavefront: A instruction wave + 4 s for s < 2 TM,
  // B instruction wave + 4 (s - 2 TM) after
  uint32_t dma_off[kDma];
#pragma unroll
  for (int s = 0; s < kDma; ++s)
    dma_off[s] = s < 2 * TM ? cell_off((wave + s * kNW) * 64 + lane, a.F - f0)
                            : cell_off((wave + (s - 2 * TM) * kNW) * 64 + lane, a.M - m0);
  typedef __attribute__((address_space(3))) char lds_char_t;
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(lds_char_t *)reinterpret_cast<char *>(ring));
  const uint16_t *wa = a.w + (int64_t)f0 * a.C;
  const uint16_t *xb = a.x + (int64_t)m0 * a.C;
  const int nk = a.C / kBK;
  // copy o of stage ks (clamped to the last stage) into ring slot `slot`
  auto dma1 = [&](int o, int ks, int slot) {
    const int c0 = __builtin_amdgcn_readfirstlane(min(ks, nk - 1)) * kBK;
    const uint32_t adst = ring_lds + (uint32_t)slot * (kStageCells * 16);
    if (o < 2 * TM)
      lds_dma16(wa + c0, dma_off[o], adst + (wave + o * kNW) * 1024);
    else
      lds_dma16(xb + c0, dma_off[o], adst + kACells * 16 + (wave + (o - 2 * TM) * kNW) * 1024);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // A stage is consumed in two halves of 32 C-values (2 sub-steps of 16);
  // fragments of one half: [sub-step][block] for A (features) and B (tokens).
  const int sw = (l32 >> 1) & 7;
  constexpr int NM = 2 * TM * TN;        // products per half
  constexpr int NF = 2 * (TM + TN);      // fragment reads per half
  // fragment f of half `h` of the stage in ring slot `slot`
  auto frag1 = [&](int f, int slot, int h, bf16x8_t (&af)[2][TM], bf16x8_t (&bfr)[2][TN]) {
    const uint4 *__restrict__ at = ring + slot * kStageCells;
    const int kk = f / (TM + TN), q = f % (TM + TN);
    const int chunk = (h * 4 + kk * 2 + hf) ^ sw;
    if (q < TM)
      af[kk][q] = __builtin_bit_cast(bf16x8_t, at[(fw * 32 * TM + q * 32 + l32) * 8 + chunk]);
    else
      bfr[kk][q - TM] = __builtin_bit_cast(bf16x8_t, at[kACells + (tw * 32 * TN + (q - TM) * 32 + l32) * 8 + chunk]);
  };
  auto mfma1 = [&](int t, const bf16x8_t (&af)[2][TM], const bf16x8_t (&bfr)[2][TN]) {
    const int kk = t / (TM * TN), i = (t / TN) % TM, j = t % TN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bfr[kk][j], acc[i][j], 0, 0, 0);
  };

  // ---- main loop.  Stage ks, first half: the matrix cores work on its
  // first 32 C-values (fragments in buffer 0) while its second half's
  // fragments are read into buffer 1.  Then wait for stage ks+1, barrier,
  // second half: products from buffer 1 while the wavefront issues the
  // copy of stage ks+NS into the slot of stage ks (every wavefront read its
  // fragments before the barrier) and reads stage ks+1's first half into
  // buffer 0.  One product, then one or two of the other operations; the
  // order is pinned with scheduling barriers.  Past the last stage the
  // copies repeat it (into slots nobody reads again), so every step has the
  // same number of copies in flight. ----
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int o = 0; o < kDma; ++o) dma1(o, s, s);
  wait_vmcnt<(NS - 1) * kDma>();  // stage 0 landed
  __syncthreads();
  bf16x8_t fa0[2][TM], fb0[2][TN], fa1[2][TM], fb1[2][TN];
#pragma unroll
  for (int f = 0; f < NF; ++f) frag1(f, 0, 0, fa0, fb0);

  constexpr int R0 = (NF + NM - 1) / NM;
  constexpr int R1 = (kDma + NF + NM - 1) / NM;
  for (int ks = 0; ks < nk; ++ks) {
    const int slot = ks % NS;
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      mfma1(t, fa0, fb0);
#pragma unroll
      for (int r = 0; r < R0; ++r)
        if (t * R0 + r < NF) frag1(t * R0 + r, slot, 1, fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // stage ks+1 has landed once only stages ks+2 .. ks+NS-1 are pending
    wait_vmcnt<(NS - 2) * kDma>();
    __syncthreads();
    const int nslot = (ks + 1) % NS;
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      mfma1(t, fa1, fb1);
#pragma unroll
      for (int r = 0; r < R1; ++r) {
        const int o = t * R1 + r;
        if (o < kDma)
          dma1(o, ks + NS, slot);
        else if (o - kDma < NF)
          frag1(o - kDma, nslot, 0, fa0, fb0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();  // no copy may still be writing LDS when the workgroup ends

  // token blocks in gather batches of 2 or 3 (4 would not fit in registers)
  rope_store_tile<TM, TN, TN == 4 ? 2 : TN, D, false>(a, acc, f0, m0, fw, tw, l32, hf, nullptr,
                                        TabView{0, (int)a.tg.base_h, (int)a.tg.base_w});
}


// One 32x32x16 bf16 product into an accumulator block held in the
// accumulation registers (AGPR) or in vector registers, through asm so that
// the register file is fixed: the compiler would otherwise put every
// accumulator in the accumulation registers.  Dependent products on one
// block are a whole sub-step apart, and the callers add the wait states
// before the results are read.
template <bool AGPR>
__device__ inline void mfma_reg(f32x16_t &c, bf16x8_t a, bf16x8_t b) {
  if constexpr (AGPR)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// An empty asm that claims to modify c: writes of c before it stay before
// it, reads after it stay after it, and it keeps its place among the other
// asm statements (where the wait states are).
template <bool AGPR>
__device__ inline void pin_reg(f32x16_t &c) {
  if constexpr (AGPR)
    asm volatile("" : "+a"(c));
  else
    asm volatile("" : "+v"(c));
}

// Wide tile: 4 wavefronts tile the workgroup 2 (features) x 2 (tokens) as
// above, but each wavefront holds TM x TN = 4 x 6 accumulator blocks (128
// features x 192 tokens), so a workgroup covers 256 features x 384 tokens
// and every byte copied into LDS feeds twice the products of the narrow
// tile's token width 3.  C is walked in stages of 32 (64-byte row segments)
// through an NS-stage ring, the copies running NS-2 stages ahead.  The
// fragments of one 16-wide sub-step are held in registers: A block i is
// re-read for the next sub-step as soon as its last product has issued, B
// alternates between two register sets.
template <int TM, int TN, int NS, int D>
__global__ void __launch_bounds__(kNW * 64, 1) qkv_rope_wide_kernel(QkvKArgs a) {
  constexpr int kBM = 64 * TM, kBN = 64 * TN;
  constexpr int kACells = kBM * 4, kBCells = kBN * 4;  // 4 cells of 16 bytes per row
  constexpr int kStageCells = kACells + kBCells;
  constexpr int kAW = kACells / 64 / kNW, kBW = kBCells / 64 / kNW;  // copies per wavefront
  static_assert(kAW * kNW * 64 == kACells && kBW * kNW * 64 == kBCells, "copies split evenly");
  constexpr int kDma = kAW + kBW;
  static_assert(NS >= 3 && (NS - 2) * kDma < 64, "ring depth, vmcnt wait range");
  static_assert(NS * kStageCells * 16 + kQkvTabBytes <= 160 * 1024, "LDS");
  __shared__ uint4 ring[NS * kStageCells];
  __shared__ f32x2_t tab[kQkvTabBytes / 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int l32 = lane & 31;
  const int fw = wave & 1, tw = wave >> 1;
  int f0, m0;
  tile_origin(a, kBM, kBN, f0, m0);
  // the table rows of the epilogue, copied while the first stages load (the
  // prologue's vmcnt wait and barrier before the first fragment reads
  // publish them: the copies are issued before the stages')
  lds_f2 *tl = (lds_f2 *)reinterpret_cast<f32x2_t *>(tab);
  typedef __attribute__((address_space(3))) char lds_char_t;
  const TabView tv = dma_table<D>(
      a, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char_t *)reinterpret_cast<char *>(tab)),
      wave, lane);

  // ---- per-lane copy offsets.  LDS row r holds its 4 chunks of 8 C-values
  // (64 bytes) in swizzled order: physical cell p has chunk p ^ ((r >> 2) &
  // 3), so the 16 rows a quarter-wavefront reads fall on distinct banks.
  // Rows past the matrix re-read its last row. ----
  auto cell_off = [&](int cell, int rows_valid) -> uint32_t {
    int row = cell >> 2;
    const int c = (cell & 3) ^ ((row >> 2) & 3);
    row = min(row, rows_valid - 1);
    return (uint32_t)row * (uint32_t)a.C * 2u + (uint32_t)(c * 16);
  };
  uint32_t dma_off[kDma];
#pragma unroll
  for (int o = 0; o < kDma; ++o)
    dma_off[o] = o < kAW ? cell_off((wave + o * kNW) * 64 + lane, a.F - f0)
                         : cell_off((wave + (o - kAW) * kNW) * 64 + lane, a.M - m0);
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(lds_char_t *)reinterpret_cast<char *>(ring));
  const uint16_t *wa = a.w + (int64_t)f0 * a.C;
  const uint16_t *xb = a.x + (int64_t)m0 * a.C;
  const int nk = a.C / 32;
  // copy o of stage ks (clamped to the last stage) into ring slot `slot`
  auto dma1 = [&](int o, int ks, int slot) {
    const int c0 = __builtin_amdgcn_readfirstlane(min(ks, nk - 1)) * 32;
    const uint32_t adst = ring_lds + (uint32_t)slot * (kStageCells * 16);
    if (o < kAW)
      lds_dma16(wa + c0, dma_off[o], adst + (wave + o * kNW) * 1024);
    else
      lds_dma16(xb + c0, dma_off[o], adst + kACells * 16 + (wave + (o - kAW) * kNW) * 1024);
  };

  // the accumulators (16 TM TN registers a lane) exceed the 256
  // accumulation registers: block columns j < kAgprCols live there, the
  // rest in vector registers
  constexpr int kAgprCols = 256 / (16 * TM);
  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto pin_acc = [&]() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if (j < kAgprCols)
          pin_reg<true>(acc[i][j]);
        else
          pin_reg<false>(acc[i][j]);
      }
  };

  // fragment of A block i / B block j for sub-step kk of the stage in `slot`
  const int sw = (l32 >> 2) & 3;
  auto frag_a = [&](int slot, int kk, int i) {
    const uint4 *__restrict__ at = ring + slot * kStageCells;
    return __builtin_bit_cast(bf16x8_t, at[(fw * 32 * TM + i * 32 + l32) * 4 + ((kk * 2 + hf) ^ sw)]);
  };
  auto frag_b = [&](int slot, int kk, int j) {
    const uint4 *__restrict__ at = ring + slot * kStageCells + kACells;
    return __builtin_bit_cast(bf16x8_t, at[(tw * 32 * TN + j * 32 + l32) * 4 + ((kk * 2 + hf) ^ sw)]);
  };

  // ---- main loop.  Step s: wait for this wavefront's copies of stage s+1,
  // barrier (every wavefront's copies of it have landed, and every
  // wavefront has finished reading stage s-1), then the two sub-steps of
  // stage s, with the copies of stage s+NS-1 into the slot of stage s-1
  // spread over both.
  // Each sub-step's products run block row by block row; the reads of the
  // next sub-step's fragments (stage s's second half, or stage s+1's first)
  // are spread between them.  Past the last stage the copies repeat it
  // (into slots nobody reads again), so every step has the same number of
  // copies in flight. ----
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
#pragma unroll
    for (int o = 0; o < kDma; ++o) dma1(o, s, s);
  wait_vmcnt<(NS - 2) * kDma>();  // stage 0 landed
  __syncthreads();
  // the zeroed accumulators are read by asm products: wait states after
  // their last write
  pin_acc();
  asm volatile("s_nop 4" ::: "memory");
  bf16x8_t fa[TM], fb0[TN], fb1[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) fa[i] = frag_a(0, 0, i);
#pragma unroll
  for (int j = 0; j < TN; ++j) fb0[j] = frag_b(0, 0, j);

  // one sub-step: products from fa and bc; copies c_lo .. c_hi-1 of stage
  // cs into slot cslot go after every fourth product (a step's copies are
  // split between its two sub-steps, so they reach the address unit evenly
  // rather than in one burst), the reads of the next sub-step's B fragments
  // (slot nslot, sub-step nkk) into bn after the odd products; A block i is
  // re-read into fa after its row of products
  auto substep = [&](const bf16x8_t (&bc)[TN], bf16x8_t (&bn)[TN], int nslot, int nkk,
                     bool read_next, int c_lo, int c_hi, int cs, int cslot) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if (j < kAgprCols)
          mfma_reg<true>(acc[i][j], fa[i], bc[j]);
        else
          mfma_reg<false>(acc[i][j], fa[i], bc[j]);
        const int t = i * TN + j;
        if (t % 4 == 0 && c_lo + t / 4 < c_hi) dma1(c_lo + t / 4, cs, cslot);
        if (read_next && (t & 1) && (t >> 1) < TN) bn[t >> 1] = frag_b(nslot, nkk, t >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (read_next) fa[i] = frag_a(nslot, nkk, i);
    }
  };
  auto step = [&](int s, auto read_next) {
    constexpr bool kRead = decltype(read_next)::value;
    // stage s+1 has landed once only stages s+2 .. s+NS-2 are pending
    wait_vmcnt<(NS - 3) * kDma>();
    __syncthreads();
    const int cslot = (s + NS - 1) % NS, slot = s % NS, nslot = (s + 1) % NS;
    substep(fb0, fb1, slot, 1, true, 0, kDma / 2, s + NS - 1, cslot);
    substep(fb1, fb0, nslot, 0, kRead, kDma / 2, kDma, s + NS - 1, cslot);
  };
  for (int s = 0; s < nk - 1; ++s) step(s, std::true_type());
  step(nk - 1, std::false_type());
  wait_vmcnt<0>();  // no copy may still be writing LDS when the workgroup ends
  // the products are issued through asm, whose results the compiler does
  // not track: 24 wait states before the accumulators are read
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  pin_acc();

  rope_store_tile_wide<TM, TN, D>(a, acc, f0, m0, fw, tw, l32, hf, tl, tv);
}

}  // namespace

hipError_t launch_qkv_rope(const QkvArgs &q, hipStream_t s) {
  const RopeSplit sp = rope_split(q.D);
  QkvKArgs a;
  a.x = static_cast<const uint16_t *>(q.x);
  a.w = static_cast<const uint16_t *>(q.w);
  a.q_out = static_cast<uint16_t *>(q.q_out);
  a.k_cache = static_cast<uint16_t *>(q.k_cache);
  a.v_cache = static_cast<uint16_t *>(q.v_cache);
  a.table = reinterpret_cast<const float2 *>(q.table);
  a.cap = q.cap;
  a.cache_pos = q.cache_pos;
  a.n = q.n;
  a.M = (int)((int64_t)q.B * q.n);
  a.F = 3 * q.H * q.D;
  a.f_begin = q.q_out != nullptr ? 0 : q.H * q.D;
  a.C = q.C;
  a.H = q.H;
  a.D = q.D;
  a.per_frame = (uint32_t)q.grid_h * (uint32_t)q.grid_w;
  a.gw = (uint32_t)q.grid_w;
  a.t0 = (uint32_t)q.t0;
  a.tok_off = (uint32_t)q.tok_off;
  a.tg.ht = (uint32_t)(sp.dt / 2);
  a.tg.hh = (uint32_t)(sp.dh / 2);
  a.tg.base_h = (uint32_t)q.max_t * a.tg.ht;
  a.tg.base_w = a.tg.base_h + (uint32_t)q.max_h * a.tg.hh;
  // token-tile width: the fewest tile-rounds over the chip's CUs, weighted
  // by the tile's width; ties go to the wider tile
  const int n_ft = (a.F - a.f_begin + 255) / 256;
  const int n_cu = device_cu_count();
  // the wide tile (6 blocks) stages the table rows in LDS beside its ring
  int t_lo;
  const int rows = q.D == 128 ? staged_rows<128>(a.t0, a.tok_off, q.n, a.per_frame, a.gw, t_lo)
                              : staged_rows<64>(a.t0, a.tok_off, q.n, a.per_frame, a.gw, t_lo);
  // (the last 256-byte copy of the rows may run past them)
  const bool wide_ok = (int64_t)rows * 8 + 256 <= kQkvTabBytes;
  int best_tn = 4;
  int64_t best_cost = -1;
  for (int tn : {6, 4, 3, 2}) {
    if (tn == 6 && !wide_ok) continue;
    const int64_t tiles = (int64_t)n_ft * ((a.M + 64 * tn - 1) / (64 * tn));
    const int64_t cost = (tiles + n_cu - 1) / n_cu * tn;
    if (best_cost < 0 || cost < best_cost) best_cost = cost, best_tn = tn;
  }
  const int64_t grid = (int64_t)n_ft * ((a.M + 64 * best_tn - 1) / (64 * best_tn));
  // 6 feature tiles per group: an XCD's 32 concurrent tiles then cover
  // about 6 x 5 tiles, near the fewest distinct rows of W and X for 32 tiles
  a.fg = min(n_ft, 6);
  // ring depth: as many stages as fit in LDS (64-wide: 2 or 3; 32-wide: 3,
  // beside the table rows)
  const dim3 g((unsigned)grid), blk(kNW * 64);
  if (q.D == 128) {
    if (best_tn == 6)
      qkv_rope_wide_kernel<4, 6, 3, 128><<<g, blk, 0, s>>>(a);
    else if (best_tn == 4)
      qkv_rope_kernel<4, 4, 2, 128><<<g, blk, 0, s>>>(a);
    else if (best_tn == 3)
      qkv_rope_kernel<4, 3, 2, 128><<<g, blk, 0, s>>>(a);
    else
      qkv_rope_kernel<4, 2, 3, 128><<<g, blk, 0, s>>>(a);
  } else {
    if (best_tn == 6)
      qkv_rope_wide_kernel<4, 6, 3, 64><<<g, blk, 0, s>>>(a);
    else if (best_tn == 4)
      qkv_rope_kernel<4, 4, 2, 64><<<g, blk, 0, s>>>(a);
    else if (best_tn == 3)
      qkv_rope_kernel<4, 3, 2, 64><<<g, blk, 0, s>>>(a);
    else
      qkv_rope_kernel<4, 2, 3, 64><<<g, blk, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace crattn
