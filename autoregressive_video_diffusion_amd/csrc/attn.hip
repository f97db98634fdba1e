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
#include "../../include/crattn.h"

#include <math.h>

#include <algorithm>

namespace crattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X

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
  float scale_log2;
  int64_t seg0_rows, tiles0, tiles_full, n_full, last_rows, n_tiles;
  int splits;
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

template <int CPR>
__device__ inline int k_cell(int row, int chunk) {
  return row * CPR + (chunk ^ (row & (CPR - 1)));
}

// V octet cell (g, d) -> index of its 16-byte cell in LDS.  The XOR spreads
// the staging writes of one row group over banks; reads of 32 consecutive d
// stay within one 512-byte run.
template <int D>
__device__ inline int v_cell(int g, int d) {
  return g * D + (d ^ ((d >> 3) & 7));
}

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

template <int D, int NW, int QB, int BN, int MINB>
__global__ void __launch_bounds__(NW * 64, MINB) attn_fwd_kernel(AttnKArgs a) {
  constexpr int kBN = BN;
  constexpr int T = NW * 64;
  constexpr int DK = D / 16;    // k-steps of the QK product
  constexpr int DB = D / 32;    // 32-dim blocks of O
  constexpr int KB = kBN / 32;  // 32-key blocks per tile
  constexpr int CPR = D / 8;    // 16-byte chunks per K row
  constexpr int BM = NW * QB * 32;
  constexpr int K_CELLS = kBN * CPR;        // 16-byte cells of a K tile
  constexpr int K_PER_T = (K_CELLS + T - 1) / T;
  constexpr int V_ITEMS = (kBN / 4) * CPR;  // (4 keys x 8 dims) items of a V tile
  constexpr int V_PER_T = (V_ITEMS + T - 1) / T;

  __shared__ uint4 k_lds[2][K_CELLS];
  __shared__ uint4 v_lds[2][kBN * D / 8];  // key-octet cells, 16 bytes each

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;
  const int l32 = lane & 31;

  // ---- which (b, h, query tile, key split) this workgroup computes ----
  // Workgroups are dealt to the 8 XCDs round-robin (XCD = blockIdx % 8).
  // Renumber so that consecutive work items -- the query tiles of one head,
  // which stream the same K/V -- land on the same XCD and share its L2.
  int64_t bid;
  {
    const int64_t G = gridDim.x;
    const int64_t xcd = blockIdx.x % kXcds, idx = blockIdx.x / kXcds;
    const int64_t q = G / kXcds, r = G % kXcds;
    bid = xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  }
  const int split = (int)(bid % a.splits);
  bid /= a.splits;
  const int64_t tile = bid % a.n_tiles;
  bid /= a.n_tiles;
  const int h = (int)(bid % a.H);
  const int b = (int)(bid / a.H);

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
  const int64_t row0 = seg_row0 + t_in * BM;
  const int64_t nrows = min((int64_t)BM, seg_rows - t_in * BM);
  const int64_t q_chunk = a.q_pos0 / a.L + seg;
  const int64_t limit = min(a.kv_len, (q_chunk + 1) * a.L);
  const int64_t nkt = (limit + kBN - 1) / kBN;
  const int64_t kt_begin = split * nkt / a.splits;
  const int64_t kt_end = (split + 1) * nkt / a.splits;

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
    const uint16_t *qp = a.q + (((int64_t)b * a.Lq + row) * a.H + h) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (ok) x = *reinterpret_cast<const uint4 *>(qp + ks * 16);
      qf[qb][ks] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

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

  // ---- global -> register prefetch of one K/V tile (rows past limit = 0) ----
  uint4 kreg[K_PER_T];
  uint4 vreg[V_PER_T][4];
  auto gload = [&](int64_t kt) {
    const int64_t key0 = kt * kBN;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int id = tid + i * T;
      kreg[i] = make_uint4(0, 0, 0, 0);
      if (id < K_CELLS) {
        const int r = id / CPR, c = id % CPR;
        if (key0 + r < limit) kreg[i] = *reinterpret_cast<const uint4 *>(kh + (key0 + r) * D + c * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int id = tid + i * T;
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[i][r] = make_uint4(0, 0, 0, 0);
      if (id < V_ITEMS) {
        const int c = id % CPR, kq = id / CPR;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t key = key0 + kq * 4 + r;
          if (key < limit) vreg[i][r] = *reinterpret_cast<const uint4 *>(vh + key * D + c * 8);
        }
      }
    }
  };
  // ---- registers -> LDS: K as swizzled rows, V transposed to key octets ----
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int id = tid + i * T;
      if (id < K_CELLS) k_lds[buf][k_cell<CPR>(id / CPR, id % CPR)] = kreg[i];
    }
    uint2 *const v_half = reinterpret_cast<uint2 *>(v_lds[buf]);
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int id = tid + i * T;
      if (id >= V_ITEMS) continue;
      const int c = id % CPR, kq = id / CPR;
      const uint32_t w0[4] = {vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w};
      const uint32_t w1[4] = {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w};
      const uint32_t w2[4] = {vreg[i][2].x, vreg[i][2].y, vreg[i][2].z, vreg[i][2].w};
      const uint32_t w3[4] = {vreg[i][3].x, vreg[i][3].y, vreg[i][3].z, vreg[i][3].w};
      const int g = kq >> 1, half = kq & 1;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        uint2 cell;
        cell.x = __builtin_amdgcn_perm(w1[dd >> 1], w0[dd >> 1], sel);
        cell.y = __builtin_amdgcn_perm(w3[dd >> 1], w2[dd >> 1], sel);
        v_half[v_cell<D>(g, c * 8 + dd) * 2 + half] = cell;
      }
    }
  };

  if (kt_begin < kt_end) gload(kt_begin);
  for (int64_t kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (int)((kt - kt_begin) & 1);
    const int64_t key0 = kt * kBN;
    lstore(buf);
    __syncthreads();
    // The next tile's loads are in flight while this tile is computed.  One
    // barrier per tile suffices: a wavefront can only overwrite this buffer
    // two tiles later, after every wavefront has passed the next barrier.
    if (kt + 1 < kt_end) gload(kt + 1);
    if (!active) continue;

    // ---- S^T = K Q^T for this wavefront's queries ----
    f32x16_t s[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int row = kb * 32 + kperm;
        const bf16x8_t kf =
            __builtin_bit_cast(bf16x8_t, k_lds[buf][k_cell<CPR>(row, 2 * ks + hf)]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], s[kb][qb], 0, 0, 0);
      }
    }
    // ---- mask keys past the visible limit (last tile only) ----
    if (key0 + kBN > limit) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool dead = key0 + kb * 32 + acc_key(r, hf) >= limit;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if (dead) s[kb][qb][r] = -INFINITY;
        }
    }
    // ---- online softmax, per query column, lazy rescale ----
    bf16x8_t pf[QB][KB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      const float m_cand = half_swap_max(mx) * a.scale_log2;
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
      const float m_use = m_run[qb];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          uint32_t pk[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 =
                __builtin_amdgcn_exp2f(fmaf(s[kb][qb][h2 * 8 + 2 * e], a.scale_log2, -m_use));
            const float p1 =
                __builtin_amdgcn_exp2f(fmaf(s[kb][qb][h2 * 8 + 2 * e + 1], a.scale_log2, -m_use));
            rs += p0 + p1;
            pk[e] = pack_bf16(p0, p1);
          }
          pf[qb][kb][h2] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
        }
      }
      l_run[qb] += rs;
    }
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int g = kb * 4 + h2 * 2 + hf;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, v_lds[buf][v_cell<D>(g, db * 32 + l32)]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kb][h2], o[db][qb], 0, 0, 0);
        }
      }
    }
  }

  if (!active) return;
  // ---- epilogue: normalise and store ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = half_swap_sum(l_run[qb]);
    const int64_t row = wrow0 + qb * 32 + l32;
    if (row >= row0 + nrows) continue;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const float lse2 = lt > 0.f ? m_run[qb] + __log2f(lt) : -INFINITY;
    if (a.splits == 1) {
      uint16_t *op = a.out + (((int64_t)b * a.Lq + row) * a.H + h) * D + hf * 4;
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
      if (hf == 0 && a.lse != nullptr) a.lse[((int64_t)b * a.H + h) * a.Lq + row] = lse2 * kLn2;
    } else {
      const int64_t prow = (((int64_t)split * a.B + b) * a.H + h) * a.Lq + row;
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
}

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

// Launch shapes: waves per workgroup, 32-query blocks per wave, minimum
// resident workgroups per compute unit.
struct FwdShape {
  int waves, qb, bn;
};
FwdShape fwd_shape(int D) {
  (void)D;
  return FwdShape{8, 1, 64};
}

template <int D, int NW, int QB, int BN, int MINB>
hipError_t launch_fwd(const AttnKArgs &k, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW, QB, BN, MINB>), dim3((unsigned)grid), dim3(NW * 64),
                     0, s, k);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int B, int H, int64_t Lq, int64_t kv_len, int64_t q_pos0,
                   int64_t chunk_tokens, int D, bool allow_split) {
  AttnPlan p{};
  p.d = D;
  const FwdShape fs = fwd_shape(D);
  p.bm = fs.waves * fs.qb * 32;
  p.bn = fs.bn;
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
  hipError_t e;
  if (a.D == 128)
    e = launch_fwd<128, 8, 1, 64, 1>(k, p.grid, s);
  else
    e = launch_fwd<64, 8, 1, 64, 1>(k, p.grid, s);
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
