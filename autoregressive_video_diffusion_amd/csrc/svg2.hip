// Semantic-aware permutation for sparse attention: k-means of the queries
// and keys of every head, the stable reordering of the tokens by cluster,
// centroid top-p selection of key clusters per query cluster, and the key
// lists and query tiles of the sparse attention, for AMD CDNA4 (gfx950).
// The attention itself is the gather instance of the attention kernel
// (attn.hip).
//
// Source: "Sparse VideoGen2" summary, §2.A (k-means on Q and K, contiguous
// clusters), §2.B (centroid score estimate, top-p), §2.C (the previous
// step's centroids start k-means; sparse key loads, dense query tiles).
//
// Everything here is small next to the attention: one Lloyd iteration reads
// the tokens twice (assignment, centroid update) and the centroids once per
// token block; the selection reads the centroids of one head per query
// cluster.  The contraction of the assignment (tokens x centroids) runs on
// bf16 MFMA with every centroid split into two bf16 parts (hi = bf16(c),
// lo = bf16(c - hi)): the tokens are bf16 already, the products are exact
// and the sums fp32, so the distances that decide the nearest centroid carry
// about 2^-17 relative error instead of bf16's 2^-8.
#include "crattn_internal.h"
#include <math.h>
#include <algorithm>
#include "../../include/crattn.h"

namespace crattn {
namespace {

constexpr int kMaxC = CRATTN_SVG2_MAX_C;
constexpr int kMaxN = CRATTN_SVG2_MAX_N;
constexpr int kMaxCand = CRATTN_SVG2_MAX_CAND;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round to nearest even), low half first.
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  f32x2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

__device__ inline float wave_sum(float s) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  return s;
}

__device__ inline const uint16_t *token_ptr(const KmArgs &a, int64_t bh, int64_t t) {
  const int64_t b = bh / a.H, h = bh - b * a.H;
  return a.x + b * a.sb + h * a.sh + t * a.sr;
}

// ---- initial centroids: centroid c = token floor(c n / C); grid B*H*C ----
template <int D>
__global__ void __launch_bounds__(D) svg2_init_kernel(KmArgs a0, KmArgs a1, uint32_t split) {
  const bool second = blockIdx.x >= split;  // two problems in one launch
  const KmArgs a = second ? a1 : a0;
  const uint32_t bid = second ? blockIdx.x - split : blockIdx.x;
  const int c = (int)(bid % (uint32_t)a.C);
  const int64_t bh = bid / (uint32_t)a.C;
  const int64_t t = (int64_t)c * a.n / a.C;
  a.cent[bh * a.cent_s + (int64_t)c * D + threadIdx.x] =
      __uint_as_float((uint32_t)token_ptr(a, bh, t)[threadIdx.x] << 16);
}

// ---- assignment: nearest centroid of every token ----
// One workgroup per 128 tokens of a head, 32 per wave.  The centroids are
// staged in LDS as bf16 hi and lo parts (rows padded by one 16-byte cell)
// with their fp32 squared norms (rows past C get +inf).  Each wave forms
// S^T = C X^T on v_mfma_f32_32x32x16_bf16, 32 centroids x 32 tokens per
// block, hi and lo products into one accumulator; lane l then holds token
// l mod 32 against centroid rows 8(r/4) + 4(l/32) + r%4 of register r, so
// the distance |c|^2 - 2 x.c and its minimum are in-lane, then one exchange
// with lane l xor 32.  Ties go to the lower centroid index.
//
// The workgroup's 128 tokens are also the block of the stable sort: each
// token's rank among the earlier tokens of the block with its cluster is
// stored with its cluster (cluster | rank << 16), and the block's count of
// every cluster goes to bcnt[head][block][cluster].
template <int D>
__global__ void __launch_bounds__(256) svg2_assign_kernel(KmArgs a0, KmArgs a1, uint32_t split) {
  const bool second = blockIdx.x >= split;  // two problems in one launch
  const KmArgs a = second ? a1 : a0;
  const uint32_t bid = second ? blockIdx.x - split : blockIdx.x;
  constexpr int CPR = D / 8, PITCH = CPR + 1, DK = D / 16;
  extern __shared__ uint4 dyn[];
  const int C = a.C, CP = (C + 31) & ~31;
  uint4 *hi = dyn;
  uint4 *lo = dyn + CP * PITCH;
  float *nrm = reinterpret_cast<float *>(dyn + 2 * CP * PITCH);
  float *npart = nrm + CP;  // [CP][CPR]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int nblk = (a.n + 127) / 128;
  const int blk = (int)(bid % (uint32_t)nblk);
  const int64_t bh = bid / (uint32_t)nblk;
  // this wave's tokens as B operands (16 dims x 32 tokens per k-step)
  const int t = blk * 128 + wave * 32 + l32;
  const uint16_t *xp = token_ptr(a, bh, min(t, a.n - 1)) + hf * 8;
  bf16x8_t xb[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks)
    xb[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(xp + ks * 16));
  // stage the centroids: 8 features per (row, cell)
  const float *cb = a.cent + bh * a.cent_s;
  for (int q = tid; q < CP * CPR; q += 256) {
    const int c = q / CPR, j = q - c * CPR;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < C) {
      const float4 u0 = *reinterpret_cast<const float4 *>(cb + (int64_t)c * D + j * 8);
      const float4 u1 = *reinterpret_cast<const float4 *>(cb + (int64_t)c * D + j * 8 + 4);
      v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
      v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
    }
    uint32_t h[4], l[4];
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = pack_bf16(v[2 * e], v[2 * e + 1]);
      const float r0 = v[2 * e] - __uint_as_float(h[e] << 16);
      const float r1 = v[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u);
      l[e] = pack_bf16(r0, r1);
      sq = fmaf(v[2 * e], v[2 * e], sq);
      sq = fmaf(v[2 * e + 1], v[2 * e + 1], sq);
    }
    hi[c * PITCH + j] = make_uint4(h[0], h[1], h[2], h[3]);
    lo[c * PITCH + j] = make_uint4(l[0], l[1], l[2], l[3]);
    npart[q] = sq;
  }
  __syncthreads();
  for (int c = tid; c < CP; c += 256) {
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < CPR; ++j) sq += npart[c * CPR + j];
    nrm[c] = c < C ? sq : INFINITY;
  }
  __syncthreads();
  float best = INFINITY;
  int bidx = 0;
  for (int cb0 = 0; cb0 < CP; cb0 += 32) {
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const int row = cb0 + l32;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, hi[row * PITCH + 2 * ks + hf]);
      const bf16x8_t al = __builtin_bit_cast(bf16x8_t, lo[row * PITCH + 2 * ks + hf]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xb[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xb[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = cb0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      const float dist = fmaf(-2.f, acc[r], nrm[c]);
      if (dist < best) {
        best = dist;
        bidx = c;
      }
    }
  }
  const float ob = __shfl_xor(best, 32, 64);
  const int oi = __shfl_xor(bidx, 32, 64);
  if (ob < best || (ob == best && oi < bidx)) bidx = oi;
  // rank in the block and the block's cluster counts (LDS reused: the
  // staged centroids are no longer read once every wave is here)
  __syncthreads();
  int *bc = reinterpret_cast<int *>(dyn);           // [128] clusters in token order
  int *cnt = bc + 128;                               // [CP] counts
  const int ti = wave * 32 + l32;
  const bool valid = t < a.n;
  if (hf == 0) bc[ti] = valid ? bidx : -1;
  for (int c = tid; c < CP; c += 256) cnt[c] = 0;
  __syncthreads();
  if (hf == 0 && valid) {
    int before = 0;
    const int4 *b4 = reinterpret_cast<const int4 *>(bc);
#pragma unroll 8
    for (int j4 = 0; j4 < 32; ++j4) {
      const int4 u = b4[j4];
      const int j = 4 * j4;
      before += (u.x == bidx && j < ti) + (u.y == bidx && j + 1 < ti) +
                (u.z == bidx && j + 2 < ti) + (u.w == bidx && j + 3 < ti);
    }
    atomicAdd(&cnt[bidx], 1);
    a.assign[bh * a.n + t] = bidx | (before << 16);
  }
  __syncthreads();
  int32_t *bcnt = a.bcnt + (bh * nblk + blk) * (int64_t)C;
  for (int c = tid; c < C; c += 256) bcnt[c] = cnt[c];
}

// Dynamic LDS bytes of the assignment for C clusters.
template <int D>
size_t assign_lds_bytes(int C) {
  const int CP = (C + 31) & ~31;
  return (size_t)2 * CP * (D / 8 + 1) * 16 + (size_t)CP * 4 + (size_t)CP * (D / 8) * 4;  // >= (128 + CP) * 4
}

// ---- stable counting sort by cluster: one workgroup of 16 waves per head ----
// The assignment left every token's cluster and rank inside its 128-token
// block, and every block's cluster counts.  The counts are scanned over the
// blocks per cluster, so the position of token t of cluster c in block b is
//   offsets[c] + (tokens of c in blocks before b) + (rank of t in b),
// which keeps every cluster's tokens in ascending order.
constexpr int kSortThreads = 1024;

__global__ void __launch_bounds__(kSortThreads) svg2_sort_kernel(KmArgs a0, KmArgs a1, uint32_t split) {
  const bool second = blockIdx.x >= split;  // two problems in one launch
  const KmArgs a = second ? a1 : a0;
  const uint32_t bid = second ? blockIdx.x - split : blockIdx.x;
  __shared__ uint16_t cnt[(kMaxN / 128) * kMaxC];  // [block][cluster]
  __shared__ int tot[kMaxC];
  __shared__ int coff[kMaxC + 1];
  __shared__ int segsum[kSortThreads];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t bh = bid;
  const int n = a.n, C = a.C;
  const int nblk = (n + 127) / 128;
  const int32_t *bc = a.bcnt + bh * nblk * (int64_t)C;
  for (int i = tid; i < nblk * C; i += kSortThreads) cnt[i] = (uint16_t)bc[i];
  __syncthreads();
  // exclusive scan of every cluster's counts over the blocks, in nseg runs
  // of consecutive blocks per cluster: run sums, a scan over the runs, then
  // each run rewritten from its base
  {
    const int nseg = min(32, kSortThreads / C);
    const int per = (nblk + nseg - 1) / nseg;
    const int c = tid % C, g = tid / C;
    const bool mine = g < nseg;
    const int b0 = min(g * per, nblk), b1 = min(b0 + per, nblk);
    if (mine) {
      int sum = 0;
      for (int blk = b0; blk < b1; ++blk) sum += cnt[blk * C + c];
      segsum[g * C + c] = sum;
    }
    __syncthreads();
    if (tid < C) {
      int run = 0;
      for (int k = 0; k < nseg; ++k) {
        const int x = segsum[k * C + tid];
        segsum[k * C + tid] = run;
        run += x;
      }
      tot[tid] = run;
    }
    __syncthreads();
    if (mine) {
      int run = segsum[g * C + c];
      for (int blk = b0; blk < b1; ++blk) {
        const int x = cnt[blk * C + c];
        cnt[blk * C + c] = (uint16_t)run;
        run += x;
      }
    }
  }
  __syncthreads();
  if (tid < 64) {
    // cluster offsets: exclusive scan of the totals, 64 clusters at a time
    int base = 0;
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const int x = c < C ? tot[c] : 0;
      int inc = x;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d, 64);
        if (lane >= d) inc += y;
      }
      if (c < C) coff[c] = base + inc - x;
      base += __shfl(inc, 63, 64);
    }
    if (lane == 0) coff[C] = base;
  }
  __syncthreads();
  int32_t *off = a.off + bh * a.off_s;
  for (int c = tid; c <= C; c += kSortThreads) off[c] = coff[c];
  int32_t *perm = a.perm + bh * a.perm_s;
  const int32_t *as = a.assign + bh * n;
#pragma unroll 4
  for (int t = tid; t < n; t += kSortThreads) {
    const int v = as[t];
    const int c = min(v & 0xffff, C - 1), r = v >> 16;
    perm[min(coff[c] + cnt[(t >> 7) * C + c] + r, n - 1)] = t;
  }
}

// ---- centroid update: the mean of each cluster's tokens, an empty cluster
// keeps its centroid.  One workgroup per cluster: D/8 lanes cover a token's
// row (16 bytes each), so a pass takes 256/(D/8) tokens; per-thread sums of
// a fixed set of tokens meet in LDS and are added in slot order. ----
template <int D>
__global__ void __launch_bounds__(256) svg2_update_kernel(KmArgs a0, KmArgs a1, uint32_t split) {
  const bool second = blockIdx.x >= split;  // two problems in one launch
  const KmArgs a = second ? a1 : a0;
  const uint32_t bid = second ? blockIdx.x - split : blockIdx.x;
  constexpr int LPR = D / 8;
  constexpr int RPP = 256 / LPR;
  __shared__ float part[RPP][D + 4];
  const int c = (int)(bid % (uint32_t)a.C);
  const int64_t bh = bid / (uint32_t)a.C;
  const int tid = threadIdx.x, sub = tid % LPR, slot = tid / LPR;
  const int32_t *off = a.off + bh * a.off_s;
  const int r0 = off[c], r1 = off[c + 1];
  if (r1 <= r0) return;
  const int32_t *pm = a.perm + bh * a.perm_s;
  const uint16_t *xb = token_ptr(a, bh, 0) + sub * 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = r0 + slot; r < r1; r += RPP) {
    const uint4 u = *reinterpret_cast<const uint4 *>(xb + (int64_t)pm[r] * a.sr);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[2 * e] += __uint_as_float(w[e] << 16);
      s[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[slot][sub * 8 + e] = s[e];
  __syncthreads();
  if (tid < D) {
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < RPP; ++k) tot += part[k][tid];
    a.cent[bh * a.cent_s + (int64_t)c * D + tid] = tot / (float)(r1 - r0);
  }
}

// ---- query tiles: every query cluster split into tiles of qtile rows, in
// cluster order; unused slots get zero rows.  Run by the first wave of the
// first query cluster's workgroup of each (b, h). ----
__device__ void write_query_tiles(const SvgPlanArgs &a, int64_t bh, int lane) {
  const int32_t *qo = a.q_off + bh * (a.Cq + 1);
  int4 *sl = reinterpret_cast<int4 *>(a.slots) + bh * a.n_slots;
  int base = 0;
  for (int i0 = 0; i0 < a.Cq; i0 += 64) {
    const int i = i0 + lane;
    const int cnt = i < a.Cq ? max(qo[i + 1] - qo[i], 0) : 0;
    const int nt = (cnt + a.qtile - 1) / a.qtile;
    int inc = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(inc, d, 64);
      if (lane >= d) inc += y;
    }
    const int first = base + inc - nt;
    for (int t = 0; t < nt && first + t < a.n_slots; ++t)
      sl[first + t] = make_int4(qo[i] + t * a.qtile, min(a.qtile, cnt - t * a.qtile), i, 0);
    base += __shfl(inc, 63, 64);
  }
  for (int s = base + lane; s < a.n_slots; s += 64) sl[s] = make_int4(0, 0, 0, 0);
}

// ---- selection and key list of one (b, h, query cluster) ----
// Scores of the candidates (4 lanes per candidate); shares
// w_j = n_j exp(s_j - max s); the candidates in decreasing share (ties:
// lower id first) are kept while the shares before them add up to less than
// p times the total -- found by radix selection of the cut, not by sorting.
// The kept ids are compacted in ascending order, their key counts scanned,
// and the list is copied in chunks of 16 entries, 16 lanes per chunk.
template <int D>
__global__ void __launch_bounds__(256) svg2_select_kernel(SvgPlanArgs a) {
  __shared__ float qc[D];
  __shared__ float w[kMaxCand];
  __shared__ unsigned long long bins[256];
  __shared__ unsigned long long sh_u[2];  // total, then the sum above the threshold
  __shared__ uint32_t sh_key;
  __shared__ int lpos_buf[kMaxCand + 1];
  __shared__ int flag[4];
  __shared__ int kept[kMaxCand];
  __shared__ int kstart[kMaxCand];
  __shared__ int cpos[kMaxCand + 1];  // first 16-entry chunk of each kept cluster
  __shared__ float redf[4];
  __shared__ int redi[4];
  __shared__ int st_s[kMaxCand];   // each candidate's first reordered row
  __shared__ int cnt_s[kMaxCand];  // and its token count
  __shared__ int4 chunk_s[256];    // a batch of list chunks: source, position, count, s L
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroups are dealt to the 8 XCDs in turn; the ones an XCD receives
  // take consecutive (b, h, cluster) items, so that its L2 fetches the
  // centroids and reorderings of about gridDim / (8 Cq) heads, not of all.
  const uint32_t nx = gridDim.x / 8, rx = gridDim.x % 8, x = blockIdx.x % 8, kx = blockIdx.x / 8;
  const uint32_t item = x < rx ? x * (nx + 1) + kx : rx * (nx + 1) + (x - rx) * nx + kx;
  const int i = (int)(item % (uint32_t)a.Cq);
  const int64_t bh = item / (uint32_t)a.Cq;
  const int NC = a.n_vis * a.Ck;
  const int32_t *qo = a.q_off + bh * (a.Cq + 1);
  int32_t *sel = a.sel + (bh * a.Cq + i) * (int64_t)NC;
  const int32_t *koff = a.k_off + bh * a.S * (int64_t)(a.Ck + 1);
  // Offsets come from svg2_kmeans; they are clamped to [0, L] anyway, so
  // that no read of k_perm leaves its slot.  Read once into LDS: every
  // phase below looks them up.
  auto start_of = [&](int j) { return st_s[j]; };
  auto count_of = [&](int j) { return cnt_s[j]; };
  if (i == 0 && wave == 0) write_query_tiles(a, bh, lane);
  if (qo[i + 1] <= qo[i]) {
    if (tid == 0) a.list_len[bh * a.Cq + i] = 0;
    for (int e = tid; e < NC; e += 256) sel[e] = -1;
    return;
  }
  if (tid < D) qc[tid] = a.q_cent[(bh * a.Cq + i) * D + tid];
  for (int j = tid; j < NC; j += 256) {
    const int sl = j / a.Ck, c = j - sl * a.Ck;
    const int64_t b0 = min(max((int64_t)koff[sl * (a.Ck + 1) + c], (int64_t)0), a.L);
    const int64_t e0 = min(max((int64_t)koff[sl * (a.Ck + 1) + c + 1], (int64_t)0), a.L);
    st_s[j] = (int)b0;
    cnt_s[j] = (int)max(e0 - b0, (int64_t)0);
  }
  __syncthreads();
  // 1. scores (-inf for empty clusters)
  {
    constexpr int TPI = 4, FPT = D / TPI;
    const int sub = tid % TPI;
    const float *kc = a.k_cent + bh * a.S * (int64_t)a.Ck * D;
    for (int j = tid / TPI; j < NC; j += 256 / TPI) {
      const float *row = kc + (int64_t)j * D + sub * FPT;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < FPT; d += 4) {
        const float4 x = *reinterpret_cast<const float4 *>(row + d);
        const int dd = sub * FPT + d;
        s += qc[dd] * x.x + qc[dd + 1] * x.y + qc[dd + 2] * x.z + qc[dd + 3] * x.w;
      }
#pragma unroll
      for (int m = TPI / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, TPI);
      if (sub == 0) w[j] = count_of(j) > 0 ? s * a.scale : -INFINITY;
    }
  }
  __syncthreads();
  // 2. shares
  float mx = -INFINITY;
  for (int j = tid; j < NC; j += 256) mx = fmaxf(mx, w[j]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  if (lane == 0) redf[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(redf[0], redf[1]), fmaxf(redf[2], redf[3]));
  for (int j = tid; j < NC; j += 256) {
    const int n = count_of(j);
    w[j] = n > 0 ? (float)n * __expf(w[j] - mx) : 0.f;
  }
  __syncthreads();
  // 3. the top-p cut without sorting.  Shares are non-negative floats, so
  // they order like their bit patterns; cumulative sums are taken in fixed
  // point (u = share x 2^24 rounded, 64-bit: exact and independent of the
  // order of addition).  A candidate is kept while the shares ranked before
  // it add up to less than cut = ceil(p x total).  Four rounds of radix
  // selection (8 bits each, from the top) find the bit pattern v of the
  // last kept share and the sum of all larger shares; of the candidates
  // equal to v, the lowest ids are kept until the cut is reached.
  auto key_of = [&](int j) { return __float_as_uint(w[j]); };
  auto u_of = [&](int j) { return (unsigned long long)rintf(w[j] * 16777216.f); };
  auto live = [&](int j) { return count_of(j) > 0; };
  {
    unsigned long long t = 0;
    for (int j = tid; j < NC; j += 256)
      if (live(j)) t += u_of(j);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
    if (tid == 0) sh_u[0] = 0;
    __syncthreads();
    if (lane == 0) atomicAdd(&sh_u[0], t);
    __syncthreads();
  }
  const bool all = a.p >= 1.f;
  const unsigned long long total = sh_u[0];
  const unsigned long long cut = (unsigned long long)ceil((double)a.p * (double)total);
  uint32_t prefix = 0, pmask = 0;
  unsigned long long above = 0;
  if (!all) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      bins[tid] = 0;
      __syncthreads();
      for (int j = tid; j < NC; j += 256) {
        const uint32_t kj = key_of(j);
        if (live(j) && (kj & pmask) == prefix) atomicAdd(&bins[(kj >> shift) & 255u], u_of(j));
      }
      __syncthreads();
      if (wave == 0) {
        // lane l holds bins 4l .. 4l+3; suffix sums over the lanes above
        unsigned long long b4[4], own = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          b4[e] = bins[4 * lane + e];
          own += b4[e];
        }
        unsigned long long suf = own;  // sum over lanes >= this one
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const unsigned long long y = __shfl_down(suf, d, 64);
          if (lane + d < 64) suf += y;
        }
        // highest bin b with above + (sum of bins >= b) >= cut
        unsigned long long acc = above + (suf - own);
        int best = -1;
        unsigned long long best_above = 0;
#pragma unroll
        for (int e = 3; e >= 0; --e) {
          if (best < 0 && acc + b4[e] >= cut) {
            best = 4 * lane + e;
            best_above = acc;
          }
          acc += b4[e];
        }
        const uint64_t bal = __builtin_amdgcn_ballot_w64(best >= 0);
        const int top = bal ? 63 - __builtin_clzll(bal) : 0;
        if (lane == top) {
          sh_key = (uint32_t)max(best, 0);
          sh_u[1] = best >= 0 ? best_above : above;
        }
      }
      __syncthreads();
      prefix |= sh_key << shift;
      pmask |= 255u << shift;
      above = sh_u[1];
      __syncthreads();
    }
  }
  // 4. the ties at the cut: each adds u(v), so the first
  // ceil((cut - above) / u(v)) of them (by id) are kept
  const uint32_t vkey = prefix;
  const unsigned long long uv = (unsigned long long)rintf(__uint_as_float(vkey) * 16777216.f);
  const unsigned long long need = cut > above ? cut - above : 0;
  const long long n_tie = all ? 0 : (uv > 0 ? (long long)((need + uv - 1) / uv) : (long long)NC);
  // 5. kept ids in ascending order: a ballot compaction, counting the ties
  // seen so far
  int n_kept = 0;
  long long ties = 0;
  for (int j0 = 0; j0 < NC; j0 += 256) {
    const int j = j0 + tid;
    const bool lv = j < NC && live(j);
    const uint32_t kj = lv ? key_of(j) : 0u;
    const bool tie = lv && !all && kj == vkey;
    const uint64_t tb = __builtin_amdgcn_ballot_w64(tie);
    if (lane == 0) flag[wave] = __builtin_popcountll(tb);
    __syncthreads();
    long long tie_rank = ties + __builtin_popcountll(tb & ((uint64_t(1) << lane) - 1));
    for (int v = 0; v < wave; ++v) tie_rank += flag[v];
    const bool k = lv && (all || kj > vkey || (tie && tie_rank < n_tie));
    ties += flag[0] + flag[1] + flag[2] + flag[3];
    __syncthreads();
    const uint64_t bal = __builtin_amdgcn_ballot_w64(k);
    if (lane == 0) redi[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int pos = n_kept;
    for (int v = 0; v < wave; ++v) pos += redi[v];
    if (k) kept[pos + __builtin_popcountll(bal & ((uint64_t(1) << lane) - 1))] = j;
    n_kept += redi[0] + redi[1] + redi[2] + redi[3];
    __syncthreads();
  }
  for (int e = tid; e < NC; e += 256) sel[e] = e < n_kept ? kept[e] : -1;
  // 6. list positions of the kept clusters (their key counts scanned in id
  // order) and of their 16-entry chunks
  int *lpos = lpos_buf;
  {
    int base = 0, cbase = 0;
    for (int k0 = 0; k0 < n_kept; k0 += 256) {
      const int k = k0 + tid;
      const int x = k < n_kept ? count_of(kept[k]) : 0;
      const int y = (x + 15) >> 4;
      if (k < n_kept) kstart[k] = start_of(kept[k]);
      int inc = x, cinc = y;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(inc, d, 64), v = __shfl_up(cinc, d, 64);
        if (lane >= d) {
          inc += u;
          cinc += v;
        }
      }
      if (lane == 63) {
        redi[wave] = inc;
        flag[wave] = cinc;
      }
      __syncthreads();
      int pre = base + inc - x, cpre = cbase + cinc - y;
      for (int v = 0; v < wave; ++v) {
        pre += redi[v];
        cpre += flag[v];
      }
      if (k < n_kept) {
        lpos[k] = pre;
        cpos[k] = cpre;
      }
      base += redi[0] + redi[1] + redi[2] + redi[3];
      cbase += flag[0] + flag[1] + flag[2] + flag[3];
      __syncthreads();
    }
    if (tid == 0) {
      a.list_len[bh * a.Cq + i] = (int32_t)min((int64_t)base, a.list_cap);
      lpos[n_kept] = base;
      cpos[n_kept] = cbase;
    }
    __syncthreads();
  }
  // 7. the list, in batches of 256 chunks of 16 entries: each thread finds
  // the kept cluster of one chunk by binary search over the chunk
  // positions and leaves the chunk's first source row, list position and
  // entry count in LDS; then each group of 16 lanes copies one chunk (lane
  // u its entry u), so that a wave's loads and stores fall in 4 contiguous
  // runs.  Entries past list_cap are dropped.
  const int n_chunks = cpos[n_kept];
  int32_t *lst = a.lists + (bh * a.Cq + i) * a.list_cap;
  const int32_t *kperm = a.k_perm + bh * a.S * a.L;
  const int u = tid & 15;
  for (int q0 = 0; q0 < n_chunks; q0 += 256) {
    const int q = q0 + tid;
    if (q < n_chunks) {
      int lo = 0, hi = n_kept - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cpos[mid] <= q)
          lo = mid;
        else
          hi = mid - 1;
      }
      const int sL = kept[lo] / a.Ck * a.L;
      const int c0 = (q - cpos[lo]) * 16;
      chunk_s[tid] = make_int4(sL + kstart[lo] + c0, lpos[lo] + c0,
                               min(16, lpos[lo + 1] - lpos[lo] - c0), sL);
    }
    __syncthreads();
    const int nb = min(256, n_chunks - q0);
    int4 c[16];
    int32_t v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int r = (tid >> 4) + 16 * m;
      c[m] = r < nb ? chunk_s[r] : make_int4(0, 0, 0, 0);
      v[m] = u < c[m].z ? kperm[c[m].x + u] : 0;
    }
#pragma unroll
    for (int m = 0; m < 16; ++m)
      if (u < c[m].z && c[m].y + u < a.list_cap) lst[c[m].y + u] = c[m].w + v[m];
    __syncthreads();
  }
}

// One or two problems (a1 == nullptr: one); with two, every launch holds
// the first problem's workgroups, then the second's.
template <int D>
hipError_t kmeans_d(const KmArgs &a0, const KmArgs *a1, int iters, bool from_tokens,
                    hipStream_t s) {
  auto gc = [](const KmArgs &a) { return (unsigned)((int64_t)a.B * a.H * a.C); };
  auto ga = [](const KmArgs &a) { return (unsigned)((int64_t)a.B * a.H * ((a.n + 127) / 128)); };
  auto gh = [](const KmArgs &a) { return (unsigned)((int64_t)a.B * a.H); };
  const KmArgs &b = a1 ? *a1 : a0;
  const unsigned c0 = gc(a0), c1 = a1 ? gc(b) : 0u;
  const unsigned s0 = ga(a0), s1 = a1 ? ga(b) : 0u;
  const unsigned h0 = gh(a0), h1 = a1 ? gh(b) : 0u;
  const size_t lds = a1 ? std::max(assign_lds_bytes<D>(a0.C), assign_lds_bytes<D>(b.C))
                        : assign_lds_bytes<D>(a0.C);
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&svg2_assign_kernel<D>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)assign_lds_bytes<D>(kMaxC));
    if (e != hipSuccess) return e;
    attr = true;
  }
  if (from_tokens)
    hipLaunchKernelGGL(svg2_init_kernel<D>, dim3(c0 + c1), dim3(D), 0, s, a0, b, c0);
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(svg2_assign_kernel<D>, dim3(s0 + s1), dim3(256), lds, s, a0, b, s0);
    hipLaunchKernelGGL(svg2_sort_kernel, dim3(h0 + h1), dim3(kSortThreads), 0, s, a0, b, h0);
    hipLaunchKernelGGL(svg2_update_kernel<D>, dim3(c0 + c1), dim3(256), 0, s, a0, b, c0);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_svg2_kmeans(const KmArgs &a, int D, int iters, bool from_tokens, hipStream_t s) {
  return D == 128 ? kmeans_d<128>(a, nullptr, iters, from_tokens, s)
                  : kmeans_d<64>(a, nullptr, iters, from_tokens, s);
}

hipError_t launch_svg2_kmeans2(const KmArgs &a0, const KmArgs &a1, int D, int iters,
                               bool from_tokens, hipStream_t s) {
  return D == 128 ? kmeans_d<128>(a0, &a1, iters, from_tokens, s)
                  : kmeans_d<64>(a0, &a1, iters, from_tokens, s);
}

hipError_t launch_svg2_plan(const SvgPlanArgs &a, int D, hipStream_t s) {
  const unsigned gq = (unsigned)((int64_t)a.B * a.H * a.Cq);
  if (D == 128)
    hipLaunchKernelGGL(svg2_select_kernel<128>, dim3(gq), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(svg2_select_kernel<64>, dim3(gq), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace crattn
