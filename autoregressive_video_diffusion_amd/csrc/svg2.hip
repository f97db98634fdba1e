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
// cluster.  The contraction of the assignment (tokens x centroids) is fp32
// on the vector ALU: it decides an integer (the nearest centroid), and fp32
// keeps that decision close to the exact one.
#include "crattn_internal.h"
#include <math.h>
#include "../../include/crattn.h"

namespace crattn {
namespace {

constexpr int kMaxC = CRATTN_SVG2_MAX_C;
constexpr int kMaxN = CRATTN_SVG2_MAX_N;
constexpr int kMaxCand = CRATTN_SVG2_MAX_CAND;

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
__global__ void __launch_bounds__(D) svg2_init_kernel(KmArgs a) {
  const int c = (int)(blockIdx.x % (uint32_t)a.C);
  const int64_t bh = blockIdx.x / (uint32_t)a.C;
  const int64_t t = (int64_t)c * a.n / a.C;
  a.cent[bh * a.cent_s + (int64_t)c * D + threadIdx.x] =
      __uint_as_float((uint32_t)token_ptr(a, bh, t)[threadIdx.x] << 16);
}

// ---- squared norms of the centroids (one wave per centroid) ----
template <int D>
__global__ void __launch_bounds__(64) svg2_norm_kernel(KmArgs a) {
  const int c = (int)(blockIdx.x % (uint32_t)a.C);
  const int64_t bh = blockIdx.x / (uint32_t)a.C;
  const float *cp = a.cent + bh * a.cent_s + (int64_t)c * D;
  float s = 0.f;
#pragma unroll
  for (int d = threadIdx.x; d < D; d += 64) s = fmaf(cp[d], cp[d], s);
  s = wave_sum(s);
  if (threadIdx.x == 0) a.norm[bh * a.C + c] = s;
}

// ---- assignment: nearest centroid of every token ----
// One workgroup per 64 tokens of a head; lane = token, its D features in
// registers.  Wave w scans centroids [w C/4, (w+1) C/4), read as wave-uniform
// (scalar) loads; the distance up to the token's own norm is
// |c|^2 - 2 x.c in fp32.  The four waves' minima meet in LDS; a tie goes to
// the lower centroid index.
template <int D>
__global__ void __launch_bounds__(256) svg2_assign_kernel(KmArgs a) {
  __shared__ float best_d[4][64];
  __shared__ int best_i[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = (a.n + 63) / 64;
  const int blk = (int)(blockIdx.x % (uint32_t)nblk);
  const int64_t bh = blockIdx.x / (uint32_t)nblk;
  const int t = blk * 64 + lane;
  const uint16_t *xp = token_ptr(a, bh, min(t, a.n - 1));
  float xv[D];
#pragma unroll
  for (int d8 = 0; d8 < D / 8; ++d8) {
    const uint4 u = *reinterpret_cast<const uint4 *>(xp + d8 * 8);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xv[d8 * 8 + 2 * e] = __uint_as_float(w[e] << 16);
      xv[d8 * 8 + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  const int c0 = wave * a.C / 4, c1 = (wave + 1) * a.C / 4;
  const float *__restrict__ cb = a.cent + bh * a.cent_s;
  const float *__restrict__ nb = a.norm + bh * a.C;
  float best = INFINITY;
  int bidx = c0;
  int c = c0;
  for (; c + 2 <= c1; c += 2) {
    const float *p0 = cb + (int64_t)c * D, *p1 = p0 + D;
    float s0a = 0.f, s0b = 0.f, s1a = 0.f, s1b = 0.f;
#pragma unroll
    for (int d = 0; d < D; d += 2) {
      s0a = fmaf(xv[d], p0[d], s0a);
      s0b = fmaf(xv[d + 1], p0[d + 1], s0b);
      s1a = fmaf(xv[d], p1[d], s1a);
      s1b = fmaf(xv[d + 1], p1[d + 1], s1b);
    }
    const float e0 = fmaf(-2.f, s0a + s0b, nb[c]);
    const float e1 = fmaf(-2.f, s1a + s1b, nb[c + 1]);
    if (e0 < best) {
      best = e0;
      bidx = c;
    }
    if (e1 < best) {
      best = e1;
      bidx = c + 1;
    }
  }
  if (c < c1) {
    const float *p0 = cb + (int64_t)c * D;
    float s0a = 0.f, s0b = 0.f;
#pragma unroll
    for (int d = 0; d < D; d += 2) {
      s0a = fmaf(xv[d], p0[d], s0a);
      s0b = fmaf(xv[d + 1], p0[d + 1], s0b);
    }
    const float e0 = fmaf(-2.f, s0a + s0b, nb[c]);
    if (e0 < best) {
      best = e0;
      bidx = c;
    }
  }
  best_d[wave][lane] = best;
  best_i[wave][lane] = bidx;
  __syncthreads();
  if (wave == 0 && t < a.n) {
    float bd = best_d[0][lane];
    int bi = best_i[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (best_d[w][lane] < bd) {
        bd = best_d[w][lane];
        bi = best_i[w][lane];
      }
    a.assign[bh * a.n + t] = bi;
  }
}

// ---- stable counting sort by cluster: one workgroup of 16 waves per head ----
// Tokens are taken in blocks of 64 (block j by wave j mod 16).  Within a
// block, a token's rank is the number of earlier tokens of the block with
// its cluster; per (block, cluster) counts are then scanned over the blocks,
// so the position of token t of cluster c is
//   offsets[c] + (tokens of c in earlier blocks) + (rank in its block),
// which keeps every cluster's tokens in ascending order.
constexpr int kSortWaves = 16;
constexpr int kBlkPerWave = kMaxN / 64 / kSortWaves;

__global__ void __launch_bounds__(kSortWaves * 64) svg2_sort_kernel(KmArgs a) {
  __shared__ uint16_t cnt[(kMaxN / 64) * kMaxC];  // [block][cluster]
  __shared__ int4 blk_ids[kSortWaves][16];
  __shared__ int tot[kMaxC];
  __shared__ int coff[kMaxC + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x;
  const int n = a.n, C = a.C;
  const int nblk = (n + 63) / 64;
  for (int i = tid; i < nblk * C; i += kSortWaves * 64) cnt[i] = 0;
  __syncthreads();
  const int32_t *as = a.assign + bh * n;
  int *ids = reinterpret_cast<int *>(blk_ids[wave]);
  int val[kBlkPerWave], rank[kBlkPerWave];
#pragma unroll
  for (int k = 0; k < kBlkPerWave; ++k) {
    const int blk = wave + kSortWaves * k;
    val[k] = -1;
    rank[k] = 0;
    if (blk < nblk) {
      const int t = blk * 64 + lane;
      const int v = t < n ? as[t] : -1;
      ids[lane] = v;
      __builtin_amdgcn_wave_barrier();
      int before = 0, after = 0;
#pragma unroll 4
      for (int j4 = 0; j4 < 16; ++j4) {
        const int4 u = blk_ids[wave][j4];
        const int j = 4 * j4;
        before += (u.x == v && j < lane) + (u.y == v && j + 1 < lane) +
                  (u.z == v && j + 2 < lane) + (u.w == v && j + 3 < lane);
        after += (u.x == v && j > lane) + (u.y == v && j + 1 > lane) +
                 (u.z == v && j + 2 > lane) + (u.w == v && j + 3 > lane);
      }
      // the last token of its cluster in the block writes the block's count
      if (v >= 0 && after == 0) cnt[blk * C + v] = (uint16_t)(before + 1);
      val[k] = v;
      rank[k] = before;
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  // exclusive scan of every cluster's counts over the blocks
  for (int c = tid; c < C; c += kSortWaves * 64) {
    int run = 0;
#pragma unroll 8
    for (int blk = 0; blk < nblk; ++blk) {
      const int x = cnt[blk * C + c];
      cnt[blk * C + c] = (uint16_t)run;
      run += x;
    }
    tot[c] = run;
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
  for (int c = tid; c <= C; c += kSortWaves * 64) off[c] = coff[c];
  int32_t *perm = a.perm + bh * a.perm_s;
#pragma unroll
  for (int k = 0; k < kBlkPerWave; ++k) {
    const int blk = wave + kSortWaves * k;
    const int v = val[k];
    if (blk < nblk && v >= 0) perm[coff[v] + cnt[blk * C + v] + rank[k]] = blk * 64 + lane;
  }
}

// ---- centroid update: the mean of each cluster's tokens (one wave per
// cluster), added in reordered (= ascending token) order; an empty cluster
// keeps its centroid.  Also the squared norm for the next assignment. ----
template <int D>
__global__ void __launch_bounds__(64) svg2_update_kernel(KmArgs a) {
  constexpr int PER = D / 64;  // features per lane
  const int c = (int)(blockIdx.x % (uint32_t)a.C);
  const int64_t bh = blockIdx.x / (uint32_t)a.C;
  const int lane = threadIdx.x;
  const int32_t *off = a.off + bh * a.off_s;
  const int r0 = off[c], r1 = off[c + 1];
  float *cp = a.cent + bh * a.cent_s + (int64_t)c * D + lane * PER;
  float cv[PER];
  if (r1 > r0) {
    float s[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) s[e] = 0.f;
    const int32_t *pm = a.perm + bh * a.perm_s;
    const uint16_t *xb = token_ptr(a, bh, 0) + lane * PER;
#pragma unroll 8
    for (int r = r0; r < r1; ++r) {
      const int64_t t = pm[r];
      if constexpr (PER == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t *>(xb + t * a.sr);
        s[0] += __uint_as_float(u << 16);
        s[1] += __uint_as_float(u & 0xffff0000u);
      } else {
        s[0] += __uint_as_float((uint32_t)xb[t * a.sr] << 16);
      }
    }
    const float cntf = (float)(r1 - r0);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      cv[e] = s[e] / cntf;
      cp[e] = cv[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) cv[e] = cp[e];
  }
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) q = fmaf(cv[e], cv[e], q);
  q = wave_sum(q);
  if (lane == 0) a.norm[bh * a.C + c] = q;
}

// ---- selection and key list of one (b, h, query cluster) ----
// Scores of the candidates (16 lanes per candidate, butterfly over the 16);
// shares w_j = n_j exp(s_j - max s); rank of each candidate in decreasing
// share (ties: lower id first); exclusive prefix of the shares in rank
// order; candidate kept while the share before it is below p times the
// total.  The kept ids are compacted in ascending order, their key counts
// scanned, and every list entry finds its cluster by binary search.
template <int D>
__global__ void __launch_bounds__(256) svg2_select_kernel(SvgPlanArgs a) {
  __shared__ float qc[D];
  __shared__ float4 w4[kMaxCand / 4 + 1];
  __shared__ float sw[kMaxCand];
  __shared__ float ex[kMaxCand];
  __shared__ int rk[kMaxCand];
  __shared__ int kept[kMaxCand];
  __shared__ int lpos[kMaxCand + 1];
  __shared__ float redf[4];
  __shared__ int redi[4];
  float *w = reinterpret_cast<float *>(w4);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = (int)(blockIdx.x % (uint32_t)a.Cq);
  const int64_t bh = blockIdx.x / (uint32_t)a.Cq;
  const int NC = a.n_vis * a.Ck;
  const int32_t *qo = a.q_off + bh * (a.Cq + 1);
  int32_t *lst = a.lists + (bh * a.Cq + i) * a.list_cap;
  int32_t *sel = a.sel ? a.sel + (bh * a.Cq + i) * (int64_t)NC : nullptr;
  const int32_t *koff = a.k_off + bh * a.S * (int64_t)(a.Ck + 1);
  // Offsets come from svg2_kmeans; they are clamped to [0, L] anyway, so
  // that no read of k_perm leaves its slot.
  auto start_of = [&](int j) {
    const int s = j / a.Ck, c = j - s * a.Ck;
    return (int)min(max((int64_t)koff[s * (a.Ck + 1) + c], (int64_t)0), a.L);
  };
  auto count_of = [&](int j) {
    const int s = j / a.Ck, c = j - s * a.Ck;
    const int64_t e = min(max((int64_t)koff[s * (a.Ck + 1) + c + 1], (int64_t)0), a.L);
    return (int)max(e - start_of(j), (int64_t)0);
  };
  if (qo[i + 1] <= qo[i]) {
    if (tid == 0) a.list_len[bh * a.Cq + i] = 0;
    if (sel)
      for (int e = tid; e < NC; e += 256) sel[e] = -1;
    return;
  }
  if (tid < D) qc[tid] = a.q_cent[(bh * a.Cq + i) * D + tid];
  __syncthreads();
  // 1. scores (-inf for empty clusters)
  {
    constexpr int TPI = 16, FPT = D / TPI;
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
  if (tid < 4) w[NC + tid] = -INFINITY;
  __syncthreads();
  // 3. rank in decreasing share, ties to the lower id; shares in rank order
  for (int j = tid; j < NC; j += 256) {
    const float wj = w[j];
    int r = 0;
#pragma unroll 4
    for (int k4 = 0; k4 < (NC + 3) / 4; ++k4) {
      const float4 v = w4[k4];
      const int k = 4 * k4;
      r += (v.x > wj || (v.x == wj && k < j)) ? 1 : 0;
      r += (v.y > wj || (v.y == wj && k + 1 < j)) ? 1 : 0;
      r += (v.z > wj || (v.z == wj && k + 2 < j)) ? 1 : 0;
      r += (v.w > wj || (v.w == wj && k + 3 < j)) ? 1 : 0;
    }
    rk[j] = r;
    sw[r] = wj;
  }
  __syncthreads();
  // 4. exclusive prefix of the ranked shares: 4 consecutive per thread,
  // then a scan over the threads (fixed order)
  {
    float loc[4], t = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * tid + e;
      loc[e] = t;
      t += r < NC ? sw[r] : 0.f;
    }
    float inc = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(inc, d, 64);
      if (lane >= d) inc += y;
    }
    if (lane == 63) redf[wave] = inc;
    __syncthreads();
    float base = inc - t;
    for (int v = 0; v < wave; ++v) base += redf[v];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * tid + e < NC) ex[4 * tid + e] = base + loc[e];
    __syncthreads();
    if (tid == 0) redf[0] = redf[0] + redf[1] + redf[2] + redf[3];  // total
    __syncthreads();
  }
  const float cut = a.p * redf[0];
  const bool all = a.p >= 1.f;
  // 5. kept ids in ascending order
  int n_kept = 0;
  for (int j0 = 0; j0 < NC; j0 += 256) {
    const int j = j0 + tid;
    const bool k = j < NC && count_of(j) > 0 && (all || ex[rk[j]] < cut);
    const uint64_t bal = __builtin_amdgcn_ballot_w64(k);
    if (lane == 0) redi[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int pos = n_kept;
    for (int v = 0; v < wave; ++v) pos += redi[v];
    if (k) kept[pos + __builtin_popcountll(bal & ((uint64_t(1) << lane) - 1))] = j;
    n_kept += redi[0] + redi[1] + redi[2] + redi[3];
    __syncthreads();
  }
  if (sel)
    for (int e = tid; e < NC; e += 256) sel[e] = e < n_kept ? kept[e] : -1;
  // 6. list positions of the kept clusters (exclusive scan of their counts)
  {
    int base = 0;
    for (int k0 = 0; k0 < n_kept; k0 += 256) {
      const int k = k0 + tid;
      const int x = k < n_kept ? count_of(kept[k]) : 0;
      int inc = x;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d, 64);
        if (lane >= d) inc += y;
      }
      if (lane == 63) redi[wave] = inc;
      __syncthreads();
      int pre = base + inc - x;
      for (int v = 0; v < wave; ++v) pre += redi[v];
      if (k < n_kept) lpos[k] = pre;
      base += redi[0] + redi[1] + redi[2] + redi[3];
      __syncthreads();
    }
    if (tid == 0) lpos[n_kept] = base;
    __syncthreads();
  }
  const int m = (int)min((int64_t)lpos[n_kept], a.list_cap);
  // 7. the list: entry e belongs to kept cluster k with lpos[k] <= e < lpos[k+1]
  const int32_t *kperm = a.k_perm + bh * a.S * a.L;
  for (int e = tid; e < m; e += 256) {
    int lo = 0, hi = n_kept - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (lpos[mid] <= e)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int j = kept[lo];
    const int s = j / a.Ck;
    const int64_t r = start_of(j) + (e - lpos[lo]);
    lst[e] = (int32_t)(s * a.L + kperm[s * a.L + r]);
  }
  if (tid == 0) a.list_len[bh * a.Cq + i] = m;
}

// ---- query tiles: every query cluster split into tiles of qtile rows, in
// cluster order; unused slots get zero rows.  One wave per (b, h). ----
__global__ void __launch_bounds__(64) svg2_slots_kernel(SvgPlanArgs a) {
  const int64_t bh = blockIdx.x;
  const int lane = threadIdx.x;
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

}  // namespace

hipError_t launch_svg2_kmeans(const KmArgs &a, int D, int iters, bool from_tokens, hipStream_t s) {
  const unsigned gc = (unsigned)((int64_t)a.B * a.H * a.C);
  const unsigned ga = (unsigned)((int64_t)a.B * a.H * ((a.n + 63) / 64));
  const unsigned gh = (unsigned)((int64_t)a.B * a.H);
  if (D == 128) {
    if (from_tokens) hipLaunchKernelGGL(svg2_init_kernel<128>, dim3(gc), dim3(128), 0, s, a);
    hipLaunchKernelGGL(svg2_norm_kernel<128>, dim3(gc), dim3(64), 0, s, a);
    for (int it = 0; it < iters; ++it) {
      hipLaunchKernelGGL(svg2_assign_kernel<128>, dim3(ga), dim3(256), 0, s, a);
      hipLaunchKernelGGL(svg2_sort_kernel, dim3(gh), dim3(kSortWaves * 64), 0, s, a);
      hipLaunchKernelGGL(svg2_update_kernel<128>, dim3(gc), dim3(64), 0, s, a);
    }
  } else {
    if (from_tokens) hipLaunchKernelGGL(svg2_init_kernel<64>, dim3(gc), dim3(64), 0, s, a);
    hipLaunchKernelGGL(svg2_norm_kernel<64>, dim3(gc), dim3(64), 0, s, a);
    for (int it = 0; it < iters; ++it) {
      hipLaunchKernelGGL(svg2_assign_kernel<64>, dim3(ga), dim3(256), 0, s, a);
      hipLaunchKernelGGL(svg2_sort_kernel, dim3(gh), dim3(kSortWaves * 64), 0, s, a);
      hipLaunchKernelGGL(svg2_update_kernel<64>, dim3(gc), dim3(64), 0, s, a);
    }
  }
  return hipGetLastError();
}

hipError_t launch_svg2_plan(const SvgPlanArgs &a, int D, hipStream_t s) {
  const unsigned gq = (unsigned)((int64_t)a.B * a.H * a.Cq);
  if (D == 128)
    hipLaunchKernelGGL(svg2_select_kernel<128>, dim3(gq), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(svg2_select_kernel<64>, dim3(gq), dim3(256), 0, s, a);
  hipLaunchKernelGGL(svg2_slots_kernel, dim3((unsigned)((int64_t)a.B * a.H)), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace crattn
