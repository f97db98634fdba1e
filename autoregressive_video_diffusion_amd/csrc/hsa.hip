// Hierarchical block-sparse attention (HSA): key pooling and the two-level
// block selection, for AMD CDNA4 (gfx950).  The attention over the selected
// blocks is the block-sparse instance of the attention kernel (attn.hip).
//
// Source: "LIGHT FORCING" technical summary, §2.2: queries and keys are
// compressed by mean pooling at block and frame level; for each query block
// a few history frames are chosen with the frame-level keys, then the
// critical blocks inside them with the block-level keys.
//
// Both are small next to the attention: the pooling reads each chunk's keys
// once when the chunk is appended (HBM-bound, one workgroup per 64-key
// block), the selection reads one query block and the pooled history keys
// per workgroup.
#include "crattn_internal.h"
#include <math.h>
#include "../../include/crattn.h"

namespace crattn {
namespace {

constexpr int kKB = CRATTN_HSA_KBLOCK;
constexpr int kQB = CRATTN_HSA_QBLOCK;

__device__ inline void add_bf16x8(float (&acc)[8], const uint4 &x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += __uint_as_float(w[e] << 16);
    acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
  }
}

// ---- key pooling, pass 1: one workgroup per (b, h, block) ----
// Thread t reads 16-byte chunk t % (D/8) of rows t / (D/8), t / (D/8) + RG,
// ...  of the block; the per-thread partial sums meet in LDS and are added
// in row-group order, so the result is the same on every run.
template <int D>
__global__ void __launch_bounds__(256) hsa_pool_blocks_kernel(HsaPoolArgs a) {
  constexpr int CPR = D / 8;
  constexpr int RG = 256 / CPR;
  __shared__ float part[RG][D];
  const int tid = threadIdx.x;
  const int c = tid % CPR, g = tid / CPR;
  const int nb = a.n_frames * a.nbf;  // blocks of the pooled range
  const int bi = (int)(blockIdx.x % (uint32_t)nb);
  const int bh = (int)(blockIdx.x / (uint32_t)nb);
  const int f = a.frame0 + bi / a.nbf, j = bi % a.nbf;
  const int rs = j * kKB, re = min(rs + kKB, a.per_frame);
  const uint16_t *kr = a.k + ((int64_t)bh * a.cap + (int64_t)f * a.per_frame) * D + c * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = rs + g; r < re; r += RG)
    add_bf16x8(acc, *reinterpret_cast<const uint4 *>(kr + (int64_t)r * D));
#pragma unroll
  for (int e = 0; e < 8; ++e) part[g][c * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < RG; ++k) s += part[k][tid];
    a.blocks[((int64_t)bh * a.nf * a.nbf + (int64_t)f * a.nbf + j) * D + tid] =
        s / (float)(re - rs);
  }
}

// ---- key pooling, pass 2: frame means from the block means, one
// workgroup of D threads per (b, h, frame): the length-weighted mean of the
// frame's block means, added in block order ----
template <int D>
__global__ void __launch_bounds__(D) hsa_pool_frames_kernel(HsaPoolArgs a) {
  const int fi = (int)(blockIdx.x % (uint32_t)a.n_frames);
  const int bh = (int)(blockIdx.x / (uint32_t)a.n_frames);
  const int f = a.frame0 + fi;
  const float *bm = a.blocks + ((int64_t)bh * a.nf * a.nbf + (int64_t)f * a.nbf) * D;
  float s = 0.f;
#pragma unroll 16
  for (int j = 0; j < a.nbf; ++j)
    s += bm[(int64_t)j * D + threadIdx.x] * (float)(min(kKB, a.per_frame - j * kKB));
  a.frames[((int64_t)bh * a.nf + f) * D + threadIdx.x] = s / (float)a.per_frame;
}

// ---- selection: one workgroup per (b, h, query block) ----
template <int D>
__global__ void __launch_bounds__(256) hsa_select_kernel(HsaSelectArgs a) {
  constexpr int CPR = D / 8;
  constexpr int RG = 256 / CPR;
  __shared__ float part[RG][D];
  __shared__ float qbar[D];
  __shared__ float4 score4[CRATTN_HSA_MAX_CAND / 4 + 1];
  float *score = reinterpret_cast<float *>(score4);
  __shared__ int wave_cnt[4];
  __shared__ int frames_kept[CRATTN_HSA_MAX_KF];
  const int tid = threadIdx.x;
  const int t = (int)(blockIdx.x % (uint32_t)a.n_qblocks);
  const int bh = (int)(blockIdx.x / (uint32_t)a.n_qblocks);
  const int b = bh / a.H, h = bh - b * a.H;
  int32_t *out = a.sel + ((int64_t)bh * a.n_qblocks + t) * a.kb;

  // 1. the query block's mean
  {
    const int c = tid % CPR, g = tid / CPR;
    const int64_t r0 = (int64_t)t * kQB, r1 = min(r0 + kQB, a.Lq);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
    for (int64_t r = r0 + g; r < r1; r += RG)
      add_bf16x8(acc, *reinterpret_cast<const uint4 *>(
                          a.q + (((int64_t)b * a.Lq + r) * a.H + h) * D + c * 8));
#pragma unroll
    for (int e = 0; e < 8; ++e) part[g][c * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < RG; ++k) s += part[k][tid];
      qbar[tid] = s / (float)(r1 - r0);
    }
    __syncthreads();
  }
  // Scores of n items (rows of pooled keys): 16 threads per item, each
  // adding D/16 products, then a butterfly over the 16 lanes.
  constexpr int TPI = 16, FPT = D / TPI;
  auto scores = [&](int n, auto row_of) {
    const int sub = tid % TPI;
    for (int base = tid / TPI; base < n; base += 256 / TPI) {
      const float *row = row_of(base) + sub * FPT;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < FPT; d += 4) {
        const float4 x = *reinterpret_cast<const float4 *>(row + d);
        const int dd = sub * FPT + d;
        s += qbar[dd] * x.x + qbar[dd + 1] * x.y + qbar[dd + 2] * x.z + qbar[dd + 3] * x.w;
      }
#pragma unroll
      for (int m = TPI / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, TPI);
      // a NaN score (NaN or infinite pooled inputs) ranks below every
      // number, so the comparisons below stay a total order
      if (sub == 0) score[base] = __builtin_isnan(s) ? -INFINITY : s;
    }
  };
  // rank of item i among n scores: how many are larger, or equal with a
  // lower index (the order of a stable descending sort; no score is NaN, so
  // the ranks of the n items are 0 .. n-1, each once).  Scores are read
  // four at a time; the caller pads score[n .. n+3] with -inf, which never
  // ranks above an item (a -inf item has the lower index).
  auto rank = [&](int i, int n) {
    const float si = score[i];
    int k = 0;
#pragma unroll 4
    for (int j4 = 0; j4 < (n + 3) / 4; ++j4) {
      const float4 v = score4[j4];
      const int j = 4 * j4;
      k += (v.x > si || (v.x == si && j < i)) ? 1 : 0;
      k += (v.y > si || (v.y == si && j + 1 < i)) ? 1 : 0;
      k += (v.z > si || (v.z == si && j + 2 < i)) ? 1 : 0;
      k += (v.w > si || (v.w == si && j + 3 < i)) ? 1 : 0;
    }
    return k;
  };
  // Items [0, n) are kept or not (keep(i)); call emit(i, pos) for each kept
  // item with pos = the number of kept items before it.  A wave ballot
  // counts the kept lanes below each lane; waves add up in LDS, 256 items
  // at a time.
  auto compact = [&](int n, auto keep, auto emit) {
    const int lane = tid & 63, wave = tid >> 6;
    int base = 0;
    for (int i0 = 0; i0 < n; i0 += 256) {
      const int i = i0 + tid;
      const bool k = i < n && keep(i);
      const uint64_t bal = __builtin_amdgcn_ballot_w64(k);
      if (lane == 0) wave_cnt[wave] = __builtin_popcountll(bal);
      __syncthreads();
      int off = base;
      for (int w = 0; w < wave; ++w) off += wave_cnt[w];
      if (k) emit(i, off + __builtin_popcountll(bal & ((uint64_t(1) << lane) - 1)));
      base += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
      __syncthreads();
    }
  };

  const int n_hist = a.n_hist;
  if (n_hist == 0) {
    for (int e = tid; e < a.kb; e += 256) out[e] = -1;
    return;
  }
  // 2. frame scores and the kf best frames, kept in ascending order.
  // Candidate c is history frame c below the own chunk and c + fc above it
  // (in a ring, the own chunk's slot may sit anywhere).
  auto frame_of = [&](int c) { return c < a.own_f0 ? c : c + a.fc; };
  const float *fm = a.frames + (int64_t)bh * a.nf * D;
  scores(n_hist, [&](int c) { return fm + (int64_t)frame_of(c) * D; });
  if (tid < 4) score[n_hist + tid] = -INFINITY;
  __syncthreads();
  // (pos < kf always holds with a total order; the test keeps a write
  // inside the array whatever the scores)
  compact(n_hist, [&](int c) { return rank(c, n_hist) < a.kf; },
          [&](int c, int pos) {
            if (pos < a.kf) frames_kept[pos] = frame_of(c);
          });
  const int n_frames = min(a.kf, n_hist);
  const int n_cand = n_frames * a.nbf;
  // 3. block scores of every block of the kept frames; candidate c is block
  // c % nbf of kept frame c / nbf, so candidates run in ascending block id
  const float *bm = a.blocks + (int64_t)bh * a.nf * a.nbf * D;
  scores(n_cand, [&](int cnd) {
    return bm + (int64_t)(frames_kept[cnd / a.nbf] * a.nbf + cnd % a.nbf) * D;
  });
  if (tid < 4) score[n_cand + tid] = -INFINITY;
  __syncthreads();
  // 4. the kept blocks in ascending id order, then -1
  compact(n_cand, [&](int cnd) { return rank(cnd, n_cand) < a.kb; },
          [&](int cnd, int pos) {
            if (pos < a.kb) out[pos] = frames_kept[cnd / a.nbf] * a.nbf + cnd % a.nbf;
          });
  for (int e = min(a.kb, n_cand) + tid; e < a.kb; e += 256) out[e] = -1;
}

}  // namespace

hipError_t launch_hsa_pool(const HsaPoolArgs &a, int D, hipStream_t s) {
  const unsigned gb = (unsigned)((int64_t)a.B * a.H * a.n_frames * a.nbf);
  const unsigned gf = (unsigned)((int64_t)a.B * a.H * a.n_frames);
  if (D == 128) {
    hipLaunchKernelGGL(hsa_pool_blocks_kernel<128>, dim3(gb), dim3(256), 0, s, a);
    hipLaunchKernelGGL(hsa_pool_frames_kernel<128>, dim3(gf), dim3(128), 0, s, a);
  } else {
    hipLaunchKernelGGL(hsa_pool_blocks_kernel<64>, dim3(gb), dim3(256), 0, s, a);
    hipLaunchKernelGGL(hsa_pool_frames_kernel<64>, dim3(gf), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_hsa_select(const HsaSelectArgs &a, int D, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.B * a.H * a.n_qblocks);
  if (D == 128)
    hipLaunchKernelGGL(hsa_select_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(hsa_select_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace crattn
