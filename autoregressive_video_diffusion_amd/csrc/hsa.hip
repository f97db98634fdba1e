// Hierarchical block-sparse attention (HSA): key pooling and the two-level
// block selection, for AMD CDNA4 (gfx950).  The attention over the selected
// blocks is the block-sparse instance of the attention kernel (attn.hip).
//
// Source: "LIGHT FORCING" technical summary, §2.2: queries and keys are
// compressed by mean pooling at block and frame level; for each query block
// a few history frames are chosen with the frame-level keys, then the
// critical blocks inside them with the block-level keys.
//
// Both kernels are small next to the attention: the pooling reads each
// chunk's keys once when the chunk is appended (HBM-bound), the selection
// reads one query block and the pooled history keys per workgroup.
#include "crattn_internal.h"
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

// ---- key pooling: one workgroup per (b, h, frame) ----
// Thread t reads 16-byte chunk t % (D/8) of rows t / (D/8), t / (D/8) + RG,
// ...: RG rows of a block at a time.  Each block's per-thread partial sums
// meet in LDS and are added in row-group order, so the result is the same
// on every run.  The frame sum is the sum of its block sums in block order.
template <int D>
__global__ void __launch_bounds__(256) hsa_pool_kernel(HsaPoolArgs a) {
  constexpr int CPR = D / 8;
  constexpr int RG = 256 / CPR;
  __shared__ float part[RG][D];
  const int tid = threadIdx.x;
  const int c = tid % CPR, g = tid / CPR;
  const int fi = (int)(blockIdx.x % (uint32_t)a.n_frames);
  const int bh = (int)(blockIdx.x / (uint32_t)a.n_frames);
  const int f = a.frame0 + fi;
  const uint16_t *kr = a.k + ((int64_t)bh * a.cap + (int64_t)f * a.per_frame) * D + c * 8;
  float *fmean = a.frames + ((int64_t)bh * a.nf + f) * D;
  float *bmean = a.blocks + ((int64_t)bh * a.nf * a.nbf + (int64_t)f * a.nbf) * D;
  float fsum = 0.f;
  for (int j = 0; j < a.nbf; ++j) {
    const int rs = j * kKB, re = min(rs + kKB, a.per_frame);
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
      bmean[(int64_t)j * D + tid] = s / (float)(re - rs);
      fsum += s;
    }
    __syncthreads();
  }
  if (tid < D) fmean[tid] = fsum / (float)a.per_frame;
}

// ---- selection: one workgroup per (b, h, query block) ----
template <int D>
__global__ void __launch_bounds__(256) hsa_select_kernel(HsaSelectArgs a) {
  constexpr int CPR = D / 8;
  constexpr int RG = 256 / CPR;
  __shared__ float part[RG][D];
  __shared__ float qbar[D];
  __shared__ float score[CRATTN_HSA_MAX_CAND];
  __shared__ unsigned char keep[CRATTN_HSA_MAX_CAND];
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
  auto dot = [&](const float *row) {
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; d += 4) {
      const float4 x = *reinterpret_cast<const float4 *>(row + d);
      s += qbar[d] * x.x + qbar[d + 1] * x.y + qbar[d + 2] * x.z + qbar[d + 3] * x.w;
    }
    return s;
  };
  // rank of item i among n scores: how many are larger, or equal with a
  // lower index (the order of a stable descending sort)
  auto rank = [&](int i, int n) {
    const float si = score[i];
    int k = 0;
    for (int j = 0; j < n; ++j) {
      const float sj = score[j];
      k += (sj > si || (sj == si && j < i)) ? 1 : 0;
    }
    return k;
  };

  const int n_hist = a.n_hist;
  if (n_hist == 0) {
    for (int e = tid; e < a.kb; e += 256) out[e] = -1;
    return;
  }
  // 2. frame scores and the kf best frames, kept in ascending order
  const float *fm = a.frames + (int64_t)bh * a.nf * D;
  for (int f = tid; f < n_hist; f += 256) score[f] = dot(fm + (int64_t)f * D);
  __syncthreads();
  for (int f = tid; f < n_hist; f += 256) keep[f] = rank(f, n_hist) < a.kf ? 1 : 0;
  __syncthreads();
  for (int f = tid; f < n_hist; f += 256)
    if (keep[f]) {
      int pos = 0;
      for (int g2 = 0; g2 < f; ++g2) pos += keep[g2];
      frames_kept[pos] = f;
    }
  __syncthreads();
  const int n_frames = min(a.kf, n_hist);
  const int n_cand = n_frames * a.nbf;
  // 3. block scores of every block of the kept frames; candidate c is block
  // c % nbf of kept frame c / nbf, so candidates run in ascending block id
  const float *bm = a.blocks + (int64_t)bh * a.nf * a.nbf * D;
  for (int cnd = tid; cnd < n_cand; cnd += 256) {
    const int id = frames_kept[cnd / a.nbf] * a.nbf + cnd % a.nbf;
    score[cnd] = dot(bm + (int64_t)id * D);
  }
  __syncthreads();
  for (int cnd = tid; cnd < n_cand; cnd += 256) keep[cnd] = rank(cnd, n_cand) < a.kb ? 1 : 0;
  __syncthreads();
  // 4. the kept blocks in ascending id order, then -1
  for (int cnd = tid; cnd < n_cand; cnd += 256)
    if (keep[cnd]) {
      int pos = 0;
      for (int g2 = 0; g2 < cnd; ++g2) pos += keep[g2];
      out[pos] = frames_kept[cnd / a.nbf] * a.nbf + cnd % a.nbf;
    }
  for (int e = min(a.kb, n_cand) + tid; e < a.kb; e += 256) out[e] = -1;
}

}  // namespace

hipError_t launch_hsa_pool(const HsaPoolArgs &a, int D, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.B * a.H * a.n_frames);
  if (D == 128)
    hipLaunchKernelGGL(hsa_pool_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(hsa_pool_kernel<64>, dim3(grid), dim3(256), 0, s, a);
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
