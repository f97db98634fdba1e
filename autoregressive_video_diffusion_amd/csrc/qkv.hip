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
//     (2j, 2j+1) are registers r, r+1 of one lane, and registers 4i..4i+3
//     are 4 consecutive features of one token, stored as one 8-byte write.
//   * A 32-feature block lies inside one of Q, K, V and one head (D is a
//     multiple of 32), so the epilogue decides per block where it goes: Q'
//     to [B, n, H, D], K' and V to the cache rows cache_pos + i.
//
// Work decomposition: a workgroup of 8 wavefronts computes 256 features x
// 128 tokens; wavefront w owns features 64*(w%4) and tokens 64*(w/4), 2 x 2
// accumulator blocks.  C is walked in steps of 32 through a 5-stage LDS ring
// filled by global -> LDS DMA four steps ahead; rows are padded to 5 cells
// (80 bytes) so that the 16 rows a quarter-wavefront reads fall on distinct
// bank groups.
#include "crattn_internal.h"
#include "rope_common.h"
#include "../../include/crattn.h"

namespace crattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 256;      // features per workgroup
constexpr int kBN = 128;      // tokens per workgroup
constexpr int kBK = 32;       // C per ring stage
constexpr int kNW = 8;        // wavefronts per workgroup
constexpr int kNS = 5;        // ring stages
constexpr int kPitch = 5;     // 16-byte cells per LDS row (4 data + 1 pad)
constexpr int kACells = kBM * kPitch;
constexpr int kBCells = kBN * kPitch;
constexpr int kStageCells = kACells + kBCells;
constexpr int kAInstr = kACells / 64;  // DMA instructions per stage
constexpr int kBInstr = kBCells / 64;
constexpr int kASlots = (kAInstr + kNW - 1) / kNW;
constexpr int kBSlots = (kBInstr + kNW - 1) / kNW;
constexpr int kDmaMin = kAInstr / kNW + kBInstr / kNW;  // fewest copies a wavefront issues per stage
static_assert(kACells % 64 == 0 && kBCells % 64 == 0, "whole DMA instructions");
static_assert(kDmaMin >= 1 && (kNS - 2) * kDmaMin < 64, "vmcnt wait range");

struct QkvKArgs {
  const uint16_t *x;   // [M = B * n][C]
  const uint16_t *w;   // [F = 3 * H * D][C]
  uint16_t *q_out;     // [B][n][H][D] or null (then features start at H*D)
  uint16_t *k_cache;   // [B][H][cap][D]
  uint16_t *v_cache;
  const float2 *table;
  int64_t cap, cache_pos, n;
  int M, F, f_begin, C, H, D;
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
#pragma clang diagnostic pop

__global__ void __launch_bounds__(kNW * 64, 1) qkv_rope_kernel(QkvKArgs a) {
  __shared__ uint4 ring[kNS * kStageCells];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5;
  const int l32 = lane & 31;
  const int fw = wave & 3, tw = wave >> 2;

  // feature tile (fastest) then token tile: the workgroups that share a
  // token tile of X run together
  const int n_ft = (a.F - a.f_begin + kBM - 1) / kBM;
  const int f0 = a.f_begin + (int)(blockIdx.x % n_ft) * kBM;
  const int m0 = (int)(blockIdx.x / n_ft) * kBN;

  // ---- per-lane DMA offsets (bytes from the tile's first row, column 0);
  // rows past the matrix re-read its last row, pad cells their row's first
  // chunk (written into a pad cell nobody reads) ----
  auto cell_off = [&](int cell, int rows_valid) -> uint32_t {
    int row = cell / kPitch;
    const int c = cell - row * kPitch;
    row = min(row, rows_valid - 1);
    return (uint32_t)row * (uint32_t)a.C * 2u + (uint32_t)(c < 4 ? c * 16 : 0);
  };
  uint32_t a_off[kASlots], b_off[kBSlots];
#pragma unroll
  for (int s = 0; s < kASlots; ++s) a_off[s] = cell_off((wave + s * kNW) * 64 + lane, a.F - f0);
#pragma unroll
  for (int s = 0; s < kBSlots; ++s) b_off[s] = cell_off((wave + s * kNW) * 64 + lane, a.M - m0);
  typedef __attribute__((address_space(3))) char lds_char_t;
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(lds_char_t *)reinterpret_cast<char *>(ring));
  const uint16_t *wa = a.w + (int64_t)f0 * a.C;
  const uint16_t *xb = a.x + (int64_t)m0 * a.C;
  auto dma = [&](int ks, int stage) {
    const int c0 = __builtin_amdgcn_readfirstlane(ks) * kBK;
    const uint32_t adst = ring_lds + (uint32_t)stage * (kStageCells * 16);
    const uint32_t bdst = adst + kACells * 16;
#pragma unroll
    for (int s = 0; s < kASlots; ++s) {
      const int j = wave + s * kNW;
      if ((s + 1) * kNW <= kAInstr || j < kAInstr) lds_dma16(wa + c0, a_off[s], adst + j * 1024);
    }
#pragma unroll
    for (int s = 0; s < kBSlots; ++s) {
      const int j = wave + s * kNW;
      if ((s + 1) * kNW <= kBInstr || j < kBInstr) lds_dma16(xb + c0, b_off[s], bdst + j * 1024);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = a.C / kBK;
#pragma unroll
  for (int s = 0; s < kNS - 1; ++s)
    if (s < nk) dma(s, s);

  for (int ks = 0; ks < nk; ++ks) {
    const int stage = ks % kNS;
    // stage ks has landed once only the later stages' copies are pending
    const int later = min(nk - 1 - ks, kNS - 2);
    if (later >= 3)
      wait_vmcnt<3 * kDmaMin>();
    else if (later == 2)
      wait_vmcnt<2 * kDmaMin>();
    else if (later == 1)
      wait_vmcnt<kDmaMin>();
    else
      wait_vmcnt<0>();
    // every wavefront sees stage ks and is done with step ks-1, whose slot
    // the next copy refills
    __syncthreads();
    if (ks + kNS - 1 < nk) dma(ks + kNS - 1, (ks + kNS - 1) % kNS);

    const uint4 *__restrict__ at = ring + stage * kStageCells;
    const uint4 *__restrict__ bt = at + kACells;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t, at[(fw * 64 + i * 32 + l32) * kPitch + kk * 2 + hf]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8_t, bt[(tw * 64 + j * 32 + l32) * kPitch + kk * 2 + hf]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: rotate Q/K pairs, store Q', K', V ----
  const int HD = a.H * a.D;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + tw * 64 + j * 32 + l32;
    if (m >= a.M) continue;
    const int64_t b = m / a.n, i_tok = m - b * a.n;
    const Pos p = decode_pos(a.tok_off + (uint32_t)i_tok, a.per_frame, a.gw, a.t0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int fb = f0 + fw * 64 + i * 32;  // first feature of the block
      if (fb >= a.F) continue;
      const int part = fb / HD;              // 0 Q, 1 K, 2 V
      const int h = (fb - part * HD) / a.D;
      const int d_blk = fb - part * HD - h * a.D;
      uint16_t *dst;
      if (part == 0)
        dst = a.q_out + ((int64_t)m * a.H + h) * a.D;
      else
        dst = (part == 1 ? a.k_cache : a.v_cache) +
              (((int64_t)b * a.H + h) * a.cap + a.cache_pos + i_tok) * a.D;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = d_blk + 8 * g + 4 * hf;  // 4 consecutive features
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * g + e];
        if (part < 2) {
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float2 cs = pair_cs(a.table, a.tg, (uint32_t)(d0 + e) >> 1, p);
            const float xr = y[e], yr = y[e + 1];
            y[e] = xr * cs.x - yr * cs.y;
            y[e + 1] = xr * cs.y + yr * cs.x;
          }
        }
        uint2 wv;
        wv.x = pack_bf16(y[0], y[1]);
        wv.y = pack_bf16(y[2], y[3]);
        *reinterpret_cast<uint2 *>(dst + d0) = wv;
      }
    }
  }
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
  const int n_ft = (a.F - a.f_begin + kBM - 1) / kBM;
  const int n_tt = (a.M + kBN - 1) / kBN;
  hipLaunchKernelGGL(qkv_rope_kernel, dim3((unsigned)(n_ft * n_tt)), dim3(kNW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace crattn
