// 3D Causal-RoPE: cos/sin table precompute and the fused rotate + KV-append
// pass, for AMD CDNA4 (gfx950).
//
// Sources: "Accelerating Video Generation Inference with Sequential-Parallel
// 3D Positional Encoding Using a Global Time Index", technical summary
// §2.B (global time index t_global = t + s, local rotation from the start
// offset and local index, no gather) and §2.C (cos/sin precomputed into
// contiguous device tensors; RoPE fused into one kernel).  The rotary code
// itself is the standard per-pair 2-D rotation, applied per axis group
// (t, h, w) of head_dim.
//
// The append pass is bound by HBM bandwidth: per token and head it reads
// Q, K, V rows and writes Q', K', V rows once, 16 bytes per lane per tensor,
// with every wavefront covering whole 256-byte rows, and streaming stores.
// The table (tens of KB) stays in L1/L2.
#include "crattn_internal.h"
#include "rope_common.h"
#include "../../include/crattn.h"


namespace crattn {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// One thread per table entry (axis, position, pair).  The angle and its
// sine/cosine are evaluated in double precision, then rounded to float: at
// positions of ~80 an fp32 angle alone would carry ~8e-6 absolute error.
__global__ void __launch_bounds__(256) rope_table_kernel(RopeTableArgs a, int total) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int nt = a.max_t * (a.dt / 2);
  const int nh = a.max_h * (a.dh / 2);
  int Da, local;
  if (e < nt) {
    Da = a.dt;
    local = e;
  } else if (e < nt + nh) {
    Da = a.dh;
    local = e - nt;
  } else {
    Da = a.dw;
    local = e - nt - nh;
  }
  const int half = Da / 2;
  const int p = local / half;
  const int j = local - p * half;
  const double freq = pow(a.theta, -2.0 * (double)j / (double)Da);
  const double phi = (double)p * freq;
  double s, c;
  sincos(phi, &s, &c);
  a.table[e] = make_float2((float)c, (float)s);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// Streaming (non-temporal) 16-byte store.  Every output of the append pass
// is written once and not re-read by this kernel; streaming stores avoid
// allocating them in the caches on the way out (measured: 19.1 -> 13.9 us on
// the 480P chunk, 4.5 -> 6.2 TB/s).  Non-temporal loads did not help.
__device__ inline void ntstore(const uint4 &x, void *p) {
  const u32x4_t v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
}
__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  f32x2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

// Rotate the bf16 pair packed in one dword (element 2j in the low half).
__device__ inline uint32_t rot_bf16(uint32_t u, float2 cs) {
  const float2 r = rotate_pair(bf_lo(u), bf_hi(u), cs);
  return pack_bf16(r.x, r.y);
}

// Unsigned division by a divisor fixed for the launch as a multiply-high, an
// add and a shift (Granlund and Montgomery, "Division by Invariant Integers
// using Multiplication", 1994: the round-up multiplier for 32-bit operands
// with a 33-bit add): l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (mulhi(n, m) + n) >> l for every 32-bit n.  d in [1, 2^31].
struct FastDiv {
  uint32_t m, l;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  return FastDiv{(uint32_t)m, l};
}
__device__ inline uint32_t fdiv(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.l);
}

struct AppendGeom {
  uint32_t total;      // B * n * H * V threads
  uint32_t V;          // 16-byte vectors per row
  uint32_t n, H;
  uint32_t per_frame, gw, t0, tok_off;
  FastDiv dV, dH, dn, dframe, dgw;  // the same divisors for the bf16 pass
};

// Where one 16-byte vector of one (b, token, head) row lives.  Vector order
// is the input order (vector, head, token, batch), so Q/K/V reads are fully
// contiguous and each cache write covers whole rows of one head.
struct VecAt {
  size_t in_off, cache_off;  // in elements
  uint32_t pair0;            // first feature pair of the vector
  Pos p;
};

__device__ inline VecAt locate(uint32_t t, const RopeAppendArgs &a, const AppendGeom &g) {
  const uint32_t row = fdiv(t, g.dV);  // (b * n + i) * H + h
  const uint32_t c = t - row * g.V;
  const uint32_t bi = fdiv(row, g.dH);
  const uint32_t h = row - bi * g.H;
  const uint32_t b = fdiv(bi, g.dn);
  const uint32_t i = bi - b * g.n;
  const uint32_t tok = g.tok_off + i;
  const uint32_t f = fdiv(tok, g.dframe);
  const uint32_t in_frame = tok - f * g.per_frame;
  const uint32_t r = fdiv(in_frame, g.dgw);
  VecAt v;
  v.p = Pos{g.t0 + f, r, in_frame - r * g.gw};
  v.in_off = (size_t)row * (size_t)a.D + (size_t)c * 8;
  v.cache_off = (((size_t)b * g.H + h) * (size_t)a.cap + (size_t)a.cache_pos + i) * (size_t)a.D +
                (size_t)c * 8;
  v.pair0 = c * 4;
  return v;
}

// The inputs of one vector: K, V, Q (zero when there is no Q) and the four
// (cos, sin) pairs it rotates by.
struct VecIn {
  uint4 k, v, q;
  float2 cs[4];
};

__device__ inline VecIn load_vec(const VecAt &at, const RopeAppendArgs &a, const TabGeom &tg) {
  VecIn x;
  x.k = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + at.in_off);
  x.v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + at.in_off);
  x.q = make_uint4(0, 0, 0, 0);
  if (a.q != nullptr)
    x.q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + at.in_off);
#pragma unroll
  for (int j = 0; j < 4; ++j) x.cs[j] = pair_cs(a.table, tg, at.pair0 + j, at.p);
  return x;
}

__device__ inline void store_vec(const VecAt &at, const VecIn &x, const RopeAppendArgs &a) {
  const uint4 ko = make_uint4(rot_bf16(x.k.x, x.cs[0]), rot_bf16(x.k.y, x.cs[1]),
                              rot_bf16(x.k.z, x.cs[2]), rot_bf16(x.k.w, x.cs[3]));
  ntstore(ko, static_cast<uint16_t *>(a.k_cache) + at.cache_off);
  ntstore(x.v, static_cast<uint16_t *>(a.v_cache) + at.cache_off);
  if (a.q != nullptr) {
    const uint4 qo = make_uint4(rot_bf16(x.q.x, x.cs[0]), rot_bf16(x.q.y, x.cs[1]),
                                rot_bf16(x.q.z, x.cs[2]), rot_bf16(x.q.w, x.cs[3]));
    ntstore(qo, static_cast<uint16_t *>(a.q_out) + at.in_off);
  }
}

// One thread per 16-byte vector.
__global__ void __launch_bounds__(256) rope_append_bf16_kernel(RopeAppendArgs a, AppendGeom g,
                                                                TabGeom tg) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  if (t >= g.total) return;
  const VecAt at = locate(t, a, g);
  store_vec(at, load_vec(at, a, tg), a);
}

__device__ inline float2 rot_f32(float x, float y, float2 cs) { return rotate_pair(x, y, cs); }

// fp32 variant: a 16-byte vector is two pairs.
__global__ void __launch_bounds__(256) rope_append_f32_kernel(RopeAppendArgs a, AppendGeom g,
                                                               TabGeom tg) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  if (t >= g.total) return;
  const uint32_t c = t % g.V;
  const uint32_t row = t / g.V;
  const uint32_t h = row % g.H;
  const uint32_t bi = row / g.H;
  const uint32_t i = bi % g.n;
  const uint32_t b = bi / g.n;
  const Pos p = decode_pos(g.tok_off + i, g.per_frame, g.gw, g.t0);

  const size_t in_off = (size_t)row * (size_t)a.D + (size_t)c * 4;
  const size_t cache_off =
      (((size_t)b * g.H + h) * (size_t)a.cap + (size_t)a.cache_pos + i) * (size_t)a.D +
      (size_t)c * 4;

  const float4 kv = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.k) + in_off);
  const float4 vv = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.v) + in_off);
  const bool has_q = a.q != nullptr;
  float4 qv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (has_q) qv = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.q) + in_off);

  const float2 cs0 = pair_cs(a.table, tg, c * 2 + 0, p);
  const float2 cs1 = pair_cs(a.table, tg, c * 2 + 1, p);
  const float2 k0 = rot_f32(kv.x, kv.y, cs0), k1 = rot_f32(kv.z, kv.w, cs1);
  ntstore(make_uint4(__float_as_uint(k0.x), __float_as_uint(k0.y), __float_as_uint(k1.x),
                     __float_as_uint(k1.y)),
          static_cast<float *>(a.k_cache) + cache_off);
  ntstore(make_uint4(__float_as_uint(vv.x), __float_as_uint(vv.y), __float_as_uint(vv.z),
                     __float_as_uint(vv.w)),
          static_cast<float *>(a.v_cache) + cache_off);
  if (has_q) {
    const float2 q0 = rot_f32(qv.x, qv.y, cs0), q1 = rot_f32(qv.z, qv.w, cs1);
    ntstore(make_uint4(__float_as_uint(q0.x), __float_as_uint(q0.y), __float_as_uint(q1.x),
                       __float_as_uint(q1.y)),
            static_cast<float *>(a.q_out) + in_off);
  }
}

}  // namespace

hipError_t launch_rope_table(const RopeTableArgs &a, hipStream_t s) {
  const int total = a.max_t * (a.dt / 2) + a.max_h * (a.dh / 2) + a.max_w * (a.dw / 2);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((total + 255) / 256), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

hipError_t launch_rope_append(const RopeAppendArgs &a, hipStream_t s) {
  const RopeSplit sp = rope_split(a.D);
  TabGeom tg;
  tg.ht = (uint32_t)(sp.dt / 2);
  tg.hh = (uint32_t)(sp.dh / 2);
  tg.base_h = (uint32_t)a.max_t * tg.ht;
  tg.base_w = tg.base_h + (uint32_t)a.max_h * tg.hh;
  AppendGeom g;
  const int esize = a.dtype == CRATTN_BF16 ? 2 : 4;
  g.V = (uint32_t)(a.D * esize / 16);
  g.n = (uint32_t)a.n;
  g.H = (uint32_t)a.H;
  g.total = (uint32_t)((uint64_t)a.B * (uint64_t)a.n * (uint64_t)a.H * g.V);
  g.per_frame = (uint32_t)a.grid_h * (uint32_t)a.grid_w;
  g.gw = (uint32_t)a.grid_w;
  g.t0 = (uint32_t)a.t0;
  g.tok_off = (uint32_t)a.tok_off;
  g.dV = make_fastdiv(g.V);
  g.dH = make_fastdiv(g.H);
  g.dn = make_fastdiv(g.n);
  g.dframe = make_fastdiv(g.per_frame);
  g.dgw = make_fastdiv(g.gw);
  const dim3 grid((g.total + 255u) / 256u);
  if (a.dtype == CRATTN_BF16)
    hipLaunchKernelGGL(rope_append_bf16_kernel, grid, dim3(256), 0, s, a, g, tg);
  else
    hipLaunchKernelGGL(rope_append_f32_kernel, grid, dim3(256), 0, s, a, g, tg);
  return hipGetLastError();
}

}  // namespace crattn
