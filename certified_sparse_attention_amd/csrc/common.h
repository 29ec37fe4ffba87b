// Internal definitions shared by the HIP kernels of the certified decode path.
// Arithmetic rules (the same written rules the CPU oracle follows; no code is
// shared with it):
//   R1  fp64 sums over the 128 channels: eight sequential partial sums over
//       channels 16p..16p+15, combined ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)).
//   R2  no fused multiply-add in the fp64/fp32 arithmetic that decides sets
//       (the library is built with -ffp-contract=off).
//   R5  first(x) = min{ j in [0, J] : x >= logtau[j] }, J+1 if none.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/csa.h"

namespace csa {

constexpr double kLn2 = 0.6931471805599453;        // fp64 rounding of ln 2
constexpr double kRsqrtD = 0.08838834764831845;    // fp64 rounding of 2^-3.5
constexpr double kPadF = 0x1p-40;                  // relative pad
constexpr int kD = 128;
constexpr int kBlk = 32;
constexpr int kMaxJ = 60;
constexpr int kMaxG = 7;
constexpr int kBlocksPerWave = 16;                 // refinement: blocks per wavefront slot
constexpr int kScanBlocks = 32;                    // streaming scan: blocks per wavefront
constexpr int kNumSeg = 64;                        // accumulate: max segments per query
constexpr int kStatW = 262;                        // per-level stats N[128] V[128] D Q k P X (X:
                                                   // exact reads outside C_max), and a pad
                                                   // column (rows 16-byte aligned and 524
                                                   // dwords apart: level-strided LDS reads
                                                   // spread over the banks)

struct BlockMeta {   // 16 bytes per packed block
  float ksmax;
  int32_t kexp;
  int32_t z1sum;
  float kmax;
};

typedef int v4i __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- fp16 <-> fp64
__host__ __device__ inline double h2d(uint16_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, h);
}
__host__ __device__ inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Round-to-nearest-even fp64 -> fp16 written from the binary16 definition
// (no intermediate fp32 rounding).
__device__ inline uint16_t d2h_rne(double x) {
  uint64_t bits = (uint64_t)__double_as_longlong(x);
  uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
  double a = fabs(x);
  if (!(a < 65520.0)) return (uint16_t)(sign | 0x7C00u);          // overflow -> inf
  if (a < 0x1p-14) {                                               // subnormal range: m 2^-24
    double m = rint(a * 0x1p24);                                   // 0..1024 (1024 = min normal)
    return (uint16_t)(sign | (uint16_t)m);
  }
  int e = ilogb(a);                                                // 2^e <= a < 2^(e+1)
  double m = rint(ldexp(a, 10 - e));                               // in [1024, 2048]
  if (m == 2048.0) { m = 1024.0; e += 1; }
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024));
}

// Smallest non-negative fp16 h with h*h >= T (h*h exact in fp64).
__device__ inline uint16_t f16_sqrt_up(double T) {
  if (!(T > 0.0)) return 0;
  uint16_t h = d2h_rne(sqrt(T));
  while (h < 0x7C00u) {
    double v = h2d(h);
    if (v * v >= T) break;
    ++h;
  }
  while (h > 0) {
    double v = h2d((uint16_t)(h - 1));
    if (v * v >= T) --h; else break;
  }
  return h;
}

// Smallest non-negative fp32 y with y*y >= T (y*y exact in fp64).
__device__ inline float f32_sqrt_up(double T) {
  if (!(T > 0.0)) return 0.0f;
  uint32_t b = __float_as_uint((float)sqrt(T));
  while (b < 0x7F800000u) {
    double v = (double)__uint_as_float(b);
    if (v * v >= T) break;
    ++b;
  }
  while (b > 0) {
    double v = (double)__uint_as_float(b - 1);
    if (v * v >= T) --b; else break;
  }
  return __uint_as_float(b);
}

// Smallest fp32 value >= x.
__device__ inline float f32_up(double x) {
  float f = (float)x;
  if ((double)f < x) f = nextafterf(f, __builtin_huge_valf());
  return f;
}

// ---------------------------------------------------------------- R1 sum
struct Canon {
  double p[8];
};
// Sum of 128 values given by a functor f(t) in the R1 order.
template <class F>
__device__ inline double canon_sum(F f) {
  double p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    double acc = f(16 * k);
#pragma unroll
    for (int t = 1; t < 16; ++t) acc = acc + f(16 * k + t);
    p[k] = acc;
  }
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// Exact score s = R1-sum(q_t k_t) * RSQRT_D of one fp16 key row (256 bytes).
__device__ inline double exact_score(const double *qd, const uint16_t *krow) {
  const uint4 *src = reinterpret_cast<const uint4 *>(krow);
  double p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint4 a = src[2 * k], b = src[2 * k + 1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    double acc = qd[16 * k] * h2d((uint16_t)(w[0] & 0xFFFFu));
#pragma unroll
    for (int t = 1; t < 16; ++t) {
      uint16_t hv = (uint16_t)((t & 1) ? (w[t >> 1] >> 16) : (w[t >> 1] & 0xFFFFu));
      acc = acc + qd[16 * k + t] * h2d(hv);
    }
    p[k] = acc;
  }
  return (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]))) * kRsqrtD;
}

// The same exact score with the query given as fp32 values (each an exact fp16 value).
__device__ inline double exact_score_qf(const float *qf, const uint16_t *krow) {
  const uint4 *src = reinterpret_cast<const uint4 *>(krow);
  const float4 *q4 = reinterpret_cast<const float4 *>(qf);
  double p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint4 a = src[2 * k], b = src[2 * k + 1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float4 qa = q4[4 * k], qb = q4[4 * k + 1], qc = q4[4 * k + 2], qe = q4[4 * k + 3];
    float q[16] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w, qc.x, qc.y, qc.z, qc.w, qe.x, qe.y, qe.z, qe.w};
    double acc = (double)q[0] * h2d((uint16_t)(w[0] & 0xFFFFu));
#pragma unroll
    for (int t = 1; t < 16; ++t) {
      uint16_t hv = (uint16_t)((t & 1) ? (w[t >> 1] >> 16) : (w[t >> 1] & 0xFFFFu));
      acc = acc + (double)q[t] * h2d(hv);
    }
    p[k] = acc;
  }
  return (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]))) * kRsqrtD;
}

// Wavefront-cooperative R1 sums: lane 8s + k holds chunk k (16 channels, summed in
// order) of item s; r1_combine8 returns ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7))
// to all 8 lanes of the item (IEEE addition is commutative, so the butterfly forms
// exactly those sums).
__device__ inline double r1_combine8(double p) {
  p = p + __shfl_xor(p, 1, 64);
  p = p + __shfl_xor(p, 2, 64);
  p = p + __shfl_xor(p, 4, 64);
  return p;
}
// Inclusive prefix sum over the wavefront's 64 lanes with DPP moves (shifts within rows of
// 16, then the row broadcasts of lanes 15 and 31), no LDS round trips.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
  return x;
}

// One DPP move of a double (both halves; lanes without a source get 0).
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, kCtrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), kCtrl, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
// The same sum as r1_combine8, ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7)) over the
// eight lanes of an item, but only in the item's first lane (lane 8 i): two quad
// exchanges and a shift by four lanes within the row, no LDS round trips.
__device__ __forceinline__ double r1_combine8_first(double p) {
  p = p + dpp_f64<0xB1>(p);    // quad_perm(1, 0, 3, 2): lane ^ 1
  p = p + dpp_f64<0x4E>(p);    // quad_perm(2, 3, 0, 1): lane ^ 2
  return p + dpp_f64<0x104>(p);   // row_shl:4: lane + 4 (the item's second half)
}

// The same sum as r1_combine8 in all eight lanes of the item (identical bits: the last
// addition is A + B in the first half and B + A in the second), by DPP moves: two quad
// exchanges, then the other half of the item by a shift of four lanes either way.
__device__ __forceinline__ double r1_combine8_all(double p) {
  p = p + dpp_f64<0xB1>(p);    // lane ^ 1
  p = p + dpp_f64<0x4E>(p);    // lane ^ 2
  const double up = dpp_f64<0x104>(p), dn = dpp_f64<0x114>(p);   // row_shl:4, row_shr:4
  return p + (((threadIdx.x & 4) != 0) ? dn : up);
}
// q . k over sixteen fp16 values held in two 16-byte words (q given as doubles), in
// index order.
__device__ inline double score_words(const double *q16, uint4 a, uint4 b) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  double acc = q16[0] * h2d((uint16_t)(w[0] & 0xFFFFu));
#pragma unroll
  for (int t = 1; t < 16; ++t) {
    const uint16_t hv = (uint16_t)((t & 1) ? (w[t >> 1] >> 16) : (w[t >> 1] & 0xFFFFu));
    acc = acc + q16[t] * h2d(hv);
  }
  return acc;
}
// Chunk k of q . k for one fp16 key row (q given as doubles of the chunk).
__device__ inline double score_chunk(const double *q16, const uint16_t *krow, int k) {
  const uint4 *src = reinterpret_cast<const uint4 *>(krow) + 2 * k;
  return score_words(q16, src[0], src[1]);
}
// |v|^2 of the sixteen fp16 values held in two 16-byte words, in index order.
__device__ inline double sumsq_words(uint4 a, uint4 b) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const double v0 = h2d((uint16_t)(w[0] & 0xFFFFu));
  double acc = v0 * v0;
#pragma unroll
  for (int t = 1; t < 16; ++t) {
    const double v = h2d((uint16_t)((t & 1) ? (w[t >> 1] >> 16) : (w[t >> 1] & 0xFFFFu)));
    acc = acc + v * v;
  }
  return acc;
}
// Chunk k of |v|^2 for one fp16 row.
__device__ inline double sumsq_chunk(const uint16_t *row, int k) {
  const uint4 *src = reinterpret_cast<const uint4 *>(row) + 2 * k;
  return sumsq_words(src[0], src[1]);
}

// First level j in [0, J + 1] with lt[j] <= x (J + 1 if none), for the table
// lt[j] = (-j ln 2) / r.  The estimate e = ceil(x / lt[1]) differs from the true
// threshold x / lt[1] by a few ulps of a number below J + 2, far less than one level,
// so the answer is e - 1, e or e + 1, settled by one step from the neighbour pair
// ltp[e] = (lt[e - 1], lt[e]) read at once (ltp[j] for j = 0..J+1, with lt[-1] = +inf
// and lt[J + 1] = -inf; fill_level_pairs writes that table).
__device__ inline void fill_level_pairs(double2 *ltp, const double *lt, int J, int t, int nt) {
  for (int j = t; j <= J + 1; j += nt)
    ltp[j] = make_double2(j > 0 ? lt[j - 1] : __builtin_huge_val(), j <= J ? lt[j] : -__builtin_huge_val());
}
__device__ inline int level_of_pairs(double x, const double2 *ltp, int J, double inv_l1) {
  const double e = ceil(x * inv_l1);
  const int j = !(e > 0.0) ? 0 : (!(e < (double)(J + 1)) ? J + 1 : (int)e);
  double below = ltp[j].x, here = ltp[j].y;
  // both values are taken as they are read (so the compiler keeps one read, not a second
  // one behind a branch)
  __asm__ volatile("" : "+v"(below), "+v"(here));
  return (here > x) ? j + 1 : ((below <= x) ? j - 1 : j);
}

// R1 sum of squares of one fp16 row.
__device__ inline double row_sumsq(const uint16_t *row) {
  const uint4 *src = reinterpret_cast<const uint4 *>(row);
  double p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint4 a = src[2 * k], b = src[2 * k + 1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    double v0 = h2d((uint16_t)(w[0] & 0xFFFFu));
    double acc = v0 * v0;
#pragma unroll
    for (int t = 1; t < 16; ++t) {
      uint16_t hv = (uint16_t)((t & 1) ? (w[t >> 1] >> 16) : (w[t >> 1] & 0xFFFFu));
      double v = h2d(hv);
      acc = acc + v * v;
    }
    p[k] = acc;
  }
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// ---------------------------------------------------------------- levels
// R5 by binary search over the strictly decreasing table lt[0..J].
__device__ inline int first_level(double x, const double *lt, int J) {
  int lo = 0, hi = J + 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (lt[mid] > x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------- hash
// SplitMix64 output function (Steele, Lea and Flood 2014; Mix13 finalizer):
// one generator step applied to state x.
__host__ __device__ inline uint64_t mix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__host__ __device__ inline uint64_t hash_prefix(uint64_t seed, uint64_t step, uint64_t layer,
                                                uint64_t kv_head) {
  uint64_t h = mix64(seed);
  h = mix64(h ^ step);
  h = mix64(h ^ layer);
  return mix64(h ^ kv_head);
}
// The steps and constants below follow fdlibm's e_log.c, which carries this notice:
//   Copyright (C) 1993 by Sun Microsystems, Inc. All rights reserved.
//   Developed at SunPro, a Sun Microsystems, Inc. business.
//   Permission to use, copy, modify, and distribute this software is freely granted,
//   provided that this notice is preserved.
// ln x for normal positive x, written from the steps of fdlibm's e_log.c (Sun
// Microsystems, 1993): x = 2^k (1 + f), s = f / (2 + f), an odd polynomial in s with
// coefficients Lg1..Lg7, ln 2 split into a high and a low part.  Evaluated in fp64
// in the written order without fused operations, so every implementation of the
// specification returns the same bits (the library's own log would differ from
// other implementations in the last bit for some inputs).
__device__ inline double log_spec(double x) {
  constexpr double ln2_hi = 0x1.62e42feep-1;           // 3fe62e42 fee00000
  constexpr double ln2_lo = 0x1.a39ef35793c76p-33;     // 3dea39ef 35793c76
  constexpr double Lg1 = 0x1.5555555555593p-1, Lg2 = 0x1.999999997fa04p-2;
  constexpr double Lg3 = 0x1.2492494229359p-2, Lg4 = 0x1.c71c51d8e78afp-3;
  constexpr double Lg5 = 0x1.7466496cb03dep-3, Lg6 = 0x1.39a09d078c69fp-3;
  constexpr double Lg7 = 0x1.2f112df3e5244p-3;
  const uint64_t bits = (uint64_t)__double_as_longlong(x);
  int32_t hx = (int32_t)(bits >> 32);
  const uint32_t lx = (uint32_t)bits;
  int32_t k = (hx >> 20) - 1023;
  hx &= 0x000fffff;
  const int32_t i = (hx + 0x95f64) & 0x100000;
  const double xn = __longlong_as_double(
      (long long)(((uint64_t)(uint32_t)(hx | (i ^ 0x3ff00000)) << 32) | (uint64_t)lx));
  k += (i >> 20);
  const double f = xn - 1.0;
  const double dk = (double)k;
  if ((0x000fffff & (2 + hx)) < 3) {   // |f| < 2^-20
    if (f == 0.0) return (k == 0) ? 0.0 : dk * ln2_hi + dk * ln2_lo;
    const double R = f * f * (0.5 - 0.33333333333333333 * f);
    return (k == 0) ? f - R : dk * ln2_hi - ((R - dk * ln2_lo) - f);
  }
  const double s = f / (2.0 + f);
  const double z = s * s;
  int32_t ii = hx - 0x6147a;
  const double w = z * z;
  const int32_t j = 0x6b851 - hx;
  const double t1 = w * (Lg2 + w * (Lg4 + w * Lg6));
  const double t2 = z * (Lg1 + w * (Lg3 + w * (Lg5 + w * Lg7)));
  ii |= j;
  const double R = t2 + t1;
  if (ii > 0) {
    const double hfsq = 0.5 * f * f;
    return (k == 0) ? f - (hfsq - s * (hfsq + R)) : dk * ln2_hi - ((hfsq - (s * (hfsq + R) + dk * ln2_lo)) - f);
  }
  return (k == 0) ? f - s * (f - R) : dk * ln2_hi - ((s * (f - R) - dk * ln2_lo) - f);
}

// E = -ln u, u = ((h >> 11) + 1) 2^-53 in (0, 1].
__device__ inline double perturbation(uint64_t prefix, int64_t pos) {
  uint64_t h = mix64(prefix ^ (uint64_t)pos);
  double u = (double)((h >> 11) + 1ull) * 0x1p-53;
  return -log_spec(u);
}

// ---------------------------------------------------------------- ordered fp64
__host__ __device__ inline unsigned long long enc_max(double x) {
  unsigned long long b = (unsigned long long)__builtin_bit_cast(long long, x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__host__ __device__ inline double dec_max(unsigned long long e) {
  unsigned long long b = (e >> 63) ? (e & 0x7FFFFFFFFFFFFFFFull) : ~e;
  return __builtin_bit_cast(double, (long long)b);
}

// ---------------------------------------------------------------- wave helpers
__device__ inline int lane_id() { return (int)(threadIdx.x & 63u); }

__device__ inline int bperm_i32(int src_lane, int v) {
  return __builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}
__device__ inline double bperm_f64(int src_lane, double v) {
  long long b = __builtin_bit_cast(long long, v);
  int lo = bperm_i32(src_lane, (int)(b & 0xFFFFFFFFll));
  int hi = bperm_i32(src_lane, (int)(b >> 32));
  long long r = ((long long)(unsigned)hi << 32) | (unsigned)lo;
  return __builtin_bit_cast(double, r);
}
__device__ inline double wave_max_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}

// ---------------------------------------------------------------- batch of items
// One call covers `nitems` items (requests, or layers of one request), each with its own
// cached length n and its own cache slot; the kernels see nitems * H_kv units, unit u
// being KV head u % H_kv of item u / H_kv.  Workspace rows are per unit (query head
// u G + g); cache rows are those of cache head slot H_kv + (u % H_kv).  Passed by value
// in every kernel's arguments.
constexpr int kMaxItems = 64;
struct Batch {
  int nitems, H_kv;
  int64_t n[kMaxItems];
  int32_t slot[kMaxItems];
};
// (a single item reads its entries at fixed offsets: no division and no load that waits
// for one)
__host__ __device__ inline int unit_item(const Batch &b, int u) { return b.nitems == 1 ? 0 : u / b.H_kv; }
__host__ __device__ inline int64_t unit_n(const Batch &b, int u) { return b.nitems == 1 ? b.n[0] : b.n[u / b.H_kv]; }
__host__ __device__ inline int64_t unit_npool(const Batch &b, int u, int W) {
  const int64_t n = unit_n(b, u);
  return n > W ? n - W : 0;
}
__host__ __device__ inline int64_t unit_kv(const Batch &b, int u) {
  if (b.nitems == 1) return (int64_t)b.slot[0] * b.H_kv + u;
  return (int64_t)b.slot[u / b.H_kv] * b.H_kv + u % b.H_kv;
}

// ---------------------------------------------------------------- workspace plan
struct Plan {
  int H_kv, G, H_q, J, W;   // H_kv, H_q: units and their query heads (all items)
  int64_t npool_cap;   // pool capacity per query head
  int64_t ntiles;      // bucket tiles per query head
  int64_t wstride;     // scan wavefronts per KV head at full pool capacity
  // offsets in bytes
  size_t qf, qconst, qA, lt, tau, prefix, sR, cR;     // per-call constants
  size_t clo, cstar, lbpart, vpart, hist, tilelist, tilehist, tilecm, cmhist, ccount, ccount1, jspec;
  size_t exdone, exdone2;  // per-head completion counters (last-workgroup reductions)
  size_t ccount2, jspec2, flags2;
  size_t pbuf, ubuf, lub, live, bmax, win, candpos, rec_s, rec_w, rec_vsq, rec_hl, rec_x;
  size_t partial, betalv, dhatlv, klv, flags, exactp;
  int nseg_cap;        // segment rows per query head in `partial`
  size_t total;
};

// Per-query constants (fp64 slots in qconst[hq][kQc])
enum { QC_BETA = 0, QC_QNP, QC_QABS, QC_CR, QC_QA, QC_QN, QC_PILOT, kQc = 8 };

constexpr int kBucketTile = 2048;   // positions per bucket tile (64 bitmap words)
constexpr int kTileList = 64;       // positions per tile listed in level order (the tile's lowest levels)
constexpr int kDefaultBudget = 32;   // candidates rescored before the first certificate pass
constexpr int kExactChunks = 8;                    // tail: workgroups (exact chunks) per query head
constexpr int kBufDword3 = 0x00020000;  // buffer resource word 3 for gfx9-family raw loads
constexpr int kMaxWin = 1024;       // largest window (recent tokens read exactly)
constexpr int kWinW = 130;          // window sums per query head: N[128], D, Q

}  // namespace csa
