// Per-call constants and the GQA-shared 4-bit scan.
//
// "Certified Sparse Attention via Perturbed Retrieval": summary page, Methodology >
// Algorithm Components items 1 (window / pool split, Exp(1) perturbations from a
// 53-bit hash) and 4 (4-bit keys bound every score with certainty; candidates are
// grouped by the first level at which they could be sampled); authors' abstract (the
// scan is shared across a GQA group and reads every key once).
//
// Bound per pool key i and query g (all integers exact; fp64 in this order):
//   shat  = (base_gb + alpha_b I_gi) * RSQRT_D
//   slack = (((alpha_b/2 C_i + qnp_g kerr_i) + eb_gb) + pad_gb) * RSQRT_D
//   UB = shat + slack, LB = shat - slack, p = UB + E_i
// with I_gi = sum_t a~_gbt c_it and C_i = sum_t c_it from one i8 MFMA chain, and
// base_gb = beta_g kappa_b sum_t q~_gt z_bt from a second one.  The integer weights
// a~ = rint(q kscale 2^(11-x)) lie in [-2048, 2048]; each is split into two int8 rows of
// the MFMA's A operand, a~ = 256 a1 + a0 (a1 in [-8, 8], a0 in [-128, 127]).
//
// MFMA operand rows (16): query g's high part at row 4(g%4) + 2(g/4), its low part
// one row below; row 14 is all ones (gives C_i); row 15 is zero.  So G <= 7.
// Output row 4k+i lands in register i of lanes 16k..16k+15, column = lane % 16.
#include "common.h"

namespace csa {

__device__ inline int op_row(int g, int part) { return 4 * (g & 3) + 2 * (g >> 2) + part; }

__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------ scan
//
// The scan is two kernels.
//   scan_kernel (streaming; reads every packed key once): for each block of 32 keys
//     and query it keeps two fp32 numbers that are rigorous upper bounds of
//     max_i UB_i and of max_i (UB_i + E^_i) over the block's keys (E^_i >= E_i from the
//     hash's leading bits, no logarithm), and a rigorous lower bound of max_i LB_i that
//     raises c_lo's running value.  Nothing is written per key.
//   refine_kernel: once every block's maxima are known, c_lo and the pilot give tight
//     lower bounds of c_lo and c*.  A block can hold a key of C_max (UB >= c_lo) or a
//     key that is sampled at some level (UB + E >= c* + log tau_J) only if its maxima
//     pass the same tests; the exact fp64 bounds, the exact perturbations and the
//     per-key outputs are computed for those blocks only.
struct ScanArgs {
  const uint16_t *K;        // fp16 keys (exact scores of C_max candidates)
  const uint8_t *codes;
  const uint16_t *kscale;
  const int8_t *zq;
  const BlockMeta *bmeta;
  const uint16_t *kerr, *vnorm;
  int64_t n_cap, nb_cap, nb_pool, npool_cap, nwords, nbw;   // nb_pool: the longest item's
  int G, U, J, r;                                            // units (item KV heads)
  Batch b;
  const uint16_t *q;        // fp16 [units G][128]
  uint64_t seed[kMaxItems], step[kMaxItems];   // hash inputs per item
  int32_t layer[kMaxItems];
  // per-call constants, written by the window workgroups for the later kernels (the
  // streaming wavefronts derive their own from q)
  float *qf;
  double *qconst;
  int8_t *qA;
  uint64_t *prefix;
  double *lt, *tau;
  int *ccount, *exdone, *exdone2;   // per-head counters, cleared by the window workgroups
  // window work (extra workgroups of the streaming kernel, one per query head)
  const uint16_t *V;
  int W;
  int64_t nstream;          // workgroups of the streaming scan; the rest do window work
  double *sR;               // [H_q][W] window scores
  double *win;              // [H_q][kWinW]: sum_R e^(s - c_R) v, sum e^(s - c_R), sum e^(s - c_R) |v|^2
  float2 *bmax;             // [H_q][nbw]: per block, bounds of max UB and of max (UB + E)
  double *pbuf, *ubuf;
  uint32_t *live;
  unsigned long long *clo, *cstar;
  // per streaming wavefront (wph of them per KV head, row stride wstride): a lower bound
  // of the largest LB of its keys per query, and the largest |v| code of its keys; plain
  // stores, reduced by the consumers (same-address atomics from every wavefront would
  // serialize at the end of the scan)
  float *lbpart;            // [H_q][wstride]
  unsigned *vpart;          // [H_kv][wstride]
  int64_t wstride;
  int diag;                 // 1: every key is live and UB/LB/E are written for all keys
  double *lb_out, *e_out;   // diagnostics (may be null)
};

// Rigorous upper bound on E = -ln u with u = N 2^-53, N = (h >> 11) + 1, from N's
// exponent k and leading mantissa bits f: ln(1 + f) >= f ln 2 on [0, 1], so
// E <= (53 - k - f) ln 2.
__device__ inline double perturbation_upper(uint64_t prefix, int64_t pos) {
  const uint64_t N = (mix64(prefix ^ (uint64_t)pos) >> 11) + 1ull;
  const int k = 63 - __clzll((long long)N);
  const uint64_t top = (k >= 23) ? (N >> (k - 23)) : (N << (23 - k));   // in [2^23, 2^24)
  const double f = (double)(top - (1ull << 23)) * 0x1p-23;             // <= mantissa fraction
  const double x = (double)(53 - k) - f;
  return (x * 0.69314718055994539725) * (1.0 + 0x1p-40) + 0x1p-40;    // ln 2 rounded up
}

// fp32 bound that is >= perturbation_upper(): f is truncated to 16 bits (x grows and is
// exact in fp32), ln 2 is taken as its fp32 rounding (which lies above ln 2), and the
// relative and absolute pads exceed the fp64 ones plus every fp32 rounding.
__device__ inline float perturbation_upper32(uint64_t prefix, int64_t pos) {
  const uint64_t N = (mix64(prefix ^ (uint64_t)pos) >> 11) + 1ull;
  const int k = 63 - __clzll((long long)N);
  const uint32_t top = (uint32_t)((k >= 16) ? (N >> (k - 16)) : (N << (16 - k)));   // [2^16, 2^17)
  const float x = (float)(53 - k) - (float)(top - (1u << 16)) * 0x1p-16f;
  return (x * 0x1.62e430p-1f) * (1.0f + 0x1p-20f) + 0x1p-30f;
}

// Constant rows of the A operand: zero everything, then the ones row (14); with
// `every_group` (groups of at most four queries, which leave rows 4k + 2 and 4k + 3
// free) also rows 2, 6 and 10, so that every lane group of the result holds the code
// sums of its tokens.
__device__ inline void init_operand(uint8_t *Abuf, int lane, bool every_group = false) {
  uint4 *A4 = reinterpret_cast<uint4 *>(Abuf);
  A4[lane] = make_uint4(0, 0, 0, 0);
  A4[64 + lane] = make_uint4(0, 0, 0, 0);
  wave_sync();
  if ((lane & 15) == 14 || (every_group && (lane & 3) == 2)) {
    A4[lane] = make_uint4(0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u);
    A4[64 + lane] = make_uint4(0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u);
  }
  wave_sync();
}


// ------------------------------------------------------------------ query constants
// The exact constants, which the window workgroups compute and store for the later
// kernels (the streaming wavefronts use fp32 bounds of them, below).
// Per query (R1 sums: the 128 channels in 8 chunks of 16 summed in channel order, then
// the fixed tree ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7)); all fp64):
//   qa    = max_t |q_t|;  beta = 2^(e - 11) for qa = f 2^e, f in [1/2, 1) (0 for q = 0)
//   qabs  = R1-sum |q_t|;  qn = the fp32 square root of R1-sum q_t^2 (1 + 2^-40),
//   rounded up;  qnp = qn (1 + 2^-40)
//   the integer grid of the offset term: qi_t = rint(q_t / beta) = 128 q1_t + q0_t with
//   q1 = floor((qi + 64) / 128), q0 = qi - 128 q1, in operand rows op_row(g, 0 / 1).
struct QueryConsts {
  double qa, beta, qabs, qn, qnp;
  float ib;   // 1 / beta (a power of two, exact in fp32; 0 when beta = 0)
};

__device__ inline QueryConsts query_consts_from(double ss, double sa, double qa) {
  QueryConsts c;
  c.qa = qa;
  c.beta = 0.0;
  c.ib = 0.0f;
  if (qa > 0.0) {
    int e;
    (void)frexp(qa, &e);
    c.beta = ldexp(1.0, e - 11);
    c.ib = ldexpf(1.0f, 11 - e);
  }
  c.qabs = sa;
  const float qn = f32_sqrt_up(ss * (1.0 + kPadF));
  c.qn = (double)qn;
  c.qnp = (double)qn * (1.0 + kPadF);
  return c;
}

// Maximum over the 16 lanes of a row with integer DPP maxima on order-preserving keys.
__device__ inline int fkey(float v) {
  const int b = __float_as_int(v);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ inline float fkey_inv(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }
// Maxima over the 16 lanes of each row of two values at once: four DPP steps (swap
// neighbours, swap pairs, mirror half-rows, mirror rows), each a max with the moved
// value.  Every source lane lies in the row, so the masks are full and no lane keeps an
// old value; every lane must be active.  The nops give the two wait states a DPP read
// needs after a VALU write of its operand.
__device__ inline void row_max16x2(float &u, float &v) {
  __asm__("s_nop 1\n\t"
          "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_max_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "s_nop 1\n\t"
          "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
          "v_max_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
          "s_nop 1\n\t"
          "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
          "v_max_f32_dpp %1, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
          "s_nop 1\n\t"
          "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"
          "v_max_f32_dpp %1, %1, %1 row_mirror row_mask:0xf bank_mask:0xf"
          : "+v"(u), "+v"(v));
}
__device__ inline int row_max16key(int k) {
  k = max(k, __builtin_amdgcn_update_dpp(k, k, 0xB1, 0xF, 0xF, false));    // quad_perm 1032
  k = max(k, __builtin_amdgcn_update_dpp(k, k, 0x4E, 0xF, 0xF, false));    // quad_perm 2301
  k = max(k, __builtin_amdgcn_update_dpp(k, k, 0x141, 0xF, 0xF, false));   // row_half_mirror
  k = max(k, __builtin_amdgcn_update_dpp(k, k, 0x140, 0xF, 0xF, false));   // row_mirror
  return k;
}
__device__ inline float row_max16k(float v) { return fkey_inv(row_max16key(fkey(v))); }
// Maximum over the 64 lanes (every lane active), the same in every lane: the rows' maxima
// by DPP, then the four rows' from scalar reads.
__device__ inline float wave_max_f32(float v) {
  const int k = row_max16key(fkey(v));
  const int r0 = __builtin_amdgcn_readlane(k, 0), r1 = __builtin_amdgcn_readlane(k, 16);
  const int r2 = __builtin_amdgcn_readlane(k, 32), r3 = __builtin_amdgcn_readlane(k, 48);
  return fkey_inv(max(max(r0, r1), max(r2, r3)));
}
// Sum over the 16 lanes of each row, the same in all of them (every lane active): pairs,
// quads, half-rows, rows, each step adding the value of a lane in the other part.
__device__ inline float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// Lane l's value of v, as a wave-uniform value (the bits move, not a converted value).
__device__ inline float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Lanes of the streaming scan: lane l takes the query slots gA = l / 16 and gB = gA + 4
// (groups of five to seven queries), each with channels 8 o .. 8 o + 7, o = l % 16, so
// the 16 lanes of a slot are one DPP row.  op_octet gives the byte offset of those eight
// channels in operand row `row` (lane L = row + 16 kg holds the bytes of channels
// 32 kg + 16 kh + b, b = 0..15, in half kh of the operand).
__device__ inline int op_octet(int row, int o) {
  return ((o >> 1) & 1) * 1024 + (row + 16 * (o >> 2)) * 16 + 8 * (o & 1);
}

// One wavefront's constants of its G queries, for the streaming bounds only (q8A, q8B:
// the lane's eight channels of slots gA and gB, zero for slots past G).  They need not
// equal the exact constants that the window workgroups store for the later kernels, only
// bound them:
//   - max |q| is exact in fp32, so beta, 1 / beta and the integer grid q~ are the exact
//     ones, and so are the offset terms base and eb;
//   - the sum of squares is taken in fp32 (squares of fp16 values are exact in fp32; at
//     most 11 roundings on any path, so the true sum S is at most s (1 + 2^-20)), and
//     qnp32 = sqrt(s (1 + 2^-10)) (1 + 2^-10) in fp32 exceeds sqrt(S) (1 + 2^-11) with a
//     square root within one ulp, above the exact qnp, which is below sqrt(S) (1 + 2^-22);
//   - 128 max |q| stands in for sum |q| in the pad 2^-40 qabs Kmax.
// A larger qnp or pad only raises every upper bound and lowers every lower bound.  The
// lane gets the values of its slots (qnp, qabs, beta), the largest |q| of the group, and
// its slice of the offset term's A operand (qa0, qa1), built in A (2 KB of LDS): rows
// op_row(g, 0 / 1) hold q~ = 128 q1 + q0 with q1 = floor((q~ + 64) / 128).
template <int G>
__device__ inline void wave_query_consts8(const float *q8A, const float *q8B, int lane, uint8_t *A, float &qmax,
                                          float &qnpA, float &qnpB, double *obeta, double *oqabs, v4i &qa0,
                                          v4i &qa1) {
  constexpr bool kTwo = G > 4;
  const int gA = lane >> 4, gB = gA + 4, o = lane & 15;
  float mA = 0.0f, sA = 0.0f, mB = 0.0f, sB = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mA = fmaxf(mA, fabsf(q8A[i]));
    sA += q8A[i] * q8A[i];
    if (kTwo) {
      mB = fmaxf(mB, fabsf(q8B[i]));
      sB += q8B[i] * q8B[i];
    }
  }
  mA = row_max16k(mA);
  sA = row_sum16(sA);
  qmax = fmaxf(fmaxf(readlane_f32(mA, 0), readlane_f32(mA, 16)), fmaxf(readlane_f32(mA, 32), readlane_f32(mA, 48)));
  if (kTwo) {
    mB = row_max16k(mB);
    sB = row_sum16(sB);
    qmax = fmaxf(qmax, fmaxf(fmaxf(readlane_f32(mB, 0), readlane_f32(mB, 16)),
                             fmaxf(readlane_f32(mB, 32), readlane_f32(mB, 48))));
  }
  // the slot's constants and its rows of the offset operand (zero rows for empty slots)
  auto slot = [&](const float *q8, float m, float ss, bool valid, int g, double &beta, double &qabs, float &qnp) {
    beta = 0.0;
    qabs = 0.0;
    qnp = 0.0f;
    float ib = 0.0f;   // 0 for a zero query: its rows stay 0
    if (valid) {
      if (m > 0.0f) {
        int e;
        (void)frexpf(m, &e);
        beta = ldexp(1.0, e - 11);
        ib = ldexpf(1.0f, 11 - e);
      }
      qnp = __builtin_sqrtf(ss * 0x1.004p0f) * 0x1.004p0f;
      qabs = 128.0 * (double)m;
    }
    uint32_t hi[2] = {0u, 0u}, lo[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int qi = (int)rintf(q8[i] * ib);
      const int q1 = (qi + 64) >> 7;
      hi[i >> 2] |= (uint32_t)(q1 & 0xFF) << (8 * (i & 3));
      lo[i >> 2] |= (uint32_t)((qi - 128 * q1) & 0xFF) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2 *>(A + op_octet(op_row(g, 0), o)) = make_uint2(hi[0], hi[1]);
    *reinterpret_cast<uint2 *>(A + op_octet(op_row(g, 1), o)) = make_uint2(lo[0], lo[1]);
  };
  slot(q8A, mA, sA, gA < G, gA, obeta[0], oqabs[0], qnpA);
  slot(q8B, mB, sB, kTwo && gB < G, gB, obeta[1], oqabs[1], qnpB);
  wave_sync();
  qa0 = *reinterpret_cast<const v4i *>(A + lane * 16);
  qa1 = *reinterpret_cast<const v4i *>(A + 1024 + lane * 16);
  wave_sync();
}

// Offset term of up to 16 blocks (block = MFMA column): base = beta kappa sum_t q~ z,
// eb = (beta/2) kappa sum_t |z|, pad = (2^-40 qabs) Kmax, into cst[0..2][block][g].
// The packed data the offset terms of blocks col0 .. col0 + 15 read (lane = (block
// column n16, channel group)): zero-point rows and the block record.
struct OffsetIn {
  v4i z1k0, z1k1, z0k0, z0k1;
  BlockMeta bm;
};

__device__ inline void offset_load(const ScanArgs &a, int64_t kvh, int64_t blk0, int nblk, int lane, int col0,
                                   OffsetIn &in) {
  const int n16 = lane & 15, grp = lane >> 4;
  in.z1k0 = in.z1k1 = in.z0k0 = in.z0k1 = v4i{0, 0, 0, 0};
  in.bm = BlockMeta{};
  const int col = col0 + n16;
  if (col < nblk) {
    const int8_t *zb = a.zq + (kvh * a.nb_cap + blk0 + col) * 256;
    in.z1k0 = *reinterpret_cast<const v4i *>(zb + 32 * grp);
    in.z1k1 = *reinterpret_cast<const v4i *>(zb + 32 * grp + 16);
    in.z0k0 = *reinterpret_cast<const v4i *>(zb + 128 + 32 * grp);
    in.z0k1 = *reinterpret_cast<const v4i *>(zb + 128 + 32 * grp + 16);
    in.bm = a.bmeta[kvh * a.nb_cap + blk0 + col];
  }
}

// Offset term of up to 16 blocks (block = MFMA column): base = beta kappa sum_t q~ z,
// eb = (beta/2) kappa sum_t |z|, pad = (2^-40 qabs) Kmax, into cst[0..2][block][g].
// qa0/qa1: the group's operand rows; beta/qabs: the lane's two query slots' constants;
// store(col, g, base, eb, pad) keeps the three terms.
template <typename Store>
__device__ inline void offset_compute(const OffsetIn &in, v4i qa0, v4i qa1, const double *beta,
                                      const double *qabs, int nblk, int G, int lane, Store &&store, int col0) {
  const int n16 = lane & 15, grp = lane >> 4;
  v4i zero = {0, 0, 0, 0};
  v4i r1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa0, in.z1k0, zero, 0, 0, 0);
  r1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa1, in.z1k1, r1, 0, 0, 0);
  v4i r0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa0, in.z0k0, zero, 0, 0, 0);
  r0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa1, in.z0k1, r0, 0, 0, 0);
  const int col = col0 + n16;
  if (col < nblk) {
    const double kappa = ldexp(1.0, in.bm.kexp);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int g = grp + 4 * s;
      if (g < G) {
        // q~ z = 16384 q1 z1 + 128 (q1 z0 + q0 z1) + q0 z0
        const int hi1 = s ? r1[2] : r1[0], lo1 = s ? r1[3] : r1[1];
        const int hi0 = s ? r0[2] : r0[0], lo0 = s ? r0[3] : r0[1];
        const int bint = 16384 * hi1 + 128 * (hi0 + lo1) + lo0;
        store(col, g, (beta[s] * kappa) * (double)bint, ((beta[s] / 2.0) * kappa) * (double)in.bm.z1sum,
              (kPadF * qabs[s]) * (double)in.bm.kmax);
      }
    }
  }
  wave_sync();
}

// The lane's query-slot constants for the offset terms.
__device__ inline void offset_consts(const ScanArgs &a, int h, int G, int lane, double *beta, double *qabs) {
  const int grp = lane >> 4;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int g = grp + 4 * s;
    beta[s] = (g < G) ? a.qconst[(int64_t)(h * G + g) * kQc + QC_BETA] : 0.0;
    qabs[s] = (g < G) ? a.qconst[(int64_t)(h * G + g) * kQc + QC_QABS] : 0.0;
  }
}

template <int NB>
__device__ inline void offset_terms(const ScanArgs &a, int h, int64_t kvh, int64_t blk0, int nblk, int G, int lane,
                                   double (*cst)[NB][8], int col0 = 0) {
  const v4i qa0 = *reinterpret_cast<const v4i *>(a.qA + (int64_t)h * 2048 + lane * 16);
  const v4i qa1 = *reinterpret_cast<const v4i *>(a.qA + (int64_t)h * 2048 + 1024 + lane * 16);
  double beta[2], qabs[2];
  offset_consts(a, h, G, lane, beta, qabs);
  OffsetIn in;
  offset_load(a, kvh, blk0, nblk, lane, col0, in);
  offset_compute(
      in, qa0, qa1, beta, qabs, nblk, G, lane,
      [&](int col, int g, double base, double eb, double pad) {
        cst[0][col][g] = base;
        cst[1][col][g] = eb;
        cst[2][col][g] = pad;
      },
      col0);
}

// The group's integer weights of one block (lanes as for
// wave_query_consts8; kk: the eight channels' fp16 scales; alpha = 2^(x - 11), the
// block's grid step, or 0).  Here a~ = 256 a1 + a0 with a1 = floor((a~ + 128) / 256) in
// [-8, 8] and a0 in [-128, 127], both signed bytes, so that each row part of the lane's
// eight channels is one 8-byte store.  The rint is one fused multiply-add of q kscale
// (exact inside the FMA) and (1.5 2^23 + 128) alpha: the sum's spacing is alpha, so it
// rounds q kscale / alpha to the nearest integer, ties to even (128 is even), and its
// mantissa bits are 0x400000 + v with v = a~ + 128.  Byte 1 of them is floor(v / 256) =
// a1 (the 0x4000 above it has a zero low byte) and byte 0 is v mod 256 = a0 + 128, a0
// once its top bit is flipped.  With alpha = 0 (a zero query group or zero scales) every
// product is 0 and the constant is taken unscaled, so that every weight is 0.
template <int G>
__device__ inline void build_operand8(uint8_t *Abuf, const float *q8A, const float *q8B, uint4 kk, float alpha,
                                      int lane) {
  constexpr bool kTwo = G > 4;
  const int gA = lane >> 4, gB = gA + 4, o = lane & 15;
  const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
  float ks[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ks[2 * j] = h2f((uint16_t)(kw[j] & 0xFFFFu));
    ks[2 * j + 1] = h2f((uint16_t)(kw[j] >> 16));
  }
  constexpr float kMagic = 0x1.8p23f + 128.0f;
  const float magic = (alpha > 0.0f) ? kMagic * alpha : kMagic;
  auto one = [&](const float *q8, int g) {
    uint32_t t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = __float_as_uint(__builtin_fmaf(q8[i], ks[i], magic));
    uint32_t pr[4];   // channels 2j, 2j + 1: a1, a1, a0 + 128, a0 + 128
#pragma unroll
    for (int j = 0; j < 4; ++j) pr[j] = __builtin_amdgcn_perm(t[2 * j + 1], t[2 * j], 0x04000501u);
    const uint32_t hi0 = __builtin_amdgcn_perm(pr[1], pr[0], 0x05040100u);
    const uint32_t hi1 = __builtin_amdgcn_perm(pr[3], pr[2], 0x05040100u);
    const uint32_t lo0 = __builtin_amdgcn_perm(pr[1], pr[0], 0x07060302u) ^ 0x80808080u;
    const uint32_t lo1 = __builtin_amdgcn_perm(pr[3], pr[2], 0x07060302u) ^ 0x80808080u;
    *reinterpret_cast<uint2 *>(Abuf + op_octet(op_row(g, 0), o)) = make_uint2(hi0, hi1);
    *reinterpret_cast<uint2 *>(Abuf + op_octet(op_row(g, 1), o)) = make_uint2(lo0, lo1);
  };
  if (gA < G) one(q8A, gA);
  if (kTwo && gB < G) one(q8B, gB);
}

// Weight grid of one block: alpha = 2^(x - 11) with m = max_t |q_t| kscale_t = f 2^x.
__device__ inline void block_grid(float qmax, float ksmax, double &alpha, float &scale) {
  const float m = qmax * ksmax;
  alpha = 0.0;
  scale = 0.0f;
  if (m > 0.0f) {
    int x;
    (void)frexpf(m, &x);
    alpha = ldexp(1.0, x - 11);
    scale = ldexpf(1.0f, 11 - x);
  }
}

// The same grid step in fp32 (a power of two, so equal to the fp32 rounding of the fp64 one).
__device__ inline void block_grid32(float qmax, float ksmax, float &alpha, float &scale) {
  const float m = qmax * ksmax;
  alpha = 0.0f;
  scale = 0.0f;
  if (m > 0.0f) {
    int x;
    (void)frexpf(m, &x);
    alpha = ldexpf(1.0f, x - 11);
    scale = ldexpf(1.0f, 11 - x);
  }
}

// fp32 bounds of one (query, key): ub >= UB, lb <= LB, ube >= UB + E^.  The fp64
// bound rounds at most ~10 times with unit 2^-53 and this fp32 evaluation at most
// ~12 times with unit 2^-24, each relative to M = (|base| + |alpha I|) R + slack, so a
// pad of 2^-17 M (plus 2^-100 for subnormal results) covers both.
struct Bound32 {
  float ub, lb, ube;
};
__device__ inline Bound32 bound32(float base, float ebpad, float alpha, float halpha, float qnp, int I,
                                  int C, float kerr, float eup) {
  constexpr float R = 0x1.6a09e6p-4f;   // fp32 rounding of 2^-3.5
  const float aI = alpha * (float)I;     // exact: |I| < 2^22, alpha a power of two
  const float s = (base + aI) * R;
  const float sl = __builtin_fmaf(halpha, (float)C, __builtin_fmaf(qnp, kerr, ebpad)) * R;
  const float M = __builtin_fmaf(fabsf(base) + fabsf(aI), R, sl);
  const float d = __builtin_fmaf(M, 0x1p-17f, 0x1p-100f);
  Bound32 r;
  r.ub = (s + sl) + d;
  r.lb = (s - sl) - d;
  const float t = r.ub + eup;
  r.ube = __builtin_fmaf(fabsf(r.ub) + eup, 0x1p-20f, t);
  return r;
}

constexpr int kPilot = 128;   // pool keys scored exactly up front (a lower bound on c*)
constexpr int kScanBufs = 3;     // streaming scan: chunk buffers (chunks in flight + 1)

// Shared memory of the streaming kernel; its window workgroups reuse it.
struct StreamSmem {
  alignas(16) uint8_t Abuf[4][2][2 * 1024];   // per wavefront, one operand per block of a chunk
  alignas(16) float ep[4][64];                 // per wavefront, E^ of the chunk's keys by (n16, tile)
  alignas(16) float ek[4][64];                 // per wavefront, key-error bounds of the chunk's keys, same order
  float2 cst[4][kScanBlocks][8];                // per block and query: fp32 base, eb + pad
  float2 mx[4][kScanBlocks][8];
};
struct WindowSmem {
  double sw[kMaxWin], vsq[kMaxWin];
  double red[2][4];
  double qd[kD];       // the query (fp64)
  double part[16];     // its R1 chunk sums of q^2 and |q|
  double smax[2];
};
union ScanSmem {
  StreamSmem st;
  WindowSmem win;
};

// Window work of query head hq (256 threads): exact window scores and c_R, a strided
// sample of the pool scored exactly (a lower bound on c*), and the window's sums
// relative to c_R, which the certificate rescales to c*.  All tokens are the window
// when n <= window.  Scores are wavefront-cooperative: 8 keys per wavefront step.  The
// workgroup shares the GPU with the streaming scan, so its reads are issued in few
// batches: the V columns of the first window rows up front, and the key rows of three
// steps at a time (more would raise the kernel's register count).
constexpr int kWinVPre = 64;   // window rows whose V columns are read up front
constexpr int kWinGrp = 3;     // wavefront steps whose rows are read together
__device__ void window_work(const ScanArgs &a, int hq, WindowSmem &sm) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int s8 = lane >> 3, k8 = lane & 7;
  const int h = hq / a.G, g = hq % a.G;                     // the unit and the query in it
  const int64_t kvh = unit_kv(a.b, h), nU = unit_n(a.b, h);  // its cache head and length
  // the call's constants of this query, stored for the later kernels (thread t < 128
  // owns channel t): level table (first query head), hash prefix (first query of a
  // unit), qf, the query constants, its rows of the offset term's A operand; and the
  // per-head counters cleared
  {
    if (hq == 0 && t <= a.J) {
      const double v = (-(double)t * kLn2) / (double)a.r;
      a.lt[t] = v;
      a.tau[t] = exp(v);
    }
    if (g == 0 && t == 0) {
      const int it = (a.U == a.b.H_kv) ? 0 : h / a.b.H_kv;
      a.prefix[h] = hash_prefix(a.seed[it], a.step[it], (uint64_t)(int64_t)a.layer[it], (uint64_t)(h % a.b.H_kv));
    }
    if (t == 0) {
      a.ccount[hq] = 0;
      a.exdone[hq] = 0;
      a.exdone2[hq] = 0;
    }
    const double qv = (t < kD) ? h2d(a.q[(int64_t)hq * kD + t]) : 0.0;
    if (t < kD) {
      a.qf[(int64_t)hq * kD + t] = (float)qv;
      sm.qd[t] = qv;
    }
    __syncthreads();
    // R1 chunk sums: threads 0..7 those of q^2, threads 8..15 those of |q|
    if (t < 16) {
      const int p = t & 7;
      double acc = (t < 8) ? sm.qd[16 * p] * sm.qd[16 * p] : fabs(sm.qd[16 * p]);
      for (int c = 1; c < 16; ++c)
        acc = acc + ((t < 8) ? sm.qd[16 * p + c] * sm.qd[16 * p + c] : fabs(sm.qd[16 * p + c]));
      sm.part[t] = acc;
    }
    double qa = fabs(qv);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qa = fmax(qa, __shfl_xor(qa, off, 64));
    if (lane == 0 && wv < 2) sm.smax[wv] = qa;
    __syncthreads();
    qa = fmax(sm.smax[0], sm.smax[1]);
    const double ss = ((sm.part[0] + sm.part[1]) + (sm.part[2] + sm.part[3])) +
                      ((sm.part[4] + sm.part[5]) + (sm.part[6] + sm.part[7]));
    const double sa = ((sm.part[8] + sm.part[9]) + (sm.part[10] + sm.part[11])) +
                      ((sm.part[12] + sm.part[13]) + (sm.part[14] + sm.part[15]));
    const QueryConsts c = query_consts_from(ss, sa, qa);
    if (t == 0) {
      double *qc = a.qconst + (int64_t)hq * kQc;
      qc[QC_BETA] = c.beta;
      qc[QC_QNP] = c.qnp;
      qc[QC_QABS] = c.qabs;
      qc[QC_QA] = c.qa;
      qc[QC_QN] = c.qn;
    }
    if (t < kD) {
      const int qi = (c.beta > 0.0) ? (int)rint(qv / c.beta) : 0;   // exact scaling
      const int q1 = (qi + 64) >> 7;
      const int q0 = qi - 128 * q1;
      const int kg = t >> 5, kh = (t >> 4) & 1, b = t & 15;
      int8_t *A = a.qA + (int64_t)h * 2048;
      A[kh * 1024 + (op_row(g, 0) + 16 * kg) * 16 + b] = (int8_t)q1;
      A[kh * 1024 + (op_row(g, 1) + 16 * kg) * 16 + b] = (int8_t)q0;
      if (g == 0)   // the rows of unused query slots
        for (int gs = a.G; gs < 8; ++gs) {
          A[kh * 1024 + (op_row(gs, 0) + 16 * kg) * 16 + b] = 0;
          A[kh * 1024 + (op_row(gs, 1) + 16 * kg) * 16 + b] = 0;
        }
    }
  }
  const int64_t w0 = (nU > a.W) ? (nU - a.W) : 0;
  const int nw = (int)(nU - w0);
  const int64_t stride = (w0 + kPilot - 1) / kPilot;
  const int npilot = (w0 > 0) ? kPilot : 0;
  const bool vcols = (t < kD) && a.V != nullptr && nw > 0;
  const uint16_t *vcol = vcols ? a.V + (kvh * a.n_cap + w0) * kD + t : nullptr;
  typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));
  ushort2v vpre[kWinVPre / 2];   // two rows per register (half-register loads)
  if (vcols) {
#pragma unroll
    for (int i = 0; i < kWinVPre / 2; ++i) {
      vpre[i].x = vcol[(int64_t)min(2 * i, nw - 1) * kD];
      vpre[i].y = vcol[(int64_t)min(2 * i + 1, nw - 1) * kD];
    }
  }
  double q16[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) q16[i] = sm.qd[16 * k8 + i];
  const uint16_t *Kh = a.K + kvh * a.n_cap * kD;
  const uint16_t *Vh = a.V ? a.V + kvh * a.n_cap * kD : nullptr;
  double m = -__builtin_huge_val(), mp = -__builtin_huge_val();
  for (int g0 = 0; g0 < nw + npilot; g0 += 32 * kWinGrp) {
    int64_t pos[kWinGrp];
    uint4 kw[kWinGrp][2], vw[kWinGrp][2];
#pragma unroll
    for (int j = 0; j < kWinGrp; ++j) {
      const int e = g0 + 32 * j + 8 * wv + s8;             // the key of this lane's group
      pos[j] = -1;
      if (e < nw) pos[j] = w0 + e;
      else if (e < nw + npilot && (int64_t)(e - nw) * stride < w0) pos[j] = (int64_t)(e - nw) * stride;
      const int64_t row = (pos[j] >= 0) ? pos[j] : 0;       // rows read by keys past the end: unused
      const uint4 *ks = reinterpret_cast<const uint4 *>(Kh + row * kD) + 2 * k8;
      kw[j][0] = ks[0];
      kw[j][1] = ks[1];
      if (Vh != nullptr && e < nw) {
        const uint4 *vs = reinterpret_cast<const uint4 *>(Vh + row * kD) + 2 * k8;
        vw[j][0] = vs[0];
        vw[j][1] = vs[1];
      } else {
        vw[j][0] = vw[j][1] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < kWinGrp; ++j) {
      const int e = g0 + 32 * j + 8 * wv + s8;
      const double p = (pos[j] >= 0) ? score_words(q16, kw[j][0], kw[j][1]) : 0.0;
      const double v = (pos[j] >= 0 && e < nw && Vh != nullptr) ? sumsq_words(vw[j][0], vw[j][1]) : 0.0;
      const double sc = r1_combine8(p) * kRsqrtD;
      const double vs = r1_combine8(v);
      if (pos[j] >= 0 && k8 == 0) {
        if (e < nw) {
          a.sR[(int64_t)hq * a.W + e] = sc;
          sm.sw[e] = sc;
          sm.vsq[e] = vs;
          m = fmax(m, sc);
        } else {
          mp = fmax(mp, sc);
        }
      }
    }
  }
  m = wave_max_f64(m);
  mp = wave_max_f64(mp);
  if (lane == 0) { sm.red[0][wv] = m; sm.red[1][wv] = mp; }
  __syncthreads();
  const double cr = fmax(fmax(sm.red[0][0], sm.red[0][1]), fmax(sm.red[0][2], sm.red[0][3]));
  const double pilot = fmax(cr, fmax(fmax(sm.red[1][0], sm.red[1][1]), fmax(sm.red[1][2], sm.red[1][3])));
  for (int i = t; i < nw; i += 256) sm.sw[i] = exp(sm.sw[i] - cr);
  __syncthreads();
  double *out = a.win + (int64_t)hq * kWinW;
  if (t < kD) {
    if (a.V) {
      double acc = 0.0;
      int i = 0;
      if (vcols) {
#pragma unroll
        for (int k = 0; k < kWinVPre; ++k)
          if (k < nw) acc += sm.sw[k] * h2d((k & 1) ? vpre[k >> 1].y : vpre[k >> 1].x);
        i = min(nw, kWinVPre);
      }
      for (; i + 8 <= nw; i += 8) {
        uint16_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = vcol[(int64_t)(i + k) * kD];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += sm.sw[i + k] * h2d(v[k]);
      }
      for (; i < nw; ++i) acc += sm.sw[i] * h2d(vcol[(int64_t)i * kD]);
      out[t] = acc;
    }
  } else if (t == kD) {
    double d = 0.0;
    for (int i = 0; i < nw; ++i) d += sm.sw[i];
    out[kD] = d;
  } else if (t == kD + 1) {
    double q = 0.0;
    for (int i = 0; i < nw; ++i) q += sm.sw[i] * sm.vsq[i];
    out[kD + 1] = q;
  } else if (t == kD + 2) {
    double *qc = a.qconst + (int64_t)hq * kQc;
    qc[QC_CR] = cr;
    qc[QC_PILOT] = pilot;
    // c_lo and c* start at c_R (nothing else writes them during the scan)
    a.clo[hq] = enc_max(cr);
    a.cstar[hq] = enc_max(cr);
  }
}


template <int G>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  __shared__ ScanSmem sm;
  if ((int64_t)blockIdx.x >= a.nstream) {
    window_work(a, (int)((int64_t)blockIdx.x - a.nstream), sm.win);
    return;
  }
  constexpr bool kTwo = G > 4;
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int64_t wph = (a.nb_pool + kScanBlocks - 1) / kScanBlocks;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wv;
  if (gw >= (int64_t)a.U * wph) return;
  const int h = (int)(gw / wph);                         // the unit
  const int64_t kvh = unit_kv(a.b, h);                   // its cache head
  const int64_t npool = unit_npool(a.b, h, a.W);
  const int64_t blk0 = (gw % wph) * kScanBlocks;
  if (blk0 * kBlk >= npool) return;                      // past this unit's pool
  const int nblk = (int)min((int64_t)kScanBlocks, (npool + kBlk - 1) / kBlk - blk0);
  const int n16 = lane & 15, grp = lane >> 4;
  uint8_t *Abuf = sm.st.Abuf[wv][0];
  uint8_t *Abuf1 = sm.st.Abuf[wv][1];
  float2(*cst)[8] = sm.st.cst[wv];
  auto keep_offsets = [&](int col, int g, double base, double eb, double pad) {
    cst[col][g] = make_float2((float)base, (float)(eb + pad));
  };
  float2(*mx)[8] = sm.st.mx[wv];
  float *ep = sm.st.ep[wv];
  float *ek = sm.st.ek[wv];

  const int gA = grp, gB = grp + 4;
  const bool hasA = gA < G, hasB = kTwo && gB < G;
  const int hq0 = h * G;
  // the group's queries (fp16 -> fp32, exact): the lane's eight channels of slots gA and
  // gB (read at clamped rows, zero for slots past G)
  float q8A[8], q8B[8];
  {
    const int o = lane & 15;
    const uint4 wa = *reinterpret_cast<const uint4 *>(a.q + (int64_t)(hq0 + min(gA, G - 1)) * kD + 8 * o);
    const uint4 wb = *reinterpret_cast<const uint4 *>(a.q + (int64_t)(hq0 + min(gB, G - 1)) * kD + 8 * o);
    const uint32_t ua[4] = {wa.x, wa.y, wa.z, wa.w}, ub[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q8A[2 * j] = hasA ? h2f((uint16_t)(ua[j] & 0xFFFFu)) : 0.0f;
      q8A[2 * j + 1] = hasA ? h2f((uint16_t)(ua[j] >> 16)) : 0.0f;
      q8B[2 * j] = hasB ? h2f((uint16_t)(ub[j] & 0xFFFFu)) : 0.0f;
      q8B[2 * j + 1] = hasB ? h2f((uint16_t)(ub[j] >> 16)) : 0.0f;
    }
  }

  // Software pipeline: the loads of chunks c + 1 .. c + kScanBufs - 1 (two blocks each)
  // are in flight while chunk c is computed.  The loads are unconditional and the loop
  // issues no global stores or atomics, so the compiler can wait for the older loads only.
  struct ChunkIn {
    uint4 cw[4];
    uint4 kk[2];        // the lane's eight channels' scales of both blocks
    float ksmax[2];
    uint16_t kerr;      // key-error code of the chunk's key `lane`
    uint16_t vn;
  };
  // Buffer resources over this wave's blocks only.  The chunk offset goes into the
  // per-lane offset, which the hardware range checks (the scalar offset is not), so the
  // reads of chunks past the wave's blocks or the pool return 0 and touch no memory.
  const int64_t tokw = min((int64_t)nblk * kBlk, npool - blk0 * kBlk);
  const __amdgpu_buffer_rsrc_t rs_codes = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.codes + (kvh * a.nb_cap + blk0) * 2048), (short)0, nblk * 2048, kBufDword3);
  const __amdgpu_buffer_rsrc_t rs_ks = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.kscale + (kvh * a.nb_cap + blk0) * kD), (short)0, nblk * 2 * kD, kBufDword3);
  const __amdgpu_buffer_rsrc_t rs_bm = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.bmeta + kvh * a.nb_cap + blk0), (short)0, nblk * (int)sizeof(BlockMeta), kBufDword3);
  const __amdgpu_buffer_rsrc_t rs_kerr = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.kerr + kvh * a.n_cap + blk0 * kBlk), (short)0, (int)tokw * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t rs_vn = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.vnorm + kvh * a.n_cap + blk0 * kBlk), (short)0, (int)tokw * 2, kBufDword3);
  auto load_chunk = [&](int c0, ChunkIn &in) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const int oc = c0 * 2048 + lane * 16, ok = c0 * 2 * kD + (lane & 15) * 16, om = c0 * (int)sizeof(BlockMeta);
    const int ov = c0 * kBlk * 2 + lane * 2;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs_codes, oc + T * 1024, 0, 0);
      in.cw[T] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const v4u k4 = __builtin_amdgcn_raw_buffer_load_b128(rs_ks, ok + bi * 2 * kD, 0, 0);
      in.kk[bi] = make_uint4(k4.x, k4.y, k4.z, k4.w);
      in.ksmax[bi] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_bm, om + bi * (int)sizeof(BlockMeta), 0, 0));
    }
    in.kerr = __builtin_amdgcn_raw_buffer_load_b16(rs_kerr, ov, 0, 0);
    in.vn = __builtin_amdgcn_raw_buffer_load_b16(rs_vn, ov, 0, 0);
  };

  // The offset terms of blocks 0..15 are formed before the stream starts and those of
  // blocks 16..31 during its first chunks; the loads of the first half and of the first
  // chunks are in flight together before the first wait, those of the second half are
  // issued once the first chunk is done.
  static_assert(kScanBlocks == 16 || kScanBlocks == 32, "offset terms are formed 16 blocks at a time");
  OffsetIn off0, off1;
  offset_load(a, kvh, blk0, nblk, lane, 0, off0);
  ChunkIn buf[kScanBufs];
#pragma unroll
  for (int k = 0; k + 1 < kScanBufs; ++k) load_chunk(2 * k, buf[k]);
  // the query constants, while the first loads are in flight (staged in the first
  // operand buffer, which is set up afterwards)
  v4i qa0, qa1;
  float qnpA, qnpB, qmax;
  double obeta[2], oqabs[2];
  wave_query_consts8<G>(q8A, q8B, lane, Abuf, qmax, qnpA, qnpB, obeta, oqabs, qa0, qa1);
  init_operand(Abuf, lane, !kTwo);
  init_operand(Abuf1, lane, !kTwo);
  offset_compute(off0, qa0, qa1, obeta, oqabs, nblk, G, lane, keep_offsets, 0);

  const int item = (a.U == a.b.H_kv) ? 0 : h / a.b.H_kv;
  const uint64_t prefix =
      hash_prefix(a.seed[item], a.step[item], (uint64_t)(int64_t)a.layer[item], (uint64_t)(h % a.b.H_kv));
  float lbA = -__builtin_huge_valf(), lbB = -__builtin_huge_valf();
  unsigned vmx = 0u;
  constexpr float kNegInf = -__builtin_huge_valf();

  // Staging a chunk: E^ of the lane's key (hash_chunk), then E^ into ep and both blocks'
  // operands into Abuf, Abuf1 (stage); al gets each block's fp32 grid step.
  auto hash_chunk = [&](const int c0, const ChunkIn &in) {
    const int nb2 = min(2, nblk - c0);
    const int64_t tok0 = (blk0 + c0) * kBlk;
    const int nval = (int)min((int64_t)(32 * nb2), npool - tok0);
    float myEup = 0.0f;
    if (lane < nval) {
      myEup = perturbation_upper32(prefix, tok0 + lane);
      vmx = max(vmx, (unsigned)in.vn);
    }
    return myEup;
  };
  auto stage = [&](const int c0, const ChunkIn &in, float myEup, float *al) {
    const int nb2 = min(2, nblk - c0);
    // key 16 T + n goes to ep[4 n + T]: a lane reads its token's four tiles at once
    ep[4 * (lane & 15) + (lane >> 4)] = myEup;
    ek[4 * (lane & 15) + (lane >> 4)] = h2f(in.kerr);
    float scales[2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) block_grid32(qmax, in.ksmax[bi], al[bi], scales[bi]);
    build_operand8<G>(Abuf, q8A, q8B, in.kk[0], al[0], lane);
    if (nb2 > 1) build_operand8<G>(Abuf1, q8A, q8B, in.kk[1], al[1], lane);
  };
  // process(c0, cur, nxt): bounds of the chunk staged before, with the next chunk hashed
  // while the operand reads are in flight and staged while the products run.  The
  // wavefront's LDS operations run in order, so the reads see the staged chunk and the
  // next chunk's writes leave them be; the syncs only keep the compiler from moving LDS
  // accesses (and the writes before the products) across them.
  auto process = [&](const int c0, const ChunkIn &cur, const ChunkIn &nxt, const float *alpha32s, float *alnext) {
    const int nb2 = min(2, nblk - c0);
    const int nval = (int)min((int64_t)(32 * nb2), npool - (blk0 + c0) * kBlk);
    wave_sync();
    float2 cA[2], cB[2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      cA[bi] = hasA ? cst[c0 + bi][gA] : make_float2(0.0f, 0.0f);
      cB[bi] = hasB ? cst[c0 + bi][gB] : make_float2(0.0f, 0.0f);
    }
    v4i Aop[2][2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const uint8_t *Ab = bi ? Abuf1 : Abuf;
      Aop[bi][0] = *reinterpret_cast<const v4i *>(Ab + lane * 16);
      Aop[bi][1] = *reinterpret_cast<const v4i *>(Ab + 1024 + lane * 16);
    }
    const float4 eup4 = *reinterpret_cast<const float4 *>(ep + 4 * n16);
    const float4 kerr4 = *reinterpret_cast<const float4 *>(ek + 4 * n16);
    wave_sync();
    const bool more = c0 + 2 < nblk;
    const float eupN = more ? hash_chunk(c0 + 2, nxt) : 0.0f;
    // all four tiles' products first, so that the matrix operations overlap
    v4i accs[4];
#pragma unroll
    for (int Tg = 0; Tg < 4; ++Tg) {
      const uint4 w = cur.cw[Tg];
      v4i lo = {(int)(w.x & 0x0F0F0F0Fu), (int)(w.y & 0x0F0F0F0Fu), (int)(w.z & 0x0F0F0F0Fu),
                (int)(w.w & 0x0F0F0F0Fu)};
      v4i hi = {(int)((w.x >> 4) & 0x0F0F0F0Fu), (int)((w.y >> 4) & 0x0F0F0F0Fu),
                (int)((w.z >> 4) & 0x0F0F0F0Fu), (int)((w.w >> 4) & 0x0F0F0F0Fu)};
      v4i acc = {0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aop[Tg >> 1][0], lo, acc, 0, 0, 0);
      accs[Tg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aop[Tg >> 1][1], hi, acc, 0, 0, 0);
    }
    wave_sync();
    if (more) stage(c0 + 2, nxt, eupN, alnext);
    // (chunks with all 64 keys in the pool, all but the last of a wavefront or pool, take
    // the copy without the per-key masks)
    auto bounds = [&](auto kFull) __attribute__((always_inline)) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      if (bi >= nb2) break;
      const int bl = c0 + bi;
      const float alpha32 = alpha32s[bi], halpha32 = 0.5f * alpha32s[bi];
      const float baseA = cA[bi].x, ebpA = cA[bi].y, baseB = cB[bi].x, ebpB = cB[bi].y;
      float uA = kNegInf, eA = kNegInf, uB = kNegInf, eB = kNegInf;
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        const int Tg = 2 * bi + T;
        const v4i acc = accs[Tg];
        const int tt = 16 * Tg + n16;            // token within chunk
        // code sums: every lane group's own ones row for groups of up to four queries
        const int Csum = kTwo ? bperm_i32(48 + n16, acc[2]) : acc[2];
        const float eup = Tg == 0 ? eup4.x : (Tg == 1 ? eup4.y : (Tg == 2 ? eup4.z : eup4.w));
        const float kerr = Tg == 0 ? kerr4.x : (Tg == 1 ? kerr4.y : (Tg == 2 ? kerr4.z : kerr4.w));
        const bool valid = decltype(kFull)::value || tt < nval;
        if (hasA) {
          const Bound32 r = bound32(baseA, ebpA, alpha32, halpha32, qnpA, acc[0] * 256 + acc[1], Csum, kerr, eup);
          uA = T ? fmaxf(uA, valid ? r.ub : kNegInf) : (valid ? r.ub : kNegInf);
          eA = T ? fmaxf(eA, valid ? r.ube : kNegInf) : (valid ? r.ube : kNegInf);
          lbA = fmaxf(lbA, valid ? r.lb : kNegInf);
        }
        if (hasB) {
          const Bound32 r = bound32(baseB, ebpB, alpha32, halpha32, qnpB, acc[2] * 256 + acc[3], Csum, kerr, eup);
          uB = T ? fmaxf(uB, valid ? r.ub : kNegInf) : (valid ? r.ub : kNegInf);
          eB = T ? fmaxf(eB, valid ? r.ube : kNegInf) : (valid ? r.ube : kNegInf);
          lbB = fmaxf(lbB, valid ? r.lb : kNegInf);
        }
      }
      row_max16x2(uA, eA);
      if (kTwo) row_max16x2(uB, eB);
      if (n16 == 0) {
        if (hasA) mx[bl][gA] = make_float2(uA, eA);
        if (hasB) mx[bl][gB] = make_float2(uB, eB);
      }
    }
    };
    if (nval == 64) bounds(std::true_type{});
    else bounds(std::false_type{});
  };
  // kScanBufs - 1 chunks in flight ahead of the one being computed, which has been staged
  float alCur[2], alNext[2];
  stage(0, buf[0], hash_chunk(0, buf[0]), alCur);
  for (int c0 = 0; c0 < nblk; c0 += 2 * kScanBufs) {
#pragma unroll
    for (int k = 0; k < kScanBufs; ++k) {
      const int c = c0 + 2 * k;
      if (c >= nblk) break;
      if (kScanBlocks > 16 && c == 8) offset_compute(off1, qa0, qa1, obeta, oqabs, nblk, G, lane, keep_offsets, 16);
      load_chunk(c + 2 * (kScanBufs - 1), buf[(k + kScanBufs - 1) % kScanBufs]);
      process(c, buf[k], buf[(k + 1) % kScanBufs], alCur, alNext);
      alCur[0] = alNext[0];
      alCur[1] = alNext[1];
      if (kScanBlocks > 16 && c == 0) offset_load(a, kvh, blk0, nblk, lane, 16, off1);
    }
  }
  wave_sync();
  // per-block maxima of the wave: [query][block] rows of float2
  for (int i = lane; i < G * kScanBlocks; i += 64) {
    const int g = i / kScanBlocks, bl = i % kScanBlocks;
    if (bl < nblk) a.bmax[(int64_t)(hq0 + g) * a.nbw + blk0 + bl] = mx[bl][g];
  }
  // c_lo >= every LB: publish the wave's lower bounds of max LB
  lbA = row_max16k(lbA);
  if (kTwo) lbB = row_max16k(lbB);
  const int64_t wih = gw % wph;   // this wavefront within its head
  if (n16 == 0) {
    if (hasA) a.lbpart[(int64_t)(hq0 + gA) * a.wstride + wih] = lbA;
    if (hasB) a.lbpart[(int64_t)(hq0 + gB) * a.wstride + wih] = lbB;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) vmx = max(vmx, (unsigned)__shfl_xor((int)vmx, off, 64));
  if (lane == 0) a.vpart[(int64_t)h * a.wstride + wih] = vmx;
}

// Everything one chunk (two blocks) of the refinement reads from the packed cache: its
// codes (four tiles), the key-error code of the lane's key and both blocks' scale maximum
// and channel scales of the lane's eight channels (8 (lane % 16) ..).
struct ChunkLoads {
  uint4 cw[4];
  uint32_t kerr;
  float ksmax[2];
  uint4 kk[2];
};

__device__ inline void load_chunk(const ScanArgs &a, int u, int64_t bA, int nb2, int lane, ChunkLoads &L) {
  const int64_t h = unit_kv(a.b, u);   // cache head of unit u
  const int64_t mypos = bA * kBlk + lane;
  L.kerr = (lane < 32 * nb2 && mypos < unit_npool(a.b, u, a.W)) ? (uint32_t)a.kerr[h * a.n_cap + mypos] : 0u;
#pragma unroll
  for (int T = 0; T < 4; ++T)
    L.cw[T] = (T < 2 * nb2)
                  ? reinterpret_cast<const uint4 *>(a.codes + (h * a.nb_cap + bA) * 2048)[T * 64 + lane]
                  : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    L.ksmax[bi] = (bi < nb2) ? a.bmeta[h * a.nb_cap + bA + bi].ksmax : 0.0f;
    L.kk[bi] = (bi < nb2) ? reinterpret_cast<const uint4 *>(a.kscale + (h * a.nb_cap + bA + bi) * kD)[lane & 15]
                          : make_uint4(0u, 0u, 0u, 0u);
  }
}

// Per wave slot: the KV head's values every wavefront of the workgroup needs when it takes
// one of the slot's chunks.
struct RefineSlot {
  float q[kMaxG][kD];              // the group's query values
  double clo[8], thr[8], qnp[8];   // c_lo snapshot, sampling threshold, |q| pad per query
  uint64_t prefix;
  float qmax;
};

__global__ __launch_bounds__(256) void refine_kernel(ScanArgs a) {
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  // wave slots of kBlocksPerWave blocks, interleaved over the KV heads: global slot s is
  // local slot s / H_kv of head s % H_kv, so one head's slots fall to different
  // workgroups and a head with many passing blocks shares them with the others' waves
  const int64_t wph = (a.nb_pool + kBlocksPerWave - 1) / kBlocksPerWave;
  const int64_t nslots = (int64_t)a.U * wph;
  auto slot_head = [&](int w) { return (int)(((int64_t)blockIdx.x * 4 + w) % a.U); };
  auto slot_blk0 = [&](int w) { return (((int64_t)blockIdx.x * 4 + w) / a.U) * kBlocksPerWave; };
  auto unit_blocks = [&](int u) { return (unit_npool(a.b, u, a.W) + kBlk - 1) / kBlk; };
  const int64_t gs = (int64_t)blockIdx.x * 4 + wv;
  const int h = slot_head(wv);
  const int64_t blk0 = slot_blk0(wv);
  const int G = a.G;
  const int n16 = lane & 15, grp = lane >> 4;

  __shared__ __attribute__((aligned(16))) uint8_t Abuf_all[4][2 * 1024];
  __shared__ double cst_all[4][3][kBlocksPerWave][8];
  __shared__ RefineSlot slot_all[4];
  __shared__ uint32_t wchunks[4];
  __shared__ uint8_t flag_all[4][64];
  __shared__ int ent_all[4][2 * 4 * 64];
  uint8_t *Abuf = Abuf_all[wv];
  uint8_t *flag = flag_all[wv];
  int *ent = ent_all[wv];
  RefineSlot &me = slot_all[wv];

  // this slot's values: one snapshot of c_lo's running value per query, shared by every
  // test of the slot's blocks; the block maxima are loaded together with it
  const int hq0 = h * G;
  const int gA = grp, gB = grp + 4;
  const bool hasA = gA < G, hasB = gB < G;
  // every load of the preamble is issued before the first use: the block maxima, the
  // queries, the per-query constants (lane g < G), the hash prefix and the scan
  // wavefronts' LB bounds (the first 128 wavefronts' of every query at once; a longer
  // pool adds a loop)
  // (block maxima at clamped positions, used below only for the slot's own blocks)
  // (read unconditionally at clamped rows, so that no load waits at a branch's end; the
  // rows of query slots past G are not used)
  const int64_t bcol = min<int64_t>(blk0 + n16, a.nbw - 1);
  const float2 mxA = a.bmax[(int64_t)(hq0 + min(gA, G - 1)) * a.nbw + bcol];
  const float2 mxB = a.bmax[(int64_t)(hq0 + min(gB, G - 1)) * a.nbw + bcol];
  const double ltJ = a.lt[a.J];
  float qv[kMaxG][2];
#pragma unroll
  for (int g = 0; g < kMaxG; ++g) {
    qv[g][0] = (g < G) ? a.qf[(int64_t)(hq0 + g) * kD + 2 * lane] : 0.0f;
    qv[g][1] = (g < G) ? a.qf[(int64_t)(hq0 + g) * kD + 2 * lane + 1] : 0.0f;
  }
  // (lane g < G takes query g; the other lanes read query G - 1's and drop the values)
  const int gq = min(lane, G - 1);
  const double *qc = a.qconst + (int64_t)(hq0 + gq) * kQc;
  const unsigned long long clo_r = __hip_atomic_load(a.clo + hq0 + gq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const double pilot_r = qc[QC_PILOT], qnp_r = qc[QC_QNP], qa_r = qc[QC_QA];
  const unsigned long long clo_enc = (lane < G) ? clo_r : 0ull;
  const double pilot = (lane < G) ? pilot_r : 0.0, qnp = (lane < G) ? qnp_r : 0.0, qa = (lane < G) ? qa_r : 0.0;
  const uint64_t prefix0 = a.prefix[h];
  const int64_t swph = (unit_blocks(h) + kScanBlocks - 1) / kScanBlocks;   // the unit's scan wavefronts
  float lbs[kMaxG][2];
#pragma unroll
  for (int g = 0; g < kMaxG; ++g)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t k = lane + 64 * i;   // (read within the row; entries past swph are masked below)
      lbs[g][i] = (g < G && k < a.wstride) ? a.lbpart[(int64_t)(hq0 + g) * a.wstride + k] : -__builtin_huge_valf();
    }
#pragma unroll
  for (int g = 0; g < kMaxG; ++g)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (lane + 64 * i >= swph) lbs[g][i] = -__builtin_huge_valf();
#pragma unroll
  for (int g = 0; g < kMaxG; ++g) {
    me.q[g][2 * lane] = qv[g][0];
    me.q[g][2 * lane + 1] = qv[g][1];
  }
  // c_lo snapshot per query: c_R (the window's atomic) and the scan wavefronts' bounds
#pragma unroll
  for (int g = 0; g < kMaxG; ++g) {
    if (g >= G) break;   // (G is the same for every lane)
    float v = fmaxf(lbs[g][0], lbs[g][1]);
    for (int64_t k = lane + 128; k < swph; k += 64) v = fmaxf(v, a.lbpart[(int64_t)(hq0 + g) * a.wstride + k]);
    lbs[g][0] = wave_max_f32(v);
  }
  // the slot's blocks (counted once the loads above are under way)
  const int nblk = (gs < nslots) ? (int)max<int64_t>(0, min<int64_t>(kBlocksPerWave, unit_blocks(h) - blk0)) : 0;
  // largest |q_t| over the group (lanes 0..7 hold the queries' values, 0 past G)
  float qm = (float)qa;
#pragma unroll
  for (int off = 4; off >= 1; off >>= 1) qm = fmaxf(qm, __shfl_xor(qm, off, 64));
  if (lane < 8) {
    double clo = 0.0, thr = 0.0;
    if (lane < G) {
      float lb = lbs[0][0];
#pragma unroll
      for (int g = 1; g < kMaxG; ++g) lb = (lane == g) ? lbs[g][0] : lb;
      clo = fmax(dec_max(clo_enc), (double)lb);
      thr = fmax(clo, pilot) + ltJ;
    }
    me.clo[lane] = clo;
    me.thr[lane] = thr;
    me.qnp[lane] = (lane < G) ? qnp : 0.0;
  }
  if (lane == 0) {
    me.qmax = qm;
    me.prefix = prefix0;
  }
  wave_sync();

  // blocks whose maxima pass a test (lane = (query slot, block))
  uint32_t alive = 0;
  if (a.diag) {
    alive = (nblk >= 32) ? 0xFFFFFFFFu : ((1u << nblk) - 1u);
  } else {
    bool pass = false;
    if (n16 < nblk) {
      if (hasA) {
        const double u = mxA.x, e = mxA.y, clo2 = me.clo[gA], thr = me.thr[gA];
        pass |= u >= clo2 - 0x1p-30 * (fabs(u) + fabs(clo2) + 1.0);
        pass |= e >= thr - 0x1p-30 * (fabs(e) + fabs(thr) + 1.0);
      }
      if (hasB) {
        const double u = mxB.x, e = mxB.y, clo2 = me.clo[gB], thr = me.thr[gB];
        pass |= u >= clo2 - 0x1p-30 * (fabs(u) + fabs(clo2) + 1.0);
        pass |= e >= thr - 0x1p-30 * (fabs(e) + fabs(thr) + 1.0);
      }
    }
    const unsigned long long b = __ballot(pass);
    alive = (uint32_t)((b | (b >> 16) | (b >> 32) | (b >> 48)) & 0xFFFFull);
  }
  // chunks (two blocks) with a block that passed
  uint32_t chunks = 0;
  for (int c = 0; 2 * c < nblk; ++c)
    if ((alive >> (2 * c)) & 3u) chunks |= 1u << c;
  if (lane == 0) wchunks[wv] = chunks;
  // the live words of blocks in chunks that are not processed (the processed ones are
  // written by their job): every pool block's word is written by this launch
  if (n16 < nblk && !((chunks >> (n16 >> 1)) & 1u)) {
    if (hasA) a.live[(int64_t)(hq0 + gA) * a.nwords + blk0 + n16] = 0u;
    if (hasB) a.live[(int64_t)(hq0 + gB) * a.nwords + blk0 + n16] = 0u;
  }
  __syncthreads();
  const uint32_t allm = wchunks[0] | (wchunks[1] << 8) | (wchunks[2] << 16) | (wchunks[3] << 24);
  if (allm == 0u) return;

  // the workgroup's chunks in order, the k-th to wavefront k mod 4 (job bit 8 w + c: chunk
  // c of slot w); each job's loads are issued while the previous job finishes, and
  // the first job's before the offset terms are formed
  uint32_t jobs = 0;
  {
    uint32_t m = allm;
    for (int k = 0; m; ++k) {
      const uint32_t bit = m & (0u - m);
      if ((k & 3) == wv) jobs |= bit;
      m ^= bit;
    }
  }
  auto job_blk = [&](int j) { return slot_blk0(j >> 3) + 2 * (j & 7); };
  auto job_nb2 = [&](int j) { return (int)min<int64_t>(2, unit_blocks(slot_head(j >> 3)) - job_blk(j)); };
  int cc = jobs ? __ffs((int)jobs) - 1 : -1;
  ChunkLoads cur, nxt;
  if (cc >= 0) load_chunk(a, slot_head(cc >> 3), job_blk(cc), job_nb2(cc), lane, cur);
  if (chunks) offset_terms(a, h, unit_kv(a.b, h), blk0, nblk, G, lane, cst_all[wv]);
  init_operand(Abuf, lane);
  __syncthreads();   // every slot's offset terms and values are in LDS

  while (cc >= 0) {
    jobs &= jobs - 1u;
    const int cn = jobs ? __ffs((int)jobs) - 1 : -1;
    // the job's slot: its head's values
    RefineSlot &S = slot_all[cc >> 3];
    const int jh = slot_head(cc >> 3), jhq0 = jh * G;   // the job's unit
    const int64_t jnpool = unit_npool(a.b, jh, a.W), jkv = unit_kv(a.b, jh);
    // the lane's eight channels of its query slots (as in the streaming scan)
    float q8A[8], q8B[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      q8A[i] = hasA ? S.q[gA][8 * (lane & 15) + i] : 0.0f;
      q8B[i] = hasB ? S.q[hasB ? gB : 0][8 * (lane & 15) + i] : 0.0f;
    }
    const float qmax = S.qmax;
    const uint64_t prefix = S.prefix;
    const double clo2A = hasA ? S.clo[gA] : 0.0, thrA = hasA ? S.thr[gA] : 0.0, qnpA = hasA ? S.qnp[gA] : 0.0;
    const double clo2B = hasB ? S.clo[gB] : 0.0, thrB = hasB ? S.thr[gB] : 0.0, qnpB = hasB ? S.qnp[gB] : 0.0;
    const int64_t rowA = (int64_t)(jhq0 + gA) * a.npool_cap, rowB = (int64_t)(jhq0 + gB) * a.npool_cap;
    double lbA = -__builtin_huge_val(), lbB = -__builtin_huge_val();
    double(*cst)[kBlocksPerWave][8] = cst_all[cc >> 3];
    const int c0 = 2 * (cc & 7);          // first block of the chunk within its slot
    const int64_t bA = job_blk(cc);
    const int nb2 = job_nb2(cc);
    const int64_t tok0 = bA * kBlk;
    const int64_t mypos = tok0 + lane;
    const bool mine = (lane < 32 * nb2) && (mypos < jnpool);
    double myEup = 0.0;
    if (mine) myEup = perturbation_upper(prefix, mypos);
    const uint32_t mykerr = cur.kerr;
    flag[lane] = 0;
    const uint4 *cw = cur.cw;
    double ubA[4], ubB[4];
    uint32_t liveA = 0, liveB = 0;     // bit Tg: the key of tile Tg is live for slot A / B
    uint32_t cmA = 0, cmB = 0;         // bit Tg: UB >= c_lo snapshot (C_max candidate)
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      if (bi >= nb2) break;
      const int64_t b = bA + bi;
      const int bl = c0 + bi;
      double alpha;
      float scale;
      block_grid(qmax, cur.ksmax[bi], alpha, scale);
      const double halpha = alpha / 2.0;
      const uint4 kk = cur.kk[bi];
      const float alpha32 = (float)alpha;   // a power of two (or 0): exact
      switch (G) {
        case 1: build_operand8<1>(Abuf, q8A, q8B, kk, alpha32, lane); break;
        case 2: build_operand8<2>(Abuf, q8A, q8B, kk, alpha32, lane); break;
        case 3: build_operand8<3>(Abuf, q8A, q8B, kk, alpha32, lane); break;
        case 4: build_operand8<4>(Abuf, q8A, q8B, kk, alpha32, lane); break;
        case 5: build_operand8<5>(Abuf, q8A, q8B, kk, alpha32, lane); break;
        case 6: build_operand8<6>(Abuf, q8A, q8B, kk, alpha32, lane); break;
        default: build_operand8<7>(Abuf, q8A, q8B, kk, alpha32, lane); break;
      }
      wave_sync();
      const v4i A0 = *reinterpret_cast<const v4i *>(Abuf + lane * 16);
      const v4i A1 = *reinterpret_cast<const v4i *>(Abuf + 1024 + lane * 16);
      wave_sync();
      const double baseA = hasA ? cst[0][bl][gA] : 0.0, ebA = hasA ? cst[1][bl][gA] : 0.0,
                   padA = hasA ? cst[2][bl][gA] : 0.0;
      const double baseB = hasB ? cst[0][bl][gB] : 0.0, ebB = hasB ? cst[1][bl][gB] : 0.0,
                   padB = hasB ? cst[2][bl][gB] : 0.0;
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        const int Tg = 2 * bi + T;
        const uint4 w = cw[Tg];
        v4i lo = {(int)(w.x & 0x0F0F0F0Fu), (int)(w.y & 0x0F0F0F0Fu), (int)(w.z & 0x0F0F0F0Fu),
                  (int)(w.w & 0x0F0F0F0Fu)};
        v4i hi = {(int)((w.x >> 4) & 0x0F0F0F0Fu), (int)((w.y >> 4) & 0x0F0F0F0Fu),
                  (int)((w.z >> 4) & 0x0F0F0F0Fu), (int)((w.w >> 4) & 0x0F0F0F0Fu)};
        v4i acc = {0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, lo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, hi, acc, 0, 0, 0);
        const int Csum = bperm_i32(48 + n16, acc[2]);
        const int tt = 16 * Tg + n16;            // token within chunk
        const int64_t pos = tok0 + tt;
        const double Eup = bperm_f64(tt, myEup);
        const double kerr = h2d((uint16_t)bperm_i32(tt, (int)mykerr));
        ubA[Tg] = 0.0;
        ubB[Tg] = 0.0;
        if (pos < jnpool) {
          if (hasA) {
            const int I = acc[0] * 256 + acc[1];
            const double shat = (baseA + alpha * (double)I) * kRsqrtD;
            const double slack = (((halpha * (double)Csum + qnpA * kerr) + ebA) + padA) * kRsqrtD;
            const double ub = shat + slack, lb = shat - slack;
            ubA[Tg] = ub;
            lbA = fmax(lbA, lb);
            if (a.lb_out) a.lb_out[(int64_t)(jhq0 + gA) * jnpool + pos] = lb;
            const double marg = 0x1p-40 * (fabs(ub) + fabs(thrA) + 1.0);
            if (ub >= clo2A - marg) cmA |= 1u << Tg;
            if (a.diag || ub + Eup >= thrA - marg || ub >= clo2A - marg) liveA |= 1u << Tg;
          }
          if (hasB) {
            const int I = acc[2] * 256 + acc[3];
            const double shat = (baseB + alpha * (double)I) * kRsqrtD;
            const double slack = (((halpha * (double)Csum + qnpB * kerr) + ebB) + padB) * kRsqrtD;
            const double ub = shat + slack, lb = shat - slack;
            ubB[Tg] = ub;
            lbB = fmax(lbB, lb);
            if (a.lb_out) a.lb_out[(int64_t)(jhq0 + gB) * jnpool + pos] = lb;
            const double marg = 0x1p-40 * (fabs(ub) + fabs(thrB) + 1.0);
            if (ub >= clo2B - marg) cmB |= 1u << Tg;
            if (a.diag || ub + Eup >= thrB - marg || ub >= clo2B - marg) liveB |= 1u << Tg;
          }
          if ((liveA | liveB) & (1u << Tg)) flag[tt] = 1;
        }
      }
    }
    // the next job's loads go out once this chunk's packed data has been used (vector
    // stores share the load counter, so loads issued before this job's stores would be
    // waited for together with them)
    if (cn >= 0) load_chunk(a, slot_head(cn >> 3), job_blk(cn), job_nb2(cn), lane, nxt);
    // exact perturbations of the chunk's live tokens (lane = token): formed while the first
    // C_max candidates' rows are on their way, or here if the chunk has none
    wave_sync();
    const bool needE = __ballot((liveA | liveB) != 0) != 0ull;
    const bool myLive = mine && flag[lane] != 0;
    double myE = 0.0;
    auto exact_E = [&]() __attribute__((always_inline)) {
      if (needE && myLive) {
        myE = perturbation(prefix, mypos);
        if (a.e_out) a.e_out[(int64_t)jh * jnpool + mypos] = myE;
      }
    };
    // exact scores of C_max candidates: c* = max(c_R, max over them), since a key with
    // UB < c_lo scores below c_lo <= c*.  Every candidate of the chunk (both slots, all
    // tiles) is listed in LDS first, then they are scored eight lanes per key.
    if (__ballot((cmA | cmB) != 0)) {
      int ne = 0;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
        for (int Tg = 0; Tg < 4; ++Tg) {
          const bool f = (((sl ? cmB : cmA) >> Tg) & 1u) != 0u;
          const unsigned long long mk = __ballot(f);
          if (f) {
            const int idx = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
            ent[ne + idx] = (16 * Tg + n16) | ((sl ? gB : gA) << 8);
          }
          ne += __popcll(mk);
        }
      }
      wave_sync();
      for (int e0 = 0; e0 < ne; e0 += 8) {
        const int e = e0 + (lane >> 3), k8 = lane & 7;
        int g2 = 0;
        int64_t pos = -1;
        if (e < ne) {
          const int v = ent[e];
          g2 = v >> 8;
          pos = tok0 + (v & 0xFF);
        }
        // the query chunk from the slot's LDS copy and the key chunk (position 0 for the
        // lanes past the list, dropped) are requested before anything waits for them
        const int64_t kpos = (pos >= 0) ? pos : 0;
        const uint4 *ksrc = reinterpret_cast<const uint4 *>(a.K + (jkv * a.n_cap + kpos) * kD) + 2 * k8;
        const uint4 kw0 = ksrc[0], kw1 = ksrc[1];
        if (e0 == 0) exact_E();
        double q16[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) q16[i] = (double)S.q[g2][16 * k8 + i];
        const double p = (pos >= 0) ? score_words(q16, kw0, kw1) : 0.0;
        const double sc = r1_combine8_first(p) * kRsqrtD;
        // c* = max(c_R, these exact scores)
        if (pos >= 0 && k8 == 0)
          __hip_atomic_fetch_max(a.cstar + jhq0 + g2, enc_max(sc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      wave_sync();
    } else {
      exact_E();
    }
    wave_sync();
#pragma unroll
    for (int Tg = 0; Tg < 4; ++Tg) {
      const int tt = 16 * Tg + n16;
      const int64_t pos = tok0 + tt;
      const bool la = (liveA >> Tg) & 1u, lbv = (liveB >> Tg) & 1u;
      const unsigned long long mA = __ballot(la), mB = __ballot(lbv);
      if (mA | mB) {
        const double E = bperm_f64(tt, myE);
        if (la) {
          a.pbuf[rowA + pos] = ubA[Tg] + E;
          a.ubuf[rowA + pos] = ubA[Tg];
        }
        if (lbv) {
          a.pbuf[rowB + pos] = ubB[Tg] + E;
          a.ubuf[rowB + pos] = ubB[Tg];
        }
      }
      // live bitmap: one 32-bit word per (query, block); tiles 2k and 2k+1 fill it
      if ((Tg & 1) == 1 && (Tg >> 1) < nb2) {
        const unsigned long long pA = __ballot((liveA >> (Tg - 1)) & 1u);
        const unsigned long long pB = __ballot((liveB >> (Tg - 1)) & 1u);
        const int64_t blk = bA + (Tg >> 1);
        if (n16 == 0) {
          if (hasA)
            a.live[(int64_t)(jhq0 + gA) * a.nwords + blk] =
                (uint32_t)((pA >> (16 * grp)) & 0xFFFFull) | ((uint32_t)((mA >> (16 * grp)) & 0xFFFFull) << 16);
          if (hasB)
            a.live[(int64_t)(jhq0 + gB) * a.nwords + blk] =
                (uint32_t)((pB >> (16 * grp)) & 0xFFFFull) | ((uint32_t)((mB >> (16 * grp)) & 0xFFFFull) << 16);
        }
      }
    }
    // exact c_lo: the processed blocks hold every key whose LB can exceed the snapshot
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      lbA = fmax(lbA, __shfl_xor(lbA, off, 64));
      lbB = fmax(lbB, __shfl_xor(lbB, off, 64));
    }
    if (n16 == 0) {
      if (hasA && lbA > clo2A)
        __hip_atomic_fetch_max(a.clo + jhq0 + gA, enc_max(lbA), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (hasB && lbB > clo2B)
        __hip_atomic_fetch_max(a.clo + jhq0 + gB, enc_max(lbB), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    cc = cn;
    if (cc >= 0) cur = nxt;
  }
}

// Streaming workgroups first, then one window workgroup per query head (a.nstream
// must be the number of streaming workgroups, 0 when the pool is empty).
int64_t scan_stream_wgs(int64_t H_kv, int64_t nb_pool) {
  const int64_t waves = H_kv * ((nb_pool + kScanBlocks - 1) / kScanBlocks);
  return (waves + 3) / 4;
}

// With events given, they take the kernel's own start and end times from its dispatch (no
// separate marker packets around it).
hipError_t launch_scan(const ScanArgs &a, hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
  const unsigned wgs = (unsigned)(a.nstream + (int64_t)a.U * a.G);
  switch (a.G) {
    case 1: hipExtLaunchKernelGGL(scan_kernel<1>, dim3(wgs), dim3(256), 0, st, ev0, ev1, 0, a); break;
    case 2: hipExtLaunchKernelGGL(scan_kernel<2>, dim3(wgs), dim3(256), 0, st, ev0, ev1, 0, a); break;
    case 3: hipExtLaunchKernelGGL(scan_kernel<3>, dim3(wgs), dim3(256), 0, st, ev0, ev1, 0, a); break;
    case 4: hipExtLaunchKernelGGL(scan_kernel<4>, dim3(wgs), dim3(256), 0, st, ev0, ev1, 0, a); break;
    case 5: hipExtLaunchKernelGGL(scan_kernel<5>, dim3(wgs), dim3(256), 0, st, ev0, ev1, 0, a); break;
    case 6: hipExtLaunchKernelGGL(scan_kernel<6>, dim3(wgs), dim3(256), 0, st, ev0, ev1, 0, a); break;
    default: hipExtLaunchKernelGGL(scan_kernel<7>, dim3(wgs), dim3(256), 0, st, ev0, ev1, 0, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_refine(const ScanArgs &a, hipStream_t st) {
  const int64_t wph = (a.nb_pool + kBlocksPerWave - 1) / kBlocksPerWave;
  const unsigned wgs = (unsigned)(((int64_t)a.U * wph + 3) / 4);
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(refine_kernel, dim3(wgs), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
