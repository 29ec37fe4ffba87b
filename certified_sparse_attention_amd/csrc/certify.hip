// Per-level Horvitz-Thompson sums, certificates, the per-head stop and the exact
// fallback.
//
// "Certified Sparse Attention via Perturbed Retrieval", summary page:
//   Methodology > Algorithm Components item 2: D^ = D_R + D_B + tau k,
//     N^ = N_R + N_B + tau sum_{S & A} v (heavy keys B with w >= tau are always in
//     the sample, light keys A enter with probability w / tau);
//   item 3: on the grid tau_j, a Chernoff interval for the number of light samples
//     (independent Bernoulli draws), a Bernstein-type bound for Hilbert-space vectors
//     on Z_c = sum_A (tau X - w)(v - c),
//     beta = (zeta + |o^ - c| dD) / (D^ - dD), stop at the first certified level;
//   Theorem 4: validity per head and per measure over all levels (union bound:
//     each level spends delta/(J+1), split over its one-sided tails);
//   Results > Certificate Validity: heads that certify nowhere fall back to exact
//     attention.
// Completion of the certificate (the pages give its shape, not its constants):
//   kl(x, mu) = mu - x + x ln(x/mu); mu_hi / mu_lo the roots above / below k of
//   kl(k, mu) = L; dD = tau max(k - mu_lo, mu_hi - k); c = N_det / D_det;
//   R_c = Vmax + |c|; y = (P - 2 c.V + k|c|^2)/R_c^2; mu_G the root above y;
//   sigma^2 = tau^2 R_c^2 mu_G; zeta = sqrt(2 sigma^2 L) + (2/3) tau R_c L;
//   value scale: mu_Q the root below P/Vmax^2, Q_lo = Q_det + tau Vmax^2 mu_Q,
//   M_lo = max(|o^| - beta_abs, sqrt(Q_lo / (D_det + tau mu_hi))).
#include "common.h"

namespace csa {

struct CertArgs {
  const uint16_t *K, *V;
  int64_t n_cap, npool_cap;
  int G, J, W, measure;
  double L;
  Batch b;                       // units: item KV heads (query head hq is in unit hq / G)
  double eps[kMaxItems];         // per item
  const float *qf;
  const double *lt, *tau, *sR;
  const double *win, *qconst;   // window sums relative to c_R; per-query constants (c_R)
  const unsigned long long *cstar, *clo;
  const double *ubuf;
  const unsigned *vpart;         // per scan wavefront: largest |v| code of its keys
  int64_t wstride;               // row stride of vpart (per unit)
  int *ccount, *candpos, *hist;  // (pass 1 writes the totals and the candidate list)
  int *rec_hl;                  // candidate records (written by the fused rescoring)
  int *cmhist;                  // [H_q][J+2] C_max keys per bucket level
  double *rec_w, *rec_vsq;
  const int8_t *lub;            // [H_q][npool_cap] l^ub of live keys (bucket count)
  const int *tilehist;          // [H_q][ntiles][J+2] per-tile cumulative level counts
  const int *tilecm;            // [H_q][ntiles][J+2] per-tile C_max keys per level
  const int *tilelist;          // [H_q][ntiles][kTileList] per-tile live keys in level order
  int64_t ntiles;               // row stride of the tile tables
  const uint32_t *live;         // [H_q][nwords] live keys (refinement)
  int64_t nwords;
  int budget, budget2;          // candidates of the first pass; of the first two (INT_MAX: all)
  int full_list;                // place every range even when pass 1 certifies (diagnostics)
  double *partial, *betalv, *dhatlv;
  int nseg_cap;                 // segment rows per query head in `partial` (seg_cap_for(npool))
  int *klv;
  int *flags;                   // [H_q] after pass 1: 0 certified, 1 exact fallback, 2 second pass
  int *flags2;                  // [H_q] after pass 2 (heads with flags 2): 0, 1, or 3 third pass
  int *exdone, *exdone2;        // [H_q] finished work items of the second / third-pass launch
  int *ccount1, *jspec;         // candidates with l^ub <= jspec come first in the list,
  int *ccount2, *jspec2;        // then those with jspec < l^ub <= jspec2, then the rest
  int H_q;
  int pass;                     // 1: levels <= jspec; 2: levels <= jspec2; 3: all levels
  const int8_t *codes8;         // the 8-bit refinement copy (csa.h)
  const float *scale8;
  const uint16_t *kerr8;
  int *rec_x;                   // per candidate: l8 | (UB >= c_lo) << 8
  int final_pass;               // the last tail launch (2 when jspec2 = J, else 3): it also
                                // takes the exact fallback
  const uint64_t *prefix;       // per KV head hash prefixes
  double *rec_s;
  double *exactp;
  float *o_hat;
  double *beta;
  int32_t *stop;
  int64_t *keys_read;
};

// Query head hq: its unit's cached length, cache head and item.
__device__ inline int64_t head_n(const CertArgs &a, int hq) { return unit_n(a.b, hq / a.G); }
__device__ inline int64_t head_kv(const CertArgs &a, int hq) { return unit_kv(a.b, hq / a.G); }
__device__ inline int head_item(const CertArgs &a, int hq) { return unit_item(a.b, hq / a.G); }

constexpr int kFusedMax = 2048;   // heads with more candidates use the segmented accumulation
constexpr int kStage = 64;        // candidates staged in LDS at a time

// Candidates this pass accumulates for query head hq (-1: the head is not in this pass).
// Pass p takes every candidate up to its deepest level: the ones earlier passes rescored
// from their records, the new ones rescored here.
__device__ inline int pass_count(const CertArgs &a, int hq) {
  if (a.pass == 1) return a.ccount1[hq];
  if (a.pass == 2) return (a.flags[hq] == 2) ? a.ccount2[hq] : -1;
  return (a.flags[hq] == 2 && a.flags2[hq] == 3) ? a.ccount[hq] : -1;
}
__device__ inline int pass_jmax(const CertArgs &a, int hq) {
  return (a.pass == 1) ? a.jspec[hq] : ((a.pass == 2) ? a.jspec2[hq] : a.J);
}
// The head's state after this pass (read by the next launch; pass 3 is the last).
__device__ inline void set_status(const CertArgs &a, int hq, int v) {
  if (a.pass == 1) a.flags[hq] = v;
  else if (a.pass == 2) a.flags2[hq] = v;
}

// Most segments a head with at most npool candidates can use (rows of `partial`).
__host__ __device__ inline int seg_cap_for(int64_t npool) {
  const int64_t need = (npool + 1023) / 1024;
  return (npool <= kFusedMax) ? 0 : (int)(need < kNumSeg ? need : kNumSeg);
}

__device__ inline void seg_range(int count, int seg, int &i0, int &i1, int &nseg) {
  nseg = (count <= kFusedMax) ? 0 : min(kNumSeg, (count + 1023) / 1024);
  if (seg >= nseg) { i0 = i1 = 0; return; }
  const int len = (count + nseg - 1) / nseg;
  i0 = seg * len;
  i1 = min(count, i0 + len);
}

// Scratch of pass 1's candidate placement (it runs before and after the level sums).
struct PlaceScratch {
  int tiles[256];   // tiles of the current chunk with candidates in the range
  int toff[256];    // the list index of each one's first candidate
  int ws[2][4];
  int slot[256];    // first range: the tile-list entry of each candidate
  int key[256];     // first range: the candidates' positions
  int sum[4][64], cms[4][64];   // per-wavefront level totals
  int th[64][64];               // the tiles' cumulative level counts (heads of at most 64 tiles)
};
struct AccSmem {
  union {
    alignas(16) double acc[kMaxJ + 1][kStatW];   // per-level increments: N[128] V[128] D Q k P X
    PlaceScratch pl;
  };
  double2 ltp[kMaxJ + 2];               // level table in neighbour pairs (for rescoring)
  uint16_t vs[kStage][kD];              // staged V rows
  alignas(16) int hl[kStage];           // read eight at a time
  int pos[kStage];
  int x[kStage];                        // l8 | (UB >= c_lo) << 8
  double w[kStage], vsq[kStage];
};

// Add one staged group of candidates (records in s.hl/w/vsq/pos, cnt <= kStage) into
// s.acc (256 threads).  Heavy keys (h <= J) add (w, w v, w |v|^2) at level h; light
// samples (l < h) add (1, v, |v|^2) at their entry level l and remove it at h, where
// they turn heavy.  Thread t < 128 owns column t of N (threads 0, 1 also D, Q), thread
// 128 + c column c of the light V sums (threads 128, 129 also k, P); each adds its
// candidates' terms in candidate order with LDS atomics that return nothing, so no cell
// is shared between threads and nothing waits on the sums.
// V rows are fetched here unless `staged`.
__device__ __forceinline__ void accumulate_stage(const CertArgs &a, AccSmem &s, int64_t h, int cnt, bool staged) {
  const int t = threadIdx.x, J = a.J;
  if (!staged) {
    // V rows of candidates that enter the sample at some level <= J
    for (int e = t; e < cnt * 16; e += 256) {
      const int r = e >> 4, part = e & 15;
      if ((s.hl[r] >> 8) <= J) {
        const int pos = s.pos[r];
        reinterpret_cast<uint4 *>(s.vs[r])[part] =
            reinterpret_cast<const uint4 *>(a.V + (h * a.n_cap + pos) * kD)[part];
      }
    }
    __syncthreads();
  }
  const bool heavy_col = t < kD;
  const int c = heavy_col ? t : t - kD;
  for (int e0 = 0; e0 < cnt; e0 += 8) {
    // eight records at once (slots past cnt hold stale values and are not used)
    const int4 h0 = *reinterpret_cast<const int4 *>(&s.hl[e0]);
    const int4 h1 = *reinterpret_cast<const int4 *>(&s.hl[e0 + 4]);
    const int raw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
    int hl[8];
    double v[8], w[8], q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int e = e0 + k;
      v[k] = h2d(s.vs[e][c]);
      w[k] = s.w[e];
      q[k] = s.vsq[e];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // the same for every thread: kept in scalar registers, so the tests below are
      // scalar branches (not a candidate: h = l = 255)
      hl[k] = (e0 + k < cnt) ? __builtin_amdgcn_readfirstlane(raw[k]) : 0xFFFF;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int hk = hl[k] & 0xFF, lk = hl[k] >> 8;
      if (heavy_col) {
        if (hk <= J) {
          atomicAdd(&s.acc[hk][t], w[k] * v[k]);
          // D and Q: threads 0 and 1, one instruction
          if (t < 2) atomicAdd(&s.acc[hk][2 * kD + t], (t == 0) ? w[k] : w[k] * q[k]);
        }
      } else if (lk < hk) {
        atomicAdd(&s.acc[lk][t], v[k]);
        if (hk <= J) atomicAdd(&s.acc[hk][t], -v[k]);
        // k and P: threads 128, 129 add (1, |v|^2) at l and remove them at h
        if (c < 2) {
          const double x = c ? q[k] : 1.0;
          atomicAdd(&s.acc[lk][2 * kD + 2 + c], x);
          if (hk <= J) atomicAdd(&s.acc[hk][2 * kD + 2 + c], -x);
        }
      }
    }
    // exact reads outside C_max: threads 130 + k count candidate e0 + k at its refined level
    // l8 (whole numbers: the order of the additions does not matter)
    if (t >= kD + 2 && t < kD + 10 && e0 + (t - kD - 2) < cnt) {
      const int x = s.x[e0 + (t - kD - 2)], l8 = x & 0xFF;
      if (l8 <= J && !(x >> 8)) atomicAdd(&s.acc[l8][2 * kD + 4], 1.0);
    }
  }
  __syncthreads();
}

// Add candidates [i0, i1) of query head hq from their stored records.
__device__ __forceinline__ void accumulate_range(const CertArgs &a, AccSmem &s, int hq, int i0, int i1) {
  const int t = threadIdx.x;
  const int64_t h = head_kv(a, hq);
  const int64_t base = (int64_t)hq * a.npool_cap;
  for (int c0 = i0; c0 < i1; c0 += kStage) {
    const int cnt = min(kStage, i1 - c0);
    if (t < cnt) {
      s.hl[t] = a.rec_hl[base + c0 + t];
      s.w[t] = a.rec_w[base + c0 + t];
      s.vsq[t] = a.rec_vsq[base + c0 + t];
      s.pos[t] = a.candpos[base + c0 + t];
      s.x[t] = a.rec_x[base + c0 + t];
    }
    __syncthreads();
    accumulate_stage(a, s, h, cnt, false);
  }
}

// Rescoring of the stage of candidates [c0, c0 + cnt) (cnt <= kStage) of query head hq.
// First the 8-bit refinement (eight lanes per key, sixteen channels each):
//   S8 = R1-sum_t q_t (scale8 k8_t), slack8 = (qnp kerr8) + 2^-40 ((128 scale8) qabs),
//   UB8 = (S8 + slack8) RSQRT_D, l8 = first((min(UB, UB8) + E) - c*),
// and the key's C_max bit (UB >= c_lo).  Then, for keys with l8 <= J only, the exact
// score and |v|^2, and (one lane per key) h, l and the weight; keys with l8 > J can be
// sampled at no level and get h = l = J + 1.  With kSpec the exact rows are requested
// together with the 8-bit row (one round trip, for the latency of a short first pass);
// otherwise only after l8 is known (the bytes of keys the refinement rules out are not
// read).  Records go into the stage (s.hl, s.x, s.w, s.vsq, staged V rows s.vs) and the
// global records.  E is hashed, and with zero_rows the level increments are cleared,
// while the rows are in flight.
struct RescoreConsts {
  double q16[16];
  double cs, inv_l1, qnp, qabs, clo;
  uint64_t prefix;
};

// Candidate positions of the first stage (placed in LDS by pass 1): the rows of the lane's
// two steps (32 step + 8 wv + lane / 8) and thread t's key.  Entries past the count are
// read but never used.
struct StagePre {
  int pos_r[2];
  int pos_t;
};
__device__ __forceinline__ void stage_positions(const int *pos, StagePre &p) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
#pragma unroll
  for (int step = 0; step < 2; ++step) p.pos_r[step] = pos[32 * step + 8 * wv + (lane >> 3)];
  p.pos_t = pos[min(t, kStage - 1)];
}

template <bool kSpec, int kSteps = 2>
__device__ __forceinline__ void rescore_stage(const CertArgs &a, AccSmem &s, int hq, int c0, int cnt,
                                              const RescoreConsts &rc, int zero_rows = 0,
                                              bool use_pre = false, StagePre pre = StagePre{}) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t h = head_kv(a, hq);
  const int s8 = lane >> 3, k8 = lane & 7;
  const int64_t base = (int64_t)hq * a.npool_cap;
  if (use_pre) {   // (c0 = 0) the positions were read with the counts
    if (t < cnt) s.pos[t] = pre.pos_t;
  } else {
    if (t < cnt) s.pos[t] = a.candpos[base + c0 + t];
    __syncthreads();
  }
  // Step k takes keys 32 k .. 32 k + 31, wavefront wv eight of them (eight lanes per key), so a
  // stage of at most 32 keys is one step of every wavefront (kSteps = 1: cnt <= 32).  Every
  // load of every step is issued before any is used (slots past cnt read position 0 and
  // drop the values).  The eight lanes of a key then form its scalars (perturbation, 8-bit
  // bound and level, exact levels and weight) alike from sums that reach all eight, so no
  // barrier separates the 8-bit bound, the exact score and the records.
  uint4 cw8[2], kw[2][2], vw[2][2];
  float sc8[2];
  double ubt[2];
  uint16_t ke8r[2];
  int pr[2];
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int r = 32 * step + 8 * wv + s8;
    pr[step] = (r < cnt) ? (use_pre ? pre.pos_r[step] : s.pos[r]) : 0;
    const int64_t tok = h * a.n_cap + pr[step];
    cw8[step] = reinterpret_cast<const uint4 *>(a.codes8 + tok * kD)[k8];
    sc8[step] = a.scale8[tok];
    ubt[step] = a.ubuf[base + pr[step]];
    ke8r[step] = a.kerr8[tok];
    kw[step][0] = kw[step][1] = vw[step][0] = vw[step][1] = make_uint4(0, 0, 0, 0);
    if (kSpec) {
      const uint4 *ksrc = reinterpret_cast<const uint4 *>(a.K + tok * kD) + 2 * k8;
      const uint4 *vsrc = reinterpret_cast<const uint4 *>(a.V + tok * kD) + 2 * k8;
      kw[step][0] = ksrc[0];
      kw[step][1] = ksrc[1];
      vw[step][0] = vsrc[0];
      vw[step][1] = vsrc[1];
    }
  }
  double E[2];
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int r = 32 * step + 8 * wv + s8;
    E[step] = (r < cnt) ? perturbation(rc.prefix, pr[step]) : 0.0;
  }
  for (int e = t; e < zero_rows * kStatW; e += 256) (&s.acc[0][0])[e] = 0.0;
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int r = 32 * step + 8 * wv + s8;
    const bool act = r < cnt;
    // the 8-bit bound and its level l8
    double p = 0.0;
    const double sc = (double)sc8[step];
    if (act) {
      const uint32_t wd[4] = {cw8[step].x, cw8[step].y, cw8[step].z, cw8[step].w};
      p = rc.q16[0] * (sc * (double)(int8_t)(wd[0] & 0xFFu));
#pragma unroll
      for (int i = 1; i < 16; ++i) p = p + rc.q16[i] * (sc * (double)(int8_t)((wd[i >> 2] >> (8 * (i & 3))) & 0xFFu));
    }
    const double S8 = r1_combine8_all(p);
    int l8 = a.J + 1, x = 0;
    if (act) {
      const double slack8 = (rc.qnp * h2d(ke8r[step])) + (kPadF * ((128.0 * sc) * rc.qabs));
      const double ub8 = (S8 + slack8) * kRsqrtD;
      l8 = level_of_pairs((fmin(ubt[step], ub8) + E[step]) - rc.cs, s.ltp, a.J, rc.inv_l1);
      x = l8 | ((ubt[step] >= rc.clo) ? 0x100 : 0);
    }
    // the exact score and |v|^2 of the keys with l8 <= J (rows read now unless speculative)
    const bool ex = act && l8 <= a.J;
    if (!kSpec && ex) {
      const int64_t tok = h * a.n_cap + pr[step];
      const uint4 *ksrc = reinterpret_cast<const uint4 *>(a.K + tok * kD) + 2 * k8;
      const uint4 *vsrc = reinterpret_cast<const uint4 *>(a.V + tok * kD) + 2 * k8;
      kw[step][0] = ksrc[0];
      kw[step][1] = ksrc[1];
      vw[step][0] = vsrc[0];
      vw[step][1] = vsrc[1];
    }
    double ps = 0.0, pv = 0.0;
    if (ex) {
      ps = score_words(rc.q16, kw[step][0], kw[step][1]);
      // the V row is staged for the accumulation while its |v|^2 is formed
      uint4 *vdst = reinterpret_cast<uint4 *>(s.vs[r]) + 2 * k8;
      vdst[0] = vw[step][0];
      vdst[1] = vw[step][1];
      pv = sumsq_words(vw[step][0], vw[step][1]);
    }
    const double scx = r1_combine8_all(ps) * kRsqrtD;
    const double vs = r1_combine8_all(pv);
    // the key's levels, weight and records (its first lane writes them)
    if (act && k8 == 0) {
      int hl = a.J + 1, ll = a.J + 1;
      double sco = 0.0, w = 0.0, vsq = 0.0;
      if (ex) {
        sco = scx;
        hl = level_of_pairs(scx - rc.cs, s.ltp, a.J, rc.inv_l1);
        ll = level_of_pairs((scx + E[step]) - rc.cs, s.ltp, a.J, rc.inv_l1);
        w = exp(scx - rc.cs);
        vsq = (ll <= a.J) ? vs : 0.0;
      }
      s.hl[r] = hl | (ll << 8);
      s.w[r] = w;
      s.vsq[r] = vsq;
      s.x[r] = x;
      a.rec_s[base + c0 + r] = sco;
      a.rec_w[base + c0 + r] = w;
      a.rec_vsq[base + c0 + r] = vsq;
      a.rec_hl[base + c0 + r] = hl | (ll << 8);
      a.rec_x[base + c0 + r] = x;
    }
  }
  __syncthreads();
}

// The per-query constants of rescoring: the query chunk of the lane (eight lanes per key,
// sixteen channels each), c*, c_lo, |q| pad and sum |q|, the hash prefix, 1 / log tau_1.
__device__ __forceinline__ void rescore_consts_load(const CertArgs &a, int hq, RescoreConsts &c) {
  const int k8 = threadIdx.x & 7;
#pragma unroll
  for (int i = 0; i < 16; ++i) c.q16[i] = (double)a.qf[(int64_t)hq * kD + 16 * k8 + i];
  c.cs = dec_max(a.cstar[hq]);
  c.clo = dec_max(a.clo[hq]);
  c.qnp = a.qconst[(int64_t)hq * kQc + QC_QNP];
  c.qabs = a.qconst[(int64_t)hq * kQc + QC_QABS];
  c.prefix = a.prefix[hq / a.G];
}
// (s.ltp must be filled and the workgroup past a barrier since)
__device__ __forceinline__ void rescore_consts(const CertArgs &a, const AccSmem &s, int hq, RescoreConsts &c) {
  rescore_consts_load(a, hq, c);
  c.inv_l1 = (a.J >= 1) ? 1.0 / s.ltp[1].y : 0.0;
}

// Exact rescoring of candidates [i0, i1) of query head hq inside the certificate
// workgroup, stage by stage, each stage added into the level increments s.acc.
__device__ __forceinline__ void rescore_accumulate(const CertArgs &a, AccSmem &s, int hq, int i0, int i1) {
  __syncthreads();              // the level table s.ltp is filled
  RescoreConsts rc;
  rescore_consts(a, s, hq, rc);
  for (int c0 = i0; c0 < i1; c0 += kStage) {
    const int cnt = min(kStage, i1 - c0);
    rescore_stage<false>(a, s, hq, c0, cnt, rc);
    accumulate_stage(a, s, head_kv(a, hq), cnt, true);
  }
}

__device__ inline void zero_acc(AccSmem &s, int J1) {
  for (int e = threadIdx.x; e < J1 * kStatW; e += blockDim.x) (&s.acc[0][0])[e] = 0.0;
  __syncthreads();
}

// Candidates [i0, i1): those below `split` from their stored records, the rest rescored
// here (records stored), in index order.
__device__ __forceinline__ void accumulate_mixed(const CertArgs &a, AccSmem &s, int hq, int i0, int i1, int split) {
  if (i0 < split) accumulate_range(a, s, hq, i0, min(i1, split));
  if (i1 > split) rescore_accumulate(a, s, hq, max(i0, split), i1);
}

// Which candidates of this pass already have records: the first pass's, when a separate
// kernel rescored them, and in later passes the earlier passes' ranges.
__device__ inline int record_split(const CertArgs &a, int hq, int count) {
  if (a.pass == 1) return 0;
  return (a.pass == 2) ? a.ccount1[hq] : a.ccount2[hq];
}

// Root of kl(x, mu) = mu - x + x ln(x / mu) = L above x: Newton from above on the convex
// increasing branch (every iterate stays above the root, so the bound is valid wherever
// it stops).  It stops when a step no longer decreases mu, or after a step that moved mu
// by at most 2^-26 of itself: Newton's relative error after such a step is about
// x / (2 (mu - x)) times its square, far below the 1e-4 the certificate is compared to.
// The step is mu - f mu / (mu - x) with f = (mu - x) + x (ln x - ln mu) - L.
__device__ inline double kl_upper(double x, double L) {
  if (!(x > 0.0)) return L;
  const double lx = log(x);
  double mu = x + L + sqrt(L * L + 2.0 * x * L);
  for (int it = 0; it < 100; ++it) {
    const double f = (mu - x) + x * (lx - log(mu)) - L;
    const double nx = mu - f * mu / (mu - x);
    if (!(nx < mu)) break;
    const bool small = mu - nx <= 0x1p-26 * mu;   // converged: the iterate stays above the root
    mu = nx;
    if (small) break;
  }
  return mu;
}
// Root of kl(x, mu) = L below x (Newton from below on the convex decreasing branch).
__device__ inline double kl_lower(double x, double L) {
  if (!(x > 0.0)) return 0.0;
  const double lx = log(x);
  double mu = fmax(x - sqrt(2.0 * x * L), x * exp(-1.0 - L / x));
  if (!(mu > 0.0)) return 0.0;
  for (int it = 0; it < 100; ++it) {
    const double f = (mu - x) + x * (lx - log(mu)) - L;
    const double nx = mu - f * mu / (mu - x);
    if (!(nx > mu) || !(nx < x)) break;
    const bool small = nx - mu <= 0x1p-26 * mu;   // converged: the iterate stays below the root
    mu = nx;
    if (small) break;
  }
  return mu;
}

// Certificate of one level from the prefix sums and the level's four KL roots
// (mu_hi, mu_lo of k; mu_G of y; mu_Q of P / Vmax^2), all in fp64.
__device__ inline double level_beta(const CertArgs &a, double D_det, double Q_det, double k, double tau,
                                    double Vmax, double cn2, double dn2, double on2, const double *root) {
  const double L = a.L;
  const double D_hat = D_det + tau * k;
  const double mu_hi = root[0], mu_lo = root[1];
  const double dD = tau * fmax(k - mu_lo, mu_hi - k);
  const double D_hi = D_det + tau * mu_hi;
  const double inf = __builtin_huge_val();
  if (a.measure == CSA_MEASURE_DENOM) return (D_hat > dD) ? dD / (D_hat - dD) : inf;
  const double cn = sqrt(cn2), Rc = Vmax + cn;
  const double mu_G = root[2];
  const double sigma2 = tau * tau * Rc * Rc * mu_G;
  const double zeta = sqrt(2.0 * sigma2 * L) + (2.0 / 3.0) * (tau * Rc) * L;
  const double dn = sqrt(dn2), on = sqrt(on2);
  const double beta_abs = (D_hat > dD) ? (zeta + dn * dD) / (D_hat - dD) : inf;
  if (a.measure == CSA_MEASURE_OUTNORM) return (on > beta_abs) ? beta_abs / (on - beta_abs) : inf;
  const double mu_Q = root[3];
  const double Q_lo = Q_det + tau * Vmax * Vmax * mu_Q;
  const double M_lo = fmax(on - beta_abs, sqrt(Q_lo / D_hi));
  return (M_lo > 0.0 && beta_abs < inf) ? beta_abs / M_lo : inf;
}

struct FinSmem {
  AccSmem s;
  double tau[kMaxJ + 1];
  int hist[kMaxJ + 2];
  int cmh[kMaxJ + 2];            // C_max keys per bucket level
  alignas(16) double nr[kD];
  double vmax;
  double dr, qr;
  double beta[kMaxJ + 1];
  double dots[kMaxJ + 1][4];     // |c|^2, c.V, |o^ - c|^2, |o^|^2 per level
  double dpart[kMaxJ + 1][4][4]; // the same over channel quarters
  double root[kMaxJ + 1][4];
  int jstar;
  long long extra[4];
};

// The certificate's inputs that depend on nothing of the pass: thresholds and level
// table, V_max from the scan's wavefront maxima, the window sums rescaled from c_R to c*,
// and (after pass 1, which has them from its own sums) the C_max counts per level.  They
// are read into registers first (head_issue) and written to LDS later (head_commit), so
// the loads travel together with whatever the caller issues in between.
struct HeadPre {
  double tau, ltx, lty;   // thread t: tau_t and the level-table pair of level t
  double win;             // thread t < kD + 2: window sum t (relative to c_R)
  double cr;
  unsigned long long cs;  // c* (encoded)
  unsigned vp0, vp1, vp2;  // wavefront 3: its lanes' V_max bits (entries lane, lane + 64, the rest)
  int vpn;                 // wavefront 3: how many of the first 128 entries exist
  int cmh;                // thread t <= J + 1: C_max keys at level t (not in pass 1)
};
template <bool kFirst>
__device__ __forceinline__ void head_issue(const CertArgs &a, int hq, HeadPre &p) {
  const int t = threadIdx.x, h = hq / a.G;
  const int lane = t & 63, wv = t >> 6, J = a.J;
  p.tau = (t <= J) ? a.tau[t] : 0.0;
  p.ltx = (t >= 1 && t <= J + 1) ? a.lt[t - 1] : __builtin_huge_val();
  p.lty = (t <= J) ? a.lt[t] : -__builtin_huge_val();
  p.win = (t < kD + 2) ? a.win[(int64_t)hq * kWinW + t] : 0.0;
  p.cr = a.qconst[(int64_t)hq * kQc + QC_CR];
  p.cs = a.cstar[hq];
  p.cmh = (!kFirst && t <= J + 1) ? a.cmhist[(int64_t)hq * (J + 2) + t] : 0;
  p.vp0 = p.vp1 = p.vp2 = 0u;
  p.vpn = 0;
  if (wv == 3) {
    // (entries past the unit's wavefronts are read within the row and not used; the two
    // loads are only combined at head_commit, so nothing waits for them here)
    const int64_t np = unit_npool(a.b, h, a.W);
    const int64_t wph = ((np + kBlk - 1) / kBlk + kScanBlocks - 1) / kScanBlocks;   // the unit's scan wavefronts
    const unsigned *vp = a.vpart + (int64_t)h * a.wstride;
    p.vp0 = vp[min<int64_t>(lane, a.wstride - 1)];
    p.vp1 = vp[min<int64_t>(lane + 64, a.wstride - 1)];
    p.vpn = (int)min<int64_t>(wph, 128);
    if (wph > 128) {   // (a separate value: no wait for the two loads above at this branch)
      unsigned v = 0u;
      for (int64_t k = lane + 128; k < wph; k += 64) v = max(v, vp[k]);
      p.vp2 = v;
    }
  }
}
template <bool kFirst>
__device__ __forceinline__ void head_commit(const CertArgs &a, FinSmem &f, const HeadPre &p) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, J = a.J;
  if (t <= J) f.tau[t] = p.tau;
  if (t <= J + 1) f.s.ltp[t] = make_double2(p.ltx, p.lty);
  if (!kFirst && t <= J + 1) f.cmh[t] = p.cmh;
  if (!kFirst && wv == 0) {   // |C_max| (pass 1 takes it from its own sums)
    const int tot = __builtin_amdgcn_readlane(wave_incl_scan(lane <= J + 1 ? p.cmh : 0), 63);
    if (lane == 0) f.extra[0] = tot;
  }
  if (wv == 3) {
    unsigned v = max(max(lane < p.vpn ? p.vp0 : 0u, lane + 64 < p.vpn ? p.vp1 : 0u), p.vp2);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, off, 64));
    if (lane == 0) f.vmax = h2d((uint16_t)v);
  }
  const double sc = exp(p.cr - dec_max(p.cs));
  if (t < kD) f.nr[t] = p.win * sc;
  if (t == kD) f.dr = p.win * sc;
  if (t == kD + 1) f.qr = p.win * sc;
}

// The certificate of query head hq in pass a.pass, by one workgroup of 256 threads: level
// sums (directly, or from the segments' increments), window sums, prefix over levels, the
// certificate of every level up to the pass's last level, the stop level and the outputs.
// Returns true when a level certifies (outputs written); otherwise the head is flagged
// for the extension pass (2) or for the exact fallback (1).  Uniform across the group.
// nparts: partial tables of this pass written by other workgroups (0: accumulate every
// candidate here; -1: as many as seg_range gives for the count).
// kFirst: pass 1 in the certificate kernel, after its placement step, which left the
// candidate count (pcount) and deepest level (pjmax) of the pass, the head_issue inputs in
// LDS, the rescoring constants (*rc0) and, when the candidates fit one stage, their
// positions in s.pos.
template <bool kFirst>
__device__ __forceinline__ bool certify_head(const CertArgs &a, FinSmem &f, int hq, int nparts, int pcount,
                             int pjmax, const RescoreConsts *rc0) {
  const int t = threadIdx.x, h = hq / a.G;
  const int lane = t & 63, wv = t >> 6;
  AccSmem &s = f.s;
  const int J1 = a.J + 1;
  // every load that does not depend on the candidate count is issued before it is used
  const int count = kFirst ? pcount : pass_count(a, hq);
  const int jmax = kFirst ? pjmax : pass_jmax(a, hq);
  // pass 1 takes its candidates (at most `budget`) in one stage when they fit: their
  // positions are in LDS, the rescoring constants are read now
  const bool spec = kFirst && (nparts < 0);
  StagePre pre{};
  RescoreConsts rc;
  if (spec) {
    stage_positions(s.pos, pre);
    rc = *rc0;
  }
  if (!kFirst) {
    HeadPre hp;
    head_issue<false>(a, hq, hp);
    head_commit<false>(a, f, hp);
  }
  if (count < 0) return false;
  int i0, i1, nseg;
  seg_range(count, 0, i0, i1, nseg);
  if (nparts >= 0) nseg = nparts;
  // a single stage rescored here: the increments are cleared while its rows arrive
  if (nseg == 0 && count <= kStage && record_split(a, hq, count) == 0) {
    __syncthreads();            // the level table s.ltp is filled
    if (spec) rc.inv_l1 = (a.J >= 1) ? 1.0 / s.ltp[1].y : 0.0;
    else rescore_consts(a, s, hq, rc);
    if (count <= 32) rescore_stage<true, 1>(a, s, hq, 0, count, rc, jmax + 1, spec, pre);
    else rescore_stage<true, 2>(a, s, hq, 0, count, rc, jmax + 1, spec, pre);
    accumulate_stage(a, s, head_kv(a, hq), count, true);
  } else if (nseg == 0) {
    zero_acc(s, jmax + 1);      // rows above jmax may receive increments but are never read
    accumulate_mixed(a, s, hq, 0, count, record_split(a, hq, count));
  } else {
    for (int e = t; e < J1 * kStatW; e += 256) {
      double v = 0.0;
      const double *col = a.partial + (int64_t)hq * a.nseg_cap * J1 * kStatW + e;
      int sg = 0;
      for (; sg + 8 <= nseg; sg += 8) {
        double x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = col[(int64_t)(sg + k) * J1 * kStatW];
#pragma unroll
        for (int k = 0; k < 8; ++k) v += x[k];
      }
      for (; sg < nseg; ++sg) v += col[(int64_t)sg * J1 * kStatW];
      (&s.acc[0][0])[e] = v;
    }
    __syncthreads();
  }
  // prefix over levels, eight rows at a time: thread t takes column t and, for t < 5, the
  // scalar column 256 + t as a second chain (the others run it on the pad column)
  {
    const int c2 = (t < 5) ? 2 * kD + t : kStatW - 1;
    double run = 0.0, run2 = 0.0;
    int j = 0;
    for (; j + 8 <= jmax + 1; j += 8) {
      double v[8], v2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = s.acc[j + i][t];
        v2[i] = s.acc[j + i][c2];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        run += v[i];
        run2 += v2[i];
        s.acc[j + i][t] = run;
        s.acc[j + i][c2] = run2;
      }
    }
    for (; j <= jmax; ++j) {
      run += s.acc[j][t];
      run2 += s.acc[j][c2];
      s.acc[j][t] = run;
      s.acc[j][c2] = run2;
    }
  }
  __syncthreads();
  // certificate of every level up to jmax: dot products per level (wavefront wv takes
  // levels wv, wv + 4, ...), then the four KL roots of every level in parallel, then beta
  const double Vmax = f.vmax;
  {
    const int j = t >> 2, qt = t & 3;
    if (j <= jmax) {
      const double tau = f.tau[j];
      const double D_det = f.dr + s.acc[j][256];
      const double D_hat = D_det + tau * s.acc[j][258];
      const double iD = 1.0 / D_det, iDh = 1.0 / D_hat;
      double cn2 = 0.0, cV = 0.0, dn2 = 0.0, on2 = 0.0;
      // two channels per 16-byte read, added in channel order
      const double2 *rN = reinterpret_cast<const double2 *>(&s.acc[j][32 * qt]);
      const double2 *rV = reinterpret_cast<const double2 *>(&s.acc[j][128 + 32 * qt]);
      const double2 *rR = reinterpret_cast<const double2 *>(&f.nr[32 * qt]);
#pragma unroll 4
      for (int c2 = 0; c2 < 16; ++c2) {
        const double2 N2 = rN[c2], V2 = rV[c2], R2 = rR[c2];
        const double Nc[2] = {N2.x, N2.y}, Vc[2] = {V2.x, V2.y}, Rc2[2] = {R2.x, R2.y};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const double nd = Rc2[e] + Nc[e];
          const double cc = nd * iD;
          const double o = (nd + tau * Vc[e]) * iDh;
          cn2 += cc * cc;
          cV += cc * Vc[e];
          dn2 += (o - cc) * (o - cc);
          on2 += o * o;
        }
      }
      f.dpart[j][qt][0] = cn2;
      f.dpart[j][qt][1] = cV;
      f.dpart[j][qt][2] = dn2;
      f.dpart[j][qt][3] = on2;
    }
  }
  __syncthreads();
  if (t < 4 * (jmax + 1)) {
    const int j = t >> 2, r = t & 3;
    f.dots[j][r] = (f.dpart[j][0][r] + f.dpart[j][1][r]) + (f.dpart[j][2][r] + f.dpart[j][3][r]);
  }
  __syncthreads();
  {
    // roots: wavefronts 0-1 the upper ones (r = 0: of k; r = 2: of the G statistic),
    // wavefronts 2-3 the lower ones (r = 1: of k; r = 3: of P / Vmax^2)
    const bool upper = t < 128;
    const int u = t & 127, j = u >> 1, r = (upper ? 0 : 1) + 2 * (u & 1);
    if (j <= jmax) {
      const double k = s.acc[j][258], P = s.acc[j][259];
      double x;
      if (r < 2) {
        x = k;
      } else if (r == 2) {
        const double cn2 = f.dots[j][0], cn = sqrt(cn2), Rc = Vmax + cn;
        x = (Rc > 0.0) ? fmax((P - 2.0 * f.dots[j][1] + k * cn * cn) / (Rc * Rc), 0.0) : 0.0;
      } else {
        x = (Vmax > 0.0) ? P / (Vmax * Vmax) : 0.0;
      }
      f.root[j][r] = upper ? kl_upper(x, a.L) : kl_lower(x, a.L);
    }
  }
  __syncthreads();
  if (t <= jmax) {
    const int j = t;
    const double tau = f.tau[j];
    const double D_det = f.dr + s.acc[j][256];
    const double Q_det = f.qr + s.acc[j][257];
    const double k = s.acc[j][258];
    const double b = level_beta(a, D_det, Q_det, k, tau, Vmax, f.dots[j][0], f.dots[j][2], f.dots[j][3],
                                f.root[j]);
    f.beta[j] = b;
    a.betalv[(int64_t)hq * J1 + j] = b;
    a.dhatlv[(int64_t)hq * J1 + j] = D_det + tau * k;
    a.klv[(int64_t)hq * J1 + j] = (int)k;
  }
  __syncthreads();
  if (wv == 0) {
    const double eps = a.eps[head_item(a, hq)];
    const unsigned long long ok = __ballot(lane <= jmax && f.beta[lane] <= eps);
    if (lane == 0) f.jstar = ok ? (__ffsll((long long)ok) - 1) : a.J + 1;
  }
  __syncthreads();
  const int js = f.jstar;
  if (js > a.J || (js > jmax)) {
    // no level up to jmax certifies: either the next pass takes deeper levels, or
    // (jmax = J) the head falls back to exact attention
    if (t == 0) {
      const bool extend = (jmax < a.J);
      set_status(a, hq, extend ? a.pass + 1 : 1);
      a.stop[hq] = a.J + 1;
      a.beta[hq] = 0.0;
      a.keys_read[hq] = head_n(a, hq);
    }
    return false;
  }
  // keys read exactly: window + |C_max| (f.extra[0], written by thread 0 before) + the
  // candidates outside C_max whose refined level l8 is at most j* (column 260 counts them
  // by l8, prefix-summed over levels)
  const double tau = f.tau[js];
  const double D_hat = (f.dr + s.acc[js][256]) + tau * s.acc[js][258];
  if (t < kD)
    a.o_hat[(int64_t)hq * kD + t] = (float)(((f.nr[t] + s.acc[js][t]) + tau * s.acc[js][128 + t]) / D_hat);
  if (t == 0) {
    set_status(a, hq, 0);
    a.stop[hq] = js;
    a.beta[hq] = f.beta[js];
    a.keys_read[hq] = (int64_t)a.W + f.extra[0] + (int64_t)s.acc[js][2 * kD + 4];
  }
  return true;
}

// Exclusive prefix of v[0..N) over the workgroup's 256 threads in thread order; tot[] gets
// the sums.  All threads take part; two barriers.
template <int N>
__device__ __forceinline__ void wg_excl_scan(int *v, int (*ws)[4], int *tot) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int x[N];
#pragma unroll
  for (int k = 0; k < N; ++k) x[k] = v[k];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int y = __shfl_up(x[k], off, 64);
      if (lane >= off) x[k] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < N; ++k) ws[k][wv] = x[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) {
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = ws[k][w];
      all += c;
      before += (w < wv) ? c : 0;
    }
    tot[k] = all;
    v[k] = before + x[k] - v[k];
  }
  __syncthreads();
}

// Pass 1's placement of the candidates with lo < l^ub <= hi (levels from the bucket
// count; lo = -1 for the first range) in position order, at list indices base, base + 1,
// ...: the tiles' counts come from their cumulative histograms, so each tile's first index
// is a prefix over tiles, and a wavefront places one tile at a time (lane = bitmap word;
// the levels of its live keys from the l^ub bytes).  Indices below nstage also go into the
// stage's positions s.pos.  Ends with the workgroup in step.
__device__ __forceinline__ void place_range(const CertArgs &a, FinSmem &f, int hq, int64_t npool, int lo, int hi, int base,
                            int nstage) {
  AccSmem &s = f.s;
  PlaceScratch &ps = s.pl;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, J2 = a.J + 2;
  const int64_t row = (int64_t)hq * a.npool_cap;
  const int64_t ntiles = (npool + kBucketTile - 1) / kBucketTile;   // this head's tiles
  const int *th = a.tilehist + (int64_t)hq * a.ntiles * J2;
  int run = base;
  for (int64_t k0 = 0; k0 < ntiles; k0 += 256) {
    const int64_t k = k0 + t;
    int c = 0;
    if (k < ntiles) {
      const int *r = th + k * J2;
      c = r[hi] - (lo >= 0 ? r[lo] : 0);
    }
    int v[2] = {c, c > 0 ? 1 : 0}, tot[2];
    wg_excl_scan<2>(v, ps.ws, tot);
    if (c > 0) {
      ps.tiles[v[1]] = (int)k;
      ps.toff[v[1]] = run + v[0];
    }
    __syncthreads();
    for (int i = wv; i < tot[1]; i += 4) {
      const int64_t tk = ps.tiles[i];
      const int64_t wi = tk * 64 + lane, p0 = wi * 32;
      const int valid = (int)max<int64_t>(0, min<int64_t>(32, npool - p0));
      uint32_t bits = 0u, m = 0u;
      if (valid > 0) bits = a.live[(int64_t)hq * a.nwords + wi] & ((valid == 32) ? 0xFFFFFFFFu : ((1u << valid) - 1u));
      if (bits) {
        const uint4 *lp = reinterpret_cast<const uint4 *>(a.lub + row + p0);
        const uint4 l0 = lp[0], l1 = lp[1];
        const uint32_t x[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
        for (int b = 0; b < 32; ++b) {
          const int l = (int)(int8_t)((x[b >> 2] >> (8 * (b & 3))) & 0xFFu);
          if (((bits >> b) & 1u) && l > lo && l <= hi) m |= 1u << b;
        }
      }
      const int n = __popc(m);
      int xs = n;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(xs, off, 64);
        if (lane >= off) xs += y;
      }
      int o = ps.toff[i] + xs - n;
      while (m) {
        const int b = __ffs((int)m) - 1;
        m &= m - 1u;
        const int pos = (int)(p0 + b);
        a.candpos[row + o] = pos;
        if (o < nstage) s.pos[o] = pos;
        ++o;
      }
    }
    run += tot[0];
    __syncthreads();
  }
}

// Lane L of the caller's quad of lanes (a DPP quad broadcast).
template <int L>
__device__ __forceinline__ int quad_lane(int x) {
  return __builtin_amdgcn_update_dpp(0, x, 0x55 * L, 0xF, 0xF, false);
}

// Pass 1's first range (l^ub <= js, tot1 candidates) from the tiles' level-ordered lists:
// tile k holds the range's keys in its first tilehist[k][js] list entries, so each
// candidate is one read; the list is then put in position order by ranking in LDS.
// Returns false, having written nothing, when the range has more candidates than threads
// or a tile holds more of them than its list; uniform across the workgroup.
__device__ __forceinline__ bool place_first_lists(const CertArgs &a, FinSmem &f, int hq, int64_t npool, int js, int tot1,
                                  int nstage) {
  AccSmem &s = f.s;
  PlaceScratch &ps = s.pl;
  const int t = threadIdx.x, J2 = a.J + 2;
  if (tot1 > 256) return false;
  const int64_t ntiles = (npool + kBucketTile - 1) / kBucketTile;
  const int *th = a.tilehist + (int64_t)hq * a.ntiles * J2;
  int run = 0;
  for (int64_t k0 = 0; k0 < ntiles; k0 += 256) {
    const int64_t k = k0 + t;
    const int c = (k < ntiles) ? th[k * J2 + js] : 0;
    int v[2] = {c, c > kTileList ? 1 : 0}, tot[2];
    wg_excl_scan<2>(v, ps.ws, tot);
    if (tot[1] > 0) return false;
    for (int e = 0; e < c; ++e) ps.slot[run + v[0] + e] = (int)(k * kTileList + e);
    run += tot[0];
  }
  __syncthreads();
  int pos = 0;
  if (t < tot1) {
    pos = a.tilelist[(int64_t)hq * a.ntiles * kTileList + ps.slot[t]];
    ps.key[t] = pos;
  }
  __syncthreads();
  if (t < tot1) {   // positions are distinct: the ranks are a permutation
    int r = 0;
    for (int i = 0; i < tot1; ++i) r += (ps.key[i] < pos) ? 1 : 0;
    a.candpos[(int64_t)hq * a.npool_cap + r] = pos;
    if (r < nstage) s.pos[r] = pos;
  }
  return true;
}

// Pass 1, one workgroup per query head (heads with n <= W go straight to exact attention):
// the head's level totals and speculative levels from the tile histograms, the first range
// of the candidate list, the certificate of the levels up to the speculative level, and,
// for heads that need a later pass (or with every range requested), the other ranges.
__global__ __launch_bounds__(256) void finish_kernel(CertArgs a) {
  const int hq = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t npool = unit_npool(a.b, hq / a.G, a.W);
  if (npool == 0) {
    if (t == 0) {
      a.flags[hq] = 1;
      a.stop[hq] = 0;
      a.beta[hq] = 0.0;
      a.keys_read[hq] = head_n(a, hq);
    }
    return;
  }
  __shared__ FinSmem f;
  PlaceScratch &ps = f.s.pl;
  const int J = a.J, J2 = J + 2;
  const int64_t ntiles = (npool + kBucketTile - 1) / kBucketTile;
  const bool small = ntiles <= 64;   // the tile rows are kept in LDS
  // the first eight entries of every tile's level-ordered list, read before it is known
  // how many of them the first range takes (thread t: tile t >> 2, entries (t & 3) + 4 i)
  const int sk = t >> 2, se = t & 3;
  // (tiles past the head's read its last tile's entries, which no candidate takes)
  int sp[2] = {0, 0};
  if (small) {
    const int *lp = a.tilelist + ((int64_t)hq * a.ntiles + min<int64_t>(sk, ntiles - 1)) * kTileList + se;
    sp[0] = lp[0];
    sp[1] = lp[4];
  }
  // the certificate's inputs and the rescoring constants travel with the tile sums
  HeadPre hp;
  head_issue<true>(a, hq, hp);
  RescoreConsts rc;
  rescore_consts_load(a, hq, rc);
  // level totals over the tiles (lane = level; wavefront wv sums tiles wv, wv + 4, ...):
  // candidates at levels <= j, C_max keys per level
  {
    // (at most 64 tiles: one straight block of loads, no loop whose header would wait for
    // every load issued before it)
    int cum = 0, cm = 0;
    if (lane < J2) {
      const int *th = a.tilehist + (int64_t)hq * a.ntiles * J2 + lane;
      const int *tc = a.tilecm + (int64_t)hq * a.ntiles * J2 + lane;
      // (rows past the head's tiles are read at its last tile and counted as 0: loads and
      // LDS writes without branches; ps.th rows past ntiles are not read)
      auto sum16 = [&](int64_t k0, bool keep) __attribute__((always_inline)) {
        int u[16], w[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int64_t kk = min<int64_t>(k0 + 4 * k, ntiles - 1);
          u[k] = th[kk * J2];
          w[k] = tc[kk * J2];
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const bool in = k0 + 4 * k < ntiles;
          u[k] = in ? u[k] : 0;
          cum += u[k];
          cm += in ? w[k] : 0;
          if (keep) ps.th[k0 + 4 * k][lane] = u[k];
        }
      };
      if (small) {
        sum16(wv, true);
      } else {
        for (int64_t k0 = wv; k0 < ntiles; k0 += 64) sum16(k0, false);
      }
    }
    ps.sum[wv][lane] = cum;
    ps.cms[wv][lane] = cm;
  }
  head_commit<true>(a, f, hp);
  __syncthreads();
  const int cum = ps.sum[0][lane] + ps.sum[1][lane] + ps.sum[2][lane] + ps.sum[3][lane];
  // the levels that fit form a prefix 0..js (cumulative counts only grow); js = -1 when
  // level 0 alone exceeds the budget, and the first pass then has no candidates
  const unsigned long long fit = __ballot(lane <= J && cum <= a.budget);
  const int js = (int)__popcll(fit) - 1;   // (the count is unsigned)
  const unsigned long long fit2 = __ballot(lane <= J && cum <= a.budget2);
  const int js2 = min(J, max(js + 1, (int)__popcll(fit2) - 1));   // at least one level past js
  // (js, js2 and J are the same in every lane: lane reads, not shuffles)
  const int tot1v = __builtin_amdgcn_readlane(cum, max(js, 0)), tot2 = __builtin_amdgcn_readlane(cum, js2);
  const int tot1 = (js >= 0) ? tot1v : 0;
  if (wv == 0) {
    const int cm = ps.cms[0][lane] + ps.cms[1][lane] + ps.cms[2][lane] + ps.cms[3][lane];
    const int below = __shfl_up(cum, 1, 64), totJ = __builtin_amdgcn_readlane(cum, J);
    const int64_t hr = (int64_t)hq * J2;
    if (lane < J2) {
      a.hist[hr + lane] = cum - (lane > 0 ? below : 0);
      a.cmhist[hr + lane] = cm;
      f.cmh[lane] = cm;
    }
    const int cm_all = __builtin_amdgcn_readlane(wave_incl_scan(lane < J2 ? cm : 0), 63);
    if (lane == 0) f.extra[0] = cm_all;   // |C_max|
    if (lane == 0) {
      a.jspec[hq] = js;
      a.ccount1[hq] = tot1;
      a.jspec2[hq] = js2;
      a.ccount2[hq] = tot2;
      a.ccount[hq] = totJ;
    }
  }
  const int nstage = (tot1 <= kStage) ? tot1 : 0;
  bool placed = js < 0;
  if (!placed && small) {
    // the first range's count per tile (lane = tile; every wavefront computes all of them)
    // and the tiles' first list indices; when no tile has more than eight, the entries
    // read above are the whole range, and a candidate's index is its tile's first index
    // plus its rank by position among the tile's entries
    const int c = (lane < ntiles) ? ps.th[lane][js] : 0;
    const int incl = wave_incl_scan(c);
    if (__ballot(c > 8) == 0ull) {
      const int ck = __shfl(c, sk, 64), first = __shfl(incl - c, sk, 64);
      // the tile's entries are in the lane's quad (lanes 4 (lane / 4) + j), both registers
      const int e0[4] = {quad_lane<0>(sp[0]), quad_lane<1>(sp[0]), quad_lane<2>(sp[0]), quad_lane<3>(sp[0])};
      const int e1[4] = {quad_lane<0>(sp[1]), quad_lane<1>(sp[1]), quad_lane<2>(sp[1]), quad_lane<3>(sp[1])};
      int r0 = 0, r1 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q0 = e0[j], q1 = e1[j];
        if (j < ck) {
          r0 += (q0 < sp[0]) ? 1 : 0;
          r1 += (q0 < sp[1]) ? 1 : 0;
        }
        if (j + 4 < ck) {
          r0 += (q1 < sp[0]) ? 1 : 0;
          r1 += (q1 < sp[1]) ? 1 : 0;
        }
      }
      // (the indices lie in [0, tot1) by construction; the bound keeps every store in the
      // head's row regardless)
      const int64_t row = (int64_t)hq * a.npool_cap;
      const int o0 = first + r0, o1 = first + r1;
      if (se < ck && o0 < tot1) {
        a.candpos[row + o0] = sp[0];
        if (o0 < nstage) f.s.pos[o0] = sp[0];
      }
      if (se + 4 < ck && o1 < tot1) {
        a.candpos[row + o1] = sp[1];
        if (o1 < nstage) f.s.pos[o1] = sp[1];
      }
      placed = true;
    }
  }
  if (!placed && !place_first_lists(a, f, hq, npool, js, tot1, nstage))
    place_range(a, f, hq, npool, -1, js, 0, nstage);
  // (more than one stage: the rescoring reads the list back from memory)
  if (tot1 > kStage) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tot1 > kStage) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const bool ok = certify_head<true>(a, f, hq, -1, tot1, js, &rc);
  if ((!ok && js < J) || a.full_list) {
    __syncthreads();
    place_range(a, f, hq, npool, js, js2, tot1, 0);
    if (js2 < J) place_range(a, f, hq, npool, js2, J, tot2, 0);
  }
}

struct ExactSmem {
  double qd[kD];
  double w[256];
  double half[kD];   // after the call: N[c] of the whole range
  double dsum[4];    // after the call: dsum[0] = D of the whole range
};

// Exact attention sums over keys [i0, i1) of query head hq relative to c*: N[c] (out[c])
// and D (out[kD]), 256 threads.  Keys in batches of 256: one key per thread for its score
// and weight, then two halves of the batch over the 128 channels.
__device__ __forceinline__ void exact_chunk(const CertArgs &a, ExactSmem &e, int hq, int64_t i0, int64_t i1, double *out) {
  const int t = threadIdx.x, c = t & (kD - 1), hf = t >> 7;
  const int64_t h = head_kv(a, hq);
  if (t < kD) e.qd[t] = (double)a.qf[(int64_t)hq * kD + t];
  const double cs = dec_max(a.cstar[hq]);
  __syncthreads();
  double accN = 0.0, accD = 0.0;
  for (int64_t b = i0; b < i1; b += 256) {
    const int cnt = (int)min<int64_t>(256, i1 - b);
    if (t < cnt) {
      const double sc = exact_score(e.qd, a.K + (h * a.n_cap + b + t) * kD);
      const double w = exp(sc - cs);
      e.w[t] = w;
      accD += w;
    }
    __syncthreads();
    for (int i = 128 * hf; i < min(cnt, 128 * hf + 128); ++i)
      accN += e.w[i] * h2d(a.V[(h * a.n_cap + b + i) * kD + c]);
    __syncthreads();
  }
  // D: wavefront sums, then the four in order; N: the two halves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) accD += __shfl_xor(accD, off, 64);
  if ((t & 63) == 0) e.dsum[t >> 6] = accD;
  if (hf == 1) e.half[c] = accN;
  __syncthreads();
  if (t < kD) {
    const double N = accN + e.half[t];
    out[t] = N;
    e.half[t] = N;
  }
  if (t == 0) {
    const double D = (e.dsum[0] + e.dsum[1]) + (e.dsum[2] + e.dsum[3]);
    out[kD] = D;
    e.dsum[0] = D;
  }
  __syncthreads();
}

constexpr int kTailWG = kExactChunks;   // tail workgroups per query head (at least 256 in all)

// What query head hq does in the tail launch of pass a.pass (2 or 3), and how much: the
// pass's candidates (kind = the pass), or, in the final launch, the exact fallback
// (kind 1).  Work units: blocks of 1024 candidates (at most one unit when the certificate
// workgroup can take them all), or the fallback's chunks.  Built from the states the
// earlier launches left, which nothing in this launch changes, so every workgroup sees
// the same plan.
__device__ inline int tail_units(const CertArgs &a, int hq, int &kind) {
  const int s1 = a.flags[hq];
  int i0, i1, nseg;
  kind = 0;
  if (a.pass == 2) {
    if (s1 == 1 && a.final_pass == 2) {
      kind = 1;
      return kExactChunks;
    }
    if (s1 != 2) return 0;
    kind = 2;
    seg_range(a.ccount2[hq], 0, i0, i1, nseg);
    return max(1, nseg);
  }
  const int s2 = (s1 == 2) ? a.flags2[hq] : -1;
  if (s2 == 3) {
    kind = 3;
    seg_range(a.ccount[hq], 0, i0, i1, nseg);
    return max(1, nseg);
  }
  if (s1 == 1 || s2 == 1) {
    kind = 1;
    return kExactChunks;
  }
  return 0;
}

// One launch per later pass (grid of at least 256 workgroups, 256 threads).  Every head
// with work gets its own contiguous group of workgroups, sized by its share of all the
// work units (at least one, at most its own units), and each workgroup of a group takes
// one contiguous range of the head's candidates (or of its keys, for the fallback) and
// writes one partial table; the group's last workgroup to finish (a counter behind a
// device-wide fence) sums the group's tables and runs the certificate, or combines the
// fallback's chunks.  A group of one accumulates everything itself.  A certificate of
// the final pass that finds no level computes the exact output by itself (slow, and
// rare: the final pass covers every level up to J).  Heads with nothing to do cost one
// read of their states.
__global__ __launch_bounds__(256) void tail_kernel(CertArgs a) {
  const int t = threadIdx.x;
  const int nwg = (int)gridDim.x, w = (int)blockIdx.x;
  __shared__ union {
    FinSmem f;
    ExactSmem e;
  } u;
  __shared__ int red[4][2];
  __shared__ int grp[2][256];     // per head of the chunk: group size, group start
  __shared__ int last;
  AccSmem &s = u.f.s;
  int *done = (a.pass == 2) ? a.exdone : a.exdone2;
  // totals over all heads: work units and heads with work
  int units = 0, busy = 0;
  for (int hq = t; hq < a.H_q; hq += 256) {
    int kind;
    const int n = tail_units(a, hq, kind);
    units += n;
    busy += (n > 0);
  }
  // (wavefront totals by DPP prefixes and a lane read)
  units = __builtin_amdgcn_readlane(wave_incl_scan(units), 63);
  busy = __builtin_amdgcn_readlane(wave_incl_scan(busy), 63);
  if ((t & 63) == 0) {
    red[t >> 6][0] = units;
    red[t >> 6][1] = busy;
  }
  __syncthreads();
  const int64_t T = (int64_t)red[0][0] + red[1][0] + red[2][0] + red[3][0];
  const int64_t B = (int64_t)red[0][1] + red[1][1] + red[2][1] + red[3][1];
  if (T == 0) return;
  const int64_t spare = max<int64_t>(0, (int64_t)nwg - B);   // nwg >= H_q >= B
  int64_t start = 0;                                         // first workgroup of this chunk
  for (int h0 = 0; h0 < a.H_q; h0 += 256) {
    __syncthreads();
    int kind = 0;
    const int hq = h0 + t;
    const int n = (hq < a.H_q) ? tail_units(a, hq, kind) : 0;
    const int g = (n > 0) ? (int)max<int64_t>(1, min<int64_t>(n, spare * n / T)) : 0;
    grp[0][t] = g;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {                // inclusive scan of group sizes
      const int v = (t >= off) ? grp[0][t - off] : 0;
      __syncthreads();
      grp[0][t] += v;
      __syncthreads();
    }
    grp[1][t] = (int)start + grp[0][t] - g;                  // this head's first workgroup
    __syncthreads();
    const int64_t chunk_end = start + grp[0][255];
    if (w >= start && w < chunk_end) {
      int lo = 0, hi = 255;                                  // the head: first k with end > w
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (start + grp[0][mid] > w) hi = mid; else lo = mid + 1;
      }
      const int h = h0 + lo;
      const int k = w - grp[1][lo];                          // this workgroup's part
      int k2 = 0;
      tail_units(a, h, k2);
      const int gsz = grp[0][lo] - (lo > 0 ? grp[0][lo - 1] : 0);
      if (k2 == 1) {
        const int64_t nh = head_n(a, h);
        const int64_t len = (nh + gsz - 1) / gsz;
        const int64_t i0 = k * len, i1 = min<int64_t>(nh, i0 + len);
        exact_chunk(a, u.e, h, i0, i1, a.exactp + ((int64_t)h * kExactChunks + k) * 130);
      } else if (gsz > 1) {
        const int count = pass_count(a, h);
        const int len = (count + gsz - 1) / gsz;
        const int i0 = min(count, k * len), i1 = min(count, i0 + len);
        const int J1 = a.J + 1;
        fill_level_pairs(s.ltp, a.lt, a.J, t, 256);
        zero_acc(s, J1);
        accumulate_mixed(a, s, h, i0, i1, record_split(a, h, count));
        double *out = a.partial + ((int64_t)h * a.nseg_cap + k) * J1 * kStatW;
        for (int e = t; e < J1 * kStatW; e += 256) out[e] = (&s.acc[0][0])[e];
      }
      bool run = true;
      if (gsz > 1) {
        __threadfence();
        __syncthreads();
        if (t == 0) last = (atomicAdd(done + h, 1) == gsz - 1);
        __syncthreads();
        run = last;
        if (run) __threadfence();
      }
      if (run) {
        if (k2 == 1) {
          if (t < kD) {
            double N = 0.0, Dn = 0.0;
            for (int c = 0; c < gsz; ++c) {
              const double *p = a.exactp + ((int64_t)h * kExactChunks + c) * 130;
              N += p[t];
              Dn += p[kD];
            }
            a.o_hat[(int64_t)h * kD + t] = (float)(N / Dn);
          }
        } else if (!certify_head<false>(a, u.f, h, gsz > 1 ? gsz : 0, -1, 0, nullptr) && a.pass == a.final_pass) {
          __syncthreads();
          exact_chunk(a, u.e, h, 0, head_n(a, h), a.exactp + (int64_t)h * kExactChunks * 130);
          if (t < kD) a.o_hat[(int64_t)h * kD + t] = (float)(u.e.half[t] / u.e.dsum[0]);
        }
      }
      return;                                                // one part per workgroup
    }
    start = chunk_end;
  }
}

hipError_t launch_certify_pass(CertArgs a, int pass, int H_q, hipStream_t st) {
  a.pass = pass;
  hipLaunchKernelGGL(finish_kernel, dim3(H_q), dim3(256), 0, st, a);
  return hipGetLastError();
}

// The later passes and the exact fallback, in launches that heads certified earlier leave
// at once: one launch when the second pass covers every level (the default), two when a
// second budget splits the remaining levels.
hipError_t launch_tail(CertArgs a, int H_q, bool three_pass, hipStream_t st) {
  // at least one workgroup per query head (every head with work gets its own group)
  const unsigned nwg = (unsigned)max(max(256, H_q), min(4096, H_q * kTailWG));
  a.H_q = H_q;
  a.final_pass = three_pass ? 3 : 2;
  a.pass = 2;
  hipLaunchKernelGGL(tail_kernel, dim3(nwg), dim3(256), 0, st, a);
  if (three_pass) {
    a.pass = 3;
    hipLaunchKernelGGL(tail_kernel, dim3(nwg), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace csa
