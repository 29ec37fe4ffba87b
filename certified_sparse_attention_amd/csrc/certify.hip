// Per-level Horvitz-Thompson sums, certificates, the per-head stop and the exact
// fallback.
//
// "Certified Sparse Attention via Perturbed Retrieval", summary page:
//   Methodology > Algorithm Components item 2: D^ = D_R + D_B + tau k,
//     N^ = N_R + N_B + tau sum_{S & A} v (heavy keys B with w >= tau are always in
//     the sample, light keys A enter with probability w / tau);
//   item 3: on the grid tau_j, a Chernoff interval for the Poisson-binomial sample
//     count, a Hilbert-space Bernstein bound on Z_c = sum_A (tau X - w)(v - c),
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
  int64_t n_cap, n, npool, npool_cap;
  int G, J, W, measure;
  double eps, L;
  const float *qf;
  const double *lt, *tau, *sR;
  const unsigned long long *cstar;
  const unsigned *vmax;
  const int *ccount, *candpos, *rec_hl, *hist, *cmcnt, *cmpos;
  const double *rec_w, *rec_vsq;
  const int8_t *lub;
  double *partial, *stats, *winsum, *betalv, *dhatlv;
  int *klv, *flags;
  double *exactp;
  float *o_hat;
  double *beta;
  int32_t *stop;
  int64_t *keys_read;
  int all_exact;
};

__device__ inline void seg_range(int count, int seg, int &i0, int &i1, int &nseg) {
  nseg = (count <= 0) ? 0 : min(kNumSeg, (count + 255) / 256);
  if (seg >= nseg) { i0 = i1 = 0; return; }
  const int len = (count + nseg - 1) / nseg;
  i0 = seg * len;
  i1 = min(count, i0 + len);
}

// grid (H_q, kNumSeg, 2 channel slices); 64 threads, thread t owns channel 64 slice + t.
__global__ __launch_bounds__(64) void accumulate_kernel(CertArgs a) {
  extern __shared__ double sm[];
  const int hq = blockIdx.x, seg = blockIdx.y, slice = blockIdx.z;
  const int h = hq / a.G, t = threadIdx.x;
  const int J1 = a.J + 1;
  int i0, i1, nseg;
  seg_range(a.ccount[hq], seg, i0, i1, nseg);
  if (seg >= nseg) return;
  double *accN = sm;                 // [J1][64]
  double *accV = sm + J1 * 64;       // [J1][64]
  double *scal = sm + 2 * J1 * 64;   // [J1][4]
  for (int j = 0; j < J1; ++j) {
    accN[j * 64 + t] = 0.0;
    accV[j * 64 + t] = 0.0;
    if (t < 4) scal[j * 4 + t] = 0.0;
  }
  const int64_t base = (int64_t)hq * a.npool_cap;
  const int ch = 64 * slice + t;
  for (int i = i0; i < i1; ++i) {
    const int hl = a.rec_hl[base + i];
    const int hlev = hl & 0xFF, llev = hl >> 8;
    if (llev > a.J) continue;
    const int pos = a.candpos[base + i];
    const double v = h2d(a.V[((int64_t)h * a.n_cap + pos) * kD + ch]);
    const double w = a.rec_w[base + i];
    if (hlev <= a.J) accN[hlev * 64 + t] += w * v;
    if (llev < hlev) {
      accV[llev * 64 + t] += v;
      if (hlev <= a.J) accV[hlev * 64 + t] -= v;
    }
    if (slice == 0 && t < 4) {
      const double vsq = a.rec_vsq[base + i];
      if (t == 0) {
        if (hlev <= a.J) scal[hlev * 4 + 0] += w;
      } else if (t == 1) {
        if (hlev <= a.J) scal[hlev * 4 + 1] += w * vsq;
      } else if (t == 2) {
        if (llev < hlev) {
          scal[llev * 4 + 2] += 1.0;
          if (hlev <= a.J) scal[hlev * 4 + 2] -= 1.0;
        }
      } else {
        if (llev < hlev) {
          scal[llev * 4 + 3] += vsq;
          if (hlev <= a.J) scal[hlev * 4 + 3] -= vsq;
        }
      }
    }
  }
  double *out = a.partial + ((int64_t)hq * kNumSeg + seg) * J1 * kStatW;
  for (int j = 0; j < J1; ++j) {
    out[j * kStatW + ch] = accN[j * 64 + t];
    out[j * kStatW + 128 + ch] = accV[j * 64 + t];
    if (slice == 0 && t < 4) out[j * kStatW + 256 + t] = scal[j * 4 + t];
  }
}

// grid H_q; thread c owns stats component c; fixed order over segments, then levels.
__global__ __launch_bounds__(kStatW) void reduce_kernel(CertArgs a) {
  const int hq = blockIdx.x, c = threadIdx.x;
  const int J1 = a.J + 1;
  int i0, i1, nseg;
  seg_range(a.ccount[hq], 0, i0, i1, nseg);
  double run = 0.0;
  for (int j = 0; j < J1; ++j) {
    double inc = 0.0;
    for (int s = 0; s < nseg; ++s) inc += a.partial[(((int64_t)hq * kNumSeg + s) * J1 + j) * kStatW + c];
    run += inc;
    a.stats[((int64_t)hq * J1 + j) * kStatW + c] = run;
  }
}

// grid H_q, 128 threads: window sums N_R, D_R, Q_R relative to c*.
__global__ __launch_bounds__(128) void window_kernel(CertArgs a) {
  const int hq = blockIdx.x, h = hq / a.G, t = threadIdx.x;
  __shared__ double wv[256], vq[256];
  const int64_t w0 = (a.n > a.W) ? a.n - a.W : 0;
  const int nw = (int)(a.n - w0);
  const double cs = dec_max(a.cstar[hq]);
  double accN = 0.0, accD = 0.0, accQ = 0.0;
  for (int base = 0; base < nw; base += 256) {
    const int cnt = min(256, nw - base);
    for (int i = t; i < cnt; i += 128) {
      wv[i] = exp(a.sR[(int64_t)hq * a.W + base + i] - cs);
      vq[i] = row_sumsq(a.V + ((int64_t)h * a.n_cap + w0 + base + i) * kD);
    }
    __syncthreads();
    for (int i = 0; i < cnt; ++i)
      accN += wv[i] * h2d(a.V[((int64_t)h * a.n_cap + w0 + base + i) * kD + t]);
    if (t == 0)
      for (int i = 0; i < cnt; ++i) {
        accD += wv[i];
        accQ += wv[i] * vq[i];
      }
    __syncthreads();
  }
  a.winsum[(int64_t)hq * 130 + t] = accN;
  if (t == 0) {
    a.winsum[(int64_t)hq * 130 + 128] = accD;
    a.winsum[(int64_t)hq * 130 + 129] = accQ;
  }
}

__device__ inline double kl_div(double x, double mu) {
  return (x > 0.0) ? (mu - x + x * log(x / mu)) : mu;
}
// Root of kl(x, mu) = L above x (Newton from above; convex increasing branch).
__device__ inline double kl_upper(double x, double L) {
  if (!(x > 0.0)) return L;
  double mu = x + L + sqrt(L * L + 2.0 * x * L);
  for (int it = 0; it < 100; ++it) {
    const double f = kl_div(x, mu) - L;
    const double d = 1.0 - x / mu;
    const double nx = mu - f / d;
    if (!(nx < mu)) break;
    mu = nx;
  }
  return mu;
}
// Root of kl(x, mu) = L below x (Newton from below; convex decreasing branch).
__device__ inline double kl_lower(double x, double L) {
  if (!(x > 0.0)) return 0.0;
  double mu = fmax(x - sqrt(2.0 * x * L), x * exp(-1.0 - L / x));
  for (int it = 0; it < 100; ++it) {
    const double f = kl_div(x, mu) - L;
    const double d = 1.0 - x / mu;
    const double nx = mu - f / d;
    if (!(nx > mu) || !(nx < x)) break;
    mu = nx;
  }
  return mu;
}

// grid H_q, 64 threads: lane j computes the certificate of level j.
__global__ __launch_bounds__(64) void certificate_kernel(CertArgs a) {
  const int hq = blockIdx.x, j = threadIdx.x, h = hq / a.G;
  if (j > a.J) return;
  const int J1 = a.J + 1;
  const double *st = a.stats + ((int64_t)hq * J1 + j) * kStatW;
  const double *ws = a.winsum + (int64_t)hq * 130;
  const double tau = a.tau[j], L = a.L;
  const double Vmax = h2d((uint16_t)a.vmax[h]);
  const double D_det = ws[128] + st[256];
  const double Q_det = ws[129] + st[257];
  const double k = st[258], P = st[259];
  const double D_hat = D_det + tau * k;
  const double mu_hi = kl_upper(k, L), mu_lo = kl_lower(k, L);
  const double dD = tau * fmax(k - mu_lo, mu_hi - k);
  const double D_hi = D_det + tau * mu_hi;
  const double inf = __builtin_huge_val();
  double beta;
  if (a.measure == CSA_MEASURE_DENOM) {
    beta = (D_hat > dD) ? dD / (D_hat - dD) : inf;
  } else {
    double cn2 = 0.0, cV = 0.0, dn2 = 0.0, on2 = 0.0;
    for (int t = 0; t < kD; ++t) {
      const double nd = ws[t] + st[t];
      const double c = nd / D_det;
      const double o = (nd + tau * st[128 + t]) / D_hat;
      cn2 += c * c;
      cV += c * st[128 + t];
      dn2 += (o - c) * (o - c);
      on2 += o * o;
    }
    const double cn = sqrt(cn2), Rc = Vmax + cn;
    const double y = (Rc > 0.0) ? fmax((P - 2.0 * cV + k * cn * cn) / (Rc * Rc), 0.0) : 0.0;
    const double mu_G = kl_upper(y, L);
    const double sigma2 = tau * tau * Rc * Rc * mu_G;
    const double zeta = sqrt(2.0 * sigma2 * L) + (2.0 / 3.0) * (tau * Rc) * L;
    const double dn = sqrt(dn2), on = sqrt(on2);
    const double beta_abs = (D_hat > dD) ? (zeta + dn * dD) / (D_hat - dD) : inf;
    if (a.measure == CSA_MEASURE_OUTNORM) {
      beta = (on > beta_abs) ? beta_abs / (on - beta_abs) : inf;
    } else {
      const double yq = (Vmax > 0.0) ? P / (Vmax * Vmax) : 0.0;
      const double mu_Q = kl_lower(yq, L);
      const double Q_lo = Q_det + tau * Vmax * Vmax * mu_Q;
      const double M_lo = fmax(on - beta_abs, sqrt(Q_lo / D_hi));
      beta = (M_lo > 0.0 && beta_abs < inf) ? beta_abs / M_lo : inf;
    }
  }
  a.betalv[(int64_t)hq * J1 + j] = beta;
  a.dhatlv[(int64_t)hq * J1 + j] = D_hat;
  a.klv[(int64_t)hq * J1 + j] = (int)k;
}

// grid H_q, 64 threads (one wavefront): the stop level and the outputs.
__global__ __launch_bounds__(64) void finalize_kernel(CertArgs a) {
  const int hq = blockIdx.x, lane = threadIdx.x;
  if (a.all_exact) {
    if (lane == 0) {
      a.flags[hq] = 1;
      a.stop[hq] = 0;
      a.beta[hq] = 0.0;
      a.keys_read[hq] = a.n;
    }
    return;
  }
  const int J1 = a.J + 1;
  const bool ok = (lane <= a.J) && (a.betalv[(int64_t)hq * J1 + lane] <= a.eps);
  const unsigned long long mask = __ballot(ok);
  const int js = mask ? (__ffsll((long long)mask) - 1) : a.J + 1;
  if (js > a.J) {
    if (lane == 0) {
      a.flags[hq] = 1;
      a.stop[hq] = a.J + 1;
      a.beta[hq] = 0.0;
      a.keys_read[hq] = a.n;
    }
    return;
  }
  const double *st = a.stats + ((int64_t)hq * J1 + js) * kStatW;
  const double *ws = a.winsum + (int64_t)hq * 130;
  const double tau = a.tau[js];
  const double D_hat = (ws[128] + st[256]) + tau * st[258];
  for (int t = lane; t < kD; t += 64)
    a.o_hat[(int64_t)hq * kD + t] = (float)(((ws[t] + st[t]) + tau * st[128 + t]) / D_hat);
  // keys read: window + |{l^ub <= j*}| + |{i in C_max : l^ub_i > j*}|
  int64_t extra = 0;
  const int ncm = a.cmcnt[hq];
  for (int i = lane; i < ncm; i += 64) {
    const int pos = a.cmpos[(int64_t)hq * a.npool_cap + i];
    extra += (a.lub[(int64_t)hq * a.npool_cap + pos] > js);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) extra += __shfl_xor(extra, off, 64);
  if (lane == 0) {
    int64_t inb = 0;
    for (int j = 0; j <= js; ++j) inb += a.hist[(int64_t)hq * (a.J + 2) + j];
    a.flags[hq] = 0;
    a.stop[hq] = js;
    a.beta[hq] = a.betalv[(int64_t)hq * J1 + js];
    a.keys_read[hq] = (int64_t)a.W + inb + extra;
  }
}

// Exact attention for heads flagged for the fallback: grid (H_q, kExactChunks), 128 threads.
__global__ __launch_bounds__(128) void exact_partial_kernel(CertArgs a) {
  const int hq = blockIdx.x, ch = blockIdx.y, t = threadIdx.x, h = hq / a.G;
  if (a.flags[hq] == 0) return;
  __shared__ double qd[kD];
  __shared__ double wv[128], wq[128];
  qd[t] = (double)a.qf[(int64_t)hq * kD + t];
  __syncthreads();
  const double cs = dec_max(a.cstar[hq]);
  const int64_t len = (a.n + kExactChunks - 1) / kExactChunks;
  const int64_t i0 = ch * len, i1 = min(a.n, i0 + len);
  double accN = 0.0, accD = 0.0, accQ = 0.0;
  for (int64_t b = i0; b < i1; b += 128) {
    const int cnt = (int)min<int64_t>(128, i1 - b);
    if (t < cnt) {
      const int64_t pos = b + t;
      const double s = exact_score(qd, a.K + ((int64_t)h * a.n_cap + pos) * kD);
      const double w = exp(s - cs);
      wv[t] = w;
      wq[t] = w * row_sumsq(a.V + ((int64_t)h * a.n_cap + pos) * kD);
    }
    __syncthreads();
    for (int i = 0; i < cnt; ++i) accN += wv[i] * h2d(a.V[((int64_t)h * a.n_cap + b + i) * kD + t]);
    if (t == 0)
      for (int i = 0; i < cnt; ++i) {
        accD += wv[i];
        accQ += wq[i];
      }
    __syncthreads();
  }
  double *out = a.exactp + ((int64_t)hq * kExactChunks + ch) * 130;
  out[t] = accN;
  if (t == 0) {
    out[128] = accD;
    out[129] = accQ;
  }
}

__global__ __launch_bounds__(128) void exact_final_kernel(CertArgs a) {
  const int hq = blockIdx.x, t = threadIdx.x;
  if (a.flags[hq] == 0) return;
  double N = 0.0, Dn = 0.0;
  for (int c = 0; c < kExactChunks; ++c) {
    const double *p = a.exactp + ((int64_t)hq * kExactChunks + c) * 130;
    N += p[t];
    Dn += p[128];
  }
  a.o_hat[(int64_t)hq * kD + t] = (float)(N / Dn);
}

hipError_t launch_certify(const CertArgs &a, int H_q, hipStream_t st) {
  if (!a.all_exact) {
    const size_t shm = (size_t)(a.J + 1) * (2 * 64 + 4) * sizeof(double);
    hipLaunchKernelGGL(accumulate_kernel, dim3(H_q, kNumSeg, 2), dim3(64), shm, st, a);
    hipLaunchKernelGGL(reduce_kernel, dim3(H_q), dim3(kStatW), 0, st, a);
    hipLaunchKernelGGL(window_kernel, dim3(H_q), dim3(128), 0, st, a);
    hipLaunchKernelGGL(certificate_kernel, dim3(H_q), dim3(64), 0, st, a);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(H_q), dim3(64), 0, st, a);
  hipLaunchKernelGGL(exact_partial_kernel, dim3(H_q, kExactChunks), dim3(128), 0, st, a);
  hipLaunchKernelGGL(exact_final_kernel, dim3(H_q), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
