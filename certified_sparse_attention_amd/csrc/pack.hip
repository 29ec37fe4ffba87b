// 4-bit per-block, per-channel key quantization with error-bound metadata, and the
// per-token 8-bit refinement copy ("Certified Sparse Attention via Perturbed
// Retrieval", summary page, Methodology > Algorithm Components item 4: 4-bit
// per-block-per-channel keys that give deterministic score bounds; an 8-bit
// refinement before exact reads).  The rules (zero points on a per-block
// power-of-two grid, round-to-nearest scales, round-up norm bounds) are stated in
// csa.h next to the packed layout.
//
// One workgroup of 128 threads per (KV head, block); thread t owns channel t.
#include "common.h"

namespace csa {

struct PackArgs {
  const uint16_t *K, *V;
  uint8_t *codes;
  uint16_t *kscale;
  int8_t *zq;
  BlockMeta *bmeta;
  uint16_t *kerr, *vnorm;
  int8_t *codes8;
  float *scale8;
  uint16_t *kerr8;
  int64_t n_cap, nb_cap, block_begin;
};

__global__ __launch_bounds__(128) void pack_kernel(PackArgs a) {
  const int t = threadIdx.x;
  const int64_t b = a.block_begin + blockIdx.x;
  const int h = blockIdx.y;
  const int64_t tok0 = b * kBlk;
  const uint16_t *Kb = a.K + ((int64_t)h * a.n_cap + tok0) * kD;
  const uint16_t *Vb = a.V + ((int64_t)h * a.n_cap + tok0) * kD;

  __shared__ double red[128];
  __shared__ double sq[kBlk][kD + 1];
  __shared__ uint8_t cd[kBlk][kD];
  __shared__ int zi[kD];
  __shared__ double sh_kappa;
  __shared__ double s8sh[kBlk];

  double k[kBlk];
  double mn = 1e300, mx = -1e300;
#pragma unroll
  for (int i = 0; i < kBlk; ++i) {
    k[i] = h2d(Kb[(int64_t)i * kD + t]);
    mn = fmin(mn, k[i]);
    mx = fmax(mx, k[i]);
  }
  // A = max_t |mn_t|; kappa = 2^(y-11) with A = f 2^y, f in [0.5, 1).
  red[t] = fabs(mn);
  __syncthreads();
  if (t == 0) {
    double A = 0.0;
    for (int i = 0; i < kD; ++i) A = fmax(A, red[i]);
    int kexp = 0;
    if (A > 0.0) {
      int y;
      (void)frexp(A, &y);
      kexp = y - 11;
    }
    sh_kappa = ldexp(1.0, kexp);
    a.bmeta[(int64_t)h * a.nb_cap + b].kexp = kexp;
    red[0] = A;  // reused below only by t == 0
  }
  __syncthreads();
  const double kappa = sh_kappa;
  const double A = red[0];
  __syncthreads();
  const double z = (A > 0.0) ? floor(mn / kappa) : 0.0;
  const double kmin = kappa * z;
  const uint16_t ks16 = d2h_rne((mx - kmin) / 15.0);
  const double ks = h2d(ks16);
  a.kscale[((int64_t)h * a.nb_cap + b) * kD + t] = ks16;
  const int zv = (int)z;
  const int z1 = (zv + 64) >> 7;
  const int z0 = zv - 128 * z1;
  a.zq[(((int64_t)h * a.nb_cap + b) * 2 + 0) * kD + t] = (int8_t)z1;
  a.zq[(((int64_t)h * a.nb_cap + b) * 2 + 1) * kD + t] = (int8_t)z0;
  zi[t] = zv;

#pragma unroll
  for (int i = 0; i < kBlk; ++i) {
    double c = 0.0;
    if (ks > 0.0) c = fmin(fmax(rint((k[i] - kmin) / ks), 0.0), 15.0);
    cd[i][t] = (uint8_t)c;
    double r = k[i] - (kmin + ks * c);
    sq[i][t] = r * r;
  }
  // per-block metadata: ksmax, Z1, Kmax (rounded up to fp32)
  red[t] = ks;
  __syncthreads();
  if (t == 0) {
    double m = 0.0;
    for (int i = 0; i < kD; ++i) m = fmax(m, red[i]);
    a.bmeta[(int64_t)h * a.nb_cap + b].ksmax = (float)m;   // an fp16 value: exact
  }
  __syncthreads();
  red[t] = fabs(kmin) + 15.0 * ks;
  __syncthreads();
  if (t == 0) {
    double m = 0.0;
    int zsum = 0;
    for (int i = 0; i < kD; ++i) {
      m = fmax(m, red[i]);
      zsum += abs(zi[i]);
    }
    a.bmeta[(int64_t)h * a.nb_cap + b].kmax = f32_up(m);
    a.bmeta[(int64_t)h * a.nb_cap + b].z1sum = zsum;
  }
  __syncthreads();
  // kerr: token thread sums its residual squares in the R1 order
  if (t < kBlk) {
    const double *row = sq[t];
    double s = canon_sum([&](int c) { return row[c]; });
    a.kerr[(int64_t)h * a.n_cap + tok0 + t] = f16_sqrt_up(s * (1.0 + kPadF));
  }
  __syncthreads();
  // the 8-bit copy, per token: scale8 = fp32(max_t |k| / 127), codes rint(k / scale8)
  // clamped to [-127, 127], kerr8 from the residual squares in the R1 order
#pragma unroll
  for (int i = 0; i < kBlk; ++i) sq[i][t] = fabs(k[i]);
  __syncthreads();
  if (t < kBlk) {
    double m = 0.0;
    for (int c = 0; c < kD; ++c) m = fmax(m, sq[t][c]);
    const float sc = (float)(m / 127.0);
    a.scale8[(int64_t)h * a.n_cap + tok0 + t] = sc;
    s8sh[t] = (double)sc;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kBlk; ++i) {
    const double sc = s8sh[i];
    const double c8 = (sc > 0.0) ? fmin(fmax(rint(k[i] / sc), -127.0), 127.0) : 0.0;
    a.codes8[((int64_t)h * a.n_cap + tok0 + i) * kD + t] = (int8_t)c8;
    const double r = k[i] - sc * c8;
    sq[i][t] = r * r;
  }
  __syncthreads();
  if (t < kBlk) {
    const double *row = sq[t];
    double s = canon_sum([&](int c) { return row[c]; });
    a.kerr8[(int64_t)h * a.n_cap + tok0 + t] = f16_sqrt_up(s * (1.0 + kPadF));
  }
  __syncthreads();
  // vnorm
#pragma unroll
  for (int i = 0; i < kBlk; ++i) {
    double v = h2d(Vb[(int64_t)i * kD + t]);
    sq[i][t] = v * v;
  }
  __syncthreads();
  if (t < kBlk) {
    const double *row = sq[t];
    double s = canon_sum([&](int c) { return row[c]; });
    a.vnorm[(int64_t)h * a.n_cap + tok0 + t] = f16_sqrt_up(s * (1.0 + kPadF));
  }
  // codes in the scan's operand layout: thread th writes chunk th (16 bytes):
  // half-block tile T = th / 64, token n = th % 16, channel group g = (th % 64) / 16.
  {
    const int T = t >> 6, l = t & 63, n = l & 15, g = l >> 4;
    const int i = 16 * T + n;
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t acc = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int jj = 4 * d + j;
        uint32_t byte = (uint32_t)cd[i][32 * g + jj] | ((uint32_t)cd[i][32 * g + 16 + jj] << 4);
        acc |= byte << (8 * j);
      }
      w[d] = acc;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(a.codes + ((int64_t)h * a.nb_cap + b) * 2048) + t;
    *dst = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_pack(const csa_shape &s, const uint16_t *K, const uint16_t *V, int64_t b0,
                       int64_t b1, const csa_packed &p, hipStream_t st) {
  if (b1 <= b0) return hipSuccess;
  PackArgs a;
  a.K = K;
  a.V = V;
  a.codes = p.codes;
  a.kscale = p.kscale;
  a.zq = p.zq;
  a.bmeta = reinterpret_cast<BlockMeta *>(p.bmeta);
  a.kerr = p.kerr;
  a.vnorm = p.vnorm;
  a.codes8 = p.codes8;
  a.scale8 = p.scale8;
  a.kerr8 = p.kerr8;
  a.n_cap = s.n_cap;
  a.nb_cap = s.n_cap / kBlk;
  a.block_begin = b0;
  dim3 grid((unsigned)(b1 - b0), (unsigned)s.num_kv_heads);
  hipLaunchKernelGGL(pack_kernel, grid, dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
