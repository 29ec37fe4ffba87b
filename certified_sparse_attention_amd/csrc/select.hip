// Exact maximum, level buckets and exact rescoring of candidates.
//
// "Certified Sparse Attention via Perturbed Retrieval", summary page, Methodology >
// Algorithm Components item 4: the exact maximum is computed over a small part of
// the pool; candidates are bucketed by their earliest possible inclusion level and
// only keys that may enter the sample get exact 16-bit reads.  Item 1: the sample
// at threshold tau is {i in P : s_i - c* + E_i >= log tau}.
//
//   c_lo  = max(c_R, max_P LB);  C_max = {i in P : UB_i >= c_lo}
//   c*    = max(c_R, max_{C_max} s_i)
//   l^ub  = first((UB + E) - c*)   (bucket; candidates are l^ub <= J)
//   h     = first(s - c*), l = first((s + E) - c*), w = exp(s - c*) for candidates
#include "common.h"

namespace csa {

struct SelectArgs {
  const uint16_t *K, *V;
  int64_t n_cap, npool, npool_cap, ntiles;
  int G, J;
  const float *qf;
  const double *lt;
  const uint64_t *prefix;
  const double *pbuf, *ubuf;
  unsigned long long *clo, *cstar;
  int *cmcnt, *cmpos;
  int *hist, *tilecnt, *tileoff, *ccount;
  int8_t *lub;
  int *candpos;
  double *rec_s, *rec_w, *rec_vsq;
  int *rec_hl;
};

// ---- exact maximum over C_max
__global__ __launch_bounds__(256) void cmax_kernel(SelectArgs a) {
  const int hq = blockIdx.x;
  const int h = hq / a.G;
  __shared__ double qd[kD];
  __shared__ double red[256];
  if (threadIdx.x < kD) qd[threadIdx.x] = (double)a.qf[(int64_t)hq * kD + threadIdx.x];
  __syncthreads();
  const double clo = dec_max(a.clo[hq]);
  double m = -__builtin_huge_val();
  for (int64_t pos = (int64_t)blockIdx.y * 256 + threadIdx.x; pos < a.npool;
       pos += (int64_t)gridDim.y * 256) {
    if (a.ubuf[(int64_t)hq * a.npool_cap + pos] >= clo) {
      const double s = exact_score(qd, a.K + ((int64_t)h * a.n_cap + pos) * kD);
      m = fmax(m, s);
      const int idx = atomicAdd(a.cmcnt + hq, 1);
      a.cmpos[(int64_t)hq * a.npool_cap + idx] = (int)pos;
    }
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0 && red[0] > -__builtin_huge_val()) atomicMax(a.cstar + hq, enc_max(red[0]));
}

// ---- buckets: count per tile and histogram of l^ub
__global__ __launch_bounds__(256) void bucket_count_kernel(SelectArgs a) {
  const int hq = blockIdx.x;
  const int64_t tile = blockIdx.y;
  __shared__ int hist[kMaxJ + 2];
  __shared__ int cnt;
  for (int j = threadIdx.x; j < a.J + 2; j += 256) hist[j] = 0;
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();
  const double cs = dec_max(a.cstar[hq]);
  int mine = 0;
  for (int k = 0; k < 4; ++k) {
    const int64_t pos = tile * kBucketTile + 4 * threadIdx.x + k;
    if (pos < a.npool) {
      const int l = first_level(a.pbuf[(int64_t)hq * a.npool_cap + pos] - cs, a.lt, a.J);
      a.lub[(int64_t)hq * a.npool_cap + pos] = (int8_t)l;
      atomicAdd(&hist[l], 1);
      mine += (l <= a.J);
    }
  }
  atomicAdd(&cnt, mine);
  __syncthreads();
  for (int j = threadIdx.x; j < a.J + 2; j += 256)
    if (hist[j]) atomicAdd(a.hist + (int64_t)hq * (a.J + 2) + j, hist[j]);
  if (threadIdx.x == 0) a.tilecnt[(int64_t)hq * a.ntiles + tile] = cnt;
}

__global__ __launch_bounds__(64) void bucket_scan_kernel(SelectArgs a) {
  const int hq = blockIdx.x;
  if (threadIdx.x != 0) return;
  int run = 0;
  for (int64_t t = 0; t < a.ntiles; ++t) {
    a.tileoff[(int64_t)hq * a.ntiles + t] = run;
    run += a.tilecnt[(int64_t)hq * a.ntiles + t];
  }
  a.ccount[hq] = run;
}

// Stable compaction: thread k owns positions 4k..4k+3 of the tile.
__global__ __launch_bounds__(256) void bucket_write_kernel(SelectArgs a) {
  const int hq = blockIdx.x;
  const int64_t tile = blockIdx.y;
  __shared__ int pre[256];
  int flags = 0, mine = 0;
  for (int k = 0; k < 4; ++k) {
    const int64_t pos = tile * kBucketTile + 4 * threadIdx.x + k;
    if (pos < a.npool && a.lub[(int64_t)hq * a.npool_cap + pos] <= a.J) {
      flags |= 1 << k;
      ++mine;
    }
  }
  pre[threadIdx.x] = mine;
  __syncthreads();
  // inclusive Hillis-Steele scan over 256 counts
  for (int off = 1; off < 256; off <<= 1) {
    const int v = ((int)threadIdx.x >= off) ? pre[threadIdx.x - off] : 0;
    __syncthreads();
    pre[threadIdx.x] += v;
    __syncthreads();
  }
  int out = a.tileoff[(int64_t)hq * a.ntiles + tile] + pre[threadIdx.x] - mine;
  for (int k = 0; k < 4; ++k)
    if (flags & (1 << k)) a.candpos[(int64_t)hq * a.npool_cap + out++] = (int)(tile * kBucketTile + 4 * threadIdx.x + k);
}

// ---- exact rescore of candidates (one lane per candidate)
__global__ __launch_bounds__(256) void rescore_kernel(SelectArgs a) {
  const int hq = blockIdx.x;
  const int h = hq / a.G;
  __shared__ double qd[kD];
  if (threadIdx.x < kD) qd[threadIdx.x] = (double)a.qf[(int64_t)hq * kD + threadIdx.x];
  __syncthreads();
  const int cnt = a.ccount[hq];
  const double cs = dec_max(a.cstar[hq]);
  const uint64_t prefix = a.prefix[h];
  for (int64_t i = (int64_t)blockIdx.y * 256 + threadIdx.x; i < cnt; i += (int64_t)gridDim.y * 256) {
    const int64_t o = (int64_t)hq * a.npool_cap + i;
    const int pos = a.candpos[o];
    const double s = exact_score(qd, a.K + ((int64_t)h * a.n_cap + pos) * kD);
    const double E = perturbation(prefix, pos);
    const int hl = first_level(s - cs, a.lt, a.J);
    const int ll = first_level((s + E) - cs, a.lt, a.J);
    double vsq = 0.0;
    if (ll <= a.J) vsq = row_sumsq(a.V + ((int64_t)h * a.n_cap + pos) * kD);
    a.rec_s[o] = s;
    a.rec_w[o] = exp(s - cs);
    a.rec_vsq[o] = vsq;
    a.rec_hl[o] = hl | (ll << 8);
  }
}

hipError_t launch_select(const SelectArgs &a, int H_q, hipStream_t st) {
  const int64_t cmc = (a.npool + 255) / 256;
  const unsigned cm_chunks = (unsigned)(cmc < 64 ? cmc : 64);
  hipLaunchKernelGGL(cmax_kernel, dim3(H_q, cm_chunks), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bucket_count_kernel, dim3(H_q, (unsigned)a.ntiles), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(H_q), dim3(64), 0, st, a);
  hipLaunchKernelGGL(bucket_write_kernel, dim3(H_q, (unsigned)a.ntiles), dim3(256), 0, st, a);
  hipLaunchKernelGGL(rescore_kernel, dim3(H_q, 64), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
