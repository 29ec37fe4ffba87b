// Dense decode attention o = softmax(q K^T / sqrt(d)) V ("Certified Sparse Attention
// via Perturbed Retrieval", summary page, Methodology > Problem Setup), the
// library's own comparison kernel.
//
// Split over tokens.  A workgroup (four wavefronts) takes one token range of one KV
// head for all G queries of its group; each wavefront takes every fourth 32-token tile
// of the range:
//   scores: v_mfma_f32_16x16x32_f16 with the tile's keys as the A operand (rows =
//     16 tokens, k = 32 channels; every lane loads its 8 channels of one key row with
//     one 16-byte load, so a tile's 8 KB arrive as 8 loads per lane) and the group's
//     queries as the B operand (columns = queries; G of the 16 columns are used);
//   online softmax per query in fp32 (max and sum across the four lanes that hold a
//     query's scores);
//   values: lane l accumulates channels 8(l%16)..+7 of tokens 4k + l/16 of the tile
//     (one 16-byte load per lane covers four whole rows), with each token's G weights
//     read from LDS as one broadcast, so no per-token cross-lane traffic.
// The four lane groups and four wavefronts are combined in LDS at the end; a second
// kernel combines the ranges of a query head with all of its threads in parallel.
#include "common.h"

namespace csa {

constexpr int kDenseStep = 32;          // tokens per wavefront step
constexpr int kDenseGrain = 4 * kDenseStep;   // token ranges are multiples of this
constexpr int kDenseWGs = 768;          // workgroups that run at once (3 per CU at this
                                        // kernel's register use): one round fills the GPU
constexpr int kDensePart = 2 + kD;      // per (query head, range): m, l, acc[128]

struct DenseArgs {
  const uint16_t *q, *K, *V;
  int64_t n_cap, n;
  int G, nsplit;
  int64_t split_len;   // tokens per workgroup (a multiple of kDenseGrain)
  float *part;   // [H_q][nsplit][kDensePart]
  float *o;
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

__device__ inline half8 as_half8(uint4 v) { return __builtin_bit_cast(half8, v); }

template <int G>
__global__ __launch_bounds__(256) void dense_split_kernel(DenseArgs a) {
  const int sp = blockIdx.x, h = blockIdx.y;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  constexpr float kNegInf = -__builtin_huge_valf();
  __shared__ float pw[4][kDenseStep][8];          // per wavefront: weights p[token][query]
  __shared__ float sc_w[4][8];                    // per wavefront: the step's rescale per query
  __shared__ float mw[4][8], lw[4][8];            // per wavefront: final m and l per query
  __shared__ float accw[4][8][kD];                // per wavefront: final acc per query

  // the queries as the B operand: column col = query, channels 32 s + 8 grp .. + 7
  half8 qb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col < G) v = *reinterpret_cast<const uint4 *>(a.q + (int64_t)(h * G + col) * kD + 32 * s + 8 * grp);
    qb[s] = as_half8(v);
  }
  const int64_t t0 = (int64_t)sp * a.split_len, t1 = min(a.n, t0 + a.split_len);
  const uint16_t *Kh = a.K + (int64_t)h * a.n_cap * kD;
  const uint16_t *Vh = a.V + (int64_t)h * a.n_cap * kD;
  float m = kNegInf, l = 0.0f;      // running max and sum of query `col` (lanes col < G)
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[g][c] = 0.0f;

  for (int64_t base = t0 + kDenseStep * wv; base < t1; base += 4 * kDenseStep) {
    // keys: rows base + 16 u + col, channels 32 s + 8 grp; values: rows base + 4 k + grp,
    // channels 8 col .. + 7.  Rows past n are clamped (their weights are zero).
    uint4 kt[2][4], vt[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t row = min(base + 16 * u + col, a.n - 1);
#pragma unroll
      for (int s = 0; s < 4; ++s) kt[u][s] = *reinterpret_cast<const uint4 *>(Kh + row * kD + 32 * s + 8 * grp);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t row = min(base + 4 * k + grp, a.n - 1);
      vt[k] = *reinterpret_cast<const uint4 *>(Vh + row * kD + 8 * col);
    }
    // scores of the tile: lane holds tokens base + 16 u + 4 grp + i for query col
    float sv[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float4v d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(kt[u][s]), qb[s], d, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t tok = base + 16 * u + 4 * grp + i;
        sv[u][i] = (tok < t1) ? d[i] * (float)kRsqrtD : kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[u][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);                     // finite: the tile holds a token < t1
    const float scale = __expf(m - mn);                // 0 on the first step (m = -inf)
    float ps = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __expf(sv[u][i] - mn);
        ps += p;
        if (col < G) pw[wv][16 * u + 4 * grp + i][col] = p;
      }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l = l * scale + ps;
    m = mn;
    if (lane < G) sc_w[wv][lane] = scale;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // values: rescale, then add p v for the lane's four tokens (one per 16-byte load)
    float scg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) scg[g] = sc_w[wv][g];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[g][c] *= scg[g];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 p0 = *reinterpret_cast<const float4 *>(&pw[wv][4 * k + grp][0]);
      const float4 p1 = *reinterpret_cast<const float4 *>(&pw[wv][4 * k + grp][4]);
      const float pg[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      const half8 vh = as_half8(vt[k]);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float v = (float)vh[c];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g][c] = __builtin_fmaf(pg[g], v, acc[g][c]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // the wavefront's sums over its four lane groups (same scale: m is per wavefront)
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = acc[g][c];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[g][c] = v;
    }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c) accw[wv][g][8 * col + c] = acc[g][c];
  }
  if (lane < G) {
    mw[wv][lane] = m;
    lw[wv][lane] = l;
  }
  __syncthreads();
  // the workgroup's range: the four wavefronts rescaled to their common maximum
  for (int i = threadIdx.x; i < G * kD; i += 256) {
    const int g = i / kD, c = i % kD;
    const float M = fmaxf(fmaxf(mw[0][g], mw[1][g]), fmaxf(mw[2][g], mw[3][g]));
    float A = 0.0f, Ls = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (mw[w][g] == kNegInf) ? 0.0f : __expf(mw[w][g] - M);
      A += accw[w][g][c] * f;
      Ls += lw[w][g] * f;
    }
    float *dst = a.part + ((int64_t)(h * G + g) * a.nsplit + sp) * kDensePart;
    dst[2 + c] = A;
    if (c == 0) {
      dst[0] = M;
      dst[1] = Ls;
    }
  }
}

// One workgroup of 1024 threads per query head: thread t takes channel t % 128 of the
// ranges t / 128, t / 128 + 8, ...; range maxima and weights first, then the eight
// partial sums per channel are added in LDS.
__global__ __launch_bounds__(1024) void dense_combine_kernel(DenseArgs a) {
  const int hq = blockIdx.x, t = threadIdx.x;
  const int c = t & (kD - 1), part = t >> 7;
  const float *p = a.part + (int64_t)hq * a.nsplit * kDensePart;
  __shared__ float red[32];
  __shared__ float accs[8][kD + 1];
  __shared__ float ls[8];
  float M = -__builtin_huge_valf();
  for (int s = t; s < a.nsplit; s += 1024) M = fmaxf(M, p[(int64_t)s * kDensePart]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if ((t & 63) == 0) red[t >> 6] = M;
  __syncthreads();
  M = red[0];
  for (int w = 1; w < 16; ++w) M = fmaxf(M, red[w]);
  float A = 0.0f, L = 0.0f;
  for (int s = part; s < a.nsplit; s += 8) {
    const float ms = p[(int64_t)s * kDensePart];
    const float f = (ms == -__builtin_huge_valf()) ? 0.0f : __expf(ms - M);
    A += p[(int64_t)s * kDensePart + 2 + c] * f;
    L += p[(int64_t)s * kDensePart + 1] * f;
  }
  accs[part][c] = A;
  if (c == 0) ls[part] = L;
  __syncthreads();
  if (t < kD) {
    float As = 0.0f, Ls = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      As += accs[q][t];
      Ls += ls[q];
    }
    a.o[(int64_t)hq * kD + t] = As / Ls;
  }
}

// Tokens per workgroup: the smallest multiple of kDenseGrain that keeps the grid within
// one round of kDenseWGs workgroups (so at most ceil(kDenseWGs / H_kv) ranges per head).
int64_t dense_split_len(int64_t n, int H_kv) {
  const int64_t per = (n * H_kv + kDenseWGs - 1) / kDenseWGs;
  const int64_t len = (per + kDenseGrain - 1) / kDenseGrain * kDenseGrain;
  return len < kDenseGrain ? kDenseGrain : len;
}
int dense_nsplit(int64_t n, int H_kv) {
  const int64_t len = dense_split_len(n, H_kv);
  return (int)((n + len - 1) / len);
}
// Most ranges any n <= n_max can use (the workspace bound).
int dense_nsplit_max(int64_t n_max, int H_kv) {
  const int64_t by_len = (n_max + kDenseGrain - 1) / kDenseGrain;
  const int64_t by_wgs = (kDenseWGs + H_kv - 1) / H_kv;
  return (int)(by_len < by_wgs ? by_len : by_wgs);
}

hipError_t launch_dense(const DenseArgs &a, int H_kv, hipStream_t st) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)H_kv);
  switch (a.G) {
    case 1: hipLaunchKernelGGL(dense_split_kernel<1>, grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(dense_split_kernel<2>, grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL(dense_split_kernel<3>, grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(dense_split_kernel<4>, grid, dim3(256), 0, st, a); break;
    case 5: hipLaunchKernelGGL(dense_split_kernel<5>, grid, dim3(256), 0, st, a); break;
    case 6: hipLaunchKernelGGL(dense_split_kernel<6>, grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL(dense_split_kernel<7>, grid, dim3(256), 0, st, a); break;
  }
  hipLaunchKernelGGL(dense_combine_kernel, dim3(H_kv * a.G), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
