// Dense decode attention o = softmax(q K^T / sqrt(d)) V ("Certified Sparse Attention
// via Perturbed Retrieval", summary page, Methodology > Problem Setup), the
// library's own comparison kernel.  Split over tokens: each workgroup streams one
// token range of one KV head for all G queries of its group with an online
// softmax in fp32; a second pass combines the ranges.
#include "common.h"

namespace csa {

constexpr int kDenseTok = 1024;   // tokens per workgroup

struct DenseArgs {
  const uint16_t *q, *K, *V;
  int64_t n_cap, n;
  int G, nsplit;
  float *part;   // [H_q][nsplit][130]: m, l, acc[128]
  float *o;
};

__global__ __launch_bounds__(256) void dense_split_kernel(DenseArgs a) {
  const int h = blockIdx.x, sp = blockIdx.y;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int G = a.G;
  __shared__ float qs[kMaxG][kD];
  __shared__ float wm[4][kMaxG], wl[4][kMaxG];
  __shared__ float wacc[4][kMaxG][kD];
  for (int i = threadIdx.x; i < G * kD; i += 256)
    qs[i / kD][i % kD] = h2f(a.q[(int64_t)(h * G) * kD + i]) * (float)kRsqrtD;
  __syncthreads();
  const int64_t t0 = (int64_t)sp * kDenseTok, t1 = min(a.n, t0 + kDenseTok);
  float m[kMaxG], l[kMaxG], acc0[kMaxG], acc1[kMaxG];
#pragma unroll
  for (int g = 0; g < kMaxG; ++g) { m[g] = -__builtin_huge_valf(); l[g] = 0.f; acc0[g] = acc1[g] = 0.f; }
  for (int64_t b = t0 + 64 * wv; b < t1; b += 256) {
    const int64_t tok = b + lane;
    float s[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) s[g] = -__builtin_huge_valf();
    if (tok < t1) {
      const uint4 *kr = reinterpret_cast<const uint4 *>(a.K + ((int64_t)h * a.n_cap + tok) * kD);
#pragma unroll
      for (int g = 0; g < kMaxG; ++g) s[g] = 0.f;
#pragma unroll 4
      for (int c = 0; c < 16; ++c) {
        const uint4 w = kr[c];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = h2f((uint16_t)(ww[e] & 0xFFFFu)), k1 = h2f((uint16_t)(ww[e] >> 16));
#pragma unroll
          for (int g = 0; g < kMaxG; ++g)
            if (g < G) s[g] = __builtin_fmaf(qs[g][8 * c + 2 * e + 1], k1, __builtin_fmaf(qs[g][8 * c + 2 * e], k0, s[g]));
        }
      }
    }
    const int cnt = (int)min<int64_t>(64, t1 - b);
    float p[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
      if (g < G) {
        float mx = s[g];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        const float mn = fmaxf(m[g], mx);
        const float sc = __expf(m[g] - mn);
        p[g] = (lane < cnt) ? __expf(s[g] - mn) : 0.f;
        float ps = p[g];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off, 64);
        l[g] = l[g] * sc + ps;
        acc0[g] *= sc;
        acc1[g] *= sc;
        m[g] = mn;
      }
    }
    for (int i = 0; i < cnt; ++i) {
      const uint32_t vv = reinterpret_cast<const uint32_t *>(a.V + ((int64_t)h * a.n_cap + b + i) * kD)[lane];
      const float v0 = h2f((uint16_t)(vv & 0xFFFFu)), v1 = h2f((uint16_t)(vv >> 16));
#pragma unroll
      for (int g = 0; g < kMaxG; ++g) {
        if (g < G) {
          const float pi = __shfl(p[g], i, 64);
          acc0[g] = __builtin_fmaf(pi, v0, acc0[g]);
          acc1[g] = __builtin_fmaf(pi, v1, acc1[g]);
        }
      }
    }
  }
  // combine the four waves
#pragma unroll
  for (int g = 0; g < kMaxG; ++g) {
    if (g < G) {
      if (lane == 0) { wm[wv][g] = m[g]; wl[wv][g] = l[g]; }
      wacc[wv][g][2 * lane] = acc0[g];
      wacc[wv][g][2 * lane + 1] = acc1[g];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * kD; i += 256) {
    const int g = i / kD, c = i % kD;
    float M = -__builtin_huge_valf();
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][g]);
    float Lsum = 0.f, A = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float sc = (wm[w][g] == -__builtin_huge_valf()) ? 0.f : __expf(wm[w][g] - M);
      Lsum += wl[w][g] * sc;
      A += wacc[w][g][c] * sc;
    }
    float *dst = a.part + ((int64_t)(h * G + g) * a.nsplit + sp) * 130;
    dst[2 + c] = A;
    if (c == 0) { dst[0] = M; dst[1] = Lsum; }
  }
}

__global__ __launch_bounds__(128) void dense_combine_kernel(DenseArgs a) {
  const int hq = blockIdx.x, t = threadIdx.x;
  const float *p = a.part + (int64_t)hq * a.nsplit * 130;
  float M = -__builtin_huge_valf();
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, p[s * 130]);
  float L = 0.f, A = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float ms = p[s * 130];
    const float sc = (ms == -__builtin_huge_valf()) ? 0.f : __expf(ms - M);
    L += p[s * 130 + 1] * sc;
    A += p[s * 130 + 2 + t] * sc;
  }
  a.o[(int64_t)hq * kD + t] = A / L;
}

int dense_nsplit(int64_t n) { return (int)((n + kDenseTok - 1) / kDenseTok); }

hipError_t launch_dense(const DenseArgs &a, int H_kv, hipStream_t st) {
  hipLaunchKernelGGL(dense_split_kernel, dim3(H_kv, a.nsplit), dim3(256), 0, st, a);
  hipLaunchKernelGGL(dense_combine_kernel, dim3(H_kv * a.G), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
