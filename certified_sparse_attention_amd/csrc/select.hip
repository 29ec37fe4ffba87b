// Exact maximum, level buckets and exact rescoring of candidates.
//
// "Certified Sparse Attention via Perturbed Retrieval", summary page, Methodology >
// Algorithm Components item 4: the exact maximum is computed over a small part of
// the pool; candidates are grouped by the first level at which they could be sampled,
// and 16-bit keys are read only for candidates.  Item 1: the sample
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
  int64_t n_cap, npool_cap, ntiles;   // ntiles: the longest item's tiles (row stride)
  int G, J, W;
  Batch b;
  const float *qf;
  const double *lt;
  const uint64_t *prefix;
  const double *pbuf, *ubuf;
  unsigned long long *clo, *cstar;
  int *hist, *tilecnt, *tileoff, *ccount;
  int8_t *lub;
  int *candpos;
  const uint32_t *live;   // [H_q][nwords] keys the scan kept (others have l^ub = J+1, UB < c_lo)
  int64_t nwords;
  int full_lub;           // write l^ub for every pool key (diagnostics)
  int *tilehist;          // [H_q][ntiles][J+2] per-tile cumulative counts of l^ub
  int *tileoff2;          // [H_q][ntiles] offsets of the second range
  int *ccount1, *jspec;   // [H_q] end of the first range and its deepest level
  int *ccount2, *jspec2;  // [H_q] end of the second range and its deepest level
  int *bdone;             // [H_q] tiles whose histogram is written
  int *tilecm;            // [H_q][ntiles][J+2] C_max keys per level and tile
  int *cmhist;            // [H_q][J+2] C_max keys per level
  const int *flags;
  int budget;             // candidates rescored before the first certificate pass
  int budget2;            // candidates (all ranges so far) before the third pass
  int pass;
};

// ---- buckets.  A tile is 64 bitmap words (2048 positions).
constexpr int kDenseTile = 512;   // live keys above which a tile's candidates are written in rounds
// Per tile: cumulative level counts tilehist[tile][j] = |{l^ub <= j}| (j = 0..J+1, the
// last one counting every pool key of the tile) and the C_max keys per level.
__global__ __launch_bounds__(64) void bucket_count_kernel(SelectArgs a) {
  const int hq = blockIdx.x, lane = threadIdx.x;
  const int64_t tile = blockIdx.y;
  // (tiles past this unit's pool find no valid keys: their rows are written as zeros and
  // never read)
  const int64_t npool = unit_npool(a.b, hq / a.G, a.W);
  __shared__ int hist[kMaxJ + 2], cmh[kMaxJ + 2];
  __shared__ double2 ltp[kMaxJ + 2];
  // this lane's bitmap word (tile word `lane`, read at a clamped position and masked
  // below), c* and c_lo are read together with the level table
  const int64_t p_tile = tile * 2048;
  const uint32_t rawword = a.live[(int64_t)hq * a.nwords + min(tile * 64 + lane, a.nwords - 1)];
  const unsigned long long cs_enc = a.cstar[hq], clo_enc = a.clo[hq];
  for (int j = lane; j < a.J + 2; j += 64) {
    hist[j] = 0;
    cmh[j] = 0;
  }
  fill_level_pairs(ltp, a.lt, a.J, lane, 64);
  __syncthreads();
  const double cs = dec_max(cs_enc);
  const double clo = dec_max(clo_enc);
  const double inv_l1 = (a.J >= 1) ? 1.0 / ltp[1].y : 0.0;
  // the word gives the dead count and the bits the lanes read below through shuffles
  const int valid = (int)max<int64_t>(0, min<int64_t>(32, npool - p_tile - 32 * lane));
  const uint32_t word = rawword & ((valid == 32) ? 0xFFFFFFFFu : ((1u << valid) - 1u));
  const int dead = valid - __popc(word);
  if (dead) atomicAdd(&hist[a.J + 1], dead);
  // positions p_tile + 64 k + lane, k = 0..31: lane reads bit (lane & 31) of tile word
  // 2k + (lane >> 5), so every load and store of a round covers 64 consecutive keys
  const bool any = __ballot(word != 0u) != 0ull;
  if (any || a.full_lub) {
    const double *pb = a.pbuf + (int64_t)hq * a.npool_cap + p_tile;
    const double *ubp = a.ubuf + (int64_t)hq * a.npool_cap + p_tile;
    int8_t *lub = a.lub + (int64_t)hq * a.npool_cap + p_tile;
    const int64_t left = npool - p_tile;
    uint32_t on = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t wk = (uint32_t)__shfl((int)word, 2 * k + (lane >> 5), 64);
      on |= ((wk >> (lane & 31)) & 1u) << k;
    }
    // all loads of the lane's live keys first, then the levels
    double pv[32], uv[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const bool o = ((on >> k) & 1u) != 0u;
      pv[k] = o ? pb[64 * k + lane] : 0.0;
      uv[k] = o ? ubp[64 * k + lane] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int i = 64 * k + lane;
      if ((on >> k) & 1u) {
        const int l = level_of_pairs(pv[k] - cs, ltp, a.J, inv_l1);
        lub[i] = (int8_t)l;
        atomicAdd(&hist[l], 1);
        if (uv[k] >= clo) atomicAdd(&cmh[l], 1);
      } else if (a.full_lub && i < left) {
        lub[i] = (int8_t)(a.J + 1);
      }
    }
  }
  __syncthreads();
  // inclusive prefix over levels (lane = level)
  if (lane < a.J + 2) {
    int c = hist[lane];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(c, off, 64);
      if (lane >= off) c += y;
    }
    a.tilehist[((int64_t)hq * a.ntiles + tile) * (a.J + 2) + lane] = c;
    a.tilecm[((int64_t)hq * a.ntiles + tile) * (a.J + 2) + lane] = cmh[lane];
  }
}

// Entry `lane` of rows of width w, summed over the ntiles tiles (*all) and over the tiles
// before `upto` (*before).  Buffer loads keep 64 tiles' loads in flight at a time; the
// per-lane offset carries the tile, so reads past the last tile are out of the buffer's
// range and return 0.
__device__ inline void sum_tiles(const int *base, int64_t ntiles, int w, int lane, int64_t upto, int *all,
                                 int *before) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)(ntiles * w * 4), kBufDword3);
  int cum = 0, pre = 0;
  for (int64_t g0 = 0; g0 < ntiles; g0 += 64) {
    int v[64];
#pragma unroll
    for (int k = 0; k < 64; ++k)
      v[k] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)((g0 + k) * w * 4) + lane * 4, 0, 0);
#pragma unroll
    for (int k = 0; k < 64; ++k) {
      cum += v[k];
      pre += (g0 + k < upto) ? v[k] : 0;
    }
  }
  *all = cum;
  *before = pre;
}

// Stable compaction of the three ranges (l^ub <= j1, then j1 < l^ub <= j2, then
// j2 < l^ub <= J, each in position order): thread = bitmap word.  Every tile's workgroup
// sums the head's tile histograms itself (they are small and L2-resident), which gives the
// level histogram, the speculative levels (j1 the deepest level whose cumulative candidate
// count fits the budget, j2 > j1 the deepest one within the second budget) and, from the
// tiles before it, the tile's offsets without a separate pass.
__global__ __launch_bounds__(64) void bucket_write_kernel(SelectArgs a) {
  const int hq = blockIdx.x, lane = threadIdx.x;
  const int64_t tile = blockIdx.y;
  const int J = a.J, J2 = J + 2;
  const int64_t npool = unit_npool(a.b, hq / a.G, a.W);
  const int64_t ntiles = (npool + kBucketTile - 1) / kBucketTile;   // this unit's tiles
  if (tile > 0 && tile >= ntiles) return;   // (tile 0 writes the head's totals, also of an empty pool)
  const int *th0 = a.tilehist + (int64_t)hq * a.ntiles * J2;
  // this lane's bitmap word (tile word `lane`) and its 32 levels are read together with
  // the histograms (unconditional reads at clamped positions; words past the pool are
  // masked out below, and the levels of keys that are not live are not used)
  const int64_t wi = tile * 64 + lane;
  const int64_t p0 = wi * 32;
  const int64_t p_tile = tile * 2048;
  const uint32_t word = a.live[(int64_t)hq * a.nwords + min(wi, a.nwords - 1)];
  const int valid = (int)max<int64_t>(0, min<int64_t>(32, npool - p0));
  const uint32_t bits = word & ((valid == 32) ? 0xFFFFFFFFu : ((1u << valid) - 1u));
  // a tile without live keys has no candidate to place (tile 0 still writes the totals)
  if (tile > 0 && __ballot(bits != 0u) == 0ull) return;
  const uint4 *lw = reinterpret_cast<const uint4 *>(a.lub + (int64_t)hq * a.npool_cap + min(p0, a.npool_cap - 32));
  const uint4 lv0 = lw[0], lv1 = lw[1];
  // cumulative level histogram of the head and of the tiles before this one (lane = level)
  int cum = 0, pre = 0;
  if (lane < J2) sum_tiles(th0, ntiles, J2, lane, tile, &cum, &pre);
  // the levels that fit form a prefix 0..js (cumulative counts only grow); js = -1 when
  // level 0 alone exceeds the budget, and the first pass then has no candidates
  const unsigned long long fit = __ballot(lane <= J && cum <= a.budget);
  const int js = __popcll(fit) - 1;
  const unsigned long long fit2 = __ballot(lane <= J && cum <= a.budget2);
  const int js2 = min(J, max(js + 1, __popcll(fit2) - 1));       // at least one level past j1
  const int tot1v = __shfl(cum, max(js, 0), 64), totJ = __shfl(cum, J, 64);
  const int pre1v = __shfl(pre, max(js, 0), 64), preJ = __shfl(pre, J, 64);
  const int tot2 = __shfl(cum, js2, 64), pre2 = __shfl(pre, js2, 64);
  const int tot1 = (js >= 0) ? tot1v : 0;
  if (tile == 0) {
    const int below = __shfl_up(cum, 1, 64);
    if (lane < J2) a.hist[(int64_t)hq * J2 + lane] = cum - (lane > 0 ? below : 0);
    if (lane == 0) {
      a.jspec[hq] = js;
      a.ccount1[hq] = tot1;
      a.jspec2[hq] = js2;
      a.ccount2[hq] = tot2;
      a.ccount[hq] = totJ;
    }
    // C_max keys per bucket level
    if (lane < J2) {
      int cm = 0, unused = 0;
      sum_tiles(a.tilecm + (int64_t)hq * a.ntiles * J2, ntiles, J2, lane, 0, &cm, &unused);
      a.cmhist[(int64_t)hq * J2 + lane] = cm;
    }
  }
  // this tile's offsets: candidates of each range in the earlier tiles
  const int b1 = (js >= 0) ? pre1v : 0;
  const int b2 = pre2 - b1;
  const int b3 = preJ - pre2;
  int *dst = a.candpos + (int64_t)hq * a.npool_cap;
  int tile_live = __popc(bits);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tile_live += __shfl_xor(tile_live, off, 64);
  if (tile_live > kDenseTile) {
    // a dense tile (a near-flat head): round k, lane i takes position p_tile + 64 k + i,
    // whose bit is bit (i & 31) of tile word 2k + (i >> 5); each round's candidates of
    // either range are consecutive in position order and go out in one store instruction.
    // The levels are read again in that layout (byte buffer loads, range checked).
    const __amdgpu_buffer_rsrc_t rs_lub = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.lub + (int64_t)hq * a.npool_cap + p_tile), (short)0,
        (int)max<int64_t>(0, a.npool_cap - p_tile), kBufDword3);
    int lv[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) lv[k] = (int)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(rs_lub, 64 * k + lane, 0, 0);
    int o1 = b1, o2 = tot1 + b2, o3 = tot2 + b3;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t wk = (uint32_t)__shfl((int)bits, 2 * k + (lane >> 5), 64);
      const bool on = ((wk >> (lane & 31)) & 1u) != 0u;
      const int l = lv[k];
      const bool in1 = on && l <= js, in2 = on && l > js && l <= js2, in3 = on && l > js2 && l <= J;
      const unsigned long long m1 = __ballot(in1), m2 = __ballot(in2), m3 = __ballot(in3);
      const int r1 = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m1 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m1, 0u));
      const int r2 = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m2 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m2, 0u));
      const int r3 = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m3 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m3, 0u));
      const int pos = (int)(p_tile + 64 * k + lane);
      if (in1) dst[o1 + r1] = pos;
      if (in2) dst[o2 + r2] = pos;
      if (in3) dst[o3 + r3] = pos;
      o1 += __popcll(m1);
      o2 += __popcll(m2);
      o3 += __popcll(m3);
    }
    return;
  }
  // a sparse tile: thread = bitmap word, its candidates in bit order after the earlier words'
  uint32_t m1 = 0, m2 = 0, m3 = 0;
  if (bits) {
    const uint32_t wds[8] = {lv0.x, lv0.y, lv0.z, lv0.w, lv1.x, lv1.y, lv1.z, lv1.w};
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      if ((bits >> b) & 1u) {
        const int l = (int)(int8_t)((wds[b >> 2] >> (8 * (b & 3))) & 0xFFu);
        if (l <= js) m1 |= 1u << b;
        else if (l <= js2) m2 |= 1u << b;
        else if (l <= J) m3 |= 1u << b;
      }
    }
  }
  const int n1 = __popc(m1), n2 = __popc(m2), n3 = __popc(m3);
  // exclusive prefix over the 64 lanes
  int x1 = n1, x2 = n2, x3 = n3;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y1 = __shfl_up(x1, off, 64), y2 = __shfl_up(x2, off, 64), y3 = __shfl_up(x3, off, 64);
    if (lane >= off) { x1 += y1; x2 += y2; x3 += y3; }
  }
  int o1 = b1 + x1 - n1;
  int o2 = tot1 + b2 + x2 - n2;
  int o3 = tot2 + b3 + x3 - n3;
  while (m1) {
    const int b = __ffs(m1) - 1;
    m1 &= m1 - 1u;
    dst[o1++] = (int)(p0 + b);
  }
  while (m2) {
    const int b = __ffs(m2) - 1;
    m2 &= m2 - 1u;
    dst[o2++] = (int)(p0 + b);
  }
  while (m3) {
    const int b = __ffs(m3) - 1;
    m3 &= m3 - 1u;
    dst[o3++] = (int)(p0 + b);
  }
}

hipError_t launch_select(const SelectArgs &a, int H_q, hipStream_t st) {
  hipLaunchKernelGGL(bucket_count_kernel, dim3(H_q, (unsigned)a.ntiles), dim3(64), 0, st, a);
  hipLaunchKernelGGL(bucket_write_kernel, dim3(H_q, (unsigned)a.ntiles), dim3(64), 0, st, a);
  return hipGetLastError();
}


}  // namespace csa
