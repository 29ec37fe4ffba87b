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
  int64_t npool_cap, ntiles;   // ntiles: the longest item's tiles (row stride)
  int G, J, W;
  Batch b;
  const double *lt;
  const double *pbuf, *ubuf;
  const unsigned long long *clo, *cstar;
  int8_t *lub;
  const uint32_t *live;   // [H_q][nwords] keys the scan kept (others have l^ub = J+1, UB < c_lo)
  int64_t nwords;
  int full_lub;           // write l^ub for every pool key (diagnostics)
  int *tilehist;          // [H_q][ntiles][J+2] per-tile cumulative counts of l^ub
  int *tilecm;            // [H_q][ntiles][J+2] C_max keys per level and tile
  int *tilelist;          // [H_q][ntiles][kTileList] the tile's lowest-level live keys
};

// ---- buckets.  A tile is 64 bitmap words (2048 positions).
// Per tile: cumulative level counts tilehist[tile][j] = |{l^ub <= j}| (j = 0..J+1, the
// last one counting every pool key of the tile), the C_max keys per level, and the
// positions of the tile's live keys ordered by level (in no set order within a level),
// the first kTileList of them: the keys with l^ub <= j are the first tilehist[tile][j]
// entries, so a level prefix of the head that holds at most kTileList keys of the tile
// is read from this list without the bitmap.
__global__ __launch_bounds__(64) void bucket_count_kernel(SelectArgs a) {
  const int hq = blockIdx.x, lane = threadIdx.x;
  const int64_t tile = blockIdx.y;
  // (tiles past this unit's pool find no valid keys: their rows are written as zeros and
  // never read)
  const int64_t npool = unit_npool(a.b, hq / a.G, a.W);
  __shared__ int hist[kMaxJ + 2], cmh[kMaxJ + 2], slot[kMaxJ + 2];
  __shared__ __attribute__((aligned(16))) uint32_t wt[2][32];   // the tile's words, even ones first
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
  // the word's bits are read by the lanes below through shuffles; the keys that are not
  // live count at level J + 1 only through the tile's total (no per-lane atomics)
  const int valid = (int)max<int64_t>(0, min<int64_t>(32, npool - p_tile - 32 * lane));
  const uint32_t word = rawword & ((valid == 32) ? 0xFFFFFFFFu : ((1u << valid) - 1u));
  const int tile_keys = (int)max<int64_t>(0, min<int64_t>(kBucketTile, npool - p_tile));
  // positions p_tile + 64 k + lane, k = 0..31: lane reads bit (lane & 31) of tile word
  // 2k + (lane >> 5), so every load and store of a round covers 64 consecutive keys
  const bool any = __ballot(word != 0u) != 0ull;
  uint32_t on = 0;
  int lv[32];
  if (any || a.full_lub) {
    const double *pb = a.pbuf + (int64_t)hq * a.npool_cap + p_tile;
    const double *ubp = a.ubuf + (int64_t)hq * a.npool_cap + p_tile;
    int8_t *lub = a.lub + (int64_t)hq * a.npool_cap + p_tile;
    const int64_t left = npool - p_tile;
    // (the words go through LDS, even ones first: a lane's 32 words are then 8 vector reads)
    wt[lane & 1][lane >> 1] = word;
    __builtin_amdgcn_wave_barrier();
    const uint4 *wrow = reinterpret_cast<const uint4 *>(wt[lane >> 5]);
#pragma unroll
    for (int k4 = 0; k4 < 8; ++k4) {
      const uint4 w4 = wrow[k4];
      const uint32_t wk[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) on |= ((wk[i] >> (lane & 31)) & 1u) << (4 * k4 + i);
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
      lv[k] = 0;
      if ((on >> k) & 1u) {
        const int l = level_of_pairs(pv[k] - cs, ltp, a.J, inv_l1);
        lv[k] = l;
        lub[i] = (int8_t)l;
        atomicAdd(&hist[l], 1);
        if (uv[k] >= clo) atomicAdd(&cmh[l], 1);
      } else if (a.full_lub && i < left) {
        lub[i] = (int8_t)(a.J + 1);
      }
    }
  }
  __syncthreads();
  // inclusive prefix over levels of the live keys (lane = level); at J + 1 the count is
  // every pool key of the tile
  if (lane < a.J + 2) {
    int c = hist[lane];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(c, off, 64);
      if (lane >= off) c += y;
    }
    a.tilehist[((int64_t)hq * a.ntiles + tile) * (a.J + 2) + lane] = (lane == a.J + 1) ? tile_keys : c;
    a.tilecm[((int64_t)hq * a.ntiles + tile) * (a.J + 2) + lane] = cmh[lane];
    slot[lane] = c - hist[lane];   // first list index of the level
  }
  if (!any) return;
  __syncthreads();
  int *list = a.tilelist + ((int64_t)hq * a.ntiles + tile) * kTileList;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int l = lv[k];
    if (((on >> k) & 1u) && slot[l] < kTileList) {
      const int at = atomicAdd(&slot[l], 1);
      if (at < kTileList) list[at] = (int)(p_tile + 64 * k + lane);
    }
  }
}

hipError_t launch_select(const SelectArgs &a, int H_q, hipStream_t st) {
  hipLaunchKernelGGL(bucket_count_kernel, dim3(H_q, (unsigned)a.ntiles), dim3(64), 0, st, a);
  return hipGetLastError();
}


}  // namespace csa
