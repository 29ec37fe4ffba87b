// C ABI of the certified decode path (declarations and contracts in include/csa.h).
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.h"

// The launchers take the kernels' argument structs, so the kernel sources are
// compiled as part of this one translation unit.
#include "scan.hip"
#include "select.hip"
#include "certify.hip"
#include "dense.hip"
#include "pack.hip"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char *where) {
  return fail(CSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int check_shape(const csa_shape *s) {
  if (!s) return fail(CSA_ERR_INVALID_ARGUMENT, "shape is null");
  if (s->head_dim != csa::kD) return fail(CSA_ERR_INVALID_ARGUMENT, "head_dim must be 128 (got %d)", s->head_dim);
  if (s->num_kv_heads < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "num_kv_heads must be >= 1");
  if (s->group_size < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "group_size must be >= 1");
  if (s->group_size > csa::kMaxG) return fail(CSA_ERR_UNSUPPORTED, "group_size must be <= %d", csa::kMaxG);
  if (s->n_cap < 32 || s->n_cap % 32 != 0 || s->n_cap >= (int64_t(1) << 31))
    return fail(CSA_ERR_UNSUPPORTED, "n_cap must be a positive multiple of 32 below 2^31");
  return CSA_OK;
}

int check_params(const csa_params *p) {
  if (!p) return fail(CSA_ERR_INVALID_ARGUMENT, "params is null");
  if (!(p->eps > 0.0) || !std::isfinite(p->eps)) return fail(CSA_ERR_INVALID_ARGUMENT, "eps must be > 0");
  if (!(p->delta > 0.0 && p->delta < 1.0)) return fail(CSA_ERR_INVALID_ARGUMENT, "delta must lie in (0, 1)");
  if (p->r < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "r must be >= 1");
  if (p->J < 0) return fail(CSA_ERR_INVALID_ARGUMENT, "J must be >= 0");
  if (p->J > csa::kMaxJ) return fail(CSA_ERR_UNSUPPORTED, "J must be <= %d", csa::kMaxJ);
  if (p->window < 32 || p->window > csa::kMaxWin)
    return fail(CSA_ERR_UNSUPPORTED, "window must lie in [32, %d]", csa::kMaxWin);
  if (p->measure < 0 || p->measure > 2) return fail(CSA_ERR_INVALID_ARGUMENT, "unknown measure %d", p->measure);
  return CSA_OK;
}

// The items of one call (a single call is one item in cache slot 0).
struct Call {
  csa::Batch b;
  double eps[csa::kMaxItems];
  uint64_t seed[csa::kMaxItems], step[csa::kMaxItems];
  int32_t layer[csa::kMaxItems];
  int64_t n_max;       // the longest item
  int64_t npool_max;   // its pool (0: every item is its window alone)
};

Call single_call(const csa_shape *s, const csa_params *p, int64_t n) {
  Call c{};
  c.b.nitems = 1;
  c.b.H_kv = s->num_kv_heads;
  c.b.n[0] = n;
  c.b.slot[0] = 0;
  c.eps[0] = p->eps;
  c.seed[0] = p->seed;
  c.step[0] = p->step;
  c.layer[0] = p->layer;
  c.n_max = n;
  c.npool_max = n > p->window ? n - p->window : 0;
  return c;
}

// Workspace layout for `nitems` items of up to n_max cached tokens each.
csa::Plan make_plan(const csa_shape *s, const csa_params *p, int64_t n_max, int nitems = 1) {
  csa::Plan P;
  P.H_kv = s->num_kv_heads * nitems;
  P.G = s->group_size;
  P.H_q = P.H_kv * P.G;
  P.J = p->J;
  P.W = p->window;
  const int64_t npool = n_max > p->window ? n_max - p->window : 0;
  // per-head pool capacity, a multiple of 32 (rows of per-key arrays start 32-byte aligned
  // and every 32-key word of them lies inside its row)
  P.npool_cap = npool > 0 ? (npool + 31) / 32 * 32 : 32;
  P.ntiles = (P.npool_cap + csa::kBucketTile - 1) / csa::kBucketTile;
  const size_t Hq = (size_t)P.H_q, J1 = (size_t)P.J + 1, J2 = (size_t)P.J + 2, npc = (size_t)P.npool_cap;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  P.qf = take(Hq * csa::kD * sizeof(float));
  P.qconst = take(Hq * csa::kQc * sizeof(double));
  P.qA = take((size_t)P.H_kv * 2048);
  P.lt = take(J1 * sizeof(double));
  P.tau = take(J1 * sizeof(double));
  P.prefix = take((size_t)P.H_kv * sizeof(uint64_t));
  P.sR = take(Hq * (size_t)P.W * sizeof(double));
  P.cR = 0;
  P.clo = take(Hq * sizeof(unsigned long long));
  P.cstar = take(Hq * sizeof(unsigned long long));
  P.wstride = std::max<int64_t>(1, ((P.npool_cap + csa::kBlk - 1) / csa::kBlk + csa::kScanBlocks - 1) / csa::kScanBlocks);
  P.lbpart = take(Hq * (size_t)P.wstride * sizeof(float));
  P.vpart = take((size_t)P.H_kv * P.wstride * sizeof(unsigned));
  P.exdone = take(Hq * sizeof(int));
  P.exdone2 = take(Hq * sizeof(int));
  P.hist = take(Hq * J2 * sizeof(int));
  P.tilelist = take(Hq * (size_t)P.ntiles * csa::kTileList * sizeof(int));
  P.tilehist = take(Hq * (size_t)P.ntiles * J2 * sizeof(int));
  P.tilecm = take(Hq * (size_t)P.ntiles * J2 * sizeof(int));
  P.cmhist = take(Hq * J2 * sizeof(int));
  P.ccount = take(Hq * sizeof(int));
  P.ccount1 = take(Hq * sizeof(int));
  P.jspec = take(Hq * sizeof(int));
  P.ccount2 = take(Hq * sizeof(int));
  P.jspec2 = take(Hq * sizeof(int));
  P.pbuf = take(Hq * npc * sizeof(double));
  P.ubuf = take(Hq * npc * sizeof(double));
  P.lub = take(Hq * npc);
  P.live = take(Hq * (size_t)(P.npool_cap / 32 + 1) * sizeof(uint32_t));
  P.bmax = take(Hq * (size_t)((P.npool_cap + csa::kBlk - 1) / csa::kBlk) * 2 * sizeof(float));
  P.win = take(Hq * (size_t)csa::kWinW * sizeof(double));
  P.candpos = take(Hq * npc * sizeof(int));
  P.rec_s = take(Hq * npc * sizeof(double));
  P.rec_w = take(Hq * npc * sizeof(double));
  P.rec_vsq = take(Hq * npc * sizeof(double));
  P.rec_hl = take(Hq * npc * sizeof(int));
  P.rec_x = take(Hq * npc * sizeof(int));
  P.nseg_cap = csa::seg_cap_for(npool);
  P.partial = take(Hq * (size_t)P.nseg_cap * J1 * csa::kStatW * sizeof(double));
  P.betalv = take(Hq * J1 * sizeof(double));
  P.dhatlv = take(Hq * J1 * sizeof(double));
  P.klv = take(Hq * J1 * sizeof(int));
  P.flags = take(Hq * sizeof(int));
  P.flags2 = take(Hq * sizeof(int));
  P.exactp = take(Hq * csa::kExactChunks * 130 * sizeof(double));
  P.total = off;
  return P;
}

template <class T>
T *at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

int check_packed(const csa_packed *p) {
  if (!p || !p->codes || !p->kscale || !p->zq || !p->bmeta || !p->kerr || !p->vnorm || !p->codes8 ||
      !p->scale8 || !p->kerr8)
    return fail(CSA_ERR_INVALID_ARGUMENT, "packed arrays must all be non-null");
  return CSA_OK;
}

// The scan (whose window workgroups also store the per-call constants) and the
// refinement, shared by the certified call and the bounds diagnostic.
int run_scan(const csa_shape *s, const csa_params *p, const Call &c, const uint16_t *q, const uint16_t *K,
                  const uint16_t *V, const csa_packed *pk, void *ws, const csa::Plan &P, double *lb_out,
                  double *e_out, double *ub_diag, void *ev0, void *ev1, hipStream_t st, int diag = 0) {
  const int64_t npool = c.npool_max;
  csa::ScanArgs sa;
  sa.K = K;
  sa.V = V;
  sa.b = c.b;
  sa.W = p->window;
  sa.q = q;
  sa.r = p->r;
  for (int i = 0; i < c.b.nitems; ++i) {
    sa.seed[i] = c.seed[i];
    sa.step[i] = c.step[i];
    sa.layer[i] = c.layer[i];
  }
  sa.sR = at<double>(ws, P.sR);
  sa.win = at<double>(ws, P.win);
  sa.cstar = at<unsigned long long>(ws, P.cstar);
  sa.tau = at<double>(ws, P.tau);
  sa.ccount = at<int>(ws, P.ccount);
  sa.exdone = at<int>(ws, P.exdone);
  sa.exdone2 = at<int>(ws, P.exdone2);
  sa.codes = pk->codes;
  sa.kscale = pk->kscale;
  sa.zq = pk->zq;
  sa.bmeta = reinterpret_cast<const csa::BlockMeta *>(pk->bmeta);
  sa.kerr = pk->kerr;
  sa.vnorm = pk->vnorm;
  sa.n_cap = s->n_cap;
  sa.nb_cap = s->n_cap / csa::kBlk;
  sa.nb_pool = (npool + csa::kBlk - 1) / csa::kBlk;
  sa.nstream = npool > 0 ? csa::scan_stream_wgs(P.H_kv, sa.nb_pool) : 0;
  sa.npool_cap = P.npool_cap;
  sa.G = P.G;
  sa.U = P.H_kv;
  sa.nbw = (P.npool_cap + csa::kBlk - 1) / csa::kBlk;
  sa.bmax = at<float2>(ws, P.bmax);
  sa.qf = at<float>(ws, P.qf);
  sa.qconst = at<double>(ws, P.qconst);
  sa.qA = at<int8_t>(ws, P.qA);
  sa.prefix = at<uint64_t>(ws, P.prefix);
  sa.pbuf = at<double>(ws, P.pbuf);
  sa.ubuf = at<double>(ws, P.ubuf);
  sa.clo = at<unsigned long long>(ws, P.clo);
  sa.lbpart = at<float>(ws, P.lbpart);
  sa.vpart = at<unsigned>(ws, P.vpart);
  sa.wstride = P.wstride;
  sa.lb_out = lb_out;
  sa.e_out = e_out;
  sa.nwords = P.npool_cap / 32 + 1;
  sa.J = P.J;
  sa.lt = at<double>(ws, P.lt);
  sa.live = at<uint32_t>(ws, P.live);
  sa.diag = diag;
  hipError_t e = csa::launch_scan(sa, st, (hipEvent_t)ev0, (hipEvent_t)ev1);
  if (e != hipSuccess) return hip_fail(e, "scan");
  if (npool <= 0) return CSA_OK;
  e = csa::launch_refine(sa, st);
  if (e != hipSuccess) return hip_fail(e, "refine");
  if (ub_diag) {
    e = hipMemcpy2DAsync(ub_diag, (size_t)npool * sizeof(double), sa.ubuf, (size_t)P.npool_cap * sizeof(double),
                         (size_t)npool * sizeof(double), (size_t)P.H_q, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "copy UB");
  }
  return CSA_OK;
}

// Trace values of a certified call, one workgroup (256 threads) per query head.  |C_max|
// counts the live keys whose stored UB reaches the final c_lo: every such key is live
// (its block passed the snapshot test and the key itself the UB >= snapshot test).
__global__ __launch_bounds__(256) void trace_kernel(const double *qconst, const unsigned long long *clo,
                                                    const unsigned long long *cstar, const uint32_t *live,
                                                    int64_t nwords, int64_t nblocks, const double *ubuf,
                                                    int64_t npool_cap, const int *ccount, double *c_R,
                                                    double *c_lo, double *c_star, int *cm, int *cc) {
  const int i = blockIdx.x, t = threadIdx.x;
  const double cl = csa::dec_max(clo[i]);
  if (t == 0) {
    if (c_R) c_R[i] = qconst[(int64_t)i * csa::kQc + csa::QC_CR];
    if (c_lo) c_lo[i] = cl;
    if (c_star) c_star[i] = csa::dec_max(cstar[i]);
    if (cc) cc[i] = ccount[i];
  }
  if (!cm) return;
  __shared__ int part[4];
  int k = 0;
  for (int64_t w = t; w < nblocks; w += 256) {
    uint32_t bits = live[(int64_t)i * nwords + w];
    while (bits) {
      const int b = __ffs((int)bits) - 1;
      bits &= bits - 1u;
      k += (ubuf[(int64_t)i * npool_cap + 32 * w + b] >= cl) ? 1 : 0;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) k += __shfl_xor(k, off, 64);
  if ((t & 63) == 0) part[t >> 6] = k;
  __syncthreads();
  if (t == 0) cm[i] = part[0] + part[1] + part[2] + part[3];
}

// Per-candidate trace, grid (H_q, ceil(npool / 256)): the candidate list and the levels
// of the entries that were rescored.  Pass p rescores the entries up to the end of its
// range (levels up to jspec, jspec2, J); a head whose stop level lies past a pass's
// deepest level went through the next one (the exact fallback only after the last
// pass, which rescored all).
__global__ __launch_bounds__(256) void cand_trace_kernel(const int *ccount, const int *ccount1, const int *jspec,
                                                         const int *ccount2, const int *jspec2,
                                                         const int32_t *stop, const int *candpos, const int *rec_hl,
                                                         const int *rec_x, int64_t npool_cap, int64_t npool,
                                                         int32_t *cand_pos, int32_t *cand_hl, int32_t *cand_l8,
                                                         int32_t *rescored) {
  const int hq = blockIdx.x;
  const int cnt = ccount[hq];
  const int st = stop[hq];
  const int nres = (st <= jspec[hq]) ? ccount1[hq] : ((st <= jspec2[hq]) ? ccount2[hq] : cnt);
  if (blockIdx.y == 0 && threadIdx.x == 0 && rescored) rescored[hq] = nres;
  const int64_t i = (int64_t)blockIdx.y * 256 + threadIdx.x;
  if (i >= cnt || i >= npool) return;
  const int64_t src = (int64_t)hq * npool_cap + i, dst = (int64_t)hq * npool + i;
  if (cand_pos) cand_pos[dst] = candpos[src];
  if (cand_hl) cand_hl[dst] = (i < nres) ? rec_hl[src] : -1;
  if (cand_l8) cand_l8[dst] = (i < nres) ? (rec_x[src] & 0xFF) : -1;
}

// One read of a buffer (16-byte loads; workgroup w streams the w-th contiguous slice) and
// the XOR of its 32-bit words per workgroup.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *src, int64_t n16, int64_t per,
                                                          uint32_t *sink) {
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(n16, b0 + per);
  uint32_t acc = 0;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += 4 * 256) {
    uint4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = (i + 256 * k < b1) ? src[i + 256 * k] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

int check_certified_args(const csa_shape *shape, const csa_params *params, const uint16_t *q, const uint16_t *K,
                         const uint16_t *V, const csa_packed *packed, int64_t n, const float *o_hat,
                         const double *beta, const int32_t *stop_level, const int64_t *keys_read) {
  int rc = check_shape(shape);
  if (rc || (rc = check_params(params))) return rc;
  if (!q || !K || !V || !o_hat || !beta || !stop_level || !keys_read)
    return fail(CSA_ERR_INVALID_ARGUMENT, "q, K, V and every output must be non-null");
  if (n < 1 || n > shape->n_cap) return fail(CSA_ERR_INVALID_ARGUMENT, "n must lie in [1, n_cap]");
  if (n > params->window && (rc = check_packed(packed))) return rc;
  return CSA_OK;
}

int certified_run(const csa_shape *shape, const csa_params *params, const Call &c, const uint16_t *q,
                  const uint16_t *K, const uint16_t *V, const csa_packed *packed, void *workspace, const csa::Plan &P,
                  float *o_hat, double *beta, int32_t *stop_level, int64_t *keys_read, const csa_trace *trace,
                  hipStream_t st);

// Scratch of the allocation-free entry point: one static array per GPU (the code object's
// device globals are instantiated on every device the library runs on), kept until the
// process ends.  Host code never passes `scratch` itself to a kernel -- in host code the
// name is a host-side stand-in -- but the device address hipGetSymbolAddress gives for the
// current device, looked up once per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CSA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(CSA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}

}  // namespace

extern "C" {

const char *csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_INVALID_ARGUMENT: return "CSA_ERR_INVALID_ARGUMENT";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE";
    case CSA_ERR_HIP: return "CSA_ERR_HIP";
    default: return "CSA_ERR_UNKNOWN";
  }
}

const char *csa_last_error(void) { return g_err; }

int csa_pack_kv_4bit(const csa_shape *shape, const uint16_t *K, const uint16_t *V, int64_t block_begin,
                     int64_t block_end, const csa_packed *out, csa_stream_t stream) {
  g_err[0] = 0;
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!K || !V) return fail(CSA_ERR_INVALID_ARGUMENT, "K and V must be non-null");
  if ((rc = check_packed(out))) return rc;
  const int64_t nb = shape->n_cap / csa::kBlk;
  if (block_begin < 0 || block_end < block_begin || block_end > nb)
    return fail(CSA_ERR_INVALID_ARGUMENT, "block range [%lld, %lld) outside [0, %lld]", (long long)block_begin,
                (long long)block_end, (long long)nb);
  hipError_t e = csa::launch_pack(*shape, K, V, block_begin, block_end, *out, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "pack");
}

size_t csa_workspace_bytes(const csa_shape *shape, const csa_params *params, int64_t n_max) {
  if (check_shape(shape) || check_params(params) || n_max < 1) return 0;
  return make_plan(shape, params, n_max).total;
}

int csa_scan_bounds(const csa_shape *shape, const csa_params *params, const uint16_t *q, const uint16_t *K,
                    const csa_packed *packed, int64_t n, void *workspace, size_t workspace_bytes, double *UB,
                    double *LB, double *E, csa_stream_t stream) {
  g_err[0] = 0;
  int rc = check_shape(shape);
  if (rc || (rc = check_params(params))) return rc;
  if (!q || !K) return fail(CSA_ERR_INVALID_ARGUMENT, "q and K must be non-null");
  if ((rc = check_packed(packed))) return rc;
  if (n < 1 || n > shape->n_cap) return fail(CSA_ERR_INVALID_ARGUMENT, "n must lie in [1, n_cap]");
  const csa::Plan P = make_plan(shape, params, n);
  if (!workspace || workspace_bytes < P.total)
    return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed", P.total);
  return run_scan(shape, params, single_call(shape, params, n), q, K, nullptr, packed, workspace, P, LB, E, UB,
                       nullptr, nullptr, (hipStream_t)stream, 1);
}

int csa_certified_decode_attention(const csa_shape *shape, const csa_params *params, const uint16_t *q,
                                   const uint16_t *K, const uint16_t *V, const csa_packed *packed, int64_t n,
                                   void *workspace, size_t workspace_bytes, float *o_hat, double *beta,
                                   int32_t *stop_level, int64_t *keys_read, const csa_trace *trace,
                                   csa_stream_t stream) {
  g_err[0] = 0;
  int rc = check_certified_args(shape, params, q, K, V, packed, n, o_hat, beta, stop_level, keys_read);
  if (rc) return rc;
  const csa::Plan P = make_plan(shape, params, n);
  if (!workspace || workspace_bytes < P.total)
    return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed", P.total);
  return certified_run(shape, params, single_call(shape, params, n), q, K, V, packed, workspace, P, o_hat, beta,
                       stop_level, keys_read, trace, (hipStream_t)stream);
}

size_t csa_workspace_bytes_batch(const csa_shape *shape, const csa_params *params, int32_t num_items,
                                 int64_t n_max) {
  if (check_shape(shape) || check_params(params) || n_max < 1 || num_items < 1 || num_items > csa::kMaxItems)
    return 0;
  return make_plan(shape, params, n_max, num_items).total;
}

int csa_certified_decode_attention_batch(const csa_shape *shape, const csa_params *params, int32_t num_slots,
                                         int32_t num_items, const csa_item *items, const uint16_t *q,
                                         const uint16_t *K, const uint16_t *V, const csa_packed *packed,
                                         void *workspace, size_t workspace_bytes, float *o_hat, double *beta,
                                         int32_t *stop_level, int64_t *keys_read, csa_stream_t stream) {
  g_err[0] = 0;
  int rc = check_shape(shape);
  if (rc || (rc = check_params(params))) return rc;
  if (num_items < 1 || num_items > csa::kMaxItems)
    return fail(CSA_ERR_UNSUPPORTED, "num_items must lie in [1, %d]", csa::kMaxItems);
  if (num_slots < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "num_slots must be >= 1");
  if ((int64_t)num_slots * shape->num_kv_heads * shape->n_cap >= (int64_t(1) << 40))
    return fail(CSA_ERR_UNSUPPORTED, "cache too large");
  if (!items || !q || !K || !V || !o_hat || !beta || !stop_level || !keys_read)
    return fail(CSA_ERR_INVALID_ARGUMENT, "items, q, K, V and every output must be non-null");
  Call c{};
  c.b.nitems = num_items;
  c.b.H_kv = shape->num_kv_heads;
  for (int i = 0; i < num_items; ++i) {
    const csa_item &it = items[i];
    if (it.n < 1 || it.n > shape->n_cap)
      return fail(CSA_ERR_INVALID_ARGUMENT, "item %d: n must lie in [1, n_cap]", i);
    if (it.slot < 0 || it.slot >= num_slots)
      return fail(CSA_ERR_INVALID_ARGUMENT, "item %d: slot %d outside [0, %d)", i, it.slot, num_slots);
    if (!(it.eps > 0.0) || !std::isfinite(it.eps)) return fail(CSA_ERR_INVALID_ARGUMENT, "item %d: eps must be > 0", i);
    c.b.n[i] = it.n;
    c.b.slot[i] = it.slot;
    c.eps[i] = it.eps;
    c.seed[i] = it.seed;
    c.step[i] = it.step;
    c.layer[i] = it.layer;
    c.n_max = std::max(c.n_max, it.n);
  }
  c.npool_max = c.n_max > params->window ? c.n_max - params->window : 0;
  if (c.npool_max > 0 && (rc = check_packed(packed))) return rc;
  const csa::Plan P = make_plan(shape, params, c.n_max, num_items);
  if (!workspace || workspace_bytes < P.total)
    return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed", P.total);
  return certified_run(shape, params, c, q, K, V, packed, workspace, P, o_hat, beta, stop_level, keys_read, nullptr,
                       (hipStream_t)stream);
}

int csa_certified_decode_attention_noalloc(const csa_shape *shape, const csa_params *params, const uint16_t *q,
                                           const uint16_t *K, const uint16_t *V, const csa_packed *packed,
                                           int64_t n, float *o_hat, double *beta, int32_t *stop_level,
                                           int64_t *keys_read, csa_stream_t stream) {
  g_err[0] = 0;
  int rc = check_certified_args(shape, params, q, K, V, packed, n, o_hat, beta, stop_level, keys_read);
  if (rc) return rc;
  const csa::Plan P = make_plan(shape, params, n);
  if (P.total > kScratchBytes)
    return fail(CSA_ERR_UNSUPPORTED,
                "this call needs %zu bytes of scratch; the library's static scratch holds %zu (use "
                "csa_certified_decode_attention with a workspace)",
                P.total, kScratchBytes);
  void *ws = nullptr;
  if ((rc = scratch_for_current_device(&ws))) return rc;
  return certified_run(shape, params, single_call(shape, params, n), q, K, V, packed, ws, P, o_hat, beta,
                       stop_level, keys_read, nullptr, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// The certified call on a workspace that holds at least plan P (arguments checked).
int certified_run(const csa_shape *shape, const csa_params *params, const Call &c, const uint16_t *q,
                  const uint16_t *K, const uint16_t *V, const csa_packed *packed, void *workspace, const csa::Plan &P,
                  float *o_hat, double *beta, int32_t *stop_level, int64_t *keys_read, const csa_trace *trace,
                  hipStream_t st) {
  int rc = 0;
  const bool all_exact = c.npool_max == 0;   // every item is its window alone
  void *ev0 = trace ? trace->ev_scan_begin : nullptr;
  void *ev1 = trace ? trace->ev_scan_end : nullptr;
  rc = run_scan(shape, params, c, q, K, V, packed, workspace, P, nullptr, nullptr, nullptr, ev0, ev1, st);
  if (rc) return rc;
  void *ws = workspace;
  const int64_t npool = c.npool_max;   // (a single call: its pool)
  hipError_t e;
  csa::SelectArgs sel{};
  // the first pass rescores inside the certificate kernel: at most kFusedMax candidates
  const int budget = params->cand_budget > 0 ? std::min(params->cand_budget, csa::kFusedMax) : csa::kDefaultBudget;
  const int budget2 = params->cand_budget2 > 0 ? params->cand_budget2 : INT_MAX;   // default: no third range
  if (!all_exact) {
    csa::SelectArgs &sa = sel;
    sa.b = c.b;
    sa.W = params->window;
    sa.npool_cap = P.npool_cap;
    sa.ntiles = (npool + csa::kBucketTile - 1) / csa::kBucketTile;
    sa.G = P.G;
    sa.J = P.J;
    sa.lt = at<double>(ws, P.lt);
    sa.pbuf = at<double>(ws, P.pbuf);
    sa.ubuf = at<double>(ws, P.ubuf);
    sa.clo = at<unsigned long long>(ws, P.clo);
    sa.cstar = at<unsigned long long>(ws, P.cstar);
    sa.tilehist = at<int>(ws, P.tilehist);
    sa.tilecm = at<int>(ws, P.tilecm);
    sa.tilelist = at<int>(ws, P.tilelist);
    sa.lub = at<int8_t>(ws, P.lub);
    sa.live = at<uint32_t>(ws, P.live);
    sa.nwords = P.npool_cap / 32 + 1;
    sa.full_lub = (trace && trace->lub) ? 1 : 0;
    if ((e = csa::launch_select(sa, P.H_q, st)) != hipSuccess) return hip_fail(e, "select");
  }
  csa::CertArgs ca{};
  ca.K = K;
  ca.V = V;
  ca.n_cap = shape->n_cap;
  ca.b = c.b;
  ca.npool_cap = P.npool_cap;
  ca.G = P.G;
  ca.J = P.J;
  ca.W = params->window;
  ca.measure = params->measure;
  for (int i = 0; i < c.b.nitems; ++i) ca.eps[i] = c.eps[i];
  {
    const int tails = params->measure == CSA_MEASURE_DENOM ? 2 : (params->measure == CSA_MEASURE_OUTNORM ? 5 : 6);
    ca.L = std::log((double)tails * (double)(params->J + 1) / params->delta);
  }
  ca.qf = at<float>(ws, P.qf);
  ca.lt = at<double>(ws, P.lt);
  ca.tau = at<double>(ws, P.tau);
  ca.sR = at<double>(ws, P.sR);
  ca.win = at<double>(ws, P.win);
  ca.qconst = at<double>(ws, P.qconst);
  ca.cstar = at<unsigned long long>(ws, P.cstar);
  ca.vpart = at<unsigned>(ws, P.vpart);
  ca.wstride = P.wstride;
  ca.ccount = at<int>(ws, P.ccount);
  ca.candpos = at<int>(ws, P.candpos);
  ca.rec_hl = at<int>(ws, P.rec_hl);
  ca.hist = at<int>(ws, P.hist);
  ca.ubuf = at<double>(ws, P.ubuf);
  ca.clo = at<unsigned long long>(ws, P.clo);
  ca.rec_w = at<double>(ws, P.rec_w);
  ca.rec_s = at<double>(ws, P.rec_s);
  ca.prefix = at<uint64_t>(ws, P.prefix);
  ca.rec_vsq = at<double>(ws, P.rec_vsq);
  ca.rec_x = at<int>(ws, P.rec_x);
  ca.codes8 = packed->codes8;
  ca.scale8 = packed->scale8;
  ca.kerr8 = packed->kerr8;
  ca.lub = at<int8_t>(ws, P.lub);
  ca.partial = at<double>(ws, P.partial);
  ca.betalv = at<double>(ws, P.betalv);
  ca.dhatlv = at<double>(ws, P.dhatlv);
  ca.klv = at<int>(ws, P.klv);
  ca.flags = at<int>(ws, P.flags);
  ca.exactp = at<double>(ws, P.exactp);
  ca.exdone = at<int>(ws, P.exdone);
  ca.exdone2 = at<int>(ws, P.exdone2);
  ca.flags2 = at<int>(ws, P.flags2);
  ca.ccount2 = at<int>(ws, P.ccount2);
  ca.jspec2 = at<int>(ws, P.jspec2);
  ca.H_q = P.H_q;
  ca.nseg_cap = P.nseg_cap;
  ca.cmhist = at<int>(ws, P.cmhist);
  ca.o_hat = o_hat;
  ca.beta = beta;
  ca.stop = stop_level;
  ca.keys_read = keys_read;
  ca.ccount1 = at<int>(ws, P.ccount1);
  ca.jspec = at<int>(ws, P.jspec);
  if (!all_exact) {   // pass 1 places the candidates from the bucket counts
    ca.tilehist = sel.tilehist;
    ca.tilecm = sel.tilecm;
    ca.tilelist = sel.tilelist;
    ca.ntiles = sel.ntiles;
    ca.live = sel.live;
    ca.nwords = sel.nwords;
    ca.budget = budget;
    ca.budget2 = budget2;
    ca.full_list = trace ? 1 : 0;
  }
  // pass 1: levels up to the speculative level (at most `budget` candidates, rescored
  // inside the certificate kernel); with all_exact, the exact attention of every head
  if ((e = csa::launch_certify_pass(ca, 1, P.H_q, st)) != hipSuccess) return hip_fail(e, "certify");
  // the tail: pass 2 for the heads that need all levels (their remaining candidates are
  // rescored there) and the exact fallback, in one launch that certified heads leave at once
  if ((e = csa::launch_tail(ca, P.H_q, params->cand_budget2 > 0, st)) != hipSuccess) return hip_fail(e, "tail");

  if (trace) {
    const int Hq = P.H_q;
    if (trace->c_R || trace->c_lo || trace->c_star || trace->cmax_count || trace->cand_count) {
      const int64_t nblocks = npool > 0 ? (npool + 31) / 32 : 0;
      hipLaunchKernelGGL(trace_kernel, dim3(Hq), dim3(256), 0, st, at<double>(ws, P.qconst),
                       at<unsigned long long>(ws, P.clo), at<unsigned long long>(ws, P.cstar),
                       at<uint32_t>(ws, P.live), (int64_t)(P.npool_cap / 32 + 1), nblocks,
                       at<double>(ws, P.ubuf), P.npool_cap, at<int>(ws, P.ccount), trace->c_R,
                       trace->c_lo, trace->c_star, trace->cmax_count, trace->cand_count);
    }
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "trace");
    const size_t J1 = (size_t)P.J + 1;
    auto cp = [&](void *dst, size_t off, size_t bytes) -> hipError_t {
      return dst ? hipMemcpyAsync(dst, at<char>(ws, off), bytes, hipMemcpyDeviceToDevice, st) : hipSuccess;
    };
    if (!all_exact && (trace->cand_pos || trace->cand_hl || trace->cand_l8 || trace->rescored_count)) {
      const unsigned ny = (unsigned)((npool + 255) / 256);
      hipLaunchKernelGGL(cand_trace_kernel, dim3(Hq, ny), dim3(256), 0, st, at<int>(ws, P.ccount),
                         at<int>(ws, P.ccount1), at<int>(ws, P.jspec), at<int>(ws, P.ccount2),
                         at<int>(ws, P.jspec2), stop_level, at<int>(ws, P.candpos),
                         at<int>(ws, P.rec_hl), at<int>(ws, P.rec_x), P.npool_cap, npool, trace->cand_pos,
                         trace->cand_hl, trace->cand_l8, trace->rescored_count);
      if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "candidate trace");
    }
    if (!all_exact) {
      if ((e = cp(trace->bucket_count, P.hist, (size_t)Hq * (J1 + 1) * sizeof(int))) != hipSuccess ||
          (e = cp(trace->beta_level, P.betalv, (size_t)Hq * J1 * sizeof(double))) != hipSuccess ||
          (e = cp(trace->dhat_level, P.dhatlv, (size_t)Hq * J1 * sizeof(double))) != hipSuccess ||
          (e = cp(trace->k_level, P.klv, (size_t)Hq * J1 * sizeof(int))) != hipSuccess ||
          (e = cp(trace->logtau, P.lt, J1 * sizeof(double))) != hipSuccess)
        return hip_fail(e, "trace copy");
      if (trace->lub && npool > 0) {
        e = hipMemcpy2DAsync(trace->lub, (size_t)npool, at<char>(ws, P.lub), (size_t)P.npool_cap, (size_t)npool,
                             (size_t)Hq, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return hip_fail(e, "trace lub");
      }
    }
  }
  return CSA_OK;
}

}  // namespace

extern "C" {

size_t csa_dense_workspace_bytes(const csa_shape *shape, int64_t n_max) {
  if (check_shape(shape) || n_max < 1) return 0;
  return align_up((size_t)shape->num_kv_heads * shape->group_size *
                  csa::dense_nsplit_max(n_max, shape->num_kv_heads) * csa::kDensePart * sizeof(float));
}

int csa_dense_decode_attention(const csa_shape *shape, const uint16_t *q, const uint16_t *K, const uint16_t *V,
                               int64_t n, void *workspace, size_t workspace_bytes, float *o, csa_stream_t stream) {
  g_err[0] = 0;
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!q || !K || !V || !o) return fail(CSA_ERR_INVALID_ARGUMENT, "q, K, V and o must be non-null");
  if (n < 1 || n > shape->n_cap) return fail(CSA_ERR_INVALID_ARGUMENT, "n must lie in [1, n_cap]");
  const size_t need = csa_dense_workspace_bytes(shape, n);
  if (!workspace || workspace_bytes < need) return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  csa::DenseArgs a;
  a.q = q;
  a.K = K;
  a.V = V;
  a.n_cap = shape->n_cap;
  a.n = n;
  a.G = shape->group_size;
  a.nsplit = csa::dense_nsplit(n, shape->num_kv_heads);
  a.split_len = csa::dense_split_len(n, shape->num_kv_heads);
  a.part = static_cast<float *>(workspace);
  a.o = o;
  hipError_t e = csa::launch_dense(a, shape->num_kv_heads, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "dense");
}

int csa_stream_read(const void *buf, int64_t bytes, int workgroups, uint32_t *sink, void *ev_begin,
                    void *ev_end, void *stream) {
  if (!buf || !sink) return fail(CSA_ERR_INVALID_ARGUMENT, "buf and sink must be device pointers");
  if (bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0)
    return fail(CSA_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 16 and buf 16-byte aligned");
  if (workgroups < 1 || workgroups > 65536) return fail(CSA_ERR_INVALID_ARGUMENT, "workgroups must be in [1, 65536]");
  const int64_t n16 = bytes / 16, per = (n16 + workgroups - 1) / workgroups;
  hipExtLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                        (hipEvent_t)ev_begin, (hipEvent_t)ev_end, 0, (const uint4 *)buf, n16, per, sink);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? CSA_OK : hip_fail(e, "stream read");
}

int csa_event_create(void **event) {
  if (!event) return fail(CSA_ERR_INVALID_ARGUMENT, "event is null");
  hipEvent_t ev;
  // timing only: no system-scope fence when the event is recorded, so recording it does not
  // write back and invalidate the caches under the kernels that follow
  hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableSystemFence);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
  *event = ev;
  return CSA_OK;
}

int csa_event_destroy(void *event) {
  hipError_t e = hipEventDestroy((hipEvent_t)event);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "hipEventDestroy");
}

int csa_event_elapsed_ms(void *begin, void *end, float *ms) {
  if (!ms) return fail(CSA_ERR_INVALID_ARGUMENT, "ms is null");
  hipError_t e = hipEventElapsedTime(ms, (hipEvent_t)begin, (hipEvent_t)end);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "hipEventElapsedTime");
}

}  // extern "C"
