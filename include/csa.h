/*
 * csa.h -- C ABI of the MI355X (gfx950) implementation of one decode step of
 * certified sparse attention via perturbed retrieval, for one layer over a 16-bit
 * KV cache.
 *
 * Sources (cited by page and section):
 *   [S] "Certified Sparse Attention via Perturbed Retrieval", structured summary:
 *       Theoretical Foundation; Methodology > Problem Setup; Methodology >
 *       Algorithm Components items 1-4; Results > Certificate Validity; Theorems 1-4.
 *   [A] "Certified Sparse Attention via Perturbed Retrieval", authors' abstract.
 *
 * Conventions for every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller unless the
 *     comment says "host".  The library never allocates, frees or retains memory;
 *     scratch space comes from the caller's workspace.
 *   - Calls are asynchronous on the given stream (a hipStream_t; NULL is the null
 *     stream).  Outputs are valid once that stream has synchronized.  Calls that
 *     share a workspace must be ordered on one stream.
 *   - Return value: CSA_OK (0) or a negative status; csa_status_string() names it
 *     and csa_last_error() gives the detail of the calling thread's last failure.
 *     On an argument error nothing is launched.  No C++ exception crosses the ABI.
 *   - Same inputs and parameters give bit-identical outputs (fixed-order
 *     reductions; floating-point atomics only on LDS cells that one thread owns).
 *   - Non-finite K, V or q values are undefined behaviour.
 *   - fp16 arrays are IEEE binary16 bit patterns (uint16_t).
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *csa_stream_t; /* hipStream_t */

enum csa_status {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARGUMENT = -1, /* null pointer, head_dim != 128, n < 1, n > n_cap,
                                    r < 1, J < 0, eps <= 0, delta outside (0,1), ... */
  CSA_ERR_UNSUPPORTED = -2,      /* group_size outside 1..7, window outside 32..1024, J > 60,
                                    n_cap not a multiple of 32 or >= 2^31 */
  CSA_ERR_WORKSPACE = -3,        /* workspace missing or smaller than csa_workspace_bytes() */
  CSA_ERR_HIP = -4               /* a HIP runtime call failed; csa_last_error() has the text */
};

enum csa_measure {
  CSA_MEASURE_DENOM = 0,   /* |D^ - D| <= eps D            ([S] Problem Setup) */
  CSA_MEASURE_OUTNORM = 1, /* |o^ - o| <= eps |o|                              */
  CSA_MEASURE_VALUE = 2    /* |o^ - o| <= eps M, M^2 = sum_i a_i |v_i|^2 (default) */
};

/* Shape of one layer's cache.  Query head hq is served by KV head hq / group_size. */
typedef struct {
  int32_t num_kv_heads; /* H_kv >= 1 */
  int32_t group_size;   /* G query heads per KV head (GQA group), 1..7 */
  int32_t head_dim;     /* d; must be 128 */
  int64_t n_cap;        /* token capacity of K, V and the packed arrays; multiple of 32 */
} csa_shape;

/*
 * Packed 4-bit keys and error-bound metadata of one layer ([S] Algorithm Components
 * item 4: 4-bit per-block, per-channel quantization giving deterministic score
 * bounds).  Blocks are 32 aligned tokens; nb_cap = n_cap / 32.  Per block b of KV
 * head h, with mn_t the block minimum of channel t and A = max_t |mn_t| = f 2^y
 * (f in [0.5, 1)):
 *   kappa = 2^kexp with kexp = y - 11 (0 when A = 0); z_t = floor(mn_t / kappa) in
 *   [-2048, 2047]; zero point kmin_t = kappa z_t; kscale_t = fp16 round-to-nearest
 *   of (max_t - kmin_t) / 15; code c = clamp(rint((k - kmin)/kscale), 0, 15).
 *   kerr_i = smallest fp16 h with h^2 >= sum_t (k_it - kmin_t - kscale_t c_it)^2 (1+2^-40)
 *   vnorm_i = smallest fp16 h with h^2 >= sum_t v_it^2 (1+2^-40).
 * Device layouts (84.5 bytes per token):
 *   codes  uint8 [H_kv][nb_cap][2048]: half-block tile T (tokens 16T..16T+15) at
 *          byte 1024 T; inside it, token n's channel group g (channels 32g..32g+31)
 *          is the 16-byte chunk at 16 (n + 16 g); its byte j holds the code of
 *          channel 32g + j in the low nibble and of channel 32g + 16 + j in the
 *          high nibble.
 *   kscale fp16  [H_kv][nb_cap][128].
 *   zq     int8  [H_kv][nb_cap][2][128]: z = 128 zq[0][t] + zq[1][t], zq[1] in [-64, 63].
 *   bmeta  16-byte records [H_kv][nb_cap]: { float ksmax = max_t kscale_t;
 *          int32 kexp; int32 Z1 = sum_t |z_t|; float Kmax = smallest fp32 >=
 *          max_t (|kmin_t| + 15 kscale_t) }.
 *   kerr, vnorm fp16 [H_kv][n_cap].
 * The 8-bit refinement copy ([S] Algorithm Components item 4: an 8-bit refinement
 * before exact 16-bit reads), per token i, read only for candidates:
 *   scale8_i = fp32 round-to-nearest of max_t |k_it| / 127; k8_it = clamp(rint(k_it /
 *   scale8_i), -127, 127) (0 for a zero key); kerr8_i = smallest fp16 h with h^2 >=
 *   sum_t (k_it - scale8_i k8_it)^2 (1+2^-40).
 *   codes8 int8 [H_kv][n_cap][128] (token-major), scale8 fp32 [H_kv][n_cap],
 *   kerr8 fp16 [H_kv][n_cap]: 134 bytes per token.
 */
typedef struct {
  uint8_t *codes;
  uint16_t *kscale;
  int8_t *zq;
  void *bmeta;
  uint16_t *kerr;
  uint16_t *vnorm;
  int8_t *codes8;
  float *scale8;
  uint16_t *kerr8;
} csa_packed;

/* Parameters of one certified call. */
typedef struct {
  double eps;      /* target error, > 0 ([S] Problem Setup) */
  double delta;    /* failure probability per head and call, in (0,1) ([S] Theorem 4) */
  int32_t r;       /* grid tau_j = 2^(-j/r), j = 0..J ([S] Algorithm Components item 3) */
  int32_t J;       /* deepest level, 0..60 */
  int32_t window;  /* recent tokens always read exactly ([S] item 1; 64 on the pages), 32..1024 */
  int32_t measure; /* enum csa_measure */
  uint64_t seed;   /* perturbation hash inputs ([S] item 1: u from 53 bits of a hash) */
  uint64_t step;   /* decode step: fresh perturbations per step ([A]) */
  int32_t layer;
  int32_t cand_budget; /* candidates rescored before the first certificate pass (0: 32;
                          values above 2048 act as 2048); heads that certify at no level up
                          to that point get a second pass over deeper levels.  Results do
                          not depend on it. */
  int32_t cand_budget2; /* 0 (default): the second pass takes every remaining level.  Else
                           the candidates (all passes so far) the second pass may take; it
                           takes at least one level more than the first, and heads still
                           uncertified get a third pass over every remaining level (one more
                           launch).  Results do not depend on it. */
} csa_params;

/*
 * Optional diagnostics of one certified call (every pointer may be NULL).  Arrays
 * are indexed by query head hq; n_pool = n - window.
 *   c_R, c_lo, c_star   fp64 [H_q]: window maximum, max(c_R, max LB), exact maximum.
 *   bucket_count        int32 [H_q][J+2]: pool keys per earliest possible level
 *                       l^ub = first((UB + E) - c*); bucket J+1 holds the rest.
 *   lub                 int8  [H_q][n_pool]: l^ub of every pool key.
 *   cmax_count          int32 [H_q]: |C_max| = |{pool keys with UB >= c_lo}|.
 *   cand_count          int32 [H_q]: keys rescored exactly (l^ub <= J).
 *   beta_level, dhat_level fp64 [H_q][J+1]: beta_j and D^_j at every level.
 *   k_level             int32 [H_q][J+1]: light sample count k_j.
 *   logtau              fp64 [J+1]: the level table used.
 *   ev_scan_begin/end   hipEvent_t that take the start and end times of the 4-bit
 *                       scan kernel's own dispatch (for timing it alone; no marker
 *                       packets are added to the stream).
 *   cand_pos            int32 [H_q][n_pool]: the candidates (l^ub <= J) in list order,
 *                       first those with l^ub up to the speculative level, then the
 *                       rest, each part in position order; entries past cand_count
 *                       are unspecified.
 *   cand_hl             int32 [H_q][n_pool]: for the first rescored_count entries of
 *                       cand_pos, h | (l << 8) with h = first(s - c*) the level from
 *                       which the key is heavy (always sampled) and l = first((s + E) - c*)
 *                       its entry level, both in [0, J+1] ([S] Algorithm Components
 *                       items 1-2: S_j = {l <= j}, B_j = {h <= j}); -1 for the other
 *                       candidates, which can enter the sample only at levels past the
 *                       stop level.
 *   rescored_count      int32 [H_q]: candidates rescored exactly in this call.
 *   cand_l8             int32 [H_q][n_pool]: for the first rescored_count entries of
 *                       cand_pos, the refined level l8 = first((min(UB, UB8) + E) - c*)
 *                       in [0, J+1] (the exact key and value are read only when l8 <= J);
 *                       -1 for the other candidates.
 */
typedef struct {
  double *c_R, *c_lo, *c_star;
  int32_t *bucket_count;
  int8_t *lub;
  int32_t *cmax_count;
  int32_t *cand_count;
  double *beta_level, *dhat_level;
  int32_t *k_level;
  double *logtau;
  void *ev_scan_begin, *ev_scan_end;
  int32_t *cand_pos, *cand_hl;
  int32_t *rescored_count;
  int32_t *cand_l8;
} csa_trace;

/*
 * Pack blocks [block_begin, block_end) of one layer (prefill, and each time an
 * append completes a block).  K, V: fp16 [H_kv][n_cap][128] of this layer.
 * Requires 0 <= block_begin <= block_end <= n_cap/32.
 */
int csa_pack_kv_4bit(const csa_shape *shape, const uint16_t *K, const uint16_t *V,
                     int64_t block_begin, int64_t block_end, const csa_packed *out,
                     csa_stream_t stream);

/* Workspace bytes a call with these shape/params needs for any n <= n_max. */
size_t csa_workspace_bytes(const csa_shape *shape, const csa_params *params, int64_t n_max);

/*
 * One certified decode step of one layer for all H_q = H_kv * G query heads
 * ([S] Algorithm Components items 1-4; [A]).
 *   q        fp16 [H_q][128]
 *   K, V     fp16 [H_kv][n_cap][128] of this layer; tokens 0..n-1 are in use.
 *   packed   this layer's packed keys; blocks 0..ceil((n - window)/32)-1 must be packed.
 *   n        cached tokens, 1 <= n <= n_cap.  Pool = [0, n - window), window = the rest.
 * Outputs per query head:
 *   o_hat      fp32 [H_q][128]  the estimate o^_{j*} = N^/D^ (exact o on fallback)
 *   beta       fp64 [H_q]       the certified bound at the stop level (0 when exact)
 *   stop_level int32 [H_q]      j* = first level with beta_j <= eps; J+1 = no level
 *                               certified and o is exact ([S] Results > Certificate
 *                               Validity); 0 when n <= window (every key is exact)
 *   keys_read  int64 [H_q]      exact 16-bit key reads: window + |C_max union
 *                               {l8 <= j*}| with l8 the level after the 8-bit
 *                               refinement (n on the exact paths)
 */
int csa_certified_decode_attention(const csa_shape *shape, const csa_params *params,
                                   const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                   const csa_packed *packed, int64_t n, void *workspace,
                                   size_t workspace_bytes, float *o_hat, double *beta,
                                   int32_t *stop_level, int64_t *keys_read,
                                   const csa_trace *trace, csa_stream_t stream);

/*
 * One item of a batched certified call: a request, or one layer of a request.  Each item
 * has its own context length, target and fresh perturbations ([S] Results > CPU Speed:
 * new perturbations at every decode step; the hash inputs of [S] Algorithm Components
 * item 1 are per item).
 */
typedef struct {
  int64_t n;       /* cached tokens of the item, 1 <= n <= n_cap */
  int32_t slot;    /* cache slot of the item's K, V and packed arrays, 0 <= slot < num_slots */
  int32_t layer;   /* hash input */
  double eps;      /* certificate target of the item, > 0 */
  uint64_t seed;   /* hash inputs */
  uint64_t step;
} csa_item;

#define CSA_MAX_ITEMS 64

/*
 * Workspace of a batched call of up to num_items items of at most n_max tokens each
 * (0 on invalid arguments).
 */
size_t csa_workspace_bytes_batch(const csa_shape *shape, const csa_params *params, int32_t num_items,
                                 int64_t n_max);

/*
 * The certified decode step of num_items items in one set of launches (every kernel of
 * the path runs once for the whole batch).  The cache holds num_slots slots of
 * num_kv_heads heads each: item b's KV head h is cache head slot_b * num_kv_heads + h.
 *   shape    per slot: num_kv_heads, group_size, head_dim 128, n_cap
 *   params   delta, r, J, window, measure, cand_budget, cand_budget2 shared by all items;
 *            its eps, seed, step and layer are not used (each item carries its own)
 *   items    host array of num_items entries, 1 <= num_items <= CSA_MAX_ITEMS
 *   q        fp16 [num_items][H_q][128]
 *   K, V     fp16 [num_slots][num_kv_heads][n_cap][128] (device)
 *   packed   the packing of K, V as num_slots * num_kv_heads heads (csa_pack_kv_4bit with
 *            num_kv_heads = num_slots * num_kv_heads); each item's blocks up to
 *            ceil((n - window) / 32) must be packed
 *   workspace at least csa_workspace_bytes_batch(shape, params, num_items, max n)
 * Outputs per item and query head, laid out [num_items][H_q] (o_hat [num_items][H_q][128])
 * with the meaning of csa_certified_decode_attention's.  Each item's outputs are those of
 * a single call on that item up to the order of floating-point sums (sets, levels, stop
 * levels and keys_read are the same).  Errors: CSA_ERR_INVALID_ARGUMENT for a bad item
 * (n, slot, eps) or pointer, CSA_ERR_UNSUPPORTED beyond CSA_MAX_ITEMS, CSA_ERR_WORKSPACE
 * for a short workspace; nothing is launched then.
 */
int csa_certified_decode_attention_batch(const csa_shape *shape, const csa_params *params,
                                         int32_t num_slots, int32_t num_items, const csa_item *items,
                                         const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                         const csa_packed *packed, void *workspace,
                                         size_t workspace_bytes, float *o_hat, double *beta,
                                         int32_t *stop_level, int64_t *keys_read,
                                         csa_stream_t stream);

/*
 * The same certified decode step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments and outputs are those of
 * csa_certified_decode_attention (no trace).  Scratch space is a static device array of
 * 64 MiB that the library holds on every GPU it runs on until the process ends; this
 * call allocates and frees nothing.  Calls whose scratch need (csa_workspace_bytes for
 * this n) exceeds 64 MiB return CSA_ERR_UNSUPPORTED without launching anything.  Every
 * call on one GPU uses that GPU's one array: calls that overlap on a GPU (two streams,
 * two threads) race and give undefined results; order them on one stream.  The per-call
 * counters in the array are reset by the call itself.
 */
int csa_certified_decode_attention_noalloc(const csa_shape *shape, const csa_params *params,
                                           const uint16_t *q, const uint16_t *K, const uint16_t *V,
                                           const csa_packed *packed, int64_t n, float *o_hat,
                                           double *beta, int32_t *stop_level, int64_t *keys_read,
                                           csa_stream_t stream);

/*
 * Diagnostic: the scan's deterministic bounds and perturbations for every pool key.
 *   UB, LB fp64 [H_q][n - window]; E fp64 [H_kv][n - window] (E = -ln u from the
 *   hash of (seed, step, layer, kv_head, position)).  Any output may be NULL.
 * Uses the same workspace as csa_certified_decode_attention.
 */
int csa_scan_bounds(const csa_shape *shape, const csa_params *params, const uint16_t *q,
                    const uint16_t *K, const csa_packed *packed, int64_t n, void *workspace,
                    size_t workspace_bytes, double *UB, double *LB, double *E,
                    csa_stream_t stream);

/*
 * Dense attention o = softmax(q K^T / sqrt(128)) V over tokens 0..n-1 for all query
 * heads ([S] Problem Setup), fp32 accumulation; the library's own comparison kernel.
 *   o fp32 [H_q][128].  Workspace: csa_dense_workspace_bytes().
 */
size_t csa_dense_workspace_bytes(const csa_shape *shape, int64_t n_max);
int csa_dense_decode_attention(const csa_shape *shape, const uint16_t *q, const uint16_t *K,
                               const uint16_t *V, int64_t n, void *workspace,
                               size_t workspace_bytes, float *o, csa_stream_t stream);

/* Name of a status code (static string). */
const char *csa_status_string(int status);
/* Detail of the calling thread's last failed call (static per thread; "" if none). */
const char *csa_last_error(void);

/* Measurement helper (not part of the certified path): reads `bytes` of device memory at
 * `buf` once with 16-byte loads, `workgroups` workgroups of 256 threads each streaming one
 * contiguous slice, and writes each workgroup's XOR of the 32-bit words it read to
 * sink[workgroup] (uint32, device, `workgroups` entries).  It times the plain read of a
 * given byte count on the caller's stream: ev_begin/ev_end (hipEvent_t or NULL) take the
 * kernel's own dispatch start and end.  bytes must be a multiple of 16 and buf 16-byte
 * aligned; workgroups in [1, 65536].  Returns CSA_ERR_INVALID_ARGUMENT otherwise. */
int csa_stream_read(const void *buf, int64_t bytes, int workgroups, uint32_t *sink, void *ev_begin,
                    void *ev_end, void *stream);

/* Event helpers for timing on the caller's stream (host side; events are hipEvent_t).  The
 * events are for timing only: they are created without the system-scope fence at record
 * time (hipEventDisableSystemFence), so synchronize the device before reading a time. */
int csa_event_create(void **event);
int csa_event_destroy(void *event);
int csa_event_elapsed_ms(void *begin, void *end, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
