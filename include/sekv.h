/*
 * sekv.h - C ABI of libsekv, an MI355X (gfx950) implementation of the
 * decode-time hot path of SeKV's resolution-adaptive semantic KV cache.
 *
 * Pages cited (by title and section):
 *   [abstract] the authors' abstract of "SeKV: Resolution-Adaptive KV Cache with
 *              Hierarchical Semantic Memory for Long-Context LLM Inference"
 *              (chatpaper.ai paper page, English part).
 *   [de-1..3]  gist.science German explainer of the same paper, "Technisches
 *              Resümee" > "Methodik", parts 1 (span segmentation), 2 (dual
 *              resolution storage), 3 (zoom-in: routing, expansion,
 *              mixed-resolution attention).
 *   [zh-1..3]  gist.science Chinese explainer, "技术摘要" > "方法论", parts 1-3.
 *
 * Conventions shared by every call
 *   - Shapes come from sekv_config.  B = batch, T = n_ctx, Hq / Hkv query / KV
 *     heads, G = Hq / Hkv (1..8), d = head_dim (64 or 128).  Query head h
 *     belongs to KV head h / G.
 *   - "dtype" arrays hold float32 or bfloat16 (raw 16-bit patterns) per
 *     sekv_config.dtype.  sigma, gate, theta and outputs are always float32.
 *   - All arrays are C-order, caller-owned, and never freed or reallocated by
 *     the library.  "device" = HBM of the context's GPU; "host" = CPU memory;
 *     "pinned" = page-locked host memory from hipHostMalloc.
 *   - Capacities (host-computable, see sekv_capacities):
 *       seg_cap  = floor((T - n_sink - n_recent) / (min_span + 1)) + 1
 *       full_cap = min(T, n_sink + seg_cap + n_recent + 1)
 *   - Errors: every call returns a sekv_status; sekv_last_error() returns a
 *     thread-local message for the last failing call of this thread.  All
 *     argument checks run on the host before anything is enqueued; a call that
 *     fails a check writes nothing.  The staged host-resident decode also
 *     checks the route list after its one host wait: a failure found then (or
 *     an injected gather fault) returns before anything writes `out`, but the
 *     device workspace may already have been written.  No C++ exception
 *     crosses the ABI.
 *   - Asynchrony: calls enqueue on the caller's stream and return, except
 *     sekv_plan_spans and sekv_build_spans (host-synchronous) and the
 *     host-resident decode (one documented host wait, see below).
 *   - One context per device.  Calls that share a context must be ordered on
 *     one stream (the context holds the host-resident path's events and
 *     staging state).
 */
#ifndef SEKV_H
#define SEKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sekv_status {
  SEKV_OK = 0,
  SEKV_EINVAL = 1,     /* null pointer, bad enum, bad parameter value        */
  SEKV_ESHAPE = 2,     /* inconsistent or unsupported shape                  */
  SEKV_ECAPACITY = 3,  /* a caller buffer or workspace is too small          */
  SEKV_EHIP = 4,       /* a HIP runtime call failed                           */
  SEKV_ENOMEM = 5      /* the library could not allocate its own state       */
} sekv_status;

typedef enum sekv_dtype { SEKV_F32 = 0, SEKV_BF16 = 1 } sekv_dtype;

/* How host-resident factors reach the expanded-span pass (sekv_ctx_set_fetch_mode). */
typedef enum sekv_fetch_mode {
  SEKV_FETCH_STAGED = 0,  /* host threads gather the listed blocks into pinned staging,
                             one copy per staging slot on the copy stream, after one
                             host wait for the route list */
  SEKV_FETCH_DIRECT = 1   /* (default) the kernels read the listed blocks from the
                             pinned pools over the bus; no host wait, graph-capturable */
} sekv_fetch_mode;

/* Where sekv_build_spans computes summaries, routing keys and factors
 * (sekv_ctx_set_build_mode). */
typedef enum sekv_build_mode {
  SEKV_BUILD_DEVICE = 0,  /* (default) GPU kernels; separate bases (basis = 1) fall
                             back to the host */
  SEKV_BUILD_HOST = 1     /* host threads (one-sided Jacobi) */
} sekv_build_mode;

/* Failures a test can force from the host (sekv_ctx_inject_fault). */
typedef enum sekv_fault { SEKV_FAULT_NONE = 0, SEKV_FAULT_GATHER = 1 } sekv_fault;

typedef struct sekv_config {
  int32_t batch, n_ctx, n_q_heads, n_kv_heads, head_dim;
  int32_t n_sink;          /* full-resolution sink [0, n_sink)                      */
  int32_t n_recent;        /* full-resolution recent window, last n_recent tokens   */
  int32_t min_span;        /* lo: data heads need >= lo body tokens on both sides   */
  int32_t max_span;        /* hi: a body of hi tokens forces the next head          */
  int32_t dtype;           /* sekv_dtype of K/V, q, summaries, rho, factors         */
  int32_t factors_on_host; /* 1: fac/sg pools are pinned host memory              */
  /* Reading variants (0 = the default reading): */
  int32_t rank_cap;        /* 0: r_i <= L_i; 1: r_i <= ceil(L_i / 2)                */
  int32_t basis;           /* 0: one basis for [K | V]; 1: separate K and V bases   */
  int32_t route_keys;      /* 0: route on rho; 1: route on kbar with key_scale and
                              the fold matrix (P^T P q) . kbar / |P kbar|         */
  /* Decode-time layout (online sealing, sekv_append_token): */
  int32_t sealed;          /* 0: prefill layout; 1: only sealed spans (below)      */
  int32_t n_ctx_max;       /* capacities are sized for max(n_ctx, n_ctx_max)       */
} sekv_config;

/*
 * The span cache: everything decode reads.  Built by sekv_plan_spans +
 * sekv_build_spans, or filled by the caller directly (same layout).
 *
 *   seg_off [B][seg_cap+1] int32: anchor i of sequence b is token seg_off[i];
 *       span body i is the open token interval (seg_off[i], seg_off[i+1]), of
 *       length L_i = seg_off[i+1] - seg_off[i] - 1 (1..max_span); the tail
 *       (full resolution) starts at seg_off[n_seg].  [de-1], [zh-1].
 *   full_k [B][Hkv][full_cap][d] dtype: full-resolution keys in token order
 *       sink, anchors (span order), tail.  n_full[b] rows valid.
 *   full_v [B][Hkv][ceil(full_cap/32)][d][32] dtype: the matching values in
 *       32-entry tiles, each tile transposed: value (entry e, dim j) of a
 *       (b, kv) block at ((e/32)*d + j)*32 + e%32.  Padding entries must be
 *       finite (zero).  (The transposed tile is the matrix-core operand of P.V.)
 *   sum_k [B][Hkv][seg_cap][d] dtype: surprisal-weighted mean key of each span
 *       body; sum_v [B][Hkv][ceil(seg_cap/32)][d][32]: the mean values, tiled
 *       and transposed like full_v.  [de-2], [zh-2].
 *   rho [B][Hkv][seg_cap][d] dtype: routing key, P^T normalize(P kbar), so that
 *       q . rho equals the routing-space score of the projected query. [de-2/3]
 *   rank [B][seg_cap] int32: r_i, 1 <= r_i <= min(L_i, 2d), shared by all KV
 *       heads of the span.  [de-2], [zh-2] (adaptive rank budget).
 *   key_scale [B][Hkv][seg_cap] f32 (route_keys = 1): 1 / |P kbar| of each
 *       span (0 if the norm is 0), kbar the unrounded summary key.
 *   fold [Hkv][d][d] f64 (route_keys = 1): M = P^T P of each KV head.
 *   fac pool (dtype): for span (b, kv, i) a block at element offset
 *       fac_off[b][kv][i] (a multiple of 8) holding, with rp = ceil(r_i/8)*8:
 *       the key part of the right singular vectors Vh_K [r_i][d], where row
 *       k stores its d/8 groups of 8 elements rotated by k (group u at
 *       position (u + k) mod d/8, so that rows read side by side fall on
 *       different LDS banks); then U [L_i][rp] (row stride rp, padding
 *       zero); then the value part transposed, W_V[j][k] = Vh[k][d + j],
 *       stored as column blocks of 16 ranks: block g = k / 16 of width
 *       wk = min(16, rp - 16 g) is [d][wk] row-major at block offset 16 g d
 *       (padding zero).  Block size r_i*d + L_i*rp + d*rp elements.
 *       With basis = 1 the block is Vh_K [r_i][d] (rotated as above) | U_K
 *       [L_i][rp] | U_V [L_i][rp] | W_V blocks of the value basis, size
 *       r_i*d + 2*L_i*rp + d*rp; keys are U_K diag(sigma_K*gate) Vh_K and
 *       values U_V diag(sigma_V*gate) W_V^T.
 *   sg pool (float32): for span (b, kv, i) an entry at offset sg_off[b][kv][i]
 *       (a multiple of 4): sigma[rq] then gate[rq], rq = ceil(r_i/4)*4,
 *       padding zero.  Token keys of the span are U diag(sigma*gate) Vh_K,
 *       token values U diag(sigma*gate) W_V^T.  With basis = 1 the entry is
 *       sigma_K[rq] | gate[rq] | sigma_V[rq] | gate[rq] (4*rq floats).
 *       [abstract], [de-2], [zh-2].
 *
 * Device arrays are required for every field; the *_host fields are host
 * copies the library reads to size grids (n_seg_host, n_full_host) and, in the
 * host-resident mode, to gather factor blocks (seg_off_host, rank_host,
 * fac_off_host, sg_off_host).  With factors_on_host = 1, fac and sg must be
 * pinned host memory.
 */
typedef struct sekv_spans {
  int32_t seg_cap, full_cap;
  const int32_t* n_seg_host;    /* [B] host */
  const int32_t* n_full_host;   /* [B] host */
  const int32_t* seg_off;       /* [B][seg_cap+1] device */
  const int32_t* rank;          /* [B][seg_cap] device */
  const void* full_k;           /* [B][Hkv][full_cap][d] device */
  const void* full_v;           /* [B][Hkv][ceil(full_cap/32)][d][32] device */
  const void* sum_k;            /* [B][Hkv][seg_cap][d] device */
  const void* sum_v;            /* [B][Hkv][ceil(seg_cap/32)][d][32] device */
  const void* rho;              /* [B][Hkv][seg_cap][d] device */
  const int64_t* fac_off;       /* [B][Hkv][seg_cap] device */
  const int64_t* sg_off;        /* [B][Hkv][seg_cap] device */
  const void* fac;              /* pool, fac_elems elements of dtype */
  const float* sg;              /* pool, sg_elems floats */
  int64_t fac_elems, sg_elems;
  const int32_t* seg_off_host;  /* [B][seg_cap+1] host (host-resident mode) */
  const int32_t* rank_host;     /* [B][seg_cap] host (host-resident mode)   */
  const int64_t* fac_off_host;  /* [B][Hkv][seg_cap] host                    */
  const int64_t* sg_off_host;   /* [B][Hkv][seg_cap] host                    */
  const float* key_scale;       /* [B][Hkv][seg_cap] device (route_keys = 1) */
  const double* fold;           /* [Hkv][d][d] device (route_keys = 1)       */
} sekv_spans;

typedef struct sekv_ctx sekv_ctx;

/* Context for one GPU: events, timing hooks and the copy-side thread pool.
 * The pool (host gathers of the staged fetch, host-side span builds) has
 * min(hardware threads, 16) threads, or SEKV_THREADS threads when that
 * environment variable holds a positive integer; it changes no result.
 * Errors: SEKV_EINVAL (out == NULL), SEKV_EHIP (bad device), SEKV_ENOMEM. */
sekv_status sekv_ctx_create(int device, sekv_ctx** out);
void sekv_ctx_destroy(sekv_ctx* ctx);
/* Thread-local message of this thread's last failing call ("" if none). */
const char* sekv_last_error(void);

/* seg_cap and full_cap of a configuration (formulas above).  Host only. */
sekv_status sekv_capacities(const sekv_config* cfg, int32_t* seg_cap, int32_t* full_cap);

/*
 * sekv_plan_spans - segmentation and pool layout (host only, no GPU).
 * [de-1], [zh-1]: high-surprisal tokens become anchors, spans are the runs
 * between neighbouring anchors.  Rule: token n_sink is the first head; for
 * t in (n_sink, T - n_recent), with body = tokens since the last head, t is a
 * head if body == max_span, or if surprisal[t] > boundary_thr[b] and
 * body >= min_span and at least min_span tokens remain before the recent
 * window; a last head with an empty body is returned to the tail.  Rank
 * r_i = min(rank_req[b][i], L_i, 2d), with ceil(L_i / 2) in place of L_i when
 * cfg->rank_cap = 1 and d in place of 2d when cfg->basis = 1 (each part of
 * separate bases is L_i x d).
 *   surprisal [B][T], boundary_thr [B], rank_req [B][seg_cap]: host, read.
 *   Outputs (host, written): n_seg [B], n_full [B], seg_off [B][seg_cap+1]
 *   (unused tail entries set to the tail start), rank [B][seg_cap] (0 past
 *   n_seg), fac_off/sg_off [B][Hkv][seg_cap] (0 past n_seg), *fac_elems,
 *   *sg_elems (pool sizes).  Errors: SEKV_EINVAL / SEKV_ESHAPE; non-finite
 *   surprisal or threshold, rank_req < 1 -> SEKV_EINVAL.
 */
sekv_status sekv_plan_spans(const sekv_config* cfg, const float* surprisal, const float* boundary_thr,
                            const int32_t* rank_req, int32_t* n_seg, int32_t* n_full, int32_t* seg_off,
                            int32_t* rank, int64_t* fac_off, int64_t* sg_off, int64_t* fac_elems,
                            int64_t* sg_elems);

/*
 * sekv_build_spans - fill the cache from the prefill K/V (host-synchronous).
 * k, v [B][Hkv][T][d] dtype: device, read.  surprisal [B][T] f32: host.
 * route_proj [Hkv][d][d] f32: host (one projection per KV head, [de-3]).
 * gate [B][Hkv][seg_cap][gate_stride] f32: host (rank gates, first r_i used).
 * spans: the plan fields (n_seg_host, n_full_host, seg_off_host, rank_host,
 * fac_off_host, sg_off_host) must hold sekv_plan_spans output; every device
 * array (and the pools, pinned host when factors_on_host) is written.
 * Summaries: weights s_t / sum s over the body (uniform if the sum is 0).
 * Routing key: rho = P^T r/|r|, r = P kbar (0 if |r| = 0); with route_keys = 1
 * instead key_scale = 1/|r| and fold = P^T P (rho may then be NULL).
 * Factors: rank-r_i truncated SVD of [K_body | V_body] (basis 0) or of K_body
 * and V_body separately (basis 1), in fp64, sign fixed so each U column's
 * largest-magnitude entry is positive.  Stored values are fp64 rounded to f32
 * (then to bf16, nearest-even).  Build mode DEVICE (the context's default,
 * basis 0): GPU kernels, one workgroup per span of a persistent grid, the
 * factors from the Jacobi eigenvectors of the fp64 Gram matrix M M^T (as
 * sekv_append_token); summaries, routing keys and key scales in the host
 * builder's fp64 operation order (same bits).  Build mode HOST, or basis 1:
 * host threads, one-sided Jacobi on M.  The segmentation scan and the fold
 * matrices are host work in both modes.
 * Errors: SEKV_EINVAL / SEKV_ESHAPE / SEKV_ECAPACITY (pool sizes) / SEKV_EHIP.
 */
sekv_status sekv_build_spans(sekv_ctx* ctx, const sekv_config* cfg, const void* k, const void* v,
                             const float* surprisal, const float* route_proj, const float* gate,
                             int32_t gate_stride, const sekv_spans* spans, hipStream_t stream);

/* Device workspace of sekv_route, in bytes (0 for an invalid configuration). */
size_t sekv_route_workspace_bytes(const sekv_config* cfg, const sekv_spans* spans);

/*
 * sekv_route - routing and compaction for one decode step.  [de-3], [zh-3]:
 * the query is scored against each span's routing summary through a sigmoid
 * relevance gate, and a per-head threshold decides expansion.  Decision for
 * query head h, span i: z > theta[b][h] (strict), where z = sum over
 * j = 0..d-1 of q[b][h][j] * rho[b][kv][i][j], evaluated in float32 in that
 * order with every product and sum rounded separately (sigma(z) > tau is
 * z > logit(tau); theta may be +/-inf).  With route_keys = 1 the score is
 * z' = fl32(z * key_scale[b][kv][i]) with z the same float32 chain over the
 * folded query q'[h][j] and kbar (sum_k) instead of q and rho, where
 * q'[h][j] = fl32(sum over m of fold[kv][j][m] * q[h][m]), a sequential fp64
 * chain in m with every product and sum rounded separately.
 *   q [B][Hq][d] dtype, theta [B][Hq] f32: device, read.
 *   exp_list [B][Hkv][seg_cap] int32: ascending span indices that any head of
 *     the group expands (first exp_count entries valid).
 *   exp_mask [B][Hkv][seg_cap] uint8: bit g set iff head kv*G+g expands it.
 *   exp_count [B][Hkv] int32.  All device, written.  A count of -1 reports
 *     that the call could not finish that group's list (an internal bounded
 *     wait ran out; not expected in normal operation): the list is then
 *     invalid and the workspace must be zero-filled again.
 *   ws: device workspace of sekv_route_workspace_bytes.  It must be
 *     zero-filled once before its first use; every call leaves it zero again.
 *     Calls that may run concurrently need workspaces of their own.
 * One kernel launch; every (b, kv) tile of 256 spans is one workgroup.
 * Errors: SEKV_EINVAL / SEKV_ESHAPE / SEKV_ECAPACITY / SEKV_EHIP.
 */
sekv_status sekv_route(sekv_ctx* ctx, const sekv_config* cfg, const sekv_spans* spans, const void* q,
                       const float* theta, int32_t* exp_list, uint8_t* exp_mask, int32_t* exp_count,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sekv_route_noalloc - sekv_route for callers that cannot allocate memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and errors as sekv_route, without the
 * workspace: the route state lives in a static device array of 1 MiB that the
 * library holds on each GPU it runs on until the process ends (created and
 * zero-filled once per device by sekv_ctx_create; every call leaves it zero).
 * Configurations whose route state (sekv_route_workspace_bytes) exceeds
 * 1 MiB are rejected with SEKV_ECAPACITY.  The call allocates nothing and
 * records no timing events.  All calls on one GPU share the array: calls that
 * may overlap on one GPU (other streams, other threads, other contexts) race
 * and must be serialized by the caller.
 */
sekv_status sekv_route_noalloc(sekv_ctx* ctx, const sekv_config* cfg, const sekv_spans* spans, const void* q,
                               const float* theta, int32_t* exp_list, uint8_t* exp_mask, int32_t* exp_count,
                               hipStream_t stream);

/*
 * sekv_reconstruct - token-level K/V of listed spans (standalone, for checks
 * and unfused use).  [de-3], [zh-3]: selected spans are rebuilt at token level;
 * K_hat = U diag(sigma*gate) Vh_K, V_hat = U diag(sigma*gate) W_V^T.
 *   exp_list, exp_count as written by sekv_route (device).
 *   tok_off [B][Hkv][seg_cap+1] int32 device, written: row offset of list entry
 *     j in the outputs (exclusive prefix of L), tok_off[count] = total rows.
 *   k_out, v_out [B][Hkv][T][d] f32 device, written: rows in list order.
 *   Host-resident factors are read directly from pinned memory.
 * Errors: SEKV_EINVAL / SEKV_ESHAPE / SEKV_EHIP.
 */
sekv_status sekv_reconstruct(sekv_ctx* ctx, const sekv_config* cfg, const sekv_spans* spans,
                             const int32_t* exp_list, const int32_t* exp_count, int32_t* tok_off,
                             float* k_out, float* v_out, hipStream_t stream);

/* Workspace sizes of sekv_mixed_attention_decode: device bytes, and pinned
 * host bytes (0 unless factors_on_host with the staged fetch).  They depend on
 * the context's split and fetch mode; ctx may be NULL (automatic split,
 * direct fetch).  0 for an invalid configuration. */
size_t sekv_decode_workspace_bytes(const sekv_ctx* ctx, const sekv_config* cfg, const sekv_spans* spans);
size_t sekv_decode_host_workspace_bytes(const sekv_ctx* ctx, const sekv_config* cfg, const sekv_spans* spans);

/* Full-resolution entries per split-K chunk of the decode (rounded up to a
 * multiple of 32); 0 (the default) lets the library choose.  The result does
 * not depend on the split beyond rounding (the log-sum-exp merge is exact in
 * real arithmetic).  Errors: SEKV_EINVAL (NULL ctx, entries outside [0, 2048]). */
sekv_status sekv_ctx_set_split(sekv_ctx* ctx, int32_t entries);

/* Fetch mode of host-resident factors (sekv_fetch_mode), default DIRECT.
 * [de-2], [de-3]: the factor tier lives in CPU memory and is loaded
 * asynchronously on expansion.  Errors: SEKV_EINVAL. */
sekv_status sekv_ctx_set_fetch_mode(sekv_ctx* ctx, int32_t mode);

/* Build mode of sekv_build_spans (sekv_build_mode), default DEVICE.
 * Errors: SEKV_EINVAL. */
sekv_status sekv_ctx_set_build_mode(sekv_ctx* ctx, int32_t mode);

/* Test hook: with SEKV_FAULT_GATHER the next staged host-resident decode of
 * this context fails its host gather after the one host wait: it returns
 * SEKV_EHIP, does not write `out`, and the context stays usable.  The fault
 * fires once.  Errors: SEKV_EINVAL. */
sekv_status sekv_ctx_inject_fault(sekv_ctx* ctx, int32_t fault);

/*
 * sekv_mixed_attention_decode - one decode step of mixed-resolution attention.
 * [de-3], [zh-3]: one softmax per query head over (a) full-resolution entries
 * (sink, anchors, tail) with logit q.k/sqrt(d); (b) for each span this head
 * does not expand, its summary with logit q.kbar/sqrt(d) + ln L_i and value
 * vbar; (c) for each span this head expands, its L_i rebuilt tokens.  The
 * rebuilt K/V never leave registers/LDS (the kernel applies the factors to the
 * query and to the softmax weights directly).
 *   q [B][Hq][d] dtype device; exp_list/exp_mask/exp_count from sekv_route.
 *   out [B][Hq][d] f32 device, written.
 *   dev_ws: device workspace (sekv_decode_workspace_bytes).
 *   host_ws: pinned host workspace (sekv_decode_host_workspace_bytes), only
 *     with factors_on_host and the staged fetch.  In that mode the call copies
 *     the list to the host and waits for it (the one host wait), gathers the
 *     listed factor blocks on host threads into host_ws, and copies them with
 *     hipMemcpyAsync on copy_stream while the full-resolution/summary pass
 *     runs on stream.  With the direct fetch the kernels read the pinned
 *     pools themselves; there is no host wait and host_ws is not used.
 *   copy_stream may be NULL (then stream is used).
 *   Device-resident factors: every kernel runs on stream, in order; no host
 *   wait (the call may be captured into a HIP graph).
 * Errors: SEKV_EINVAL / SEKV_ESHAPE / SEKV_ECAPACITY / SEKV_EHIP.
 */
sekv_status sekv_mixed_attention_decode(sekv_ctx* ctx, const sekv_config* cfg, const sekv_spans* spans,
                                        const void* q, const int32_t* exp_list, const uint8_t* exp_mask,
                                        const int32_t* exp_count, float* out, void* dev_ws,
                                        size_t dev_ws_bytes, void* host_ws, size_t host_ws_bytes,
                                        hipStream_t stream, hipStream_t copy_stream);

/*
 * sekv_decode_step - sekv_route and sekv_mixed_attention_decode of one decode
 * step in one call, with the full-resolution entries' attention (sink,
 * anchors, tail: the part that does not depend on the routing decision,
 * [de-3]) running on a second stream of the context while the route runs on
 * `stream`; the summaries, the expanded spans and the merge follow on
 * `stream` after both.  Results are bit-identical to sekv_route followed by
 * sekv_mixed_attention_decode with the same context and workspaces.
 *   Arguments as in those two calls: q, theta, exp_list/exp_mask/exp_count
 *   (written), out (written), route_ws (sekv_route_workspace_bytes, same
 *   zero-between-calls contract), dev_ws (sekv_decode_workspace_bytes).
 *   Device-resident factors or the direct host fetch only; with the staged
 *   host fetch the call returns SEKV_EINVAL.
 *   Everything the call enqueues is ordered after the work already on
 *   `stream`, and later work on `stream` is ordered after all of it (the
 *   second stream forks from and joins `stream` through events, so the call
 *   may be captured into a HIP graph).  Calls on one context must not overlap
 *   in time (they share its second stream and events).
 * Errors: as sekv_route and sekv_mixed_attention_decode; nothing is enqueued
 * when the arguments are rejected.
 */
sekv_status sekv_decode_step(sekv_ctx* ctx, const sekv_config* cfg, const sekv_spans* spans, const void* q,
                             const float* theta, int32_t* exp_list, uint8_t* exp_mask, int32_t* exp_count,
                             float* out, void* route_ws, size_t route_ws_bytes, void* dev_ws, size_t dev_ws_bytes,
                             hipStream_t stream);

/*
 * Online span sealing (decode-time layout).  [de-1], [zh-1] place span
 * boundaries at high-surprisal tokens and define the segmentation at prefill;
 * during decode new tokens keep leaving the recent window.  Reading: the
 * boundary rule of sekv_plan_spans decides token t for good once
 * t <= T - n_recent - 1 - min_span (its room before the recent window then
 * holds at every longer context, and the forced-head test never depended on
 * it); a span seals when its closing head is decided.  With cfg->sealed = 1,
 * sekv_plan_spans returns only the sealed spans of a context: heads up to that
 * token, the last of them starting the full-resolution tail (which then also
 * holds the undecided tokens and the open span's body).  Capacities (seg_cap,
 * full_cap) follow max(n_ctx, n_ctx_max), so a cache can be allocated once for
 * the longest context it will reach.
 */
size_t sekv_append_workspace_bytes(const sekv_config* cfg, const sekv_spans* spans);

/*
 * sekv_append_token - one decode step of online sealing: the context grows
 * from cfg->n_ctx to n_ctx + 1 tokens.  The new token's key and value are
 * appended to every (b, kv) full-resolution tail; the one token this step
 * decides (T + 1 - n_recent - 1 - min_span) becomes a head when its body since
 * the last sealed head has reached max_span, or when surprisal[b][t] >
 * boundary_thr[b] and the body holds at least min_span tokens; a new head
 * seals the span before it ([de-1], [zh-1]), which is then summarised, given
 * its routing key (or key scale) and factored exactly as sekv_build_spans does
 * ([de-2], [zh-2]; summaries and routing keys in the builder's fp64 operation
 * order, the rank-r factors from the fp64 Gram matrix's Jacobi eigenvectors),
 * its body rows leave the full-resolution tail and its factor block and
 * sigma|gate entry are appended to the pools.
 *   cfg: sealed = 1, basis = 0; n_ctx = T, the context before the call.
 *   spans: the cache of the sealed layout of T tokens.  Written in place:
 *     device arrays, pools (pinned host pools through their device
 *     addresses) and the host arrays n_seg_host, n_full_host, seg_off_host,
 *     rank_host, fac_off_host, sg_off_host (the pointers must be writable).
 *     Entries of seg_off (device and host) past n_seg are left as they were.
 *   k_new, v_new [B][Hkv][d] dtype: device, read.
 *   surprisal [B][s_stride] f32: host, entries [0, T] (the new token's at T).
 *   boundary_thr [B] f32: host.  route_proj [Hkv][d][d] f32: device.
 *   gate [B][Hkv][seg_cap][gate_stride] f32, rank_req [B][seg_cap]: host,
 *     indexed by span as in sekv_build_spans.
 *   fac_used, sg_used: in/out, pool elements in use (sekv_plan_spans'
 *     fac_elems / sg_elems after a build); spans->fac_elems / sg_elems are
 *     the pools' capacities.
 *   sealed_out [B] int32 host (may be NULL): 1 where a span sealed.
 *   ws: device workspace of sekv_append_workspace_bytes.
 * Enqueued on stream (small host-to-device copies, then two kernels); the
 * host arrays are updated before the call returns.  After it the cache holds
 * the sealed layout of T + 1 tokens: set cfg->n_ctx = T + 1 for later calls.
 * Errors (nothing written): SEKV_EINVAL / SEKV_ESHAPE / SEKV_ECAPACITY
 * (n_ctx_max, seg_cap, full_cap or the pools would overflow) / SEKV_EHIP.
 */
sekv_status sekv_append_token(sekv_ctx* ctx, const sekv_config* cfg, const sekv_spans* spans, const void* k_new,
                              const void* v_new, const float* surprisal, int32_t s_stride,
                              const float* boundary_thr, const float* route_proj, const float* gate,
                              int32_t gate_stride, const int32_t* rank_req, int64_t* fac_used, int64_t* sg_used,
                              int32_t* sealed_out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Device factor cache for host-resident factors.  [de-2], [abstract]: the
 * factor tier lives in CPU memory and a span's factors are loaded when it is
 * expanded; the pages name the CPU-GPU bandwidth this costs as the method's
 * limitation ("Bedeutung und Ansprüche").  The cache keeps the factor blocks
 * (factor block + sigma|gate entry) of recently expanded spans in an HBM arena
 * across decode steps and layers, so a span expanded again is read from HBM.
 *
 * Policy: the arena is cut into 2 MiB pages, split evenly among `partitions`
 * partitions; the blocks of KV group g = b * Hkv + kv belong to partition
 * g mod partitions, which manages its own pages: a block takes a slot of the
 * smallest size class that holds it (classes grow by about 1.25x from 1 KiB in
 * 256-byte steps); a class takes a free page of its partition when it has no
 * free slot, and once every page is assigned it evicts its least recently used
 * block.  Blocks used by the current call are never evicted by that call: a
 * block that finds every slot of its class in use by the call is read over the
 * bus directly (a bypass).  Blocks are keyed by (layer, g, span index); a key
 * whose host address or size changed is refilled.  After rebuilding a layer's
 * spans in place, invalidate that layer.
 *
 * sekv_factor_cache_create: an arena of floor(bytes / 2 MiB) pages on ctx's
 *   device (hipMalloc), owned by the cache; partitions 1..256, 0 for the
 *   default 8.  ctx may be NULL: then the cache has no arena and serves only
 *   sekv_factor_cache_lookup (the bookkeeping, on the host).  Errors:
 *   SEKV_EINVAL, SEKV_ESHAPE (less than one page per partition), SEKV_EHIP,
 *   SEKV_ENOMEM.
 * sekv_factor_cache_destroy: waits for the last cached decode that read the
 *   arena, then frees it.
 * sekv_factor_cache_invalidate: drops every block of `layer` (0..65535);
 *   layer = -1 drops everything and returns every page to the free pool.
 * sekv_factor_cache_stats: counters since the last reset (lookups = hits +
 *   fills + bypasses; bytes are block bytes) and the current residency;
 *   reset != 0 zeroes the counters afterwards.
 */
typedef struct sekv_factor_cache sekv_factor_cache;
typedef struct sekv_cache_stats {
  int64_t lookups, hits, fills, bypasses, evictions;
  int64_t bytes_hit, bytes_filled, bytes_bypassed;
  int64_t resident_blocks, resident_bytes;
  int64_t pages_used, pages_total;
} sekv_cache_stats;

sekv_status sekv_factor_cache_create(sekv_ctx* ctx, size_t bytes, int32_t partitions, sekv_factor_cache** out);
void sekv_factor_cache_destroy(sekv_factor_cache* cache);
sekv_status sekv_factor_cache_invalidate(sekv_factor_cache* cache, int32_t layer);
sekv_status sekv_factor_cache_stats(sekv_factor_cache* cache, sekv_cache_stats* out, int32_t reset);

/*
 * sekv_factor_cache_lookup - the cache bookkeeping of one decode call, on the
 * host only (no GPU work; what sekv_cached_attention_decode does after its
 * host wait).  Every listed entry is checked first (counts, span indices,
 * pool bounds); a bad list changes nothing.  Then the entries are looked up
 * in list order (group-major).
 *   exp_list [B][Hkv][seg_cap], exp_count [B][Hkv]: host, read.
 *   spans: only seg_cap, n_seg_host, seg_off_host, rank_host, fac_off_host,
 *     sg_off_host, fac (the tag address), fac_elems and sg_elems are read.
 *   status [B][Hkv][seg_cap] int32: host, written for entries j < count:
 *     0 hit, 1 fill (a slot was assigned; the cached decode copies the block
 *     there), 2 bypass.
 *   offset [B][Hkv][seg_cap] int64: host, written: the slot's byte offset in
 *     the arena (the sigma|gate entry follows the factor block), -1 for a
 *     bypass.
 * Errors: SEKV_EINVAL / SEKV_ESHAPE / SEKV_EHIP (list out of range).
 */
sekv_status sekv_factor_cache_lookup(sekv_factor_cache* cache, int32_t layer, const sekv_config* cfg,
                                     const sekv_spans* spans, const int32_t* exp_list, const int32_t* exp_count,
                                     int32_t* status, int64_t* offset);

/* Workspaces of sekv_cached_attention_decode: device bytes and pinned host
 * bytes (0 for an invalid configuration); ctx may be NULL (automatic split). */
size_t sekv_cached_decode_workspace_bytes(const sekv_ctx* ctx, const sekv_config* cfg, const sekv_spans* spans);
size_t sekv_cached_decode_host_workspace_bytes(const sekv_ctx* ctx, const sekv_config* cfg, const sekv_spans* spans);

/*
 * sekv_cached_attention_decode - sekv_mixed_attention_decode for host-resident
 * factors (cfg->factors_on_host = 1) through a device factor cache; the
 * result is bit-identical to the direct and staged fetches.  One call serves
 * one layer; layers of a model share one cache, each under its own `layer`
 * index (0..65535).
 *   Sequence: the list is copied to the host and the full-resolution +
 *   summary pass starts on `stream`; after the one host wait the cache
 *   bookkeeping assigns slots partition by partition, and after every
 *   quarter of the partitions a fill kernel pulls that part's missing blocks
 *   from the pinned pools into their slots on copy_stream (reading its item
 *   list from host_ws) while the host goes on; the stage table is copied;
 *   all of this runs beside the full-resolution pass; the
 *   expanded-span pass then reads hits and fills from HBM (bypassed blocks
 *   from the pinned pools), followed by the merge on `stream`.
 *   A layer's route needs that layer's query, which in a model comes from the
 *   layer below: the fill of a layer overlaps that layer's own
 *   full-resolution pass, not a later layer's.
 *   Arguments as sekv_mixed_attention_decode; dev_ws and host_ws (pinned,
 *   required) sized by the two functions above; copy_stream may be NULL.
 *   The cache must live on ctx's device.  Calls that share a context or a
 *   cache must be ordered on one stream.
 * Errors: as sekv_mixed_attention_decode; a bad route list found after the
 * host wait returns SEKV_EHIP (out not written, the cache unchanged).
 */
sekv_status sekv_cached_attention_decode(sekv_ctx* ctx, sekv_factor_cache* cache, int32_t layer,
                                         const sekv_config* cfg, const sekv_spans* spans, const void* q,
                                         const int32_t* exp_list, const uint8_t* exp_mask, const int32_t* exp_count,
                                         float* out, void* dev_ws, size_t dev_ws_bytes, void* host_ws,
                                         size_t host_ws_bytes, hipStream_t stream, hipStream_t copy_stream);

/*
 * sekv_dense_attention_decode - the dense baseline: plain softmax attention of
 * each query head over all T cached tokens (logit q.k/sqrt(d)), with the same
 * split-K matrix-core pass and log-sum-exp merge as the full-resolution part
 * of sekv_mixed_attention_decode.  It is the full-KV decode that the pages
 * compare SeKV's latency with ("Experimentelle Ergebnisse", efficiency).
 *   k [B][Hkv][T][d] dtype device (token order).
 *   v [B][Hkv][ceil(T/32)][d][32] dtype device: values in 32-token tiles, each
 *     tile transposed (value (t, j) at ((t/32)*d + j)*32 + t%32; padding
 *     entries finite).
 *   q [B][Hq][d] dtype device; out [B][Hq][d] f32 device, written.
 *   ws: device workspace of sekv_dense_workspace_bytes (contents ignored).
 * Only batch, n_ctx, head counts, head_dim and dtype of cfg are used (the
 * span fields must still pass the usual checks).  The context's split setting
 * applies.  Timed under "full" by the measurement hook.
 * Errors: SEKV_EINVAL / SEKV_ESHAPE / SEKV_ECAPACITY / SEKV_EHIP.
 */
size_t sekv_dense_workspace_bytes(const sekv_ctx* ctx, const sekv_config* cfg);
sekv_status sekv_dense_attention_decode(sekv_ctx* ctx, const sekv_config* cfg, const void* k, const void* v,
                                        const void* q, float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Measurement hook.  While enabled, sekv_route and sekv_mixed_attention_decode
 * record a timing-event pair around each of their main kernels, on the stream
 * the kernel runs on: the route kernels ("route"); the attention kernels
 * ("full": the full-resolution + summary pass, which with device-resident
 * factors and ranks up to 64 is one launch together with the expanded-span
 * pass; "expand": the expanded-span pass when it is a launch of its own).
 * sekv_profile_read waits for the recorded events,
 * returns the summed milliseconds and launch counts since the last read, and
 * resets them.  Errors: SEKV_EINVAL (NULL ctx/outputs), SEKV_EHIP.
 */
sekv_status sekv_profile_enable(sekv_ctx* ctx, int32_t enable);
sekv_status sekv_profile_read(sekv_ctx* ctx, double* route_ms, int64_t* route_launches, double* full_ms,
                              int64_t* full_launches, double* expand_ms, int64_t* expand_launches);
/* The same for the full-resolution pass that sekv_decode_step runs on its
 * second stream beside the route ("overlap"; in that call "full" times only
 * the summary + expanded-span launch). */
sekv_status sekv_profile_read_overlap(sekv_ctx* ctx, double* ms, int64_t* launches);

/* The same for the cache fill kernels of sekv_cached_attention_decode ("fill"). */
sekv_status sekv_profile_read_fill(sekv_ctx* ctx, double* ms, int64_t* launches);

/* Host-side phases of staged and cached host-resident decode calls since the
 * last read (always recorded): the host wait for the route list, the threaded
 * gather of factor blocks into pinned staging (staged) or the cache
 * bookkeeping (cached), and the whole call, in milliseconds summed over
 * `calls` calls; then reset.  Errors: SEKV_EINVAL. */
sekv_status sekv_profile_read_host(sekv_ctx* ctx, double* wait_ms, double* gather_ms, double* call_ms,
                                   int64_t* calls);

#ifdef __cplusplus
}
#endif
#endif /* SEKV_H */
