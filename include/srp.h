/*
 * srp.h -- C ABI of libsrp.so, the selective-recompute prefill layer ("KV cache
 * fusor") for AMD MI355X (gfx950).
 *
 * One layer of the method: the concatenated, independently precomputed KV caches
 * of retrieved chunks are moved to their global positions, a subset of token rows is
 * recomputed, chosen by KV deviation, their fresh K/V overwrite the cache, and the
 * selected rows attend over the whole fused cache (CacheBlend walkthrough,
 * "Selective KV recompute" and "Implementation"; CacheClip paper, sections 4.1-4.3).
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers owned by the caller, row-major and
 *    contiguous. The library keeps no pointer after a call returns.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream). No
 *    entry point synchronises the host except srp_validate_batch. Outputs are valid
 *    once the caller has synchronised with the stream.
 *  - Return value: SRP_OK (0) or a negative srp_status. Host-checkable errors are
 *    reported before anything is enqueued; srp_last_error() returns a message for
 *    the last failure on the calling thread. No exception or abort crosses the ABI.
 *  - Device arrays (offsets, positions, candidate lists) are trusted: malformed
 *    contents give undefined results. srp_validate_batch checks them on request.
 *  - Identical inputs give bitwise-identical outputs (no floating-point atomics).
 */
#ifndef SRP_H_
#define SRP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *srp_stream_t; /* hipStream_t */

/* Status codes. A call reports failure by a negative return value, as the
 * CacheBlend walkthrough's loader does ("Implementation": fetch_kv returns -1 when a
 * chunk's cache is missing); the codes below tell the failures apart. */
typedef enum {
  SRP_OK = 0,
  SRP_E_INVALID = -1,     /* bad argument (shape, dtype, ratio, null pointer...)  */
  SRP_E_WORKSPACE = -2,   /* workspace smaller than srp_workspace_size()          */
  SRP_E_UNSUPPORTED = -3, /* valid but not implemented (e.g. head_dim 96)          */
  SRP_E_HIP = -4,         /* a HIP runtime call failed                            */
  SRP_E_BATCH = -5        /* srp_validate_batch found malformed device arrays     */
} srp_status;

typedef enum { SRP_F32 = 0, SRP_BF16 = 1 } srp_dtype;

/* Selection modes (CacheBlend walkthrough, "Implementation": a per-layer
 * check_flag says whether the layer selects tokens by deviation or uses the
 * indices it was given; CacheClip paper 4.2 and SpecCache notes 2.2 rank tokens by
 * scores from a small auxiliary model instead). */
typedef enum {
  SRP_SEL_TOPK = 0,  /* score candidates by KV deviation, keep the top k      */
  SRP_SEL_GIVEN = 1, /* keep the candidates as given (no scoring)            */
  SRP_SEL_SCORES = 2 /* rank candidates by caller-supplied per-row scores;
                        only the chosen rows are recomputed                  */
} srp_sel_mode;

/* How k follows from the ratio: round half up (CacheClip walkthrough 6.2) or
 * ceiling (SpecCache notes 2.2); the product ratio * N is taken in double. */
typedef enum { SRP_K_ROUND = 0, SRP_K_CEIL = 1 } srp_k_rule;

/* What the deviation measures (the CacheBlend walkthrough compares K and V; the
 * CacheClip paper's account of CacheBlend compares value matrices only). */
typedef enum { SRP_DEV_KV = 0, SRP_DEV_V = 1 } srp_dev_mode;

/* Model shape of one layer. Weights W_qkv are [(nh + 2 nkv) * d, hidden]: the
 * n_heads*d query rows, then n_kv_heads*d key rows, then n_kv_heads*d value rows,
 * each row one output feature (so Q = X W_q^T). Rotary embedding: rotate-half
 * pairing (i, i + d/2), angle p * rope_base^(-2i/d). Supported: head_dim 64 or
 * 128, n_heads a multiple of n_kv_heads with at most 8 query heads per KV head
 * (SRP_E_UNSUPPORTED beyond), hidden a multiple of 64. */
typedef struct {
  int32_t hidden;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  double rope_base;
  int32_t dtype; /* srp_dtype: storage and compute type of every tensor */
} srp_dims;

/* A varlen batch of total_rows token rows (CacheClip paper 4.1: concatenated chunk
 * caches with rearranged position IDs). Rows are partitioned into requests and,
 * independently, into segments; every segment lies inside one request. A segment
 * is a cached chunk whose first row was encoded at position chunk_src_pos[c] (its
 * rows at consecutive positions), or a fresh segment (chunk_src_pos[c] = -1: the
 * query tail or a chunk whose cache is missing), whose rows are always recomputed
 * and whose input cache rows are ignored.
 *
 * Cache layout. block_rows = 0: row j of the batch is row j of k_cache / v_cache.
 * block_rows > 0 (paged; Cache-Craft summary, section 4: each chunk maps to
 * 16-token memory blocks through address pointers, padded at its end): k_cache /
 * v_cache point at a pool of blocks of block_rows rows, and row i of segment c
 * lives at pool row block_table[seg_block[c] + i / block_rows] * block_rows +
 * i % block_rows. Fresh segments need blocks too (their fresh K/V are written
 * there). Distinct rows must map to distinct pool rows (srp_validate_batch checks
 * this). Only srp_fuse_layer, srp_rerotate_kv and srp_fuse_stack without host
 * loads read this layout; srp_encode_kv writes rows contiguously. */
typedef struct {
  int32_t n_req;        /* host: number of requests (>= 1)                         */
  int32_t n_chunks;     /* host: number of segments (>= 1)                         */
  int32_t total_rows;   /* host: T (>= 0)                                          */
  int32_t max_req_rows; /* host: upper bound on the rows of any one request        */
  int32_t max_position; /* host: every position, encode position and |pos - src|
                           is < max_position (sizes the rotary tables)            */
  const int32_t *req_offsets;   /* device [n_req+1], req_offsets[0] = 0,
                                   req_offsets[n_req] = T, non-decreasing          */
  const int32_t *chunk_offsets; /* device [n_chunks+1], same rules               */
  const int32_t *chunk_src_pos; /* device [n_chunks], >= 0 cached, -1 fresh       */
  const int32_t *positions;     /* device [T], global positions, strictly
                                   increasing inside each request                 */
  int32_t block_rows;           /* host: 0 = contiguous cache rows; else the rows
                                   per block of a paged cache pool (16 on the
                                   pages), 1..4096                               */
  const int32_t *seg_block;     /* device [n_chunks], paged only: index into
                                   block_table of each segment's first block      */
  const int32_t *block_table;   /* device, paged only: pool block ids             */
} srp_batch;

/* Token selection of one layer. k = round(ratio * N_ctx) per request (halves up;
 * k_rule SRP_K_CEIL: ceil), N_ctx = the request's cached rows, clamped to its
 * candidate count (CacheClip walkthrough 6.2). Ties in the ranking go to the lower
 * row index. window > 0 turns on sliding-window grouping (CacheClip paper 4.3): over
 * the request's cached rows in order, a window of `window` rows starting on a top-k
 * row that holds at least `tau` top-k rows is recomputed whole; top-k rows covered
 * by no such window are dropped. Grouping requires cand == NULL. Candidates
 * (gradual filtering across layers, CacheBlend walkthrough "The chicken-and-egg
 * problem"): cand == NULL means every cached row; otherwise cand/cand_offsets is a
 * CSR list per request of row ids, ascending inside each request -- the
 * sel_idx/sel_offsets of the previous layer can be passed as is (fresh rows in it
 * are ignored, they are always recomputed).
 *
 * SRP_SEL_SCORES ranks the candidates by scores[row] (device, fp32, finite; e.g.
 * an auxiliary model's attention column means, CacheClip paper 4.2, or its
 * deep-layer hidden-state norms, SpecCache notes 2.2) and keeps the top k; grouping
 * then applies as above, or span completion (SpecCache notes 2.3) when span_max > 0:
 * the request's cached rows in order are cut into spans of at most span_max rows,
 * a row joining its predecessor's span while |s~_j - s~_i| / s~_i < tau_smooth for
 * the min-max normalised scores s~ (evaluated in double; a NaN or infinite change
 * starts a new span); every span in which the top-k rows make up a share >=
 * tau_cover (in double) is added whole; then, if cap_ratio > 0, only the
 * k(cap_ratio) highest-scored rows of the result are kept. Span completion requires
 * cand == NULL and window == 0; SCORES mode requires max_req_rows <= 22528. The
 * rows not chosen are not recomputed; dev_out then reports the deviation of the
 * chosen cached rows.
 *
 * fresh_all = 1 writes fresh K/V into the cache for every recomputed row (every
 * candidate in TOPK mode), not only the selected ones, as in the CacheBlend
 * walkthrough's figure of gradual filtering; attention and sel_idx are unchanged
 * by it. All fields past cand_offsets are zero for the defaults. */
typedef struct {
  int32_t mode;     /* srp_sel_mode                                             */
  double ratio;     /* in [0, 1]                                                */
  int32_t window;   /* 0 = no grouping                                          */
  int32_t tau;      /* grouping threshold, 1 <= tau <= window                   */
  int32_t dev_mode; /* srp_dev_mode                                             */
  const int32_t *cand;        /* device, NULL = all cached rows                  */
  const int32_t *cand_offsets; /* device [n_req+1], required with cand            */
  int32_t k_rule;   /* srp_k_rule                                               */
  int32_t span_max; /* SCORES: 0 = no span completion, else 1..1024 (pages: 16) */
  const float *scores; /* device [T], SCORES mode only (NULL otherwise)          */
  double tau_smooth;   /* span segmentation threshold, >= 0 (pages: 0.4)        */
  double tau_cover;    /* span coverage threshold, in [0, 1] (pages: 0.7)       */
  double cap_ratio;    /* budget after completion: 0 = none, else in [ratio, 1] */
  int32_t fresh_all;   /* 0 or 1                                                */
} srp_select;

/* Bytes of device scratch that srp_fuse_layer needs for these arguments (written
 * to *bytes). No passage of the pages defines this call: it is the engineering
 * convention that keeps allocation off the hot path (the caller allocates once and
 * reuses the buffer across layers, as the per-layer calls of the CacheBlend
 * walkthrough's "Implementation" run back to back). Host arithmetic only; the same
 * argument checks as srp_fuse_layer, with the same error codes. */
int srp_workspace_size(const srp_dims *dims, const srp_batch *batch,
                       const srp_select *sel, size_t *bytes);

/* One fused layer (CacheBlend walkthrough, "Selective KV recompute": mask the input
 * to the selected rows, project Q/K/V, expand K/V with the reused rows, attend).
 *   hidden    [T, hidden]                 layer input
 *   w_qkv     [(nh+2nkv)*d, hidden]       weights (layout above)
 *   k_cache   [T, nkv, d]  in/out         in: K of cached rows at their encode
 *             positions; out: fused K (re-rotated cache rows, fresh K on
 *             selected rows)
 *   v_cache   [T, nkv, d]  in/out         in: cached V; out: fused V
 *   sel_idx   [T] out                     selected rows, ascending per request,
 *             fresh rows included; only the first sel_offsets[n_req] are written
 *   sel_offsets [n_req+1] out             CSR offsets of sel_idx per request
 *   attn_out  [T, nh, d] out              attention output of selected row
 *             sel_idx[s] in row s; rows past sel_offsets[n_req] are not written
 *   dev_out   [T] out, optional (NULL)    fp32 deviation per row, NaN where the
 *             row was not scored
 *   workspace device scratch of workspace_bytes >= srp_workspace_size()
 * k_cache/v_cache are updated in place: a caller that must keep its stored chunk
 * caches intact passes a copy (Cache-Craft summary, section 4: the fixed cache is
 * swapped in only after use). */
int srp_fuse_layer(const srp_dims *dims, const srp_batch *batch,
                   const srp_select *sel, const void *hidden, const void *w_qkv,
                   void *k_cache, void *v_cache, int32_t *sel_idx,
                   int32_t *sel_offsets, void *attn_out, float *dev_out,
                   void *workspace, size_t workspace_bytes, srp_stream_t stream);

/* srp_fuse_layer without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, outputs and errors as srp_fuse_layer minus
 * workspace / workspace_bytes. Its scratch space (the layer's workspace with 16
 * split-K partial-tile slots instead of 256, and a rotary table built on the device
 * for the call's head_dim, rope_base and max_position) lives in a static device
 * array of 128 MiB that every GPU the library runs on holds until the process
 * ends; the call allocates nothing. A layer whose scratch exceeds 128 MiB gets
 * SRP_E_WORKSPACE before anything is enqueued (bf16, head_dim 128: about 5,600 rows
 * at hidden 8192 with 64/8 heads, 7,600 at 5120 with 40/8, 8,600 at 4096 with
 * 32/8). Every call on one GPU uses that GPU's
 * one array, which keeps the last call's contents (the next call sets everything it
 * reads before reading it): calls that overlap on one GPU (different streams or
 * threads) race and must be serialised by the caller. */
int srp_fuse_layer_noalloc(const srp_dims *dims, const srp_batch *batch,
                           const srp_select *sel, const void *hidden, const void *w_qkv,
                           void *k_cache, void *v_cache, int32_t *sel_idx,
                           int32_t *sel_offsets, void *attn_out, float *dev_out,
                           srp_stream_t stream);

/* Offline chunk encoding (CacheClip walkthrough, Figure 4, offline phase: each
 * chunk's KV cache is computed once, at chunk-local positions):
 *   k_out[j] = R(positions[j]) W_k hidden[j],  v_out[j] = W_v hidden[j]
 * for j < n_rows. hidden [n_rows, hidden], positions device [n_rows] with
 * 0 <= positions[j] < max_position; k_out, v_out [n_rows, nkv, d]. */
int srp_encode_kv(const srp_dims *dims, int32_t n_rows, int32_t max_position,
                  const void *hidden, const void *w_qkv, const int32_t *positions,
                  void *k_out, void *v_out, srp_stream_t stream);

/* Positional recovery alone (CacheBlend walkthrough, "Selective KV recompute";
 * SpecCache notes 2.1): every cached row's K is rotated in place from its encode
 * position to its global position, K <- R(pos - src) K. Fresh rows and V are not
 * touched. Equals srp_fuse_layer's cache output at ratio 0 without fresh rows. */
int srp_rerotate_kv(const srp_dims *dims, const srp_batch *batch, void *k_cache,
                    srp_stream_t stream);

/* Chain step between stacked layers (CacheBlend walkthrough, "The chicken-and-egg
 * problem": the rows a layer recomputes carry their hidden state into the next
 * layer, which checks only them; "The system": the fusor runs the layers one after
 * another). The pages give no block internals; the step taken is a unit-weight
 * RMSNorm after the residual. For every selected row
 * j = sel_idx[s], s < sel_offsets[n_req]:
 *   hidden[j] <- y / sqrt(mean(y^2) + eps),  y = hidden[j] + attn_out[s]
 * (requires n_heads * head_dim == hidden, else SRP_E_INVALID). hidden [T, hidden]
 * is updated in place; attn_out [sel_capacity, n_heads, head_dim] holds the layer's
 * attention rows in sel_idx order; sel_idx / sel_offsets are device arrays as
 * srp_fuse_layer writes them. sel_capacity bounds sel_offsets[n_req] (normally T);
 * rows past it are ignored. Enqueued on `stream`; SRP_E_INVALID on a NULL pointer,
 * n_req < 1 or eps < 0. */
int srp_residual_rmsnorm(const srp_dims *dims, void *hidden, const void *attn_out,
                         const int32_t *sel_idx, const int32_t *sel_offsets,
                         int32_t n_req, int32_t sel_capacity, float eps,
                         srp_stream_t stream);

/* ------------------------------------------------------------------------- */
/* A stack of layers with its caches loaded from host memory while it runs.    */
/* ------------------------------------------------------------------------- */

/* One layer of srp_fuse_stack. */
typedef struct {
  const void *w_qkv;  /* device [(nh+2nkv)*d, hidden] weights (layout above)          */
  void *k_cache;      /* device [T, nkv, d]: the layer's chunk caches, fused in place */
  void *v_cache;      /* device [T, nkv, d]                                            */
  const void *k_host; /* host [T, nkv, d] copied into k_cache before the layer runs;
                         page-locked memory (hipHostMalloc) for an asynchronous copy;
                         NULL: k_cache already holds the cache                        */
  const void *v_host; /* same for V; given exactly when k_host is                      */
  double ratio;       /* the layer's recompute ratio, in [0, 1]                        */
  int32_t mode;       /* layers >= 1 (CacheBlend walkthrough, "Implementation": the
                         per-layer check_flag): SRP_SEL_TOPK (0) checks the layer, ranking
                         the previous layer's selection by KV deviation at `ratio`;
                         SRP_SEL_GIVEN recomputes exactly the previous layer's selection
                         (ratio unused). Layer 0 selects with `first` instead.          */
} srp_layer;

/* Bytes of device scratch that srp_fuse_stack needs (written to *bytes):
 * srp_workspace_size plus room for the candidate list carried from layer to layer
 * (CacheBlend walkthrough, "Implementation": the per-layer dictionary passes the
 * indices chosen by one layer to the next). The allocation itself is the same
 * engineering convention as srp_workspace_size. Host arithmetic only; errors as for
 * srp_workspace_size. */
int srp_stack_workspace_size(const srp_dims *dims, const srp_batch *batch,
                             const srp_select *first, size_t *bytes);

/* n_layers stacked layers with gradual filtering (CacheBlend walkthrough, "The
 * chicken-and-egg problem") and their cache loads overlapped with the recompute
 * (CacheBlend walkthrough, "Making the recompute free": a layer can be recomputed as
 * soon as its cache has landed in GPU memory; Cache-Craft summary, section 4: the
 * caches of later layers are loaded ahead).
 *   Layer 0 selects with `first` (its ratio field is ignored; layers[0].ratio
 *   applies); layer l >= 1 starts from the previous layer's selection (fresh rows
 *   are always recomputed) and, with layers[l].mode SRP_SEL_TOPK, ranks it by KV
 *   deviation at layers[l].ratio with first's dev_mode, k_rule and fresh_all, or,
 *   with SRP_SEL_GIVEN, recomputes it as it is (check on the first layers, then pass
 *   the indices on). After every layer hidden[j] <- RMSNorm(hidden[j] +
 *   attn[j]) on its selected rows (srp_residual_rmsnorm, eps rms_eps), so hidden
 *   ends as the stack's output. sel_idx, sel_offsets and attn_out end as the last
 *   layer's; every layer's fused cache stays in its k_cache / v_cache.
 *   Loads: the host key caches are copied on copy_stream in layer order and the
 *   value caches on a second copy stream that the library creates once per device
 *   (default priority, kept until the process ends), each layer's copies followed by
 *   events that `stream` waits for before that layer, so the loads of layer l+1 run
 *   while layer l computes and the two copy engines share the link. The copies are
 *   not ordered after earlier work: when the call is made, no pending work on any
 *   stream may still use a destination k_cache / v_cache (a caller issuing stacks
 *   back to back alternates two sets of destinations, or waits for the call before
 *   last). Making a copy stream wait for pending work on the compute stream was
 *   measured to stall the host inside hipMemcpyAsync for milliseconds at times, which
 *   idles the GPU. copy_stream == stream (e.g. both NULL) puts all copies in line,
 *   ordered as usual. Work is only enqueued: synchronising with `stream` covers the
 *   copies too. The host caches must stay valid until then.
 * Errors as for srp_fuse_layer; nothing is enqueued when an argument check fails. */
int srp_fuse_stack(const srp_dims *dims, const srp_batch *batch, const srp_select *first,
                   int32_t n_layers, const srp_layer *layers, void *hidden, float rms_eps,
                   int32_t *sel_idx, int32_t *sel_offsets, void *attn_out, void *workspace,
                   size_t workspace_bytes, srp_stream_t stream, srp_stream_t copy_stream);

/* The loading controller's recompute ratio (CacheBlend walkthrough, "Making the
 * recompute free"): recompute delay = ratio x full_layer_ms (the profiled full
 * prefill of a layer), load delay = load_ms (a layer's KV bytes over the measured
 * load throughput); *ratio = the ratio at which the two are equal, raised to r_floor
 * (15% on the page) and capped at 1. Host arithmetic only. SRP_E_INVALID unless
 * full_layer_ms > 0, load_ms >= 0 and 0 <= r_floor <= 1. */
int srp_controller_ratio(double full_layer_ms, double load_ms, double r_floor, double *ratio);

/* Debug check of a batch's device arrays against the rules of srp_batch (copies
 * them to the host and synchronises `stream`). SRP_OK or SRP_E_BATCH with a
 * message. No passage of the pages defines it: it is the engineering counterpart of
 * the synchronisation point that the CacheBlend walkthrough's "Implementation" puts
 * before each layer (synchronize), a place where device-side layout errors can be
 * reported to the host instead of giving undefined results. The only entry point
 * that blocks the host. */
int srp_validate_batch(const srp_batch *batch, srp_stream_t stream);

/* Stage timing (the pages report per-stage latency breakdowns of this path, e.g.
 * the CacheClip paper's Table 6). After srp_profile_begin(max_calls), each of the
 * next max_calls srp_fuse_layer calls records hipEvents on its stream between its
 * SRP_N_STAGES launch stages (events only, the kernels are unchanged).
 * srp_profile_end waits for those events and writes ms[c * SRP_N_STAGES + i], the
 * GPU time of stage i of call c, for up to max_calls calls (*n_calls = number
 * written). Stage names: srp_profile_stage_name(i). Process-wide; not meant for
 * concurrent callers. */
#define SRP_N_STAGES 6
int srp_profile_begin(int32_t max_calls);
int srp_profile_end(float *ms, int32_t max_calls, int32_t *n_calls);
const char *srp_profile_stage_name(int32_t i);

/* Message for the last failing call on this thread ("" if none; the pointer stays
 * valid until the thread's next libsrp call). Engineering convention that goes with
 * the negative status codes (CacheBlend walkthrough, "Implementation": fetch_kv
 * reports a miss as -1): the code says what kind of failure, this says which
 * argument. */
const char *srp_last_error(void);

/* Library version string (static storage). Engineering convention; no passage of
 * the pages defines it. */
const char *srp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SRP_H_ */
