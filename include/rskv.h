/*
 * rskv.h - span-routed mixed-resolution KV-cache decode for AMD MI355X.
 *
 * C ABI of librskv.so.  Plain pointers and sizes only; every device pointer
 * is a HIP device allocation owned by the caller unless stated otherwise.
 * Streams are passed as `void*` holding a hipStream_t (NULL = the legacy
 * default stream).  No C++ exception crosses this boundary: every entry
 * point returns an rskv_status and leaves a message for rskv_last_error().
 *
 * The method is SEKV's ("SEKV - KV Cache Adattiva alla Risoluzione con
 * Memoria Semantica Gerarchica", gist.science 2606.31145):
 *   - Metodologia 1 (entropy-guided segmentation): the highest-surprisal
 *     tokens are anchors kept at full resolution; the tokens between two
 *     neighbouring anchors form a span.
 *   - Metodologia 2 (dual-resolution span representation): each span keeps a
 *     normalised surprisal-weighted summary of its keys for coarse routing
 *     and a low-rank SVD basis from which its token K/V can be rebuilt.
 *   - Metodologia 3 (zoom-in): the query is projected into the routing
 *     space, a sigmoid gate scores every span, spans over the threshold are
 *     expanded, and one softmax runs over anchors (full K/V), expanded spans
 *     (rebuilt tokens) and unexpanded spans (summary plus a size
 *     correction).
 * Where the page leaves a step open, the library takes these readings:
 *   n_a = floor(p*T) anchors, ties to the lower position; lead and tail runs
 *   stay at full resolution; summary s = normalise(sum_t H_t k_t); the value
 *   of an unexpanded span is the mean of its values and its logit is
 *   <q,s>/sqrt(d) + ln|S|; routing per KV head from the mean of its query
 *   group, rho = P qbar, z = alpha <rho, s>, gate sigmoid(z - tau), expand
 *   iff z > tau, at most k_max spans (largest z, ties to the lower index);
 *   factors A = U_r S_r, W_r with r_j = min(r, |S|, d).
 */
#ifndef RSKV_H_
#define RSKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rskv_status {
  RSKV_OK = 0,
  RSKV_EINVAL = -1,     /* null pointer, bad shape or argument */
  RSKV_EDTYPE = -2,     /* unsupported dtype */
  RSKV_ENOMEM = -3,     /* device or host allocation failed */
  RSKV_ECAPACITY = -4,  /* tail capacity or k_max_cap exceeded */
  RSKV_EHIP = -5,       /* a HIP runtime call failed (message names it) */
  RSKV_ESTATE = -6      /* handle not valid (destroyed or foreign) */
} rskv_status;

typedef enum rskv_dtype {
  RSKV_F32 = 0,   /* IEEE binary32 */
  RSKV_BF16 = 1   /* bfloat16, stored values rounded to nearest, ties to even */
} rskv_dtype;

typedef struct rskv_cache rskv_cache; /* opaque, owned by the library */

/* Device-memory allocator of a cache: every device array it holds, its
 * build temporaries and its decode workspace come from here.
 *   alloc(ctx, bytes, stream): a device pointer to at least `bytes` bytes,
 *     aligned to 256 bytes, usable by work queued on `stream` (the stream
 *     of the call that allocates), or NULL on failure; the library then
 *     releases what it already holds and returns RSKV_ENOMEM.
 *   free(ctx, ptr, stream): releases a pointer that alloc returned, once
 *     the library has synchronised `stream`, the last stream that used it.
 *   ctx: passed back unchanged.
 * alloc == NULL selects hipMalloc / hipFree (hipFree may itself wait for
 * the whole device; a caching allocator such as a framework's avoids it).
 * Pinned host memory (the host tiers) is always hipHostMalloc'd. */
typedef struct rskv_allocator {
  void* (*alloc)(void* ctx, size_t bytes, void* stream);
  void (*free)(void* ctx, void* ptr, void* stream);
  void* ctx;
} rskv_allocator;

/* Shapes and options of a cache.  K, V, q and every stored array use
 * `dtype`; surprisal, ln|S|, the projection and the output are fp32. */
typedef struct rskv_build_opts {
  int32_t batch;         /* B >= 1 sequences */
  int32_t n_q_heads;     /* Hq, a multiple of n_kv_heads, Hq / Hkv <= 16 */
  int32_t n_kv_heads;    /* Hkv >= 1; query head h uses KV head h / (Hq/Hkv) */
  int32_t head_dim;      /* d in {64, 128} */
  int32_t context_len;   /* T >= 1 prefilled tokens per sequence */
  int32_t dtype;         /* rskv_dtype */
  double anchor_frac;    /* p in [0, 1]; n_a = floor(p*T), product in fp64 */
  float alpha;           /* routing gain in z = alpha <rho, s> (8 if <= 0) */
  const float* proj;     /* device fp32 [n_proj][d][d] routing projection P,
                            row-major (rho_i = sum_c P[i][c] qbar_c); NULL
                            means identity.  Copied into the cache. */
  int32_t n_proj;        /* 1 (shared) or n_kv_heads; ignored if proj NULL */
  int32_t tail_capacity; /* slots reserved for decode-time appends (>= 0) */
  int32_t k_max_cap;     /* largest k_max decode_step accepts; <= 0 means no
                            limit (at most n_spans are ever expanded) */
  int32_t factor_tier;   /* where the span factors (A_K, A_V, W_K, W_V) live:
                            RSKV_TIER_HBM, or RSKV_TIER_HOST: pinned host
                            memory that the kernels read over the host link
                            (SEKV keeps the low-rank bases in CPU memory and
                            fetches the expanded spans on demand; Metodologia
                            2 and 3).  Results are identical; only the
                            expanded spans' factors cross the link. */
  rskv_allocator allocator; /* device memory of the cache (zeroed struct:
                               hipMalloc / hipFree) */
} rskv_build_opts;

typedef enum rskv_factor_tier {
  RSKV_TIER_HBM = 0,
  RSKV_TIER_HOST = 1
} rskv_factor_tier;

/* Build a cache from prefilled contexts (Metodologia 1 and 2).
 *   surprisal: device fp32 [B][T] token surprisal H_t (no NaN).
 *   K, V:      device [B][Hkv][T][d] in opts->dtype, row-major.
 *   rank:      r >= 1 of the per-span factors.
 * Segments every sequence, writes span summaries, span value means, ln|S|,
 * rank-r SVD factors of each span's K and V (fp64 one-sided Jacobi), and a
 * packed copy of the full-resolution rows (anchors, lead and tail runs) with
 * tail_capacity free rows.  The inputs are only read.  The call copies the
 * per-sequence counts to the host to size the cache and returns after the
 * work queued on `stream` has finished, so the inputs may be freed at once.
 * On success *out receives a new cache; on failure *out is NULL. */
int rskv_build_spans(const float* surprisal, const void* K, const void* V,
                     int32_t rank, const rskv_build_opts* opts, void* stream,
                     rskv_cache** out);

/* One decode step for every (sequence, KV head) unit (Metodologia 3).
 *   q:     device [B][Hq][d] in the cache dtype.
 *   tau:   expansion threshold in logit units (may be +-inf, not NaN).
 *   k_max: 0 <= k_max <= k_max_cap, spans expanded per KV head at most.
 *   out:   device fp32 [B][Hq][d], written.
 *   sel:   device int32 [B][Hkv][k_max] or NULL: expanded span indices,
 *          ascending, -1 padded.
 *   n_sel: device int32 [B][Hkv] or NULL: number of expanded spans.
 * Asynchronous on `stream`; no host synchronisation, no allocation and no
 * memset node (three or four kernel launches), so it can be captured in a
 * HIP graph: a replay decodes the query then in the buffer `q` with the
 * tau, k_max and output pointers of the captured call.  Profiling (below)
 * must be off while capturing.  Calls on one cache must not overlap (they
 * share the cache's workspace). */
int rskv_decode_step(rskv_cache* cache, const void* q, float tau, int32_t k_max,
                     float* out, int32_t* sel, int32_t* n_sel, void* stream);

/* rskv_decode_step for callers that cannot allocate device memory or must
 * not rely on a per-cache workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same kernels and
 * results, with the decode workspace (routing scores, summary logits,
 * selection lists, work ranges, partial softmax states) taken from a
 * library-owned static device array of rskv_decode_static_capacity() bytes
 * (32 MiB) per GPU, held until the process ends, instead of the cache's
 * own.  Calls nothing that allocates (no hipMalloc, no events; profiling is
 * not recorded).  The device of the cache must be current.
 * Returns RSKV_ECAPACITY when the cache's workspace is larger than the
 * array (rskv_decode_step then still works).  Every call on one GPU shares
 * that GPU's array, so calls that overlap on one GPU race, even on
 * different caches or streams; serialise them.  No part of the array needs
 * clearing between calls (each step writes what it reads). */
int rskv_decode_step_static(rskv_cache* cache, const void* q, float tau, int32_t k_max,
                            float* out, int32_t* sel, int32_t* n_sel, void* stream);

/* Bytes of the static decode workspace array of one GPU. */
size_t rskv_decode_static_capacity(void);

/* Routing scores of the last rskv_decode_step on this cache (Metodologia
 * 3: the gate's argument before the threshold), z_j = alpha <rho, s_j> in
 * fp64, copied to the host array z [B][Hkv][S] (S = n_spans_max of
 * rskv_cache_info; entries past n_spans[b] are unspecified), and the span
 * counts of that step to the host array n_spans [B] (or NULL).
 * Synchronous: waits for the cache's last stream.  Meant for reports on
 * selection ambiguity (scores within a band of tau or of the k-th largest
 * score). */
int rskv_decode_scores(const rskv_cache* cache, double* z, int32_t* n_spans);

/* Append one decoded token per sequence, with streaming segmentation
 * (Metodologia 1 applied to decoded tokens; the page fixes the anchor rule
 * only for a whole context, and the library reads it this way):
 *   k, v: device [B][Hkv][d] in the cache dtype.
 *   h:    device fp32 [B] surprisal of the new tokens, or NULL (then every
 *         token counts as surprisal 0 and is never an anchor).
 * The token joins the full-resolution rows at position T + (appends so
 * far).  It is an anchor iff h[b] > theta_b, the smallest surprisal among
 * the prefill anchors of sequence b (no decoded anchor when the prefill had
 * none).  Before a decoded anchor is stored, the non-empty run of
 * full-resolution rows after the previous anchor becomes a new span j =
 * n_spans[b], exactly as the build would make it from a run between two
 * anchors (summary weighted by the rows' surprisal, value mean, ln|S|,
 * rank-r factors of the stored rows), and those rows leave the
 * full-resolution set.  Later decode steps route and attend the new span
 * like any other; span_id covers only the prefill positions.
 * Returns RSKV_ECAPACITY when tail_capacity appends have already been made.
 * Asynchronous on `stream` (two kernel launches when h is given and some
 * sequence has an anchor, else one); no allocation.  Must not overlap a
 * decode step or another append on the same cache. */
int rskv_append_token(rskv_cache* cache, const void* k, const void* v, const float* h,
                      void* stream);

/* rskv_append_token with h = NULL: the token joins the trailing
 * full-resolution run (attended at full resolution, never routed). */
int rskv_append_kv(rskv_cache* cache, const void* k, const void* v, void* stream);

/* Sizes of a cache.  S, F and N are the padded dimensions of the exported
 * arrays: S >= every n_spans[b], F >= every n_full[b] + remaining tail
 * capacity, N >= every n_span_tokens[b], including the spans and span
 * tokens that decoded anchors may still add (with a tail capacity t, at
 * most ceil(t/2) more spans per sequence). */
typedef struct rskv_cache_info {
  int32_t batch, n_q_heads, n_kv_heads, head_dim, context_len, rank, dtype;
  int32_t n_spans_max;       /* S */
  int32_t n_full_cap;        /* F */
  int32_t n_span_tokens_max; /* N */
  int32_t tail_capacity, appended, k_max_cap;
  float alpha;
  size_t device_bytes;       /* HBM held by the cache, workspace included */
  int32_t factor_tier;       /* rskv_factor_tier */
  size_t host_bytes;         /* pinned host memory held (host factor tier) */
} rskv_cache_info;

int rskv_cache_info_get(const rskv_cache* cache, rskv_cache_info* info);

/* Host arrays of a cache in the canonical layout (row-major, padding zero;
 * padding of the int32 tables is 0, of full_pos -1).  Element type of the
 * `void*` members is the cache dtype.  The caller owns every buffer. */
typedef struct rskv_host_arrays {
  int32_t* n_anchor;       /* [B] */
  int32_t* n_spans;        /* [B] */
  int32_t* n_full;         /* [B] full-resolution rows incl. appended ones */
  int32_t* n_span_tokens;  /* [B] sum of span lengths */
  int32_t* span_id;        /* [B][T]: j in span j, -1 anchor, -2 lead/tail */
  int32_t* span_start;     /* [B][S] first position of span j */
  int32_t* span_len;       /* [B][S] |S_j| */
  int32_t* full_pos;       /* [B][F] position of full-resolution row i
                              (appended token a has position T + a) */
  void* summary;           /* [B][Hkv][S][d] s_j */
  void* vmean;             /* [B][Hkv][S][d] mean value of span j */
  float* log_len;          /* [B][S] ln|S_j| */
  void* k_full;            /* [B][Hkv][F][d] */
  void* v_full;            /* [B][Hkv][F][d] */
  void* a_k;               /* [B][Hkv][N][r] rows of span j start at
                              sum_{i<j} |S_i|; A = U_r S_r */
  void* a_v;               /* [B][Hkv][N][r] */
  void* w_k;               /* [B][Hkv][S][r][d] row k = k-th right singular
                              vector; K-hat of span j = A_K(j) @ W_K(j) */
  void* w_v;               /* [B][Hkv][S][r][d] */
  /* streaming segmentation state (see rskv_append_token) */
  float* h_full;           /* [B][F] surprisal of full-resolution row i
                              (0 for tokens appended without one) */
  float* theta;            /* [B] anchor threshold, +inf without anchors */
  int32_t* last_anchor;    /* [B] full-resolution row of the last anchor, -1 */
} rskv_host_arrays;

/* Copy every stored array of the cache to host memory (synchronous). */
int rskv_cache_export(const rskv_cache* cache, rskv_host_arrays* arrays);

/* Create a cache from host arrays in the canonical layout (padded with the
 * given S, F, N; F counts rows, the new cache adds opts->tail_capacity).
 * h_full, theta and last_anchor may be NULL: then no decoded token is an
 * anchor (theta = +inf, last_anchor = -1, h_full = 0).
 * Lets tests and benchmarks decode on a cache built elsewhere.  K/V inputs
 * are not needed, and opts->proj, if given, is a HOST pointer here.
 * Synchronous. */
int rskv_cache_import(const rskv_host_arrays* arrays, const rskv_build_opts* opts,
                      int32_t rank, int32_t S, int32_t F, int32_t N, void* stream,
                      rskv_cache** out);

/* Release the cache and its device memory.  Waits only for the work queued
 * on the cache's last stream (the stream of its last build, decode or append
 * call), then returns every allocation to the cache's allocator; work on
 * other streams is not waited for (hipFree, the default allocator's release,
 * may still wait for the device on its own).  NULL is accepted. */
void rskv_cache_destroy(rskv_cache* cache);

/* Per-kernel timing of decode_step: each of its four kernels (routing GEMV,
 * top-k cap, attention partials, merge) is dispatched with a start and a stop
 * HIP event of its own, so the totals are kernel execution times (the gaps
 * between launches are not included); the same holds for the two kernels of
 * rskv_append_token.  Enabling clears the totals. */
typedef struct rskv_profile {
  int64_t steps;
  double route_ms, topk_ms, attend_ms, merge_ms; /* summed over steps */
  int64_t appends;                /* rskv_append_token calls recorded */
  double close_ms, append_ms;     /* span-closing and append kernels */
} rskv_profile;

int rskv_profile_enable(rskv_cache* cache, int32_t on);
/* Synchronises the recorded events and returns the totals. */
int rskv_profile_read(rskv_cache* cache, rskv_profile* prof);

/* Message of the last failing call on this thread ("" if none). */
const char* rskv_last_error(void);

/* Library version string. */
const char* rskv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RSKV_H_ */
