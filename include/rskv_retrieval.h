/*
 * rskv_retrieval.h - token-retrieval router for decode on AMD MI355X.
 *
 * Second router of librskv.so, beside the span router of rskv.h: instead
 * of routing spans by their summaries it retrieves single tokens, following
 * "ParisKV: Fast and Drift-Robust KV-Cache Retrieval for Long-Context
 * LLMs" (gist.science 2602.07721), section "Metodologia: Il Framework
 * ParisKV":
 *   - "Centroidi Analitici Robusti al Drift": keys and queries are
 *     l2-normalised and rotated by one random orthogonal transform (SRHT);
 *     the centroids are fixed sign patterns, independent of the data.
 *   - "Pipeline di Recupero Nativa su GPU in Due Stadi": per subspace every
 *     key sits in the bucket of its nearest centroid; the query's top-rho
 *     centroids of each subspace hand tiered votes to their buckets; the
 *     keys with the largest vote totals are the candidates; the candidates
 *     are reranked by the RSQ-IP estimate ||q|| sum_b w_b <v_b, q~_b> from
 *     4-bit codes (1 sign + 3 magnitude bits) and a per-key, per-subspace
 *     calibration w, and the best k_ret are retrieved.
 *   - the sliding-window regions (system level): Sink (first tokens) and
 *     Local (last tokens) are always attended; retrieval covers the rest.
 * Readings where the page leaves a step open:
 *   x~ = H diag(sigma) x / (||x|| sqrt(d)) with H the Sylvester Hadamard
 *   matrix and sigma the caller's signs; subspaces of m = 8 contiguous
 *   coordinates, centroid p has entry i negative iff bit i of p is set, a
 *   key's bucket is its sign pattern (zero counts as positive); retrieval
 *   runs once per KV head on the mean of its query group; the query ranks
 *   the 256 patterns by <q~_b, c_p> (ties to the lower pattern) and rank r
 *   < rho gives rho - r votes; candidates are the ceil(cand_frac N) keys of
 *   largest vote total (ties to the lower position); a code's magnitude bins
 *   are the octiles of |y|, y a coordinate of a uniform unit vector of R^m,
 *   dequantised to the bin means; w_b = ||k|| ||x~_b|| / <v_b, u_b> is
 *   stored in fp32; the estimate is formed in fp64 and the retrieval
 *   decision taken on its fp32 rounding (ties to the lower position);
 *   attention is one exact softmax per query head over Sink, retrieved and
 *   Local tokens with their stored K/V, logits <q, k> / sqrt(d).
 *
 * Conventions as in rskv.h: plain pointers and sizes, device pointers are
 * HIP allocations owned by the caller unless stated, `stream` is a
 * hipStream_t (NULL = legacy default stream), every call returns an
 * rskv_status and leaves a message for rskv_last_error().
 */
#ifndef RSKV_RETRIEVAL_H_
#define RSKV_RETRIEVAL_H_

#include <stddef.h>
#include <stdint.h>

#include "rskv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque retrieval index: the cache's own copy of K/V (Sink and Local rows
 * always in device memory, the retrieval region in device memory or in
 * pinned host memory by kv_tier), the buckets and RSQ-IP records of the
 * retrieval region, and the decode workspace. */
typedef struct rskv_retrieval rskv_retrieval;

typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads, Hq / Hkv <= 8 */
  int32_t n_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t context_len;  /* T >= 1 tokens per sequence */
  int32_t dtype;        /* RSKV_F32 or RSKV_BF16: K, V and q storage type */
  int32_t m;            /* subspace width; 8 (one byte per bucket) */
  int32_t rho;          /* centroids voted per subspace, 1..16 */
  double cand_frac;     /* candidate fraction gamma in [0, 1] */
  int32_t k_ret;        /* tokens retrieved per KV head, >= 0 */
  int32_t n_sink;       /* Sink tokens, >= 0 */
  int32_t n_local;      /* Local tokens, >= 0 */
  int32_t kv_tier;      /* RSKV_TIER_HBM or RSKV_TIER_HOST: where the
                           retrieval region's K/V rows live (host: pinned
                           memory read by the kernels over the host link,
                           as the page's unified-addressing offload) */
  rskv_allocator allocator; /* device memory of the index (rskv.h; zeroed:
                               hipMalloc / hipFree) */
} rskv_retrieval_opts;

/* Builds the index.  K, V: device [B][Hkv][T][d] in dtype (copied; the
 * caller may free them afterwards).  signs: HOST array of d entries, each
 * +1 or -1 (the SRHT's random signs).  Rotates and encodes every key of the
 * retrieval region (positions [s, l0) with s = min(n_sink, T), l0 =
 * max(s, T - n_local)).  Errors: RSKV_EINVAL for a bad option, a NULL
 * pointer, a sign not +-1, or an empty attention set (no Sink, no Local and
 * nothing retrievable); RSKV_ENOMEM; RSKV_EHIP.  On error *out is NULL and
 * nothing is leaked.  Returns after the work queued on `stream` has
 * finished, so K and V may be freed at once. */
int rskv_retrieval_build(const void* K, const void* V, const int8_t* signs,
                         const rskv_retrieval_opts* opts, void* stream, rskv_retrieval** out);

/* One decode step.  q: device [B][Hq][d] in dtype.  out: device fp32
 * [B][Hq][d].  retrieved: device int32 [B][Hkv][k_ret] or NULL; receives
 * the retrieved positions of each KV head in ascending order, padded with
 * -1 past the n_sel = min(k_ret, C) retrieved.  At most ten
 * stream-ordered launches (two when nothing can be retrieved, three to pad
 * `retrieved`), no
 * host synchronisation, no allocation; calls on one index must
 * not overlap (they share its workspace).  Errors: RSKV_ESTATE (bad
 * handle), RSKV_EINVAL (NULL q or out), RSKV_EHIP. */
int rskv_retrieval_decode(rskv_retrieval* index, const void* q, float* out, int32_t* retrieved,
                          void* stream);

typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim, context_len, dtype, m, rho, k_ret;
  int32_t n_sink;       /* effective Sink rows s = min(n_sink, T) */
  int32_t local_start;  /* l0: first Local position */
  int32_t n_retrieval;  /* N = l0 - s keys in the retrieval region */
  int32_t n_cand;       /* C = min(N, ceil(cand_frac N)), at most 2^21 */
  int32_t n_sel;        /* min(k_ret, C) retrieved per KV head */
  int32_t n_attend;     /* s + n_sel + (T - l0) tokens attended per head */
  int32_t record_bytes; /* bytes of one key's RSQ-IP record (codes + w) */
  int32_t kv_tier;
  double cand_frac;
  size_t device_bytes;  /* device memory held */
  size_t host_bytes;    /* pinned host memory held */
} rskv_retrieval_info;

int rskv_retrieval_info_get(const rskv_retrieval* index, rskv_retrieval_info* info);

/* Host copies of the index (any field may be NULL to skip it).  Units u =
 * b * Hkv + h; i indexes the retrieval region (position s + i). */
typedef struct {
  uint8_t* buckets;  /* [U][N][d/8]: bit t set iff coordinate t of the
                        rotated subspace is negative */
  uint8_t* codes;    /* [U][N][d/2]: coordinate 2c in the low nibble of
                        byte c, 2c+1 in the high one; per nibble bit 3 =
                        sign, bits 0-2 = magnitude bin */
  float* w;          /* [U][N][d/8] stored calibration */
  double* beta;      /* [9] bin boundaries of |u_t| */
  double* lambda;    /* [8] dequantised magnitudes */
} rskv_retrieval_host;

/* Synchronises with the index's last stream, then copies.  Errors:
 * RSKV_ESTATE, RSKV_EHIP. */
int rskv_retrieval_export(const rskv_retrieval* index, rskv_retrieval_host* arrays);

/* Intermediates of the last decode step, copied to host (any field NULL to
 * skip).  For testing and inspection; synchronises. */
typedef struct {
  double* q_rot;       /* [U][d] rotated unit query of each unit (q~) */
  double* q_norm;      /* [U] ||q-bar|| */
  uint8_t* votes;      /* [U][d/8][256] vote table */
  uint16_t* scores;    /* [U][N] vote totals */
  int32_t* threshold;  /* [U][2] smallest candidate score, candidates
                          taken at that score */
  int32_t* cand;       /* [U][C] candidate indices i (ascending) */
  float* est;          /* [U][C] fp32 rounding of each candidate's estimate */
  int32_t* retrieved;  /* [U][n_sel] retrieved positions (ascending) */
} rskv_retrieval_trace;

int rskv_retrieval_trace_get(const rskv_retrieval* index, rskv_retrieval_trace* trace);

/* Kernel time of the decode steps while enabled (per-dispatch start/stop
 * events, summed): [0] query rotation and vote table, [1] vote totals,
 * [2] candidate threshold and compaction, [3] rerank, [4] estimate
 * histogram, [5] crossing bin and its members, [6] exact top-k threshold,
 * [7] ordered top-k output, [8] attention, [9] merge. */
typedef struct {
  int64_t steps;
  double ms[10];
} rskv_retrieval_profile;

int rskv_retrieval_profile_enable(rskv_retrieval* index, int32_t on);
int rskv_retrieval_profile_read(rskv_retrieval* index, rskv_retrieval_profile* prof);

/* Releases the index: waits only for the work queued on its last stream,
 * then returns every device block to its allocator.  NULL is accepted. */
void rskv_retrieval_destroy(rskv_retrieval* index);

#ifdef __cplusplus
}
#endif
#endif /* RSKV_RETRIEVAL_H_ */
