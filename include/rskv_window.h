/*
 * rskv_window.h - window-routed three-tier KV cache for decode on AMD MI355X.
 *
 * Third router of librskv.so, beside the span router of rskv.h and the
 * token-retrieval router of rskv_retrieval.h.  It follows the QEvict summary
 * ("QEvict", gist.science 2608.05326), section "Metodologia: QEvict" and its
 * key mechanisms:
 *   - the cached history is cut into contiguous windows, and routing
 *     decisions are taken per window, not per token;
 *   - under a fixed memory budget every window is in one of three tiers:
 *     full precision, a recoverable low-bit tier (INT2) that is still
 *     attended and may be promoted back, or evicted for good;
 *   - a window's importance is its attention mass accumulated over the
 *     routing events; windows whose importance falls are demoted, INT2
 *     windows whose importance rises are dequantised and promoted;
 *   - write-once ledger: a window is quantised once, at its first demotion,
 *     and that code serves every later promotion and demotion.
 * Readings where the page leaves a step open:
 *   windows of RSKV_WINDOW_ROWS = 64 positions (the last one may be
 *   shorter); the budget is given as window counts n_full and n_quant per KV
 *   head; before the first routing event every window is full precision;
 *   routing events at decode steps 0, R, 2R, ...: the step attends with the
 *   tiers in force, adds every window's attention mass (softmax
 *   probabilities of the KV head's query group, summed over the heads and
 *   the window's positions) to its score, then ranks the windows not evicted
 *   by score (descending, ties to the lower window): the first n_full are
 *   full precision, the next n_quant INT2, the rest evicted; INT2 code per
 *   position and group of RSKV_WINDOW_GROUP = 64 coordinates, for K and V
 *   alike: mn = min, scale = (max - min) / 3, code = rint((x - mn) / scale)
 *   clamped to 0..3 (0 when scale = 0), all in fp32, dequantised value
 *   mn + code * scale (product and sum each rounded to fp32); promotion
 *   stores the dequantised values rounded to the cache dtype; attention per
 *   query head is one softmax over the full and INT2 windows (INT2 windows
 *   with their dequantised values), logits <q, k> / sqrt(d).
 *
 * Conventions as in rskv.h: plain pointers and sizes, device pointers are
 * HIP allocations owned by the caller unless stated, `stream` is a
 * hipStream_t (NULL = legacy default stream), every call returns an
 * rskv_status and leaves a message for rskv_last_error().
 */
#ifndef RSKV_WINDOW_H_
#define RSKV_WINDOW_H_

#include <stddef.h>
#include <stdint.h>

#include "rskv.h"

#ifdef __cplusplus
extern "C" {
#endif

#define RSKV_WINDOW_ROWS 64   /* positions per window */
#define RSKV_WINDOW_GROUP 64  /* coordinates per INT2 scale group */

/* Tier of a window. */
enum {
  RSKV_TIER_FULL = 0,
  RSKV_TIER_INT2 = 1,
  RSKV_TIER_EVICTED = 2
};

/* Opaque window cache: its own copy of K/V (the full-precision store), the
 * INT2 ledger, tiers, scores and the decode workspace. */
typedef struct rskv_window rskv_window;

typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads, Hq / Hkv <= 16 */
  int32_t n_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t context_len;  /* T >= 1 positions per sequence, at most 2^20 */
  int32_t dtype;        /* RSKV_F32 or RSKV_BF16: K, V and q storage type */
  int32_t n_full;       /* windows per KV head kept at full precision by a
                           routing event, >= 0 */
  int32_t n_quant;      /* windows per KV head kept in INT2 by a routing
                           event, >= 0; n_full + n_quant >= 1 */
  int32_t route_every;  /* R >= 1: routing events at steps 0, R, 2R, ... */
  rskv_allocator allocator; /* device memory of the cache (rskv.h; zeroed:
                               hipMalloc / hipFree) */
} rskv_window_opts;

/* Builds the cache.  K, V: device [B][Hkv][T][d] in dtype (copied; the
 * caller may free them afterwards).  Every window starts full precision
 * with score 0 and no ledger entry.  Errors: RSKV_EINVAL for a bad option
 * or a NULL pointer; RSKV_ENOMEM; RSKV_EHIP.  On error *out is NULL and
 * nothing is leaked.  Returns after the work queued on `stream` has
 * finished, so K and V may be freed at once. */
int rskv_window_build(const void* K, const void* V, const rskv_window_opts* opts, void* stream,
                      rskv_window** out);

/* One decode step.  q: device [B][Hq][d] in dtype.  out: device fp32
 * [B][Hq][d].  Attends with the tiers in force; when the step is a routing
 * event it then updates the scores, re-tiers, quantises the windows demoted
 * for the first time into the ledger and restores promoted windows.  At
 * most three stream-ordered launches on other steps, five on routing
 * events; no host
 * synchronisation, no allocation; calls on one cache must not overlap (they
 * share its workspace and state).  Errors: RSKV_ESTATE (bad handle),
 * RSKV_EINVAL (NULL q or out), RSKV_EHIP. */
int rskv_window_decode(rskv_window* cache, const void* q, float* out, void* stream);

typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim, context_len, dtype;
  int32_t n_full, n_quant, route_every;
  int32_t n_windows;     /* nW = ceil(T / 64) per KV head */
  int64_t step;          /* decode steps done */
  int32_t next_full;     /* windows attended at full precision by the next step */
  int32_t next_quant;    /* windows attended in INT2 by the next step */
  int32_t next_splits;   /* attention workgroups per KV head the next step launches
                            (each writes one partial softmax state per query head) */
  int32_t full_bytes;    /* bytes read per full-precision window (K and V) */
  int32_t quant_bytes;   /* bytes read per INT2 window (codes, scales, minima) */
  size_t device_bytes;   /* device memory held */
} rskv_window_info;

int rskv_window_info_get(const rskv_window* cache, rskv_window_info* info);

/* Host copies of the cache state (any field may be NULL to skip it).  Units
 * u = b * Hkv + h; windows j = 0..nW-1; rows r = 0..63 of a window are
 * positions 64 j + r. */
typedef struct {
  int8_t* tier;       /* [U][nW] RSKV_TIER_* */
  double* score;      /* [U][nW] cumulative attention mass */
  double* mass;       /* [U][nW] masses credited by the last routing event */
  uint8_t* has_code;  /* [U][nW] 1 once the window holds a ledger entry */
  uint8_t* code_k;    /* [U][nW][64][d] INT2 codes 0..3 (ledger; 0 where
                         has_code is 0) */
  uint8_t* code_v;
  float* scale_k;     /* [U][nW][64][d/64] */
  float* min_k;
  float* scale_v;
  float* min_v;
  void* k;            /* [U][nW*64][d] full-precision store in dtype, rows
                         past T zero */
  void* v;
} rskv_window_state;

/* Synchronises with the cache's last stream, then copies.  Errors:
 * RSKV_ESTATE, RSKV_EHIP. */
int rskv_window_state_get(const rskv_window* cache, rskv_window_state* state);

/* Kernel time of the decode steps while enabled (per-dispatch start/stop
 * events, summed): [0] attention over the full-precision windows (fp32
 * caches: over all windows), [1] attention over the INT2 windows (bf16
 * caches), [2] merge of the partial softmax states, [3] routing (masses,
 * scores, ranking, tiers), [4] ledger writes and promotions. */
typedef struct {
  int64_t steps;
  int64_t events;
  double ms[5];
} rskv_window_profile;

int rskv_window_profile_enable(rskv_window* cache, int32_t on);
int rskv_window_profile_read(rskv_window* cache, rskv_window_profile* prof);

/* Releases the cache: waits only for the work queued on its last stream,
 * then returns every device block to its allocator.  NULL is accepted. */
void rskv_window_destroy(rskv_window* cache);

#ifdef __cplusplus
}
#endif
#endif /* RSKV_WINDOW_H_ */
