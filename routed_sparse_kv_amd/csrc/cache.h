// Host-side cache object and kernel launchers of librskv.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <tuple>
#include <vector>

#include "../../include/rskv.h"
#include "devmem.h"
#include "layout.h"

namespace rskv {

// Device memory of a cache.  U = B*Hkv units, unit u = b*Hkv + h.  S, F, N
// are the batch maxima of spans, full-resolution rows (incl. tail capacity)
// and span tokens; Sp = round_up(S, 32), Fp = round_up(F, 32) and Np (span
// tokens with every span padded to 16 rows) size the tiled arrays (see
// layout.h).
struct DeviceArrays {
  // segmentation tables
  int32_t* span_id = nullptr;     // [B][T]
  int32_t* span_start = nullptr;  // [B][S]
  int32_t* span_len = nullptr;    // [B][S]
  int32_t* tok_off = nullptr;     // [B][S+1] exclusive prefix of span_len
  int32_t* tok_pad = nullptr;     // [B][S+1] same with lengths rounded up to 16
  int32_t* full_pos = nullptr;    // [B][F]
  int32_t* n_spans = nullptr;     // [B]
  int32_t* n_full = nullptr;      // [B] current full rows (grows on append)
  int32_t* n_full0 = nullptr;     // [B] full rows at build time
  // streaming segmentation state
  float* h_full = nullptr;        // [B][F] surprisal of each full-resolution row
  float* theta = nullptr;         // [B] anchor threshold (smallest prefill anchor
                                  // surprisal, +inf without anchors)
  int32_t* last_anchor = nullptr; // [B] full-resolution row of the last anchor, -1
  // stored representation (cache dtype unless noted)
  void* summary = nullptr;        // [U][S][d] row-major (routing GEMV rows)
  void* vmean = nullptr;          // [U] V32 tiles over Sp spans
  float* log_len = nullptr;       // [B][S]
  void* k_full = nullptr;         // [U] K16 tiles over Fp rows
  void* v_full = nullptr;         // [U] V32 tiles over Fp rows
  void* a_k = nullptr;            // [U][Np][r]
  void* a_v = nullptr;            // [U] transposed 16-row tiles over Np rows
  void* w_k = nullptr;            // [U][S][r][d]
  void* w_v = nullptr;            // [U][S][d][r]
  float* proj = nullptr;          // [n_proj][d][d] or null
  // decode workspace
  double* z = nullptr;            // [U][S] routing scores
  float* slogit = nullptr;        // [U] summary logits incl. ln|S| (slogit_off, Sp spans)
  int32_t* sel = nullptr;         // [U][S] expanded spans, ascending
  int32_t* sel_desc = nullptr;    // [U][S][4] per expanded span: j, |S_j|, padded offset,
                                  // exclusive work-cost prefix
  int32_t* n_sel = nullptr;       // [U]
  int32_t* wstart = nullptr;      // [U][4 nsplit_max + 1] first work item of each wave
  float* part = nullptr;          // [U][nsplit_max][G][d + 2] partial states
};

// Decode workspace of one step, written and read only by the decode kernels
// of that step: routing scores, summary logits, selection lists, per-wave
// work ranges and partial softmax states.  Every entry a kernel reads was
// written earlier in the same step (padding reads are masked), so none of
// it needs clearing.  rskv_decode_step uses the cache's own workspace;
// rskv_decode_step_static carves one out of the library's static scratch.
struct DecodeWs {
  double* z = nullptr;         // [U][S]
  float* slogit = nullptr;     // [U] Sp spans x G heads (slogit_off)
  int32_t* sel = nullptr;      // [U][S]
  int32_t* sel_desc = nullptr; // [U][S][4]
  int32_t* n_sel = nullptr;    // [U]
  int32_t* wstart = nullptr;   // [U][4 nsplit_max + 1]
  float* part = nullptr;       // [U][nsplit_max][G][d + 2]
};

// Decode kernels timed per profiled step (route, top-k, attend, merge); each
// has a start and a stop event carried by its own dispatch.
constexpr int kProfileKernels = 4;

struct Profile {
  bool on = false;
  int64_t steps = 0;
  double ms[kProfileKernels] = {0, 0, 0, 0};
  std::vector<hipEvent_t> pending;  // 2 * kProfileKernels per recorded step
  // appends: close start/stop (null when not launched), append start/stop
  int64_t appends = 0;
  double close_ms = 0, append_ms = 0;
  std::vector<hipEvent_t> app_pending;
  std::vector<hipEvent_t> pool;
};

// Start/stop events of one kernel dispatch (timestamps of the kernel itself).
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launches `kernel`; with `ev`, the dispatch records ev->start and ev->stop.
// Without events it is a plain launch, which a HIP graph can capture.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                  const KernelEvents* ev, Args... args) {
  if (ev != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, ev->start, ev->stop, 0u, args...);
  } else {
    std::tuple<KArgs...> formals{static_cast<KArgs>(args)...};
    void* argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    pArgs<0>(formals, argv);
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

// Integer work cost (64-byte units) of the attention kernel's items, used by
// the top-k kernel to give each wave a contiguous, balanced item range.
struct WorkCost {
  int span_base;   // an expanded span: factor matrices W_K, W_V + overhead
  int span_row;    // bytes of A_K and A_V per padded row
  int span_extra;  // each further 32 rows past the first 64 (a load round)
  int full;        // 32 full-resolution rows
  int summ;        // 32 summary entries
  // (fits in int for spans of up to 2^24 rows)
  __host__ __device__ int span(int len) const {
    const int pad = (len + 15) & ~15;
    const int extra = len > 64 ? (len - 33) >> 5 : 0;
    return span_base + ((pad * span_row) >> 6) + extra * span_extra;
  }
};

}  // namespace rskv

struct rskv_cache {
  uint32_t magic = 0;
  int B = 0, Hq = 0, Hkv = 0, d = 0, T = 0, rank = 0, dtype = 0, G = 0;
  float alpha = 8.f;
  int n_proj = 0;
  int S = 1, F = 1, N = 1, Sp = 32, Fp = 32, Np = 16;
  int tail_cap = 0, appended = 0, k_max_cap = 0;
  // span closing at append time: longest run a closing can see (0: no
  // decoded token can be an anchor) and the close kernel's workgroups
  int close_rows = 0;
  int close_grid = 0;
  int nsplit_max = 1;
  std::vector<int32_t> h_n_anchor, h_n_spans, h_n_full0, h_n_span_tokens, h_n_tok_pad;
  rskv::DeviceArrays dev;
  rskv::DevMem mem;                // allocator of the device memory
  std::vector<void*> allocs;       // device memory
  size_t bytes = 0;
  int factor_tier = 0;             // RSKV_TIER_HBM or RSKV_TIER_HOST
  std::vector<void*> host_allocs;  // pinned host memory (host factor tier)
  size_t host_bytes = 0;
  hipStream_t last_stream = nullptr;
  rskv::Profile prof;
};

namespace rskv {

constexpr uint32_t kMagic = 0x52534b56u;  // "RSKV"

// Records `msg` as the calling thread's last error (rskv_last_error) and
// returns `code`.
int report_error(int code, const std::string& msg);

// ---- launchers (each returns hipSuccess or the first launch error)

// Segmentation of every sequence; writes span_id, span starts/lengths,
// token offsets (plain and padded), full-resolution positions (pitch T) and
// counts[B][7] = {n_anchor (-1: NaN surprisal), n_spans, n_full,
// n_span_tokens, n_tok_pad, full-resolution row of the last anchor (-1 if
// none), bits of the anchor threshold (fp32; +inf if none)}.
constexpr int kCounts = 7;
hipError_t launch_segment(const float* H, int B, int T, int n_anchor, int32_t* span_id,
                          int32_t* start_tmp, int32_t* len_tmp, int32_t* tokoff_tmp,
                          int32_t* tokpad_tmp, int32_t* full_tmp, int32_t* counts,
                          hipStream_t st);

// dst[b][i] = i < counts[b*stride+index] + extra ? src[b][i] : pad.
hipError_t launch_copy_rows(int32_t* dst, int dst_pitch, const int32_t* src, int src_pitch,
                            const int32_t* counts, int count_stride, int count_index,
                            int extra, int32_t pad, int B, hipStream_t st);

// Summaries, value means and ln|S| (fp64 accumulation).
hipError_t launch_summary(const rskv_cache* c, const float* H, const void* K, const void* V,
                          hipStream_t st);

// Packs full-resolution rows of K and V and their surprisal.
hipError_t launch_pack(const rskv_cache* c, const float* H, const void* K, const void* V,
                       hipStream_t st);

// Per-span rank-r factors of K and V (fp64 one-sided Jacobi).
hipError_t launch_factor(rskv_cache* c, const void* K, const void* V, hipStream_t st,
                         std::string* err);

// Decode, four launches in stream order: routing GEMV (z, summary logits),
// top-k cap (and the attention work partition when `nwaves` > 0),
// attention partials, merge of the partials into `out`, all with the
// workspace `ws`.  `ev` (may be null) receives the kernel's own start and
// stop times.
hipError_t launch_route(const rskv_cache* c, const DecodeWs& ws, const void* q, hipStream_t st,
                        const KernelEvents* ev);
hipError_t launch_topk(const rskv_cache* c, const DecodeWs& ws, float tau, int k_max, int nwaves,
                       int32_t* sel_out, int32_t* nsel_out, hipStream_t st,
                       const KernelEvents* ev);
int decode_nsplit(const rskv_cache* c, int k_max);
int decode_nsplit_max(int B, int Hkv, int S, int F, int k_max_cap);
bool attend_uses_mfma(const rskv_cache* c);
WorkCost work_cost(const rskv_cache* c);

// Arguments of the attention launch when it also makes the top-k selection
// (attend_fuses_topk): the spans of a unit fit in the kernel's LDS.
struct SelectArgs {
  float tau;
  int k_max;
  int32_t* sel_out;   // may be null
  int32_t* nsel_out;  // may be null
};
bool attend_fuses_topk(const rskv_cache* c, int k_max);
hipError_t launch_attend(const rskv_cache* c, const DecodeWs& ws, const void* q, int nsplit,
                         const SelectArgs* sel, hipStream_t st, const KernelEvents* ev);
hipError_t launch_merge(const rskv_cache* c, const DecodeWs& ws, int nsplit, float* out,
                        hipStream_t st, const KernelEvents* ev);

// The cache's own decode workspace; the bytes a workspace of this cache
// needs (each array 256-byte aligned) and one laid out from `base`.
DecodeWs cache_ws(const rskv_cache* c);
size_t decode_ws_bytes(const rskv_cache* c);
DecodeWs carve_ws(const rskv_cache* c, void* base);

// One decode step with workspace `ws` (the body of rskv_decode_step; with
// `profile` false no event is used and nothing is allocated).
int decode_with(rskv_cache* c, const DecodeWs& ws, const void* q, float tau, int k_max,
                float* out, int32_t* sel, int32_t* n_sel, hipStream_t st, bool profile);
// Argument checks of the decode entry points (sets the error message).
int check_decode(const rskv_cache* c, const void* q, float tau, int k_max, const float* out);

// Streaming segmentation at append time, two launches: launch_close turns
// the full-resolution run after the last anchor into a new span for every
// sequence whose new token (surprisal h[b], device) is an anchor;
// launch_append then stores the token (surprisal h[b], or 0 when h is null)
// at position `pos` and updates the counts; `closed` tells it whether
// launch_close ran before it.  `ev` may be null.
hipError_t launch_close(const rskv_cache* c, const float* h, hipStream_t st,
                        const KernelEvents* ev);
hipError_t launch_append(const rskv_cache* c, const void* k, const void* v, const float* h,
                         bool closed, int pos, hipStream_t st, const KernelEvents* ev);

}  // namespace rskv
