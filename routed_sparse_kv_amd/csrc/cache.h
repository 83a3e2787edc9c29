// Host-side cache object and kernel launchers of librskv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/rskv.h"

namespace rskv {

// Device memory layout of a cache (all row-major; U = B*Hkv units, unit
// u = b*Hkv + h; S, F, N are the padded span, full-row and span-token
// dimensions).
struct DeviceArrays {
  // segmentation tables
  int32_t* span_id = nullptr;     // [B][T]
  int32_t* span_start = nullptr;  // [B][S]
  int32_t* span_len = nullptr;    // [B][S]
  int32_t* tok_off = nullptr;     // [B][S+1] exclusive prefix of span_len
  int32_t* full_pos = nullptr;    // [B][F]
  int32_t* n_spans = nullptr;     // [B]
  int32_t* n_full = nullptr;      // [B] current full rows (grows on append)
  int32_t* n_full0 = nullptr;     // [B] full rows at build time
  // stored representation (cache dtype unless noted)
  void* summary = nullptr;        // [U][S][d]
  void* vmean = nullptr;          // [U][S][d]
  float* log_len = nullptr;       // [B][S]
  void* k_full = nullptr;         // [U][F][d]
  void* v_full = nullptr;         // [U][F][d]
  void* a_k = nullptr;            // [U][N][r]
  void* a_v = nullptr;            // [U][N][r]
  void* w_k = nullptr;            // [U][S][r][d]
  void* w_v = nullptr;            // [U][S][r][d]
  float* proj = nullptr;          // [n_proj][d][d] or null
  // decode workspace
  double* z = nullptr;            // [U][S] routing scores
  float* slogit = nullptr;        // [U][S][G] summary logits incl. ln|S|
  uint8_t* expanded = nullptr;    // [U][S] 1 if span j expanded this step
  int32_t* sel = nullptr;         // [U][kcap] expanded spans, ascending
  int32_t* n_sel = nullptr;       // [U]
  float* part = nullptr;          // [U][nsplit_max][G][d + 2] partial states
};

struct Profile {
  bool on = false;
  int64_t steps = 0;
  double ms[4] = {0, 0, 0, 0};
  std::vector<hipEvent_t> pending;  // 5 events per recorded step
  std::vector<hipEvent_t> pool;
};

}  // namespace rskv

struct rskv_cache {
  uint32_t magic = 0;
  int B = 0, Hq = 0, Hkv = 0, d = 0, T = 0, rank = 0, dtype = 0, G = 0;
  float alpha = 8.f;
  int n_proj = 0;
  int S = 1, F = 1, N = 1;
  int tail_cap = 0, appended = 0, k_max_cap = 0;
  int nsplit_max = 1;
  std::vector<int32_t> h_n_anchor, h_n_spans, h_n_full0, h_n_span_tokens;
  rskv::DeviceArrays dev;
  std::vector<void*> allocs;
  size_t bytes = 0;
  hipStream_t last_stream = nullptr;
  rskv::Profile prof;
};

namespace rskv {

constexpr uint32_t kMagic = 0x52534b56u;  // "RSKV"

// ---- launchers (each returns hipSuccess or the first launch error)

// Segmentation of every sequence; writes span_id, span starts/lengths,
// token offsets, full-resolution positions (pitch T) and counts[B][4] =
// {n_anchor, n_spans, n_full, n_span_tokens}.
hipError_t launch_segment(const float* H, int B, int T, int n_anchor, int32_t* span_id,
                          int32_t* start_tmp, int32_t* len_tmp, int32_t* tokoff_tmp,
                          int32_t* full_tmp, int32_t* counts, hipStream_t st);

// dst[b][i] = i < counts[b*stride+index] + extra ? src[b][i] : pad.
hipError_t launch_copy_rows(int32_t* dst, int dst_pitch, const int32_t* src, int src_pitch,
                            const int32_t* counts, int count_stride, int count_index,
                            int extra, int32_t pad, int B, hipStream_t st);

// Summaries, value means and ln|S| (fp64 accumulation).
hipError_t launch_summary(const rskv_cache* c, const float* H, const void* K, const void* V,
                          hipStream_t st);

// Packs full-resolution rows of K and V.
hipError_t launch_pack(const rskv_cache* c, const void* K, const void* V, hipStream_t st);

// Per-span rank-r factors of K and V (fp64 one-sided Jacobi).
hipError_t launch_factor(rskv_cache* c, const void* K, const void* V, hipStream_t st,
                         std::string* err);

// Decode: route (z, summary logits), top-k, attention partials, merge.
hipError_t launch_route(const rskv_cache* c, const void* q, hipStream_t st);
hipError_t launch_topk(const rskv_cache* c, float tau, int k_max, int32_t* sel_out,
                       int32_t* nsel_out, hipStream_t st);
int decode_nsplit(const rskv_cache* c, int k_max);
int decode_nsplit_max(int B, int Hkv, int S, int F, int k_max_cap);
hipError_t launch_attend(const rskv_cache* c, const void* q, int k_max, int nsplit,
                         hipStream_t st);
hipError_t launch_merge(const rskv_cache* c, int nsplit, float* out, hipStream_t st);

hipError_t launch_append(rskv_cache* c, const void* k, const void* v, hipStream_t st);

}  // namespace rskv
