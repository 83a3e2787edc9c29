// Entropy-guided segmentation (SEKV, Metodologia 1): the n_a tokens with the
// largest surprisal are anchors (ties to the lower position); the non-empty
// runs strictly between two neighbouring anchors are spans; the lead and tail
// runs stay at full resolution with the anchors.
//
// One 1024-thread workgroup per sequence:
//   1. radix select (4 passes of 8 bits over an order-preserving uint32 key of
//      H) finds the n_a-th largest key K* and how many tokens equal to K* are
//      anchors (the lowest positions among them);
//   2. a chunked block scan marks anchors and finds the first/last anchor;
//   3. a second chunked scan numbers spans, records span starts/ends and
//      compacts the full-resolution positions;
//   4. a scan over spans turns ends into lengths and token offsets.
// It also reports what streaming segmentation needs at append time: the
// anchor threshold (the smallest anchor surprisal, whose order key is K*)
// and the full-resolution row of the last anchor (the rows after it are
// the tail run).  The sequence is read a handful of times; segmentation runs
// once per cache.
#include "cache.h"
#include "common.h"

namespace rskv {
namespace {

constexpr int kSegThreads = 1024;

// Inverse of f32_order_key (a folded zero comes back as +0).
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

__global__ __launch_bounds__(kSegThreads) void segment_kernel(
    const float* __restrict__ H_all, int T, int n_a, int32_t* __restrict__ span_id_all,
    int32_t* __restrict__ start_all, int32_t* __restrict__ len_all,
    int32_t* __restrict__ tokoff_all, int32_t* __restrict__ tokpad_all,
    int32_t* __restrict__ full_all, int32_t* __restrict__ counts) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const float* H = H_all + static_cast<size_t>(b) * T;
  int32_t* span_id = span_id_all + static_cast<size_t>(b) * T;
  int32_t* starts = start_all + static_cast<size_t>(b) * T;
  int32_t* ends = len_all + static_cast<size_t>(b) * T;  // ends first, lengths later
  int32_t* tokoff = tokoff_all + static_cast<size_t>(b) * (T + 1);
  int32_t* tokpad = tokpad_all + static_cast<size_t>(b) * (T + 1);
  int32_t* full = full_all + static_cast<size_t>(b) * T;

  __shared__ unsigned hist[256];
  __shared__ int scan_tmp[17];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining, s_first, s_last, s_nan;

  if (tid == 0) {
    s_first = T;
    s_last = -1;
    s_nan = 0;
  }
  __syncthreads();

  // ---- 1. radix select of the n_a-th largest key
  uint32_t prefix = 0u, pmask = 0u;
  int remaining = n_a;
  if (n_a > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSegThreads) hist[i] = 0u;
      __syncthreads();
      for (int t = tid; t < T; t += kSegThreads) {
        const float h = H[t];
        if (h != h) s_nan = 1;
        const uint32_t k = f32_order_key(h);
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int acc = 0, dg = 255;
        for (; dg > 0; --dg) {
          const int c = static_cast<int>(hist[dg]);
          if (acc + c >= remaining) break;
          acc += c;
        }
        s_prefix = prefix | (static_cast<uint32_t>(dg) << shift);
        s_remaining = remaining - acc;
      }
      __syncthreads();
      prefix = s_prefix;
      remaining = s_remaining;
      pmask |= (255u << shift);
      __syncthreads();
    }
  }
  const uint32_t kstar = prefix;
  const int need = remaining;  // anchors among the keys equal to K*

  // ---- 2. anchors, first and last anchor
  int eq_seen = 0;
  for (int base = 0; base < T; base += kSegThreads) {
    const int t = base + tid;
    const bool valid = t < T;
    uint32_t k = 0u;
    if (valid) k = f32_order_key(H[t]);
    const bool gt = valid && n_a > 0 && k > kstar;
    const bool eq = valid && n_a > 0 && k == kstar;
    int eq_total;
    const int eq_before = block_excl_scan(eq ? 1 : 0, scan_tmp, &eq_total);
    const bool anchor = gt || (eq && eq_seen + eq_before < need);
    if (valid) {
      span_id[t] = anchor ? -1 : -3;
      if (anchor) {
        atomicMin(&s_first, t);
        atomicMax(&s_last, t);
      }
    }
    eq_seen += eq_total;
  }
  __syncthreads();
  const int first = s_first, last = s_last;

  // ---- 3. span numbering, starts/ends, full-resolution positions
  int n_spans = 0, n_full = 0;
  for (int base = 0; base < T; base += kSegThreads) {
    const int t = base + tid;
    const bool valid = t < T;
    bool is_anchor = false, in_span = false, is_start = false, is_end = false;
    if (valid) {
      is_anchor = span_id[t] == -1;
      in_span = !is_anchor && t > first && t < last;
      if (in_span) {
        is_start = span_id[t - 1] == -1;
        is_end = span_id[t + 1] == -1;
      }
    }
    const bool is_full = valid && !in_span;
    int tot;
    const int packed = block_excl_scan((is_start ? 1 : 0) + (is_full ? 65536 : 0), scan_tmp, &tot);
    const int start_before = packed & 0xFFFF;
    const int full_before = packed >> 16;
    if (valid) {
      if (in_span) {
        const int j = n_spans + start_before + (is_start ? 1 : 0) - 1;
        span_id[t] = j;
        if (is_start) starts[j] = t;
        if (is_end) ends[j] = t + 1;
      } else {
        span_id[t] = is_anchor ? -1 : -2;
        full[n_full + full_before] = t;
      }
    }
    n_spans += tot & 0xFFFF;
    n_full += tot >> 16;
  }
  __syncthreads();

  // ---- 4. lengths and token offsets (plain, and with spans padded to 16)
  int n_tok = 0, n_pad = 0;
  for (int base = 0; base < n_spans; base += kSegThreads) {
    const int j = base + tid;
    int len = 0;
    if (j < n_spans) len = ends[j] - starts[j];
    int tot, tot_pad;
    const int before = block_excl_scan(len, scan_tmp, &tot);
    const int before_pad = block_excl_scan(round_up(len, 16), scan_tmp, &tot_pad);
    if (j < n_spans) {
      ends[j] = len;
      tokoff[j] = n_tok + before;
      tokpad[j] = n_pad + before_pad;
    }
    n_tok += tot;
    n_pad += tot_pad;
  }
  if (tid == 0) {
    tokoff[n_spans] = n_tok;
    tokpad[n_spans] = n_pad;
    int32_t* cnt = counts + kCounts * b;
    cnt[0] = s_nan ? -1 : n_a;  // -1 flags NaN surprisal
    cnt[1] = n_spans;
    cnt[2] = n_full;
    cnt[3] = n_tok;
    cnt[4] = n_pad;
    // the tail run holds the T - 1 - last positions after the last anchor
    cnt[5] = last >= 0 ? n_full - (T - 1 - last) - 1 : -1;
    const float inf = __builtin_huge_valf();
    cnt[6] = __float_as_int(last >= 0 ? f32_from_order_key(kstar) : inf);
  }
}

// dst[b][i] = i < count[b] ? src[b][i] : pad, for i < dst_pitch.
__global__ void copy_rows_kernel(int32_t* __restrict__ dst, int dst_pitch,
                                 const int32_t* __restrict__ src, int src_pitch,
                                 const int32_t* __restrict__ counts, int count_stride,
                                 int count_index, int extra, int32_t pad) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= dst_pitch) return;
  const int n = counts[count_stride * b + count_index] + extra;
  dst[static_cast<size_t>(b) * dst_pitch + i] =
      i < n ? src[static_cast<size_t>(b) * src_pitch + i] : pad;
}

}  // namespace

hipError_t launch_segment(const float* H, int B, int T, int n_anchor, int32_t* span_id,
                          int32_t* start_tmp, int32_t* len_tmp, int32_t* tokoff_tmp,
                          int32_t* tokpad_tmp, int32_t* full_tmp, int32_t* counts,
                          hipStream_t st) {
  hipLaunchKernelGGL(segment_kernel, dim3(B), dim3(kSegThreads), 0, st, H, T, n_anchor,
                     span_id, start_tmp, len_tmp, tokoff_tmp, tokpad_tmp, full_tmp, counts);
  return hipGetLastError();
}

hipError_t launch_copy_rows(int32_t* dst, int dst_pitch, const int32_t* src, int src_pitch,
                            const int32_t* counts, int count_stride, int count_index,
                            int extra, int32_t pad, int B, hipStream_t st) {
  dim3 grid((dst_pitch + 255) / 256, B);
  hipLaunchKernelGGL(copy_rows_kernel, grid, dim3(256), 0, st, dst, dst_pitch, src, src_pitch,
                     counts, count_stride, count_index, extra, pad);
  return hipGetLastError();
}

}  // namespace rskv
