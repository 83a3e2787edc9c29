// Coarse representation of each span and the full-resolution store.
//
// SEKV, Metodologia 2: every span keeps a normalised, surprisal-weighted
// summary of its keys for coarse routing; Metodologia 3: an unexpanded span
// enters attention with its summary and a size correction.  Here
//   s_j   = u / ||u||, u = sum_{t in S_j} H_t k_t   (s_j = 0 if u = 0),
//   vbar_j = mean of the span's value rows,
//   ell_j  = ln |S_j|,
// accumulated in fp64 and rounded once to the cache dtype.  The anchors and
// the lead/tail runs are copied row by row into the packed full-resolution
// store, which also receives decode-time appends (with streaming
// segmentation: a decoded anchor closes the run before it into a span).
#include "cache.h"
#include "common.h"

namespace rskv {
namespace {

// One 128-thread workgroup per (span, unit); thread c owns column c.
template <int DT>
__global__ __launch_bounds__(128) void summary_kernel(
    const float* __restrict__ H_all, const typename Elem<DT>::T* __restrict__ K,
    const typename Elem<DT>::T* __restrict__ V, const int32_t* __restrict__ span_start,
    const int32_t* __restrict__ span_len, const int32_t* __restrict__ n_spans, int T, int d,
    int S, int Sp, int Hkv, typename Elem<DT>::T* __restrict__ s_out,
    typename Elem<DT>::T* __restrict__ v_out, float* __restrict__ log_len) {
  typedef Elem<DT> E;
  const int j = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  if (j >= n_spans[b]) return;
  const int st = span_start[static_cast<size_t>(b) * S + j];
  const int len = span_len[static_cast<size_t>(b) * S + j];
  const int c = threadIdx.x;
  const float* H = H_all + static_cast<size_t>(b) * T + st;
  const size_t row0 = (static_cast<size_t>(u) * T + st) * d;

  double us = 0.0, vs = 0.0;
  if (c < d) {
    for (int t = 0; t < len; ++t) {
      const size_t idx = row0 + static_cast<size_t>(t) * d + c;
      us += static_cast<double>(H[t]) * static_cast<double>(E::ld(K, idx));
      vs += static_cast<double>(E::ld(V, idx));
    }
  }
  __shared__ double red[2];
  double sq = wave_sum(us * us);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = sq;
  __syncthreads();
  const double norm2 = red[0] + red[1];
  if (c < d) {
    s_out[(static_cast<size_t>(u) * S + j) * d + c] =
        E::from_f64(norm2 > 0.0 ? us / sqrt(norm2) : 0.0);
    v_out[static_cast<size_t>(u) * Sp * d + v32_off(j, c, d)] =
        E::from_f64(vs / static_cast<double>(len));
  }
  if (c == 0 && h == 0)
    log_len[static_cast<size_t>(b) * S + j] = static_cast<float>(log(static_cast<double>(len)));
}

// Row i < n_full0[b] of unit u: K/V row full_pos[b][i] of the context; the
// blocks of KV head 0 also keep the row's surprisal (streaming segmentation
// weighs the rows of a later span by it).
template <int DT>
__global__ __launch_bounds__(128) void pack_kernel(
    const float* __restrict__ H, const typename Elem<DT>::T* __restrict__ K,
    const typename Elem<DT>::T* __restrict__ V, const int32_t* __restrict__ full_pos,
    const int32_t* __restrict__ n_full0, int T, int d, int F, int Fp, int Hkv,
    typename Elem<DT>::T* __restrict__ kf, typename Elem<DT>::T* __restrict__ vf,
    float* __restrict__ h_full) {
  const int i = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  if (i >= n_full0[b]) return;
  const int pos = full_pos[static_cast<size_t>(b) * F + i];
  const size_t src = (static_cast<size_t>(u) * T + pos) * d;
  const size_t dst = static_cast<size_t>(u) * Fp * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    kf[dst + k16_off(i, c, d)] = K[src + c];
    vf[dst + v32_off(i, c, d)] = V[src + c];
  }
  if (u == b * Hkv && threadIdx.x == 0)
    h_full[static_cast<size_t>(b) * F + i] = H[static_cast<size_t>(b) * T + pos];
}

// One workgroup per sequence: store the decoded token (k, v of every KV
// head, surprisal h[b] or 0 without h) as a full-resolution row at
// position `pos`.  Streaming segmentation (SEKV, Metodologia 1, applied to
// decoded tokens): the token is an anchor iff its surprisal exceeds the
// sequence's threshold.  If it is and the run after the previous anchor is
// non-empty, the close kernel has just turned that run into span
// n_spans[b]: the run's rows are released and the token takes the first of
// them (only when `closed` says the close kernel ran).  The token then
// becomes the last anchor.
template <int DT>
__global__ __launch_bounds__(256) void append_kernel(
    const typename Elem<DT>::T* __restrict__ k, const typename Elem<DT>::T* __restrict__ v,
    const float* __restrict__ h_new, int closed, int pos, int Hkv, int d, int F, int Fp,
    const float* __restrict__ theta, int32_t* __restrict__ n_full, int32_t* __restrict__ n_spans,
    int32_t* __restrict__ last_anchor, int32_t* __restrict__ full_pos,
    float* __restrict__ h_full, typename Elem<DT>::T* __restrict__ kf,
    typename Elem<DT>::T* __restrict__ vf) {
  const int b = blockIdx.x;
  const int nf = n_full[b];
  const int la = last_anchor[b];
  const float hb = h_new != nullptr ? h_new[b] : 0.f;
  const bool anchor = h_new != nullptr && hb > theta[b];
  const bool close = closed && anchor && la >= 0 && nf - la - 1 > 0;
  const int row = close ? la + 1 : nf;
  float* hf = h_full + static_cast<size_t>(b) * F;
  int32_t* fp = full_pos + static_cast<size_t>(b) * F;
  __syncthreads();  // every thread has read the counts
  for (int i = row + threadIdx.x; i < nf; i += blockDim.x) {
    fp[i] = -1;
    hf[i] = 0.f;
  }
  for (int idx = threadIdx.x; idx < Hkv * d; idx += blockDim.x) {
    const int h = idx / d;
    const int c = idx - h * d;
    const size_t u = static_cast<size_t>(b) * Hkv + h;
    kf[u * Fp * d + k16_off(row, c, d)] = k[u * d + c];
    vf[u * Fp * d + v32_off(row, c, d)] = v[u * d + c];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    fp[row] = pos;
    hf[row] = hb;
    n_full[b] = row + 1;
    if (close) n_spans[b] += 1;
    if (anchor) last_anchor[b] = row;
  }
}

template <int DT>
hipError_t summary_impl(const rskv_cache* c, const float* H, const void* K, const void* V,
                        hipStream_t st) {
  typedef typename Elem<DT>::T T;
  dim3 grid(c->S, c->B * c->Hkv);
  hipLaunchKernelGGL(summary_kernel<DT>, grid, dim3(128), 0, st, H,
                     static_cast<const T*>(K), static_cast<const T*>(V), c->dev.span_start,
                     c->dev.span_len, c->dev.n_spans, c->T, c->d, c->S, c->Sp, c->Hkv,
                     static_cast<T*>(c->dev.summary), static_cast<T*>(c->dev.vmean),
                     c->dev.log_len);
  return hipGetLastError();
}

template <int DT>
hipError_t pack_impl(const rskv_cache* c, const float* H, const void* K, const void* V,
                     hipStream_t st) {
  typedef typename Elem<DT>::T T;
  dim3 grid(c->F, c->B * c->Hkv);
  hipLaunchKernelGGL(pack_kernel<DT>, grid, dim3(128), 0, st, H, static_cast<const T*>(K),
                     static_cast<const T*>(V), c->dev.full_pos, c->dev.n_full0, c->T, c->d,
                     c->F, c->Fp, c->Hkv, static_cast<T*>(c->dev.k_full),
                     static_cast<T*>(c->dev.v_full), c->dev.h_full);
  return hipGetLastError();
}

template <int DT>
hipError_t append_impl(const rskv_cache* c, const void* k, const void* v, const float* h,
                       bool closed, int pos, hipStream_t st, const KernelEvents* ev) {
  typedef typename Elem<DT>::T T;
  const auto& a = c->dev;
  return launch(append_kernel<DT>, dim3(c->B), dim3(256), 0, st, ev, static_cast<const T*>(k),
                static_cast<const T*>(v), h, closed ? 1 : 0, pos, c->Hkv, c->d, c->F, c->Fp,
                static_cast<const float*>(a.theta), a.n_full, a.n_spans, a.last_anchor,
                a.full_pos, a.h_full, static_cast<T*>(a.k_full), static_cast<T*>(a.v_full));
}

}  // namespace

hipError_t launch_summary(const rskv_cache* c, const float* H, const void* K, const void* V,
                          hipStream_t st) {
  return c->dtype == kBF16 ? summary_impl<kBF16>(c, H, K, V, st)
                           : summary_impl<kF32>(c, H, K, V, st);
}

hipError_t launch_pack(const rskv_cache* c, const float* H, const void* K, const void* V,
                       hipStream_t st) {
  return c->dtype == kBF16 ? pack_impl<kBF16>(c, H, K, V, st) : pack_impl<kF32>(c, H, K, V, st);
}

hipError_t launch_append(const rskv_cache* c, const void* k, const void* v, const float* h,
                         bool closed, int pos, hipStream_t st, const KernelEvents* ev) {
  return c->dtype == kBF16 ? append_impl<kBF16>(c, k, v, h, closed, pos, st, ev)
                           : append_impl<kF32>(c, k, v, h, closed, pos, st, ev);
}

}  // namespace rskv
