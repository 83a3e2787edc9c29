// Zoom-in routing (SEKV, Metodologia 3): the query is projected into the
// routing space of the summaries and a sigmoid gate scores every span.
//
// Per unit (sequence b, KV head h) with query group q_{hG..hG+G-1}:
//   rho  = P (1/G sum_g q_g)                       (P = identity if absent)
//   z_j  = alpha <rho, s_j>       in fp64, so that the expansion decision
//                                  z_j > tau is exact up to fp64 rounding
//   gate = sigmoid(z_j - tau);     expand iff z_j > tau (gate > 1/2), at
//                                  most k_max spans: largest z, ties to the
//                                  lower index
// The routing pass also stores, for every span and query head, the logit
// the span would carry if left unexpanded: <q_h, s_j>/sqrt(d) + ln|S_j|,
// so the summaries are read from HBM exactly once per step.
//
// route_kernel: HBM-bound GEMV; 16 lanes share one span row (16-byte
// vector loads for bf16), 4 spans per wave instruction, 64 spans per
// 256-thread workgroup.  topk_kernel: one 1024-thread workgroup per unit,
// radix select over an order-preserving uint64 key of z, then compaction
// of the selected indices in ascending order.
#include "cache.h"
#include "common.h"

namespace rskv {
namespace {

constexpr int kMaxG = 8;
constexpr int kRouteThreads = 256;
constexpr int kSpansPerBlock = 64;
constexpr int kTopkThreads = 1024;

template <int DT>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ summ,
    const float* __restrict__ log_len, const int32_t* __restrict__ n_spans,
    const float* __restrict__ proj, int n_proj, int Hkv, int G, int d, int S, float alpha,
    float inv_sqrt_d, double* __restrict__ z_out, float* __restrict__ slogit) {
  typedef Elem<DT> E;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int tid = threadIdx.x;
  const int ns = n_spans[b];
  const int j0 = blockIdx.x * kSpansPerBlock;
  if (j0 >= ns) return;

  __shared__ double qbar[128];
  __shared__ double rho[128];
  __shared__ float qh[kMaxG][128];
  const size_t qbase = (static_cast<size_t>(b) * Hkv * G + static_cast<size_t>(h) * G) * d;
  if (tid < d) {
    double sum = 0.0;
    for (int g = 0; g < G; ++g) {
      const float x = E::ld(q, qbase + static_cast<size_t>(g) * d + tid);
      qh[g][tid] = x;
      sum += static_cast<double>(x);
    }
    qbar[tid] = sum / static_cast<double>(G);
  }
  __syncthreads();
  if (tid < d) {
    if (proj != nullptr) {
      const float* P = proj + static_cast<size_t>(n_proj == 1 ? 0 : h) * d * d +
                       static_cast<size_t>(tid) * d;
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += static_cast<double>(P[c]) * qbar[c];
      rho[tid] = acc;
    } else {
      rho[tid] = qbar[tid];
    }
  }
  __syncthreads();

  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int grp = lane >> 4;      // span within the wave instruction
  const int li = lane & 15;       // lane within the span's 16
  const int epl = d / 16;         // elements per lane (8 or 4)
  for (int it = 0; it < kSpansPerBlock / 16; ++it) {
    const int j = j0 + wave * (kSpansPerBlock / 4) + it * 4 + grp;
    const bool valid = j < ns;
    double zacc = 0.0;
    float lacc[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) lacc[g] = 0.f;
    if (valid) {
      const size_t row = (static_cast<size_t>(u) * S + j) * d + static_cast<size_t>(li) * epl;
      for (int e = 0; e < epl; ++e) {
        const float sv = E::ld(summ, row + e);
        const int c = li * epl + e;
        zacc += rho[c] * static_cast<double>(sv);
#pragma unroll
        for (int g = 0; g < kMaxG; ++g)
          if (g < G) lacc[g] += qh[g][c] * sv;
      }
    }
    zacc = group_sum(zacc, 16);
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) lacc[g] = group_sum(lacc[g], 16);
    if (valid && li == 0) {
      z_out[static_cast<size_t>(u) * S + j] = static_cast<double>(alpha) * zacc;
      const float ell = log_len[static_cast<size_t>(b) * S + j];
      float* sl = slogit + (static_cast<size_t>(u) * S + j) * G;
      for (int g = 0; g < G; ++g) sl[g] = lacc[g] * inv_sqrt_d + ell;
    }
  }
}

// Count of keys (over the unit's spans) with key > thr, block-wide.
__device__ int block_count_gt(const double* z, int n, unsigned long long thr, int* red) {
  int cnt = 0;
  for (int j = threadIdx.x; j < n; j += kTopkThreads) cnt += f64_order_key(z[j]) > thr ? 1 : 0;
  int tot;
  block_excl_scan(cnt, red, &tot);
  return tot;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const double* __restrict__ z_all, const int32_t* __restrict__ n_spans, int Hkv, int S,
    double tau, int k_max, int k_ws, uint8_t* __restrict__ expanded_all,
    int32_t* __restrict__ sel_ws, int32_t* __restrict__ nsel_ws, int32_t* __restrict__ sel_out,
    int32_t* __restrict__ nsel_out) {
  const int u = blockIdx.x;
  const int b = u / Hkv;
  const int tid = threadIdx.x;
  const int n = n_spans[b];
  const double* z = z_all + static_cast<size_t>(u) * S;
  uint8_t* expanded = expanded_all + static_cast<size_t>(u) * S;
  int32_t* sel = sel_ws + static_cast<size_t>(u) * k_ws;

  __shared__ int red[17];
  __shared__ unsigned hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_remaining;

  const unsigned long long ktau = f64_order_key(tau);
  const int n_cand = block_count_gt(z, n, ktau, red);

  // Selection rule: key > kstar, plus the first `need` (by index) of the
  // keys equal to kstar.
  unsigned long long kstar = ktau;
  int need = 0;
  if (k_max == 0) {
    kstar = ~0ull;  // nothing is greater
  } else if (n_cand > k_max) {
    unsigned long long prefix = 0ull, pmask = 0ull;
    int remaining = k_max;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0u;
      __syncthreads();
      for (int j = tid; j < n; j += kTopkThreads) {
        const unsigned long long k = f64_order_key(z[j]);
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255ull], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int acc = 0, dg = 255;
        for (; dg > 0; --dg) {
          const int c = static_cast<int>(hist[dg]);
          if (acc + c >= remaining) break;
          acc += c;
        }
        s_prefix = prefix | (static_cast<unsigned long long>(dg) << shift);
        s_remaining = remaining - acc;
      }
      __syncthreads();
      prefix = s_prefix;
      remaining = s_remaining;
      pmask |= (255ull << shift);
      __syncthreads();
    }
    kstar = prefix;
    need = remaining;
  }

  int eq_seen = 0, n_sel = 0;
  for (int base = 0; base < S; base += kTopkThreads) {
    const int j = base + tid;
    const bool valid = j < n;
    unsigned long long k = 0ull;
    if (valid) k = f64_order_key(z[j]);
    const bool gt = valid && k > kstar;
    const bool eq = valid && need > 0 && k == kstar;
    int tot;
    const int packed = block_excl_scan(eq ? 1 : 0, red, &tot);
    const bool pick = gt || (eq && eq_seen + packed < need);
    eq_seen += tot;
    int stot;
    const int pos = block_excl_scan(pick ? 1 : 0, red, &stot);
    if (j < S) expanded[j] = pick ? 1 : 0;
    if (pick) sel[n_sel + pos] = j;
    n_sel += stot;
  }
  if (tid == 0) nsel_ws[u] = n_sel;
  if (sel_out != nullptr || nsel_out != nullptr) {
    __syncthreads();
    if (sel_out != nullptr)
      for (int i = tid; i < k_max; i += kTopkThreads)
        sel_out[static_cast<size_t>(u) * k_max + i] = i < n_sel ? sel[i] : -1;
    if (nsel_out != nullptr && tid == 0) nsel_out[u] = n_sel;
  }
}

template <int DT>
hipError_t route_impl(const rskv_cache* c, const void* q, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  dim3 grid((c->S + kSpansPerBlock - 1) / kSpansPerBlock, c->B * c->Hkv);
  hipLaunchKernelGGL(route_kernel<DT>, grid, dim3(kRouteThreads), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(c->dev.summary),
                     c->dev.log_len, c->dev.n_spans, c->dev.proj, c->n_proj, c->Hkv, c->G, c->d,
                     c->S, c->alpha, 1.0f / sqrtf(static_cast<float>(c->d)), c->dev.z,
                     c->dev.slogit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const rskv_cache* c, const void* q, hipStream_t st) {
  return c->dtype == kBF16 ? route_impl<kBF16>(c, q, st) : route_impl<kF32>(c, q, st);
}

hipError_t launch_topk(const rskv_cache* c, float tau, int k_max, int32_t* sel_out,
                       int32_t* nsel_out, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3(c->B * c->Hkv), dim3(kTopkThreads), 0, st, c->dev.z,
                     c->dev.n_spans, c->Hkv, c->S, static_cast<double>(tau), k_max, c->S,
                     c->dev.expanded, c->dev.sel, c->dev.n_sel, sel_out, nsel_out);
  return hipGetLastError();
}

}  // namespace rskv
