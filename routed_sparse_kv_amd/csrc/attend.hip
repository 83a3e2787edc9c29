// Mixed-resolution attention (SEKV, Metodologia 3): one softmax over
//   - full-resolution rows (anchors, lead/tail runs, appended tokens) with
//     their exact K/V;
//   - every token of an expanded span, rebuilt from its factors:
//     k-hat_i = A_K[i] W_K, v-hat_i = A_V[i] W_V;
//   - every other span as one entry: key s_j with logit <q, s_j>/sqrt(d) +
//     ln|S_j| (precomputed by the routing pass), value the span mean.
//
// Split-K: the unit's work items (32-row full-resolution chunks, expanded
// spans, 32-span summary chunks) are dealt round-robin to `nsplit`
// workgroups; each keeps an online-softmax state (m, l, acc) per query head
// and writes it as a partial; merge_kernel combines the partials with the
// log-sum-exp rule.
//
// The rank-r contraction is applied to the small operands instead of
// materialising K-hat and V-hat:  <q, A_i W_K> = A_i (W_K q)  and
// sum_i p_i A_i W_V = (sum_i p_i A_i) W_V,  which is the same arithmetic up
// to association and reads each factor exactly once.
#include "cache.h"
#include "common.h"

namespace rskv {
namespace {

constexpr int kAttThreads = 256;
constexpr int kChunk = 32;
constexpr int kMaxG = 8;
constexpr int kMaxRank = 32;
constexpr int kMaxOut = 4;  // outputs per thread: G * d <= 1024

struct SoftmaxState {
  float m[kMaxG];
  float l[kMaxG];
  float sc[kMaxG];
};

// Turns the chunk logits lg[i][g] into probabilities relative to the new
// running max, and updates the running max, scale and sum.  All threads.
__device__ __forceinline__ void chunk_softmax(float (*lg)[kMaxG + 1], SoftmaxState* st, int G) {
  const int tid = threadIdx.x;
  if (tid < G) {
    float cm = -INFINITY;
    for (int i = 0; i < kChunk; ++i) cm = fmaxf(cm, lg[i][tid]);
    const float mo = st->m[tid];
    const float mn = fmaxf(mo, cm);
    st->sc[tid] = (mn == -INFINITY) ? 1.f : expf(mo - mn);
    st->m[tid] = mn;
  }
  __syncthreads();
  for (int pi = tid; pi < kChunk * G; pi += kAttThreads) {
    const int i = pi / G;
    const int g = pi - i * G;
    const float x = lg[i][g];
    lg[i][g] = (x == -INFINITY) ? 0.f : expf(x - st->m[g]);
  }
  __syncthreads();
  if (tid < G) {
    float sum = 0.f;
    for (int i = 0; i < kChunk; ++i) sum += lg[i][tid];
    st->l[tid] = st->l[tid] * st->sc[tid] + sum;
  }
}

template <int DT>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(
    const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ kf,
    const typename Elem<DT>::T* __restrict__ vf, const int32_t* __restrict__ n_full,
    const typename Elem<DT>::T* __restrict__ vmean, const float* __restrict__ slogit,
    const uint8_t* __restrict__ expanded, const int32_t* __restrict__ n_spans,
    const typename Elem<DT>::T* __restrict__ a_k, const typename Elem<DT>::T* __restrict__ a_v,
    const typename Elem<DT>::T* __restrict__ w_k, const typename Elem<DT>::T* __restrict__ w_v,
    const int32_t* __restrict__ span_len, const int32_t* __restrict__ tok_off,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel, int Hkv, int G, int d,
    int S, int F, int N, int rank, int k_slots, int nsplit, int nsplit_max, int nFC, int nSC,
    float inv_sqrt_d, float* __restrict__ part) {
  typedef Elem<DT> E;
  const int s = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int tid = threadIdx.x;

  __shared__ float qs[kMaxG][128];
  __shared__ float lg[kChunk][kMaxG + 1];
  __shared__ SoftmaxState st;
  __shared__ float uk[kMaxG][kMaxRank];
  __shared__ float wv[kMaxG][kMaxRank];

  const size_t qbase = (static_cast<size_t>(b) * Hkv * G + static_cast<size_t>(h) * G) * d;
  for (int idx = tid; idx < G * d; idx += kAttThreads) {
    const int g = idx / d;
    qs[g][idx - g * d] = E::ld(q, qbase + idx);
  }
  if (tid < kMaxG) {
    st.m[tid] = -INFINITY;
    st.l[tid] = 0.f;
    st.sc[tid] = 1.f;
  }
  float acc[kMaxOut];
#pragma unroll
  for (int i = 0; i < kMaxOut; ++i) acc[i] = 0.f;
  const int nout = G * d;
  __syncthreads();

  const int nf = n_full[b];
  const int ns = n_spans[b];
  const int nsel = n_sel[u];
  const int NI = nFC + k_slots + nSC;
  const size_t ubase_f = static_cast<size_t>(u) * F;
  const size_t ubase_s = static_cast<size_t>(u) * S;

  for (int it = s; it < NI; it += nsplit) {
    if (it < nFC) {
      // ---------------- full-resolution rows r0 .. r0+31
      const int r0 = it * kChunk;
      if (r0 >= nf) continue;
      {
        const int i = tid >> 3;
        const int p = tid & 7;
        const int row = r0 + i;
        const bool valid = row < nf;
        float dot[kMaxG];
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) dot[g] = 0.f;
        if (valid) {
          const int cpl = d / 8;
          const size_t base = (ubase_f + row) * d + static_cast<size_t>(p) * cpl;
          for (int e = 0; e < cpl; ++e) {
            const float kv = E::ld(kf, base + e);
            const int c = p * cpl + e;
#pragma unroll
            for (int g = 0; g < kMaxG; ++g)
              if (g < G) dot[g] += qs[g][c] * kv;
          }
        }
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) dot[g] = group_sum(dot[g], 8);
        if (p == 0)
          for (int g = 0; g < G; ++g) lg[i][g] = valid ? dot[g] * inv_sqrt_d : -INFINITY;
      }
      __syncthreads();
      chunk_softmax(lg, &st, G);
#pragma unroll
      for (int oi = 0; oi < kMaxOut; ++oi) {
        const int o = tid + oi * kAttThreads;
        if (o < nout) {
          const int g = o / d;
          const int c = o - g * d;
          float a = acc[oi] * st.sc[g];
          const int nr = min(kChunk, nf - r0);
          for (int i = 0; i < nr; ++i)
            a += lg[i][g] * E::ld(vf, (ubase_f + r0 + i) * d + c);
          acc[oi] = a;
        }
      }
      __syncthreads();
    } else if (it < nFC + k_slots) {
      // ---------------- expanded span sel[e], rebuilt from its factors
      const int e = it - nFC;
      if (e >= nsel) continue;
      const int j = sel[ubase_s + e];
      const int len = span_len[static_cast<size_t>(b) * S + j];
      const size_t toff = static_cast<size_t>(u) * N + tok_off[static_cast<size_t>(b) * (S + 1) + j];
      const size_t wbase = (ubase_s + j) * rank;
      for (int pi = tid; pi < G * rank; pi += kAttThreads) {
        const int g = pi / rank;
        const int k = pi - g * rank;
        const size_t wrow = (wbase + k) * d;
        float a = 0.f;
        for (int c = 0; c < d; ++c) a += E::ld(w_k, wrow + c) * qs[g][c];
        uk[g][k] = a;
        wv[g][k] = 0.f;
      }
      __syncthreads();
      for (int i0 = 0; i0 < len; i0 += kChunk) {
        for (int pi = tid; pi < kChunk * G; pi += kAttThreads) {
          const int i = pi / G;
          const int g = pi - i * G;
          const int t = i0 + i;
          float a = -INFINITY;
          if (t < len) {
            const size_t arow = (toff + t) * rank;
            a = 0.f;
            for (int k = 0; k < rank; ++k) a += E::ld(a_k, arow + k) * uk[g][k];
            a *= inv_sqrt_d;
          }
          lg[i][g] = a;
        }
        __syncthreads();
        chunk_softmax(lg, &st, G);
        const int nr = min(kChunk, len - i0);
        for (int pi = tid; pi < G * rank; pi += kAttThreads) {
          const int g = pi / rank;
          const int k = pi - g * rank;
          float a = wv[g][k] * st.sc[g];
          for (int i = 0; i < nr; ++i) a += lg[i][g] * E::ld(a_v, (toff + i0 + i) * rank + k);
          wv[g][k] = a;
        }
#pragma unroll
        for (int oi = 0; oi < kMaxOut; ++oi) {
          const int o = tid + oi * kAttThreads;
          if (o < nout) acc[oi] *= st.sc[o / d];
        }
        __syncthreads();
      }
#pragma unroll
      for (int oi = 0; oi < kMaxOut; ++oi) {
        const int o = tid + oi * kAttThreads;
        if (o < nout) {
          const int g = o / d;
          const int c = o - g * d;
          float a = acc[oi];
          for (int k = 0; k < rank; ++k) a += wv[g][k] * E::ld(w_v, (wbase + k) * d + c);
          acc[oi] = a;
        }
      }
      __syncthreads();
    } else {
      // ---------------- unexpanded spans j0 .. j0+31 (summary entries)
      const int j0 = (it - nFC - k_slots) * kChunk;
      if (j0 >= ns) continue;
      for (int pi = tid; pi < kChunk * G; pi += kAttThreads) {
        const int i = pi / G;
        const int g = pi - i * G;
        const int j = j0 + i;
        float a = -INFINITY;
        if (j < ns && !expanded[ubase_s + j]) a = slogit[(ubase_s + j) * G + g];
        lg[i][g] = a;
      }
      __syncthreads();
      chunk_softmax(lg, &st, G);
      const int nr = min(kChunk, ns - j0);
#pragma unroll
      for (int oi = 0; oi < kMaxOut; ++oi) {
        const int o = tid + oi * kAttThreads;
        if (o < nout) {
          const int g = o / d;
          const int c = o - g * d;
          float a = acc[oi] * st.sc[g];
          for (int i = 0; i < nr; ++i) {
            const float p = lg[i][g];
            if (p != 0.f) a += p * E::ld(vmean, (ubase_s + j0 + i) * d + c);
          }
          acc[oi] = a;
        }
      }
      __syncthreads();
    }
  }

  float* P = part + (static_cast<size_t>(u) * nsplit_max + s) * G * (d + 2);
  if (tid < G) {
    P[tid * (d + 2)] = st.m[tid];
    P[tid * (d + 2) + 1] = st.l[tid];
  }
#pragma unroll
  for (int oi = 0; oi < kMaxOut; ++oi) {
    const int o = tid + oi * kAttThreads;
    if (o < nout) {
      const int g = o / d;
      P[g * (d + 2) + 2 + (o - g * d)] = acc[oi];
    }
  }
}

// out[b][h*G+g][c] = sum_s e^{m_s-M} acc_s / sum_s e^{m_s-M} l_s.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part, int nsplit,
                                                    int nsplit_max, int Hkv, int G, int d,
                                                    float* __restrict__ out) {
  const int u = blockIdx.x;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const size_t ps = static_cast<size_t>(G) * (d + 2);
  const float* P = part + static_cast<size_t>(u) * nsplit_max * ps;
  for (int o = threadIdx.x; o < G * d; o += blockDim.x) {
    const int g = o / d;
    const int c = o - g * d;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, P[s * ps + g * (d + 2)]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        const float* ps_g = P + s * ps + g * (d + 2);
        const float w = expf(ps_g[0] - M);
        num += w * ps_g[2 + c];
        den += w * ps_g[1];
      }
    }
    out[(static_cast<size_t>(b) * Hkv * G + static_cast<size_t>(h) * G + g) * d + c] =
        M == -INFINITY ? 0.f : num / den;
  }
}

template <int DT>
hipError_t attend_impl(const rskv_cache* c, const void* q, int k_max, int nsplit,
                       hipStream_t st) {
  typedef typename Elem<DT>::T T;
  const int nFC = (c->F + kChunk - 1) / kChunk;
  const int nSC = (c->S + kChunk - 1) / kChunk;
  const int k_slots = k_max < c->S ? k_max : c->S;
  dim3 grid(nsplit, c->B * c->Hkv);
  hipLaunchKernelGGL(attend_kernel<DT>, grid, dim3(kAttThreads), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(c->dev.k_full),
                     static_cast<const T*>(c->dev.v_full), c->dev.n_full,
                     static_cast<const T*>(c->dev.vmean), c->dev.slogit, c->dev.expanded,
                     c->dev.n_spans, static_cast<const T*>(c->dev.a_k),
                     static_cast<const T*>(c->dev.a_v), static_cast<const T*>(c->dev.w_k),
                     static_cast<const T*>(c->dev.w_v), c->dev.span_len, c->dev.tok_off,
                     c->dev.sel, c->dev.n_sel, c->Hkv, c->G, c->d, c->S, c->F, c->N, c->rank,
                     k_slots, nsplit, c->nsplit_max, nFC, nSC,
                     1.0f / sqrtf(static_cast<float>(c->d)), c->dev.part);
  return hipGetLastError();
}

}  // namespace

int decode_nsplit(const rskv_cache* c, int k_max) {
  const int nFC = (c->F + kChunk - 1) / kChunk;
  const int nSC = (c->S + kChunk - 1) / kChunk;
  const int k_slots = k_max < c->S ? k_max : c->S;
  const int NI = nFC + k_slots + nSC;
  const int U = c->B * c->Hkv;
  int ns = (2048 + U - 1) / U;
  if (ns > NI) ns = NI;
  if (ns > c->nsplit_max) ns = c->nsplit_max;
  return ns < 1 ? 1 : ns;
}

int decode_nsplit_max(int B, int Hkv, int S, int F, int k_max_cap) {
  const int nFC = (F + kChunk - 1) / kChunk;
  const int nSC = (S + kChunk - 1) / kChunk;
  const int k_slots = k_max_cap < S ? k_max_cap : S;
  const int NI = nFC + k_slots + nSC;
  const int U = B * Hkv;
  int ns = (2048 + U - 1) / U;
  if (ns > NI) ns = NI;
  return ns < 1 ? 1 : ns;
}

hipError_t launch_attend(const rskv_cache* c, const void* q, int k_max, int nsplit,
                         hipStream_t st) {
  return c->dtype == kBF16 ? attend_impl<kBF16>(c, q, k_max, nsplit, st)
                           : attend_impl<kF32>(c, q, k_max, nsplit, st);
}

hipError_t launch_merge(const rskv_cache* c, int nsplit, float* out, hipStream_t st) {
  hipLaunchKernelGGL(merge_kernel, dim3(c->B * c->Hkv), dim3(256), 0, st, c->dev.part, nsplit,
                     c->nsplit_max, c->Hkv, c->G, c->d, out);
  return hipGetLastError();
}

}  // namespace rskv
