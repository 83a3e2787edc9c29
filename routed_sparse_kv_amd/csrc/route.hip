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
// The same pass stores, for every span and query head, the logit the span
// carries if it stays unexpanded, <q_h, s_j>/sqrt(d) + ln|S_j|, so the
// summaries are read from HBM once per step.
//
// route_kernel (bf16): a wave takes 16-span tiles of the summary matrix as
// the A operand of 16x16x32 MFMAs against the G queries (the summary logits,
// fp32 accumulation of exact bf16 products); the same registers hold 32
// elements of one span row per lane, so z needs 32 fp64 FMAs per lane and a
// two-step reduction over the four lane groups.  fp32 caches use a VALU
// version (16 lanes per span row).
// topk_kernel (next launch, one workgroup per unit): keys are order-
// preserving uint64 images of z, staged in LDS when they fit; an 8-bit-digit
// radix select from the top stops as soon as the bucket holding the k-th
// largest key is taken whole, and a block scan writes the selected indices
// in ascending order.  It also overwrites the summary logits of the
// selected spans with -inf, so that attention skips their summary entries.
// (Handing z from one workgroup to another inside one kernel would need a
// device-scope release per workgroup, which on gfx950 writes back the XCD's
// L2 and serialises; the kernel boundary is cheaper.)
#include "cache.h"
#include "common.h"

namespace rskv {
namespace {

constexpr int kMaxG = 8;
constexpr int kRouteThreads = 256;               // 4 waves
constexpr int kTilesPerWave = 2;                 // 16 spans per tile
constexpr int kSpansPerBlock = 4 * kTilesPerWave * 16;
constexpr int kTopkThreads = 1024;
constexpr int kTopkLds = 6144;                   // keys staged in LDS (48 KB)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 summaries: MFMA logits, fp64 VALU z (see the file comment).
template <int D>
__device__ __forceinline__ void route_tiles_bf16(const uint16_t* __restrict__ q,
                                                 const uint16_t* __restrict__ summ,
                                                 const float* __restrict__ log_len, int b,
                                                 int u, int h, int Hkv, int ns, int S, int G,
                                                 float alpha, float inv_sqrt_d,
                                                 const double* rho, double* __restrict__ z_out,
                                                 float* __restrict__ slogit_u) {
  constexpr int KK = D / 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g16 = lane & 15;
  const int grp = lane >> 4;
  const bool head_ok = g16 < G;
  bf16x8 qb[KK];
  {
    const uint16_t* qp = q + (static_cast<size_t>(b) * Hkv * G + static_cast<size_t>(h) * G +
                              (head_ok ? g16 : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qb[kk] = *reinterpret_cast<const bf16x8*>(qp + 32 * kk + 8 * grp);
      if (!head_ok) qb[kk] = bf16x8{};
    }
  }
  const int jw = blockIdx.x * kSpansPerBlock + wave * kTilesPerWave * 16;
  bf16x8 sa[kTilesPerWave][KK];
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int j = jw + 16 * t + g16;  // row of the A operand held by this lane
    const uint16_t* row = summ + (static_cast<size_t>(u) * S + (j < ns ? j : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      sa[t][kk] = *reinterpret_cast<const bf16x8*>(row + 32 * kk + 8 * grp);
      if (j >= ns) sa[t][kk] = bf16x8{};
    }
  }
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int j0 = jw + 16 * t;
    if (j0 >= ns) break;
    f32x4 lg = {0.f, 0.f, 0.f, 0.f};
    double zp = 0.0;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      lg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa[t][kk], qb[kk], lg, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        zp += rho[32 * kk + 8 * grp + e] * static_cast<double>(static_cast<float>(sa[t][kk][e]));
    }
    zp += __shfl_xor(zp, 16, kWave);
    zp += __shfl_xor(zp, 32, kWave);
    if (grp == 0 && j0 + g16 < ns) z_out[static_cast<size_t>(u) * S + j0 + g16] = alpha * zp;
    if (head_ok) {
      // lane holds spans j0 + 4 grp + i of head g16
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * grp + i;
        o[i] = j < ns ? lg[i] * inv_sqrt_d + log_len[static_cast<size_t>(b) * S + j] : 0.f;
      }
      *reinterpret_cast<f32x4*>(slogit_u + slogit_off(j0 + 4 * grp, g16, G)) = o;
    }
  }
}

// fp32 summaries: 16 lanes per span row, 4 spans per wave instruction.
template <int D>
__device__ __forceinline__ void route_spans_f32(const float* __restrict__ summ,
                                                const float* __restrict__ log_len, int b, int u,
                                                int ns, int S, int G, float alpha,
                                                float inv_sqrt_d, const double* rho,
                                                const float (*qh)[D], double* __restrict__ z_out,
                                                float* __restrict__ slogit_u) {
  constexpr int kEpl = D / 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int grp = lane >> 4;
  const int li = lane & 15;
  const int j_base = blockIdx.x * kSpansPerBlock + wave * kTilesPerWave * 16;
  for (int it = 0; it < kTilesPerWave * 4; ++it) {
    const int j = j_base + it * 4 + grp;
    const bool valid = j < ns;
    float sv[kEpl];
#pragma unroll
    for (int e = 0; e < kEpl; ++e)
      sv[e] = valid ? summ[(static_cast<size_t>(u) * S + j) * D + li * kEpl + e] : 0.f;
    double zacc = 0.0;
    float lacc[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) lacc[g] = 0.f;
#pragma unroll
    for (int e = 0; e < kEpl; ++e) {
      const int c = li * kEpl + e;
      zacc += rho[c] * static_cast<double>(sv[e]);
#pragma unroll
      for (int g = 0; g < kMaxG; ++g)
        if (g < G) lacc[g] += qh[g][c] * sv[e];
    }
    zacc = group_sum(zacc, 16);
#pragma unroll
    for (int g = 0; g < kMaxG; ++g)
      if (g < G) lacc[g] = group_sum(lacc[g], 16);
    if (valid && li == 0) {
      z_out[static_cast<size_t>(u) * S + j] = static_cast<double>(alpha) * zacc;
      const float ell = log_len[static_cast<size_t>(b) * S + j];
#pragma unroll
      for (int g = 0; g < kMaxG; ++g)
        if (g < G) slogit_u[slogit_off(j, g, G)] = lacc[g] * inv_sqrt_d + ell;
    }
  }
}

template <int DT, int D>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ summ,
    const float* __restrict__ log_len, const int32_t* __restrict__ n_spans,
    const float* __restrict__ proj, int n_proj, int Hkv, int G, int S, int Sp, float alpha,
    float inv_sqrt_d, double* __restrict__ z_all, float* __restrict__ slogit) {
  typedef Elem<DT> E;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int tid = threadIdx.x;
  const int ns = n_spans[b];
  if (static_cast<int>(blockIdx.x) * kSpansPerBlock >= ns) return;
  float* slogit_u = slogit + static_cast<size_t>(u) * Sp * G;

  __shared__ double qbar[D];
  __shared__ double rho[D];
  __shared__ float qh[kMaxG][D];
  const size_t qbase = (static_cast<size_t>(b) * Hkv * G + static_cast<size_t>(h) * G) * D;
  if (tid < D) {
    double sum = 0.0;
    for (int g = 0; g < G; ++g) {
      const float x = E::ld(q, qbase + static_cast<size_t>(g) * D + tid);
      qh[g][tid] = x;
      sum += static_cast<double>(x);
    }
    qbar[tid] = sum / static_cast<double>(G);
  }
  __syncthreads();
  if (tid < D) {
    if (proj != nullptr) {
      const float* P = proj + static_cast<size_t>(n_proj == 1 ? 0 : h) * D * D +
                       static_cast<size_t>(tid) * D;
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc += static_cast<double>(P[c]) * qbar[c];
      rho[tid] = acc;
    } else {
      rho[tid] = qbar[tid];
    }
  }
  __syncthreads();
  if constexpr (DT == kBF16) {
    route_tiles_bf16<D>(q, summ, log_len, b, u, h, Hkv, ns, S, G, alpha, inv_sqrt_d, rho,
                        z_all, slogit_u);
  } else {
    route_spans_f32<D>(summ, log_len, b, u, ns, S, G, alpha, inv_sqrt_d, rho, qh, z_all,
                       slogit_u);
  }
}

// Top-k cap of one unit by a whole 1024-thread workgroup.  Thread t owns the
// contiguous indices [t*kpt, t*kpt + kpt).
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const double* __restrict__ z_all, const int32_t* __restrict__ n_spans,
    const int32_t* __restrict__ span_len, const int32_t* __restrict__ tok_pad, int Hkv, int G,
    int S, int Sp, double tau, int k_max, float* __restrict__ slogit,
    int32_t* __restrict__ sel_ws, int32_t* __restrict__ desc_ws, int32_t* __restrict__ nsel_ws,
    int32_t* __restrict__ sel_out, int32_t* __restrict__ nsel_out) {
  const int u = blockIdx.x;
  const int b = u / Hkv;
  const int tid = threadIdx.x;
  const int n = n_spans[b];
  const double* z = z_all + static_cast<size_t>(u) * S;
  int32_t* sel = sel_ws + static_cast<size_t>(u) * S;
  int4* desc = reinterpret_cast<int4*>(desc_ws) + static_cast<size_t>(u) * S;
  float* slogit_u = slogit + static_cast<size_t>(u) * Sp * G;
  const int kpt = (n + kTopkThreads - 1) / kTopkThreads;
  const int i0 = tid * kpt;
  const int mine = max(0, min(kpt, n - i0));  // valid indices of this thread

  __shared__ unsigned long long skey[kTopkLds];
  __shared__ int red[17];
  __shared__ unsigned hist[256];
  __shared__ int s_dg, s_above, s_cnt;

  const bool staged = n <= kTopkLds;
  if (staged) {
    for (int i = tid; i < n; i += kTopkThreads) skey[i] = f64_order_key(z[i]);
    __syncthreads();
  }
  // f(i, key) for this thread's valid keys, in index order
  auto for_keys = [&](auto&& f) {
    if (staged) {
      for (int i = 0; i < mine; ++i) f(i, skey[i0 + i]);
    } else {
      for (int i = 0; i < mine; ++i) f(i, f64_order_key(z[i0 + i]));
    }
  };

  const unsigned long long ktau = f64_order_key(tau);
  int c_loc = 0;
  for_keys([&](int, unsigned long long k) { c_loc += k > ktau ? 1 : 0; });
  int n_cand;
  block_excl_scan(c_loc, red, &n_cand);

  // selection rule: (key & M) > P, or (key & M) == P among the first `rem`
  unsigned long long P = ktau, M = ~0ull;
  int rem = 0;
  if (k_max == 0) {
    P = ~0ull;  // nothing above
  } else if (n_cand > k_max) {
    P = 0ull;
    M = 0ull;
    rem = k_max;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0u;
      __syncthreads();
      for_keys([&](int, unsigned long long k) {
        if ((k & M) == P) atomicAdd(&hist[(k >> shift) & 255ull], 1u);
      });
      __syncthreads();
      if (tid < kWave) {
        // lane l covers bins 255-4l .. 252-4l, highest first
        int hb[4], ts = 0;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          hb[qq] = static_cast<int>(hist[255 - 4 * tid - qq]);
          ts += hb[qq];
        }
        const int incl = wave_incl_scan(ts);
        const unsigned long long hit = __ballot(incl >= rem);
        const int first = __ffsll(static_cast<long long>(hit)) - 1;
        if (tid == first) {
          int acc = incl - ts;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            if (acc + hb[qq] >= rem) {
              s_dg = 255 - 4 * tid - qq;
              s_above = acc;
              s_cnt = hb[qq];
              break;
            }
            acc += hb[qq];
          }
        }
      }
      __syncthreads();
      P |= static_cast<unsigned long long>(s_dg) << shift;
      M |= 255ull << shift;
      rem -= s_above;
      const bool whole = s_cnt == rem;
      __syncthreads();
      if (whole) break;
    }
  }

  // flags, rank among the keys equal to P under M, compaction
  int eq_loc = 0;
  for_keys([&](int, unsigned long long k) { eq_loc += (k & M) == P ? 1 : 0; });
  int eq_tot;
  const int eq_before = block_excl_scan(eq_loc, red, &eq_tot);
  int pick_loc = 0;
  {
    int eb = eq_before;
    for_keys([&](int, unsigned long long k) {
      const unsigned long long km = k & M;
      pick_loc += (km > P || (km == P && eb < rem)) ? 1 : 0;
      eb += km == P ? 1 : 0;
    });
  }
  int n_sel;
  int pos = block_excl_scan(pick_loc, red, &n_sel);
  {
    int eb = eq_before;
    for_keys([&](int i, unsigned long long k) {
      const unsigned long long km = k & M;
      const bool pick = km > P || (km == P && eb < rem);
      eb += km == P ? 1 : 0;
      if (pick) {
        const int j = i0 + i;
        desc[pos] = make_int4(j, span_len[static_cast<size_t>(b) * S + j],
                              tok_pad[static_cast<size_t>(b) * (S + 1) + j], 0);
        sel[pos++] = j;
        for (int g = 0; g < G; ++g) slogit_u[slogit_off(j, g, G)] = -INFINITY;
      }
    });
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

template <int DT, int D>
hipError_t route_impl(const rskv_cache* c, const void* q, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  const int nblk = (c->S + kSpansPerBlock - 1) / kSpansPerBlock;
  dim3 grid(nblk, c->B * c->Hkv);
  hipLaunchKernelGGL((route_kernel<DT, D>), grid, dim3(kRouteThreads), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(c->dev.summary),
                     c->dev.log_len, c->dev.n_spans, c->dev.proj, c->n_proj, c->Hkv, c->G, c->S,
                     c->Sp, c->alpha, 1.0f / sqrtf(static_cast<float>(D)), c->dev.z,
                     c->dev.slogit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const rskv_cache* c, const void* q, hipStream_t st) {
  if (c->dtype == kBF16)
    return c->d == 128 ? route_impl<kBF16, 128>(c, q, st) : route_impl<kBF16, 64>(c, q, st);
  return c->d == 128 ? route_impl<kF32, 128>(c, q, st) : route_impl<kF32, 64>(c, q, st);
}

hipError_t launch_topk(const rskv_cache* c, float tau, int k_max, int32_t* sel_out,
                       int32_t* nsel_out, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3(c->B * c->Hkv), dim3(kTopkThreads), 0, st, c->dev.z,
                     c->dev.n_spans, c->dev.span_len, c->dev.tok_pad, c->Hkv, c->G, c->S, c->Sp,
                     static_cast<double>(tau), k_max, c->dev.slogit, c->dev.sel,
                     c->dev.sel_desc, c->dev.n_sel, sel_out, nsel_out);
  return hipGetLastError();
}

}  // namespace rskv
