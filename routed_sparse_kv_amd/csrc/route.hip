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
// topk_kernel (next launch, one workgroup per unit): exact selection by a
// narrowing fp64 histogram search for the k-th entry, compaction in index
// order, -inf over the summary logits of the selected spans (attention then
// skips their summary entries), and the per-wave work partition of the
// attention kernel.  (Handing z from one workgroup to another inside one
// kernel would need a device-scope release per workgroup, which on gfx950
// writes back the XCD's L2 and serialises; the kernel boundary is cheaper.)
#include "cache.h"
#include "common.h"
#include "lanes.h"

namespace rskv {
namespace {

constexpr int kMaxG = 16;
constexpr int kRouteThreads = 256;               // 4 waves
constexpr int kTilesPerWave = 2;                 // 16 spans per tile
constexpr int kSpansPerBlock = 4 * kTilesPerWave * 16;
constexpr int kTopkThreads = 1024;
constexpr int kTopkLds = 6144;                   // values staged in LDS (48 KB)
constexpr int kTopkBins = kTopkThreads;          // histogram bins of the threshold search

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 summaries: MFMA logits, fp64 VALU z (see the file comment).  The
// summary tiles are loaded by route_load_bf16 before rho is formed.
template <int D>
struct RouteTiles {
  bf16x8 sa[kTilesPerWave][D / 32];
  bf16x8 qb[D / 32];
  float ll[kTilesPerWave][4];  // ln|S_j| of spans j0 + 4 (lane / 16) + i
};

template <int D>
__device__ __forceinline__ void route_load_bf16(const uint16_t* __restrict__ q,
                                                const uint16_t* __restrict__ summ,
                                                const float* __restrict__ log_len, int b, int u,
                                                int h, int Hkv, int ns, int S, int G,
                                                RouteTiles<D>& rt) {
  constexpr int KK = D / 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g16 = lane & 15;
  const int grp = lane >> 4;
  const bool head_ok = g16 < G;
  const int jw = blockIdx.x * kSpansPerBlock + wave * kTilesPerWave * 16;
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int j = jw + 16 * t + g16;  // row of the A operand held by this lane
    const uint16_t* row = summ + (static_cast<size_t>(u) * S + (j < ns ? j : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      rt.sa[t][kk] = *reinterpret_cast<const bf16x8*>(row + 32 * kk + 8 * grp);
    // the logits' size bias, loaded with the tiles (not after the products)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jl = jw + 16 * t + 4 * grp + i;
      rt.ll[t][i] = log_len[static_cast<size_t>(b) * S + (jl < ns ? jl : 0)];
    }
  }
  const uint16_t* qp = q + (static_cast<size_t>(b) * Hkv * G + static_cast<size_t>(h) * G +
                            (head_ok ? g16 : 0)) * D;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    rt.qb[kk] = *reinterpret_cast<const bf16x8*>(qp + 32 * kk + 8 * grp);
}

template <int D>
__device__ __forceinline__ void route_tiles_bf16(RouteTiles<D>& rt, int u, int ns, int S, int G,
                                                 float alpha,
                                                 float inv_sqrt_d, const double* rho,
                                                 double* __restrict__ z_out,
                                                 float* __restrict__ slogit_u) {
  constexpr int KK = D / 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g16 = lane & 15;
  const int grp = lane >> 4;
  const bool head_ok = g16 < G;
  const int jw = blockIdx.x * kSpansPerBlock + wave * kTilesPerWave * 16;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    if (!head_ok) rt.qb[kk] = bf16x8{};
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int j0 = jw + 16 * t;
    if (j0 >= ns) break;
    if (j0 + g16 >= ns)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) rt.sa[t][kk] = bf16x8{};
    f32x4 lg = {0.f, 0.f, 0.f, 0.f};
    double zp = 0.0;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      lg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rt.sa[t][kk], rt.qb[kk], lg, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        zp += rho[32 * kk + 8 * grp + e] * static_cast<double>(static_cast<float>(rt.sa[t][kk][e]));
    }
    zp += xor_lane<16>(zp);
    zp += xor_lane<32>(zp);
    if (grp == 0 && j0 + g16 < ns) z_out[static_cast<size_t>(u) * S + j0 + g16] = alpha * zp;
    if (head_ok) {
      // lane holds spans j0 + 4 grp + i of head g16
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * grp + i;
        o[i] = j < ns ? lg[i] * inv_sqrt_d + rt.ll[t][i] : 0.f;
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

  // summary tiles first: their loads overlap forming rho
  [[maybe_unused]] RouteTiles<D> rt;
  if constexpr (DT == kBF16) route_load_bf16<D>(q, summ, log_len, b, u, h, Hkv, ns, S, G, rt);

  __shared__ double qbar[D];
  __shared__ double rho[D];
  __shared__ float qh[kMaxG][D];
  const size_t qbase = (static_cast<size_t>(b) * Hkv * G + static_cast<size_t>(h) * G) * D;
  if (tid < D) {
    // the group's loads are issued together, then summed in head order
    float x[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g)
      x[g] = g < G ? E::ld(q, qbase + static_cast<size_t>(g) * D + tid) : 0.f;
    double sum = 0.0;
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
      if (g < G) {
        qh[g][tid] = x[g];
        sum += static_cast<double>(x[g]);
      }
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
    route_tiles_bf16<D>(rt, u, ns, S, G, alpha, inv_sqrt_d, rho, z_all, slogit_u);
  } else {
    route_spans_f32<D>(summ, log_len, b, u, ns, S, G, alpha, inv_sqrt_d, rho, qh, z_all,
                       slogit_u);
  }
}

// Top-k cap of one unit by a whole 1024-thread workgroup, then the
// compaction of the selection and the work partition of the attention pass.
//
// Selection.  The kept set is the first k entries of the order (z
// descending, index ascending) restricted to z > tau, so it is fixed by its
// last entry (z*, j*): pick j iff z_j > tau and (z_j > z* or (z_j == z* and
// j <= j*)).  z* is found by narrowing a value interval [lo, hi] that holds
// it: a 1024-bin histogram of the values in the interval, bin
// floor((z - lo) / (hi - lo) * 1024) (monotone in z under fp64 rounding),
// locates the bin holding the k-th largest, whose own value range becomes
// the next interval.  Each round shrinks the interval about 1024-fold, so
// smooth data needs two or three rounds; once lo == hi, j* is the rem-th
// lowest index among the values equal to lo.
//
// Partition.  The attention kernel's work items of a unit, in order, are
// the expanded spans (ascending index), 32-row full-resolution chunks and
// 32-span summary chunks.  Each item has an integer cost (bytes / 64 plus
// a fixed overhead, plus a round-trip penalty per 32 rows of a span past
// the 64 its first load covers); item i goes to wave
// floor((2 P_i + c_i) W / (2 C)) (P_i the exclusive cost prefix, C the
// total), so every wave receives a contiguous item range of about C / W.
// wstart[u][w] is the first item of wave w, wstart[u][W] the item count.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const double* __restrict__ z_all, const int32_t* __restrict__ n_spans,
    const int32_t* __restrict__ n_full, const int32_t* __restrict__ span_len,
    const int32_t* __restrict__ tok_pad, int Hkv, int G, int S, int Sp, double tau, int k_max,
    float* __restrict__ slogit, int32_t* __restrict__ sel_ws, int32_t* __restrict__ desc_ws,
    int32_t* __restrict__ nsel_ws, int32_t* __restrict__ sel_out, int32_t* __restrict__ nsel_out,
    WorkCost wc, int nwaves, int wpitch, int32_t* __restrict__ wstart) {
  const int u = blockIdx.x;
  const int b = u / Hkv;
  const int tid = threadIdx.x;
  const int n = n_spans[b];
  const double* z = z_all + static_cast<size_t>(u) * S;
  int32_t* sel = sel_ws + static_cast<size_t>(u) * S;
  int4* desc = reinterpret_cast<int4*>(desc_ws) + static_cast<size_t>(u) * S;
  float* slogit_u = slogit + static_cast<size_t>(u) * Sp * G;
  const int32_t* len_b = span_len + static_cast<size_t>(b) * S;
  const int kpt = (n + kTopkThreads - 1) / kTopkThreads;
  const int i0 = tid * kpt;
  const int i1 = min(n, i0 + kpt);  // this thread's indices [i0, i1)

  __shared__ double sz[kTopkLds];
  __shared__ int hist[kTopkBins];
  __shared__ int red[17];
  __shared__ long long red64[17];
  __shared__ double redd[32];
  __shared__ int s_bin, s_above, s_cnt, s_js;

  const bool staged = n <= kTopkLds;
  if (staged) {
    for (int i = tid; i < n; i += kTopkThreads) sz[i] = z[i];
    __syncthreads();
  }
  auto zat = [&](int i) -> double { return staged ? sz[i] : z[i]; };

  // candidates z > tau: count and value range
  int c_loc = 0;
  double mn = INFINITY, mx = -INFINITY;
  for (int i = i0; i < i1; ++i) {
    const double v = zat(i);
    if (v > tau) {
      ++c_loc;
      mn = fmin(mn, v);
      mx = fmax(mx, v);
    }
  }
  int n_cand;
  block_excl_scan(c_loc, red, &n_cand);
  block_min_max(mn, mx, redd);

  double zs = INFINITY;  // pick: z > tau && (z > zs || (z == zs && j <= js))
  int js = -1;
  if (k_max > 0 && n_cand > 0) {
    if (n_cand <= k_max) {
      zs = mn;  // every candidate
      js = 0x7fffffff;
    } else {
      double lo = mn, hi = mx;
      int rem = k_max;  // entries still to take from [lo, hi]
      for (int round = 0; round < 256; ++round) {
        if (lo == hi) {
          // rem lowest indices among the values equal to lo
          int e_loc = 0;
          for (int i = i0; i < i1; ++i) e_loc += zat(i) == lo ? 1 : 0;
          int e_tot;
          const int e_before = block_excl_scan(e_loc, red, &e_tot);
          if (e_before < rem && rem <= e_before + e_loc) {
            int cnt = e_before;
            for (int i = i0; i < i1; ++i) {
              if (zat(i) == lo && ++cnt == rem) {
                s_js = i;
                break;
              }
            }
          }
          __syncthreads();
          zs = lo;
          js = s_js;
          break;
        }
        const double w = hi - lo;
        auto bin_of = [&](double v) {
          return min(kTopkBins - 1, static_cast<int>((v - lo) / w * kTopkBins));
        };
        hist[tid] = 0;
        __syncthreads();
        for (int i = i0; i < i1; ++i) {
          const double v = zat(i);
          if (v >= lo && v <= hi) atomicAdd(&hist[bin_of(v)], 1);
        }
        __syncthreads();
        // thread t holds bin 1023 - t: the exclusive scan counts the bins above
        const int cnt = hist[kTopkBins - 1 - tid];
        int tot;
        const int above = block_excl_scan(cnt, red, &tot);
        if (above < rem && rem <= above + cnt) {
          s_bin = kTopkBins - 1 - tid;
          s_above = above;
          s_cnt = cnt;
        }
        __syncthreads();
        const int bs = s_bin;
        rem -= s_above;
        const int cb = s_cnt;
        mn = INFINITY;
        mx = -INFINITY;
        for (int i = i0; i < i1; ++i) {
          const double v = zat(i);
          if (v >= lo && v <= hi && bin_of(v) == bs) {
            mn = fmin(mn, v);
            mx = fmax(mx, v);
          }
        }
        block_min_max(mn, mx, redd);
        if (cb == rem) {  // the whole bin is taken
          zs = mn;
          js = 0x7fffffff;
          break;
        }
        lo = mn;
        hi = mx;
      }
    }
  }

  // compaction in index order; the scan carries (count << 40) + cost
  auto picked = [&](int i, double v) { return v > tau && (v > zs || (v == zs && i <= js)); };
  long long loc = 0;
  for (int i = i0; i < i1; ++i)
    if (picked(i, zat(i))) loc += (1ll << 40) + wc.span(len_b[i]);
  long long tot;
  long long before = block_excl_scan(loc, red64, &tot);
  const int n_sel = static_cast<int>(tot >> 40);
  const long long e_cost = tot & ((1ll << 40) - 1);
  {
    int pos = static_cast<int>(before >> 40);
    int pre = static_cast<int>(before & ((1ll << 40) - 1));
    for (int i = i0; i < i1; ++i) {
      if (picked(i, zat(i))) {
        const int len = len_b[i];
        desc[pos] = make_int4(i, len, tok_pad[static_cast<size_t>(b) * (S + 1) + i], pre);
        sel[pos++] = i;
        pre += wc.span(len);
        for (int g = 0; g < G; ++g) slogit_u[slogit_off(i, g, G)] = -INFINITY;
      }
    }
  }
  if (tid == 0) nsel_ws[u] = n_sel;
  __syncthreads();  // desc and sel visible to the whole workgroup
  if (sel_out != nullptr)
    for (int i = tid; i < k_max; i += kTopkThreads)
      sel_out[static_cast<size_t>(u) * k_max + i] = i < n_sel ? sel[i] : -1;
  if (nsel_out != nullptr && tid == 0) nsel_out[u] = n_sel;

  if (nwaves > 0) {
    int32_t* ws = wstart + static_cast<size_t>(u) * wpitch;
    const int nFI = (n_full[b] + 31) / 32;
    const int nSI = (n + 31) / 32;
    const int NI = n_sel + nFI + nSI;
    const long long C = e_cost + static_cast<long long>(nFI) * wc.full +
                        static_cast<long long>(nSI) * wc.summ;
    const long long W = nwaves;
    if (NI == 0) {
      for (int w = tid; w <= nwaves; w += kTopkThreads) ws[w] = 0;
    }
    // cost of item i, and its exclusive prefix
    auto item = [&](int i, long long* P) -> long long {
      if (i < n_sel) {
        const int4 d = desc[i];
        *P = d.w;
        return wc.span(d.y);
      }
      if (i < n_sel + nFI) {
        *P = e_cost + static_cast<long long>(i - n_sel) * wc.full;
        return wc.full;
      }
      *P = e_cost + static_cast<long long>(nFI) * wc.full +
           static_cast<long long>(i - n_sel - nFI) * wc.summ;
      return wc.summ;
    };
    for (int i = tid; i < NI; i += kTopkThreads) {
      long long P, Pp;
      const long long c = item(i, &P);
      const long long a = (2 * P + c) * W / (2 * C);
      long long ap = -1;
      if (i > 0) {
        const long long cp = item(i - 1, &Pp);
        ap = (2 * Pp + cp) * W / (2 * C);
      }
      for (long long w = ap + 1; w <= a; ++w) ws[w] = i;
      if (i == NI - 1)
        for (long long w = a + 1; w <= W; ++w) ws[w] = NI;
    }
  }
}

template <int DT, int D>
hipError_t route_impl(const rskv_cache* c, const DecodeWs& ws, const void* q, hipStream_t st,
                      const KernelEvents* ev) {
  typedef typename Elem<DT>::T T;
  const int nblk = (c->S + kSpansPerBlock - 1) / kSpansPerBlock;
  dim3 grid(nblk, c->B * c->Hkv);
  return launch(route_kernel<DT, D>, grid, dim3(kRouteThreads), 0, st, ev,
                static_cast<const T*>(q), static_cast<const T*>(c->dev.summary), c->dev.log_len,
                c->dev.n_spans, c->dev.proj, c->n_proj, c->Hkv, c->G, c->S, c->Sp, c->alpha,
                1.0f / sqrtf(static_cast<float>(D)), ws.z, ws.slogit);
}

}  // namespace

hipError_t launch_route(const rskv_cache* c, const DecodeWs& ws, const void* q, hipStream_t st,
                        const KernelEvents* ev) {
  if (c->dtype == kBF16)
    return c->d == 128 ? route_impl<kBF16, 128>(c, ws, q, st, ev)
                       : route_impl<kBF16, 64>(c, ws, q, st, ev);
  return c->d == 128 ? route_impl<kF32, 128>(c, ws, q, st, ev)
                     : route_impl<kF32, 64>(c, ws, q, st, ev);
}

hipError_t launch_topk(const rskv_cache* c, const DecodeWs& ws, float tau, int k_max, int nwaves,
                       int32_t* sel_out, int32_t* nsel_out, hipStream_t st,
                       const KernelEvents* ev) {
  const WorkCost wc = work_cost(c);
  return launch(topk_kernel, dim3(c->B * c->Hkv), dim3(kTopkThreads), 0, st, ev, ws.z,
                c->dev.n_spans, c->dev.n_full, c->dev.span_len, c->dev.tok_pad, c->Hkv, c->G, c->S,
                c->Sp, static_cast<double>(tau), k_max, ws.slogit, ws.sel, ws.sel_desc, ws.n_sel,
                sel_out, nsel_out, wc, nwaves, 4 * c->nsplit_max + 1, ws.wstart);
}

}  // namespace rskv
