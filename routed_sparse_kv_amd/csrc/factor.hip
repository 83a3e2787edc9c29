// Low-rank span factors (SEKV, Metodologia 2: each span's token-level K/V
// is encoded by a low-rank SVD basis and rebuilt on demand at decode time).
//
// For every span j of every unit and for X = K or V rows of the span
// (|S| x d), the rank r_j = min(r, |S|, d) truncated SVD X ~ A W with
// A = U_r S_r (|S| x r) and W = W_r^T (r x d), zero-padded beyond r_j.
//
// Method: fp64 one-sided Jacobi (Hestenes) on the shorter side of X.
//   |S| <= d: rotate pairs of rows until all rows are orthogonal, X' = J X;
//             the rows of X' are sigma_i w_i^T, and A = X W_r.
//   |S| >  d: rotate pairs of columns, X' = X J; the columns of X' are
//             sigma_i u_i, so A = X'[:, top] and w_i = X^T x'_i / sigma_i^2.
// Only the working matrix is stored (no accumulated rotation), in LDS when
// it fits (<= 48 KB) and otherwise in a per-workgroup global slab.  Pairs of
// a sweep follow the round-robin (circle) ordering, so each round rotates
// cnt/2 disjoint pairs in parallel; a group of lanes handles one pair.
// Build-time only: this kernel is not on the decode path.
#include <algorithm>
#include <string>
#include <vector>

#include "cache.h"
#include "common.h"

namespace rskv {
namespace {

constexpr int kFacThreads = 256;
constexpr int kLdsWork = 6144;   // doubles of LDS working matrix (48 KB)
constexpr int kMaxSweeps = 40;
constexpr double kOrthTol = 1e-15;

template <int DT, bool kLds>
__global__ __launch_bounds__(kFacThreads) void factor_kernel(
    const typename Elem<DT>::T* __restrict__ K, const typename Elem<DT>::T* __restrict__ V,
    const int32_t* __restrict__ span_start, const int32_t* __restrict__ span_len,
    const int32_t* __restrict__ tok_pad, const int32_t* __restrict__ n_spans, int T, int d,
    int S, int Np, int Hkv, int rank, long long n_items, typename Elem<DT>::T* __restrict__ a_k,
    typename Elem<DT>::T* __restrict__ a_v, typename Elem<DT>::T* __restrict__ w_k,
    typename Elem<DT>::T* __restrict__ w_v, double* __restrict__ scratch, size_t slab) {
  typedef Elem<DT> E;
  typedef typename E::T ST;
  const int tid = threadIdx.x;
  __shared__ double sig[128];
  __shared__ int top[128];
  __shared__ int s_rot;
  double* work;
  if constexpr (kLds) {
    __shared__ double lds_work[kLdsWork];
    work = lds_work;
  } else {
    work = scratch + static_cast<size_t>(blockIdx.x) * slab;
  }

  for (long long item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int kv = static_cast<int>(item & 1);
    const long long rest = item >> 1;
    const int j = static_cast<int>(rest % S);
    const int u = static_cast<int>(rest / S);
    const int b = u / Hkv;
    if (j >= n_spans[b]) continue;
    const int n = span_len[static_cast<size_t>(b) * S + j];
    const bool small = static_cast<long long>(n) * d <= kLdsWork;
    if (small != kLds) continue;
    const int st = span_start[static_cast<size_t>(b) * S + j];
    const ST* X = (kv ? V : K) + (static_cast<size_t>(u) * T + st) * d;
    const bool by_rows = n <= d;
    const int cnt = by_rows ? n : d;  // vectors to orthogonalise
    const int L = by_rows ? d : n;    // their length

    for (int idx = tid; idx < n * d; idx += kFacThreads) {
      const int t = idx / d;
      const int c = idx - t * d;
      const double x = static_cast<double>(E::ld(X, idx));
      if (by_rows)
        work[t * d + c] = x;
      else
        work[static_cast<size_t>(c) * n + t] = x;
    }
    __syncthreads();

    // ---- one-sided Jacobi sweeps
    const int cnt2 = cnt + (cnt & 1);
    const int npairs = cnt2 / 2;
    int gs = kWave;
    while (gs > 1 && gs * npairs > kFacThreads) gs >>= 1;
    const int g = tid / gs;
    const int li = tid - g * gs;
    for (int sweep = 0; sweep < kMaxSweeps && cnt2 > 1; ++sweep) {
      if (tid == 0) s_rot = 0;
      __syncthreads();
      for (int r = 0; r < cnt2 - 1; ++r) {
        if (g < npairs) {
          const int pa = g == 0 ? 0 : ((g - 1 + r) % (cnt2 - 1)) + 1;
          const int pb = ((cnt2 - 2 - g + r) % (cnt2 - 1)) + 1;
          if (pa < cnt && pb < cnt) {
            double* xa = work + static_cast<size_t>(pa) * L;
            double* xb = work + static_cast<size_t>(pb) * L;
            double al = 0.0, be = 0.0, ga = 0.0;
            for (int e = li; e < L; e += gs) {
              const double x = xa[e], y = xb[e];
              al += x * x;
              be += y * y;
              ga += x * y;
            }
            al = group_sum(al, gs);
            be = group_sum(be, gs);
            ga = group_sum(ga, gs);
            if (ga != 0.0 && fabs(ga) > kOrthTol * sqrt(al * be)) {
              const double zeta = (be - al) / (2.0 * ga);
              const double t = copysign(1.0, zeta) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
              const double cs = 1.0 / sqrt(1.0 + t * t);
              const double sn = cs * t;
              for (int e = li; e < L; e += gs) {
                const double x = xa[e], y = xb[e];
                xa[e] = cs * x - sn * y;
                xb[e] = sn * x + cs * y;
              }
              if (li == 0) s_rot = 1;
            }
          }
        }
        __syncthreads();
      }
      const int rotated = s_rot;
      __syncthreads();
      if (!rotated) break;
    }

    // ---- singular values, top r_j (largest first, ties to lower index)
    for (int i = tid; i < cnt; i += kFacThreads) {
      double s2 = 0.0;
      const double* xi = work + static_cast<size_t>(i) * L;
      for (int e = 0; e < L; ++e) s2 += xi[e] * xi[e];
      sig[i] = sqrt(s2);
    }
    __syncthreads();
    const int rj = min(rank, cnt);
    if (tid < kWave) {
      bool taken0 = tid >= cnt, taken1 = tid + kWave >= cnt;
      for (int k = 0; k < rj; ++k) {
        double bv = -1.0;
        int bi = 1 << 30;
        if (!taken0) { bv = sig[tid]; bi = tid; }
        if (!taken1 && sig[tid + kWave] > bv) { bv = sig[tid + kWave]; bi = tid + kWave; }
        for (int o = kWave / 2; o > 0; o >>= 1) {
          const double ov = __shfl_xor(bv, o, kWave);
          const int oi = __shfl_xor(bi, o, kWave);
          if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        if (bi == tid) taken0 = true;
        if (bi == tid + kWave) taken1 = true;
        if (tid == 0) top[k] = bi;
      }
    }
    __syncthreads();

    // ---- factors: A_K rows (padded span offsets), A_V transposed 16-row
    // tiles, W_K rows [r][d], W_V transposed [d][r] (layout.h)
    const int tp = tok_pad[static_cast<size_t>(b) * (S + 1) + j];
    auto a_at = [&](int t, int k) -> ST& {
      if (kv) return a_v[static_cast<size_t>(u) * Np * rank + avt_off(tp + t, k, rank)];
      return a_k[(static_cast<size_t>(u) * Np + tp + t) * rank + k];
    };
    auto w_at = [&](int k, int e) -> ST& {
      if (kv) return w_v[static_cast<size_t>(u) * S * d * rank4(rank) + wvt_off(j, k, e, d, rank)];
      return w_k[((static_cast<size_t>(u) * S + j) * rank + k) * d + e];
    };
    if (by_rows) {
      for (int idx = tid; idx < rj * d; idx += kFacThreads) {
        const int k = idx / d;
        const int e = idx - k * d;
        const double s = sig[top[k]];
        w_at(k, e) = E::from_f64(s > 0.0 ? work[static_cast<size_t>(top[k]) * L + e] / s : 0.0);
      }
      for (int idx = tid; idx < n * rj; idx += kFacThreads) {
        const int t = idx / rj;
        const int k = idx - t * rj;
        const double s = sig[top[k]];
        double acc = 0.0;
        if (s > 0.0) {
          const double* wi = work + static_cast<size_t>(top[k]) * L;
          for (int e = 0; e < d; ++e)
            acc += static_cast<double>(E::ld(X, static_cast<size_t>(t) * d + e)) * wi[e];
          acc /= s;
        }
        a_at(t, k) = E::from_f64(acc);
      }
    } else {
      for (int idx = tid; idx < n * rj; idx += kFacThreads) {
        const int t = idx / rj;
        const int k = idx - t * rj;
        a_at(t, k) = E::from_f64(work[static_cast<size_t>(top[k]) * L + t]);
      }
      for (int idx = tid; idx < rj * d; idx += kFacThreads) {
        const int k = idx / d;
        const int e = idx - k * d;
        const double s = sig[top[k]];
        double acc = 0.0;
        if (s > 0.0) {
          const double* xi = work + static_cast<size_t>(top[k]) * L;
          for (int t = 0; t < n; ++t)
            acc += static_cast<double>(E::ld(X, static_cast<size_t>(t) * d + e)) * xi[t];
          acc /= s * s;
        }
        w_at(k, e) = E::from_f64(acc);
      }
    }
    __syncthreads();
  }
}

template <int DT>
hipError_t factor_impl(rskv_cache* c, const void* K, const void* V, hipStream_t st,
                       std::string* err) {
  typedef typename Elem<DT>::T T;
  const int U = c->B * c->Hkv;
  const long long n_items = 2ll * U * c->S;
  // Longest span decides the global slab size of the large-span pass.
  std::vector<int32_t> lens(static_cast<size_t>(c->B) * c->S);
  hipError_t e = hipMemcpyAsync(lens.data(), c->dev.span_len, lens.size() * sizeof(int32_t),
                                hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  long long n_large = 0;
  int max_len = 0;
  for (int b = 0; b < c->B; ++b)
    for (int j = 0; j < c->h_n_spans[b]; ++j) {
      const int n = lens[static_cast<size_t>(b) * c->S + j];
      max_len = std::max(max_len, n);
      if (static_cast<long long>(n) * c->d > kLdsWork) n_large += 2 * U / c->B;
    }
  const int grid_small = static_cast<int>(std::min<long long>(n_items, 1 << 20));
  if (n_items > 0) {
    hipLaunchKernelGGL((factor_kernel<DT, true>), dim3(grid_small), dim3(kFacThreads), 0, st,
                       static_cast<const T*>(K), static_cast<const T*>(V), c->dev.span_start,
                       c->dev.span_len, c->dev.tok_pad, c->dev.n_spans, c->T, c->d, c->S, c->Np,
                       c->Hkv, c->rank, n_items, static_cast<T*>(c->dev.a_k),
                       static_cast<T*>(c->dev.a_v), static_cast<T*>(c->dev.w_k),
                       static_cast<T*>(c->dev.w_v), nullptr, size_t(0));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_large > 0) {
    const size_t slab = static_cast<size_t>(max_len) * c->d;
    const size_t budget = size_t(512) << 20;
    long long nb = static_cast<long long>(budget / (slab * sizeof(double)));
    nb = std::max<long long>(1, std::min<long long>({nb, n_large, 1024}));
    double* scratch = nullptr;
    e = hipMalloc(&scratch, static_cast<size_t>(nb) * slab * sizeof(double));
    if (e != hipSuccess) {
      if (err) *err = "factor scratch allocation failed";
      return e;
    }
    hipLaunchKernelGGL((factor_kernel<DT, false>), dim3(static_cast<unsigned>(nb)),
                       dim3(kFacThreads), 0, st, static_cast<const T*>(K),
                       static_cast<const T*>(V), c->dev.span_start, c->dev.span_len,
                       c->dev.tok_pad, c->dev.n_spans, c->T, c->d, c->S, c->Np, c->Hkv, c->rank,
                       n_items, static_cast<T*>(c->dev.a_k), static_cast<T*>(c->dev.a_v),
                       static_cast<T*>(c->dev.w_k), static_cast<T*>(c->dev.w_v), scratch, slab);
    e = hipGetLastError();
    const hipError_t e2 = hipStreamSynchronize(st);
    (void)hipFree(scratch);
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_factor(rskv_cache* c, const void* K, const void* V, hipStream_t st,
                         std::string* err) {
  return c->dtype == kBF16 ? factor_impl<kBF16>(c, K, V, st, err)
                           : factor_impl<kF32>(c, K, V, st, err);
}

}  // namespace rskv
