// Low-rank span factors (SEKV, Metodologia 2: each span's token-level K/V
// is encoded by a low-rank SVD basis and rebuilt on demand at decode time).
//
// For every span j of every unit and for X = K or V rows of the span
// (|S| x d), the rank r_j = min(r, |S|, d) truncated SVD X ~ A W with
// A = U_r S_r (|S| x r) and W = W_r^T (r x d), zero-padded beyond r_j.
//
// Two methods, both in fp64:
// - factor_kernel (build, spans whose |S| x d working matrix fits 48 KB of
//   LDS): one-sided Jacobi (Hestenes) on the shorter side of X.
//     |S| <= d: rotate pairs of rows until all rows are orthogonal,
//               X' = J X; the rows of X' are sigma_i w_i^T, and A = X W_r.
//     |S| >  d: rotate pairs of columns, X' = X J; the columns of X' are
//               sigma_i u_i, so A = X'[:, top] and w_i = X^T x'_i / sigma_i^2.
//   Only the working matrix is stored (no accumulated rotation).  Pairs of
//   a sweep follow the round-robin (circle) ordering, so each round rotates
//   cnt/2 disjoint pairs in parallel; a group of lanes handles one pair.
// - factor_run (build of longer spans in factor_gram_kernel, and span
//   closing in close_kernel): the r_j largest eigenpairs of the Gram matrix
//   (see the comment above tridiagonalize), Jacobi on the Gram matrix for
//   clustered spectra.
// Build and closing only: none of this is on the decode path.
#include <algorithm>
#include <type_traits>
#include <string>
#include <vector>

#include "cache.h"
#include "common.h"

namespace rskv {
namespace {

constexpr int kFacThreads = 256;
constexpr int kLdsWork = 6144;   // doubles of LDS working matrix (48 KB)
constexpr int kMaxSweeps = 40;
// A pair of rows counts as orthogonal once |<a,b>| <= L eps ||a|| ||b||:
// the rounding error of a length-L fp64 dot product can reach that size,
// so a tighter test would keep rotating on rounding noise.
constexpr double kEps = 2.220446049250313e-16;

// One DPP lane exchange of a double (both halves with the same control).
// bound_ctrl: a disabled source lane reads 0 and no old value has to be
// set up first (two instructions fewer per exchange).
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long i = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(i), kCtrl, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(i >> 32), kCtrl, 0xf, 0xf, true);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

// Sums of three values over aligned groups of GS lanes (a power of two
// <= 64), left in every lane of the group.  Inside a 16-lane row the
// partners come from DPP (quad xor 1, quad xor 2, half-row mirror, row
// mirror: each step adds the other half of the current block, so every lane
// ends with the same sum); across rows from lane shuffles.
template <int GS>
__device__ __forceinline__ void group_sum3(double& a, double& b, double& c) {
  if constexpr (GS >= 2) {
    a += dpp_f64<0xb1>(a); b += dpp_f64<0xb1>(b); c += dpp_f64<0xb1>(c);
  }
  if constexpr (GS >= 4) {
    a += dpp_f64<0x4e>(a); b += dpp_f64<0x4e>(b); c += dpp_f64<0x4e>(c);
  }
  if constexpr (GS >= 8) {
    a += dpp_f64<0x141>(a); b += dpp_f64<0x141>(b); c += dpp_f64<0x141>(c);
  }
  if constexpr (GS >= 16) {
    a += dpp_f64<0x140>(a); b += dpp_f64<0x140>(b); c += dpp_f64<0x140>(c);
  }
#pragma unroll
  for (int o = 16; o < GS; o <<= 1) {
    const double pa = __shfl_xor(a, o, kWave);
    const double pb = __shfl_xor(b, o, kWave);
    const double pc = __shfl_xor(c, o, kWave);
    a += pa;
    b += pb;
    c += pc;
  }
}

// 1/x and 1/sqrt(x): the hardware estimate refined by one Newton step,
// which squares its relative error (a rotation then stays orthogonal to
// far below the storage rounding, and its angle is accurate enough for the
// sweep's quadratic convergence).
__device__ __forceinline__ double recip(double x) {
  const double r = __builtin_amdgcn_rcp(x);
  return fma(r, fma(-x, r, 1.0), r);
}
__device__ __forceinline__ double rsqrt_nr(double x) {
  const double y = __builtin_amdgcn_rsq(x);
  return y * fma(-0.5 * x * y, y, 1.5);
}

// LDS of one factorisation: singular values, the order of the top ones and
// the "a pair was rotated" flag of the current sweep.
struct FactorShared {
  double sig[128];
  int top[128];
  int rot;
};

// One-sided Jacobi sweeps over the `cnt` rows (length L, pitch P) of
// `work` until no pair of rows needs a rotation (or kMaxSweeps).  A round
// rotates cnt/2 disjoint pairs in parallel (round-robin ordering) with GS
// lanes per pair.  The cost of a round is its instruction count (a wave64
// VALU instruction takes 4 cycles), so the rotation comes from reciprocal
// and rsqrt estimates, the pair indices need no integer division, and with
// E > 0 (L = E * GS) a lane keeps its E elements of both rows in registers
// (addressed with immediate offsets, loaded together without branches)
// between the dot products and the rotation; E = 0 loops over L with
// stride GS instead.  NW waves take part: with one
// wave the rounds need no workgroup barrier (a wave's LDS accesses complete
// in order) and the "rotated" flag is a wave vote.  Returns the number of
// sweeps; ends with a barrier of the NW waves.
template <int GS, int NW, int E>
__device__ __forceinline__ int jacobi_sweeps_gs(double* work, int cnt, int L, int P,
                                                FactorShared& sh) {
  constexpr int kReg = E > 0 ? E : 1;
  const int tid = threadIdx.x;
  const int cnt2 = cnt + (cnt & 1);
  const int m = cnt2 - 1;  // rounds per sweep
  const int npairs = cnt2 / 2;
  const int g = tid / GS;
  const int li = tid - g * GS;
  const double tol2 = (L * kEps) * (L * kEps);
  auto round_sync = [] {
    if constexpr (NW == 1) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      __syncthreads();
    }
  };
  for (int sweep = 0; sweep < kMaxSweeps && cnt2 > 1; ++sweep) {
    bool did = false;
    if constexpr (NW > 1) {
      if (tid == 0) sh.rot = 0;
      __syncthreads();
    }
    for (int r = 0; r < m; ++r) {
      if (g < npairs) {
        int pa = 0;
        if (g > 0) {
          pa = g - 1 + r;  // < 2m
          pa = (pa >= m ? pa - m : pa) + 1;
        }
        int pb = cnt2 - 2 - g + r;  // in [0, 2m)
        pb = (pb >= m ? pb - m : pb) + 1;
        if (pa < cnt && pb < cnt) {
          double* xa = work + static_cast<size_t>(pa) * P + li;
          double* xb = work + static_cast<size_t>(pb) * P + li;
          double al = 0.0, be = 0.0, ga = 0.0;
          double va[kReg], vb[kReg];
          if constexpr (E > 0) {
#pragma unroll
            for (int i = 0; i < E; ++i) {
              va[i] = xa[i * GS];
              vb[i] = xb[i * GS];
            }
#pragma unroll
            for (int i = 0; i < E; ++i) {
              al = fma(va[i], va[i], al);
              be = fma(vb[i], vb[i], be);
              ga = fma(va[i], vb[i], ga);
            }
          } else {
            for (int e = 0; e < L - li; e += GS) {
              const double p = xa[e], q = xb[e];
              al = fma(p, p, al);
              be = fma(q, q, be);
              ga = fma(p, q, ga);
            }
          }
          group_sum3<GS>(al, be, ga);
          if (ga != 0.0 && ga * ga > tol2 * (al * be)) {
            // tan of the angle that zeroes <a,b>: t = sign(tau) rho /
            // (|tau| + sqrt(tau^2 + rho^2)), tau = be - al, rho = 2 ga
            const double tau = be - al, rho = 2.0 * ga;
            const double q = fma(tau, tau, rho * rho);
            const double root = q * rsqrt_nr(q);
            const double t = copysign(1.0, tau) * rho * recip(fabs(tau) + root);
            const double cs = rsqrt_nr(fma(t, t, 1.0));
            const double sn = cs * t;
            if constexpr (E > 0) {
#pragma unroll
              for (int i = 0; i < E; ++i) {
                xa[i * GS] = cs * va[i] - sn * vb[i];
                xb[i * GS] = sn * va[i] + cs * vb[i];
              }
            } else {
              for (int e = 0; e < L - li; e += GS) {
                const double p = xa[e], q = xb[e];
                xa[e] = cs * p - sn * q;
                xb[e] = sn * p + cs * q;
              }
            }
            did = true;
            if constexpr (NW > 1) {
              if (li == 0) sh.rot = 1;
            }
          }
        }
      }
      round_sync();
    }
    int rotated;
    if constexpr (NW == 1) {
      rotated = __any(did);
    } else {
      rotated = sh.rot;
      __syncthreads();
    }
    if (!rotated) return sweep + 1;
  }
  return kMaxSweeps;
}

// Lanes per pair that make a Jacobi round over `cnt` rows occupy about NT
// threads: the largest power of two <= 64 with lanes * pairs <= NT.
template <int NT>
__device__ __forceinline__ int jacobi_group(int cnt) {
  const int npairs = (cnt + 1) / 2;
  int gs = kWave;
  while (gs > 1 && gs * npairs > NT) gs >>= 1;
  return gs;
}

// Row pitch (doubles) of an LDS working matrix with rows of length L for
// Jacobi with gs lanes per pair.  A wave reads rows of consecutive indices
// (the round-robin ordering advances pairs by one row), so a pitch of
// gs (mod 32) doubles starts each row 2 gs banks after the previous one and
// the wave's groups tile the 64 banks instead of colliding.
__device__ __forceinline__ int jacobi_pitch(int L, int gs) {
  return gs >= 32 ? L : L + (((gs - L) % 32) + 32) % 32;
}

// jacobi_sweeps_gs with E = L / GS registers per lane when that is a power
// of two (and GS * E <= 128), else the strided loop.
template <int GS, int NW>
__device__ __forceinline__ int jacobi_sweeps_e(double* work, int cnt, int L, int P,
                                               FactorShared& sh) {
  const int e = L % GS == 0 ? L / GS : 0;
  switch (e) {
    case 1: return jacobi_sweeps_gs<GS, NW, 1>(work, cnt, L, P, sh);
    case 2:
      if constexpr (2 * GS <= 128) return jacobi_sweeps_gs<GS, NW, 2>(work, cnt, L, P, sh);
      break;
    case 4:
      if constexpr (4 * GS <= 128) return jacobi_sweeps_gs<GS, NW, 4>(work, cnt, L, P, sh);
      break;
    case 8:
      if constexpr (8 * GS <= 128) return jacobi_sweeps_gs<GS, NW, 8>(work, cnt, L, P, sh);
      break;
    case 16:
      if constexpr (16 * GS <= 128) return jacobi_sweeps_gs<GS, NW, 16>(work, cnt, L, P, sh);
      break;
    case 32:
      if constexpr (32 * GS <= 128) return jacobi_sweeps_gs<GS, NW, 32>(work, cnt, L, P, sh);
      break;
    default:
      break;
  }
  return jacobi_sweeps_gs<GS, NW, 0>(work, cnt, L, P, sh);
}

// Jacobi sweeps (see jacobi_sweeps_gs) by the first NT threads (a multiple
// of the wave size) with jacobi_group<NT>(cnt) lanes per pair.
template <int NT>
__device__ __forceinline__ int jacobi_sweeps(double* work, int cnt, int L, int P,
                                             FactorShared& sh) {
  constexpr int NW = NT / kWave;
  switch (jacobi_group<NT>(cnt)) {
    case 64: return jacobi_sweeps_e<64, NW>(work, cnt, L, P, sh);
    case 32: return jacobi_sweeps_e<32, NW>(work, cnt, L, P, sh);
    case 16: return jacobi_sweeps_e<16, NW>(work, cnt, L, P, sh);
    case 8: return jacobi_sweeps_e<8, NW>(work, cnt, L, P, sh);
    case 4: return jacobi_sweeps_e<4, NW>(work, cnt, L, P, sh);
    case 2: return jacobi_sweeps_gs<2, NW, 0>(work, cnt, L, P, sh);
    default: return jacobi_sweeps_gs<1, NW, 0>(work, cnt, L, P, sh);
  }
}

// Norms of the `cnt` rows (length L, pitch P) of `work` into sh.sig and the indices of the
// min(rank, cnt) largest into sh.top (largest first, ties to the lower
// index).  Returns that count.  Ends with a barrier.
template <int NT>
__device__ int top_rows(const double* work, int cnt, int L, int P, int rank,
                        FactorShared& sh) {
  const int tid = threadIdx.x;
  for (int i = tid; i < cnt; i += NT) {
    double s2 = 0.0;
    const double* xi = work + static_cast<size_t>(i) * P;
    for (int e = 0; e < L; ++e) s2 += xi[e] * xi[e];
    sh.sig[i] = sqrt(s2);
  }
  __syncthreads();
  const int rj = min(rank, cnt);
  if (tid < kWave) {
    bool taken0 = tid >= cnt, taken1 = tid + kWave >= cnt;
    for (int k = 0; k < rj; ++k) {
      double bv = -1.0;
      int bi = 1 << 30;
      if (!taken0) { bv = sh.sig[tid]; bi = tid; }
      if (!taken1 && sh.sig[tid + kWave] > bv) { bv = sh.sig[tid + kWave]; bi = tid + kWave; }
      for (int o = kWave / 2; o > 0; o >>= 1) {
        const double ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (bi == tid) taken0 = true;
      if (bi == tid + kWave) taken1 = true;
      if (tid == 0) sh.top[k] = bi;
    }
  }
  __syncthreads();
  return rj;
}

// Rank-r factors of the n x d matrix X whose element (t, c) is x(t, c), in
// fp64 (build path, kFacThreads threads).  `work` holds n*d doubles of LDS.
// Jacobi runs on the shorter side of X:
//   n <= d: rows of X; the rotated rows are sigma_i w_i^T and A = X W_r;
//   n >  d: columns of X; they become sigma_i u_i, so A = X'[:, top] and
//           w_i = X^T x'_i / sigma_i^2.
// A (n x r_j) goes out through a_out(t, k, value), W (r_j x d) through
// w_out(k, e, value); entries beyond r_j are not written.  Every thread of
// the block calls it; it ends with a barrier.
template <class Ld, class AOut, class WOut>
__device__ void factor_matrix(const Ld& x, int n, int d, int rank, double* work,
                              FactorShared& sh, const AOut& a_out, const WOut& w_out) {
  const int tid = threadIdx.x;
  const bool by_rows = n <= d;
  const int cnt = by_rows ? n : d;  // vectors to orthogonalise
  const int L = by_rows ? d : n;    // their length

  for (int idx = tid; idx < n * d; idx += kFacThreads) {
    const int t = idx / d;
    const int c = idx - t * d;
    const double v = x(t, c);
    if (by_rows)
      work[t * d + c] = v;
    else
      work[static_cast<size_t>(c) * n + t] = v;
  }
  __syncthreads();
  jacobi_sweeps<kFacThreads>(work, cnt, L, L, sh);
  const int rj = top_rows<kFacThreads>(work, cnt, L, L, rank, sh);

  if (by_rows) {
    for (int idx = tid; idx < rj * d; idx += kFacThreads) {
      const int k = idx / d;
      const int e = idx - k * d;
      const double s = sh.sig[sh.top[k]];
      w_out(k, e, s > 0.0 ? work[static_cast<size_t>(sh.top[k]) * L + e] / s : 0.0);
    }
    for (int idx = tid; idx < n * rj; idx += kFacThreads) {
      const int t = idx / rj;
      const int k = idx - t * rj;
      const double s = sh.sig[sh.top[k]];
      double acc = 0.0;
      if (s > 0.0) {
        const double* wi = work + static_cast<size_t>(sh.top[k]) * L;
        for (int e = 0; e < d; ++e) acc += x(t, e) * wi[e];
        acc /= s;
      }
      a_out(t, k, acc);
    }
  } else {
    for (int idx = tid; idx < n * rj; idx += kFacThreads) {
      const int t = idx / rj;
      const int k = idx - t * rj;
      a_out(t, k, work[static_cast<size_t>(sh.top[k]) * L + t]);
    }
    for (int idx = tid; idx < rj * d; idx += kFacThreads) {
      const int k = idx / d;
      const int e = idx - k * d;
      const double s = sh.sig[sh.top[k]];
      double acc = 0.0;
      if (s > 0.0) {
        const double* xi = work + static_cast<size_t>(sh.top[k]) * L;
        for (int t = 0; t < n; ++t) acc += x(t, e) * xi[t];
        acc /= s * s;
      }
      w_out(k, e, acc);
    }
  }
  __syncthreads();
}

// Build: one item per (unit, span, K or V) for the spans whose rows fit the
// LDS working matrix (longer ones go to factor_gram_kernel); the span's rows
// are read from the row-major K/V inputs.  A_K rows at the span's padded
// offset, A_V in transposed 16-row tiles, W_K rows [r][d], W_V in the
// paired layout (layout.h).
template <int DT>
__global__ __launch_bounds__(kFacThreads) void factor_kernel(
    const typename Elem<DT>::T* __restrict__ K, const typename Elem<DT>::T* __restrict__ V,
    const int32_t* __restrict__ span_start, const int32_t* __restrict__ span_len,
    const int32_t* __restrict__ tok_pad, const int32_t* __restrict__ n_spans, int T, int d,
    int S, int Np, int Hkv, int rank, long long n_items, typename Elem<DT>::T* __restrict__ a_k,
    typename Elem<DT>::T* __restrict__ a_v, typename Elem<DT>::T* __restrict__ w_k,
    typename Elem<DT>::T* __restrict__ w_v) {
  typedef Elem<DT> E;
  typedef typename E::T ST;
  __shared__ FactorShared sh;
  __shared__ double work[kLdsWork];

  for (long long item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int kv = static_cast<int>(item & 1);
    const long long rest = item >> 1;
    const int j = static_cast<int>(rest % S);
    const int u = static_cast<int>(rest / S);
    const int b = u / Hkv;
    if (j >= n_spans[b]) continue;
    const int n = span_len[static_cast<size_t>(b) * S + j];
    if (static_cast<long long>(n) * d > kLdsWork) continue;
    const int st = span_start[static_cast<size_t>(b) * S + j];
    const ST* X = (kv ? V : K) + (static_cast<size_t>(u) * T + st) * d;
    const int tp = tok_pad[static_cast<size_t>(b) * (S + 1) + j];
    auto x = [&](int t, int c) -> double {
      return static_cast<double>(E::ld(X, static_cast<size_t>(t) * d + c));
    };
    auto a_out = [&](int t, int k, double val) {
      if (kv)
        a_v[static_cast<size_t>(u) * Np * rank + avt_off(tp + t, k, rank)] = E::from_f64(val);
      else
        a_k[(static_cast<size_t>(u) * Np + tp + t) * rank + k] = E::from_f64(val);
    };
    auto w_out = [&](int k, int e, double val) {
      if (kv)
        w_v[static_cast<size_t>(u) * S * d * rank4(rank) + wvt_off(j, k, e, d, rank)] =
            E::from_f64(val);
      else
        w_k[((static_cast<size_t>(u) * S + j) * rank + k) * d + e] = E::from_f64(val);
    };
    factor_matrix(x, n, d, rank, work, sh, a_out, w_out);
  }
}

// Streaming segmentation (SEKV, Metodologia 1 and 2 applied to decoded
// tokens): a sequence whose new token is an anchor (surprisal above the
// threshold) closes the non-empty full-resolution run after its previous
// anchor into span j = n_spans[b], with the build's summary, value mean,
// ln|S| and factors, computed from the stored rows.  One workgroup per
// (unit, K or V) item; the K item also writes the summary, the V item the
// value mean, and the K item of KV head 0 the span tables.  Each item then
// zeroes its unit's rows of the run, which leave the full-resolution set
// (the append kernel, next in stream order, updates counts and positions).
//
// A closing sits on the decode loop's critical path, so this kernel is built
// for latency: one wave per SIMD (a Jacobi round costs the dependency depth
// of its fp64 arithmetic, not parallelism), the run's rows X (n x d) read
// once from the tiled store with 16-byte lane loads, and an LDS-resident
// fp64 Gram matrix:
//   rows form, G = X X^T = U S^2 U^T (n x n), when X fits in LDS beside it:
//     the rotated rows are sigma_i^2 u_i^T, so A = U_r S_r and
//     W = S_r^-1 U_r^T X;
//   cols form, G = X^T X = W S^2 W^T (d x d), otherwise (X streamed in
//     32-row blocks): the rotated rows are sigma_i^2 w_i^T, so W = W_r^T
//     and A = X W_r.
// Squaring the singular values costs accuracy only in the small ones, far
// below the storage rounding for the leading r.
constexpr int kCloseThreads = 256;
constexpr int kCloseWaves = kCloseThreads / kWave;
constexpr int kCloseWork = 128 * 132;  // doubles: G with its padded pitch (+ X)
constexpr int kBlock = 32;             // rows of X per streamed block

// 8 consecutive stored elements (16-byte aligned) as floats.
template <int DT>
__device__ __forceinline__ void load8(const typename Elem<DT>::T* p, float (&v)[8]) {
  if constexpr (DT == kBF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Visits the lane vectors of a unit's tiled full-resolution store (K16 for
// keys, V32 for values) that hold rows [lo, hi): f(p, row[8], col[8]) gets
// the vector's address and the row and column of each of its 8 elements
// (row -1: outside [lo, hi)).  Vectors are dealt to the block's waves.
template <class Fn>
__device__ __forceinline__ void for_row_vectors(bool vtile, int lo, int hi, int d, const Fn& f) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  if (!vtile) {  // K16: 16 rows x 32 columns per block; a lane holds 8 columns of one row
    const int ncb = d >> 5, tb0 = lo >> 4, nt = ((hi - 1) >> 4) - tb0 + 1;
    for (int blk = wave; blk < nt * ncb; blk += kCloseWaves) {
      const int tile = tb0 + blk / ncb, kk = blk % ncb;
      const int row = tile * 16 + (lane & 15);
      int rr[8], cc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        rr[e] = row >= lo && row < hi ? row : -1;
        cc[e] = kk * 32 + (lane >> 4) * 8 + e;
      }
      f(static_cast<size_t>(tile * ncb + kk) * 512 + lane * 8, rr, cc);
    }
  } else {  // V32: 32 rows x 16 columns per block; a lane holds 8 rows of one column
    const int ncb = d >> 4, tb0 = lo >> 5, nt = ((hi - 1) >> 5) - tb0 + 1;
    for (int blk = wave; blk < nt * ncb; blk += kCloseWaves) {
      const int tile = tb0 + blk / ncb, cb = blk % ncb;
      const int g = lane >> 4;
      int rr[8], cc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = tile * 32 + v32_row(g, e);
        rr[e] = row >= lo && row < hi ? row : -1;
        cc[e] = cb * 16 + (lane & 15);
      }
      f(static_cast<size_t>(tile * ncb + cb) * 512 + lane * 8, rr, cc);
    }
  }
}


// ---- top eigenpairs of the Gram matrix (closing path)
//
// The closing needs only the r_j largest eigenpairs of the m x m Gram
// matrix G.  G is reduced to a symmetric tridiagonal T = Q^T G Q by m - 2
// Householder reflectors (two barriers each); the r_j + 1 largest
// eigenvalues of T come from Sturm counts by multisection (a group of
// lanes per eigenvalue, no barriers); the eigenvectors of T from twisted
// factorisations T - lambda I = N_t D_t N_t^T (one lane per eigenvalue,
// three O(m) passes), which are accurate while each eigenvalue is
// separated from its neighbours; Q's reflectors map them back to
// eigenvectors of G.  When two of the r_j + 1 largest eigenvalues lie
// within kClusterGap of the largest (the truncation or the basis inside
// the cluster is then ill-determined for this method), the closing takes
// the Jacobi path instead.
constexpr int kMaxEig = 33;          // r_j <= 32 eigenpairs and the first one left out
constexpr double kClusterGap = 1e-7; // relative to the largest eigenvalue
constexpr double kSignificant = 1e-9;
constexpr double kPivot = 1e-150;    // smallest pivot magnitude of the scaled T

struct EigShared {
  double d[128];    // diagonal of T (scaled after the reduction)
  double e[128];    // e[k] = T[k][k+1]
  double tau[128];  // reflector k: I - tau_k v v^T
  double vb[2][128];  // the current and next reflector vector, 0 outside k + 1 .. m - 1
  double p[128];    // tau_k G v of the current step, 0 outside the trailing block
  double red[2][kCloseWaves];
  double lam[kMaxEig];  // eigenvalues of the scaled T, largest first
  double zn[16];        // the two halves of ||z||^2 of a batch's tridiagonal eigenvectors
  int tw[8];            // their twist indices
  double lim[3];        // Gershgorin interval of the scaled T, and the scale
};

// Sums over aligned groups of V lanes (V a power of two <= 16) by DPP
// (quad xor 1, quad xor 2, half-row mirror, row mirror: each step adds the
// other half of the current block, so every lane ends with the sum).
template <int V>
__device__ __forceinline__ double group_sum_dpp(double a) {
  if constexpr (V >= 2) a += dpp_f64<0xb1>(a);
  if constexpr (V >= 4) a += dpp_f64<0x4e>(a);
  if constexpr (V >= 8) a += dpp_f64<0x141>(a);
  if constexpr (V >= 16) a += dpp_f64<0x140>(a);
  return a;
}

// N such sums, step by step across the N values: the chains are
// independent, so their DPP latencies overlap (one sum after another would
// wait out each chain in turn).
template <int V, int N>
__device__ __forceinline__ void group_sums_dpp(double (&a)[N]) {
  auto step = [&](auto ctrl) {
    double t[N];
#pragma unroll
    for (int q = 0; q < N; ++q) t[q] = dpp_f64<decltype(ctrl)::value>(a[q]);
#pragma unroll
    for (int q = 0; q < N; ++q) a[q] += t[q];
  };
  if constexpr (V >= 2) step(std::integral_constant<int, 0xb1>{});
  if constexpr (V >= 4) step(std::integral_constant<int, 0x4e>{});
  if constexpr (V >= 8) step(std::integral_constant<int, 0x141>{});
  if constexpr (V >= 16) step(std::integral_constant<int, 0x140>{});
}

// Sum over a wave by DPP within rows of 16 lanes and lane reads across
// them (no LDS traffic); the result is uniform.
__device__ __forceinline__ double wave_sum_dpp(double a) {
  a = group_sum_dpp<16>(a);
  auto rl = [&](int l) {
    const long long v = __double_as_longlong(a);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(v), l);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), l);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
  };
  return (rl(0) + rl(16)) + (rl(32) + rl(48));
}

// Householder reduction of the symmetric m x m matrix A (m <= 128, both
// triangles stored in LDS with pitch P) to tridiagonal form: reflector k,
// H_k = I - tau_k v v^T with v_{k+1} = 1, zeroes row and column k beyond
// the first off-diagonal entry.  The matrix lives in registers: the lanes
// form groups of L (group g = tid / L, lane h = tid % L), and lane h of
// group g holds rows g + (T / L) r (r < R) at columns h + L c (c < C), so
// that one LDS read of v_j or p_j serves R rows.  Once row k + 1 is final
// its lanes copy it to LDS, and one wave forms reflector k + 1 from the
// copy (two entries per lane, one wave sum for the norm): v scaled, zero
// outside k + 2 .. m - 1, goes to vb (double buffered) and back into row
// k + 1 of A (kept for the back-transform, with zeros left of v_{k+2}).
// Each step is then
//   p = tau A v (one multiply-add per entry, a DPP sum per row; p = 0 on
//   the rows outside the trailing block), barrier,
//   A -= v w^T + w v^T with w = p - (tau/2)(p.v) v, written as
//   a_ij -= v_i p_j + (p_i - tau (p.v) v_i) v_j (two multiply-adds per
//   entry; v and p vanish outside the trailing block, so no entry needs a
//   branch), the next reflector, barrier.
// Column blocks and row slots left of / above the trailing block are
// skipped.  d, e receive T; tau the reflectors.  Ends with a barrier.
// A loaded value marked as used unconditionally (an empty asm statement
// that takes and returns it in a register): a load whose result is then
// selected against a constant stays one unconditional load, issued with
// its neighbours, instead of becoming a branch around a load that waits
// on its own.
__device__ __forceinline__ double keep(double x) {
  asm volatile("" : "+v"(x));
  return x;
}

typedef __attribute__((address_space(3))) double lds_f64;
typedef __attribute__((address_space(3))) EigShared lds_eig;
typedef __attribute__((address_space(3))) float lds_f32;
typedef double f64x4 __attribute__((ext_vector_type(4)));

// G[a][b] (a, b < m <= 128, pitch P) = sum over q of Y(q, a) Y(q, b), in
// fp64 on 16 x 16 x 4 matrix-core products.  The 16 x 16 tiles (ta, tb) of
// G with ta <= tb are dealt to the four waves in turn (at most kT each; G
// is symmetric, a tile off the diagonal is stored twice), and a wave
// advances all of its tiles through the rows q of Y four at a time.  A wave
// always runs kT tiles, so that the loads of all of them are issued
// together; the ones past the last tile repeat tile (0, 0) and are not
// stored.  Operands of lane l for rows q0 .. q0 + 3: A[i][k] = Y(q0 + l /
// 16, 16 ta + l % 16) and B[k][j] = Y(q0 + l / 16, 16 tb + l % 16); lane l
// holds D[l / 16 + 4 e][l % 16] of the product.  kByRow: Y(q, i) = y[i ys
// + q] (X rows: G = X X^T); otherwise Y(q, i) = y[q ys + i] (G = X^T X).
// Rows q >= len read 0; indices a >= m read what the buffer holds there
// (row a of an operand reaches only row a or column a of its tile, and
// those entries are not stored).
template <int kT>
struct GramTiles {
  f64x4 acc[kT];
  int ta[kT], tb[kT];
  int nt, ntiles, wv;

  __device__ __forceinline__ void init(int m) {
    nt = (m + 15) / 16;
    ntiles = nt * (nt + 1) / 2;
    wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      int r = wv + 4 * i, a = 0;  // upper-triangle tile r, row by row
      if (r >= ntiles) r = 0;
      while (a < nt && r >= nt - a) {
        r -= nt - a;
        ++a;
      }
      ta[i] = a;
      tb[i] = a + r;
    }
  }

  // partial sums of earlier blocks (upper tiles as store() left them), or 0
  __device__ __forceinline__ void load(bool zero, int m, const lds_f64* G, int P) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      const int b = 16 * tb[i] + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 16 * ta[i] + (lane >> 4) + 4 * e;
        acc[i][e] = zero || a >= m || b >= m ? 0.0 : G[a * P + b];
      }
    }
  }

  template <bool kByRow>
  __device__ __forceinline__ void accumulate(const lds_f32* y, int ys, int m, int len) {
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 15, lk = lane >> 4;
    for (int q0 = 0; q0 < len; q0 += 4) {
      const int q = q0 + lk;
      const int qc = min(q, len - 1);
      double xa[kT], xb[kT];
#pragma unroll
      for (int i = 0; i < kT; ++i) {
        const int a = 16 * ta[i] + li, b = 16 * tb[i] + li;  // < 128
        const float fa = kByRow ? y[a * ys + q] : y[qc * ys + a];
        const float fb = kByRow ? y[b * ys + q] : y[qc * ys + b];
        // rows a, b >= m need no mask: row a of the operand only reaches row a
        // of the tile, and tile entries past m - 1 are never stored; the K
        // tail past len does reach every entry and is masked
        const bool ok = kByRow || q < len;
        xa[i] = ok ? static_cast<double>(fa) : 0.0;
        xb[i] = ok ? static_cast<double>(fb) : 0.0;
      }
#pragma unroll
      for (int i = 0; i < kT; ++i)
        acc[i] = __builtin_amdgcn_mfma_f64_16x16x4f64(xa[i], xb[i], acc[i], 0, 0, 0);
      // all operand reads of the step, then their conversions, then the
      // products: the reads are in flight together (one LDS latency per
      // step, overlapping the previous step's products) instead of each
      // product waiting for its own two reads
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kT, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2 * kT, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, kT, 0);
    }
  }

  // upper tiles; with both, the mirror images of the tiles off the diagonal
  __device__ __forceinline__ void store(bool both, int m, lds_f64* G, int P) const {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      if (wv + 4 * i >= ntiles) break;
      const int b = 16 * tb[i] + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 16 * ta[i] + (lane >> 4) + 4 * e;
        if (a < m && b < m) {
          G[a * P + b] = acc[i][e];
          if (both && ta[i] != tb[i]) G[b * P + a] = acc[i][e];
        }
      }
    }
  }
};

// One block of rows of Y into G (GramTiles): `first` starts from zero,
// otherwise from the upper tiles that the previous block stored; `last`
// stores both triangles.  By rows, Y is X at the place of G, so the waves
// meet at a barrier between the last read of X and the first store.  A
// call of its own (its registers are not shared with the caller's).
template <int kT, bool kByRow>
__device__ __noinline__ void gram_block(const float* y_, int ys_, int m_, int len_, double* G_,
                                        int P_, int first_, int last_) {
  const int ys = __builtin_amdgcn_readfirstlane(ys_);
  const int m = __builtin_amdgcn_readfirstlane(m_);
  const int len = __builtin_amdgcn_readfirstlane(len_);
  const int P = __builtin_amdgcn_readfirstlane(P_);
  const bool first = __builtin_amdgcn_readfirstlane(first_) != 0;
  const bool last = __builtin_amdgcn_readfirstlane(last_) != 0;
  lds_f64* G = (lds_f64*)G_;
  GramTiles<kT> gt;
  gt.init(m);
  gt.load(first, m, G, P);
  gt.template accumulate<kByRow>((const lds_f32*)y_, ys, m, len);
  if (kByRow) __syncthreads();
  gt.store(last, m, G, P);
}

// G = X X^T of a run's rows held in LDS (Y(q, i) = y[i ys + q], q < len, a
// multiple of 4), in one pass, with the tiles dealt so that each wave reads
// few row blocks per K step: the 16-row blocks [0, 2H) cover m, waves 0 and
// 1 take the upper triangles of blocks [0, H) and [H, 2H), waves 2 and 3
// the two halves (by rows) of the rectangle [0, H) x [H, 2H).  A wave loads
// each of its row blocks once per K step and reuses it for every tile
// that has it (the dealing of gram_block reads two blocks per tile).
// Operand and output lane layouts as in GramTiles.  Tiles of rows >= m are
// computed and not stored.  A call of its own; X may share its LDS with
// G: every read of X comes before the barrier, every store after it.
template <int NR, int NC, bool kTri>
__device__ __forceinline__ void gram_rows_tiles(const lds_f32* y, int ys, int m, int len,
                                                lds_f64* G, int P, int r0, int c0) {
  constexpr int kTiles = kTri ? NR * (NR + 1) / 2 : NR * NC;
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & 15, lk = lane >> 4;
  f64x4 acc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) acc[t] = f64x4{0.0, 0.0, 0.0, 0.0};
  const lds_f32* yr = y + (16 * r0 + li) * ys + lk;
  const lds_f32* yc = y + (16 * c0 + li) * ys + lk;
#pragma unroll 2
  for (int q0 = 0; q0 < len; q0 += 4) {
    double xr[NR], xc[kTri ? 1 : NC];
#pragma unroll
    for (int i = 0; i < NR; ++i) xr[i] = static_cast<double>(yr[16 * i * ys + q0]);
    if constexpr (!kTri) {
#pragma unroll
      for (int j = 0; j < NC; ++j) xc[j] = static_cast<double>(yc[16 * j * ys + q0]);
    }
    int t = 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
#pragma unroll
      for (int j = kTri ? i : 0; j < (kTri ? NR : NC); ++j, ++t)
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(xr[i], kTri ? xr[j] : xc[kTri ? 0 : j],
                                                      acc[t], 0, 0, 0);
    }
  }
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
#pragma unroll
    for (int j = kTri ? i : 0; j < (kTri ? NR : NC); ++j, ++t) {
      const int ta = r0 + i, tb = (kTri ? r0 : c0) + j;
      const int b = 16 * tb + li;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int a = 16 * ta + lk + 4 * e;
        if (a < m && b < m) {
          G[a * P + b] = acc[t][e];
          if (ta != tb) G[b * P + a] = acc[t][e];
        }
      }
    }
  }
}

template <int H>
__device__ __noinline__ void gram_rows(const float* y_, int ys_, int m_, int len_, double* G_,
                                       int P_) {
  const int ys = __builtin_amdgcn_readfirstlane(ys_);
  const int m = __builtin_amdgcn_readfirstlane(m_);
  const int len = __builtin_amdgcn_readfirstlane(len_);
  const int P = __builtin_amdgcn_readfirstlane(P_);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const lds_f32* y = (const lds_f32*)y_;
  lds_f64* G = (lds_f64*)G_;
  constexpr int kRa = (H + 1) / 2;  // rectangle rows of wave 2; wave 3 takes H - kRa
  if (wv < 2) {
    gram_rows_tiles<H, H, true>(y, ys, m, len, G, P, wv * H, wv * H);
  } else if (wv == 2) {
    gram_rows_tiles<kRa, H, false>(y, ys, m, len, G, P, 0, H);
  } else if constexpr (H - kRa > 0) {
    gram_rows_tiles<H - kRa, H, false>(y, ys, m, len, G, P, kRa, H);
  } else {
    __syncthreads();  // no tiles: only the barrier the others wait at
  }
}

// S[k][e] = sum over t < n of X[t][e] R[k][t] (k < rj <= 32, e < d, d a
// multiple of 16; X: n rows of floats with pitch xp, R: rows of doubles
// with pitch P, S: pitch d), in fp64 on 16 x 16 x 4 matrix-core products:
// the output tiles (16 rows k, 16 columns e), at most 2 x 8, are dealt to
// the waves in turn (tiles wv + 4 i), each advanced over the rows t four at
// a time (16 rows per pass); A[k][t] = R[k][t] and B[t][e] = X[t][e], with rows t >= n and k >=
// rj read as 0.  Lane layouts as in GramTiles.  A call of its own; ends
// with a barrier.
__device__ __noinline__ void rows_product(const float* x_, int xp_, int n_, int d_, int rj_,
                                          const double* r_, int P_, double* s_) {
  const int xp = __builtin_amdgcn_readfirstlane(xp_);
  const int n = __builtin_amdgcn_readfirstlane(n_);
  const int d = __builtin_amdgcn_readfirstlane(d_);
  const int rj = __builtin_amdgcn_readfirstlane(rj_);
  const int P = __builtin_amdgcn_readfirstlane(P_);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const lds_f32* x = (const lds_f32*)x_;
  const lds_f64* r = (const lds_f64*)r_;
  lds_f64* s = (lds_f64*)s_;
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & 15, lk = lane >> 4;
  const int net = d / 16;
  const int ntile = (rj + 15) / 16 * net;  // <= 16
  f64x4 acc[4];
  int tk[4], te[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tile = wv + 4 * i;
    tk[i] = tile / net;
    te[i] = tile - tk[i] * net;
    acc[i] = f64x4{0.0, 0.0, 0.0, 0.0};
  }
  // four K steps per pass: their operand reads are issued together
  for (int t0 = 0; t0 < n; t0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (wv + 4 * i >= ntile) break;  // uniform
      const int k = 16 * tk[i] + li;
      const int kc = min(k, rj - 1);
      double a[4], b[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        // reads at clamped indices (no branch around them), masked after
        const int t = t0 + 4 * st + lk;
        const int tc = min(t, n - 1);
        const double ra = r[kc * P + tc];
        const double xb = static_cast<double>(x[tc * xp + 16 * te[i] + li]);
        a[st] = t < n && k < rj ? ra : 0.0;
        b[st] = t < n ? xb : 0.0;
      }
#pragma unroll
      for (int st = 0; st < 4; ++st)
        acc[i] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[st], b[st], acc[i], 0, 0, 0);
      // the eight reads first, then the conversions and masks, then the
      // products (one LDS latency per pass instead of one per K step)
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (wv + 4 * i >= ntile) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = 16 * tk[i] + lk + 4 * q;
      if (k < rj) s[k * d + 16 * te[i] + li] = acc[i][q];
    }
  }
  __syncthreads();
}

template <int L, int R, int C, bool kScalarLoop>
__device__ __noinline__ void tridiagonalize(double* A_, int m_, int P_, EigShared& es_) {
  // arguments of a call arrive in vector registers; kScalarLoop makes them
  // wave-uniform, so that the step loop and its block tests run on scalar
  // registers
  const int m = kScalarLoop ? __builtin_amdgcn_readfirstlane(m_) : m_;
  const int P = kScalarLoop ? __builtin_amdgcn_readfirstlane(P_) : P_;
  constexpr int kGroups = kCloseThreads / L;  // row groups of L lanes
  constexpr int kGw = kWave / L;              // row groups per wave
  constexpr int kBlk = kScalarLoop ? (C < 4 ? C : 4) : (C < 8 ? C : 8);
  static_assert(kGroups * R <= 128 && L * C <= 128 && kGroups * R >= L * C, "tile");
  lds_f64* A = (lds_f64*)A_;
  lds_eig* es = (lds_eig*)&es_;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int g = tid / L;
  const int h = tid - g * L;
  // whole rows of 128 entries are read: i, j < 128 and P <= 130 keep every
  // address inside the LDS work array; entries past m are replaced by 0
  double a[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) a[r][c] = A[(g + kGroups * r) * P + h + L * c];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const double kx = keep(a[r][c]);
      a[r][c] = g + kGroups * r < m && h + L * c < m ? kx : 0.0;
    }
  if (tid < 128) es->p[tid] = 0.0;
  // reflector r (r <= m - 3) from row r of A in LDS, by the 64 lanes of
  // one wave (two entries each): v scaled to v_{r+1} = 1 into vb and back
  // into row r (kept for the back-transform), d_r, e_r = beta, tau_r
  auto reflector = [&](int r) {
    lds_f64* row = A + r * P;
    double xa = row[lane], xb = row[lane + kWave];
    const double al = row[r + 1];
    const double dr = row[r];
    xa = keep(xa);
    xb = keep(xb);
    const bool ia = lane > r + 1 && lane < m, ib = lane + kWave > r + 1 && lane + kWave < m;
    const double ya = ia ? xa : 0.0, yb = ib ? xb : 0.0;
    const double q = wave_sum_dpp(fma(ya, ya, yb * yb));
    double tau = 0.0, scl = 0.0, beta = al;
    if (q > 0.0) {
      const double s2 = fma(al, al, q);
      beta = -copysign(s2 * rsqrt_nr(s2), al);
      const double ib_ = recip(beta);
      tau = (beta - al) * ib_;
      scl = recip(al - beta);
    }
    lds_f64* vb = es->vb[r & 1];
    const double va = lane == r + 1 ? 1.0 : ya * scl;
    const double vc = lane + kWave == r + 1 ? 1.0 : yb * scl;
    vb[lane] = va;
    vb[lane + kWave] = vc;
    // row r keeps v for the back-transform, with zeros left of v_{r+1}
    // (entries past m - 1 stay as they are: no write leaves the row)
    if (lane < m) row[lane] = va;
    if (lane + kWave < m) row[lane + kWave] = vc;
    if (lane == 0) {
      es->d[r] = dr;
      es->e[r] = beta;
      es->tau[r] = tau;
    }
  };
  if (m >= 3 && tid < kWave) reflector(0);
  __syncthreads();
  for (int k = 0; k + 2 < m; ++k) {
    const double tau = es->tau[k];
    const bool refl =
        kScalarLoop ? __builtin_amdgcn_readfirstlane(tau != 0.0 ? 1 : 0) != 0 : tau != 0.0;
    const lds_f64* vb = es->vb[k & 1];
    // slot r of this wave holds rows kGroups r + kGw wv + [0, kGw): live
    // while one of them lies in the trailing block k + 1 .. m - 1; column
    // block b (lane h's columns h + L c, c in [kBlk b, kBlk b + kBlk)) is
    // live while one of its columns does
    auto slot_live = [&](int r) {
      const int lo = kGroups * r + kGw * wv;
      return lo + kGw - 1 > k && lo < m;
    };
    auto blk_live = [&](int b) { return (L - 1) + L * (kBlk * b + kBlk - 1) > k; };
    double pi[R], vi[R];
    double xv[C];  // v_j of this lane's columns (live blocks only)
    double pvl = 0.0;
    if (refl) {
      double part[R];
#pragma unroll
      for (int r = 0; r < R; ++r) part[r] = 0.0;
#pragma unroll
      for (int b = 0; b < C / kBlk; ++b) {
        if (!blk_live(b)) continue;
#pragma unroll
        for (int u = 0; u < kBlk; ++u) xv[kBlk * b + u] = vb[h + L * (kBlk * b + u)];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (!slot_live(r)) continue;
#pragma unroll
        for (int b = 0; b < C / kBlk; ++b) {
          if (!blk_live(b)) continue;
#pragma unroll
          for (int u = 0; u < kBlk; ++u)
            part[r] = fma(a[r][kBlk * b + u], xv[kBlk * b + u], part[r]);
        }
      }
      group_sums_dpp<L>(part);  // rows outside the trailing block sum zeros
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = g + kGroups * r;
        const bool act = i > k && i < m;
        const double v = vb[i];
        pi[r] = act ? tau * part[r] : 0.0;
        vi[r] = act ? v : 0.0;
        pvl = fma(pi[r], vi[r], pvl);
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) pi[r] = vi[r] = 0.0;
    }
    if (h == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) es->p[g + kGroups * r] = pi[r];
    }
    const double pv = wave_sum_dpp(h == 0 ? pvl : 0.0);
    if (lane == 0) es->red[1][wv] = pv;
    __syncthreads();
    if (refl) {
      const double tpv = tau * ((es->red[1][0] + es->red[1][1]) + (es->red[1][2] + es->red[1][3]));
      double ci[R];
#pragma unroll
      for (int r = 0; r < R; ++r) ci[r] = pi[r] - tpv * vi[r];  // w_i - (tau/2)(p.v) v_i
#pragma unroll
      for (int b = 0; b < C / kBlk; ++b) {
        if (!blk_live(b)) continue;
        double pj[kBlk];
#pragma unroll
        for (int u = 0; u < kBlk; ++u) pj[u] = es->p[h + L * (kBlk * b + u)];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (!slot_live(r)) continue;
#pragma unroll
          for (int u = 0; u < kBlk; ++u) {
            const double x = fma(-vi[r], pj[u], a[r][kBlk * b + u]);
            a[r][kBlk * b + u] = fma(-ci[r], xv[kBlk * b + u], x);
          }
        }
      }
    }
    if (k + 3 < m) {
      // row k + 1 is final: to LDS as whole rows of L C entries (what
      // spills past column m - 1 lands on later rows' LDS copies, which are
      // not read before their own rows overwrite them), then the next
      // reflector from it
      const int g1 = (k + 1) % kGroups;
      const int r1 = (k + 1) / kGroups;
      if (g == g1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r != r1) continue;
#pragma unroll
          for (int b = 0; b < C / kBlk; ++b) {
            if (!blk_live(b)) continue;
#pragma unroll
            for (int u = 0; u < kBlk; ++u)
              A[(k + 1) * P + h + L * (kBlk * b + u)] = a[r][kBlk * b + u];
          }
        }
      }
      if (wv == g1 / kGw) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        reflector(k + 1);
      }
    } else {  // last step: the trailing 2 x 2 block
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int i = g + kGroups * r;
          const int j = h + L * c;
          if (i == m - 2 && j == m - 2) es->d[m - 2] = a[r][c];
          if (i == m - 2 && j == m - 1) es->e[m - 2] = a[r][c];
          if (i == m - 1 && j == m - 1) es->d[m - 1] = a[r][c];
        }
    }
    __syncthreads();
  }
  if (m <= 2) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int i = g + kGroups * r;
        const int j = h + L * c;
        if (i < m && j == i) es->d[i] = a[r][c];
        if (i == 0 && j == 1 && m == 2) es->e[0] = a[r][c];
      }
    __syncthreads();
  }
}

// Rescales two consecutive terms of a three-term recurrence by the same
// power of two (their ratio is kept) so that they stay near 1.
__device__ __forceinline__ void rescale2(double& a, double& b) {
  const int ex = __builtin_amdgcn_frexp_exp(fabs(a) + fabs(b));
  a = __builtin_amdgcn_ldexp(a, -ex);
  b = __builtin_amdgcn_ldexp(b, -ex);
}

// Number of eigenvalues of the tridiagonal T below x: the sign changes
// along the leading principal minors det(T_i - x I), i = 0..m (Sturm),
// from their three-term recurrence (de[i] = (d_i, e_{i-1}^2)); a zero minor
// counts as positive (the next minor then has the sign opposite to the one
// before, so the count is unchanged).  Also the Newton step -f(x) / f'(x)
// for f(x) = det(T - x I): the derivatives of the minors follow p'_i =
// (d_i - x) p'_{i-1} - p_{i-1} - e_{i-1}^2 p'_{i-2}.  Every 4 steps the
// last two minors and derivatives are rescaled by one power of two.
__device__ __forceinline__ int sturm_newton(const double2* __restrict__ de, int m, double x,
                                            double& step) {
  double p0 = 1.0, p1 = de[0].x - x, q0 = 0.0, q1 = -1.0;
  int cnt = p1 < 0.0;
  auto one = [&](const double2 qq) {
    const double a = qq.x - x;
    const double p2 = fma(a, p1, -qq.y * p0);
    const double q2 = fma(a, q1, -fma(qq.y, q0, p1));
    cnt += (p2 < 0.0) != (p1 < 0.0);
    p0 = p1;
    p1 = p2;
    q0 = q1;
    q1 = q2;
  };
  int i = 1;
  // de is padded to 128 + 4 entries: the block loaded ahead stays in bounds
  double2 qn[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) qn[u] = de[1 + u];
  for (; i + 4 <= m; i += 4) {
    double2 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      q[u] = qn[u];
      qn[u] = de[i + 4 + u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) one(q[u]);
    const int ex =
        __builtin_amdgcn_frexp_exp((fabs(p0) + fabs(p1)) + (fabs(q0) + fabs(q1)));
    p0 = __builtin_amdgcn_ldexp(p0, -ex);
    p1 = __builtin_amdgcn_ldexp(p1, -ex);
    q0 = __builtin_amdgcn_ldexp(q0, -ex);
    q1 = __builtin_amdgcn_ldexp(q1, -ex);
  }
  for (; i < m; ++i) one(de[i]);
  step = q1 != 0.0 ? -p1 / q1 : 0.0;
  return cnt;
}

// Minimum and maximum over aligned groups of g lanes (g a power of two).
template <class T>
__device__ __forceinline__ void group_min_max(T& mn, T& mx, int g) {
  for (int o = 1; o < g; o <<= 1) {
    mn = min(mn, __shfl_xor(mn, o, kWave));
    mx = max(mx, __shfl_xor(mx, o, kWave));
  }
}

// The nev largest eigenvalues of T (es.d, es.e; m) into es.lam, largest
// first, for T scaled by a power of two to entries of magnitude <= 1
// (es.d and es.e are scaled in place, the scale goes to es.lim[2], and
// de receives (d_i, e_{i-1}^2)).  A group of g lanes per eigenvalue
// evaluates Sturm counts at g - 1 points spread evenly over its bracket and
// at a Newton iterate, and keeps the smallest bracket the counts certify;
// once the bracket holds this eigenvalue alone and the Newton step is at
// rounding level the iterate is the eigenvalue, else the bracket narrows to
// a few ulps.  Ends with a barrier.
__device__ __forceinline__ void top_eigenvalues(int m, int nev, EigShared& es, double2* de) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  if (tid < kWave) {
    double mx = 0.0;
    for (int i = lane; i < m; i += kWave) {
      mx = fmax(mx, fabs(es.d[i]));
      if (i + 1 < m) mx = fmax(mx, fabs(es.e[i]));
    }
    mx = wave_max(mx);
    const double sc =
        mx > 0.0 ? __builtin_amdgcn_ldexp(1.0, -__builtin_amdgcn_frexp_exp(mx)) : 1.0;
    double lo = 1e300, hi = -1e300;
    for (int i = lane; i < m; i += kWave) {
      const double di = es.d[i] * sc;
      const double el = i > 0 ? es.e[i - 1] * sc : 0.0;
      const double er = i + 1 < m ? es.e[i] * sc : 0.0;
      lo = fmin(lo, di - fabs(el) - fabs(er));
      hi = fmax(hi, di + fabs(el) + fabs(er));
      de[i] = make_double2(di, el * el);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int i = lane; i < m; i += kWave) {
      es.d[i] *= sc;
      if (i + 1 < m) es.e[i] *= sc;
    }
    wave_min_max_f64(lo, hi);
    if (lane == 0) {
      es.lim[0] = lo;
      es.lim[1] = hi;
      es.lim[2] = sc;
    }
  }
  __syncthreads();
  constexpr double kEps = 2.220446049250313e-16;
  double lo0 = es.lim[0], hi0 = es.lim[1];
  {
    const double pad = 4.0 * kEps * fmax(fabs(lo0), fabs(hi0)) + 4.0 * kEps;
    lo0 -= pad;
    hi0 += pad;
  }
  // one round with every lane first: the counts at 256 evenly spaced
  // points x_c = lo0 + (c + 1) w0 (x_255 = hi0) bracket every eigenvalue to
  // a 256th of the interval (es.p is free once T is formed)
  const double w0 = (hi0 - lo0) / static_cast<double>(kCloseThreads);
  static_assert(sizeof(es.p) >= kCloseThreads * sizeof(int), "one count per lane");
  int* cnt0 = reinterpret_cast<int*>(es.p);
  {
    double step;
    const double x = tid == kCloseThreads - 1 ? hi0 : fma(w0, static_cast<double>(tid + 1), lo0);
    cnt0[tid] = sturm_newton(de, m, x, step);
  }
  __syncthreads();
  int g = kWave;
  while (g > 1 && g * nev > kCloseThreads) g >>= 1;
  const int kk = tid / g;
  const int l = tid - kk * g;
  if (kk < nev) {
    const int idx = m - 1 - kk;  // ascending index of the kk-th largest
    // the first point whose count exceeds idx (x_255 = hi0 counts all m):
    // the bracket (x_{jp-1}, x_jp] holds eigenvalue idx with its counts
    // certifying it, whether or not the rounded counts grow monotonically
    int jp = kCloseThreads - 1;
    for (int c = l; c < kCloseThreads; c += g)
      if (cnt0[c] > idx) jp = min(jp, c);
    for (int o = 1; o < g; o <<= 1) jp = min(jp, __shfl_xor(jp, o, kWave));
    double lo = jp == 0 ? lo0 : fma(w0, static_cast<double>(jp), lo0);
    double hi = jp == kCloseThreads - 1 ? hi0 : fma(w0, static_cast<double>(jp + 1), lo0);
    int clo = jp == 0 ? 0 : cnt0[jp - 1];  // eigenvalues below lo and below hi
    int chi = cnt0[jp];
    double xn = 0.5 * (lo + hi), lam = xn;
    const int base = lane & ~(g - 1);
    bool done = false;
    for (int it = 0; it < 64 && !done; ++it) {
      if (hi - lo <= 2.0 * kEps * fmax(fabs(lo), fabs(hi)) + 2.0 * kEps) break;
      // g - 1 points spread evenly over (lo, hi), and the Newton iterate
      const double w = (hi - lo) / static_cast<double>(g);
      const double x = l < g - 1 ? fma(w, static_cast<double>(l + 1), lo) : xn;
      double step;
      const int cnt = sturm_newton(de, m, x, step);
      const bool above = cnt > idx;
      // bracket from the even points (the first one above idx, by ballot),
      // with the counts there
      const unsigned long long bal = __ballot(above && l < g - 1);
      const unsigned long long gm = g == kWave ? bal : (bal >> base) & ((1ull << g) - 1ull);
      const int sa = gm ? __builtin_ctzll(gm) : g - 1;  // even points 0 .. g - 2
      const int c_hi = __shfl(cnt, base + min(sa, g - 2), kWave);
      const int c_lo = __shfl(cnt, base + max(sa - 1, 0), kWave);
      double nlo = sa == 0 ? lo : fma(w, static_cast<double>(sa), lo);
      double nhi = sa == g - 1 ? hi : fma(w, static_cast<double>(sa + 1), lo);
      int nclo = sa == 0 ? clo : c_lo;
      int nchi = sa == g - 1 ? chi : c_hi;
      // and the Newton point, when it falls inside
      const int cs = __shfl(cnt, base + g - 1, kWave);
      {
        const double xq = __shfl(x, base + g - 1, kWave);
        if (xq > nlo && xq < nhi) {
          if (cs > idx) {
            nhi = xq;
            nchi = cs;
          } else {
            nlo = xq;
            nclo = cs;
          }
        }
      }
      // the Newton point and its step, from the group's last lane
      const double xs = __shfl(x, base + g - 1, kWave);
      const double ss = __shfl(step, base + g - 1, kWave);
      const double xt = xs + ss;
      if (nchi - nclo == 1 && fabs(ss) <= 4.0 * kEps * fabs(xs) && xt >= nlo && xt <= nhi) {
        lam = xt;  // isolated, and the Newton step is at rounding level
        done = true;
      }
      if (!(nhi - nlo < hi - lo) && !done) break;  // no progress left at this width
      lo = nlo;
      hi = nhi;
      clo = nclo;
      chi = nchi;
      xn = xt > lo && xt < hi ? xt : 0.5 * (lo + hi);
    }
    if (!done) lam = 0.5 * (lo + hi);
    if (l == 0) es.lam[kk] = lam;
  }
  __syncthreads();
}

// A pivot of a factorisation of T - lam I kept away from zero and
// infinity (its sign kept).
__device__ __forceinline__ double guard_pivot(double x) {
  const double y = fabs(x) < kPivot ? (x < 0.0 ? -kPivot : kPivot) : x;
  return fmin(fmax(y, -1.0 / kPivot), 1.0 / kPivot);
}

// One (d_i, e_{i-1}^2) pair from an LDS view of the pair array.
struct Pair {
  double x, y;
};
__device__ __forceinline__ Pair pair_at(const lds_f64* de, int i) {
  return Pair{de[2 * i], de[2 * i + 1]};
}

// Eigenvectors of the scaled tridiagonal T (de[i] = (d_i, e_{i-1}^2), e)
// by twisted factorisations of T - lam I.  The top-down pivots D+_i =
// P_{i+1} / P_i and the bottom-up pivots D-_i = Q_i / Q_{i+1} are ratios of
// the leading and trailing minors; gamma_i = D+_i + D-_i - (d_i -
// lam), and at the twist t = argmin |gamma_i| the vector is z_t = 1, z_i =
// -(e_i / D+_i) z_{i+1} above t and z_i = -(e_{i-1} / D-_i) z_{i-1} below.
// The two directions of a vector run on two lanes of one wave in lockstep
// (the same instructions on different rows), each in its own column of z
// (stride 16 doubles): twisted_pivots, then twist_index by the whole wave,
// then twisted_solve, which overwrites the pivots it has used with z.

// dir 0: D+_i at row s of step s; dir 1: D-_i at row m - 1 - s, by the
// pivot recurrences D+_i = (d_i - lam) - e_{i-1}^2 / D+_{i-1} and D-_i =
// (d_i - lam) - e_i^2 / D-_{i+1} (the ratios of successive minors; a pivot
// is kept away from zero and infinity before it is divided by); fewer
// instructions per step than the minors' own recurrence with rescaling,
// and measured faster.
__device__ void twisted_pivots(const double2* de_, int m, double lam, int dir, double* z_) {
  // LDS views; de has m + 4 readable pairs.  The operands of the next two
  // steps are loaded ahead of the current one.
  const lds_f64* de = (const lds_f64*)de_;
  lds_f64* z = (lds_f64*)z_;
  // row of step s (prefetches past the last row stay inside de) and its
  // pair: d_i with e_{i-1}^2 top-down, e_i^2 bottom-up
  auto row = [&](int s) { return dir ? max(m - 1 - s, 0) : s; };
  auto ld = [&](int s) {
    const int i = row(s);
    return Pair{de[2 * i], de[2 * (i + dir) + 1]};
  };
  const int i0 = row(0);
  double D = guard_pivot(de[2 * i0] - lam);
  z[16 * i0] = D;
  Pair q1 = ld(1), q2 = ld(2);
#pragma unroll 4
  for (int s = 1; s < m; ++s) {
    const Pair q = q1;
    q1 = q2;
    q2 = ld(s + 2);
    D = guard_pivot(fma(-q.y, recip(D), q.x - lam));
    z[16 * row(s)] = D;
  }
}

// The twist of one vector, by the whole wave: argmin |gamma_i| over i < m
// with gamma_{m-1} = D+_{m-1}, the largest such index on ties.
__device__ int twist_index(const double2* de_, const double* zp_, const double* zm_, int m,
                           double lam) {
  const lds_f64* de = (const lds_f64*)de_;
  const lds_f64* zp = (const lds_f64*)zp_;
  const lds_f64* zm = (const lds_f64*)zm_;
  const int lane = threadIdx.x & (kWave - 1);
  double best = INFINITY;
  int bi = -1;
  for (int i = lane; i < m; i += kWave) {
    const double dp = zp[16 * i];
    const double gam = i == m - 1 ? fabs(dp) : fabs(dp + zm[16 * i] - (de[2 * i] - lam));
    if (gam <= best) {
      best = gam;
      bi = i;
    }
  }
  double mn = best;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) mn = fmin(mn, __shfl_xor(mn, o, kWave));
  int t = best == mn ? bi : -1;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) t = max(t, __shfl_xor(t, o, kWave));
  return t >= 0 ? t : m - 1;
}

// dir 0: z_i for i = t - 1 .. 0 over the D+ column; dir 1: i = t + 1 ..
// m - 1 over the D- column.  Returns the lane's sum of z_i^2 (dir 1 counts
// z_t = 1 as well).
__device__ double twisted_solve(const double* e_, int m, int t, int dir, double* z_) {
  const lds_f64* e = (const lds_f64*)e_;
  lds_f64* z = (lds_f64*)z_;
  const int n = dir ? m - 1 - t : t;  // steps of this lane
  auto row = [&](int s) { return dir ? t + s : t - s; };
  auto eix = [&](int s) { return max(dir ? t + s - 1 : t - s, 0); };
  double zi = 1.0, nrm = dir ? 1.0 : 0.0;
  double dn = z[16 * row(min(1, n))], en = e[eix(min(1, n))];
#pragma unroll 4
  for (int s = 1; s <= n; ++s) {
    const double dd = dn, ee = en;
    const int s1 = min(s + 1, n);
    dn = z[16 * row(s1)];
    en = e[eix(s1)];
    zi = -(ee * recip(dd)) * zi;
    z[16 * row(s)] = zi;
    nrm = fma(zi, zi, nrm);
  }
  return nrm;
}

// Eigenvectors of G for the rj largest eigenvalues in es.lam (rj <= 32):
// the twisted vectors of T (two lanes each, two vectors per wave, in
// batches of 8 held in `zs`, 16 m doubles of LDS: a column of top-down and
// one of bottom-up pivots per vector), normalised and spread over groups of
// V lanes (EV elements per lane), mapped back through the reflectors kept in A (the
// next reflector's entries are loaded while the current one is applied),
// then written as rows lambda_k u_k^T of A (pitch P) with sig[k] =
// lambda_k, top[k] = k.  Ends with a barrier.
template <int V, int EV>
__device__ __noinline__ void top_eigenvectors(double* A, int m, int P, int rj, EigShared& es,
                                 const double2* de, double* zs, FactorShared& sh) {
  const int tid = threadIdx.x;
  const int kk = tid / V;
  const int l = tid - kk * V;
  double y[EV];
#pragma unroll
  for (int c = 0; c < EV; ++c) y[c] = 0.0;
  // vector c of a batch of 8 belongs to wave c / 2: its top-down pass on
  // lane 2 (c % 2), its bottom-up pass on the next lane (columns c and
  // c + 8 of zs); the passes are serial recurrences, so each wave runs four
  // at a time
  const int wl = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int vec = 2 * wv + (wl >> 1);
  const int dir = wl & 1;
  for (int b0 = 0; b0 < rj; b0 += 8) {
    const bool piv = wl < 4 && b0 + vec < rj;
    if (piv) twisted_pivots(de, m, es.lam[b0 + vec], dir, zs + vec + 8 * dir);
    // the pivots of this wave's vectors are read by the whole wave: LDS
    // operations of a wave complete in order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int tw[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (b0 + 2 * wv + j < rj)
        tw[j] = twist_index(de, zs + 2 * wv + j, zs + 2 * wv + j + 8, m, es.lam[b0 + 2 * wv + j]);
    if (wl < 2) es.tw[2 * wv + wl] = tw[wl];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (piv)
      es.zn[2 * vec + dir] =
          twisted_solve(es.e, m, (wl >> 1) ? tw[1] : tw[0], dir, zs + vec + 8 * dir);
    __syncthreads();
    if (kk >= b0 && kk < b0 + 8 && kk < rj) {
      const int c0 = kk - b0;
      const int t = es.tw[c0];
      const double f = rsqrt_nr(es.zn[2 * c0 + 1] + es.zn[2 * c0]);
#pragma unroll
      for (int c = 0; c < EV; ++c) {
        const int i = l + V * c;
        if (i < m) {
          const double za = zs[16 * i + c0], zb = zs[16 * i + c0 + 8];
          y[c] = (i < t ? za : (i > t ? zb : 1.0)) * f;
        }
      }
    }
    __syncthreads();
  }
  // u = H_0 H_1 ... H_{m-3} z, by blocks of four reflectors (a, b, c, d) =
  // (4 j, ..., 4 j + 3), the last block first.  With alpha_i = v_i . z for
  // the current z and g_ik = v_i . v_k,
  //   H_a H_b H_c H_d z = z - f_a v_a - f_b v_b - f_c v_c - f_d v_d,
  //   f_d = tau_d alpha_d,  f_c = tau_c (alpha_c - g_cd f_d),
  //   f_b = tau_b (alpha_b - g_bc f_c - g_bd f_d),
  //   f_a = tau_a (alpha_a - g_ab f_b - g_ac f_c - g_ad f_d):
  // four group sums per block, interleaved, instead of one per reflector
  // (the loop is bound by instruction issue, one wave per SIMD, and the
  // sums are most of its instructions).  Row s of A holds reflector s
  // scaled (v_{s+1} = 1), with zeros left of v_{s+1}; reflectors past
  // m - 3 (the first block's padding) count as v = 0, tau = 0.  Reads stay
  // inside the work array for i < 128 and s < 128; entries past m - 1
  // (another row's, or never written) are replaced by 0.
  const int ms = __builtin_amdgcn_readfirstlane(m);  // uniform: scalar loop control
  const int nblk = (max(ms - 2, 0) + 3) / 4;
  // LDS views, converted once (generic pointers would make flat accesses)
  const lds_f64* const Al = (const lds_f64*)A;
  const lds_f64* const tl = (const lds_f64*)es.tau;
  lds_f64* const gk = (lds_f64*)es.vb[0];  // [block][6]: g_ab g_ac g_ad g_bc g_bd g_cd
  static_assert(sizeof(es.vb) >= 6 * 32 * sizeof(double), "products of 32 blocks");
  {
    // one block per group of 16 lanes, lane h holding entries h + 16 c
    const int grp = tid >> 4;
    const int h = tid & 15;
    for (int j0 = 0; j0 < nblk; j0 += kCloseThreads / 16) {
      const int j = min(j0 + grp, nblk - 1);
      double g6[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int i = h + 16 * c;
        if (16 * c < ms) {
          double w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            w[q] = (i < ms && 4 * j + q <= ms - 3) ? Al[(4 * j + q) * P + i] : 0.0;
          g6[0] = fma(w[0], w[1], g6[0]);
          g6[1] = fma(w[0], w[2], g6[1]);
          g6[2] = fma(w[0], w[3], g6[2]);
          g6[3] = fma(w[1], w[2], g6[3]);
          g6[4] = fma(w[1], w[3], g6[4]);
          g6[5] = fma(w[2], w[3], g6[5]);
        }
      }
      group_sums_dpp<16>(g6);
      if (h < 6 && j0 + grp < nblk) {
        double gv = g6[0];
#pragma unroll
        for (int q = 1; q < 6; ++q) gv = h == q ? g6[q] : gv;
        gk[6 * j + h] = gv;
      }
    }
  }
  __syncthreads();
  bool inm[EV];
#pragma unroll
  for (int c = 0; c < EV; ++c) inm[c] = l + V * c < ms;
  auto apply = [&](int j, auto first) {
    double v[4][EV], t[4], g[6];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int s = 4 * j + q;
      const lds_f64* rs = Al + s * P;
      if constexpr (decltype(first)::value) {
        const bool live = s <= ms - 3;
#pragma unroll
        for (int c = 0; c < EV; ++c) v[q][c] = live ? rs[l + V * c] : 0.0;
        t[q] = live ? tl[s] : 0.0;
      } else {
#pragma unroll
        for (int c = 0; c < EV; ++c) v[q][c] = rs[l + V * c];
        t[q] = tl[s];
      }
    }
#pragma unroll
    for (int q = 0; q < 6; ++q) g[q] = gk[6 * j + q];
    // only column blocks that reach past m - 1 need the mask (a uniform test)
#pragma unroll
    for (int c = 0; c < EV; ++c)
      if (V * (c + 1) > ms) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q][c] = inm[c] ? v[q][c] : 0.0;
      }
    double al[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      double d0 = v[q][0] * y[0], d1 = 0.0;
#pragma unroll
      for (int c = 1; c < EV; ++c) {
        if (c & 1)
          d1 = fma(v[q][c], y[c], d1);
        else
          d0 = fma(v[q][c], y[c], d0);
      }
      al[q] = EV > 1 ? d0 + d1 : d0;
    }
    group_sums_dpp<V>(al);
    const double fd = t[3] * al[3];
    const double fc = t[2] * fma(-g[5], fd, al[2]);
    const double fb = t[1] * fma(-g[4], fd, fma(-g[3], fc, al[1]));
    const double fa = t[0] * fma(-g[2], fd, fma(-g[1], fc, fma(-g[0], fb, al[0])));
#pragma unroll
    for (int c = 0; c < EV; ++c)
      y[c] = fma(-fa, v[0][c], fma(-fb, v[1][c], fma(-fc, v[2][c], fma(-fd, v[3][c], y[c]))));
  };
  if (nblk > 0) apply(nblk - 1, std::true_type{});
  for (int j = nblk - 2; j >= 0; --j) apply(j, std::false_type{});
  __syncthreads();
  if (kk < rj) {
    const double lam = es.lam[kk] / es.lim[2];
#pragma unroll
    for (int c = 0; c < EV; ++c) {
      const int i = l + V * c;
      if (i < m) A[kk * P + i] = lam * y[c];
    }
    if (l == 0) {
      sh.sig[kk] = lam;
      sh.top[kk] = kk;
    }
  }
  __syncthreads();
}

// Rank-r_j factors of a run of n rows X (n x d) in fp64 through the Gram
// matrix (SEKV, Metodologia 2: a span's rows are encoded by a truncated
// SVD basis), for the closing and the build of long spans.
// load_rows(t0, rb, dst) brings rows [t0, t0 + rb) of X into LDS as floats
// with row pitch d + 4 and ends with a barrier; pre(x_pre, for_blocks) runs
// once X is staged (the closing's summary); a_store(t, k, value) and
// w_store(k, e, value) receive A (n x r_j) and W (r_j x d).  Every thread of
// the workgroup calls it; it ends with a barrier.
struct RunLds {
  double* work;   // kCloseWork doubles
  float* stage;   // kBlock rows of 128 + 4 floats
  double* part;   // kCloseThreads + 8 doubles
  EigShared* es;
  FactorShared* sh;
};

template <class LoadRows, class Pre, class AOut, class WOut>
__device__ __forceinline__ void factor_run(int n, int d, int rank, const RunLds& L,
                                           const LoadRows& load_rows, const Pre& pre,
                                           const AOut& a_store, const WOut& w_store) {
  const int tid = threadIdx.x;
  double* const work = L.work;
  float* const stage = L.stage;
  double* const part = L.part;
  EigShared& es = *L.es;
  FactorShared& sh = *L.sh;
  // ---- layout.  Rows form (G = X X^T, m = n) when n <= d, else cols
  // form (G = X^T X, m = d).  X rows are staged as floats with pitch
  // xp = d + 4 (rows start 4 banks apart, so a wave reading one element
  // of 16 rows hits 16 bank groups, and stay 16-byte aligned).  While the
  // rows form accumulates G in registers, X sits at the start of `work`,
  // where G goes afterwards; X is kept after G (x_after) when both fit,
  // and is otherwise streamed from global memory in 32-row blocks.
  const int xp = d + 4;
  const bool rows_form = n <= d;
  const int m = rows_form ? n : d;
  const int gs = jacobi_group<kCloseThreads>(m);
  int Lp = gs;  // rows of G padded with zeros to gs * E columns, E a power of two
  while (Lp < m) Lp *= 2;
  const int Pj = jacobi_pitch(Lp, gs);
  const bool x_after = sizeof(double) * m * Pj + sizeof(float) * static_cast<size_t>(n) * xp <=
                       sizeof(double) * kCloseWork;
  float* const x_post = x_after ? reinterpret_cast<float*>(work + m * Pj) : nullptr;
  float* const x_pre = rows_form ? reinterpret_cast<float*>(work) : x_post;
  // visits X in order of rows: f(rows pointer, t0, rb), whole when
  // resident at x, else in 32-row blocks through `stage`
  auto for_blocks = [&](const float* x, const auto& f) {
    if (x != nullptr) {
      f(x, 0, n);
      return;
    }
    for (int t0 = 0; t0 < n; t0 += kBlock) {
      const int rb = min(kBlock, n - t0);
      load_rows(t0, rb, stage);
      f(static_cast<const float*>(stage), t0, rb);
      __syncthreads();
    }
  };
  if (x_pre != nullptr) load_rows(0, n, x_pre);
  pre(x_pre, for_blocks);

  // ---- Gram matrix and its r_j largest eigenpairs (sig = sigma^2): the
  // tridiagonal path, or Jacobi when the spectrum is clustered there
  auto gram = [&](int Lg, int Pg) {
    auto run = [&](auto tiles, auto half) {
      constexpr int kT = decltype(tiles)::value;
      if (rows_form) {
        gram_rows<decltype(half)::value>(x_pre, xp, m, d, work, Pg);
      } else {
        for_blocks(x_pre, [&](const float* xr, int t0, int rb) {
          gram_block<kT, false>(xr, xp, m, rb, work, Pg, t0 == 0, t0 + rb == n);
        });
      }
    };
    // tiles per wave: ceil(nt (nt + 1) / 8) for nt = ceil(m / 16) tiles a
    // side (gram_block); half the blocks a side, ceil(nt / 2) (gram_rows)
    if (m > 96)
      run(std::integral_constant<int, 9>(), std::integral_constant<int, 4>());
    else if (m > 64)
      run(std::integral_constant<int, 6>(), std::integral_constant<int, 3>());
    else if (m > 32)
      run(std::integral_constant<int, 3>(), std::integral_constant<int, 2>());
    else
      run(std::integral_constant<int, 1>(), std::integral_constant<int, 1>());
    for (int idx = tid; idx < m * (Lg - m); idx += kCloseThreads) {  // Jacobi's padding
      const int a = idx / (Lg - m);
      work[a * Pg + m + (idx - a * (Lg - m))] = 0.0;
    }
    __syncthreads();
  };
  const int rmax = min(rank, m);
  int P = Pj;
  int rj = 0;
  bool tri = rmax <= kMaxEig - 1;
  if (tri) {
    const int Pt = m + 1 + (m & 1);  // odd pitch: a wave's rows fall in distinct banks
    gram(m, Pt);
    if (m > 64)
      tridiagonalize<8, 4, 16, true>(work, m, Pt, es);
    else if (m > 32)
      tridiagonalize<4, 1, 16, false>(work, m, Pt, es);
    else if (m > 16)
      tridiagonalize<8, 1, 4, false>(work, m, Pt, es);
    else
      tridiagonalize<16, 1, 1, false>(work, m, Pt, es);
    const int nev = min(rmax + 1, m);
    double2* de = reinterpret_cast<double2*>(part);  // free after the summary
    top_eigenvalues(m, nev, es, de);
    const double l0 = es.lam[0];
    for (int k = 0; k + 1 < nev; ++k)
      if (es.lam[k] - es.lam[k + 1] <= kClusterGap * l0 && es.lam[k] > kSignificant * l0)
        tri = false;
    if (tri) {
      double* zs = reinterpret_cast<double*>(stage);
      // groups of V lanes per vector, EV >= m / V entries per lane (the
      // back-transform's steps cost about EV instructions each)
      if (rmax <= 16) {
        if (m > 64)
          top_eigenvectors<16, 8>(work, m, Pt, rmax, es, de, zs, sh);
        else if (m > 32)
          top_eigenvectors<16, 4>(work, m, Pt, rmax, es, de, zs, sh);
        else if (m > 16)
          top_eigenvectors<16, 2>(work, m, Pt, rmax, es, de, zs, sh);
        else
          top_eigenvectors<16, 1>(work, m, Pt, rmax, es, de, zs, sh);
      } else {
        if (m > 64)
          top_eigenvectors<8, 16>(work, m, Pt, rmax, es, de, zs, sh);
        else if (m > 32)
          top_eigenvectors<8, 8>(work, m, Pt, rmax, es, de, zs, sh);
        else
          top_eigenvectors<8, 4>(work, m, Pt, rmax, es, de, zs, sh);
      }
      P = Pt;
      rj = rmax;
    } else if (rows_form) {
      load_rows(0, n, x_pre);  // G took X's place
    }
  }
  if (!tri) {
    gram(Lp, Pj);
    jacobi_sweeps<kCloseThreads>(work, m, Lp, Pj, sh);
    rj = top_rows<kCloseThreads>(work, m, Lp, Pj, rank, sh);
  }
  // rows form after the tridiagonal path: the rj eigenvector rows are rows
  // 0 .. rj - 1 of work (top[k] = k); X goes back to LDS right after them
  // and the products S = R X after X (rj P + n xp / 2 + rj d doubles fit:
  // n <= d <= 128, P <= 130, rj <= 32)
  float* const x_out = rows_form && tri ? reinterpret_cast<float*>(work + rj * P) : x_post;
  double* const s_out = rows_form && tri ? work + rj * P + (n * xp + 1) / 2 : nullptr;
  if (rows_form && x_out != nullptr) load_rows(0, n, x_out);

  if (rows_form) {
    // A[t][k] = sigma_k u_k[t] = row_k[t] / sigma_k
    for (int o = tid; o < n * rj; o += kCloseThreads) {
      const int t = o / rj;
      const int k = o - t * rj;
      const double lam = sh.sig[sh.top[k]];
      a_store(t, k, lam > 0.0 ? work[sh.top[k] * P + t] / sqrt(lam) : 0.0);
    }
    if (s_out != nullptr) {
      // W[k][e] = sum_t X[t][e] row_k[t] / sigma_k^3
      rows_product(x_out, xp, n, d, rj, work, P, s_out);
      for (int o = tid; o < rj * d; o += kCloseThreads) {
        const int k = o / d;
        const double lam = sh.sig[k];
        w_store(k, o - k * d, lam > 0.0 ? s_out[o] / (lam * sqrt(lam)) : 0.0);
      }
    } else {
      // W[k][e] = sum_t X[t][e] row_k[t] / sigma_k^3: thread -> outputs
      // o = tid + q T (k = o / d, e = o % d), q < nq; the outputs advance
      // through the rows together, four chains of four rows at a time, so
      // that 32 loads are in flight per round trip (indices past the last
      // output are clamped and their sums dropped)
      constexpr int kOut = 32 * 128 / kCloseThreads;
      const int nq = __builtin_amdgcn_readfirstlane((rj * d + kCloseThreads - 1) / kCloseThreads);
      const int last = rj * d > 0 ? rj * d - 1 : 0;
      int eo[kOut], uo[kOut];
#pragma unroll
      for (int q = 0; q < kOut; ++q) {
        const int o = min(tid + q * kCloseThreads, last);
        const int k = o / d;
        eo[q] = o - k * d;
        uo[q] = sh.top[k] * P;
      }
      double wacc[kOut] = {};
      for_blocks(x_post, [&](const float* xr, int t0, int rb) {
        const double* ub = work + t0;
        int t = 0;
        for (; t + 4 <= rb; t += 4) {
#pragma unroll
          for (int q0 = 0; q0 < kOut; q0 += 4) {
            if (q0 >= nq) break;
            float xv[4][4];
            double uv[4][4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                xv[q][i] = xr[(t + i) * xp + eo[q0 + q]];
                uv[q][i] = ub[uo[q0 + q] + t + i];
              }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                wacc[q0 + q] = fma(static_cast<double>(xv[q][i]), uv[q][i], wacc[q0 + q]);
          }
        }
        for (; t < rb; ++t) {
#pragma unroll
          for (int q0 = 0; q0 < kOut; q0 += 4) {
            if (q0 >= nq) break;
#pragma unroll
            for (int q = q0; q < q0 + 4; ++q)
              wacc[q] = fma(static_cast<double>(xr[t * xp + eo[q]]), ub[uo[q] + t], wacc[q]);
          }
        }
      });
#pragma unroll
      for (int q = 0; q < kOut; ++q) {
        const int o = tid + q * kCloseThreads;
        if (o < rj * d) {
          const int k = o / d;
          const double lam = sh.sig[sh.top[k]];
          w_store(k, o - k * d, lam > 0.0 ? wacc[q] / (lam * sqrt(lam)) : 0.0);
        }
      }
    }
  } else {
    // W[k] = w_k = row_k / sigma_k^2
    for (int o = tid; o < rj * d; o += kCloseThreads) {
      const int k = o / d;
      const int e = o - k * d;
      const double lam = sh.sig[sh.top[k]];
      w_store(k, e, lam > 0.0 ? work[sh.top[k] * P + e] / lam : 0.0);
    }
    // A[t][k] = X[t] . w_k, as four interleaved partial sums (d % 4 == 0)
    for_blocks(x_post, [&](const float* xr, int t0, int rb) {
      for (int o = tid; o < rb * rj; o += kCloseThreads) {
        const int t = o / rj;
        const int k = o - t * rj;
        const double lam = sh.sig[sh.top[k]];
        const double* wk = work + sh.top[k] * P;
        const float* xt = xr + t * xp;
        double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
        for (int e = 0; e < d; e += 4) {
          s0 = fma(static_cast<double>(xt[e]), wk[e], s0);
          s1 = fma(static_cast<double>(xt[e + 1]), wk[e + 1], s1);
          s2 = fma(static_cast<double>(xt[e + 2]), wk[e + 2], s2);
          s3 = fma(static_cast<double>(xt[e + 3]), wk[e + 3], s3);
        }
        a_store(t0 + t, k, lam > 0.0 ? ((s0 + s1) + (s2 + s3)) / lam : 0.0);
      }
    });
  }
  __syncthreads();

}

template <int DT>
__global__ __launch_bounds__(kCloseThreads) void close_kernel(
    const float* __restrict__ h_new, const float* __restrict__ theta,
    const int32_t* __restrict__ last_anchor, const int32_t* __restrict__ n_full,
    const int32_t* __restrict__ n_spans, const float* __restrict__ h_full,
    const int32_t* __restrict__ full_pos, int32_t* __restrict__ span_start,
    int32_t* __restrict__ span_len, int32_t* __restrict__ tok_off,
    int32_t* __restrict__ tok_pad, float* __restrict__ log_len, int32_t* __restrict__ span_id,
    typename Elem<DT>::T* __restrict__ k_full, typename Elem<DT>::T* __restrict__ v_full,
    typename Elem<DT>::T* __restrict__ summary, typename Elem<DT>::T* __restrict__ vmean,
    typename Elem<DT>::T* __restrict__ a_k, typename Elem<DT>::T* __restrict__ a_v,
    typename Elem<DT>::T* __restrict__ w_k, typename Elem<DT>::T* __restrict__ w_v, int T,
    int d, int S, int Sp, int F, int Fp, int Np, int Hkv, int rank, int n_items) {
  typedef Elem<DT> E;
  typedef typename E::T ST;
  __shared__ FactorShared sh;
  __shared__ __align__(16) double work[kCloseWork];
  __shared__ __align__(16) float stage[kBlock * (128 + 4)];  // a streamed block of X rows
  __shared__ __align__(16) double part[kCloseThreads + 8];  // partial column sums; (d, e^2) pairs
  __shared__ double red[kCloseWaves];
  __shared__ EigShared es;
  const int tid = threadIdx.x;
  const RunLds L{work, stage, part, &es, &sh};

  // one item per workgroup (the grid is the item count) and no item loop:
  // with a loop the compiler computes much of the item's addressing ahead of
  // it and keeps it in scratch memory across the phase calls
  const int item = blockIdx.x;
  if (item >= n_items) return;
  {
    const int kv = item & 1;
    const int u = item >> 1;
    const int b = u / Hkv;
    const int h = u - b * Hkv;
    // the sequence's table entries, read together (one round trip before
    // the test, one more for the span's padded offset)
    const int la = last_anchor[b];
    const int nf = n_full[b];
    const float hn = h_new[b];
    const float th = theta[b];
    const int j = n_spans[b];
    const int n = nf - la - 1;
    // (j >= 0 always: testing it keeps its read in the first round trip)
    if (!(hn > th) || la < 0 || n <= 0 || j < 0) return;
    const int r0 = la + 1;
    const int tp = tok_pad[static_cast<size_t>(b) * (S + 1) + j];
    ST* xs = (kv ? v_full : k_full) + static_cast<size_t>(u) * Fp * d;

    // rows [t0, t0 + rb) of X into dst (row pitch xp)
    const int xp = d + 4;
    auto load_rows = [&](int t0, int rb, float* dst) {
      for_row_vectors(kv != 0, r0 + t0, r0 + t0 + rb, d, [&](size_t off, const int (&rr)[8],
                                                               const int (&cc)[8]) {
        float v[8];
        load8<DT>(xs + off, v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (rr[e] >= 0) dst[(rr[e] - r0 - t0) * xp + cc[e]] = v[e];
      });
      __syncthreads();
    };
    auto pre = [&](const float* x_pre, const auto& for_blocks) {
      // ---- summary (K item) or value mean (V item): column sums in fp64, in
      // row order; ng groups of d threads take interleaved rows, then the
      // groups are added in order
      const int ng = kCloseThreads / d;
      const int gi = tid / d;
      const int c = tid - gi * d;
      const float* hr = h_full + static_cast<size_t>(b) * F + r0;
      // the weights (surprisal for K, 1 for V) of up to 256 rows at a time
      // go to LDS first (es.tau is free until the reduction), so that the
      // sum's loads are LDS loads, four rows' issued together
      static_assert(sizeof(es.tau) >= 256 * sizeof(float), "weights of 256 rows");
      float* wbuf = reinterpret_cast<float*>(es.tau);
      double acc = 0.0;
      for_blocks(x_pre, [&](const float* xr, int t0, int rb) {
        for (int c0 = 0; c0 < rb; c0 += 256) {
          const int cn = min(256, rb - c0);
          __syncthreads();  // the previous chunk's weights are read
          if (tid < cn) wbuf[tid] = kv ? 1.0f : hr[t0 + c0 + tid];
          __syncthreads();
          const float* xc = xr + c0 * xp + c;
          int t = gi;
          for (; t + 3 * ng < cn; t += 4 * ng) {
            float w[4], x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              w[i] = wbuf[t + i * ng];
              x[i] = xc[(t + i * ng) * xp];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) acc += static_cast<double>(w[i]) * static_cast<double>(x[i]);
          }
          for (; t < cn; t += ng) acc += static_cast<double>(wbuf[t]) * static_cast<double>(xc[t * xp]);
        }
      });
      part[gi * d + c] = acc;
      __syncthreads();
      double tot = 0.0;
      if (tid < d)
        for (int q = 0; q < ng; ++q) tot += part[q * d + tid];
      if (kv == 0) {
        const double sq = wave_sum(tot * tot);
        if ((tid & (kWave - 1)) == 0) red[tid / kWave] = sq;
        __syncthreads();
        double norm2 = 0.0;
        for (int w = 0; w < d / kWave; ++w) norm2 += red[w];
        if (tid < d)
          summary[(static_cast<size_t>(u) * S + j) * d + tid] =
              E::from_f64(norm2 > 0.0 ? tot / sqrt(norm2) : 0.0);
      } else if (tid < d) {
        vmean[static_cast<size_t>(u) * Sp * d + v32_off(j, tid, d)] =
            E::from_f64(tot / static_cast<double>(n));
      }
      if (kv == 0 && h == 0) {
        const int st = full_pos[static_cast<size_t>(b) * F + r0];
        if (tid == 0) {
          span_start[static_cast<size_t>(b) * S + j] = st;
          span_len[static_cast<size_t>(b) * S + j] = n;
          tok_off[static_cast<size_t>(b) * (S + 1) + j + 1] =
              tok_off[static_cast<size_t>(b) * (S + 1) + j] + n;
          tok_pad[static_cast<size_t>(b) * (S + 1) + j + 1] = tp + round_up(n, 16);
          log_len[static_cast<size_t>(b) * S + j] = static_cast<float>(log(static_cast<double>(n)));
        }
        for (int p = st + tid; p < min(st + n, T); p += kCloseThreads)
          span_id[static_cast<size_t>(b) * T + p] = j;
      }
      __syncthreads();
    };
    auto a_store = [&](int t, int k, double val) {
      if (kv)
        a_v[static_cast<size_t>(u) * Np * rank + avt_off(tp + t, k, rank)] = E::from_f64(val);
      else
        a_k[(static_cast<size_t>(u) * Np + tp + t) * rank + k] = E::from_f64(val);
    };
    auto w_store = [&](int k, int e, double val) {
      if (kv)
        w_v[static_cast<size_t>(u) * S * d * rank4(rank) + wvt_off(j, k, e, d, rank)] =
            E::from_f64(val);
      else
        w_k[((static_cast<size_t>(u) * S + j) * rank + k) * d + e] = E::from_f64(val);
    };
    factor_run(n, d, rank, L, load_rows, pre, a_store, w_store);

    // ---- the run leaves the full-resolution set
    for_row_vectors(kv != 0, r0, r0 + n, d, [&](size_t off, const int (&rr)[8],
                                                const int (&cc)[8]) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (rr[e] >= 0) xs[off + e] = E::from_f64(0.0);
      (void)cc;
    });
    __syncthreads();
  }
}

// Build, spans whose rows exceed factor_kernel's LDS working matrix: one
// item per (unit, span, K or V) from the list `items` ((u S + j) 2 + kv),
// factored through the Gram matrix as a closing is, with the rows read from
// the row-major K/V input (16-byte vectors).
template <int DT>
__global__ __launch_bounds__(kCloseThreads) void factor_gram_kernel(
    const typename Elem<DT>::T* __restrict__ K, const typename Elem<DT>::T* __restrict__ V,
    const int32_t* __restrict__ span_start, const int32_t* __restrict__ span_len,
    const int32_t* __restrict__ tok_pad, const int32_t* __restrict__ items, int n_items, int T,
    int d, int S, int Np, int Hkv, int rank, typename Elem<DT>::T* __restrict__ a_k,
    typename Elem<DT>::T* __restrict__ a_v, typename Elem<DT>::T* __restrict__ w_k,
    typename Elem<DT>::T* __restrict__ w_v) {
  typedef Elem<DT> E;
  typedef typename E::T ST;
  __shared__ FactorShared sh;
  __shared__ __align__(16) double work[kCloseWork];
  __shared__ __align__(16) float stage[kBlock * (128 + 4)];
  __shared__ __align__(16) double part[kCloseThreads + 8];
  __shared__ EigShared es;
  const int tid = threadIdx.x;
  const RunLds L{work, stage, part, &es, &sh};
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int item = items[it];
    const int kv = item & 1;
    const int rest = item >> 1;
    const int j = rest % S;
    const int u = rest / S;
    const int b = u / Hkv;
    const int n = span_len[static_cast<size_t>(b) * S + j];
    const int st = span_start[static_cast<size_t>(b) * S + j];
    const int tp = tok_pad[static_cast<size_t>(b) * (S + 1) + j];
    const ST* X = (kv ? V : K) + (static_cast<size_t>(u) * T + st) * d;
    const int xp = d + 4;
    auto load_rows = [&](int t0, int rb, float* dst) {
      const int vpr = d / 8;  // 8-element vectors per row
      for (int idx = tid; idx < rb * vpr; idx += kCloseThreads) {
        const int t = idx / vpr;
        const int c8 = idx - t * vpr;
        float v[8];
        load8<DT>(X + static_cast<size_t>(t0 + t) * d + 8 * c8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[t * xp + 8 * c8 + e] = v[e];
      }
      __syncthreads();
    };
    auto pre = [](const float*, const auto&) {};
    auto a_store = [&](int t, int k, double val) {
      if (kv)
        a_v[static_cast<size_t>(u) * Np * rank + avt_off(tp + t, k, rank)] = E::from_f64(val);
      else
        a_k[(static_cast<size_t>(u) * Np + tp + t) * rank + k] = E::from_f64(val);
    };
    auto w_store = [&](int k, int e, double val) {
      if (kv)
        w_v[static_cast<size_t>(u) * S * d * rank4(rank) + wvt_off(j, k, e, d, rank)] =
            E::from_f64(val);
      else
        w_k[((static_cast<size_t>(u) * S + j) * rank + k) * d + e] = E::from_f64(val);
    };
    factor_run(n, d, rank, L, load_rows, pre, a_store, w_store);
  }
}

template <int DT>
hipError_t factor_impl(rskv_cache* c, const void* K, const void* V, hipStream_t st,
                       std::string* err) {
  typedef typename Elem<DT>::T T;
  const int U = c->B * c->Hkv;
  const long long n_items = 2ll * U * c->S;
  // spans whose rows do not fit factor_kernel's LDS working matrix go to
  // factor_gram_kernel through a list built from the span lengths
  std::vector<int32_t> lens(static_cast<size_t>(c->B) * c->S);
  hipError_t e = hipMemcpyAsync(lens.data(), c->dev.span_len, lens.size() * sizeof(int32_t),
                                hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  std::vector<int32_t> large;
  for (int u = 0; u < U; ++u) {
    const int b = u / c->Hkv;
    for (int j = 0; j < c->h_n_spans[b]; ++j) {
      const int n = lens[static_cast<size_t>(b) * c->S + j];
      if (static_cast<long long>(n) * c->d > kLdsWork) {
        const int32_t it = static_cast<int32_t>((static_cast<long long>(u) * c->S + j) * 2);
        large.push_back(it);
        large.push_back(it + 1);
      }
    }
  }
  const int grid_small = static_cast<int>(std::min<long long>(n_items, 1 << 20));
  if (n_items > 0) {
    hipLaunchKernelGGL((factor_kernel<DT>), dim3(grid_small), dim3(kFacThreads), 0, st,
                       static_cast<const T*>(K), static_cast<const T*>(V), c->dev.span_start,
                       c->dev.span_len, c->dev.tok_pad, c->dev.n_spans, c->T, c->d, c->S, c->Np,
                       c->Hkv, c->rank, n_items, static_cast<T*>(c->dev.a_k),
                       static_cast<T*>(c->dev.a_v), static_cast<T*>(c->dev.w_k),
                       static_cast<T*>(c->dev.w_v));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!large.empty()) {
    const size_t bytes = large.size() * sizeof(int32_t);
    int32_t* items = static_cast<int32_t*>(c->mem.alloc(bytes, st));
    if (items == nullptr) {
      if (err) *err = "device allocation failed: long-span item list";
      return hipErrorOutOfMemory;
    }
    e = hipMemcpyAsync(items, large.data(), bytes, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) {
      const int n_large = static_cast<int>(large.size());
      hipLaunchKernelGGL((factor_gram_kernel<DT>), dim3(std::min(n_large, 2048)),
                         dim3(kCloseThreads), 0, st, static_cast<const T*>(K),
                         static_cast<const T*>(V), c->dev.span_start, c->dev.span_len,
                         c->dev.tok_pad, items, n_large, c->T, c->d, c->S, c->Np, c->Hkv, c->rank,
                         static_cast<T*>(c->dev.a_k), static_cast<T*>(c->dev.a_v),
                         static_cast<T*>(c->dev.w_k), static_cast<T*>(c->dev.w_v));
      e = hipGetLastError();
    }
    // the host list must outlive the copy, the device list the kernel
    const hipError_t e2 = hipStreamSynchronize(st);
    c->mem.release(items, st);
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
  }
  return hipSuccess;
}

template <int DT>
hipError_t close_impl(const rskv_cache* c, const float* h, hipStream_t st,
                      const KernelEvents* ev) {
  typedef typename Elem<DT>::T T;
  const auto& v = c->dev;
  const int n_items = 2 * c->B * c->Hkv;
  return launch(close_kernel<DT>, dim3(c->close_grid), dim3(kCloseThreads), 0, st, ev, h,
                static_cast<const float*>(v.theta), static_cast<const int32_t*>(v.last_anchor),
                static_cast<const int32_t*>(v.n_full), static_cast<const int32_t*>(v.n_spans),
                static_cast<const float*>(v.h_full), static_cast<const int32_t*>(v.full_pos),
                v.span_start, v.span_len, v.tok_off, v.tok_pad, v.log_len, v.span_id,
                static_cast<T*>(v.k_full), static_cast<T*>(v.v_full), static_cast<T*>(v.summary),
                static_cast<T*>(v.vmean), static_cast<T*>(v.a_k), static_cast<T*>(v.a_v),
                static_cast<T*>(v.w_k), static_cast<T*>(v.w_v), c->T, c->d, c->S, c->Sp, c->F,
                c->Fp, c->Np, c->Hkv, c->rank, n_items);
}

}  // namespace

hipError_t launch_close(const rskv_cache* c, const float* h, hipStream_t st,
                        const KernelEvents* ev) {
  return c->dtype == kBF16 ? close_impl<kBF16>(c, h, st, ev) : close_impl<kF32>(c, h, st, ev);
}

hipError_t launch_factor(rskv_cache* c, const void* K, const void* V, hipStream_t st,
                         std::string* err) {
  return c->dtype == kBF16 ? factor_impl<kBF16>(c, K, V, st, err)
                           : factor_impl<kF32>(c, K, V, st, err);
}

}  // namespace rskv
