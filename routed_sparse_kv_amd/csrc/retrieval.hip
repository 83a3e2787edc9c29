// Token-retrieval router after "ParisKV: Fast and Drift-Robust KV-Cache
// Retrieval for Long-Context LLMs" (gist.science 2602.07721), section
// "Metodologia: Il Framework ParisKV".
//
// Build: every key of the retrieval region is rotated (SRHT, "Centroidi
// Analitici Robusti al Drift"), its sign pattern in each 8-wide subspace is
// its bucket, and its RSQ-IP record (4-bit codes and calibration w,
// "Reranking dei Candidati (RSQ-IP)") is stored.
//
// Decode ("Pipeline di Recupero Nativa su GPU in Due Stadi"), per unit
// (sequence b, KV head h), seven launches:
//   query     rotated group-mean query, vote table of every subspace
//   vote      vote total of every key; per-chunk and per-unit histograms
//   compact   smallest candidate score (prologue), then the candidates in
//             position order (ties to the lower position)
//   rerank    RSQ-IP estimate of every candidate (fp64, decided in fp32)
//   select    k_ret largest estimates (radix select, ties to lower position)
//   attend    one softmax over Sink, retrieved and Local rows, split in
//             64-row slices
//   merge     the slices' partial softmax states
// The vote kernel reads one byte per key and subspace: it streams the
// bucket array and is the HBM-bound step.
#include "common.h"
#include "retrieval.h"

namespace rskv {
namespace ret {
namespace {

// ------------------------------------------------------------- helpers

// Eight consecutive stored elements (16-byte aligned) as fp64.
template <int DT>
__device__ __forceinline__ void load8_f64(const typename Elem<DT>::T* p, double* x) {
  if constexpr (DT == kBF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = static_cast<double>(__uint_as_float(w[i] << 16));
      x[2 * i + 1] = static_cast<double>(__uint_as_float(w[i] & 0xffff0000u));
    }
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <int DT>
__device__ __forceinline__ void load8_f32(const typename Elem<DT>::T* p, float* x) {
  if constexpr (DT == kBF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

__device__ __forceinline__ bool sign_negative(const SignMask& s, int c) {
  return (s.w[c >> 5] >> (c & 31)) & 1u;
}

// Suffix sums over the lanes of a wave: lane l gets sum_{l' >= l} v_l'.
template <typename T>
__device__ __forceinline__ T wave_suffix_incl(T v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const T t = __shfl_down(v, o, kWave);
    if (lane + o < kWave) v += t;
  }
  return v;
}

// Exclusive prefix sum over a workgroup of NT threads (NT/64 <= 64 waves);
// `buf` holds NT/64 + 1 entries.  Returns the thread's exclusive prefix;
// *total receives the workgroup total.
template <int NT, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* buf, T* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const T incl = wave_incl_scan(v);
  if (lane == kWave - 1) buf[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const T w = lane < NW ? buf[lane] : T(0);
    const T wi = wave_incl_scan(w);
    if (lane < NW) buf[lane] = wi - w;
    if (lane == NW - 1) buf[NW] = wi;
  }
  __syncthreads();
  const T out = buf[wave] + incl - v;
  *total = buf[NW];
  __syncthreads();
  return out;
}

// Sum over a workgroup of NT threads; `buf` holds NT/64 entries.
template <int NT, typename T>
__device__ __forceinline__ T block_sum(T v, T* buf) {
  constexpr int NW = NT / kWave;
  v = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) buf[threadIdx.x / kWave] = v;
  __syncthreads();
  T s = T(0);
#pragma unroll
  for (int w = 0; w < NW; ++w) s += buf[w];
  __syncthreads();
  return s;
}

// Suffix counts over the vote totals: out[s] = sum_{s' >= s} cnt[s'] for
// s < nbins (nbins <= kMaxBins <= 320), computed by wave 0 with five bins
// per lane.  Other waves pass through.
template <typename In, typename Out>
__device__ __forceinline__ void suffix_counts(const In* cnt, int nbins, Out* out) {
  if (threadIdx.x >= kWave) return;
  const int lo = threadIdx.x * 5;
  uint32_t v[5];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    v[j] = lo + j < nbins ? static_cast<uint32_t>(cnt[lo + j]) : 0u;
    tot += v[j];
  }
  uint32_t run = wave_suffix_incl(tot) - tot;
#pragma unroll
  for (int j = 4; j >= 0; --j) {
    run += v[j];
    if (lo + j < nbins) out[lo + j] = static_cast<Out>(run);
  }
}

// ------------------------------------------------------------- build

// d/8 lanes per key, lane `sub` owns coordinates 8 sub .. 8 sub + 7, i.e.
// exactly subspace `sub`.  The Hadamard transform runs in fp64: its first
// three levels inside the lane, the others across lanes.  For keys stored
// in bf16 or fp32 every partial sum is exact, so the signs are exact.
template <int DT, int D>
__global__ __launch_bounds__(256) void encode_kernel(const typename Elem<DT>::T* __restrict__ K,
                                                     int T, int ns, int N, SignMask sg,
                                                     Codebook cb, uint8_t* __restrict__ buckets,
                                                     uint8_t* __restrict__ rec) {
  constexpr int LPK = D / 8;
  constexpr int KPW = kWave / LPK;
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = lane & (LPK - 1);
  const int64_t key =
      (static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave) * KPW +
      lane / LPK;
  const int u = blockIdx.y;
  const bool live = key < N;
  double x[8];
  if (live) {
    load8_f64<DT>(K + (static_cast<size_t>(u) * T + ns + key) * D + sub * 8, x);
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = 0.0;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t)
    if (sign_negative(sg, sub * 8 + t)) x[t] = -x[t];
  // (a, b) -> (a + b, a - b) on every bit level of the coordinate index
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const double a = x[i], b = x[i + h];
      x[i] = a + b;
      x[i + h] = a - b;
    }
  }
#pragma unroll
  for (int o = 1; o < LPK; o <<= 1) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const double p = __shfl_xor(x[t], o, kWave);
      x[t] = (sub & o) ? p - x[t] : x[t] + p;
    }
  }
  uint32_t bucket = 0;
  double nb2 = 0.0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    bucket |= (x[t] < 0.0 ? 1u : 0u) << t;
    nb2 += x[t] * x[t];
  }
  const double nb = sqrt(nb2);
  uint32_t code = 0;
  double den = 0.0;
  if (nb > 0.0) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const double ut = x[t] / nb;
      const double a = fabs(ut);
      double v = cb.lam[0];
      uint32_t j = 0;
#pragma unroll
      for (int jj = 1; jj < 8; ++jj) {
        if (a >= cb.beta[jj]) {
          v = cb.lam[jj];
          j = jj;
        }
      }
      const bool neg = ut < 0.0;
      den += (neg ? -v : v) * ut;
      code |= ((neg ? 8u : 0u) | j) << (4 * t);
    }
  }
  // w = ||k|| ||x~_b|| / <v, u> with ||x~_b|| = nb / (||k|| sqrt(d))
  const float w = (nb > 0.0 && den != 0.0)
                      ? static_cast<float>(nb / (sqrt(static_cast<double>(D)) * den))
                      : 0.f;
  if (live) {
    const size_t k = static_cast<size_t>(u) * N + key;
    buckets[k * (D / 8) + sub] = static_cast<uint8_t>(bucket);
    uint8_t* rp = rec + k * D;
    *reinterpret_cast<uint32_t*>(rp + sub * 4) = code;
    *reinterpret_cast<float*>(rp + D / 2 + sub * 4) = w;
  }
}

// ------------------------------------------------------------- decode

// Grid (d/8 subspaces, U).  Every workgroup rotates the unit's group-mean
// query (fp64, Hadamard levels through LDS), then ranks the 256 sign
// patterns of its subspace by <q~_b, c_p> (ties to the lower pattern) and
// writes the votes rho - rank for the top rho.  Workgroup 0 of the unit also
// stores q~ and ||q-bar|| and clears the unit's vote-total histogram.
template <int DT>
__global__ __launch_bounds__(256) void query_kernel(const typename Elem<DT>::T* __restrict__ q,
                                                    int Hq, int Hkv, int G, int d, SignMask sg,
                                                    int rho, double* __restrict__ qt_out,
                                                    double* __restrict__ qn_out,
                                                    uint8_t* __restrict__ votes,
                                                    uint32_t* __restrict__ tot) {
  typedef Elem<DT> E;
  const int sb = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int t = threadIdx.x;
  __shared__ double y[128];
  __shared__ double red[4];
  __shared__ double sc[256];
  double qb = 0.0;
  if (t < d) {
    const size_t base = (static_cast<size_t>(b) * Hq + static_cast<size_t>(h) * G) * d + t;
    for (int g = 0; g < G; ++g) qb += static_cast<double>(E::ld(q, base + static_cast<size_t>(g) * d));
    qb /= static_cast<double>(G);
  }
  const double nq2 = block_sum<256>(qb * qb, red);
  if (t < d) y[t] = sign_negative(sg, t) ? -qb : qb;
  __syncthreads();
  for (int hh = 1; hh < d; hh <<= 1) {
    if (t < d / 2) {
      const int i = (t / hh) * 2 * hh + (t % hh);
      const double a = y[i], c = y[i + hh];
      y[i] = a + c;
      y[i + hh] = a - c;
    }
    __syncthreads();
  }
  const double qn = sqrt(nq2);
  const double scale = qn * sqrt(static_cast<double>(d));
  if (sb == 0) {
    if (t < d) qt_out[static_cast<size_t>(u) * d + t] = scale > 0.0 ? y[t] / scale : 0.0;
    if (t == 0) qn_out[u] = qn;
    for (int i = t; i < kMaxBins; i += blockDim.x) tot[static_cast<size_t>(u) * kMaxBins + i] = 0u;
  }
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double v = scale > 0.0 ? y[sb * 8 + i] / scale : 0.0;
    s += ((t >> i) & 1) ? -v : v;
  }
  sc[t] = s;
  __syncthreads();
  int rank = 0;
  for (int p = 0; p < 256; ++p) {
    const double o = sc[p];
    rank += (o > s || (o == s && p < t)) ? 1 : 0;
  }
  votes[(static_cast<size_t>(u) * (d / 8) + sb) * 256 + t] =
      static_cast<uint8_t>(rank < rho ? rho - rank : 0);
}

// Grid (nchunk, U): kChunk consecutive keys per workgroup.  Vote totals by
// table lookups in LDS; per-chunk counts of totals >= s (for the ordered
// compaction) and the unit's histogram (global atomics, no return).
template <int BS>
__global__ __launch_bounds__(256) void vote_kernel(const uint8_t* __restrict__ buckets,
                                                   const uint8_t* __restrict__ votes, int N,
                                                   size_t npad, int nbins, int nchunk,
                                                   uint16_t* __restrict__ scores,
                                                   uint16_t* __restrict__ chist,
                                                   uint32_t* __restrict__ tot) {
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int t = threadIdx.x;
  __shared__ __align__(16) uint8_t vt[BS * 256];
  __shared__ uint32_t hist[kMaxBins];
  if (t < BS * 16)
    reinterpret_cast<uint4*>(vt)[t] =
        reinterpret_cast<const uint4*>(votes + static_cast<size_t>(u) * BS * 256)[t];
  for (int i = t; i < kMaxBins; i += blockDim.x) hist[i] = 0u;
  __syncthreads();
  const uint8_t* bk = buckets + static_cast<size_t>(u) * N * BS;
  uint16_t* sc = scores + static_cast<size_t>(u) * npad;
  const int i0 = c * kChunk;
#pragma unroll 4
  for (int k = 0; k < kChunk / 256; ++k) {
    const int i = i0 + k * 256 + t;
    if (i < N) {
      uint32_t w[BS / 4];
      if constexpr (BS == 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(bk + static_cast<size_t>(i) * 16);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(bk + static_cast<size_t>(i) * 8);
        w[0] = v.x; w[1] = v.y;
      }
      uint32_t s = 0;
#pragma unroll
      for (int j = 0; j < BS; ++j) s += vt[j * 256 + ((w[j >> 2] >> (8 * (j & 3))) & 255u)];
      sc[i] = static_cast<uint16_t>(s);
      atomicAdd(&hist[s], 1u);
    }
  }
  __syncthreads();
  suffix_counts(hist, nbins, chist + (static_cast<size_t>(u) * nchunk + c) * kMaxBins);
  for (int s = t; s < nbins; s += blockDim.x) {
    const uint32_t n = hist[s];
    if (n) atomicAdd(&tot[static_cast<size_t>(u) * kMaxBins + s], n);
  }
}

// Grid (nchunk, U).  Prologue (the threshold): s* = the largest total with
// at least C keys at or above it; quota = C - #(total > s*) keys at s* are
// taken, the first ones by position.  The chunk's output offset follows
// from the counts of the chunks before it.  Each thread then takes 16
// consecutive keys and writes the chunk's candidates in position order.
__global__ __launch_bounds__(256) void compact_kernel(const uint16_t* __restrict__ scores,
                                                      size_t npad,
                                                      const uint16_t* __restrict__ chist,
                                                      const uint32_t* __restrict__ tot, int N,
                                                      int nchunk, int nbins, int C,
                                                      int32_t* __restrict__ cand,
                                                      int32_t* __restrict__ thr) {
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int t = threadIdx.x;
  __shared__ uint32_t suf[kMaxBins + 1];
  __shared__ int red[4];
  __shared__ unsigned long long sbuf[5];
  suffix_counts(tot + static_cast<size_t>(u) * kMaxBins, nbins, suf);
  if (t == 0) suf[nbins] = 0u;
  __syncthreads();
  int cand_s = -1;
  for (int s = t; s < nbins; s += blockDim.x)
    if (suf[s] >= static_cast<uint32_t>(C)) cand_s = s;
  {
    int v = cand_s;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    if ((t & (kWave - 1)) == 0) red[t / kWave] = v;
    __syncthreads();
    cand_s = max(max(red[0], red[1]), max(red[2], red[3]));
    __syncthreads();
  }
  const int s_star = max(cand_s, 0);  // suf[0] = N >= C, so cand_s >= 0
  const int quota = C - static_cast<int>(suf[s_star + 1]);
  // counts of the chunks before this one
  const uint16_t* hrow = chist + static_cast<size_t>(u) * nchunk * kMaxBins;
  long long gt_b = 0, eq_b = 0;
  for (int cc = t; cc < c; cc += blockDim.x) {
    const int a = hrow[static_cast<size_t>(cc) * kMaxBins + s_star];
    const int bb = s_star + 1 < nbins ? hrow[static_cast<size_t>(cc) * kMaxBins + s_star + 1] : 0;
    gt_b += bb;
    eq_b += a - bb;
  }
  const unsigned long long packed =
      block_sum<256>(static_cast<unsigned long long>(gt_b) | (static_cast<unsigned long long>(eq_b) << 32),
                     sbuf);
  const int gtB = static_cast<int>(packed & 0xffffffffull);
  const int eqB = static_cast<int>(packed >> 32);
  const int out0 = gtB + min(quota, eqB);
  const int q_here = max(0, quota - eqB);
  // this thread's 16 keys
  const int i0 = c * kChunk + t * 16;
  const uint16_t* sp = scores + static_cast<size_t>(u) * npad + i0;
  uint16_t v[16];
  {
    const uint4 a = reinterpret_cast<const uint4*>(sp)[0];
    const uint4 b = reinterpret_cast<const uint4*>(sp)[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = static_cast<uint16_t>(w[j] & 0xffffu);
      v[2 * j + 1] = static_cast<uint16_t>(w[j] >> 16);
    }
  }
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const bool in = i0 + j < N;
    gt += (in && v[j] > s_star) ? 1u : 0u;
    eq += (in && v[j] == s_star) ? 1u : 0u;
  }
  unsigned long long total;
  const unsigned long long ex = block_excl_scan<256>(
      static_cast<unsigned long long>(gt) | (static_cast<unsigned long long>(eq) << 32), sbuf, &total);
  int tie = static_cast<int>(ex >> 32);
  int off = out0 + static_cast<int>(ex & 0xffffffffull) + min(q_here, tie);
  int32_t* cd = cand + static_cast<size_t>(u) * C;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = i0 + j;
    if (i >= N) break;
    bool take = v[j] > s_star;
    if (v[j] == s_star) {
      take = tie < q_here;
      ++tie;
    }
    if (take) {
      if (off < C) cd[off] = i;
      ++off;
    }
  }
  if (c == 0 && t == 0) {
    thr[2 * u] = s_star;
    thr[2 * u + 1] = quota;
  }
}

// Grid (ceil(C/256), U), one candidate per thread.  LDS table tq[c][nib] =
// (+-lambda_j) q~_c makes <v_b, q~_b> eight lookups per subspace.
template <int D>
__global__ __launch_bounds__(256) void rerank_kernel(const uint8_t* __restrict__ rec, int N,
                                                     const int32_t* __restrict__ cand, int C,
                                                     const double* __restrict__ qt_all,
                                                     const double* __restrict__ qn_all,
                                                     Codebook cb, float* __restrict__ est) {
  const int u = blockIdx.y;
  const int t = threadIdx.x;
  const int k = blockIdx.x * 256 + t;
  __shared__ double tq[D * 16];
  __shared__ double lam[8];
  if (t < 8) lam[t] = cb.lam[t];
  __syncthreads();
  const double* qt = qt_all + static_cast<size_t>(u) * D;
  for (int e = t; e < D * 16; e += 256) {
    const double p = lam[e & 7] * qt[e >> 4];
    tq[e] = (e & 8) ? -p : p;
  }
  __syncthreads();
  if (k >= C) return;
  // candidate indices lie in [0, N); the clamp only keeps a bad index in bounds
  const int i = min(max(cand[static_cast<size_t>(u) * C + k], 0), N - 1);
  const uint4* rp = reinterpret_cast<const uint4*>(rec + (static_cast<size_t>(u) * N + i) * D);
  uint32_t code[D / 8];
  float w[D / 8];
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const uint4 a = rp[j];
    code[4 * j] = a.x; code[4 * j + 1] = a.y; code[4 * j + 2] = a.z; code[4 * j + 3] = a.w;
    const uint4 b = rp[D / 32 + j];
    w[4 * j] = __uint_as_float(b.x); w[4 * j + 1] = __uint_as_float(b.y);
    w[4 * j + 2] = __uint_as_float(b.z); w[4 * j + 3] = __uint_as_float(b.w);
  }
  double acc = 0.0;
#pragma unroll
  for (int b = 0; b < D / 8; ++b) {
    double dot = 0.0;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) dot += tq[(b * 8 + tt) * 16 + ((code[b] >> (4 * tt)) & 15u)];
    acc += static_cast<double>(w[b]) * dot;
  }
  est[static_cast<size_t>(u) * C + k] = static_cast<float>(qn_all[u] * acc);
}

// Grid U, 1024 threads.  Radix select (8-bit digits from the top, per-wave
// histograms in LDS) of the n_sel largest fp32 estimates; then an ordered
// pass writes the retrieved positions ascending: keys above the threshold
// key, and the first `quota` keys equal to it.
__global__ __launch_bounds__(1024) void select_kernel(const float* __restrict__ est,
                                                      const int32_t* __restrict__ cand, int C,
                                                      int n_sel, int k_ret, int first,
                                                      int32_t* __restrict__ sel,
                                                      int32_t* __restrict__ retrieved) {
  constexpr int NT = 1024, NW = NT / kWave;
  const int u = blockIdx.x;
  const int t = threadIdx.x;
  const int wave = t / kWave;
  const int lane = t & (kWave - 1);
  __shared__ uint32_t wh[NW][256];
  __shared__ uint32_t total[256];
  __shared__ uint32_t s_digit, s_above;
  __shared__ unsigned long long sbuf[NW + 1];
  const float* e = est + static_cast<size_t>(u) * C;
  const int32_t* cd = cand + static_cast<size_t>(u) * C;
  uint32_t prefix = 0, pmask = 0;
  uint32_t remaining = static_cast<uint32_t>(n_sel);
  const bool all = n_sel >= C;
  if (!all) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = t; i < NW * 256; i += NT) (&wh[0][0])[i] = 0u;
      __syncthreads();
      for (int k = t; k < C; k += NT) {
        const uint32_t key = f32_order_key(e[k]);
        if ((key & pmask) == prefix) atomicAdd(&wh[wave][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (t < 256) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += wh[w][t];
        total[t] = s;
      }
      __syncthreads();
      if (t < kWave) {
        // lane l holds digits 4l .. 4l+3; suffix counts from the top digit
        uint32_t v[4], tot4 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = total[4 * lane + j];
          tot4 += v[j];
        }
        uint32_t run = wave_suffix_incl(tot4) - tot4;  // digits above this lane's
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          const uint32_t above = run;
          run += v[j];
          if (above < remaining && run >= remaining) {
            s_digit = static_cast<uint32_t>(4 * lane + j);
            s_above = above;
          }
        }
      }
      __syncthreads();
      remaining -= s_above;
      prefix |= s_digit << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
  }
  // ordered output over contiguous blocks of candidates
  const int per = (C + NT - 1) / NT;
  const int k0 = min(C, t * per);
  const int k1 = min(C, k0 + per);
  uint32_t gt = 0, eq = 0;
  for (int k = k0; k < k1; ++k) {
    const uint32_t key = f32_order_key(e[k]);
    gt += (all || key > prefix) ? 1u : 0u;
    eq += (!all && key == prefix) ? 1u : 0u;
  }
  unsigned long long tot;
  const unsigned long long ex = block_excl_scan<NT>(
      static_cast<unsigned long long>(gt) | (static_cast<unsigned long long>(eq) << 32), sbuf, &tot);
  uint32_t tie = static_cast<uint32_t>(ex >> 32);
  int off = static_cast<int>(ex & 0xffffffffull) + static_cast<int>(min(remaining, tie));
  int32_t* so = sel + static_cast<size_t>(u) * n_sel;
  int32_t* ro = retrieved ? retrieved + static_cast<size_t>(u) * k_ret : nullptr;
  for (int k = k0; k < k1; ++k) {
    const uint32_t key = f32_order_key(e[k]);
    bool take = all || key > prefix;
    if (!all && key == prefix) {
      take = tie < remaining;
      ++tie;
    }
    if (take && off < n_sel) {
      const int32_t p = first + cd[k];
      so[off] = p;
      if (ro) ro[off] = p;
    }
    off += take ? 1 : 0;
  }
  if (ro)
    for (int j = n_sel + t; j < k_ret; j += NT) ro[j] = -1;
}

// Grid (nsplit, U): 64 attended rows per workgroup (Sink rows, then the
// retrieved rows, then the Local rows).  Partial softmax state per query
// head: acc[d], running max, running sum.
template <int DT, int D>
__global__ __launch_bounds__(256) void attend_kernel(
    const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ k_near,
    const typename Elem<DT>::T* __restrict__ v_near, const typename Elem<DT>::T* k_far,
    const typename Elem<DT>::T* v_far, const int32_t* __restrict__ sel, int Hq, int Hkv, int G,
    int ns, int n_sel, int N, int n_near, int n_att, int nsplit, float* __restrict__ part) {
  typedef Elem<DT> E;
  typedef typename Elem<DT>::T T;
  const int split = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  __shared__ float qs[8][D];
  __shared__ float ks[kRows][D + 1];
  __shared__ float vs[kRows][D];
  __shared__ float pl[8][kRows];
  const int r0 = split * kRows;
  const int nr = min(kRows, n_att - r0);
  const size_t qbase = (static_cast<size_t>(b) * Hq + static_cast<size_t>(h) * G) * D;
  for (int e = t; e < G * D; e += 256) qs[e / D][e % D] = E::ld(q, qbase + e);
  for (int e = t; e < kRows * (D / 8); e += 256) {
    const int r = e / (D / 8);
    const int c8 = (e - r * (D / 8)) * 8;
    if (r >= nr) continue;
    const int rr = r0 + r;
    const T* kp;
    const T* vp;
    if (rr < ns) {
      const size_t o = (static_cast<size_t>(u) * n_near + rr) * D + c8;
      kp = k_near + o;
      vp = v_near + o;
    } else if (rr < ns + n_sel) {
      // retrieved positions lie in [ns, ns + N); the clamp only keeps a bad
      // index in bounds
      const int i = min(max(sel[static_cast<size_t>(u) * n_sel + (rr - ns)] - ns, 0), N - 1);
      const size_t o = (static_cast<size_t>(u) * N + i) * D + c8;
      kp = k_far + o;
      vp = v_far + o;
    } else {
      const size_t o = (static_cast<size_t>(u) * n_near + ns + (rr - ns - n_sel)) * D + c8;
      kp = k_near + o;
      vp = v_near + o;
    }
    float kx[8], vx[8];
    load8_f32<DT>(kp, kx);
    load8_f32<DT>(vp, vx);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ks[r][c8 + j] = kx[j];
      vs[r][c8 + j] = vx[j];
    }
  }
  __syncthreads();
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  for (int e = t; e < G * kRows; e += 256) {
    const int g = e / kRows;
    const int r = e - g * kRows;
    float s = -INFINITY;
    if (r < nr) {
      float a = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; ++c) a += qs[g][c] * ks[r][c];
      s = a * scale;
    }
    pl[g][r] = s;
  }
  __syncthreads();
  float* pbase = part + (static_cast<size_t>(u) * nsplit + split) * G * (D + 2);
  for (int g = wave; g < G; g += 4) {
    const float s = pl[g][lane];
    const float mx = wave_max(s);
    const float p = lane < nr ? expf(s - mx) : 0.f;
    const float l = wave_sum(p);
    pl[g][lane] = p;
    if (lane == 0) {
      pbase[g * (D + 2) + D] = mx;
      pbase[g * (D + 2) + D + 1] = l;
    }
  }
  __syncthreads();
  for (int e = t; e < G * D; e += 256) {
    const int g = e / D;
    const int c = e - g * D;
    float a = 0.f;
    for (int r = 0; r < nr; ++r) a += pl[g][r] * vs[r][c];
    pbase[g * (D + 2) + c] = a;
  }
}

// Grid U: out = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part, int nsplit,
                                                    int G, int D, int Hq, int Hkv,
                                                    float* __restrict__ out) {
  const int u = blockIdx.x;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const size_t stride = static_cast<size_t>(G) * (D + 2);
  const float* p0 = part + static_cast<size_t>(u) * nsplit * stride;
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int g = e / D;
    const int c = e - g * D;
    const float* p = p0 + static_cast<size_t>(g) * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, p[s * stride + D]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float f = expf(p[s * stride + D] - M);
      num += f * p[s * stride + c];
      den += f * p[s * stride + D + 1];
    }
    out[(static_cast<size_t>(b) * Hq + static_cast<size_t>(h) * G + g) * D + c] = num / den;
  }
}

template <int DT>
hipError_t encode_impl(const rskv_retrieval* r, const void* K, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  if (r->N == 0) return hipSuccess;
  const int U = r->B * r->Hkv;
  const int kpb = 4 * (kWave / (r->d / 8));  // keys per workgroup
  dim3 grid((r->N + kpb - 1) / kpb, U);
  if (r->d == 128)
    hipLaunchKernelGGL((encode_kernel<DT, 128>), grid, dim3(256), 0, st, static_cast<const T*>(K),
                       r->T, r->ns, r->N, r->signs, r->cb, r->buckets, r->rec);
  else
    hipLaunchKernelGGL((encode_kernel<DT, 64>), grid, dim3(256), 0, st, static_cast<const T*>(K),
                       r->T, r->ns, r->N, r->signs, r->cb, r->buckets, r->rec);
  return hipGetLastError();
}

template <int DT>
hipError_t decode_impl(const rskv_retrieval* r, const void* qv, float* out, int32_t* retrieved,
                       hipStream_t st, const KernelEvents* ev, bool* recorded) {
  typedef typename Elem<DT>::T T;
  const T* q = static_cast<const T*>(qv);
  const int U = r->B * r->Hkv;
  const bool active = r->n_sel > 0;
  auto E = [&](int k) -> const KernelEvents* {
    if (recorded) recorded[k] = true;
    return ev ? ev + k : nullptr;
  };
  if (recorded)
    for (int k = 0; k < kKernels; ++k) recorded[k] = false;
  hipError_t e = hipSuccess;
  if (active) {
    e = launch(query_kernel<DT>, dim3(r->Bs, U), dim3(256), 0, st, E(0), q, r->Hq, r->Hkv, r->G,
               r->d, r->signs, r->rho, r->qt, r->qn, r->votes, r->tot);
    if (e != hipSuccess) return e;
    if (r->Bs == 16)
      e = launch(vote_kernel<16>, dim3(r->nchunk, U), dim3(256), 0, st, E(1),
                 static_cast<const uint8_t*>(r->buckets), static_cast<const uint8_t*>(r->votes),
                 r->N, r->npad, r->nbins, r->nchunk, r->scores, r->chist, r->tot);
    else
      e = launch(vote_kernel<8>, dim3(r->nchunk, U), dim3(256), 0, st, E(1),
                 static_cast<const uint8_t*>(r->buckets), static_cast<const uint8_t*>(r->votes),
                 r->N, r->npad, r->nbins, r->nchunk, r->scores, r->chist, r->tot);
    if (e != hipSuccess) return e;
    e = launch(compact_kernel, dim3(r->nchunk, U), dim3(256), 0, st, E(2),
               static_cast<const uint16_t*>(r->scores), r->npad,
               static_cast<const uint16_t*>(r->chist), static_cast<const uint32_t*>(r->tot), r->N,
               r->nchunk, r->nbins, r->C, r->cand, r->thr);
    if (e != hipSuccess) return e;
    if (r->d == 128)
      e = launch(rerank_kernel<128>, dim3((r->C + 255) / 256, U), dim3(256), 0, st, E(3),
                 static_cast<const uint8_t*>(r->rec), r->N, static_cast<const int32_t*>(r->cand),
                 r->C, static_cast<const double*>(r->qt), static_cast<const double*>(r->qn),
                 r->cb, r->est);
    else
      e = launch(rerank_kernel<64>, dim3((r->C + 255) / 256, U), dim3(256), 0, st, E(3),
                 static_cast<const uint8_t*>(r->rec), r->N, static_cast<const int32_t*>(r->cand),
                 r->C, static_cast<const double*>(r->qt), static_cast<const double*>(r->qn),
                 r->cb, r->est);
    if (e != hipSuccess) return e;
  }
  if (active || (retrieved != nullptr && r->k_ret > 0)) {
    e = launch(select_kernel, dim3(U), dim3(1024), 0, st, E(4), static_cast<const float*>(r->est),
               static_cast<const int32_t*>(r->cand), active ? r->C : 0, r->n_sel, r->k_ret, r->ns,
               r->sel, retrieved);
    if (e != hipSuccess) return e;
  }
  const T* kn = static_cast<const T*>(r->k_near);
  const T* vn = static_cast<const T*>(r->v_near);
  const T* kf = static_cast<const T*>(r->k_far);
  const T* vf = static_cast<const T*>(r->v_far);
  if (r->d == 128)
    e = launch(attend_kernel<DT, 128>, dim3(r->nsplit, U), dim3(256), 0, st, E(5), q, kn, vn, kf,
               vf, static_cast<const int32_t*>(r->sel), r->Hq, r->Hkv, r->G, r->ns, r->n_sel, r->N,
               r->n_near, r->n_att, r->nsplit, r->part);
  else
    e = launch(attend_kernel<DT, 64>, dim3(r->nsplit, U), dim3(256), 0, st, E(5), q, kn, vn, kf,
               vf, static_cast<const int32_t*>(r->sel), r->Hq, r->Hkv, r->G, r->ns, r->n_sel, r->N,
               r->n_near, r->n_att, r->nsplit, r->part);
  if (e != hipSuccess) return e;
  return launch(merge_kernel, dim3(U), dim3(256), 0, st, E(6), static_cast<const float*>(r->part),
                r->nsplit, r->G, r->d, r->Hq, r->Hkv, out);
}

}  // namespace

hipError_t launch_encode(const rskv_retrieval* r, const void* K, hipStream_t st) {
  return r->dtype == kBF16 ? encode_impl<kBF16>(r, K, st) : encode_impl<kF32>(r, K, st);
}

hipError_t launch_decode(const rskv_retrieval* r, const void* q, float* out, int32_t* retrieved,
                         hipStream_t st, const KernelEvents* ev, bool* recorded) {
  return r->dtype == kBF16 ? decode_impl<kBF16>(r, q, out, retrieved, st, ev, recorded)
                           : decode_impl<kF32>(r, q, out, retrieved, st, ev, recorded);
}

}  // namespace ret
}  // namespace rskv
