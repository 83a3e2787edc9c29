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
// (sequence b, KV head h), at most ten launches:
//   query     rotated group-mean query, vote table of every subspace
//   vote      vote total of every key; per-chunk and per-unit histograms
//   compact   smallest candidate score (prologue), then the candidates in
//             position order (ties to the lower position)
//   rerank    RSQ-IP estimate of every candidate (fp64, decided in fp32)
//   top-k     k_ret largest estimates over the whole chip in four launches
//             (histogram, crossing bin, exact threshold, ordered output;
//             ties to the lower position)
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

// Grid (d/8 subspaces, U), 1024 threads.  Every workgroup rotates the
// unit's group-mean query (fp64, in wave 0: Hadamard levels by shuffles,
// the top level of d = 128 within the lane), then ranks the
// 256 sign patterns of its subspace by <q~_b, c_p> (ties to the lower
// pattern): four threads per pattern each count the better patterns among
// an interleaved quarter, and two shuffles add the counts.  The top rho
// patterns get rho - rank votes.  Workgroup 0 of the unit also stores q~ and
// ||q-bar|| and clears the unit's vote-total histogram; the workgroups
// together clear the unit's estimate histogram and top-k member count.
template <int DT>
__global__ __launch_bounds__(1024) void query_kernel(const typename Elem<DT>::T* __restrict__ q,
                                                     int Hq, int Hkv, int G, int d, SignMask sg,
                                                     int rho, double* __restrict__ qt_out,
                                                     double* __restrict__ qn_out,
                                                     uint8_t* __restrict__ votes,
                                                     uint32_t* __restrict__ tot,
                                                     uint32_t* __restrict__ ehtot,
                                                     uint32_t* __restrict__ lcnt) {
  typedef Elem<DT> E;
  const int sb = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int t = threadIdx.x;
  __shared__ double y[128];  // q~ (scaled)
  __shared__ double sc[256];
  if (t < kWave) {
    // wave 0: group mean, norm and Hadamard levels in registers and
    // shuffles; lane l holds coordinates l and l + 64 (d = 128)
    const size_t base = (static_cast<size_t>(b) * Hq + static_cast<size_t>(h) * G) * d;
    double x[2] = {0.0, 0.0};
    const int nv = d / kWave;  // 1 or 2 coordinates per lane
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      if (v < nv) {
        const int c = t + v * kWave;
        double a = 0.0;
        for (int g = 0; g < G; ++g) a += static_cast<double>(E::ld(q, base + static_cast<size_t>(g) * d + c));
        x[v] = a / static_cast<double>(G);
      }
    }
    const double qn = sqrt(wave_sum(x[0] * x[0] + x[1] * x[1]));
#pragma unroll
    for (int v = 0; v < 2; ++v)
      if (v < nv && sign_negative(sg, t + v * kWave)) x[v] = -x[v];
    // (a, b) -> (a + b, a - b) on every bit level of the coordinate index
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const double pv = __shfl_xor(x[v], o, kWave);
        x[v] = (t & o) ? pv - x[v] : x[v] + pv;
      }
    }
    if (nv == 2) {
      const double a = x[0], c = x[1];
      x[0] = a + c;
      x[1] = a - c;
    }
    const double scale = qn * sqrt(static_cast<double>(d));
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      if (v < nv) {
        const double qt = scale > 0.0 ? x[v] / scale : 0.0;
        y[t + v * kWave] = qt;
        if (sb == 0) qt_out[static_cast<size_t>(u) * d + t + v * kWave] = qt;
      }
    }
    if (sb == 0 && t == 0) {
      qn_out[u] = qn;
      lcnt[u] = 0u;
    }
  }
  if (sb == 0)
    for (int i = t; i < kMaxBins; i += blockDim.x) tot[static_cast<size_t>(u) * kMaxBins + i] = 0u;
  for (int i = sb * blockDim.x + t; i < kSelBins; i += gridDim.x * blockDim.x)
    ehtot[static_cast<size_t>(u) * kSelBins + i] = 0u;
  __syncthreads();
  const int p = t >> 2;
  const int part = t & 3;
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double v = y[sb * 8 + i];
    s += ((p >> i) & 1) ? -v : v;
  }
  if (part == 0) sc[p] = s;
  __syncthreads();
  int rank = 0;
#pragma unroll 16
  for (int jj = 0; jj < 64; ++jj) {
    const int o_p = 4 * jj + part;
    const double o = sc[o_p];
    rank += (o > s || (o == s && o_p < p)) ? 1 : 0;
  }
  rank += __shfl_xor(rank, 1, kWave);
  rank += __shfl_xor(rank, 2, kWave);
  if (part == 0)
    votes[(static_cast<size_t>(u) * (d / 8) + sb) * 256 + p] =
        static_cast<uint8_t>(rank < rho ? rho - rank : 0);
}

// Grid (nchunk, U): kChunk consecutive keys per workgroup.  Vote totals by
// table lookups in LDS; per-chunk counts of totals >= s (for the ordered
// compaction) and the unit's histogram (global atomics, no return).  Totals
// of 0, a third of the keys, are counted per wave.  (Measured on MI355X:
// tables replicated per LDS bank with one persistent workgroup per compute
// unit, and 4-bit conflict-free tables, were both slower; the kernel is
// bound by its ~32 VALU + 16 LDS instructions per key beside 18 HBM bytes.)
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
    bool zero = false;
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
      if (s != 0) atomicAdd(&hist[s], 1u);
      zero = s == 0;
    }
    // totals of 0, a third of the keys, are counted per wave
    const unsigned long long z = __ballot(i < N && zero);
    if ((t & (kWave - 1)) == 0 && z) atomicAdd(&hist[0], static_cast<uint32_t>(__popcll(z)));
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
  // this thread's 16 keys (loaded first: independent of the threshold)
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
  suffix_counts(tot + static_cast<size_t>(u) * kMaxBins, nbins, suf);
  if (t == 0) suf[nbins] = 0u;
  __syncthreads();
  int cand_s = -1;
  for (int s = t; s < nbins; s += blockDim.x)
    if (suf[s] >= static_cast<uint32_t>(C)) cand_s = s;
  {
    int mv = cand_s;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) mv = max(mv, __shfl_xor(mv, o, kWave));
    if ((t & (kWave - 1)) == 0) red[t / kWave] = mv;
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
                                                     Codebook cb, float* __restrict__ est,
                                                     uint32_t* __restrict__ rmm) {
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
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  if (k < C) {
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
    const float ev = static_cast<float>(qn_all[u] * acc);
    est[static_cast<size_t>(u) * C + k] = ev;
    kmin = kmax = f32_order_key(ev);
  }
  // this workgroup's estimate range (order keys), for the top-k histogram
  __shared__ uint32_t red[8];
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o, kWave)));
    kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o, kWave)));
  }
  if ((t & (kWave - 1)) == 0) {
    red[t / kWave] = kmin;
    red[4 + t / kWave] = kmax;
  }
  __syncthreads();
  if (t == 0) {
    uint2 mm;
    mm.x = min(min(red[0], red[1]), min(red[2], red[3]));
    mm.y = max(max(red[4], red[5]), max(red[6], red[7]));
    reinterpret_cast<uint2*>(rmm)[static_cast<size_t>(u) * gridDim.x + blockIdx.x] = mm;
  }
}

// Block-wide minimum / maximum over NT threads (`buf` holds NT/64 floats).
template <int NT>
__device__ __forceinline__ float block_min(float v, float* buf) {
  constexpr int NW = NT / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) buf[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = buf[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fminf(r, buf[w]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float* buf) {
  constexpr int NW = NT / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) buf[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = buf[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, buf[w]);
  __syncthreads();
  return r;
}

// Lanes of this wave below the calling lane, as a mask.
__device__ __forceinline__ unsigned long long lanes_below() {
  return (1ull << (threadIdx.x & (kWave - 1))) - 1ull;
}

// Monotone bin of x in [lo, hi] over NB bins, scale = NB / (hi - lo) (the
// width formed in fp64, so it is finite for any fp32 pair).  Rounding of
// x - lo and of the product preserves order (an fp32 overflow to +inf
// included, clamped before the conversion), so every key of a higher bin is
// larger than every key of a lower bin; lo falls in bin 0 and hi in bin
// NB - 1.
template <int NB>
__device__ __forceinline__ int range_bin(float x, float lo, float scale) {
  return static_cast<int>(fminf((x - lo) * scale, static_cast<float>(NB - 1)));
}

// Inverse of f32_order_key (for keys of finite values).
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The unit's estimate range [lo, hi] (from the order keys in rng) and the
// bin scale over it, identical in every kernel that bins estimates.
struct EstRange {
  float lo, hi, scale;
};

__device__ __forceinline__ EstRange est_range(uint32_t kmin, uint32_t kmax) {
  EstRange r;
  r.lo = f32_from_order_key(kmin);
  r.hi = f32_from_order_key(kmax);
  r.scale = r.lo < r.hi
                ? static_cast<float>(kSelBins / (static_cast<double>(r.hi) - static_cast<double>(r.lo)))
                : 0.f;
  return r;
}

// Crossing bin of a histogram held in LDS (NB bins, counts from the top):
// the bin where the count of keys in higher bins stays below `rem` and the
// count including it reaches `rem`.  Sets *bin and *above (keys in higher
// bins); every thread of the workgroup calls it.
template <int NT, int NB>
__device__ __forceinline__ void crossing_bin(const uint32_t* hist, uint32_t rem,
                                             unsigned long long* sbuf, int* s_bin,
                                             uint32_t* s_above) {
  constexpr int BPT = NB / NT;
  const int t = threadIdx.x;
  uint32_t s4 = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) s4 += hist[NB - 1 - (BPT * t + i)];
  unsigned long long total;
  uint32_t above =
      static_cast<uint32_t>(block_excl_scan<NT>(static_cast<unsigned long long>(s4), sbuf, &total));
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const uint32_t ci = hist[NB - 1 - (BPT * t + i)];
    if (above < rem && above + ci >= rem) {
      *s_bin = NB - 1 - (BPT * t + i);
      *s_above = above;
    }
    above += ci;
  }
  __syncthreads();
}

// Value-range refinement over the `len` keys at `src` (LDS or global
// memory, read with stride NT): histogram the keys inside [lo, hi] over NB
// equal-width bins, keep the crossing bin, shrink [lo, hi] to its smallest
// and largest key, until lo == hi.  Each round shrinks the range at least
// NB-fold, so fp32 needs at most a few dozen rounds.  Returns the value all
// remaining keys share; *rem becomes the number of them to take.
template <int NT, int NB>
__device__ float refine_range(const float* src, int len, float lo, float hi, uint32_t* rem,
                              uint32_t* hist, float* fbuf, unsigned long long* sbuf, int* s_bin,
                              uint32_t* s_above) {
  const int t = threadIdx.x;
  for (int round = 0; round < 64 && lo < hi; ++round) {
    for (int i = t; i < NB; i += NT) hist[i] = 0u;
    __syncthreads();
    const float scale =
        static_cast<float>(NB / (static_cast<double>(hi) - static_cast<double>(lo)));
    for (int k = t; k < len; k += NT) {
      const float x = src[k];
      if (x >= lo && x <= hi) atomicAdd(&hist[range_bin<NB>(x, lo, scale)], 1u);
    }
    __syncthreads();
    crossing_bin<NT, NB>(hist, *rem, sbuf, s_bin, s_above);
    const int bsel = *s_bin;
    *rem -= *s_above;
    float nlo = INFINITY, nhi = -INFINITY;
    for (int k = t; k < len; k += NT) {
      const float x = src[k];
      if (x >= lo && x <= hi && range_bin<NB>(x, lo, scale) == bsel) {
        nlo = x < nlo ? x : nlo;
        nhi = x > nhi ? x : nhi;
      }
    }
    lo = block_min<NT>(nlo, fbuf);
    hi = block_max<NT>(nhi, fbuf);
  }
  return lo;
}

// The top-k selection of each unit (the n_sel largest fp32 estimates, ties
// to the lower candidate index, output ascending) runs over the whole chip
// in four launches, with blocks of kSelBlock candidates:
//   ehist_kernel   the unit's range [lo, hi] from the rerank workgroups, and
//                  the histogram of the estimates over kSelBins equal-width
//                  bins of it (binning is monotone in the value, so every
//                  key of a higher bin exceeds every key of a lower one);
//   cross_kernel   the crossing bin b1 (keys of higher bins are all taken,
//                  keys of lower bins none); per block, the keys above b1;
//                  the keys inside b1 go to a member list;
//   thresh_kernel  exact value-range refinement over the members gives the
//                  threshold T and the number of ties at T to take, a radix
//                  select over the tied members' indices the last tied index
//                  taken; per block, the output offset;
//   output_kernel  each block writes its taken candidates in index order.
// When every estimate is equal the first n_sel candidates are taken; when
// n_sel >= C all are, and only the output kernel runs.

// Grid (nsb, U), 256 threads.
__global__ __launch_bounds__(256) void ehist_kernel(const float* __restrict__ est, int C, int nrwg,
                                                    const uint32_t* __restrict__ rmm,
                                                    uint32_t* __restrict__ rng,
                                                    uint32_t* __restrict__ ehtot) {
  const int blk = blockIdx.x;
  const int u = blockIdx.y;
  const int t = threadIdx.x;
  __shared__ uint32_t hist[kSelBins];
  __shared__ uint32_t red[8];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  const uint2* mm = reinterpret_cast<const uint2*>(rmm) + static_cast<size_t>(u) * nrwg;
  for (int i = t; i < nrwg; i += 256) {
    const uint2 v = mm[i];
    kmin = min(kmin, v.x);
    kmax = max(kmax, v.y);
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o, kWave)));
    kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o, kWave)));
  }
  if ((t & (kWave - 1)) == 0) {
    red[t / kWave] = kmin;
    red[4 + t / kWave] = kmax;
  }
  for (int i = t; i < kSelBins; i += 256) hist[i] = 0u;
  __syncthreads();
  kmin = min(min(red[0], red[1]), min(red[2], red[3]));
  kmax = max(max(red[4], red[5]), max(red[6], red[7]));
  if (blk == 0 && t == 0) {
    rng[2 * u] = kmin;
    rng[2 * u + 1] = kmax;
  }
  const EstRange r = est_range(kmin, kmax);
  if (!(r.lo < r.hi)) return;  // every estimate equal: no histogram needed
  const float* e = est + static_cast<size_t>(u) * C + static_cast<size_t>(blk) * kSelBlock;
  const int n = min(kSelBlock, C - blk * kSelBlock);
#pragma unroll
  for (int j = 0; j < kSelBlock / 256; ++j) {
    const int k = j * 256 + t;
    if (k < n) atomicAdd(&hist[range_bin<kSelBins>(e[k], r.lo, r.scale)], 1u);
  }
  __syncthreads();
  uint32_t* out = ehtot + static_cast<size_t>(u) * kSelBins;
  for (int i = t; i < kSelBins; i += 256) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&out[i], c);
  }
}

// Loads the unit's estimate histogram into LDS (NT threads).
template <int NT>
__device__ __forceinline__ void load_hist(const uint32_t* __restrict__ ehtot, int u, uint32_t* hist) {
  const uint4* src = reinterpret_cast<const uint4*>(ehtot + static_cast<size_t>(u) * kSelBins);
  for (int i = threadIdx.x; i < kSelBins / 4; i += NT) reinterpret_cast<uint4*>(hist)[i] = src[i];
  __syncthreads();
}

// Grid (nsb, U), 256 threads.
__global__ __launch_bounds__(256) void cross_kernel(const float* __restrict__ est, int C, int n_sel,
                                                    int nsb, const uint32_t* __restrict__ rng,
                                                    const uint32_t* __restrict__ ehtot,
                                                    int32_t* __restrict__ gtb,
                                                    float* __restrict__ lval,
                                                    int32_t* __restrict__ lidx,
                                                    uint32_t* __restrict__ lcnt) {
  const int blk = blockIdx.x;
  const int u = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  __shared__ uint32_t hist[kSelBins];
  __shared__ unsigned long long sbuf[5];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  const EstRange r = est_range(rng[2 * u], rng[2 * u + 1]);
  if (!(r.lo < r.hi)) return;
  load_hist<256>(ehtot, u, hist);
  crossing_bin<256, kSelBins>(hist, static_cast<uint32_t>(n_sel), sbuf, &s_bin, &s_above);
  const int b1 = s_bin;
  const float* e = est + static_cast<size_t>(u) * C;
  uint32_t gt = 0;
  const unsigned long long below = lanes_below();
#pragma unroll
  for (int j = 0; j < kSelBlock / 256; ++j) {
    const int k = blk * kSelBlock + j * 256 + t;
    float x = 0.f;
    int b = -1;
    if (k < C) {
      x = e[k];
      b = range_bin<kSelBins>(x, r.lo, r.scale);
    }
    gt += b > b1 ? 1u : 0u;
    // members of the crossing bin: one atomic per wave
    const unsigned long long bm = __ballot(b == b1);
    if (bm) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&lcnt[u], static_cast<uint32_t>(__popcll(bm)));
      base = static_cast<uint32_t>(__shfl(static_cast<int>(base), 0, kWave));
      if (b == b1) {
        const uint32_t slot = base + static_cast<uint32_t>(__popcll(bm & below));
        if (slot < static_cast<uint32_t>(C)) {
          lval[static_cast<size_t>(u) * C + slot] = x;
          lidx[static_cast<size_t>(u) * C + slot] = k;
        }
      }
    }
  }
  const uint32_t g = block_sum<256>(gt, reinterpret_cast<uint32_t*>(sbuf));
  if (t == 0) gtb[static_cast<size_t>(u) * nsb + blk] = static_cast<int32_t>(g);
}

// Grid U, 1024 threads.  Members of the crossing bin up to kRankCap are
// ranked directly in LDS; more fall back to value-range refinement and a
// radix select of the last tied index over the member list in memory.
constexpr int kRankCap = kSelBins / 2;

__global__ __launch_bounds__(1024) void thresh_kernel(int C, int n_sel, int nsb,
                                                      const uint32_t* __restrict__ rng,
                                                      const uint32_t* __restrict__ ehtot,
                                                      const int32_t* __restrict__ gtb,
                                                      const float* __restrict__ lval,
                                                      const int32_t* __restrict__ lidx,
                                                      const uint32_t* __restrict__ lcnt,
                                                      int32_t* __restrict__ soff,
                                                      int32_t* __restrict__ selp) {
  constexpr int NT = 1024, NW = NT / kWave, NB = kSelBins;
  const int u = blockIdx.x;
  const int t = threadIdx.x;
  __shared__ uint32_t hist[NB];
  __shared__ uint32_t cntb[kSelMaxBlocks];
  __shared__ float fbuf[NW];
  __shared__ unsigned long long sbuf[NW + 1];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  const EstRange r = est_range(rng[2 * u], rng[2 * u + 1]);
  float T = r.lo;
  int k_tie = n_sel - 1;
  if (r.lo < r.hi) {
    uint32_t rem = static_cast<uint32_t>(n_sel);
    load_hist<NT>(ehtot, u, hist);
    crossing_bin<NT, NB>(hist, rem, sbuf, &s_bin, &s_above);
    rem -= s_above;
    const int m = static_cast<int>(min(lcnt[u], static_cast<uint32_t>(C)));
    const float* lv = lval + static_cast<size_t>(u) * C;
    const int32_t* li = lidx + static_cast<size_t>(u) * C;
    if (m <= kRankCap) {
      // few members (the usual case): copy them to LDS (into the histogram's
      // space) and rank them by (estimate descending, index ascending); the
      // member of rank rem - 1 is the last one taken, so it gives T and the
      // last tied index at once
      float* mv = reinterpret_cast<float*>(hist);
      int32_t* mi = reinterpret_cast<int32_t*>(hist) + kRankCap;
      for (int i = t; i < m; i += NT) {
        mv[i] = lv[i];
        mi[i] = li[i];
      }
      __syncthreads();
      for (int i = t; i < m; i += NT) {
        const float v = mv[i];
        const int k = mi[i];
        uint32_t rank = 0;
        for (int j = 0; j < m; ++j) {
          const float o = mv[j];
          rank += (o > v || (o == v && mi[j] < k)) ? 1u : 0u;
        }
        if (rank == rem - 1) {
          s_bin = k;
          fbuf[0] = v;
        }
      }
      __syncthreads();
      T = fbuf[0];
      k_tie = s_bin;
      for (int i = t; i < nsb; i += NT) cntb[i] = 0u;
      __syncthreads();
      for (int i = t; i < m; i += NT) {
        const float x = mv[i];
        const int k = mi[i];
        if ((x > T || (x == T && k <= k_tie)) && k >= 0 && k < C) atomicAdd(&cntb[k / kSelBlock], 1u);
      }
      __syncthreads();
    } else {
    float nlo = INFINITY, nhi = -INFINITY;
    for (int i = t; i < m; i += NT) {
      const float x = lv[i];
      nlo = x < nlo ? x : nlo;
      nhi = x > nhi ? x : nhi;
    }
    const float lo = block_min<NT>(nlo, fbuf);
    const float hi = block_max<NT>(nhi, fbuf);
    T = refine_range<NT, NB>(lv, m, lo, hi, &rem, hist, fbuf, sbuf, &s_bin, &s_above);
    // the rem-th smallest index among the members equal to T: radix select,
    // 11 + 11 bits (indices are below 2^21 + 2^11)
    uint32_t want = rem, hb = 0;
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 11 : 0;
      for (int i = t; i < 2048; i += NT) hist[i] = 0u;
      __syncthreads();
      for (int i = t; i < m; i += NT) {
        const int k = li[i];
        if (lv[i] == T && (pass == 0 || (static_cast<uint32_t>(k) >> 11) == hb))
          atomicAdd(&hist[(static_cast<uint32_t>(k) >> shift) & 2047u], 1u);
      }
      __syncthreads();
      // ascending crossing: two bins per thread, counts from the bottom
      const uint32_t c0 = hist[2 * t], c1 = hist[2 * t + 1];
      unsigned long long tot;
      const uint32_t below_cnt = static_cast<uint32_t>(
          block_excl_scan<NT>(static_cast<unsigned long long>(c0 + c1), sbuf, &tot));
      if (below_cnt < want && below_cnt + c0 >= want) {
        s_bin = 2 * t;
        s_above = below_cnt;
      } else if (below_cnt + c0 < want && below_cnt + c0 + c1 >= want) {
        s_bin = 2 * t + 1;
        s_above = below_cnt + c0;
      }
      __syncthreads();
      want -= s_above;
      if (pass == 0)
        hb = static_cast<uint32_t>(s_bin);
      else
        k_tie = static_cast<int>((hb << 11) | static_cast<uint32_t>(s_bin));
      __syncthreads();
    }
    // members taken, per block
    for (int i = t; i < nsb; i += NT) cntb[i] = 0u;
    __syncthreads();
    for (int i = t; i < m; i += NT) {
      const float x = lv[i];
      const int k = li[i];
      if ((x > T || (x == T && k <= k_tie)) && k >= 0 && k < C) atomicAdd(&cntb[k / kSelBlock], 1u);
    }
    __syncthreads();
    }
  }
  // output offsets of the blocks (one block per thread)
  const int b = t;
  uint32_t taken = 0;
  if (b < nsb) {
    if (r.lo < r.hi)
      taken = cntb[b] + static_cast<uint32_t>(gtb[static_cast<size_t>(u) * nsb + b]);
    else  // every estimate equal: the first n_sel candidates
      taken = static_cast<uint32_t>(min(max(n_sel - b * kSelBlock, 0), kSelBlock));
  }
  unsigned long long tot;
  const unsigned long long ex =
      block_excl_scan<NT>(static_cast<unsigned long long>(taken), sbuf, &tot);
  if (b < nsb) soff[static_cast<size_t>(u) * nsb + b] = static_cast<int32_t>(ex);
  if (t == 0) {
    selp[2 * u] = __float_as_int(T);
    selp[2 * u + 1] = k_tie;
  }
}

// Grid (max(nsb, 1), U), 256 threads: block blk writes its taken candidates
// in index order (slot j, wave, lane) from its output offset; with n_sel >=
// C every candidate is taken and block blk starts at blk * kSelBlock.  The
// caller's buffer is padded with -1 past n_sel by block 0.
__global__ __launch_bounds__(256) void output_kernel(const float* __restrict__ est,
                                                     const int32_t* __restrict__ cand, int C,
                                                     int n_sel, int k_ret, int first, int nsb,
                                                     const int32_t* __restrict__ soff,
                                                     const int32_t* __restrict__ selp,
                                                     int32_t* __restrict__ sel,
                                                     int32_t* __restrict__ retrieved) {
  constexpr int NW = 256 / kWave, NS = kSelBlock / 256;
  const int blk = blockIdx.x;
  const int u = blockIdx.y;
  const int t = threadIdx.x;
  const int wave = t / kWave;
  const int lane = t & (kWave - 1);
  __shared__ uint32_t cnt[NS * NW];
  const bool all = n_sel >= C;
  float T = 0.f;
  int k_tie = -1, base = blk * kSelBlock;
  if (!all) {
    T = __int_as_float(selp[2 * u]);
    k_tie = selp[2 * u + 1];
    base = soff[static_cast<size_t>(u) * nsb + blk];
  }
  const float* e = est + static_cast<size_t>(u) * C;
  bool take[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int k = blk * kSelBlock + j * 256 + t;
    bool tk = false;
    if (k < C) {
      if (all) {
        tk = true;
      } else {
        const float x = e[k];
        tk = x > T || (x == T && k <= k_tie);
      }
    }
    take[j] = tk;
    const unsigned long long b = __ballot(tk);
    if (lane == 0) cnt[j * NW + wave] = static_cast<uint32_t>(__popcll(b));
  }
  __syncthreads();
  if (t < kWave) {
    const uint32_t c = t < NS * NW ? cnt[t] : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (t < NS * NW) cnt[t] = incl - c;
  }
  __syncthreads();
  int32_t* so = sel + static_cast<size_t>(u) * n_sel;
  int32_t* ro = retrieved ? retrieved + static_cast<size_t>(u) * k_ret : nullptr;
  const unsigned long long below = lanes_below();
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const unsigned long long b = __ballot(take[j]);
    const int off = base + static_cast<int>(cnt[j * NW + wave]) + __popcll(b & below);
    if (take[j] && off < n_sel) {
      const int32_t p = first + cand[static_cast<size_t>(u) * C + blk * kSelBlock + j * 256 + t];
      so[off] = p;
      if (ro) ro[off] = p;
    }
  }
  if (ro && blk == 0)
    for (int j = n_sel + t; j < k_ret; j += 256) ro[j] = -1;
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

// Grid (G, U), d threads: out = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s
// for query head g of unit u.  The maximum and the denominator are reduced
// over the slices in parallel; each thread then sums its column.
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(const float* __restrict__ part, int nsplit,
                                                  int G, int Hq, int Hkv,
                                                  float* __restrict__ out) {
  constexpr int NW = D / kWave;
  const int g = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int c = threadIdx.x;
  __shared__ float buf[NW];
  const size_t stride = static_cast<size_t>(G) * (D + 2);
  const float* p = part + static_cast<size_t>(u) * nsplit * stride + static_cast<size_t>(g) * (D + 2);
  float mx = -INFINITY;
  for (int s = c; s < nsplit; s += D) mx = fmaxf(mx, p[s * stride + D]);
  const float M = block_max<D>(mx, buf);
  float dl = 0.f;
  for (int s = c; s < nsplit; s += D) dl += expf(p[s * stride + D] - M) * p[s * stride + D + 1];
  const float den = block_sum<D>(dl, buf);
  float num = 0.f;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) num += expf(p[s * stride + D] - M) * p[s * stride + c];
  out[(static_cast<size_t>(b) * Hq + static_cast<size_t>(h) * G + g) * D + c] = num / den;
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
    e = launch(query_kernel<DT>, dim3(r->Bs, U), dim3(1024), 0, st, E(0), q, r->Hq, r->Hkv, r->G,
               r->d, r->signs, r->rho, r->qt, r->qn, r->votes, r->tot, r->ehtot, r->lcnt);
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
                 r->cb, r->est, r->rmm);
    else
      e = launch(rerank_kernel<64>, dim3((r->C + 255) / 256, U), dim3(256), 0, st, E(3),
                 static_cast<const uint8_t*>(r->rec), r->N, static_cast<const int32_t*>(r->cand),
                 r->C, static_cast<const double*>(r->qt), static_cast<const double*>(r->qn),
                 r->cb, r->est, r->rmm);
    if (e != hipSuccess) return e;
  }
  if (active && r->n_sel < r->C) {
    e = launch(ehist_kernel, dim3(r->nsb, U), dim3(256), 0, st, E(4),
               static_cast<const float*>(r->est), r->C, r->nrwg,
               static_cast<const uint32_t*>(r->rmm), r->rng, r->ehtot);
    if (e != hipSuccess) return e;
    e = launch(cross_kernel, dim3(r->nsb, U), dim3(256), 0, st, E(5),
               static_cast<const float*>(r->est), r->C, r->n_sel, r->nsb,
               static_cast<const uint32_t*>(r->rng), static_cast<const uint32_t*>(r->ehtot),
               r->gtb, r->lval, r->lidx, r->lcnt);
    if (e != hipSuccess) return e;
    e = launch(thresh_kernel, dim3(U), dim3(1024), 0, st, E(6), r->C, r->n_sel, r->nsb,
               static_cast<const uint32_t*>(r->rng), static_cast<const uint32_t*>(r->ehtot),
               static_cast<const int32_t*>(r->gtb), static_cast<const float*>(r->lval),
               static_cast<const int32_t*>(r->lidx), static_cast<const uint32_t*>(r->lcnt),
               r->soff, r->selp);
    if (e != hipSuccess) return e;
  }
  if (active || (retrieved != nullptr && r->k_ret > 0)) {
    const int Ca = active ? r->C : 0;
    e = launch(output_kernel, dim3(active ? r->nsb : 1, U), dim3(256), 0, st, E(7),
               static_cast<const float*>(r->est), static_cast<const int32_t*>(r->cand), Ca, r->n_sel,
               r->k_ret, r->ns, r->nsb, static_cast<const int32_t*>(r->soff),
               static_cast<const int32_t*>(r->selp), r->sel, retrieved);
    if (e != hipSuccess) return e;
  }
  const T* kn = static_cast<const T*>(r->k_near);
  const T* vn = static_cast<const T*>(r->v_near);
  const T* kf = static_cast<const T*>(r->k_far);
  const T* vf = static_cast<const T*>(r->v_far);
  if (r->d == 128)
    e = launch(attend_kernel<DT, 128>, dim3(r->nsplit, U), dim3(256), 0, st, E(8), q, kn, vn, kf,
               vf, static_cast<const int32_t*>(r->sel), r->Hq, r->Hkv, r->G, r->ns, r->n_sel, r->N,
               r->n_near, r->n_att, r->nsplit, r->part);
  else
    e = launch(attend_kernel<DT, 64>, dim3(r->nsplit, U), dim3(256), 0, st, E(8), q, kn, vn, kf,
               vf, static_cast<const int32_t*>(r->sel), r->Hq, r->Hkv, r->G, r->ns, r->n_sel, r->N,
               r->n_near, r->n_att, r->nsplit, r->part);
  if (e != hipSuccess) return e;
  if (r->d == 128)
    return launch(merge_kernel<128>, dim3(r->G, U), dim3(128), 0, st, E(9),
                  static_cast<const float*>(r->part), r->nsplit, r->G, r->Hq, r->Hkv, out);
  return launch(merge_kernel<64>, dim3(r->G, U), dim3(64), 0, st, E(9),
                static_cast<const float*>(r->part), r->nsplit, r->G, r->Hq, r->Hkv, out);
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
