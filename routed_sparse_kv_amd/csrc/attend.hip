// Mixed-resolution attention (SEKV, Metodologia 3): one softmax over
//   - full-resolution rows (anchors, lead/tail runs, appended tokens) with
//     their exact K/V;
//   - every token of an expanded span, rebuilt from its factors:
//     k-hat_i = A_K[i] W_K, v-hat_i = A_V[i] W_V;
//   - every other span as one entry: key s_j with logit <q, s_j>/sqrt(d) +
//     ln|S_j| (written by the routing pass, -inf once the span is expanded),
//     value the span mean.
//
// The rank-r contraction is applied to the small operands instead of
// materialising K-hat and V-hat:  <q, A_i W_K> = A_i (W_K q)  and
// sum_i p_i A_i W_V = (sum_i p_i A_i) W_V,  the same arithmetic up to
// association, reading every factor exactly once.
//
// bf16 caches, r in {8, 16}: attend_mfma_kernel.  The work items of a unit
// (expanded spans, 32-row full-resolution chunks, 32-span summary chunks)
// are split by the top-k kernel into one contiguous, cost-balanced range
// per wave.  A wave loads each item with MFMA-operand loads from the tiled
// layouts of layout.h, one item ahead of the one it computes, and keeps its
// online-softmax state (max, sum, out^T) in the MFMA accumulator layout; all
// products are 16x16 MFMAs with fp32 accumulation (fp32 intermediates enter
// as a bf16 hi + lo pair).  The workgroup merges its four waves in LDS and
// writes one partial.
//
// Other caches (fp32, or other ranks): attend_valu_kernel, a block-
// cooperative fp32 version of the same computation.
//
// merge_kernel (next launch) combines the partials of a unit with the
// log-sum-exp rule.  Merging inside the attention kernel would need a
// device-scope release per workgroup, which on gfx950 writes back the XCD's
// L2 and serialises across workgroups (measured at the 128K-context shape:
// 150 us per attention launch instead of 54); the kernel boundary is
// cheaper.
#include <stdlib.h>

#include "cache.h"
#include "common.h"
#include "lanes.h"

namespace rskv {
namespace {

constexpr int kAttThreads = 256;
constexpr int kXcds = 8;  // accelerator dies of the device
constexpr int kChunk = 32;
constexpr int kMaxG = 16;
constexpr int kMaxRank = 32;
constexpr int kMaxOut = 8;           // VALU path: outputs per thread, G*d <= 2048
constexpr int kMaxSplitMfma = 256;   // partials per unit of the MFMA path

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8b(const uint16_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ bf16x8 as8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x4 lo4(const u32x4& v) {
  return __builtin_bit_cast(bf16x4, u32x2{v.x, v.y});
}
__device__ __forceinline__ bf16x4 hi4(const u32x4& v) {
  return __builtin_bit_cast(bf16x4, u32x2{v.z, v.w});
}
__device__ __forceinline__ f32x4 asf(const u32x4& v) { return __builtin_bit_cast(f32x4, v); }

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// fp32 x as bf16 hi + lo (hi + lo equals x to ~16 significant bits)
__device__ __forceinline__ void split4(const float* x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 hb = static_cast<__bf16>(x[e]);
    hi[e] = hb;
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(hb));
  }
}
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 hb = static_cast<__bf16>(x[e]);
    hi[e] = hb;
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(hb));
  }
}


// Online-softmax update of a wave for 8 logits per lane (lane: head l % 16,
// rows 4 g + i and 16 + 4 g + i).  Turns x into probabilities relative to
// the new running max and returns the factor that rescales older state.
__device__ __forceinline__ float wave_softmax8(float* x, float& m, float& l) {
  float cm = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) cm = fmaxf(cm, x[e]);
  cm = fmaxf(cm, xor_lane<16>(cm));
  cm = fmaxf(cm, xor_lane<32>(cm));
  const float mn = fmaxf(m, cm);
  const float sc = mn == -INFINITY ? 1.f : __expf(m - mn);
  float ps = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = x[e] == -INFINITY ? 0.f : __expf(x[e] - mn);
    ps += x[e];
  }
  ps += xor_lane<16>(ps);
  ps += xor_lane<32>(ps);
  l = l * sc + ps;
  m = mn;
  return sc;
}

// Loads per work item and register slots (16 bytes per lane each) of the
// MFMA kernel; a wave issues all loads of an item before it waits:
//   full-resolution chunk (32 rows): K as 2 x KK tiles, V as CB tiles;
//   summary chunk (32 spans): CB mean tiles + 2 logit vectors;
//   expanded span: KK W_K rows, CB/2 W_V column pairs, and the first 64 rows
//   of A_K and A_V (4 + 4 eight-byte loads packed two per slot).
template <int D>
struct ItemPlan {
  static constexpr int KK = D / 32;
  static constexpr int CB = D / 16;
  static constexpr int kF = 2 * KK + CB;
  static constexpr int kS = CB + 2;
  static constexpr int kE = KK + CB / 2 + 8;
  static constexpr int NL = kF > kS ? (kF > kE ? kF : kE) : (kS > kE ? kS : kE);
  static constexpr int kEA = KK + CB / 2;  // first A slot of a span item
};

// LDS of the fused variant (spans of one unit held in LDS; indices padded by
// one slot per 16 so that a thread's contiguous run avoids bank conflicts).
constexpr int kFuseSpans = 4096;
constexpr int kFuseSel = 1024;
constexpr int kFusePad = kFuseSpans + kFuseSpans / 16;
__device__ __forceinline__ int pidx(int i) { return i + (i >> 4); }

struct FusedLds {
  union {
    double z[kFusePad];        // selection: routing scores (-inf past the last span)
    int2 elist[kFuseSel];      // item loop: {span, exclusive work-cost prefix}
    float merge[4 * 128 * 16]; // end: per-wave out^T
  };
  int len[kFusePad];
  int tpad[kFusePad];
  int hist[1024];
  unsigned mask[kFuseSpans / 32];  // expanded spans
  int rowcnt[kFuseSpans / 256][4];
  int rowcost[kFuseSpans / 256][4];
  int ired[3][4];
  double dred[2][4];
  double cand_z[256];
  int cand_j[256];
  double s_zs;
  int s_bin, s_above, s_cnt, s_js;
  int s_ncand;  // values gathered for the exact rank (reset with each histogram)
  int rng[5];
};

// Block (4 waves) reductions over the LDS scratch rows; `slot` selects a
// row (consecutive calls use different rows, so a single barrier per call
// suffices).
// Exclusive prefix of v over the block (thread order) and the total.
__device__ __forceinline__ int block4_excl(int v, FusedLds& L, int slot, int* total) {
  const int wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan_dpp(v);
  if ((threadIdx.x & 63) == 63) L.ired[slot][wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int x = L.ired[slot][w];
    before += w < wave ? x : 0;
    tot += x;
  }
  *total = tot;
  return before + incl - v;
}
__device__ __forceinline__ void block4_min_max_f64(double& mn, double& mx, FusedLds& L) {
  const int wave = threadIdx.x >> 6;
  wave_min_max_f64(mn, mx);
  if ((threadIdx.x & 63) == 0) {
    L.dred[0][wave] = mn;
    L.dred[1][wave] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mn = fmin(mn, L.dred[0][w]);
    mx = fmax(mx, L.dred[1][w]);
  }
  __syncthreads();
}

template <int D, int R, bool FUSED>
__global__ __launch_bounds__(kAttThreads) __attribute__((amdgpu_waves_per_eu(2))) void
attend_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kf,
                   const uint16_t* __restrict__ vf, const int32_t* __restrict__ n_full,
                   const uint16_t* __restrict__ vmean, const float* __restrict__ slogit,
                   const int32_t* __restrict__ n_spans, const uint16_t* __restrict__ a_k,
                   const uint16_t* __restrict__ a_v, const uint16_t* __restrict__ w_k,
                   const uint16_t* __restrict__ w_v, const int32_t* __restrict__ sel_desc,
                   const int32_t* __restrict__ n_sel, const int32_t* __restrict__ wstart,
                   const double* __restrict__ z_all, const int32_t* __restrict__ span_len,
                   const int32_t* __restrict__ tok_pad, double tau, int k_max, WorkCost wc,
                   int32_t* __restrict__ sel_out, int32_t* __restrict__ nsel_out, int Hkv,
                   int G, int S, int Sp, int Fp, int Np, int wpitch, int nsplit_max,
                   float inv_sqrt_d, float* __restrict__ part) {
  typedef ItemPlan<D> IP;
  constexpr int KK = IP::KK;
  constexpr int CB = IP::CB;
  constexpr int NL = IP::NL;
  constexpr int R4 = (R + 3) & ~3;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g16 = lane & 15;
  const int grp = lane >> 4;
  // Workgroups reach the XCDs round-robin in linear id order; when the units
  // divide evenly, all workgroups of a unit go to one XCD, whose L2 then
  // serves the unit's shared reads (scores, span tables, queries) once.
  int s = blockIdx.x, u = blockIdx.y;
  if (gridDim.y % kXcds == 0) {
    const int L = blockIdx.x + gridDim.x * blockIdx.y;
    const int m = L / kXcds;
    u = (L % kXcds) * (gridDim.y / kXcds) + m / gridDim.x;
    s = m % gridDim.x;
  }
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const bool head_ok = g16 < G;

  // Q as the B operand: head g16, columns 32 kk + 8 grp + 0..7
  bf16x8 qb[KK];
  {
    const uint16_t* qp = q + (static_cast<size_t>(b) * Hkv * G + static_cast<size_t>(h) * G +
                              (head_ok ? g16 : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qb[kk] = ld8(qp + 32 * kk + 8 * grp);
      if (!head_ok) qb[kk] = bf16x8{};
    }
  }
  float m = -INFINITY, l = 0.f;
  f32x4 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* kf_u = kf + static_cast<size_t>(u) * Fp * D;
  const uint16_t* vf_u = vf + static_cast<size_t>(u) * Fp * D;
  const uint16_t* vm_u = vmean + static_cast<size_t>(u) * Sp * D;
  const float* sl_u = slogit + static_cast<size_t>(u) * Sp * G;
  const uint16_t* ak_u = a_k + static_cast<size_t>(u) * Np * R;
  const uint16_t* av_u = a_v + static_cast<size_t>(u) * Np * R;
  const uint16_t* wk_u = w_k + static_cast<size_t>(u) * S * R * D;
  const uint16_t* wv_u = w_v + static_cast<size_t>(u) * S * D * R4;

  const int nf = n_full[b];
  const int ns = n_spans[b];
  const int nFI = (nf + kChunk - 1) / kChunk;

  // softmax over 8 logits per lane, then acc += V^T p with V the A operand
  auto attend8 = [&](float* x, int r0, int lim, const u32x4* vbuf) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = r0 + (e < 4 ? 4 * grp + e : 16 + 4 * grp + (e - 4));
      if (!head_ok || row >= lim) x[e] = -INFINITY;
    }
    const float sc = wave_softmax8(x, m, l);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] *= sc;
    bf16x8 phi, plo;
    split8(x, phi, plo);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      acc[cb] = mma32(as8(vbuf[cb]), phi, acc[cb]);
      acc[cb] = mma32(as8(vbuf[cb]), plo, acc[cb]);
    }
  };

  // a 32-row full-resolution chunk: K as 2 x KK tiles, V as CB tiles
  auto issue_full = [&](int r0, u32x4* buf) {
    const uint16_t* kt = kf_u + static_cast<size_t>(r0 >> 4) * KK * 512 + lane * 8;
#pragma unroll
    for (int t = 0; t < 2 * KK; ++t) buf[t] = ld16(kt + t * 512);
    const uint16_t* vt = vf_u + static_cast<size_t>(r0 >> 5) * CB * 512 + lane * 8;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) buf[2 * KK + cb] = ld16(vt + cb * 512);
  };
  auto compute_full = [&](int r0, const u32x4* buf) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s0 = mma32(as8(buf[kk]), qb[kk], s0);
      s1 = mma32(as8(buf[KK + kk]), qb[kk], s1);
    }
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = s0[e] * inv_sqrt_d;
      x[4 + e] = s1[e] * inv_sqrt_d;
    }
    attend8(x, r0, nf, buf + 2 * KK);
  };

  // ---- expanded spans and this wave's item range
  __shared__ __align__(16) unsigned char lds_raw[FUSED ? sizeof(FusedLds) : 4 * (2 * 16 + D * 16) * 4];
  int nsel, i0, i1;
  int fb = 0;  // first full-resolution chunk that belongs to the item ranges
  // Fused variant: every full-resolution chunk is assigned statically (wave
  // w of the unit takes chunks w, w + W, ...) and processed between the
  // selection steps, each step computing the chunk whose loads are in
  // flight and issuing the next; the cost-balanced ranges cover the
  // expanded spans and the summary chunks.
  const int wglob = 4 * s + wave;
  const int Wu = 4 * static_cast<int>(gridDim.x);
  const int nfr = FUSED && wglob < nFI ? (nFI - 1 - wglob) / Wu + 1 : 0;
  int fr = 0;  // next of this wave's chunks to compute
  u32x4 pbuf[2 * KK + CB];
  auto f_step = [&]() {
    if (fr < nfr) {
      compute_full((wglob + fr * Wu) * kChunk, pbuf);
      ++fr;
      if (fr < nfr) issue_full((wglob + fr * Wu) * kChunk, pbuf);
    }
  };
  if constexpr (FUSED) {
    // Selection of the unit by the same rule as the top-k kernel (the kept
    // set is fixed by its last entry (z*, j*)), compaction with work costs,
    // and the cost-balanced ranges of this workgroup's four waves.  Thread
    // t owns spans t + 256 k (k < 16) and keeps their scores and lengths in
    // registers; ordering by (k, t) is ordering by span index.
    FusedLds& L = *reinterpret_cast<FusedLds*>(lds_raw);
    const double* z_u = z_all + static_cast<size_t>(u) * S;
    const int32_t* len_b = span_len + static_cast<size_t>(b) * S;
    const int32_t* tp_b = tok_pad + static_cast<size_t>(b) * (S + 1);
    constexpr int KR = kFuseSpans / kAttThreads;
    // a pass loads this thread's scores from LDS (16 batched reads); they
    // are dead between passes, where the chunk computations run
    auto load_z = [&](double* zr) {
#pragma unroll
      for (int k = 0; k < KR; ++k) zr[k] = L.z[pidx(tid + kAttThreads * k)];
    };
    // candidates z > tau: count and value range (padding slots hold -inf)
    int c_loc = 0;
    double lo = INFINITY, hi = -INFINITY;
    {
      double zr[KR];
      int lr[KR], tr[KR];
      // slots past the last span read span 0 and hold z = -inf (no branch)
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const int i = tid + kAttThreads * k;
        const int ic = i < ns ? i : 0;
        zr[k] = z_u[ic];
        lr[k] = len_b[ic];
        tr[k] = tp_b[ic];
      }
#pragma unroll
      for (int k = 0; k < KR; ++k)
        if (tid + kAttThreads * k >= ns) zr[k] = -INFINITY;
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        if (zr[k] > tau) {
          ++c_loc;
          lo = fmin(lo, zr[k]);
          hi = fmax(hi, zr[k]);
        }
      }
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const int i = tid + kAttThreads * k;  // < kFuseSpans
        L.z[pidx(i)] = zr[k];
        L.len[pidx(i)] = lr[k];
        L.tpad[pidx(i)] = tr[k];
      }
      // the first chunk of this wave is in flight while the workgroup
      // selects; it is issued once the scores have arrived (issued earlier,
      // it delays them), unconditionally (a wave without chunks re-reads the
      // last one and drops it)
      issue_full(min(wglob, max(nFI, 1) - 1) * kChunk, pbuf);
    }
    // Position in index order of this thread's flagged slots: ballots per
    // slot row, wave totals in LDS, one barrier.  Returns the count before
    // slot k of this thread through base[k] and the total.
    const unsigned long long below = (1ull << lane) - 1ull;
    auto order_prefix = [&](const bool* flag, int* base, int* total) {
      unsigned long long bal[KR];
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        bal[k] = __ballot(flag[k]);
        if (lane == 0) L.rowcnt[k][wave] = __popcll(bal[k]);
      }
      __syncthreads();
      int run = 0;
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        int before_w = 0, row = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int c = L.rowcnt[k][w];
          before_w += w < wave ? c : 0;
          row += c;
        }
        base[k] = run + before_w + __popcll(bal[k] & below);
        run += row;
      }
      *total = run;
      __syncthreads();
    };
    // Bin bs holds the k-th largest and cb <= 256 values: rank them exactly,
    // (z descending, index ascending); the one of rank rem - 1 is the last
    // kept entry (z*, j*).
    auto rank_bin = [&](const double* zr, const int* bin, int bs, int cb, int rem, double& zs_,
                        int& js_) {
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        if (bin[k] == bs) {
          const int slot = atomicAdd(&L.s_ncand, 1);
          if (slot < kAttThreads) {
            L.cand_z[slot] = zr[k];
            L.cand_j[slot] = tid + kAttThreads * k;
          }
        }
      }
      __syncthreads();
      if (tid < cb) {
        const double v = L.cand_z[tid];
        const int j = L.cand_j[tid];
        int rank = 0;
        for (int y = 0; y < cb; ++y) {
          const double vy = L.cand_z[y];
          rank += (vy > v || (vy == v && L.cand_j[y] < j)) ? 1 : 0;
        }
        if (rank == rem - 1) {
          L.s_zs = v;
          L.s_js = j;
        }
      }
      __syncthreads();
      zs_ = L.s_zs;
      js_ = L.s_js;
    };
    // the bin holding the rem-th largest among the 1024 counts c (thread t
    // holds bins 1023 - 4t .. 1020 - 4t, highest first): sets s_bin,
    // s_above (values in higher bins) and s_cnt
    auto find_bin = [&](const int* c4, int rem, int* total) {
      const int cs = c4[0] + c4[1] + c4[2] + c4[3];
      const int above = block4_excl(cs, L, 1, total);
      if (above < rem && rem <= above + cs) {
        int a2 = above;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          if (a2 < rem && rem <= a2 + c4[x]) {
            L.s_bin = 1023 - 4 * tid - x;
            L.s_above = a2;
            L.s_cnt = c4[x];
          }
          a2 += c4[x];
        }
      }
      __syncthreads();
    };
    int n_cand;
    {
      const int cw = __builtin_amdgcn_readlane(wave_incl_scan_dpp(c_loc), 63);
      wave_min_max_f64(lo, hi);
      if (lane == 0) {
        L.ired[0][wave] = cw;
        L.dred[0][wave] = lo;
        L.dred[1][wave] = hi;
      }
      __syncthreads();
      n_cand = L.ired[0][0] + L.ired[0][1] + L.ired[0][2] + L.ired[0][3];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        lo = fmin(lo, L.dred[0][w]);
        hi = fmax(hi, L.dred[1][w]);
      }
    }
    double zs = INFINITY;  // pick: z > tau && (z > zs || (z == zs && j <= js))
    int js = -1;
    if (k_max > 0 && n_cand > 0) {
      if (n_cand <= k_max) {
        zs = -INFINITY;  // every candidate
      } else {
        int rem = k_max;  // entries still to take from [lo, hi]
        // narrow [lo, hi] with 1024-bin histograms of the values in it until
        // the bin holding the rem-th largest has few enough values to rank
        for (int round = 0; round < 256; ++round) {
          double zr[KR];
          load_z(zr);
          if (lo == hi) {
            // rem lowest indices among the values equal to lo
            bool f[KR];
            int base[KR], tot;
#pragma unroll
            for (int k = 0; k < KR; ++k) f[k] = zr[k] == lo;
            order_prefix(f, base, &tot);
#pragma unroll
            for (int k = 0; k < KR; ++k)
              if (f[k] && base[k] == rem - 1) L.s_js = tid + kAttThreads * k;
            __syncthreads();
            zs = lo;
            js = L.s_js;
            break;
          }
          // 1024 bins over [lo, hi]: any map that is monotone in z gives an
          // exact answer; fp32 arithmetic is used unless the range is too
          // small for it, where fp64 division takes over (a uniform branch,
          // so only one of the two formulas is executed)
          const double w = hi - lo;
          const float wf = static_cast<float>(w);
          const bool f32ok = wf > 1e-30f;
          const float sr = 1024.f / wf;
          int bin[KR];  // -1 outside [lo, hi]
          if (f32ok) {
#pragma unroll
            for (int k = 0; k < KR; ++k)
              bin[k] = (zr[k] >= lo && zr[k] <= hi)
                           ? min(1023, static_cast<int>(static_cast<float>(zr[k] - lo) * sr))
                           : -1;
          } else {
#pragma unroll
            for (int k = 0; k < KR; ++k)
              bin[k] = (zr[k] >= lo && zr[k] <= hi)
                           ? min(1023, static_cast<int>((zr[k] - lo) / w * 1024.0))
                           : -1;
          }
          for (int x = tid; x < 1024; x += kAttThreads) L.hist[x] = 0;
          if (tid == 0) L.s_ncand = 0;
          __syncthreads();
#pragma unroll
          for (int k = 0; k < KR; ++k)
            if (bin[k] >= 0) atomicAdd(&L.hist[bin[k]], 1);
          __syncthreads();
          int c4[4], tot;
#pragma unroll
          for (int x = 0; x < 4; ++x) c4[x] = L.hist[1023 - 4 * tid - x];
          find_bin(c4, rem, &tot);
          const int bs = L.s_bin;
          rem -= L.s_above;
          const int cb = L.s_cnt;
          if (cb <= kAttThreads) {
            rank_bin(zr, bin, bs, cb, rem, zs, js);
            break;
          }
          // many values left: narrow to their range and repeat
          double nlo = INFINITY, nhi = -INFINITY;
#pragma unroll
          for (int k = 0; k < KR; ++k) {
            if (bin[k] == bs) {
              nlo = fmin(nlo, zr[k]);
              nhi = fmax(nhi, zr[k]);
            }
          }
          block4_min_max_f64(nlo, nhi, L);
          lo = nlo;
          hi = nhi;
        }
      }
    }
    f_step();
    // compaction in index order: per slot row a ballot; lane k of each
    // wave turns the row counts into the wave's base position for row k
    unsigned pm = 0u;  // picked slots of this thread
    {
      double zr[KR];
      load_z(zr);
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const int i = tid + kAttThreads * k;
        if (zr[k] > tau && (zr[k] > zs || (zr[k] == zs && i <= js))) pm |= 1u << k;
      }
    }
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const unsigned long long bal = __ballot((pm >> k) & 1u);
      if (lane == 0) L.rowcnt[k][wave] = __popcll(bal);
    }
    __syncthreads();
    int rbase = 0;  // lane k < KR: slots of rows < k plus earlier waves of row k
    {
      int rowtot = 0, before_w = 0;
      if (lane < KR) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int c = L.rowcnt[lane][w];
          rowtot += c;
          before_w += w < wave ? c : 0;
        }
      }
      const int incl = wave_incl_scan_dpp(rowtot);
      rbase = incl - rowtot + before_w;
      nsel = __builtin_amdgcn_readlane(incl, KR - 1);
    }
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const bool f = (pm >> k) & 1u;
      const unsigned long long bal = __ballot(f);
      const int base = __builtin_amdgcn_readlane(rbase, k);
      if (f) L.elist[base + __popcll(bal & below)].x = tid + kAttThreads * k;
      // the row's ballot is the bitmask of spans 256 k + 64 wave .. +63
      if (lane == 0) {
        const int w0 = (kAttThreads * k + kWave * wave) >> 5;
        L.mask[w0] = static_cast<unsigned>(bal);
        L.mask[w0 + 1] = static_cast<unsigned>(bal >> 32);
      }
    }
    __syncthreads();
    // exclusive work-cost prefix over the list (4 consecutive entries per
    // thread; nsel <= 1024)
    int e_cost;
    {
      const int q0 = 4 * tid;
      int c4[4], csum = 0;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        c4[x] = q0 + x < nsel ? wc.span(L.len[pidx(L.elist[q0 + x].x)]) : 0;
        csum += c4[x];
      }
      int pre = block4_excl(csum, L, 2, &e_cost);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if (q0 + x < nsel) L.elist[q0 + x].y = pre;
        pre += c4[x];
      }
    }
    fb = nFI;  // every chunk is assigned statically
    const int nFP = nFI - fb;
    const int nSI = (ns + kChunk - 1) / kChunk;
    const int NI = nsel + nFP + nSI;  // items of the ranges
    if (tid < 5) L.rng[tid] = NI;     // (boundaries no item reaches)
    __syncthreads();
    if (s == 0) {
      if (sel_out != nullptr)
        for (int i = tid; i < k_max; i += kAttThreads)
          sel_out[static_cast<size_t>(u) * k_max + i] = i < nsel ? L.elist[i].x : -1;
      if (nsel_out != nullptr && tid == 0) nsel_out[u] = nsel;
    }
    f_step();
    // Ranges of the remaining items [expanded spans | chunks fb.. | summary
    // chunks]: item i goes to wave floor((2 P_i + c_i) W / (2 C)), so the
    // first item of wave w is the first i with (2 P_i + c_i) W >= 2 C w;
    // each thread tests its items against the five boundaries of this
    // workgroup.
    const long long W = 4ll * gridDim.x;
    {
      const long long C = static_cast<long long>(e_cost) + static_cast<long long>(nFP) * wc.full +
                          static_cast<long long>(nSI) * wc.summ;
      auto mid2 = [&](int i) -> long long {  // 2 P_i + c_i
        if (i < nsel) {
          const int2 e = L.elist[i];
          return 2ll * e.y + wc.span(L.len[pidx(e.x)]);
        }
        if (i < nsel + nFP)
          return 2ll * (e_cost + static_cast<long long>(i - nsel) * wc.full) + wc.full;
        return 2ll * (e_cost + static_cast<long long>(nFP) * wc.full +
                      static_cast<long long>(i - nsel - nFP) * wc.summ) + wc.summ;
      };
      for (int i = tid; i < NI; i += kAttThreads) {
        const long long mi = mid2(i) * W;
        const long long mp = i > 0 ? mid2(i - 1) * W : -1;
#pragma unroll
        for (int k = 0; k < 5; ++k) {
          const long long t = 2 * C * (4ll * s + k);
          if (mp < t && t <= mi) L.rng[k] = i;
        }
      }
      __syncthreads();
    }
    i0 = L.rng[wave];
    i1 = L.rng[wave + 1];
  } else {
    nsel = n_sel[u];
    const int* ws = wstart + static_cast<size_t>(u) * wpitch + s * 4 + wave;
    i0 = ws[0];
    i1 = ws[1];
  }
  const int nFP = nFI - fb;  // full-resolution chunks inside the item ranges
  const int4* desc_u = reinterpret_cast<const int4*>(sel_desc) + static_cast<size_t>(u) * S;

  // lane-constant parts of the span addresses (ranks past R read rank 0 and
  // are zeroed after the load)
  const bool krow_ok = g16 < R;        // W_K row / A_V rank held by this lane
  const bool kgrp_ok = grp < R / 4;    // ranks 4 grp..4 grp+3 exist
  const int wk_lane = (krow_ok ? g16 : 0) * D + 8 * grp;
  const int wv_lane = (g16 * (R4 / 4) + (grp < R4 / 4 ? grp : 0)) * 8;
  const int ak_lane = g16 * R + 4 * (kgrp_ok ? grp : 0);
  const int av_lane = (krow_ok ? g16 : 0) * 16 + 4 * grp;

  auto issue = [&](int i, const int4& dsc, u32x4 (&buf)[NL]) {
    if (i < nsel) {
      const int j = dsc.x;
      const int len = dsc.y;
      const int tp = dsc.z;
      const uint16_t* wk = wk_u + static_cast<size_t>(j) * R * D + wk_lane;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) buf[kk] = ld16(wk + 32 * kk);
      const uint16_t* wv = wv_u + static_cast<size_t>(j) * D * R4 + wv_lane;
#pragma unroll
      for (int p = 0; p < CB / 2; ++p) buf[KK + p] = ld16(wv + p * 32 * R4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 16 * t < len ? 16 * t : 0;
        const u32x2 k2 = ld8b(ak_u + static_cast<size_t>(tp + r) * R + ak_lane);
        const u32x2 v2 = ld8b(av_u + static_cast<size_t>((tp + r) >> 4) * R * 16 + av_lane);
        u32x4& ks = buf[IP::kEA + t / 2];
        u32x4& vs = buf[IP::kEA + 2 + t / 2];
        if (t & 1) {
          ks.z = k2.x;
          ks.w = k2.y;
          vs.z = v2.x;
          vs.w = v2.y;
        } else {
          ks.x = k2.x;
          ks.y = k2.y;
          vs.x = v2.x;
          vs.y = v2.y;
        }
      }
    } else if (i < nsel + nFP) {
      issue_full((i - nsel + fb) * kChunk, buf);
    } else {
      const int r0 = (i - nsel - nFP) * kChunk;
      const uint16_t* vt = vm_u + static_cast<size_t>(r0 >> 5) * CB * 512 + lane * 8;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) buf[cb] = ld16(vt + cb * 512);
      const float* lp = sl_u + (static_cast<size_t>(r0 >> 4) * G + (head_ok ? g16 : 0)) * 16 + 4 * grp;
      buf[CB] = *reinterpret_cast<const u32x4*>(lp);
      buf[CB + 1] = *reinterpret_cast<const u32x4*>(lp + G * 16);
    }
  };

  auto compute = [&](int i, const int4& dsc, const u32x4 (&buf)[NL], const unsigned* xmask) {
    if (i < nsel) {
      // ---- expanded span: logits A_K (W_K q), softmax, w += A_V^T p,
      // then out^T += W_V^T w
      const int j = dsc.x;
      const int len = dsc.y;
      const int tp = dsc.z;
      (void)j;
      f32x4 uk = {0.f, 0.f, 0.f, 0.f};  // uk[k = 4 grp + i][head]
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        bf16x8 w8 = as8(buf[kk]);
        if (!krow_ok) w8 = bf16x8{};
        uk = mma32(w8, qb[kk], uk);
      }
      bf16x4 uhi, ulo;
      {
        float t4[4] = {uk[0], uk[1], uk[2], uk[3]};
        split4(t4, uhi, ulo);
      }
      f32x4 wacc = {0.f, 0.f, 0.f, 0.f};  // w[k = 4 grp + i][head]
      auto chunk = [&](int t0, bf16x4 ak0, bf16x4 ak1, bf16x4 av0, bf16x4 av1) {
        f32x4 sv0 = mma16(ak0, uhi, f32x4{0.f, 0.f, 0.f, 0.f});
        sv0 = mma16(ak0, ulo, sv0);
        f32x4 sv1 = mma16(ak1, uhi, f32x4{0.f, 0.f, 0.f, 0.f});
        sv1 = mma16(ak1, ulo, sv1);
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = (head_ok && t0 + 4 * grp + e < len) ? sv0[e] * inv_sqrt_d : -INFINITY;
          x[4 + e] = (head_ok && t0 + 16 + 4 * grp + e < len) ? sv1[e] * inv_sqrt_d : -INFINITY;
        }
        const float sc = wave_softmax8(x, m, l);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[cb] *= sc;
        wacc *= sc;
        bf16x4 phi, plo;
        split4(x, phi, plo);
        wacc = mma16(av0, phi, wacc);
        wacc = mma16(av0, plo, wacc);
        split4(x + 4, phi, plo);
        wacc = mma16(av1, phi, wacc);
        wacc = mma16(av1, plo, wacc);
      };
      auto tile_k = [&](const u32x4& v, int half, int t) {
        bf16x4 r = half ? hi4(v) : lo4(v);
        if (!kgrp_ok || 16 * t >= len) r = bf16x4{};
        return r;
      };
      auto tile_v = [&](const u32x4& v, int half, int t) {
        bf16x4 r = half ? hi4(v) : lo4(v);
        if (!krow_ok || 16 * t >= len) r = bf16x4{};
        return r;
      };
      chunk(0, tile_k(buf[IP::kEA], 0, 0), tile_k(buf[IP::kEA], 1, 1),
            tile_v(buf[IP::kEA + 2], 0, 0), tile_v(buf[IP::kEA + 2], 1, 1));
      if (len > 32)
        chunk(32, tile_k(buf[IP::kEA + 1], 0, 2), tile_k(buf[IP::kEA + 1], 1, 3),
              tile_v(buf[IP::kEA + 3], 0, 2), tile_v(buf[IP::kEA + 3], 1, 3));
      if (len > 64) {
        // rows past 64: 32 at a time, one group of loads kept in flight
        auto load_a = [&](int t0, bf16x4* ak, bf16x4* av) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bool ok = t0 + 16 * t < len;
            const int r = ok ? t0 + 16 * t : t0;
            ak[t] = __builtin_bit_cast(bf16x4, ld8b(ak_u + static_cast<size_t>(tp + r) * R + ak_lane));
            av[t] = __builtin_bit_cast(bf16x4, ld8b(av_u + static_cast<size_t>((tp + r) >> 4) * R * 16 + av_lane));
            if (!ok || !kgrp_ok) ak[t] = bf16x4{};
            if (!ok || !krow_ok) av[t] = bf16x4{};
          }
        };
        bf16x4 akc[2], avc[2], akn[2], avn[2];
        load_a(64, akc, avc);
        for (int t0 = 64; t0 < len; t0 += kChunk) {
          load_a(t0 + kChunk < len ? t0 + kChunk : t0, akn, avn);
          chunk(t0, akc[0], akc[1], avc[0], avc[1]);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            akc[t] = akn[t];
            avc[t] = avn[t];
          }
        }
      }
      bf16x4 whi, wlo;
      {
        float t4[4] = {wacc[0], wacc[1], wacc[2], wacc[3]};
        split4(t4, whi, wlo);
      }
#pragma unroll
      for (int p = 0; p < CB / 2; ++p) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x4 wv4 = hh ? hi4(buf[KK + p]) : lo4(buf[KK + p]);
          if (!kgrp_ok) wv4 = bf16x4{};
          acc[2 * p + hh] = mma16(wv4, whi, acc[2 * p + hh]);
          acc[2 * p + hh] = mma16(wv4, wlo, acc[2 * p + hh]);
        }
      }
    } else if (i < nsel + nFP) {
      // ---- 32 full-resolution rows
      compute_full((i - nsel + fb) * kChunk, buf);
    } else {
      // ---- 32 summary entries (expanded spans enter through their tokens)
      const int r0 = (i - nsel - nFP) * kChunk;
      const f32x4 l0 = asf(buf[CB]);
      const f32x4 l1 = asf(buf[CB + 1]);
      const unsigned xm = xmask != nullptr ? xmask[r0 >> 5] : 0u;
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = (xm >> (4 * grp + e)) & 1u ? -INFINITY : l0[e];
        x[4 + e] = (xm >> (16 + 4 * grp + e)) & 1u ? -INFINITY : l1[e];
      }
      attend8(x, r0, ns, buf);
    }
  };

  while (fr < nfr) f_step();

  // Item loop: all loads of an item are issued before any of them is
  // waited for.
  if (i0 < i1) {
    if constexpr (FUSED) {
      const FusedLds& L = *reinterpret_cast<const FusedLds*>(lds_raw);
      for (int i = i0; i < i1; ++i) {
        int4 dc = make_int4(0, 0, 0, 0);
        if (i < nsel) {
          const int j = L.elist[i].x;
          dc = make_int4(j, L.len[pidx(j)], L.tpad[pidx(j)], 0);
        }
        u32x4 buf[NL];
        issue(i, dc, buf);
        __builtin_amdgcn_sched_barrier(0);
        compute(i, dc, buf, L.mask);
      }
    } else {
      // the next span descriptor is fetched (scalar) while an item is in flight
      auto desc_at = [&](int i) { return i < nsel ? desc_u[i] : make_int4(0, 0, 0, 0); };
      int4 dn = desc_at(i0);
      for (int i = i0; i < i1; ++i) {
        const int4 dc = dn;
        dn = desc_at(min(i + 1, i1 - 1));
        u32x4 buf[NL];
        issue(i, dc, buf);
        __builtin_amdgcn_sched_barrier(0);
        compute(i, dc, buf, static_cast<const unsigned*>(nullptr));
      }
    }
  }

  // ---- merge the four waves of the workgroup in LDS, write one partial
  float (*sm_m)[16] = reinterpret_cast<float (*)[16]>(
      lds_raw + (FUSED ? offsetof(FusedLds, hist) : 0));
  float (*sm_l)[16] = sm_m + 4;
  float* sm_buf = FUSED ? reinterpret_cast<float*>(lds_raw)
                        : reinterpret_cast<float*>(lds_raw) + 2 * 4 * 16;
  if constexpr (FUSED) __syncthreads();  // the span list is no longer read
  if (grp == 0) {
    sm_m[wave][g16] = m;
    sm_l[wave][g16] = l;
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_buf[(wave * D + 16 * cb + 4 * grp + i) * 16 + g16] = acc[cb][i];
  __syncthreads();
  const size_t ps = static_cast<size_t>(G) * (D + 2);
  float* Pb = part + (static_cast<size_t>(u) * nsplit_max + s) * ps;
  for (int o = tid; o < G * D; o += kAttThreads) {
    const int g = o / D;
    const int c = o - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][g]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = __expf(sm_m[w][g] - M);
        num += f * sm_buf[(w * D + c) * 16 + g];
        den += f * sm_l[w][g];
      }
    }
    Pb[g * (D + 2) + 2 + c] = num;
    if (c == 0) {
      Pb[g * (D + 2)] = M;
      Pb[g * (D + 2) + 1] = den;
    }
  }
}

// ------------------------------------------------------------------------
// fp32 (and any-rank) path: block-cooperative fp32 attention

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
__global__ __launch_bounds__(kAttThreads) void attend_valu_kernel(
    const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ kf,
    const typename Elem<DT>::T* __restrict__ vf, const int32_t* __restrict__ n_full,
    const typename Elem<DT>::T* __restrict__ vmean, const float* __restrict__ slogit,
    const int32_t* __restrict__ n_spans, const typename Elem<DT>::T* __restrict__ a_k,
    const typename Elem<DT>::T* __restrict__ a_v, const typename Elem<DT>::T* __restrict__ w_k,
    const typename Elem<DT>::T* __restrict__ w_v, const int32_t* __restrict__ span_len,
    const int32_t* __restrict__ tok_pad, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ n_sel, int Hkv, int G, int d, int S, int Sp, int Fp, int Np,
    int rank, int nsplit, int nsplit_max, float inv_sqrt_d, float* __restrict__ part) {
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
  const int nFI = (nf + kChunk - 1) / kChunk;
  const int nSI = (ns + kChunk - 1) / kChunk;
  const int NI = nFI + nsel + nSI;
  const size_t fbase = static_cast<size_t>(u) * Fp * d;
  const size_t sbase = static_cast<size_t>(u) * Sp * d;
  const float* sl_u = slogit + static_cast<size_t>(u) * Sp * G;

  for (int it = s; it < NI; it += nsplit) {
    if (it < nFI) {
      // ---------------- full-resolution rows r0 .. r0+31
      const int r0 = it * kChunk;
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
          for (int e = 0; e < cpl; ++e) {
            const int c = p * cpl + e;
            const float kv = E::ld(kf, fbase + k16_off(row, c, d));
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
      const int nr = min(kChunk, nf - r0);
#pragma unroll
      for (int oi = 0; oi < kMaxOut; ++oi) {
        const int o = tid + oi * kAttThreads;
        if (o < nout) {
          const int g = o / d;
          const int c = o - g * d;
          float a = acc[oi] * st.sc[g];
          for (int i = 0; i < nr; ++i) a += lg[i][g] * E::ld(vf, fbase + v32_off(r0 + i, c, d));
          acc[oi] = a;
        }
      }
      __syncthreads();
    } else if (it < nFI + nsel) {
      // ---------------- expanded span sel[e], rebuilt from its factors
      const int j = sel[static_cast<size_t>(u) * S + (it - nFI)];
      const int len = span_len[static_cast<size_t>(b) * S + j];
      const int tp = tok_pad[static_cast<size_t>(b) * (S + 1) + j];
      const size_t abase = static_cast<size_t>(u) * Np * rank;
      const size_t wkbase = (static_cast<size_t>(u) * S + j) * rank * d;
      const size_t wvbase = static_cast<size_t>(u) * S * d * rank4(rank);
      for (int pi = tid; pi < G * rank; pi += kAttThreads) {
        const int g = pi / rank;
        const int k = pi - g * rank;
        float a = 0.f;
        for (int c = 0; c < d; ++c) a += E::ld(w_k, wkbase + static_cast<size_t>(k) * d + c) * qs[g][c];
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
            const size_t arow = abase + static_cast<size_t>(tp + t) * rank;
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
          for (int i = 0; i < nr; ++i)
            a += lg[i][g] * E::ld(a_v, abase + avt_off(tp + i0 + i, k, rank));
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
          for (int k = 0; k < rank; ++k) a += wv[g][k] * E::ld(w_v, wvbase + wvt_off(j, k, c, d, rank));
          acc[oi] = a;
        }
      }
      __syncthreads();
    } else {
      // ---------------- unexpanded spans j0 .. j0+31 (summary entries)
      const int j0 = (it - nFI - nsel) * kChunk;
      for (int pi = tid; pi < kChunk * G; pi += kAttThreads) {
        const int i = pi / G;
        const int g = pi - i * G;
        const int j = j0 + i;
        lg[i][g] = j < ns ? sl_u[slogit_off(j, g, G)] : -INFINITY;
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
            if (p != 0.f) a += p * E::ld(vmean, sbase + v32_off(j0 + i, c, d));
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
// One workgroup per (unit, query head).  The split weights e^{m_s - M} and
// the denominator are formed once in LDS; thread c then sums its column over
// the splits with independent loads.
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part, int nsplit,
                                                    int nsplit_max, int Hkv, int G, int d,
                                                    float* __restrict__ out) {
  const int u = blockIdx.x;
  const int g = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int tid = threadIdx.x;

  const size_t ps = static_cast<size_t>(G) * (d + 2);
  const float* P = part + static_cast<size_t>(u) * nsplit_max * ps + static_cast<size_t>(g) * (d + 2);
  __shared__ float w[kMaxSplitMfma > 2048 ? kMaxSplitMfma : 2048];
  __shared__ float red[2];
  // max over splits
  float M = -INFINITY;
  for (int s = tid; s < nsplit; s += blockDim.x) {
    const float m = P[s * ps];
    w[s] = m;
    M = fmaxf(M, m);
  }
  M = wave_max(M);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  __syncthreads();
  float den = 0.f;
  for (int s = tid; s < nsplit; s += blockDim.x) {
    const float f = (M == -INFINITY || w[s] == -INFINITY) ? 0.f : expf(w[s] - M);
    w[s] = f;
    den += f * P[s * ps + 1];
  }
  den = wave_sum(den);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = den;
  __syncthreads();
  den = red[0] + red[1];
  for (int c = tid; c < d; c += blockDim.x) {
    float num = 0.f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) num += w[s] * P[s * ps + 2 + c];
    out[(static_cast<size_t>(b) * Hkv * G + static_cast<size_t>(h) * G + g) * d + c] =
        den > 0.f ? num / den : 0.f;
  }
}

bool use_mfma(const rskv_cache* c) {
  return c->dtype == kBF16 && (c->rank == 8 || c->rank == 16) && (c->d == 64 || c->d == 128);
}

template <int D, int R>
hipError_t attend_mfma_impl(const rskv_cache* c, const DecodeWs& ws, const void* q, int nsplit,
                            const SelectArgs* sa, hipStream_t st, const KernelEvents* ev) {
  dim3 grid(nsplit, c->B * c->Hkv);
  const WorkCost wc = work_cost(c);
  const double tau = sa ? static_cast<double>(sa->tau) : 0.0;
  const int k_max = sa ? sa->k_max : 0;
  int32_t* so = sa ? sa->sel_out : nullptr;
  int32_t* no = sa ? sa->nsel_out : nullptr;
  auto kern = sa ? attend_mfma_kernel<D, R, true> : attend_mfma_kernel<D, R, false>;
  return launch(kern, grid, dim3(kAttThreads), 0, st, ev, static_cast<const uint16_t*>(q),
                static_cast<const uint16_t*>(c->dev.k_full),
                static_cast<const uint16_t*>(c->dev.v_full), c->dev.n_full,
                static_cast<const uint16_t*>(c->dev.vmean), ws.slogit, c->dev.n_spans,
                static_cast<const uint16_t*>(c->dev.a_k), static_cast<const uint16_t*>(c->dev.a_v),
                static_cast<const uint16_t*>(c->dev.w_k), static_cast<const uint16_t*>(c->dev.w_v),
                ws.sel_desc, ws.n_sel, ws.wstart, ws.z, c->dev.span_len, c->dev.tok_pad, tau,
                k_max, wc, so, no, c->Hkv, c->G, c->S, c->Sp, c->Fp, c->Np,
                4 * c->nsplit_max + 1, c->nsplit_max, 1.0f / sqrtf(static_cast<float>(D)),
                ws.part);
}

template <int DT>
hipError_t attend_valu_impl(const rskv_cache* c, const DecodeWs& ws, const void* q, int nsplit,
                            hipStream_t st, const KernelEvents* ev) {
  typedef typename Elem<DT>::T T;
  dim3 grid(nsplit, c->B * c->Hkv);
  return launch(attend_valu_kernel<DT>, grid, dim3(kAttThreads), 0, st, ev,
                static_cast<const T*>(q), static_cast<const T*>(c->dev.k_full),
                static_cast<const T*>(c->dev.v_full), c->dev.n_full,
                static_cast<const T*>(c->dev.vmean), ws.slogit, c->dev.n_spans,
                static_cast<const T*>(c->dev.a_k), static_cast<const T*>(c->dev.a_v),
                static_cast<const T*>(c->dev.w_k), static_cast<const T*>(c->dev.w_v),
                c->dev.span_len, c->dev.tok_pad, ws.sel, ws.n_sel, c->Hkv, c->G, c->d,
                c->S, c->Sp, c->Fp, c->Np, c->rank, nsplit, c->nsplit_max,
                1.0f / sqrtf(static_cast<float>(c->d)), ws.part);
}

}  // namespace

bool attend_uses_mfma(const rskv_cache* c) { return use_mfma(c); }

bool attend_fuses_topk(const rskv_cache* c, int k_max) {
  const int k_slots = k_max < c->S ? k_max : c->S;
  return use_mfma(c) && c->S <= kFuseSpans && k_slots <= kFuseSel;
}

// Work cost model of the attention items (64-byte units): bytes an item
// reads plus a fixed per-item overhead, plus one load round trip for every
// 32 rows of a span past the 64 loaded with its factor matrices.
WorkCost work_cost(const rskv_cache* c) {
  constexpr int kItemOverhead = 16;
  constexpr int kSpanRoundTrip = 64;
  const int be = c->dtype == kBF16 ? 2 : 4;
  WorkCost wc;
  wc.span_base = (2 * c->rank * c->d * be) / 64 + kItemOverhead;
  wc.span_row = 2 * c->rank * be;
  wc.span_extra = kSpanRoundTrip;
  wc.full = (2 * kChunk * c->d * be) / 64 + kItemOverhead;
  wc.summ = (kChunk * c->d * be + kChunk * c->G * 4) / 64 + kItemOverhead;
  return wc;
}

// Workgroups per unit.  MFMA path: about two resident workgroups per CU
// (512 over all units; each wave then works through a long item range with
// its loads pipelined), at most one wave per item.  VALU path: about 2048
// workgroups, at most one per item.
static int nsplit_for(int B, int Hkv, int S, int F, int k_slots, bool mfma) {
  const int U = B * Hkv;
  const int NI = (F + kChunk - 1) / kChunk + k_slots + (S + kChunk - 1) / kChunk;
  const int target = mfma ? 512 : 2048;
  int ns = (target + U - 1) / U;
  const int per_block = mfma ? 4 : 1;
  if (ns > (NI + per_block - 1) / per_block) ns = (NI + per_block - 1) / per_block;
  if (mfma && ns > kMaxSplitMfma) ns = kMaxSplitMfma;
  return ns < 1 ? 1 : ns;
}

int decode_nsplit(const rskv_cache* c, int k_max) {
  const int k_slots = k_max < c->S ? k_max : c->S;
  int ns = nsplit_for(c->B, c->Hkv, c->S, c->F, k_slots, use_mfma(c));
  // RSKV_ATTEND_SPLITS overrides the workgroups per unit (tuning only)
  if (const char* e = getenv("RSKV_ATTEND_SPLITS")) {
    const int v = atoi(e);
    if (v > 0) ns = use_mfma(c) && v > kMaxSplitMfma ? kMaxSplitMfma : v;
  }
  return ns > c->nsplit_max ? c->nsplit_max : ns;
}

int decode_nsplit_max(int B, int Hkv, int S, int F, int k_max_cap) {
  const int k_slots = k_max_cap < S ? k_max_cap : S;
  const int a = nsplit_for(B, Hkv, S, F, k_slots, true);
  const int v = nsplit_for(B, Hkv, S, F, k_slots, false);
  // room for the tuning override as well (at most one workgroup per item)
  const int NI = (F + kChunk - 1) / kChunk + k_slots + (S + kChunk - 1) / kChunk;
  const int o = NI < kMaxSplitMfma ? NI : kMaxSplitMfma;
  const int m = a > v ? a : v;
  return m > o ? m : o;
}

hipError_t launch_attend(const rskv_cache* c, const DecodeWs& ws, const void* q, int nsplit,
                         const SelectArgs* sa, hipStream_t st, const KernelEvents* ev) {
  if (use_mfma(c)) {
    if (c->d == 128)
      return c->rank == 16 ? attend_mfma_impl<128, 16>(c, ws, q, nsplit, sa, st, ev)
                           : attend_mfma_impl<128, 8>(c, ws, q, nsplit, sa, st, ev);
    return c->rank == 16 ? attend_mfma_impl<64, 16>(c, ws, q, nsplit, sa, st, ev)
                         : attend_mfma_impl<64, 8>(c, ws, q, nsplit, sa, st, ev);
  }
  return c->dtype == kBF16 ? attend_valu_impl<kBF16>(c, ws, q, nsplit, st, ev)
                           : attend_valu_impl<kF32>(c, ws, q, nsplit, st, ev);
}

hipError_t launch_merge(const rskv_cache* c, const DecodeWs& ws, int nsplit, float* out,
                        hipStream_t st, const KernelEvents* ev) {
  return launch(merge_kernel, dim3(c->B * c->Hkv, c->G), dim3(128), 0, st, ev, ws.part, nsplit,
                c->nsplit_max, c->Hkv, c->G, c->d, out);
}

}  // namespace rskv
