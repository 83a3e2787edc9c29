// Window-routed three-tier cache (QEvict summary, "Metodologia: QEvict"):
// decode kernels.
//
//   attend_full_kernel  bf16 caches, full-precision windows.  Each wave
//       walks a contiguous range of the unit's full windows with an online
//       softmax per query head; QK and PV products on 16x16x32 bf16 MFMAs
//       straight from the K16 / V32 tiles, all loads of a window issued
//       before its first product.
//   attend_int2_kernel  bf16 caches, INT2 windows, same structure: the codes
//       are widened in registers (one packed fp4 conversion per code pair)
//       and fed to 16x16x32 MFMAs; the fp32 scales and minima, staged per
//       wave in LDS, are applied around the products:
//         <q, k_r> = sum_grp scale_r,grp <q_grp, code_r,grp> + min_r,grp sum(q_grp)
//         sum_r p_r v_r = sum_r (p_r scale_r,grp) code_r + sum_r p_r min_r,grp
//       which is the dequantised arithmetic up to association.  The QK
//       product is exact (bf16 codes times the bf16 query, fp32 sums), so
//       the logits, hence the masses that route the windows, keep fp32
//       accuracy; in the PV product the weights p_r scale_r,grp enter as
//       fp16 (relative rounding 2^-11, far inside the output tolerance of
//       bf16 caches).  In the full-window kernel p enters as a bf16 hi + lo
//       pair.  In both kernels the four waves of a workgroup merge in LDS
//       and write one partial.
//   attend_valu_kernel  fp32 caches: a block-cooperative fp32 version that
//       dequantises INT2 rows exactly (mn + code * scale, two roundings).
//   merge_kernel        log-sum-exp merge of a unit's partials; on routing
//       steps it also keeps each head's maximum and denominator.
//   route_kernel        routing event: window masses from the per-window
//       softmax statistics, cumulative scores, ranking of the windows not
//       evicted (bitonic sort in LDS), new tiers, the next attended list and
//       the lists of ledger writes and promotions.
//   transition_kernel   first demotions quantise a window into the ledger;
//       promotions write the dequantised values back into the full store.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "lanes.h"
#include "window.h"

namespace rskv {
namespace win {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCostFull = 2;  // work cost of a full-precision window (measured
constexpr int kCostQuant = 1; // attention time ratio to an INT2 window)
constexpr float kMaxSlack = 11.f;  // base-2 logits may exceed the running softmax reference by this
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTargetWaves = 8192;

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// fp32 x as bf16 hi + lo (hi + lo equals x to ~16 significant bits).
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 hb = static_cast<__bf16>(x[e]);
    hi[e] = hb;
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(hb));
  }
}

// The eight codes of MFMA operand `half` of a ledger word as bf16 0.0 ..
// 3.0: masked to one code per nibble they are e2m1 values c / 2, which the
// packed fp4 -> bf16 conversion widens two at a time with scale 2.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 decode8(uint32_t word, int half) {
  const uint32_t nib = (word >> (2 * half)) & 0x33333333u;
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(nib, 2.0f, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(nib, 2.0f, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(nib, 2.0f, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(nib, 2.0f, 3);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The same eight codes as fp16 0.0 .. 3.0 (packed fp4 -> fp16 conversion).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8 decode8h(uint32_t word, int half) {
  const uint32_t nib = (word >> (2 * half)) & 0x33333333u;
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 0);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 1);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 2);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 3);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ f32x4 mmah(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Dequantised INT2 value mn + code * scale: the product is rounded to fp32
// before the sum (contraction into a fused multiply-add is switched off).
__device__ __forceinline__ float dequant(float code, float scale, float mn) {
#pragma clang fp contract(off)
  const float p = code * scale;
  return mn + p;
}

// First attended window of range v of nv (ranges balanced by cost).
__device__ __forceinline__ int range_start(int v, int nv, int nf, int nit) {
  const long long fullc = static_cast<long long>(kCostFull) * nf;
  const long long tot = fullc + static_cast<long long>(kCostQuant) * (nit - nf);
  const long long b = tot * v / nv;
  if (b <= fullc) return static_cast<int>((b + kCostFull - 1) / kCostFull);
  return nf + static_cast<int>((b - fullc + kCostQuant - 1) / kCostQuant);
}

// ---------------------------------------------------------------- build

template <int DT, int D>
__global__ __launch_bounds__(256) void build_kernel(const typename Elem<DT>::T* __restrict__ K,
                                                    const typename Elem<DT>::T* __restrict__ V,
                                                    int T, int rows_pad,
                                                    typename Elem<DT>::T* __restrict__ kf,
                                                    typename Elem<DT>::T* __restrict__ vf) {
  typedef typename Elem<DT>::T E;
  const int u = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;  // (row, 8-column chunk)
  if (e >= rows_pad * (D / 8)) return;
  const int r = e / (D / 8);
  const int c0 = (e - r * (D / 8)) * 8;
  const size_t src = (static_cast<size_t>(u) * T + r) * D + c0;
  const size_t dst = static_cast<size_t>(u) * rows_pad * D;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const E kx = r < T ? K[src + j] : E(0);
    const E vx = r < T ? V[src + j] : E(0);
    kf[dst + k16_off(r, c0 + j, D)] = kx;
    vf[dst + v32_off(r, c0 + j, D)] = vx;
  }
}

// --------------------------------------------------------- attention (MFMA)

// Query operand of a wave (head n = lane % 16, columns 32 kb + 8 (lane / 16)
// + 0..7; zero for heads >= G) and, per 64-column group, the sum of the
// head's query over the group.
template <int D>
struct QOperand {
  static constexpr int KB = D / 32;
  static constexpr int NG = D / kGroup;
  bf16x8 qb[KB];
  float qsum[NG];
  __device__ __forceinline__ void load(const uint16_t* q, size_t base, int lane, int G) {
    const int n = lane & 15, g = lane >> 4;
    const bool hv = n < G;
    const uint16_t* qp = q + base + static_cast<size_t>(hv ? n : 0) * D + 8 * g;
#pragma unroll
    for (int x = 0; x < NG; ++x) qsum[x] = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qp + kb * 32);
      if (!hv) x = u32x4{0u, 0u, 0u, 0u};
      qb[kb] = as8(x);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s += __uint_as_float(x[e] << 16) + __uint_as_float(x[e] & 0xffff0000u);
      qsum[kb / 2] += s;
    }
#pragma unroll
    for (int x = 0; x < NG; ++x) {
      qsum[x] += xor_lane<16>(qsum[x]);
      qsum[x] += xor_lane<32>(qsum[x]);
    }
  }
};

// Online-softmax state of a wave for head n = lane % 16 over the rows its
// lane group holds, in base 2: reference m, sum l, out^T in the MFMA
// accumulator layout (coordinates 16 cb + 4 (lane / 16) + i).
template <int D>
struct SoftState {
  static constexpr int CB = D / 16;
  static constexpr int NG = D / kGroup;
  float m = -INFINITY, l = 0.f;
  f32x4 acc[CB];
  float amn[NG];  // INT2 windows: sum_r p_r min_r,grp over the lane's rows
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < NG; ++x) amn[x] = 0.f;
  }
  // s: the window's 64 scores of head n (16 per lane), whose base-2 logits
  // are s sl (sl > 0, applied inside the maximum and the exponentials) ->
  // probabilities relative to m.  On routing steps the window's own maximum
  // and sum go to *ws (natural-log maximum).
  template <bool MASS>
  __device__ __forceinline__ void update(float (&s)[4][4], float sl, int nvalid, int g,
                                         bool store, float2* ws) {
    if (nvalid < kRows) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (rb * 16 + 4 * g + i >= nvalid) s[rb][i] = -INFINITY;
    }
    float cm = s[0][0];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) cm = fmaxf(cm, s[rb][i]);
    cm = fmaxf(cm, xor_lane<16>(cm));
    cm = fmaxf(cm, xor_lane<32>(cm));
    cm *= sl;
    if (MASS) {
      float w = 0.f;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) w += __builtin_amdgcn_exp2f(fmaf(s[rb][i], sl, -cm));
      w += xor_lane<16>(w);
      w += xor_lane<32>(w);
      if (store) *ws = make_float2(cm * kLn2, w);
    }
    // the reference m moves only when a logit exceeds it by more than
    // kMaxSlack (p <= 2^11 stays exact enough in fp32), so the state is
    // rarely rescaled
    const float mnew = cm > m + kMaxSlack ? cm : m;
    if (__any(mnew != m)) {
      const float fac = __builtin_amdgcn_exp2f(m - mnew);
      l *= fac;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb] *= fac;
#pragma unroll
      for (int x = 0; x < NG; ++x) amn[x] *= fac;
      m = mnew;
    }
    float ps = 0.f;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[rb][i] = __builtin_amdgcn_exp2f(fmaf(s[rb][i], sl, -m));
        ps += s[rb][i];
      }
    ps += xor_lane<16>(ps);
    ps += xor_lane<32>(ps);
    l += ps;
  }
};

// Merge of the four waves of a workgroup (LDS, `mbuf` holds >= 4 * G * D +
// 8 * kMaxG floats) and the workgroup's partial: per head
// [out^T (D), max (natural log), sum].
template <int D>
__device__ __forceinline__ void block_partial(SoftState<D>& st, float* mbuf, int G, float* pb) {
  constexpr int CB = D / 16;
  constexpr int NG = D / kGroup;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  // minima terms of the INT2 values, summed over the lane groups' rows
#pragma unroll
  for (int x = 0; x < NG; ++x) {
    st.amn[x] += xor_lane<16>(st.amn[x]);
    st.amn[x] += xor_lane<32>(st.amn[x]);
  }
  float* sm = mbuf;                 // [4][kMaxG]
  float* sl4 = mbuf + 4 * kMaxG;    // [4][kMaxG]
  float* so = mbuf + 8 * kMaxG;     // [4][G][D]
  __syncthreads();  // the buffer may alias a wave's staging area
  if (g == 0) {
    sm[wave * kMaxG + n] = st.m * kLn2;  // natural-log units for the merge
    sl4[wave * kMaxG + n] = st.l;
  }
  if (n < G) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        so[(wave * G + n) * D + cb * 16 + 4 * g + i] = st.acc[cb][i] + st.amn[cb >> 2];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    const int hh = e / D;
    const int c = e - hh * D;
    float mw[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) mw[x] = sm[x * kMaxG + hh];
    const float M = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
    float o = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float f = mw[x] == -INFINITY ? 0.f : __expf(mw[x] - M);
        o += f * so[(x * G + hh) * D + c];
        L += f * sl4[x * kMaxG + hh];
      }
    }
    pb[hh * (D + 2) + c] = o;
    if (c == 0) {
      pb[hh * (D + 2) + D] = M;
      pb[hh * (D + 2) + D + 1] = L;
    }
  }
}

// Full-precision windows [0, nf) of the attended list; grid (nsf, U), four
// waves per workgroup each on a contiguous range.  Partials at slots
// [0, nsf) of the unit's nsplit.
template <int D, bool MASS>
__global__ __launch_bounds__(256) void attend_full_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kf,
    const uint16_t* __restrict__ vf, const int32_t* __restrict__ items, int nW, int T, int Hq,
    int Hkv, int G, int nf, int nsplit, float* __restrict__ part, float2* __restrict__ wstat) {
  constexpr int KB = D / 32;
  constexpr int CB = D / 16;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int nv = gridDim.x * 4;
  const int v = blockIdx.x * 4 + wave;
  const int k0 = static_cast<int>(static_cast<long long>(nf) * v / nv);
  const int k1 = static_cast<int>(static_cast<long long>(nf) * (v + 1) / nv);
  QOperand<D> qo;
  qo.load(q, (static_cast<size_t>(b) * Hq + static_cast<size_t>(h) * G) * D, lane, G);
  const float sl = kLog2e / sqrtf(static_cast<float>(D));
  SoftState<D> st;
  st.init();
  for (int k = k0; k < k1; ++k) {
    // the routing kernel only lists windows < nW; the clamp keeps a bad entry in bounds
    const int w = min(max(items[static_cast<size_t>(u) * nW + k], 0), nW - 1);
    const int nvalid = min(kRows, T - w * kRows);
    const size_t wb = static_cast<size_t>(u) * nW + w;
    const uint16_t* kt = kf + wb * kRows * D + lane * 8;
    const uint16_t* vt = vf + wb * kRows * D + lane * 8;
    u32x4 ka[4][KB], va[2][CB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        ka[rb][kb] = *reinterpret_cast<const u32x4*>(kt + (rb * KB + kb) * 512);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        va[rb][cb] = *reinterpret_cast<const u32x4*>(vt + (rb * CB + cb) * 512);
    float s[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 c{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) c = mma(as8(ka[rb][kb]), qo.qb[kb], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[rb][i] = c[i] * sl;
    }
    st.template update<MASS>(s, 1.f, nvalid, g, g == 0 && n < G,
                             wstat + (static_cast<size_t>(u) * nW + k) * G + n);
    // PV: A = values (column 16 cb + n, rows v32_row(g, .)), B = p (head n)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float pp[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pp[e] = s[2 * rb][e];
        pp[4 + e] = s[2 * rb + 1][e];
      }
      bf16x8 hi, lo;
      split8(pp, hi, lo);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        st.acc[cb] = mma(as8(va[rb][cb]), hi, st.acc[cb]);
        st.acc[cb] = mma(as8(va[rb][cb]), lo, st.acc[cb]);
      }
    }
  }
  __shared__ float mbuf[8 * kMaxG + 4 * kMaxG * D];
  block_partial<D>(st, mbuf, G,
                   part + (static_cast<size_t>(u) * nsplit + blockIdx.x) * G * (D + 2));
}

// INT2 windows [nf, nit) of the attended list; grid (nsq, U).  Each wave
// stages a window's scales and minima (256 (d / 64) floats) in its own LDS
// area with coalesced loads and reads them back as broadcasts.  Partials
// at slots [split0, split0 + nsq).  The path is VALU-bound (code widening,
// scale arithmetic, softmax); four waves per SIMD measured fastest (a
// handful of registers spill; three or two waves leave issue slots idle).
template <int D, bool MASS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void attend_int2_kernel(
    const uint16_t* __restrict__ q, const uint32_t* __restrict__ codes,
    const float* __restrict__ qsc, const int32_t* __restrict__ items, int nW, int T, int Hq,
    int Hkv, int G, int nf, int nit, int split0, int nsplit, float* __restrict__ part,
    float2* __restrict__ wstat) {
  constexpr int NG = D / kGroup;
  constexpr int KB = D / 32;
  constexpr int CB = D / 16;
  constexpr int SQ4 = 64 * NG;  // float4 of scales per window
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int nq = nit - nf;
  const int nv = gridDim.x * 4;
  const int v = blockIdx.x * 4 + wave;
  const int k0 = nf + static_cast<int>(static_cast<long long>(nq) * v / nv);
  const int k1 = nf + static_cast<int>(static_cast<long long>(nq) * (v + 1) / nv);
  QOperand<D> qo;
  qo.load(q, (static_cast<size_t>(b) * Hq + static_cast<size_t>(h) * G) * D, lane, G);
  const float sl = kLog2e / sqrtf(static_cast<float>(D));
  SoftState<D> st;
  st.init();
  // per wave: two staging areas of one window's scales (alternating), later
  // reused by the workgroup merge
  constexpr int kStage = 4 * 2 * SQ4 * 4;
  constexpr int kMerge = 8 * kMaxG + 4 * kMaxG * D;
  __shared__ float lds[kStage > kMerge ? kStage : kMerge];
  float4* stage = reinterpret_cast<float4*>(lds) + wave * 2 * SQ4;
  for (int k = k0; k < k1; ++k) {
    const int w = min(max(items[static_cast<size_t>(u) * nW + k], 0), nW - 1);
    const int nvalid = min(kRows, T - w * kRows);
    const size_t wb = static_cast<size_t>(u) * nW + w;
    const uint32_t* cw = codes + wb * (8 * D);
    u32x4 kw[NG], vw[NG];
#pragma unroll
    for (int p = 0; p < NG; ++p) {
      kw[p] = *reinterpret_cast<const u32x4*>(cw + (p * 64 + lane) * 4);
      vw[p] = *reinterpret_cast<const u32x4*>(cw + 4 * D + (p * 64 + lane) * 4);
    }
    float4* sq = stage + (k & 1) * SQ4;
    {
      const float4* src = reinterpret_cast<const float4*>(qsc + wb * (256 * NG));
#pragma unroll
      for (int x = 0; x < NG; ++x) sq[x * 64 + lane] = src[x * 64 + lane];
    }
    // LDS operations of a wave complete in order: the reads below see the
    // whole block
    float s[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 cg[NG];
      float4 a4[NG], b4[NG];
#pragma unroll
      for (int x = 0; x < NG; ++x) {
        // group x of rows 16 rb + 4 g + i: the two 32-column blocks of the
        // group, then [i][scale, min]
        cg[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int kb = 2 * x + kh;
          const int o = rb * KB + kb;
          const int t = o >> 1;
          cg[x] = mma(decode8(kw[t >> 2][t & 3], o & 1), qo.qb[kb], cg[x]);
        }
        a4[x] = sq[((rb * 4 + g) * NG + x) * 2];
        b4[x] = sq[((rb * 4 + g) * NG + x) * 2 + 1];
      }
      // the minimum terms first, then one multiply-add per group for the
      // scaled code products
      float z[4] = {a4[0].y * qo.qsum[0], a4[0].w * qo.qsum[0], b4[0].y * qo.qsum[0],
                    b4[0].w * qo.qsum[0]};
#pragma unroll
      for (int x = 1; x < NG; ++x) {
        z[0] = fmaf(a4[x].y, qo.qsum[x], z[0]);
        z[1] = fmaf(a4[x].w, qo.qsum[x], z[1]);
        z[2] = fmaf(b4[x].y, qo.qsum[x], z[2]);
        z[3] = fmaf(b4[x].w, qo.qsum[x], z[3]);
      }
#pragma unroll
      for (int x = 0; x < NG; ++x) {
        z[0] = fmaf(a4[x].x, cg[x][0], z[0]);
        z[1] = fmaf(a4[x].z, cg[x][1], z[1]);
        z[2] = fmaf(b4[x].x, cg[x][2], z[2]);
        z[3] = fmaf(b4[x].z, cg[x][3], z[3]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[rb][i] = z[i];
    }
    st.template update<MASS>(s, sl, nvalid, g, g == 0 && n < G,
                             wstat + (static_cast<size_t>(u) * nW + k) * G + n);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float pp[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pp[e] = s[2 * rb][e];
        pp[4 + e] = s[2 * rb + 1][e];
      }
#pragma unroll
      for (int x = 0; x < NG; ++x) {
        // rows v32_row(g, e) of block rb, group x: [e][scale, min]
        float sc[16];
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const float4 t4 = sq[32 * NG + ((rb * 4 + g) * NG + x) * 4 + y];
          sc[4 * y] = t4.x;
          sc[4 * y + 1] = t4.y;
          sc[4 * y + 2] = t4.z;
          sc[4 * y + 3] = t4.w;
        }
        // B = p_r scale_r,x in fp16 (one rounding, relative 2^-11: these
        // products only weigh values, the logits above stay exact)
        f16x8 pw;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pw[e] = static_cast<_Float16>(pp[e] * sc[2 * e]);
          st.amn[x] += pp[e] * sc[2 * e + 1];
        }
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const int cb = 4 * x + c4;  // the 16-column blocks of group x
          const int o = rb * CB + cb;
          const int t = o >> 1;
          st.acc[cb] = mmah(decode8h(vw[t >> 2][t & 3], o & 1), pw, st.acc[cb]);
        }
      }
    }
  }
  block_partial<D>(st, lds, G,
                   part + (static_cast<size_t>(u) * nsplit + split0 + blockIdx.x) * G * (D + 2));
}

// --------------------------------------------------------- attention (VALU)

template <int DT, int D, bool MASS>
__global__ __launch_bounds__(256) void attend_valu_kernel(
    const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ kf,
    const typename Elem<DT>::T* __restrict__ vf, const uint32_t* __restrict__ codes,
    const float* __restrict__ qsc, const int32_t* __restrict__ items, int nW, int T, int Hq,
    int Hkv, int G, int nf, int nit, int nsplit, float* __restrict__ part,
    float2* __restrict__ wstat) {
  typedef Elem<DT> E;
  constexpr int NG = D / kGroup;
  constexpr int SQ = 256 * NG;
  constexpr int NO = (kMaxG * D + 255) / 256;  // outputs per thread
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int k0 = range_start(blockIdx.x, nsplit, nf, nit);
  const int k1 = range_start(blockIdx.x + 1, nsplit, nf, nit);
  __shared__ float qs[kMaxG][D];
  __shared__ float xs[kRows][D + 1];
  __shared__ float pl[kMaxG][kRows];
  __shared__ float mrun[kMaxG], lrun[kMaxG], fac[kMaxG];
  const size_t qbase = (static_cast<size_t>(b) * Hq + static_cast<size_t>(h) * G) * D;
  for (int e = tid; e < G * D; e += 256) qs[e / D][e % D] = E::ld(q, qbase + e);
  if (tid < kMaxG) {
    mrun[tid] = -INFINITY;
    lrun[tid] = 0.f;
  }
  float acc[NO];
#pragma unroll
  for (int j = 0; j < NO; ++j) acc[j] = 0.f;
  const float sl = 1.0f / sqrtf(static_cast<float>(D));
  const size_t ub = static_cast<size_t>(u) * nW * kRows * D;

  // rows of window w, side 0 (K) or 1 (V), as fp32 into xs
  auto stage = [&](int w, bool full, int side) {
    const size_t wb = static_cast<size_t>(u) * nW + w;
    const uint32_t* cw = codes + wb * (8 * D);
    const float* qw = qsc + wb * SQ;
    for (int e = tid; e < kRows * D; e += 256) {
      const int r = e / D;
      const int c = e - r * D;
      float x;
      if (full) {
        const size_t o = ub + (side == 0 ? k16_off(w * kRows + r, c, D) : v32_off(w * kRows + r, c, D));
        x = E::ld(side == 0 ? kf : vf, o);
      } else {
        int bit;
        const int wd = code_word(side, r, c, D, &bit);
        const float code = static_cast<float>((cw[wd] >> bit) & 3u);
        const int grp = c / kGroup;
        const float sc = qw[side == 0 ? kq_off(r, grp, 0, D) : vq_off(r, grp, 0, D)];
        const float mn = qw[side == 0 ? kq_off(r, grp, 1, D) : vq_off(r, grp, 1, D)];
        x = dequant(code, sc, mn);
      }
      xs[r][c] = x;
    }
  };

  for (int k = k0; k < k1; ++k) {
    const int w = min(max(items[static_cast<size_t>(u) * nW + k], 0), nW - 1);
    const int nvalid = min(kRows, T - w * kRows);
    const bool full = k < nf;
    __syncthreads();
    stage(w, full, 0);
    __syncthreads();
    for (int e = tid; e < G * kRows; e += 256) {
      const int hh = e / kRows;
      const int r = e - hh * kRows;
      float a = 0.f;
      for (int c = 0; c < D; ++c) a += qs[hh][c] * xs[r][c];
      pl[hh][r] = r < nvalid ? a * sl : -INFINITY;
    }
    __syncthreads();
    for (int hh = wave; hh < G; hh += 4) {
      const float s = pl[hh][lane];
      const float cm = wave_max(s);
      if (MASS) {
        const float ws = wave_sum(expf(s - cm));
        if (lane == 0) wstat[(static_cast<size_t>(u) * nW + k) * G + hh] = make_float2(cm, ws);
      }
      const float mo = mrun[hh];
      const float mnew = fmaxf(mo, cm);
      const float p = expf(s - mnew);
      const float ps = wave_sum(p);
      pl[hh][lane] = p;
      if (lane == 0) {
        const float f = expf(mo - mnew);
        fac[hh] = f;
        lrun[hh] = lrun[hh] * f + ps;
        mrun[hh] = mnew;
      }
    }
    stage(w, full, 1);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NO; ++j) {
      const int e = tid + 256 * j;
      if (e < G * D) {
        const int hh = e / D;
        const int c = e - hh * D;
        float a = acc[j] * fac[hh];
        for (int r = 0; r < kRows; ++r) a += pl[hh][r] * xs[r][c];
        acc[j] = a;
      }
    }
  }
  __syncthreads();
  float* pb = part + (static_cast<size_t>(u) * nsplit + blockIdx.x) * G * (D + 2);
#pragma unroll
  for (int j = 0; j < NO; ++j) {
    const int e = tid + 256 * j;
    if (e < G * D) {
      const int hh = e / D;
      const int c = e - hh * D;
      pb[hh * (D + 2) + c] = acc[j];
      if (c == 0) {
        pb[hh * (D + 2) + D] = mrun[hh];
        pb[hh * (D + 2) + D + 1] = lrun[hh];
      }
    }
  }
}

// ---------------------------------------------------------------- merge

// Grid (G, U), D threads: out = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s
// for query head g of unit u.  The maximum, the weights e^{m_s - M} (kept
// in LDS) and the denominator are reduced over the partials in parallel;
// each thread then sums its column, eight independent loads at a time.
constexpr int kMergeChunk = 1024;

template <int D, bool MASS>
__global__ __launch_bounds__(D) void merge_kernel(const float* __restrict__ part, int nsplit, int G,
                                                  int Hq, int Hkv, float* __restrict__ out,
                                                  float2* __restrict__ hstat) {
  constexpr int NW = D / kWave;
  const int g = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int h = u - b * Hkv;
  const int c = threadIdx.x;
  __shared__ float buf[NW];
  __shared__ float wgt[kMergeChunk];
  const size_t stride = static_cast<size_t>(G) * (D + 2);
  const float* p = part + static_cast<size_t>(u) * nsplit * stride + static_cast<size_t>(g) * (D + 2);
  float mx = -INFINITY;
  for (int s = c; s < nsplit; s += D) mx = fmaxf(mx, p[s * stride + D]);
  mx = wave_max(mx);
  if ((c & 63) == 0) buf[c >> 6] = mx;
  __syncthreads();
  float M = buf[0];
#pragma unroll
  for (int x = 1; x < NW; ++x) M = fmaxf(M, buf[x]);
  __syncthreads();
  float dl = 0.f, num = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += kMergeChunk) {
    const int ns = min(kMergeChunk, nsplit - s0);
    for (int s = c; s < ns; s += D) {
      const float ms = p[(s0 + s) * stride + D];
      const float wv = ms == -INFINITY ? 0.f : expf(ms - M);
      wgt[s] = wv;
      dl += wv * p[(s0 + s) * stride + D + 1];
    }
    __syncthreads();
    const float* pc = p + static_cast<size_t>(s0) * stride + c;
    int s = 0;
    for (; s + 8 <= ns; s += 8) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = pc[(s + j) * stride];
#pragma unroll
      for (int j = 0; j < 8; ++j) num += wgt[s + j] * x[j];
    }
    for (; s < ns; ++s) num += wgt[s] * pc[s * stride];
    __syncthreads();
  }
  dl = wave_sum(dl);
  if ((c & 63) == 0) buf[c >> 6] = dl;
  __syncthreads();
  float den = 0.f;
#pragma unroll
  for (int x = 0; x < NW; ++x) den += buf[x];
  out[(static_cast<size_t>(b) * Hq + static_cast<size_t>(h) * G + g) * D + c] = num / den;
  if (MASS && c == 0) hstat[static_cast<size_t>(u) * G + g] = make_float2(M, den);
}

// ---------------------------------------------------------------- routing

// One workgroup per unit.  Sort keys: ((~bits(score)) >> 1) with the low
// 14 bits replaced by the window, ascending = score descending, ties to the
// lower window (scores are >= 0, so their bit patterns order like them);
// evicted windows and padding sort last.
template <int NP>
__global__ __launch_bounds__(1024) void route_kernel(
    const float2* __restrict__ wstat, const float2* __restrict__ hstat, int G, int nW, int nit,
    int n_full, int n_quant, int32_t* __restrict__ items, int8_t* __restrict__ tier,
    double* __restrict__ score, double* __restrict__ mass, const uint8_t* __restrict__ has_code,
    int32_t* __restrict__ trans, int32_t* __restrict__ ntrans) {
  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  constexpr int NR = NP >= 1024 ? NP / 1024 : 1;
  __shared__ unsigned long long key[NP];
  __shared__ uint8_t ost[NP];  // old tier (bits 0-1), ledger flag (bit 2)
  __shared__ int cnt[2];
  const size_t ub = static_cast<size_t>(u) * nW;
  // every independent load first: the state of this thread's windows
  // w = tid + 1024 r and the masses of its attended windows k = tid + 1024 r
  double sc0[NR];
  int t0[NR], h0[NR], wk[NR];
  double mk[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int w = tid + 1024 * r;
    const bool in = w < nW;
    sc0[r] = in ? score[ub + w] : 0.0;
    t0[r] = in ? tier[ub + w] : RSKV_TIER_EVICTED;
    h0[r] = in ? has_code[ub + w] : 0;
    const int k = tid + 1024 * r;
    wk[r] = -1;
    mk[r] = 0.0;
    if (k < nit) {
      wk[r] = items[ub + k];
      double ms = 0.0;
      for (int hh = 0; hh < G; ++hh) {
        const float2 ws = wstat[(ub + k) * G + hh];
        const float2 hs = hstat[static_cast<size_t>(u) * G + hh];
        ms += static_cast<double>(ws.y) * exp(static_cast<double>(ws.x) - static_cast<double>(hs.x)) /
              static_cast<double>(hs.y);
      }
      mk[r] = ms;
    }
  }
  double* mw = reinterpret_cast<double*>(key);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int w = tid + 1024 * r;
    if (w < NP) {
      mw[w] = 0.0;
      ost[w] = static_cast<uint8_t>((t0[r] & 3) | (h0[r] ? 4 : 0));
    }
  }
  if (tid < 2) cnt[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NR; ++r)
    if (wk[r] >= 0 && wk[r] < nW) mw[wk[r]] = mk[r];
  __syncthreads();
  double msw[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) msw[r] = tid + 1024 * r < NP ? mw[tid + 1024 * r] : 0.0;
  __syncthreads();  // mw aliases the keys written below
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int w = tid + 1024 * r;
    unsigned long long kk = ~0ull;
    if (w < nW) {
      mass[ub + w] = msw[r];
      const double sc = sc0[r] + msw[r];
      score[ub + w] = sc;
      if (t0[r] != RSKV_TIER_EVICTED) {
        const unsigned long long bits = static_cast<unsigned long long>(__double_as_longlong(sc));
        kk = (((~bits) >> 1) & ~0x3fffull) | static_cast<unsigned long long>(w);
      }
    }
    if (w < NP) key[w] = kk;
  }
  __syncthreads();
  // bitonic sort, ascending.  Thread t holds elements t + 1024 r (r <
  // NP / 1024, at least one).  Partners at stride j < 64 sit in the same
  // wave (wave shuffles), at j >= 1024 in the same thread (registers); only
  // strides 64..512 go through LDS.
  const int lane = tid & 63;
  unsigned long long v[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) v[r] = tid + 1024 * r < NP ? key[tid + 1024 * r] : ~0ull;
  for (int kk = 2; kk <= NP; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      if (j >= 1024) {
        const int jr = j / 1024;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int i = tid + 1024 * r;
          if ((r & jr) == 0) {
            const bool up = (i & kk) == 0;
            const unsigned long long a = v[r], c = v[r | jr];
            if ((a > c) == up) {
              v[r] = c;
              v[r | jr] = a;
            }
          }
        }
      } else if (j >= 64) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < NR; ++r)
          if (tid + 1024 * r < NP) key[tid + 1024 * r] = v[r];
        __syncthreads();
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int i = tid + 1024 * r;
          if (i < NP) {
            const unsigned long long c = key[i ^ j];
            const bool up = (i & kk) == 0;
            const bool lower = (i & j) == 0;  // i is the first of its pair
            // the pair's first element keeps the smaller key when ascending
            const bool take = lower == up ? c < v[r] : c > v[r];
            if (take) v[r] = c;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int i = tid + 1024 * r;
          const unsigned long long c = static_cast<unsigned long long>(
              __shfl_xor(static_cast<long long>(v[r]), j, kWave));
          const bool up = (i & kk) == 0;
          const bool lower = (lane & j) == 0;
          const bool take = lower == up ? c < v[r] : c > v[r];
          if (take) v[r] = c;
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NR; ++r)
    if (tid + 1024 * r < NP) key[tid + 1024 * r] = v[r];
  __syncthreads();
  for (int pos = tid; pos < nW; pos += 1024) {
    const unsigned long long kk = key[pos];
    if (kk == ~0ull) continue;
    const int w = static_cast<int>(kk & 0x3fffull);
    const int old = ost[w] & 3;
    const int nt = pos < n_full ? RSKV_TIER_FULL
                   : pos < n_full + n_quant ? RSKV_TIER_INT2 : RSKV_TIER_EVICTED;
    tier[ub + w] = static_cast<int8_t>(nt);
    if (nt != RSKV_TIER_EVICTED) items[ub + pos] = w;
    if (nt == RSKV_TIER_INT2 && old == RSKV_TIER_FULL && !(ost[w] & 4))
      trans[(static_cast<size_t>(u) * 2) * nW + atomicAdd(&cnt[0], 1)] = w;
    if (nt == RSKV_TIER_FULL && old == RSKV_TIER_INT2)
      trans[(static_cast<size_t>(u) * 2 + 1) * nW + atomicAdd(&cnt[1], 1)] = w;
  }
  __syncthreads();
  if (tid < 2) ntrans[u * 2 + tid] = cnt[tid];
}

// ---------------------------------------------------------- transitions

// One workgroup per listed window at a time.  Quantise: a side (K, then V)
// of the window's full-precision block, contiguous in the tiled store, is
// staged in LDS with 16-byte loads (code_elem maps a tile slot to its row
// and column), quantised row by row and packed into ledger words.
// Promote: each 16-byte chunk of the store is rebuilt from one ledger word
// and the window's scales (staged in LDS) and written back.
template <int DT, int D>
__global__ __launch_bounds__(256) void transition_kernel(
    typename Elem<DT>::T* __restrict__ kf, typename Elem<DT>::T* __restrict__ vf,
    uint32_t* __restrict__ codes, float* __restrict__ qsc, uint8_t* __restrict__ has_code,
    const int32_t* __restrict__ trans, const int32_t* __restrict__ ntrans, int nW) {
  typedef Elem<DT> E;
  typedef typename Elem<DT>::T T;
  constexpr int NG = D / kGroup;
  constexpr int SQ = 256 * NG;
  constexpr int WPS = 64 * (D / 16);   // code words per side
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CH = kRows * D / EPC;  // chunks per side of a window
  const int u = blockIdx.y;
  const int tid = threadIdx.x;
  const int nq = ntrans[u * 2];
  const int np = ntrans[u * 2 + 1];
  __shared__ float xs[kRows][D + 1];
  __shared__ uint8_t cb[kRows][D];
  __shared__ float qs[SQ];  // a promoted window's scales and minima
  for (int idx = blockIdx.x; idx < nq + np; idx += gridDim.x) {
    const bool quant = idx < nq;
    const int w = quant ? trans[(static_cast<size_t>(u) * 2) * nW + idx]
                        : trans[(static_cast<size_t>(u) * 2 + 1) * nW + (idx - nq)];
    const size_t wb = static_cast<size_t>(u) * nW + w;
    uint32_t* cw = codes + wb * (8 * D);
    float* qw = qsc + wb * SQ;
    if (!quant) {
      for (int i = tid; i < SQ; i += 256) qs[i] = qw[i];
      __syncthreads();
    }
    for (int side = 0; side < 2; ++side) {
      T* tile = (side == 0 ? kf : vf) + wb * kRows * D;
      if (quant) {
        for (int ch = tid; ch < CH; ch += 256) {
          const uint4 raw = reinterpret_cast<const uint4*>(tile)[ch];
          const T* el = reinterpret_cast<const T*>(&raw);
#pragma unroll
          for (int j = 0; j < EPC; ++j) {
            const int o = ch * EPC + j;
            int r, c;
            code_elem(side, o >> 9, (o >> 3) & 63, o & 7, D, &r, &c);
            xs[r][c] = E::ld(el, j);
          }
        }
        __syncthreads();
        // one (row, group) per thread: minimum, maximum, scale, codes
        for (int task = tid; task < kRows * NG; task += 256) {
          const int r = task / NG;
          const int grp = task - r * NG;
          float mn = INFINITY, mx = -INFINITY;
          for (int j = 0; j < kGroup; ++j) {
            const float x = xs[r][grp * kGroup + j];
            mn = fminf(mn, x);
            mx = fmaxf(mx, x);
          }
          const float sc = __fdiv_rn(__fsub_rn(mx, mn), 3.0f);
          for (int j = 0; j < kGroup; ++j) {
            int code = 0;
            if (sc > 0.f) {
              const float t = rintf(__fdiv_rn(__fsub_rn(xs[r][grp * kGroup + j], mn), sc));
              code = static_cast<int>(fminf(fmaxf(t, 0.f), 3.f));
            }
            cb[r][grp * kGroup + j] = static_cast<uint8_t>(code);
          }
          qw[side == 0 ? kq_off(r, grp, 0, D) : vq_off(r, grp, 0, D)] = sc;
          qw[side == 0 ? kq_off(r, grp, 1, D) : vq_off(r, grp, 1, D)] = mn;
        }
        __syncthreads();
        for (int wd = tid; wd < WPS; wd += 256) {
          const int lane = wd / (D / 16);
          const int t = wd - lane * (D / 16);
          uint32_t x = 0;
#pragma unroll
          for (int oh = 0; oh < 2; ++oh)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              int r, c;
              code_elem(side, 2 * t + oh, lane, j, D, &r, &c);
              x |= static_cast<uint32_t>(cb[r][c]) << (4 * j + 2 * oh);
            }
          cw[side * 4 * D + ((t >> 2) * 64 + lane) * 4 + (t & 3)] = x;
        }
      } else {
        // a 16-byte chunk of the tiled store holds elements e0..e0+EPC-1 of
        // tile slot (blk, lane): codes j = e of operand blk in that lane's
        // ledger word
        for (int ch = tid; ch < CH; ch += 256) {
          const int o0 = ch * EPC;
          const int blk = o0 >> 9;
          const int lane = (o0 >> 3) & 63;
          const int t = blk >> 1;
          const uint32_t word = cw[side * 4 * D + ((t >> 2) * 64 + lane) * 4 + (t & 3)];
          uint4 raw;
          T* el = reinterpret_cast<T*>(&raw);
#pragma unroll
          for (int j = 0; j < EPC; ++j) {
            const int e = (o0 & 7) + j;
            int r, c;
            code_elem(side, blk, lane, e, D, &r, &c);
            const int grp = c / kGroup;
            const float sc = qs[side == 0 ? kq_off(r, grp, 0, D) : vq_off(r, grp, 0, D)];
            const float mn = qs[side == 0 ? kq_off(r, grp, 1, D) : vq_off(r, grp, 1, D)];
            const float code = static_cast<float>((word >> (4 * e + 2 * (blk & 1))) & 3u);
            el[j] = E::from_f32(dequant(code, sc, mn));
          }
          reinterpret_cast<uint4*>(tile)[ch] = raw;
        }
      }
      __syncthreads();
    }
    if (quant && tid == 0) has_code[wb] = 1;
  }
}

template <int DT, int D>
hipError_t decode_impl(const rskv_window* W, const void* qv, float* out, bool event, int nf, int nq,
                       hipStream_t st, const KernelEvents* ev, bool* recorded) {
  typedef typename Elem<DT>::T T;
  const int U = W->B * W->Hkv;
  const int nit = nf + nq;
  int nsf = 0, nsq = 0;
  attend_splits(W, nf, nq, &nsf, &nsq);
  const int nsplit = nsf + nsq;
  auto E = [&](int k) -> const KernelEvents* {
    if (recorded) recorded[k] = true;
    return ev ? ev + k : nullptr;
  };
  if (recorded)
    for (int k = 0; k < kKernels; ++k) recorded[k] = false;
  const T* q = static_cast<const T*>(qv);
  const T* kf = static_cast<const T*>(W->kf);
  const T* vf = static_cast<const T*>(W->vf);
  const uint32_t* codes = W->codes;
  const float* qsc = W->qsc;
  const int32_t* items = W->items;
  hipError_t e = hipSuccess;
  if constexpr (DT == kBF16) {
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
    const uint16_t* k16 = reinterpret_cast<const uint16_t*>(kf);
    const uint16_t* v16 = reinterpret_cast<const uint16_t*>(vf);
    if (nsf > 0) {
      if (event)
        e = launch(attend_full_kernel<D, true>, dim3(nsf, U), dim3(256), 0, st, E(0), q16, k16, v16,
                   items, W->nW, W->T, W->Hq, W->Hkv, W->G, nf, nsplit, W->part, W->wstat);
      else
        e = launch(attend_full_kernel<D, false>, dim3(nsf, U), dim3(256), 0, st, E(0), q16, k16,
                   v16, items, W->nW, W->T, W->Hq, W->Hkv, W->G, nf, nsplit, W->part, W->wstat);
      if (e != hipSuccess) return e;
    }
    if (nsq > 0) {
      if (event)
        e = launch(attend_int2_kernel<D, true>, dim3(nsq, U), dim3(256), 0, st, E(1), q16, codes,
                   qsc, items, W->nW, W->T, W->Hq, W->Hkv, W->G, nf, nit, nsf, nsplit, W->part,
                   W->wstat);
      else
        e = launch(attend_int2_kernel<D, false>, dim3(nsq, U), dim3(256), 0, st, E(1), q16, codes,
                   qsc, items, W->nW, W->T, W->Hq, W->Hkv, W->G, nf, nit, nsf, nsplit, W->part,
                   W->wstat);
      if (e != hipSuccess) return e;
    }
  } else {
    if (event)
      e = launch(attend_valu_kernel<DT, D, true>, dim3(nsplit, U), dim3(256), 0, st, E(0), q, kf, vf,
                 codes, qsc, items, W->nW, W->T, W->Hq, W->Hkv, W->G, nf, nit, nsplit, W->part,
                 W->wstat);
    else
      e = launch(attend_valu_kernel<DT, D, false>, dim3(nsplit, U), dim3(256), 0, st, E(0), q, kf,
                 vf, codes, qsc, items, W->nW, W->T, W->Hq, W->Hkv, W->G, nf, nit, nsplit, W->part,
                 W->wstat);
    if (e != hipSuccess) return e;
  }
  if (event)
    e = launch(merge_kernel<D, true>, dim3(W->G, U), dim3(D), 0, st, E(2),
               static_cast<const float*>(W->part), nsplit, W->G, W->Hq, W->Hkv, out, W->hstat);
  else
    e = launch(merge_kernel<D, false>, dim3(W->G, U), dim3(D), 0, st, E(2),
               static_cast<const float*>(W->part), nsplit, W->G, W->Hq, W->Hkv, out, W->hstat);
  if (e != hipSuccess || !event) return e;
  const float2* ws = W->wstat;
  const float2* hs = W->hstat;
#define RSKV_ROUTE(NP)                                                                         \
  launch(route_kernel<NP>, dim3(U), dim3(1024), 0, st, E(3), ws, hs, W->G, W->nW, nit,         \
         W->n_full, W->n_quant, W->items, W->tier, W->score, W->mass,                           \
         static_cast<const uint8_t*>(W->has_code), W->trans, W->ntrans)
  if (W->nW <= 1024)
    e = RSKV_ROUTE(1024);
  else if (W->nW <= 2048)
    e = RSKV_ROUTE(2048);
  else if (W->nW <= 4096)
    e = RSKV_ROUTE(4096);
  else if (W->nW <= 8192)
    e = RSKV_ROUTE(8192);
  else
    e = RSKV_ROUTE(16384);
#undef RSKV_ROUTE
  if (e != hipSuccess) return e;
  const int nb = std::max(1, std::min(64, W->nW));
  return launch(transition_kernel<DT, D>, dim3(nb, U), dim3(256), 0, st, E(4),
                static_cast<T*>(W->kf), static_cast<T*>(W->vf), W->codes, W->qsc, W->has_code,
                static_cast<const int32_t*>(W->trans), static_cast<const int32_t*>(W->ntrans), W->nW);
}

template <int DT, int D>
hipError_t build_impl(const rskv_window* W, const void* K, const void* V, hipStream_t st) {
  typedef typename Elem<DT>::T T;
  const int U = W->B * W->Hkv;
  const int rows = W->nW * kRows;
  dim3 grid((rows * (D / 8) + 255) / 256, U);
  hipLaunchKernelGGL((build_kernel<DT, D>), grid, dim3(256), 0, st, static_cast<const T*>(K),
                     static_cast<const T*>(V), W->T, rows, static_cast<T*>(W->kf),
                     static_cast<T*>(W->vf));
  return hipGetLastError();
}

}  // namespace

void attend_splits(const rskv_window* W, int nf, int nq, int* nsf, int* nsq) {
  const int U = W->B * W->Hkv;
  if (W->dtype == RSKV_BF16) {
    // one wave per window at most, and one round of resident waves: about
    // 2048 waves of the full-window kernel (two per SIMD) and 4096 of the
    // INT2 one (four per SIMD) in all (measured: more waves lengthen the
    // tail and the merge)
    const int wf = std::min(nf, (2048 + U - 1) / U);
    const int wq = std::min(nq, (4096 + U - 1) / U);
    *nsf = (wf + 3) / 4;
    *nsq = (wq + 3) / 4;
    return;
  }
  // block-cooperative kernel: one range per workgroup, ranges of at least
  // one full window's cost
  const long long cost = static_cast<long long>(kCostFull) * nf + static_cast<long long>(kCostQuant) * nq;
  long long waves = std::min<long long>((cost + kCostFull - 1) / kCostFull, (kTargetWaves + U - 1) / U);
  *nsf = static_cast<int>(std::max<long long>(waves, 1));
  *nsq = 0;
}

hipError_t launch_build(const rskv_window* W, const void* K, const void* V, hipStream_t st) {
  if (W->dtype == RSKV_BF16)
    return W->d == 128 ? build_impl<kBF16, 128>(W, K, V, st) : build_impl<kBF16, 64>(W, K, V, st);
  return W->d == 128 ? build_impl<kF32, 128>(W, K, V, st) : build_impl<kF32, 64>(W, K, V, st);
}

hipError_t launch_decode(const rskv_window* W, const void* q, float* out, bool event, int nf, int nq,
                         hipStream_t st, const KernelEvents* ev, bool* recorded) {
  if (W->dtype == RSKV_BF16)
    return W->d == 128 ? decode_impl<kBF16, 128>(W, q, out, event, nf, nq, st, ev, recorded)
                       : decode_impl<kBF16, 64>(W, q, out, event, nf, nq, st, ev, recorded);
  return W->d == 128 ? decode_impl<kF32, 128>(W, q, out, event, nf, nq, st, ev, recorded)
                     : decode_impl<kF32, 64>(W, q, out, event, nf, nq, st, ev, recorded);
}

}  // namespace win
}  // namespace rskv
