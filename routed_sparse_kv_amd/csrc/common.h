// Device helpers shared by the rskv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace rskv {

constexpr int kWave = 64;

enum : int { kF32 = 0, kBF16 = 1 };

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp64 -> bf16, round to nearest, ties to even, done on the fp64 pattern:
// bf16 keeps 7 explicit mantissa bits of the 52, so 45 low bits are dropped.
// The rounded value has 8 significant bits and converts to fp32 exactly.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(x));
  u += ((1ull << 44) - 1ull) + ((u >> 45) & 1ull);
  u &= ~((1ull << 45) - 1ull);
  const float f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));
  return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

// Element access by storage type.  F32 arrays hold float, BF16 raw bits.
template <int DT> struct Elem;
template <> struct Elem<kF32> {
  typedef float T;
  static __device__ __forceinline__ float ld(const T* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ T from_f64(double x) { return static_cast<float>(x); }
  static __device__ __forceinline__ T from_f32(float x) { return x; }
};
template <> struct Elem<kBF16> {
  typedef uint16_t T;
  static __device__ __forceinline__ float ld(const T* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ T from_f64(double x) { return f64_to_bf16(x); }
  static __device__ __forceinline__ T from_f32(float x) { return f64_to_bf16(static_cast<double>(x)); }
};

// -------------------------------------------------------------- orderings

// Monotone map of fp32 onto uint32 (ascending), with -0 folded onto +0.
__device__ __forceinline__ uint32_t f32_order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Monotone map of fp64 onto uint64 (ascending), with -0 folded onto +0.
__device__ __forceinline__ unsigned long long f64_order_key(double x) {
  unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(x));
  if ((u << 1) == 0ull) u = 0ull;
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// ------------------------------------------------------------ reductions

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <typename T>
__device__ __forceinline__ T group_sum(T v, int width) {
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum over a wave.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const T t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Inclusive prefix sum over a wave with DPP row shifts and row broadcasts
// (no LDS traffic): shifts by 1, 2, 4, 8 scan each row of 16 lanes, then
// lane 15 of rows 0 and 2 is added to rows 1 and 3, and lane 31 to rows 2
// and 3.
__device__ __forceinline__ int wave_incl_scan_dpp(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Wave-wide minimum and maximum of 64-bit unsigned keys (result in every
// lane).  Each DPP step moves both 32-bit halves; lanes without a source
// keep their own value, the identity of min and max.
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v, int ctrl_id) {
  const int lo = static_cast<int>(v & 0xffffffffull);
  const int hi = static_cast<int>(v >> 32);
  int a, b;
  switch (ctrl_id) {
    case 0: a = __builtin_amdgcn_update_dpp(lo, lo, 0x111, 0xf, 0xf, false);
            b = __builtin_amdgcn_update_dpp(hi, hi, 0x111, 0xf, 0xf, false); break;
    case 1: a = __builtin_amdgcn_update_dpp(lo, lo, 0x112, 0xf, 0xf, false);
            b = __builtin_amdgcn_update_dpp(hi, hi, 0x112, 0xf, 0xf, false); break;
    case 2: a = __builtin_amdgcn_update_dpp(lo, lo, 0x114, 0xf, 0xf, false);
            b = __builtin_amdgcn_update_dpp(hi, hi, 0x114, 0xf, 0xf, false); break;
    case 3: a = __builtin_amdgcn_update_dpp(lo, lo, 0x118, 0xf, 0xf, false);
            b = __builtin_amdgcn_update_dpp(hi, hi, 0x118, 0xf, 0xf, false); break;
    case 4: a = __builtin_amdgcn_update_dpp(lo, lo, 0x142, 0xa, 0xf, false);
            b = __builtin_amdgcn_update_dpp(hi, hi, 0x142, 0xa, 0xf, false); break;
    default: a = __builtin_amdgcn_update_dpp(lo, lo, 0x143, 0xc, 0xf, false);
             b = __builtin_amdgcn_update_dpp(hi, hi, 0x143, 0xc, 0xf, false); break;
  }
  return (static_cast<unsigned long long>(static_cast<unsigned>(b)) << 32) |
         static_cast<unsigned>(a);
}
__device__ __forceinline__ void wave_min_max_u64(unsigned long long& mn, unsigned long long& mx) {
#pragma unroll
  for (int c = 0; c < 6; ++c) {
    const unsigned long long a = dpp_u64(mn, c);
    const unsigned long long b = dpp_u64(mx, c);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  // lane 63 holds the wave result
  mn = (static_cast<unsigned long long>(static_cast<unsigned>(
            __builtin_amdgcn_readlane(static_cast<int>(mn >> 32), 63))) << 32) |
       static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(mn & 0xffffffffull), 63));
  mx = (static_cast<unsigned long long>(static_cast<unsigned>(
            __builtin_amdgcn_readlane(static_cast<int>(mx >> 32), 63))) << 32) |
       static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(mx & 0xffffffffull), 63));
}

// Wave-wide minimum and maximum of doubles (result in every lane; NaN-free
// inputs).
__device__ __forceinline__ void wave_min_max_f64(double& mn, double& mx) {
#pragma unroll
  for (int c = 0; c < 6; ++c) {
    const double a = __longlong_as_double(static_cast<long long>(
        dpp_u64(static_cast<unsigned long long>(__double_as_longlong(mn)), c)));
    const double b = __longlong_as_double(static_cast<long long>(
        dpp_u64(static_cast<unsigned long long>(__double_as_longlong(mx)), c)));
    mn = fmin(mn, a);
    mx = fmax(mx, b);
  }
  const long long a = __double_as_longlong(mn), b = __double_as_longlong(mx);
  const int alo = __builtin_amdgcn_readlane(static_cast<int>(a & 0xffffffffll), 63);
  const int ahi = __builtin_amdgcn_readlane(static_cast<int>(a >> 32), 63);
  const int blo = __builtin_amdgcn_readlane(static_cast<int>(b & 0xffffffffll), 63);
  const int bhi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), 63);
  mn = __longlong_as_double((static_cast<long long>(ahi) << 32) | static_cast<unsigned>(alo));
  mx = __longlong_as_double((static_cast<long long>(bhi) << 32) | static_cast<unsigned>(blo));
}

// Inverse of f64_order_key.
__device__ __forceinline__ double f64_from_order_key(unsigned long long k) {
  const unsigned long long b = (k & 0x8000000000000000ull) ? (k ^ 0x8000000000000000ull) : ~k;
  return __longlong_as_double(static_cast<long long>(b));
}

// Exclusive prefix sum over the whole block (blockDim.x a multiple of 64,
// at most 1024).  `scratch` holds >= 17 values of shared memory.  Returns
// the exclusive prefix of v and the block total in *total.  Contains
// barriers: every thread of the block must call it.
template <typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* scratch, T* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const T incl = wave_incl_scan(v);
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const T w = lane < nw ? scratch[lane] : T(0);
    const T ws = wave_incl_scan(w);
    if (lane < nw) scratch[lane] = ws - w;
    if (lane == nw - 1) scratch[16] = ws;
  }
  __syncthreads();
  const T r = scratch[wid] + incl - v;
  *total = scratch[16];
  __syncthreads();
  return r;
}

// Block-wide minimum and maximum (same calling rules as block_excl_scan;
// `scratch` holds >= 32 doubles of shared memory).
__device__ __forceinline__ void block_min_max(double& mn, double& mx, double* scratch) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    mn = fmin(mn, __shfl_xor(mn, o, kWave));
    mx = fmax(mx, __shfl_xor(mx, o, kWave));
  }
  if (lane == 0) {
    scratch[wid] = mn;
    scratch[16 + wid] = mx;
  }
  __syncthreads();
  mn = scratch[0];
  mx = scratch[16];
  for (int w = 1; w < nw; ++w) {
    mn = fmin(mn, scratch[w]);
    mx = fmax(mx, scratch[16 + w]);
  }
  __syncthreads();
}

}  // namespace rskv
