// Token-retrieval index (ParisKV-style router) of librskv: host object and
// kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/rskv_retrieval.h"
#include "cache.h"

namespace rskv {
namespace ret {

constexpr int kChunk = 4096;    // keys per vote / compaction workgroup
constexpr int kMaxBins = 264;   // vote totals 0 .. (d/8) * rho <= 256, padded
constexpr int kRows = 64;       // attention rows per workgroup (one per lane)
constexpr int kMaxRho = 16;
constexpr int kKernels = 10;    // decode launches (profile slots)
constexpr int kSelBlock = 2048; // estimates per top-k workgroup (one block)
constexpr int kSelBins = 4096;  // value bins of the top-k histogram
constexpr int kSelMaxBlocks = 1024;  // blocks per unit the top-k handles

// sigma as bits: bit c of w[c / 32] set <=> sigma_c = -1 (d <= 128).
struct SignMask {
  uint32_t w[4];
};

// Magnitude bins of a code: bin j covers beta[j] <= |u_t| < beta[j+1]
// (beta[0] = 0, beta[8] = 1 implied), dequantised to lam[j].
struct Codebook {
  double beta[8];
  double lam[8];
};

}  // namespace ret
}  // namespace rskv

struct rskv_retrieval {
  uint32_t magic = 0;
  int B = 0, Hq = 0, Hkv = 0, G = 0, d = 0, T = 0, dtype = 0, m = 8, Bs = 0, rho = 0;
  int k_ret = 0, kv_tier = 0;
  double cand_frac = 0;
  // regions: Sink [0, ns), retrieval [ns, l0) (N keys), Local [l0, T) (nl)
  int ns = 0, l0 = 0, nl = 0, N = 0, C = 0, n_sel = 0, n_att = 0, n_near = 0;
  int rec_bytes = 0, nchunk = 0, nbins = 0, nsplit = 0;
  int nsb = 0;      // top-k blocks per unit, ceil(C / kSelBlock)
  int nrwg = 0;     // rerank workgroups per unit, ceil(C / 256)
  size_t npad = 0;  // pitch of the per-unit score arrays
  rskv::ret::SignMask signs{};
  rskv::ret::Codebook cb{};
  // stored K/V: Sink then Local rows [U][n_near][d]; retrieval rows [U][N][d]
  void* k_near = nullptr;
  void* v_near = nullptr;
  void* k_far = nullptr;
  void* v_far = nullptr;
  uint8_t* buckets = nullptr;  // [U][N][Bs]
  uint8_t* rec = nullptr;      // [U][N][rec_bytes]: codes d/2 bytes, w Bs fp32
  // decode workspace
  double* qt = nullptr;        // [U][d]
  double* qn = nullptr;        // [U]
  uint8_t* votes = nullptr;    // [U][Bs][256]
  uint32_t* tot = nullptr;     // [U][kMaxBins] vote-total histogram
  uint16_t* scores = nullptr;  // [U][npad]
  uint16_t* chist = nullptr;   // [U][nchunk][kMaxBins] per-chunk counts >= s
  int32_t* thr = nullptr;      // [U][2]
  int32_t* cand = nullptr;     // [U][C]
  float* est = nullptr;        // [U][C]
  uint32_t* rmm = nullptr;     // [U][nrwg][2] smallest / largest estimate (order keys)
                               // of each rerank workgroup
  uint32_t* rng = nullptr;     // [U][2] the unit's estimate range (order keys)
  uint32_t* ehtot = nullptr;   // [U][kSelBins] histogram of the estimates over the range
  int32_t* gtb = nullptr;      // [U][nsb] keys above the crossing bin, per block
  float* lval = nullptr;       // [U][C] crossing-bin members: estimate
  int32_t* lidx = nullptr;     // [U][C] crossing-bin members: candidate index
  uint32_t* lcnt = nullptr;    // [U] crossing-bin members
  int32_t* soff = nullptr;     // [U][nsb] first output slot of each block
  int32_t* selp = nullptr;     // [U][2] threshold (fp32 bits), last tied index taken
  int32_t* sel = nullptr;      // [U][n_sel]
  float* part = nullptr;       // [U][nsplit][G][d + 2]
  rskv::DevMem mem;  // allocator of the device memory
  std::vector<void*> allocs;
  std::vector<void*> host_allocs;
  size_t bytes = 0, host_bytes = 0;
  hipStream_t last_stream = nullptr;
  // per-kernel timing
  bool prof_on = false;
  int64_t prof_steps = 0;
  double prof_ms[rskv::ret::kKernels] = {};
  std::vector<hipEvent_t> pending;  // 2 * kKernels per recorded step
  std::vector<hipEvent_t> pool;
};

namespace rskv {
namespace ret {

constexpr uint32_t kMagic = 0x52534b52u;  // "RSKR"

// Rotates and encodes the retrieval region of every unit, reading the
// caller's K [U][T][d].
hipError_t launch_encode(const rskv_retrieval* r, const void* K, hipStream_t st);

// One decode step (at most ten launches); `ev` is null or holds kKernels start/stop
// pairs, one per launch (a skipped launch leaves its pair unrecorded and
// `recorded[k]` false).
hipError_t launch_decode(const rskv_retrieval* r, const void* q, float* out, int32_t* retrieved,
                         hipStream_t st, const KernelEvents* ev, bool* recorded);

}  // namespace ret
}  // namespace rskv
