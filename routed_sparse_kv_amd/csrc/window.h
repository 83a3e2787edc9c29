// Window-routed three-tier cache (QEvict form) of librskv: host object,
// ledger layouts and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/rskv_window.h"
#include "cache.h"
#include "layout.h"

namespace rskv {
namespace win {

constexpr int kRows = RSKV_WINDOW_ROWS;    // positions per window
constexpr int kGroup = RSKV_WINDOW_GROUP;  // coordinates per INT2 scale group
constexpr int kMaxG = 16;                  // query heads per KV head (MFMA columns)
constexpr int kMaxWindows = 16384;         // windows per unit the routing sort holds
constexpr int kKernels = 5;  // attend (full windows), attend (INT2 windows), merge, route, transition
constexpr uint32_t kMagic = 0x52534b57u;   // "RSKW"

// Ledger of one window (INT2 codes of K and V plus fp32 scales and minima).
//
// Codes: 8 d uint32 words, K side then V side, 4 d words each, laid out as
// [part = t / 4][lane 0..63][t % 4] for the lane's word t < d / 16, so that
// a wave reads one side with d / 64 16-byte loads per lane.  Word t of a
// lane holds the 8-code MFMA operands o = 2 t and 2 t + 1; code j of
// operand o (o' = o % 2) sits at bit 4 j + 2 o', so that
// (word >> 2 o') & 0x33333333 holds the operand's codes as the 4-bit
// floating-point (e2m1) values 0, 0.5, 1, 1.5, one per nibble, which the
// hardware widens to bf16 two at a time.
//   K side, operand o = rb16 * (d / 32) + kb: lane l holds row 16 rb16 + l % 16,
//     columns 32 kb + 8 (l / 16) + j (the A operand of the QK product).
//   V side, operand o = rb32 * (d / 16) + cb: lane l holds column
//     16 cb + l % 16 of rows 32 rb32 + v32_row(l / 16, j) (the A operand of
//     the transposed PV product).
RSKV_HD int code_words(int d) { return 8 * d; }
RSKV_HD void code_elem(int side, int o, int lane, int j, int d, int* r, int* c) {
  if (side == 0) {
    const int kbn = d >> 5;
    *r = (o / kbn) * 16 + (lane & 15);
    *c = (o % kbn) * 32 + 8 * (lane >> 4) + j;
  } else {
    const int cbn = d >> 4;
    *r = (o / cbn) * 32 + v32_row(lane >> 4, j);
    *c = (o % cbn) * 16 + (lane & 15);
  }
}
// Word (within the window's 8 d words) and bit of the code of row r,
// column c of `side`.
RSKV_HD int code_word(int side, int r, int c, int d, int* bit) {
  int lane, o, j;
  if (side == 0) {
    lane = (r & 15) | (((c & 31) >> 3) << 4);
    o = (r >> 4) * (d >> 5) + (c >> 5);
    j = c & 7;
  } else {
    const int rr = r & 31;
    lane = (((rr & 15) >> 2) << 4) | (c & 15);
    o = (r >> 5) * (d >> 4) + (c >> 4);
    j = (rr & 3) + 4 * (rr >> 4);
  }
  const int t = o >> 1;
  *bit = 4 * j + 2 * (o & 1);
  return side * 4 * d + ((t >> 2) * 64 + lane) * 4 + (t & 3);
}

// Scales and minima: 256 (d / 64) floats per window, in the order the lane
// groups of the attention kernel read them.  K block first,
// [rb16][g][group][i][scale, min] for row 16 rb16 + 4 g + i (the rows of a
// QK output lane group); V block next, [rb32][g][group][e][scale, min] for
// row 32 rb32 + v32_row(g, e) (the rows of a PV operand lane group).
RSKV_HD int scale_floats(int d) { return 256 * (d / kGroup); }
RSKV_HD int kq_off(int r, int grp, int which, int d) {
  const int ng = d / kGroup;
  return (((r >> 2) * ng + grp) * 4 + (r & 3)) * 2 + which;
}
RSKV_HD int vq_off(int r, int grp, int which, int d) {
  const int ng = d / kGroup;
  const int rr = r & 31;
  const int g = (rr & 15) >> 2;
  const int e = (rr & 3) + 4 * (rr >> 4);
  return 128 * ng + ((((r >> 5) * 4 + g) * ng + grp) * 8 + e) * 2 + which;
}

}  // namespace win
}  // namespace rskv

struct rskv_window {
  uint32_t magic = 0;
  int B = 0, Hq = 0, Hkv = 0, G = 0, d = 0, T = 0, dtype = 0;
  int n_full = 0, n_quant = 0, R = 1;
  int nW = 0;                // windows per unit
  int64_t step = 0;          // decode steps done
  int nf_next = 0, nq_next = 0;
  int nsplit_max = 0;        // attention workgroups per unit, largest of the two phases
  // full-precision store [U][nW * 64 rows] in K16 / V32 tiles (layout.h)
  void* kf = nullptr;
  void* vf = nullptr;
  uint32_t* codes = nullptr;   // [U][nW][8 d] ledger codes
  float* qsc = nullptr;        // [U][nW][256 d / 64] ledger scales and minima
  uint8_t* has_code = nullptr; // [U][nW]
  int8_t* tier = nullptr;      // [U][nW]
  double* score = nullptr;     // [U][nW]
  double* mass = nullptr;      // [U][nW] masses of the last routing event
  int32_t* items = nullptr;    // [U][nW] attended windows, full ones first
  int32_t* trans = nullptr;    // [U][2][nW] windows to quantise, to promote
  int32_t* ntrans = nullptr;   // [U][2]
  float* part = nullptr;       // [U][nsplit][G][d + 2]
  float2* wstat = nullptr;     // [U][nW][G] per attended window: max and sum of e^(s - max)
  float2* hstat = nullptr;     // [U][G] per head: softmax max and denominator
  rskv::DevMem mem;  // allocator of the device memory
  std::vector<void*> allocs;
  size_t bytes = 0;
  hipStream_t last_stream = nullptr;
  bool prof_on = false;
  int64_t prof_steps = 0, prof_events = 0;
  double prof_ms[rskv::win::kKernels] = {};
  std::vector<hipEvent_t> pending;  // 2 * kKernels per recorded step
  std::vector<hipEvent_t> pool;
};

namespace rskv {
namespace win {

// Attention workgroups per unit for nf full and nq INT2 windows: *nsf of
// the full-window kernel (of the block-cooperative kernel for fp32
// caches, which takes both) and *nsq of the INT2 kernel.
void attend_splits(const rskv_window* w, int nf, int nq, int* nsf, int* nsq);

// Copies the caller's K, V [U][T][d] into the tiled store (rows past T zero).
hipError_t launch_build(const rskv_window* w, const void* K, const void* V, hipStream_t st);

// One decode step: attention and merge, then on routing events the routing
// and the ledger transitions.  `ev` is null or holds kKernels start/stop
// pairs; `recorded[k]` tells which were recorded.
hipError_t launch_decode(const rskv_window* w, const void* q, float* out, bool event, int nf, int nq,
                         hipStream_t st, const KernelEvents* ev, bool* recorded);

}  // namespace win
}  // namespace rskv
