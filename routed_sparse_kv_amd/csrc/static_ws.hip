// Allocation-free decode: rskv_decode_step with its decode workspace in a
// file-scope device array of the library instead of the cache's own, for
// callers that cannot allocate device memory (see rskv.h).
#include <mutex>
#include <string>

#include "cache.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per device
constexpr int kMaxDevices = 64;

// One copy per GPU the library runs on, held until the process ends.  In
// host code `scratch` names a host-side stand-in: the kernels receive the
// device address of the current GPU's copy (scratch_base), never the name.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_base[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current.
int scratch_base(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return rskv::report_error(RSKV_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return rskv::report_error(RSKV_EINVAL, "device index outside the static scratch table");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_base[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return rskv::report_error(RSKV_EHIP, std::string("hipGetSymbolAddress(scratch): ") +
                                               hipGetErrorString(e));
    g_base[dev] = p;
  }
  *out = g_base[dev];
  return RSKV_OK;
}

}  // namespace

extern "C" int rskv_decode_step_static(rskv_cache* c, const void* q, float tau, int32_t k_max,
                                       float* out, int32_t* sel, int32_t* n_sel, void* stream) {
  try {
    int rc = rskv::check_decode(c, q, tau, k_max, out);
    if (rc != RSKV_OK) return rc;
    const size_t need = rskv::decode_ws_bytes(c);
    if (need > kScratchBytes)
      return rskv::report_error(
          RSKV_ECAPACITY, "decode workspace of this cache needs " + std::to_string(need) +
                              " bytes; the static scratch holds " +
                              std::to_string(kScratchBytes) + " (use rskv_decode_step)");
    void* base = nullptr;
    if ((rc = scratch_base(&base)) != RSKV_OK) return rc;
    return rskv::decode_with(c, rskv::carve_ws(c, base), q, tau, k_max, out, sel, n_sel,
                             static_cast<hipStream_t>(stream), false);
  } catch (...) {
    return rskv::report_error(RSKV_EINVAL, "unexpected error in rskv_decode_step_static");
  }
}

extern "C" size_t rskv_decode_static_capacity(void) { return kScratchBytes; }
