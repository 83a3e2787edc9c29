// Device memory of a library object through the caller's allocator hook
// (rskv_allocator in rskv.h) or, without one, hipMalloc / hipFree.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/rskv.h"

namespace rskv {

struct DevMem {
  rskv_allocator hook{};

  // A device block of at least `bytes` bytes usable on `st`, or null.
  void* alloc(size_t bytes, hipStream_t st) const {
    if (hook.alloc != nullptr) return hook.alloc(hook.ctx, bytes, static_cast<void*>(st));
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    return p;
  }

  // Releases a block from alloc(); `st` has been synchronised by the caller.
  void release(void* p, hipStream_t st) const {
    if (p == nullptr) return;
    if (hook.alloc != nullptr) {
      if (hook.free != nullptr) hook.free(hook.ctx, p, static_cast<void*>(st));
      return;
    }
    (void)hipFree(p);
  }
};

// A hook needs both functions, or neither.
inline bool valid_hook(const rskv_allocator& a) {
  return (a.alloc == nullptr) == (a.free == nullptr);
}

}  // namespace rskv
