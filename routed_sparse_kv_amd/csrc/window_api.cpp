// C ABI of the window-routed three-tier cache (rskv_window.h): option
// checks, allocation, build, decode orchestration (the routing-event
// schedule and the tier counts the next step attends), state export and
// per-kernel timing.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "window.h"

namespace {

using rskv::report_error;
namespace W = rskv::win;

int hip_fail(hipError_t e, const char* what) {
  return report_error(RSKV_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define WIN_HIP(expr, what)                          \
  do {                                               \
    hipError_t e_ = (expr);                          \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool valid(const rskv_window* w) { return w != nullptr && w->magic == W::kMagic; }

size_t esize(int dtype) { return dtype == RSKV_BF16 ? 2 : 4; }

int dev_alloc(rskv_window* w, void** p, size_t bytes, const char* what) {
  *p = nullptr;
  bytes = std::max<size_t>(bytes, 16);
  void* q = w->mem.alloc(bytes, w->last_stream);
  if (q == nullptr)
    return report_error(RSKV_ENOMEM, std::string("device allocation failed: ") + what);
  w->allocs.push_back(q);
  w->bytes += bytes;
  *p = q;
  return RSKV_OK;
}

template <typename T>
int dev_array(rskv_window* w, T** p, size_t count, const char* what) {
  void* q = nullptr;
  int rc = dev_alloc(w, &q, count * sizeof(T), what);
  *p = static_cast<T*>(q);
  return rc;
}

void free_cache(rskv_window* w) {
  if (w == nullptr) return;
  // the last stream only; then every block goes back to the allocator
  (void)hipStreamSynchronize(w->last_stream);
  for (void* p : w->allocs) w->mem.release(p, w->last_stream);
  for (hipEvent_t e : w->pending)
    if (e != nullptr) (void)hipEventDestroy(e);
  for (hipEvent_t e : w->pool) (void)hipEventDestroy(e);
  w->magic = 0;
  delete w;
}

struct Guard {
  rskv_window* w;
  ~Guard() {
    if (w) free_cache(w);
  }
};

int check_opts(const rskv_window_opts* o) {
  if (o == nullptr) return report_error(RSKV_EINVAL, "opts is NULL");
  if (o->dtype != RSKV_F32 && o->dtype != RSKV_BF16)
    return report_error(RSKV_EDTYPE, "dtype must be RSKV_F32 or RSKV_BF16");
  if (o->batch < 1 || o->n_q_heads < 1 || o->n_kv_heads < 1 || o->context_len < 1)
    return report_error(RSKV_EINVAL, "batch, heads and context_len must be >= 1");
  if (o->n_q_heads % o->n_kv_heads)
    return report_error(RSKV_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
  if (o->n_q_heads / o->n_kv_heads > W::kMaxG)
    return report_error(RSKV_EINVAL, "query group size above 16 is not supported");
  if (o->head_dim != 64 && o->head_dim != 128)
    return report_error(RSKV_EINVAL, "head_dim must be 64 or 128");
  if (o->context_len > W::kMaxWindows * W::kRows)
    return report_error(RSKV_EINVAL, "context_len must be <= 2^20");
  if (o->n_full < 0 || o->n_quant < 0 || o->n_full + o->n_quant < 1)
    return report_error(RSKV_EINVAL, "n_full and n_quant must be >= 0 with n_full + n_quant >= 1");
  if (!rskv::valid_hook(o->allocator))
    return report_error(RSKV_EINVAL, "allocator needs both alloc and free, or neither");
  if (o->route_every < 1) return report_error(RSKV_EINVAL, "route_every must be >= 1");
  const long long nW = (o->context_len + W::kRows - 1) / W::kRows;
  if (static_cast<long long>(o->batch) * o->n_kv_heads * nW * W::kRows * o->head_dim > (1ll << 40))
    return report_error(RSKV_EINVAL, "cache too large");
  return RSKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int rskv_window_build(const void* K, const void* V, const rskv_window_opts* o, void* stream,
                      rskv_window** out) {
  try {
    if (out == nullptr) return report_error(RSKV_EINVAL, "out is NULL");
    *out = nullptr;
    int rc = check_opts(o);
    if (rc != RSKV_OK) return rc;
    if (K == nullptr || V == nullptr) return report_error(RSKV_EINVAL, "K and V must be non-NULL");
    rskv_window* w = new rskv_window();
    Guard guard{w};
    hipStream_t st = static_cast<hipStream_t>(stream);
    w->last_stream = st;
    w->mem.hook = o->allocator;
    w->B = o->batch;
    w->Hq = o->n_q_heads;
    w->Hkv = o->n_kv_heads;
    w->G = w->Hq / w->Hkv;
    w->d = o->head_dim;
    w->T = o->context_len;
    w->dtype = o->dtype;
    w->n_full = o->n_full;
    w->n_quant = o->n_quant;
    w->R = o->route_every;
    w->nW = (w->T + W::kRows - 1) / W::kRows;
    w->nf_next = w->nW;
    w->nq_next = 0;
    const int nf1 = std::min(w->n_full, w->nW);
    const int nq1 = std::min(w->n_quant, w->nW - nf1);
    int a0, b0, a1, b1;
    W::attend_splits(w, w->nW, 0, &a0, &b0);
    W::attend_splits(w, nf1, nq1, &a1, &b1);
    w->nsplit_max = std::max(a0 + b0, a1 + b1);

    const size_t U = static_cast<size_t>(w->B) * w->Hkv;
    const size_t nW = static_cast<size_t>(w->nW);
    const size_t d = static_cast<size_t>(w->d);
    if ((rc = dev_alloc(w, &w->kf, U * nW * W::kRows * d * esize(w->dtype), "full-precision keys")) ||
        (rc = dev_alloc(w, &w->vf, U * nW * W::kRows * d * esize(w->dtype), "full-precision values")) ||
        (rc = dev_array(w, &w->codes, U * nW * W::code_words(w->d), "ledger codes")) ||
        (rc = dev_array(w, &w->qsc, U * nW * W::scale_floats(w->d), "ledger scales")) ||
        (rc = dev_array(w, &w->has_code, U * nW, "ledger flags")) ||
        (rc = dev_array(w, &w->tier, U * nW, "tiers")) ||
        (rc = dev_array(w, &w->score, U * nW, "scores")) ||
        (rc = dev_array(w, &w->mass, U * nW, "masses")) ||
        (rc = dev_array(w, &w->items, U * nW, "attended windows")) ||
        (rc = dev_array(w, &w->trans, U * 2 * nW, "transition lists")) ||
        (rc = dev_array(w, &w->ntrans, U * 2, "transition counts")) ||
        (rc = dev_array(w, &w->part, U * w->nsplit_max * w->G * (d + 2), "partials")) ||
        (rc = dev_array(w, &w->wstat, U * nW * w->G, "window statistics")) ||
        (rc = dev_array(w, &w->hstat, U * w->G, "head statistics")))
      return rc;
    WIN_HIP(hipMemsetAsync(w->codes, 0, U * nW * W::code_words(w->d) * sizeof(uint32_t), st), "clear");
    WIN_HIP(hipMemsetAsync(w->qsc, 0, U * nW * W::scale_floats(w->d) * sizeof(float), st), "clear");
    WIN_HIP(hipMemsetAsync(w->has_code, 0, U * nW, st), "clear");
    WIN_HIP(hipMemsetAsync(w->tier, 0, U * nW, st), "clear");
    WIN_HIP(hipMemsetAsync(w->score, 0, U * nW * sizeof(double), st), "clear");
    WIN_HIP(hipMemsetAsync(w->mass, 0, U * nW * sizeof(double), st), "clear");
    WIN_HIP(hipMemsetAsync(w->ntrans, 0, U * 2 * sizeof(int32_t), st), "clear");
    std::vector<int32_t> ident(U * nW);
    for (size_t u = 0; u < U; ++u)
      for (size_t j = 0; j < nW; ++j) ident[u * nW + j] = static_cast<int32_t>(j);
    WIN_HIP(hipMemcpyAsync(w->items, ident.data(), ident.size() * sizeof(int32_t),
                           hipMemcpyHostToDevice, st),
            "list upload");
    WIN_HIP(W::launch_build(w, K, V, st), "build launch");
    WIN_HIP(hipStreamSynchronize(st), "build synchronize");
    w->magic = W::kMagic;
    *out = w;
    guard.w = nullptr;
    return RSKV_OK;
  } catch (const std::bad_alloc&) {
    return report_error(RSKV_ENOMEM, "host allocation failed");
  } catch (...) {
    return report_error(RSKV_EINVAL, "unexpected error in rskv_window_build");
  }
}

int rskv_window_decode(rskv_window* w, const void* q, float* out, void* stream) {
  try {
    if (!valid(w)) return report_error(RSKV_ESTATE, "invalid window cache handle");
    if (q == nullptr || out == nullptr) return report_error(RSKV_EINVAL, "q and out must be non-NULL");
    if (!aligned16(q)) return report_error(RSKV_EINVAL, "q must be 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    w->last_stream = st;
    const bool event = w->step % w->R == 0;
    const int nf = w->nf_next, nq = w->nq_next;
    hipError_t e;
    if (!w->prof_on) {
      e = W::launch_decode(w, q, out, event, nf, nq, st, nullptr, nullptr);
      if (e != hipSuccess) return hip_fail(e, "decode launch");
    } else {
      rskv::KernelEvents ev[W::kKernels];
      for (auto& k : ev)
        for (hipEvent_t* p : {&k.start, &k.stop}) {
          if (w->pool.empty()) {
            hipEvent_t n;
            WIN_HIP(hipEventCreate(&n), "event create");
            w->pool.push_back(n);
          }
          *p = w->pool.back();
          w->pool.pop_back();
        }
      bool rec[W::kKernels];
      e = W::launch_decode(w, q, out, event, nf, nq, st, ev, rec);
      for (int k = 0; k < W::kKernels; ++k) {
        if (rec[k] && e == hipSuccess) {
          w->pending.push_back(ev[k].start);
          w->pending.push_back(ev[k].stop);
        } else {
          w->pending.push_back(nullptr);
          w->pending.push_back(nullptr);
          w->pool.push_back(ev[k].start);
          w->pool.push_back(ev[k].stop);
        }
      }
      if (e != hipSuccess) return hip_fail(e, "decode launch");
      if (event) ++w->prof_events;
    }
    if (event) {
      // every window still attended is ranked; the first n_full stay (or
      // become) full precision, the next n_quant INT2
      const int live = nf + nq;
      w->nf_next = std::min(w->n_full, live);
      w->nq_next = std::min(w->n_quant, live - w->nf_next);
    }
    ++w->step;
    return RSKV_OK;
  } catch (const std::bad_alloc&) {
    return report_error(RSKV_ENOMEM, "host allocation failed");
  } catch (...) {
    return report_error(RSKV_EINVAL, "unexpected error in rskv_window_decode");
  }
}

int rskv_window_info_get(const rskv_window* w, rskv_window_info* i) {
  if (!valid(w)) return report_error(RSKV_ESTATE, "invalid window cache handle");
  if (i == nullptr) return report_error(RSKV_EINVAL, "info is NULL");
  i->batch = w->B;
  i->n_q_heads = w->Hq;
  i->n_kv_heads = w->Hkv;
  i->head_dim = w->d;
  i->context_len = w->T;
  i->dtype = w->dtype;
  i->n_full = w->n_full;
  i->n_quant = w->n_quant;
  i->route_every = w->R;
  i->n_windows = w->nW;
  i->step = w->step;
  i->next_full = w->nf_next;
  i->next_quant = w->nq_next;
  int a, b;
  W::attend_splits(w, w->nf_next, w->nq_next, &a, &b);
  i->next_splits = a + b;
  i->full_bytes = static_cast<int32_t>(2 * W::kRows * w->d * esize(w->dtype));
  i->quant_bytes = static_cast<int32_t>(W::code_words(w->d) * 4 + W::scale_floats(w->d) * 4);
  i->device_bytes = w->bytes;
  return RSKV_OK;
}

int rskv_window_state_get(const rskv_window* w, rskv_window_state* s) {
  try {
    if (!valid(w)) return report_error(RSKV_ESTATE, "invalid window cache handle");
    if (s == nullptr) return report_error(RSKV_EINVAL, "state is NULL");
    WIN_HIP(hipStreamSynchronize(w->last_stream), "state synchronize");
    const size_t U = static_cast<size_t>(w->B) * w->Hkv;
    const size_t nW = static_cast<size_t>(w->nW);
    const int d = w->d;
    const size_t rows = nW * W::kRows;
    auto cp = [&](void* dst, const void* src, size_t bytes) -> hipError_t {
      if (dst == nullptr || bytes == 0) return hipSuccess;
      return hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
    };
    WIN_HIP(cp(s->tier, w->tier, U * nW), "state");
    WIN_HIP(cp(s->score, w->score, U * nW * sizeof(double)), "state");
    WIN_HIP(cp(s->mass, w->mass, U * nW * sizeof(double)), "state");
    WIN_HIP(cp(s->has_code, w->has_code, U * nW), "state");
    if (s->code_k || s->code_v || s->scale_k || s->min_k || s->scale_v || s->min_v) {
      std::vector<uint32_t> cw(U * nW * W::code_words(d));
      std::vector<float> qs(U * nW * W::scale_floats(d));
      WIN_HIP(cp(cw.data(), w->codes, cw.size() * 4), "state");
      WIN_HIP(cp(qs.data(), w->qsc, qs.size() * 4), "state");
      const int ng = d / W::kGroup;
      for (size_t wi = 0; wi < U * nW; ++wi) {
        const uint32_t* c = cw.data() + wi * W::code_words(d);
        const float* q = qs.data() + wi * W::scale_floats(d);
        for (int r = 0; r < W::kRows; ++r) {
          for (int col = 0; col < d; ++col) {
            int bit;
            const size_t o = (wi * W::kRows + r) * d + col;
            if (s->code_k) s->code_k[o] = (c[W::code_word(0, r, col, d, &bit)] >> bit) & 3u;
            if (s->code_v) s->code_v[o] = (c[W::code_word(1, r, col, d, &bit)] >> bit) & 3u;
          }
          for (int g = 0; g < ng; ++g) {
            const size_t o = (wi * W::kRows + r) * ng + g;
            if (s->scale_k) s->scale_k[o] = q[W::kq_off(r, g, 0, d)];
            if (s->min_k) s->min_k[o] = q[W::kq_off(r, g, 1, d)];
            if (s->scale_v) s->scale_v[o] = q[W::vq_off(r, g, 0, d)];
            if (s->min_v) s->min_v[o] = q[W::vq_off(r, g, 1, d)];
          }
        }
      }
    }
    const size_t es = esize(w->dtype);
    for (int kv = 0; kv < 2; ++kv) {
      char* dst = static_cast<char*>(kv ? s->v : s->k);
      if (dst == nullptr) continue;
      std::vector<char> tiled(U * rows * d * es);
      WIN_HIP(cp(tiled.data(), kv ? w->vf : w->kf, tiled.size()), "state");
      for (size_t u = 0; u < U; ++u)
        for (size_t r = 0; r < rows; ++r)
          for (int col = 0; col < d; ++col) {
            const size_t src = u * rows * d + (kv ? rskv::v32_off(static_cast<int>(r), col, d)
                                                  : rskv::k16_off(static_cast<int>(r), col, d));
            memcpy(dst + ((u * rows + r) * d + col) * es, tiled.data() + src * es, es);
          }
    }
    return RSKV_OK;
  } catch (const std::bad_alloc&) {
    return report_error(RSKV_ENOMEM, "host allocation failed");
  }
}

int rskv_window_profile_enable(rskv_window* w, int32_t on) {
  if (!valid(w)) return report_error(RSKV_ESTATE, "invalid window cache handle");
  w->prof_on = on != 0;
  return RSKV_OK;
}

int rskv_window_profile_read(rskv_window* w, rskv_window_profile* p) {
  if (!valid(w)) return report_error(RSKV_ESTATE, "invalid window cache handle");
  if (p == nullptr) return report_error(RSKV_EINVAL, "prof is NULL");
  constexpr int kEv = 2 * W::kKernels;
  for (size_t s = 0; s + kEv <= w->pending.size(); s += kEv) {
    for (int k = 0; k < W::kKernels; ++k) {
      hipEvent_t a = w->pending[s + 2 * k], b = w->pending[s + 2 * k + 1];
      if (a == nullptr) continue;
      WIN_HIP(hipEventSynchronize(b), "event synchronize");
      float ms = 0.f;
      WIN_HIP(hipEventElapsedTime(&ms, a, b), "event elapsed");
      w->prof_ms[k] += ms;
    }
    ++w->prof_steps;
  }
  for (hipEvent_t e : w->pending)
    if (e != nullptr) w->pool.push_back(e);
  w->pending.clear();
  p->steps = w->prof_steps;
  p->events = w->prof_events;
  for (int k = 0; k < W::kKernels; ++k) p->ms[k] = w->prof_ms[k];
  return RSKV_OK;
}

void rskv_window_destroy(rskv_window* w) {
  if (valid(w)) free_cache(w);
}

}  // extern "C"
