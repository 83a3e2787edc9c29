// C ABI of librskv: argument checks, cache allocation, build orchestration,
// the decode step, appends, import/export and per-kernel timing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "cache.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return RSKV_EHIP;
}

#define RSKV_HIP(expr, what)                         \
  do {                                               \
    hipError_t e_ = (expr);                          \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr int kMaxG = 16;
constexpr int kMaxRank = 32;

size_t elem_size(int dtype) { return dtype == RSKV_BF16 ? 2 : 4; }

bool valid_cache(const rskv_cache* c) { return c != nullptr && c->magic == rskv::kMagic; }

int check_opts(const rskv_build_opts* o, int rank) {
  if (o == nullptr) return fail(RSKV_EINVAL, "opts is NULL");
  if (o->dtype != RSKV_F32 && o->dtype != RSKV_BF16)
    return fail(RSKV_EDTYPE, "dtype must be RSKV_F32 or RSKV_BF16");
  if (o->batch < 1 || o->n_kv_heads < 1 || o->n_q_heads < 1 || o->context_len < 1)
    return fail(RSKV_EINVAL, "batch, heads and context_len must be >= 1");
  if (o->n_q_heads % o->n_kv_heads != 0)
    return fail(RSKV_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
  if (o->n_q_heads / o->n_kv_heads > kMaxG)
    return fail(RSKV_EINVAL, "query group size above 16 is not supported");
  if (o->head_dim != 64 && o->head_dim != 128)
    return fail(RSKV_EINVAL, "head_dim must be 64 or 128");
  if (!(o->anchor_frac >= 0.0 && o->anchor_frac <= 1.0))
    return fail(RSKV_EINVAL, "anchor_frac must lie in [0, 1]");
  if (rank < 1 || rank > kMaxRank) return fail(RSKV_EINVAL, "rank must lie in [1, 32]");
  if (o->tail_capacity < 0) return fail(RSKV_EINVAL, "tail_capacity must be >= 0");
  if (o->proj != nullptr && o->n_proj != 1 && o->n_proj != o->n_kv_heads)
    return fail(RSKV_EINVAL, "n_proj must be 1 or n_kv_heads");
  if (!(o->alpha == o->alpha)) return fail(RSKV_EINVAL, "alpha is NaN");
  if (o->factor_tier != RSKV_TIER_HBM && o->factor_tier != RSKV_TIER_HOST)
    return fail(RSKV_EINVAL, "factor_tier must be RSKV_TIER_HBM or RSKV_TIER_HOST");
  if (!rskv::valid_hook(o->allocator))
    return fail(RSKV_EINVAL, "allocator needs both alloc and free, or neither");
  return RSKV_OK;
}

// Allocation of one device array, tracked by the cache.
template <typename T>
int dev_alloc(rskv_cache* c, T** p, size_t count, const char* what) {
  *p = nullptr;
  const size_t bytes = std::max<size_t>(count, 1) * sizeof(T);
  void* q = c->mem.alloc(bytes, c->last_stream);
  if (q == nullptr) return fail(RSKV_ENOMEM, std::string("device allocation failed: ") + what);
  c->allocs.push_back(q);
  c->bytes += bytes;
  *p = static_cast<T*>(q);
  return RSKV_OK;
}

int dev_alloc_bytes(rskv_cache* c, void** p, size_t bytes, const char* what) {
  char* q = nullptr;
  int rc = dev_alloc(c, &q, bytes, what);
  *p = q;
  return rc;
}

// Zero-filled pinned host memory, tracked by the cache; the kernels use the
// same address (unified addressing) and read it over the host link.
int host_alloc_bytes(rskv_cache* c, void** p, size_t bytes, const char* what) {
  *p = nullptr;
  bytes = std::max<size_t>(bytes, 1);
  void* q = nullptr;
  hipError_t e = hipHostMalloc(&q, bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(RSKV_ENOMEM, std::string("pinned host allocation failed: ") + what);
  }
  memset(q, 0, bytes);
  c->host_allocs.push_back(q);
  c->host_bytes += bytes;
  *p = q;
  return RSKV_OK;
}

// Waits for the cache's last stream only, then releases its memory.
void free_cache(rskv_cache* c) {
  if (c == nullptr) return;
  (void)hipStreamSynchronize(c->last_stream);
  for (void* p : c->allocs) c->mem.release(p, c->last_stream);
  for (void* p : c->host_allocs) (void)hipHostFree(p);
  for (auto* list : {&c->prof.pending, &c->prof.app_pending})
    for (hipEvent_t e : *list)
      if (e != nullptr) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->prof.pool) (void)hipEventDestroy(e);
  c->magic = 0;
  delete c;
}

struct CacheGuard {
  rskv_cache* c;
  ~CacheGuard() {
    if (c) free_cache(c);
  }
};

// Sizes of the stored arrays, in elements.
struct Sizes {
  size_t summary, vmean, full, a, w, wv, slogit;
};

Sizes sizes_of(const rskv_cache* c) {
  const size_t U = static_cast<size_t>(c->B) * c->Hkv;
  const size_t d = c->d, r = c->rank;
  return Sizes{U * c->S * d, U * c->Sp * d, U * c->Fp * d, U * c->Np * r, U * c->S * r * d,
               U * c->S * rskv::rank4(c->rank) * d, U * c->Sp * c->G};
}

// Allocates the stored arrays and the decode workspace once the padded
// dimensions are known.  Everything is zero-filled.
int alloc_arrays(rskv_cache* c, hipStream_t st) {
  const size_t U = static_cast<size_t>(c->B) * c->Hkv;
  const size_t es = elem_size(c->dtype);
  const size_t d = c->d, S = c->S;
  const Sizes z = sizes_of(c);
  auto& v = c->dev;
  int rc;
#define ALLOC(ptr, n, what) \
  if ((rc = dev_alloc(c, &(ptr), (n), what)) != RSKV_OK) return rc
#define ALLOCB(ptr, n, what) \
  if ((rc = dev_alloc_bytes(c, &(ptr), (n), what)) != RSKV_OK) return rc
  ALLOC(v.span_start, c->B * S, "span_start");
  ALLOC(v.span_len, c->B * S, "span_len");
  ALLOC(v.tok_off, c->B * (S + 1), "tok_off");
  ALLOC(v.tok_pad, c->B * (S + 1), "tok_pad");
  ALLOC(v.full_pos, static_cast<size_t>(c->B) * c->F, "full_pos");
  ALLOC(v.n_spans, c->B, "n_spans");
  ALLOC(v.n_full, c->B, "n_full");
  ALLOC(v.n_full0, c->B, "n_full0");
  ALLOC(v.h_full, static_cast<size_t>(c->B) * c->F, "h_full");
  ALLOC(v.theta, c->B, "theta");
  ALLOC(v.last_anchor, c->B, "last_anchor");
  ALLOCB(v.summary, z.summary * es, "summary");
  ALLOCB(v.vmean, z.vmean * es, "vmean");
  ALLOC(v.log_len, c->B * S, "log_len");
  ALLOCB(v.k_full, z.full * es, "k_full");
  ALLOCB(v.v_full, z.full * es, "v_full");
  const bool host = c->factor_tier == RSKV_TIER_HOST;
#define ALLOCF(ptr, n, what)                                                      \
  if ((rc = host ? host_alloc_bytes(c, &(ptr), (n), what)                         \
                 : dev_alloc_bytes(c, &(ptr), (n), what)) != RSKV_OK) return rc
  ALLOCF(v.a_k, z.a * es, "a_k");
  ALLOCF(v.a_v, z.a * es, "a_v");
  ALLOCF(v.w_k, z.w * es, "w_k");
  ALLOCF(v.w_v, z.wv * es, "w_v");
#undef ALLOCF
  ALLOC(v.z, U * S, "z");
  ALLOC(v.slogit, z.slogit, "slogit");
  ALLOC(v.sel, U * S, "sel");
  ALLOC(v.sel_desc, U * S * 4, "sel_desc");
  ALLOC(v.n_sel, U, "n_sel");
  c->nsplit_max = rskv::decode_nsplit_max(c->B, c->Hkv, c->S, c->F, c->k_max_cap);
  ALLOC(v.wstart, U * (4 * c->nsplit_max + 1), "wstart");
  ALLOC(v.part, U * c->nsplit_max * c->G * (d + 2), "part");
  // span closing: one workgroup per (unit, K or V), launched only when some
  // sequence can see a decoded anchor
  c->close_grid = c->close_rows > 0 ? static_cast<int>(2 * U) : 0;
#undef ALLOC
#undef ALLOCB
  RSKV_HIP(hipMemsetAsync(v.summary, 0, z.summary * es, st), "memset summary");
  RSKV_HIP(hipMemsetAsync(v.vmean, 0, z.vmean * es, st), "memset vmean");
  RSKV_HIP(hipMemsetAsync(v.k_full, 0, z.full * es, st), "memset k_full");
  RSKV_HIP(hipMemsetAsync(v.v_full, 0, z.full * es, st), "memset v_full");
  if (!host) {  // host-tier factors are zeroed at allocation
    RSKV_HIP(hipMemsetAsync(v.a_k, 0, z.a * es, st), "memset a_k");
    RSKV_HIP(hipMemsetAsync(v.a_v, 0, z.a * es, st), "memset a_v");
    RSKV_HIP(hipMemsetAsync(v.w_k, 0, z.w * es, st), "memset w_k");
    RSKV_HIP(hipMemsetAsync(v.w_v, 0, z.wv * es, st), "memset w_v");
  }
  RSKV_HIP(hipMemsetAsync(v.log_len, 0, c->B * S * sizeof(float), st), "memset log_len");
  RSKV_HIP(hipMemsetAsync(v.slogit, 0, z.slogit * sizeof(float), st), "memset slogit");
  RSKV_HIP(hipMemsetAsync(v.n_sel, 0, U * sizeof(int32_t), st), "memset n_sel");
  RSKV_HIP(hipMemsetAsync(v.h_full, 0, static_cast<size_t>(c->B) * c->F * sizeof(float), st),
           "memset h_full");
  return RSKV_OK;
}

void init_header(rskv_cache* c, const rskv_build_opts* o, int rank) {
  c->magic = rskv::kMagic;
  c->B = o->batch;
  c->Hq = o->n_q_heads;
  c->Hkv = o->n_kv_heads;
  c->G = c->Hq / c->Hkv;
  c->d = o->head_dim;
  c->T = o->context_len;
  c->rank = rank;
  c->dtype = o->dtype;
  c->alpha = o->alpha > 0.f ? o->alpha : 8.f;
  c->tail_cap = o->tail_capacity;
  c->n_proj = o->proj != nullptr ? o->n_proj : 0;
  c->factor_tier = o->factor_tier;
  c->mem.hook = o->allocator;
}

int copy_proj(rskv_cache* c, const rskv_build_opts* o, hipStream_t st, bool from_host) {
  if (o->proj == nullptr) return RSKV_OK;
  const size_t n = static_cast<size_t>(c->n_proj) * c->d * c->d;
  int rc = dev_alloc(c, &c->dev.proj, n, "proj");
  if (rc != RSKV_OK) return rc;
  RSKV_HIP(hipMemcpyAsync(c->dev.proj, o->proj, n * sizeof(float),
                          from_host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDevice, st),
           "copy proj");
  return RSKV_OK;
}

// Padded dimensions from the per-sequence counts.  `la` holds the
// full-resolution row of each sequence's last anchor (-1 if none) and
// `theta` its anchor threshold: with a tail capacity, decoded anchors may
// close spans (streaming segmentation), so the span and span-token
// dimensions reserve room for them.  A closing needs a decoded anchor, and
// two closings at least one decoded non-anchor between them, so a sequence
// closes at most ceil(tail/2) spans, holding at most its tail run after the
// last anchor plus the decoded tokens.
void finish_sizes(rskv_cache* c, const rskv_build_opts* o, const std::vector<int>& la,
                  const std::vector<float>& theta) {
  int s_max = 0, f_max = 0, n_max = 0, p_max = 0, trail_max = 0;
  bool anchors = false;  // some sequence may see a decoded anchor
  for (int b = 0; b < c->B; ++b) {
    s_max = std::max(s_max, c->h_n_spans[b]);
    f_max = std::max(f_max, c->h_n_full0[b]);
    n_max = std::max(n_max, c->h_n_span_tokens[b]);
    p_max = std::max(p_max, c->h_n_tok_pad[b]);
    if (la[b] >= 0) trail_max = std::max(trail_max, c->h_n_full0[b] - la[b] - 1);
    anchors = anchors || la[b] >= 0 || theta[b] < HUGE_VALF;
  }
  const int closings = anchors && c->tail_cap > 0 ? (c->tail_cap + 1) / 2 : 0;
  c->close_rows = closings > 0 ? trail_max + c->tail_cap : 0;
  c->S = std::max(1, s_max + closings);
  c->F = std::max(1, f_max + c->tail_cap);
  c->N = std::max(1, n_max + c->close_rows);
  c->Sp = rskv::round_up(c->S, 32);
  c->Fp = rskv::round_up(c->F, 32);
  c->Np = std::max(16, p_max + (closings > 0 ? rskv::round_up(c->close_rows, 16) + 16 * closings
                                              : 0));
  c->k_max_cap = o->k_max_cap > 0 ? o->k_max_cap : 0x7fffffff;  // <= 0: no limit
}

// Host-side offsets of every span: plain and padded to 16 rows.
void span_offsets(const int32_t* len, int ns, std::vector<int>* off, std::vector<int>* pad) {
  off->assign(ns + 1, 0);
  pad->assign(ns + 1, 0);
  for (int j = 0; j < ns; ++j) {
    (*off)[j + 1] = (*off)[j] + len[j];
    (*pad)[j + 1] = (*pad)[j] + rskv::round_up(len[j], 16);
  }
}

// Conversion between the device layouts (layout.h) and the canonical
// row-major layout of rskv_host_arrays.  E is the element type by size.
template <typename E>
struct Relayout {
  const rskv_cache* c;
  const int32_t* span_len;  // [B][S_host], pitch ls
  int ls;
  const int* n_spans;       // [B] spans per sequence

  // dir = +1: device -> canonical; -1: canonical -> device.
  void full(E* canon, int F_c, E* dev, bool keys, int dir) const {
    const int d = c->d;
    for (int u = 0; u < c->B * c->Hkv; ++u)
      for (int r = 0; r < std::min(F_c, c->F); ++r)
        for (int k = 0; k < d; ++k) {
          const size_t dv = static_cast<size_t>(u) * c->Fp * d +
                            (keys ? rskv::k16_off(r, k, d) : rskv::v32_off(r, k, d));
          E& cv = canon[(static_cast<size_t>(u) * F_c + r) * d + k];
          if (dir > 0) cv = dev[dv]; else dev[dv] = cv;
        }
  }
  void vmean(E* canon, int S_c, E* dev, int dir) const {
    const int d = c->d;
    for (int u = 0; u < c->B * c->Hkv; ++u)
      for (int j = 0; j < std::min(S_c, c->S); ++j)
        for (int k = 0; k < d; ++k) {
          const size_t dv = static_cast<size_t>(u) * c->Sp * d + rskv::v32_off(j, k, d);
          E& cv = canon[(static_cast<size_t>(u) * S_c + j) * d + k];
          if (dir > 0) cv = dev[dv]; else dev[dv] = cv;
        }
  }
  void factors_a(E* canon, int N_c, E* dev, bool transposed, int dir) const {
    const int r = c->rank;
    std::vector<int> off, pad;
    for (int b = 0; b < c->B; ++b) {
      const int ns = n_spans[b];
      span_offsets(span_len + static_cast<size_t>(b) * ls, ns, &off, &pad);
      for (int h = 0; h < c->Hkv; ++h) {
        const size_t u = static_cast<size_t>(b) * c->Hkv + h;
        for (int j = 0; j < ns; ++j)
          for (int t = 0; t < off[j + 1] - off[j]; ++t)
            for (int k = 0; k < r; ++k) {
              const int tp = pad[j] + t;
              const size_t dv = u * c->Np * r + (transposed ? rskv::avt_off(tp, k, r)
                                                            : static_cast<size_t>(tp) * r + k);
              E& cv = canon[(u * N_c + off[j] + t) * r + k];
              if (dir > 0) cv = dev[dv]; else dev[dv] = cv;
            }
      }
    }
  }
  void factors_wv(E* canon, int S_c, E* dev, int dir) const {
    const int r = c->rank, d = c->d;
    for (int u = 0; u < c->B * c->Hkv; ++u)
      for (int j = 0; j < std::min(S_c, c->S); ++j)
        for (int k = 0; k < r; ++k)
          for (int e = 0; e < d; ++e) {
            const size_t dv = static_cast<size_t>(u) * c->S * d * rskv::rank4(r) + rskv::wvt_off(j, k, e, d, r);
            E& cv = canon[((static_cast<size_t>(u) * S_c + j) * r + k) * d + e];
            if (dir > 0) cv = dev[dv]; else dev[dv] = cv;
          }
  }
};

template <typename E>
int export_arrays(const rskv_cache* c, const std::vector<int>& ns, rskv_host_arrays* a) {
  const auto& v = c->dev;
  const Sizes z = sizes_of(c);
  const size_t U = static_cast<size_t>(c->B) * c->Hkv;
  const int S = c->S, F = c->F, N = c->N, d = c->d, r = c->rank;
  std::vector<int32_t> lens(static_cast<size_t>(c->B) * S);
  RSKV_HIP(hipMemcpy(lens.data(), v.span_len, lens.size() * 4, hipMemcpyDeviceToHost), "export");
  Relayout<E> rl{c, lens.data(), S, ns.data()};
  std::vector<E> tmp;
  auto fetch = [&](const void* src, size_t n) -> int {
    tmp.assign(n, E(0));
    hipError_t e = hipMemcpy(tmp.data(), src, n * sizeof(E), hipMemcpyDefault);
    return e == hipSuccess ? RSKV_OK : hip_fail(e, "export copy");
  };
  int rc;
  if (a->summary) {
    RSKV_HIP(hipMemcpy(a->summary, v.summary, z.summary * sizeof(E), hipMemcpyDeviceToHost),
             "export summary");
  }
  if (a->w_k) {
    RSKV_HIP(hipMemcpy(a->w_k, v.w_k, z.w * sizeof(E), hipMemcpyDefault), "export w_k");
  }
  if (a->vmean) {
    if ((rc = fetch(v.vmean, z.vmean))) return rc;
    rl.vmean(static_cast<E*>(a->vmean), S, tmp.data(), +1);
  }
  if (a->k_full) {
    if ((rc = fetch(v.k_full, z.full))) return rc;
    rl.full(static_cast<E*>(a->k_full), F, tmp.data(), true, +1);
  }
  if (a->v_full) {
    if ((rc = fetch(v.v_full, z.full))) return rc;
    rl.full(static_cast<E*>(a->v_full), F, tmp.data(), false, +1);
  }
  if (a->a_k) {
    if ((rc = fetch(v.a_k, z.a))) return rc;
    memset(a->a_k, 0, U * N * r * sizeof(E));
    rl.factors_a(static_cast<E*>(a->a_k), N, tmp.data(), false, +1);
  }
  if (a->a_v) {
    if ((rc = fetch(v.a_v, z.a))) return rc;
    memset(a->a_v, 0, U * N * r * sizeof(E));
    rl.factors_a(static_cast<E*>(a->a_v), N, tmp.data(), true, +1);
  }
  if (a->w_v) {
    if ((rc = fetch(v.w_v, z.wv))) return rc;
    rl.factors_wv(static_cast<E*>(a->w_v), S, tmp.data(), +1);
  }
  (void)d;
  return RSKV_OK;
}

template <typename E>
int import_arrays(rskv_cache* c, const rskv_host_arrays* a, int S_in, int F_in, int N_in) {
  auto& v = c->dev;
  const Sizes z = sizes_of(c);
  const size_t U = static_cast<size_t>(c->B) * c->Hkv;
  const int d = c->d, r = c->rank;
  Relayout<E> rl{c, a->span_len, S_in, c->h_n_spans.data()};
  std::vector<E> tmp;
  auto put = [&](void* dst, size_t n, const char* what) -> int {
    hipError_t e = hipMemcpy(dst, tmp.data(), n * sizeof(E), hipMemcpyDefault);
    return e == hipSuccess ? RSKV_OK : hip_fail(e, what);
  };
  int rc;
  // summary and W_K: canonical on both sides, re-pitched
  tmp.assign(z.summary, E(0));
  for (size_t u = 0; u < U; ++u)
    for (int j = 0; j < std::min(S_in, c->S); ++j)
      memcpy(&tmp[(u * c->S + j) * d], static_cast<const E*>(a->summary) + (u * S_in + j) * d,
             d * sizeof(E));
  if ((rc = put(v.summary, z.summary, "import summary"))) return rc;
  tmp.assign(z.w, E(0));
  for (size_t u = 0; u < U; ++u)
    for (int j = 0; j < std::min(S_in, c->S); ++j)
      memcpy(&tmp[(u * c->S + j) * r * d],
             static_cast<const E*>(a->w_k) + (u * S_in + j) * r * d, r * d * sizeof(E));
  if ((rc = put(v.w_k, z.w, "import w_k"))) return rc;
  tmp.assign(z.vmean, E(0));
  rl.vmean(static_cast<E*>(const_cast<void*>(static_cast<const void*>(a->vmean))), S_in,
           tmp.data(), -1);
  if ((rc = put(v.vmean, z.vmean, "import vmean"))) return rc;
  tmp.assign(z.full, E(0));
  rl.full(static_cast<E*>(a->k_full), F_in, tmp.data(), true, -1);
  if ((rc = put(v.k_full, z.full, "import k_full"))) return rc;
  tmp.assign(z.full, E(0));
  rl.full(static_cast<E*>(a->v_full), F_in, tmp.data(), false, -1);
  if ((rc = put(v.v_full, z.full, "import v_full"))) return rc;
  tmp.assign(z.a, E(0));
  rl.factors_a(static_cast<E*>(a->a_k), N_in, tmp.data(), false, -1);
  if ((rc = put(v.a_k, z.a, "import a_k"))) return rc;
  tmp.assign(z.a, E(0));
  rl.factors_a(static_cast<E*>(a->a_v), N_in, tmp.data(), true, -1);
  if ((rc = put(v.a_v, z.a, "import a_v"))) return rc;
  tmp.assign(z.wv, E(0));
  rl.factors_wv(static_cast<E*>(a->w_v), S_in, tmp.data(), -1);
  if ((rc = put(v.w_v, z.wv, "import w_v"))) return rc;
  return RSKV_OK;
}

}  // namespace

namespace rskv {
int report_error(int code, const std::string& msg) { return fail(code, msg); }

DecodeWs cache_ws(const rskv_cache* c) {
  const auto& v = c->dev;
  DecodeWs w;
  w.z = v.z;
  w.slogit = v.slogit;
  w.sel = v.sel;
  w.sel_desc = v.sel_desc;
  w.n_sel = v.n_sel;
  w.wstart = v.wstart;
  w.part = v.part;
  return w;
}

namespace {
// Bytes of the workspace arrays, in DecodeWs order (sizes as alloc_arrays).
void ws_array_bytes(const rskv_cache* c, size_t* b) {
  const size_t U = static_cast<size_t>(c->B) * c->Hkv;
  b[0] = U * c->S * sizeof(double);
  b[1] = U * c->Sp * c->G * sizeof(float);
  b[2] = U * c->S * sizeof(int32_t);
  b[3] = U * c->S * 4 * sizeof(int32_t);
  b[4] = U * sizeof(int32_t);
  b[5] = U * (4 * c->nsplit_max + 1) * sizeof(int32_t);
  b[6] = U * c->nsplit_max * c->G * (c->d + 2) * sizeof(float);
}
size_t align256(size_t x) { return (std::max<size_t>(x, 1) + 255) & ~size_t(255); }
}  // namespace

size_t decode_ws_bytes(const rskv_cache* c) {
  size_t b[7], total = 0;
  ws_array_bytes(c, b);
  for (size_t x : b) total += align256(x);
  return total;
}

DecodeWs carve_ws(const rskv_cache* c, void* base) {
  size_t b[7];
  ws_array_bytes(c, b);
  char* p = static_cast<char*>(base);
  void* a[7];
  for (int i = 0; i < 7; ++i) {
    a[i] = p;
    p += align256(b[i]);
  }
  DecodeWs w;
  w.z = static_cast<double*>(a[0]);
  w.slogit = static_cast<float*>(a[1]);
  w.sel = static_cast<int32_t*>(a[2]);
  w.sel_desc = static_cast<int32_t*>(a[3]);
  w.n_sel = static_cast<int32_t*>(a[4]);
  w.wstart = static_cast<int32_t*>(a[5]);
  w.part = static_cast<float*>(a[6]);
  return w;
}

int decode_with(rskv_cache* c, const DecodeWs& ws, const void* q, float tau, int k_max,
                float* out, int32_t* sel, int32_t* n_sel, hipStream_t st, bool profile) {
  c->last_stream = st;
  const int nsplit = decode_nsplit(c, k_max);
  const int nwaves = attend_uses_mfma(c) ? 4 * nsplit : 0;
  constexpr int kK = kProfileKernels;
  KernelEvents ev[kK];
  const bool prof = profile && c->prof.on;
  if (prof) {
    for (int i = 0; i < kK; ++i) {
      for (hipEvent_t* e : {&ev[i].start, &ev[i].stop}) {
        if (c->prof.pool.empty()) {
          hipEvent_t n;
          RSKV_HIP(hipEventCreate(&n), "event create");
          c->prof.pool.push_back(n);
        }
        *e = c->prof.pool.back();
        c->prof.pool.pop_back();
      }
    }
  }
  RSKV_HIP(launch_route(c, ws, q, st, prof ? &ev[0] : nullptr), "route kernel");
  const bool fused = attend_fuses_topk(c, k_max);
  const SelectArgs sa{tau, k_max, sel, n_sel};
  if (fused) {
    // the attention kernel selects: the top-k slot of the profile stays at 0
    if (prof) {
      c->prof.pool.push_back(ev[1].start);
      c->prof.pool.push_back(ev[1].stop);
      ev[1] = KernelEvents{};
    }
  } else {
    RSKV_HIP(launch_topk(c, ws, tau, k_max, nwaves, sel, n_sel, st, prof ? &ev[1] : nullptr),
             "topk kernel");
  }
  RSKV_HIP(launch_attend(c, ws, q, nsplit, fused ? &sa : nullptr, st, prof ? &ev[2] : nullptr),
           "attend kernel");
  RSKV_HIP(launch_merge(c, ws, nsplit, out, st, prof ? &ev[3] : nullptr), "merge kernel");
  if (prof) {
    for (int i = 0; i < kK; ++i) {
      c->prof.pending.push_back(ev[i].start);
      c->prof.pending.push_back(ev[i].stop);
    }
  }
  return RSKV_OK;
}

// Argument checks shared by the decode entry points.
int check_decode(const rskv_cache* c, const void* q, float tau, int k_max, const float* out) {
  if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
  if (q == nullptr || out == nullptr) return fail(RSKV_EINVAL, "q and out must be non-NULL");
  if (tau != tau) return fail(RSKV_EINVAL, "tau is NaN");
  if (k_max < 0) return fail(RSKV_EINVAL, "k_max must be >= 0");
  if (k_max > c->k_max_cap) return fail(RSKV_ECAPACITY, "k_max exceeds k_max_cap");
  return RSKV_OK;
}
}  // namespace rskv

extern "C" {

const char* rskv_last_error(void) { return g_err.c_str(); }

const char* rskv_version(void) { return "rskv 0.2.0 (gfx950)"; }

int rskv_build_spans(const float* surprisal, const void* K, const void* V, int32_t rank,
                     const rskv_build_opts* opts, void* stream, rskv_cache** out) {
  try {
    if (out == nullptr) return fail(RSKV_EINVAL, "out is NULL");
    *out = nullptr;
    int rc = check_opts(opts, rank);
    if (rc != RSKV_OK) return rc;
    if (surprisal == nullptr || K == nullptr || V == nullptr)
      return fail(RSKV_EINVAL, "surprisal, K and V must be device pointers");
    hipStream_t st = static_cast<hipStream_t>(stream);
    rskv_cache* c = new rskv_cache();
    CacheGuard guard{c};
    init_header(c, opts, rank);
    c->last_stream = st;
    const int B = c->B, T = c->T;
    const int n_anchor = static_cast<int>(floor(opts->anchor_frac * static_cast<double>(T)));

    // ---- segmentation into temporaries of pitch T (T + 1 for offsets)
    rc = dev_alloc(c, &c->dev.span_id, static_cast<size_t>(B) * T, "span_id");
    if (rc != RSKV_OK) return rc;
    std::vector<void*> tmps;
    auto tmp_alloc = [&](int32_t** p, size_t n) -> int {
      void* q = c->mem.alloc(std::max<size_t>(n, 1) * sizeof(int32_t), st);
      if (q == nullptr)
        return fail(RSKV_ENOMEM, "device allocation failed: segmentation temporaries");
      tmps.push_back(q);
      *p = static_cast<int32_t*>(q);
      return RSKV_OK;
    };
    struct TmpFree {
      std::vector<void*>* v;
      const rskv::DevMem* mem;
      hipStream_t st;
      ~TmpFree() {
        if (!v->empty()) (void)hipStreamSynchronize(st);
        for (void* p : *v) mem->release(p, st);
      }
    } tmp_free{&tmps, &c->mem, st};
    int32_t *start_tmp, *len_tmp, *tokoff_tmp, *tokpad_tmp, *full_tmp, *counts;
    const size_t BT = static_cast<size_t>(B) * T, BT1 = static_cast<size_t>(B) * (T + 1);
    if ((rc = tmp_alloc(&start_tmp, BT)) != RSKV_OK) return rc;
    if ((rc = tmp_alloc(&len_tmp, BT)) != RSKV_OK) return rc;
    if ((rc = tmp_alloc(&tokoff_tmp, BT1)) != RSKV_OK) return rc;
    if ((rc = tmp_alloc(&tokpad_tmp, BT1)) != RSKV_OK) return rc;
    if ((rc = tmp_alloc(&full_tmp, BT)) != RSKV_OK) return rc;
    if ((rc = tmp_alloc(&counts, static_cast<size_t>(B) * rskv::kCounts)) != RSKV_OK) return rc;
    RSKV_HIP(rskv::launch_segment(surprisal, B, T, n_anchor, c->dev.span_id, start_tmp, len_tmp,
                                  tokoff_tmp, tokpad_tmp, full_tmp, counts, st),
             "segment kernel");
    std::vector<int32_t> hc(static_cast<size_t>(B) * rskv::kCounts);
    RSKV_HIP(hipMemcpyAsync(hc.data(), counts, hc.size() * sizeof(int32_t),
                            hipMemcpyDeviceToHost, st),
             "copy counts");
    RSKV_HIP(hipStreamSynchronize(st), "segment kernel");
    c->h_n_anchor.resize(B);
    c->h_n_spans.resize(B);
    c->h_n_full0.resize(B);
    c->h_n_span_tokens.resize(B);
    c->h_n_tok_pad.resize(B);
    std::vector<int> la(B);
    std::vector<float> theta(B);
    for (int b = 0; b < B; ++b) {
      const int32_t* cb = &hc[rskv::kCounts * b];
      if (cb[0] < 0) return fail(RSKV_EINVAL, "surprisal holds NaN");
      c->h_n_anchor[b] = cb[0];
      c->h_n_spans[b] = cb[1];
      c->h_n_full0[b] = cb[2];
      c->h_n_span_tokens[b] = cb[3];
      c->h_n_tok_pad[b] = cb[4];
      la[b] = cb[5];
      memcpy(&theta[b], &cb[6], sizeof(float));
    }
    finish_sizes(c, opts, la, theta);
    if ((rc = alloc_arrays(c, st)) != RSKV_OK) return rc;
    if ((rc = copy_proj(c, opts, st, false)) != RSKV_OK) return rc;
    auto& v = c->dev;
    RSKV_HIP(hipMemcpyAsync(v.last_anchor, la.data(), B * sizeof(int32_t), hipMemcpyHostToDevice,
                            st),
             "copy last_anchor");
    RSKV_HIP(hipMemcpyAsync(v.theta, theta.data(), B * sizeof(float), hipMemcpyHostToDevice, st),
             "copy theta");
    const int kc = rskv::kCounts;
    RSKV_HIP(rskv::launch_copy_rows(v.span_start, c->S, start_tmp, T, counts, kc, 1, 0, 0, B, st),
             "copy span_start");
    RSKV_HIP(rskv::launch_copy_rows(v.span_len, c->S, len_tmp, T, counts, kc, 1, 0, 0, B, st),
             "copy span_len");
    RSKV_HIP(rskv::launch_copy_rows(v.tok_off, c->S + 1, tokoff_tmp, T + 1, counts, kc, 1, 1, 0,
                                    B, st),
             "copy tok_off");
    RSKV_HIP(rskv::launch_copy_rows(v.tok_pad, c->S + 1, tokpad_tmp, T + 1, counts, kc, 1, 1, 0,
                                    B, st),
             "copy tok_pad");
    RSKV_HIP(rskv::launch_copy_rows(v.full_pos, c->F, full_tmp, T, counts, kc, 2, 0, -1, B, st),
             "copy full_pos");
    RSKV_HIP(hipMemcpyAsync(v.n_spans, c->h_n_spans.data(), B * sizeof(int32_t),
                            hipMemcpyHostToDevice, st),
             "copy n_spans");
    RSKV_HIP(hipMemcpyAsync(v.n_full, c->h_n_full0.data(), B * sizeof(int32_t),
                            hipMemcpyHostToDevice, st),
             "copy n_full");
    RSKV_HIP(hipMemcpyAsync(v.n_full0, c->h_n_full0.data(), B * sizeof(int32_t),
                            hipMemcpyHostToDevice, st),
             "copy n_full0");
    // ---- summaries, packed rows, factors
    RSKV_HIP(rskv::launch_summary(c, surprisal, K, V, st), "summary kernel");
    RSKV_HIP(rskv::launch_pack(c, surprisal, K, V, st), "pack kernel");
    std::string ferr;
    hipError_t fe = rskv::launch_factor(c, K, V, st, &ferr);
    if (fe != hipSuccess) {
      if (!ferr.empty()) return fail(RSKV_ENOMEM, ferr);
      return hip_fail(fe, "factor kernel");
    }
    RSKV_HIP(hipStreamSynchronize(st), "build");
    guard.c = nullptr;
    *out = c;
    return RSKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(RSKV_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(RSKV_EINVAL, "unexpected error in rskv_build_spans");
  }
}

int rskv_decode_step(rskv_cache* c, const void* q, float tau, int32_t k_max, float* out,
                     int32_t* sel, int32_t* n_sel, void* stream) {
  try {
    int rc = rskv::check_decode(c, q, tau, k_max, out);
    if (rc != RSKV_OK) return rc;
    return rskv::decode_with(c, rskv::cache_ws(c), q, tau, k_max, out, sel, n_sel,
                             static_cast<hipStream_t>(stream), true);
  } catch (const std::bad_alloc&) {
    return fail(RSKV_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(RSKV_EINVAL, "unexpected error in rskv_decode_step");
  }
}

int rskv_decode_scores(const rskv_cache* c, double* z, int32_t* n_spans) {
  try {
    if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
    if (z == nullptr) return fail(RSKV_EINVAL, "z is NULL");
    RSKV_HIP(hipStreamSynchronize(c->last_stream), "scores synchronize");
    const size_t n = static_cast<size_t>(c->B) * c->Hkv * c->S;
    RSKV_HIP(hipMemcpy(z, c->dev.z, n * sizeof(double), hipMemcpyDeviceToHost), "scores copy");
    if (n_spans != nullptr)
      RSKV_HIP(hipMemcpy(n_spans, c->dev.n_spans, c->B * sizeof(int32_t), hipMemcpyDeviceToHost),
               "span counts copy");
    return RSKV_OK;
  } catch (...) {
    return fail(RSKV_EINVAL, "unexpected error in rskv_decode_scores");
  }
}

int rskv_append_token(rskv_cache* c, const void* k, const void* v, const float* h,
                      void* stream) {
  try {
    if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
    if (k == nullptr || v == nullptr) return fail(RSKV_EINVAL, "k and v must be non-NULL");
    if (c->appended >= c->tail_cap) return fail(RSKV_ECAPACITY, "tail capacity exhausted");
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    auto& pr = c->prof;
    rskv::KernelEvents ev[2];
    if (pr.on) {
      for (auto* e : {&ev[0].start, &ev[0].stop, &ev[1].start, &ev[1].stop}) {
        if (pr.pool.empty()) {
          hipEvent_t n;
          RSKV_HIP(hipEventCreate(&n), "event create");
          pr.pool.push_back(n);
        }
        *e = pr.pool.back();
        pr.pool.pop_back();
      }
    }
    // a closing needs an anchor threshold and the surprisal of the token
    const bool may_close = h != nullptr && c->close_grid > 0;
    if (may_close) {
      RSKV_HIP(rskv::launch_close(c, h, st, pr.on ? &ev[0] : nullptr), "close kernel");
    } else if (pr.on) {
      pr.pool.push_back(ev[0].start);
      pr.pool.push_back(ev[0].stop);
      ev[0] = rskv::KernelEvents{};
    }
    RSKV_HIP(rskv::launch_append(c, k, v, h, may_close, c->T + c->appended, st,
                                 pr.on ? &ev[1] : nullptr),
             "append kernel");
    if (pr.on)
      for (const auto& e : ev) {
        pr.app_pending.push_back(e.start);
        pr.app_pending.push_back(e.stop);
      }
    c->appended += 1;
    return RSKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(RSKV_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(RSKV_EINVAL, "unexpected error in rskv_append_token");
  }
}

int rskv_append_kv(rskv_cache* c, const void* k, const void* v, void* stream) {
  return rskv_append_token(c, k, v, nullptr, stream);
}

int rskv_cache_info_get(const rskv_cache* c, rskv_cache_info* info) {
  if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
  if (info == nullptr) return fail(RSKV_EINVAL, "info is NULL");
  info->batch = c->B;
  info->n_q_heads = c->Hq;
  info->n_kv_heads = c->Hkv;
  info->head_dim = c->d;
  info->context_len = c->T;
  info->rank = c->rank;
  info->dtype = c->dtype;
  info->n_spans_max = c->S;
  info->n_full_cap = c->F;
  info->n_span_tokens_max = c->N;
  info->tail_capacity = c->tail_cap;
  info->appended = c->appended;
  info->k_max_cap = c->k_max_cap;
  info->alpha = c->alpha;
  info->device_bytes = c->bytes;
  info->factor_tier = c->factor_tier;
  info->host_bytes = c->host_bytes;
  return RSKV_OK;
}

int rskv_cache_export(const rskv_cache* c, rskv_host_arrays* a) {
  try {
    if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
    if (a == nullptr) return fail(RSKV_EINVAL, "arrays is NULL");
    RSKV_HIP(hipDeviceSynchronize(), "export sync");
    const int B = c->B;
    const size_t S = c->S, F = c->F;
    const auto& v = c->dev;
    // counts as they stand on the device (appends and closings change them)
    std::vector<int> ns(B), nf(B), la(B), off(static_cast<size_t>(B) * (S + 1));
    RSKV_HIP(hipMemcpy(ns.data(), v.n_spans, B * 4, hipMemcpyDeviceToHost), "export n_spans");
    RSKV_HIP(hipMemcpy(nf.data(), v.n_full, B * 4, hipMemcpyDeviceToHost), "export n_full");
    RSKV_HIP(hipMemcpy(la.data(), v.last_anchor, B * 4, hipMemcpyDeviceToHost), "export la");
    RSKV_HIP(hipMemcpy(off.data(), v.tok_off, off.size() * 4, hipMemcpyDeviceToHost),
             "export tok_off");
    for (int b = 0; b < B; ++b) {
      if (a->n_anchor) a->n_anchor[b] = c->h_n_anchor[b];
      if (a->n_spans) a->n_spans[b] = ns[b];
      if (a->n_full) a->n_full[b] = nf[b];
      if (a->n_span_tokens) a->n_span_tokens[b] = off[static_cast<size_t>(b) * (S + 1) + ns[b]];
      if (a->last_anchor) a->last_anchor[b] = la[b];
    }
    auto cp = [&](void* dst, const void* src, size_t bytes, const char* what) -> int {
      if (dst == nullptr) return RSKV_OK;
      hipError_t e = hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
      return e == hipSuccess ? RSKV_OK : hip_fail(e, what);
    };
    int rc;
    if ((rc = cp(a->span_id, v.span_id, static_cast<size_t>(B) * c->T * 4, "export span_id")))
      return rc;
    if ((rc = cp(a->span_start, v.span_start, B * S * 4, "export span_start"))) return rc;
    if ((rc = cp(a->span_len, v.span_len, B * S * 4, "export span_len"))) return rc;
    if ((rc = cp(a->full_pos, v.full_pos, B * F * 4, "export full_pos"))) return rc;
    if ((rc = cp(a->log_len, v.log_len, B * S * 4, "export log_len"))) return rc;
    if ((rc = cp(a->h_full, v.h_full, B * F * 4, "export h_full"))) return rc;
    if ((rc = cp(a->theta, v.theta, B * 4, "export theta"))) return rc;
    return c->dtype == RSKV_BF16 ? export_arrays<uint16_t>(c, ns, a)
                                 : export_arrays<uint32_t>(c, ns, a);
  } catch (const std::bad_alloc&) {
    return fail(RSKV_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(RSKV_EINVAL, "unexpected error in rskv_cache_export");
  }
}

int rskv_cache_import(const rskv_host_arrays* a, const rskv_build_opts* opts, int32_t rank,
                      int32_t S_in, int32_t F_in, int32_t N_in, void* stream, rskv_cache** out) {
  try {
    if (out == nullptr) return fail(RSKV_EINVAL, "out is NULL");
    *out = nullptr;
    int rc = check_opts(opts, rank);
    if (rc != RSKV_OK) return rc;
    if (a == nullptr || a->n_spans == nullptr || a->n_full == nullptr ||
        a->n_span_tokens == nullptr || a->span_start == nullptr || a->span_len == nullptr ||
        a->full_pos == nullptr || a->summary == nullptr || a->vmean == nullptr ||
        a->log_len == nullptr || a->k_full == nullptr || a->v_full == nullptr ||
        a->a_k == nullptr || a->a_v == nullptr || a->w_k == nullptr || a->w_v == nullptr)
      return fail(RSKV_EINVAL, "import needs every array except span_id and n_anchor");
    if (S_in < 1 || F_in < 1 || N_in < 1) return fail(RSKV_EINVAL, "S, F, N must be >= 1");
    hipStream_t st = static_cast<hipStream_t>(stream);
    rskv_cache* c = new rskv_cache();
    CacheGuard guard{c};
    init_header(c, opts, rank);
    c->last_stream = st;
    const int B = c->B;
    c->h_n_anchor.assign(B, 0);
    c->h_n_spans.resize(B);
    c->h_n_full0.resize(B);
    c->h_n_span_tokens.resize(B);
    c->h_n_tok_pad.resize(B);
    std::vector<int> la(B, -1);
    std::vector<float> theta(B, HUGE_VALF);
    for (int b = 0; b < B; ++b) {
      const int ns = a->n_spans[b], nf = a->n_full[b], nt = a->n_span_tokens[b];
      if (ns < 0 || ns > S_in || nf < 0 || nf > F_in || nt < 0 || nt > N_in)
        return fail(RSKV_EINVAL, "counts exceed the padded dimensions");
      if (a->last_anchor != nullptr) {
        la[b] = a->last_anchor[b];
        if (la[b] < -1 || la[b] >= nf)
          return fail(RSKV_EINVAL, "last_anchor must be -1 or a full-resolution row");
      }
      if (a->theta != nullptr) {
        theta[b] = a->theta[b];
        if (theta[b] != theta[b]) return fail(RSKV_EINVAL, "theta holds NaN");
      }
      long long sum = 0, pad = 0;
      for (int j = 0; j < ns; ++j) {
        const int len = a->span_len[static_cast<size_t>(b) * S_in + j];
        if (len < 1) return fail(RSKV_EINVAL, "span lengths must be >= 1");
        sum += len;
        pad += rskv::round_up(len, 16);
      }
      if (sum != nt) return fail(RSKV_EINVAL, "n_span_tokens differs from the sum of lengths");
      c->h_n_anchor[b] = a->n_anchor ? a->n_anchor[b] : 0;
      c->h_n_spans[b] = ns;
      c->h_n_full0[b] = nf;
      c->h_n_span_tokens[b] = nt;
      c->h_n_tok_pad[b] = static_cast<int>(pad);
    }
    finish_sizes(c, opts, la, theta);
    if ((rc = alloc_arrays(c, st)) != RSKV_OK) return rc;
    rc = dev_alloc(c, &c->dev.span_id, static_cast<size_t>(B) * c->T, "span_id");
    if (rc != RSKV_OK) return rc;
    if ((rc = copy_proj(c, opts, st, true)) != RSKV_OK) return rc;
    RSKV_HIP(hipStreamSynchronize(st), "import memset");
    auto& v = c->dev;
    // span tables and offsets
    std::vector<int32_t> starts(static_cast<size_t>(B) * c->S, 0), lens(starts.size(), 0),
        off(static_cast<size_t>(B) * (c->S + 1), 0), pad(off.size(), 0),
        fpos(static_cast<size_t>(B) * c->F, -1);
    std::vector<float> ell(starts.size(), 0.f), hfull(fpos.size(), 0.f);
    std::vector<int> o, p;
    for (int b = 0; b < B; ++b) {
      const int ns = c->h_n_spans[b];
      const int32_t* L = a->span_len + static_cast<size_t>(b) * S_in;
      span_offsets(L, ns, &o, &p);
      for (int j = 0; j < ns; ++j) {
        starts[static_cast<size_t>(b) * c->S + j] = a->span_start[static_cast<size_t>(b) * S_in + j];
        lens[static_cast<size_t>(b) * c->S + j] = L[j];
        ell[static_cast<size_t>(b) * c->S + j] = a->log_len[static_cast<size_t>(b) * S_in + j];
      }
      for (int j = 0; j <= ns; ++j) {
        off[static_cast<size_t>(b) * (c->S + 1) + j] = o[j];
        pad[static_cast<size_t>(b) * (c->S + 1) + j] = p[j];
      }
      for (int i = 0; i < c->h_n_full0[b]; ++i) {
        fpos[static_cast<size_t>(b) * c->F + i] = a->full_pos[static_cast<size_t>(b) * F_in + i];
        if (a->h_full != nullptr)
          hfull[static_cast<size_t>(b) * c->F + i] = a->h_full[static_cast<size_t>(b) * F_in + i];
      }
    }
    auto put = [&](void* dst, const void* src, size_t bytes, const char* what) -> int {
      hipError_t e = hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice);
      return e == hipSuccess ? RSKV_OK : hip_fail(e, what);
    };
    if ((rc = put(v.span_start, starts.data(), starts.size() * 4, "import span_start"))) return rc;
    if ((rc = put(v.span_len, lens.data(), lens.size() * 4, "import span_len"))) return rc;
    if ((rc = put(v.log_len, ell.data(), ell.size() * 4, "import log_len"))) return rc;
    if ((rc = put(v.tok_off, off.data(), off.size() * 4, "import tok_off"))) return rc;
    if ((rc = put(v.tok_pad, pad.data(), pad.size() * 4, "import tok_pad"))) return rc;
    if ((rc = put(v.full_pos, fpos.data(), fpos.size() * 4, "import full_pos"))) return rc;
    if ((rc = put(v.h_full, hfull.data(), hfull.size() * 4, "import h_full"))) return rc;
    if ((rc = put(v.theta, theta.data(), theta.size() * 4, "import theta"))) return rc;
    if ((rc = put(v.last_anchor, la.data(), la.size() * 4, "import last_anchor"))) return rc;
    if (a->span_id != nullptr &&
        (rc = put(v.span_id, a->span_id, static_cast<size_t>(B) * c->T * 4, "import span_id")))
      return rc;
    if ((rc = put(v.n_spans, c->h_n_spans.data(), B * 4, "import n_spans"))) return rc;
    if ((rc = put(v.n_full, c->h_n_full0.data(), B * 4, "import n_full"))) return rc;
    if ((rc = put(v.n_full0, c->h_n_full0.data(), B * 4, "import n_full0"))) return rc;
    rc = c->dtype == RSKV_BF16 ? import_arrays<uint16_t>(c, a, S_in, F_in, N_in)
                               : import_arrays<uint32_t>(c, a, S_in, F_in, N_in);
    if (rc != RSKV_OK) return rc;
    RSKV_HIP(hipDeviceSynchronize(), "import");
    guard.c = nullptr;
    *out = c;
    return RSKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(RSKV_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(RSKV_EINVAL, "unexpected error in rskv_cache_import");
  }
}

void rskv_cache_destroy(rskv_cache* c) {
  if (!valid_cache(c)) return;
  free_cache(c);
}

int rskv_profile_enable(rskv_cache* c, int32_t on) {
  if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
  for (auto* list : {&c->prof.pending, &c->prof.app_pending}) {
    for (hipEvent_t e : *list)
      if (e != nullptr) c->prof.pool.push_back(e);
    list->clear();
  }
  c->prof.on = on != 0;
  c->prof.steps = 0;
  c->prof.appends = 0;
  for (double& m : c->prof.ms) m = 0.0;
  c->prof.close_ms = c->prof.append_ms = 0.0;
  return RSKV_OK;
}

int rskv_profile_read(rskv_cache* c, rskv_profile* p) {
  if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
  if (p == nullptr) return fail(RSKV_EINVAL, "profile is NULL");
  auto& pr = c->prof;
  constexpr int kEv = 2 * rskv::kProfileKernels;
  for (size_t i = 0; i + kEv <= pr.pending.size(); i += kEv) {
    int last = kEv - 1;  // the step's last recorded event
    while (last > 0 && pr.pending[i + last] == nullptr) --last;
    RSKV_HIP(hipEventSynchronize(pr.pending[i + last]), "event sync");
    for (int k = 0; k < rskv::kProfileKernels; ++k) {
      if (pr.pending[i + 2 * k] == nullptr) continue;  // kernel not launched this step
      float ms = 0.f;
      RSKV_HIP(hipEventElapsedTime(&ms, pr.pending[i + 2 * k], pr.pending[i + 2 * k + 1]),
               "elapsed");
      pr.ms[k] += ms;
    }
    pr.steps += 1;
  }
  for (size_t i = 0; i + 4 <= pr.app_pending.size(); i += 4) {
    RSKV_HIP(hipEventSynchronize(pr.app_pending[i + 3]), "event sync");
    float ms = 0.f;
    if (pr.app_pending[i] != nullptr) {
      RSKV_HIP(hipEventElapsedTime(&ms, pr.app_pending[i], pr.app_pending[i + 1]), "elapsed");
      pr.close_ms += ms;
    }
    RSKV_HIP(hipEventElapsedTime(&ms, pr.app_pending[i + 2], pr.app_pending[i + 3]), "elapsed");
    pr.append_ms += ms;
    pr.appends += 1;
  }
  for (auto* list : {&pr.pending, &pr.app_pending}) {
    for (hipEvent_t e : *list)
      if (e != nullptr) pr.pool.push_back(e);
    list->clear();
  }
  p->steps = pr.steps;
  p->appends = pr.appends;
  p->close_ms = pr.close_ms;
  p->append_ms = pr.append_ms;
  p->route_ms = pr.ms[0];
  p->topk_ms = pr.ms[1];
  p->attend_ms = pr.ms[2];
  p->merge_ms = pr.ms[3];
  return RSKV_OK;
}

}  // extern "C"
