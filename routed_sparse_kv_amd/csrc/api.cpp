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

constexpr int kMaxG = 8;
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
    return fail(RSKV_EINVAL, "query group size above 8 is not supported");
  if (o->head_dim != 64 && o->head_dim != 128)
    return fail(RSKV_EINVAL, "head_dim must be 64 or 128");
  if (!(o->anchor_frac >= 0.0 && o->anchor_frac <= 1.0))
    return fail(RSKV_EINVAL, "anchor_frac must lie in [0, 1]");
  if (rank < 1 || rank > kMaxRank) return fail(RSKV_EINVAL, "rank must lie in [1, 32]");
  if (o->tail_capacity < 0) return fail(RSKV_EINVAL, "tail_capacity must be >= 0");
  if (o->proj != nullptr && o->n_proj != 1 && o->n_proj != o->n_kv_heads)
    return fail(RSKV_EINVAL, "n_proj must be 1 or n_kv_heads");
  if (!(o->alpha == o->alpha)) return fail(RSKV_EINVAL, "alpha is NaN");
  return RSKV_OK;
}

// Allocation of one device array, tracked by the cache.
template <typename T>
int dev_alloc(rskv_cache* c, T** p, size_t count, const char* what) {
  *p = nullptr;
  const size_t bytes = std::max<size_t>(count, 1) * sizeof(T);
  void* q = nullptr;
  hipError_t e = hipMalloc(&q, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(RSKV_ENOMEM, std::string("device allocation failed: ") + what);
  }
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

void free_cache(rskv_cache* c) {
  if (c == nullptr) return;
  if (c->last_stream != nullptr) (void)hipStreamSynchronize(c->last_stream);
  (void)hipDeviceSynchronize();
  for (void* p : c->allocs) (void)hipFree(p);
  for (hipEvent_t e : c->prof.pending) (void)hipEventDestroy(e);
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

// Allocates the stored arrays and the decode workspace once S, F, N and the
// counts are known.  Everything is zero-filled.
int alloc_arrays(rskv_cache* c, hipStream_t st) {
  const size_t U = static_cast<size_t>(c->B) * c->Hkv;
  const size_t es = elem_size(c->dtype);
  const size_t d = c->d, S = c->S, F = c->F, N = c->N, r = c->rank;
  auto& v = c->dev;
  int rc;
#define ALLOC(ptr, n, what) \
  if ((rc = dev_alloc(c, &(ptr), (n), what)) != RSKV_OK) return rc
#define ALLOCB(ptr, n, what) \
  if ((rc = dev_alloc_bytes(c, &(ptr), (n), what)) != RSKV_OK) return rc
  ALLOC(v.span_start, c->B * S, "span_start");
  ALLOC(v.span_len, c->B * S, "span_len");
  ALLOC(v.tok_off, c->B * (S + 1), "tok_off");
  ALLOC(v.full_pos, c->B * F, "full_pos");
  ALLOC(v.n_spans, c->B, "n_spans");
  ALLOC(v.n_full, c->B, "n_full");
  ALLOC(v.n_full0, c->B, "n_full0");
  ALLOCB(v.summary, U * S * d * es, "summary");
  ALLOCB(v.vmean, U * S * d * es, "vmean");
  ALLOC(v.log_len, c->B * S, "log_len");
  ALLOCB(v.k_full, U * F * d * es, "k_full");
  ALLOCB(v.v_full, U * F * d * es, "v_full");
  ALLOCB(v.a_k, U * N * r * es, "a_k");
  ALLOCB(v.a_v, U * N * r * es, "a_v");
  ALLOCB(v.w_k, U * S * r * d * es, "w_k");
  ALLOCB(v.w_v, U * S * r * d * es, "w_v");
  ALLOC(v.z, U * S, "z");
  ALLOC(v.slogit, U * S * c->G, "slogit");
  ALLOC(v.expanded, U * S, "expanded");
  ALLOC(v.sel, U * S, "sel");
  ALLOC(v.n_sel, U, "n_sel");
  c->nsplit_max = rskv::decode_nsplit_max(c->B, c->Hkv, c->S, c->F, c->k_max_cap);
  ALLOC(v.part, U * c->nsplit_max * c->G * (d + 2), "part");
#undef ALLOC
#undef ALLOCB
  RSKV_HIP(hipMemsetAsync(v.summary, 0, U * S * d * es, st), "memset summary");
  RSKV_HIP(hipMemsetAsync(v.vmean, 0, U * S * d * es, st), "memset vmean");
  RSKV_HIP(hipMemsetAsync(v.k_full, 0, U * F * d * es, st), "memset k_full");
  RSKV_HIP(hipMemsetAsync(v.v_full, 0, U * F * d * es, st), "memset v_full");
  RSKV_HIP(hipMemsetAsync(v.a_k, 0, U * N * r * es, st), "memset a_k");
  RSKV_HIP(hipMemsetAsync(v.a_v, 0, U * N * r * es, st), "memset a_v");
  RSKV_HIP(hipMemsetAsync(v.w_k, 0, U * S * r * d * es, st), "memset w_k");
  RSKV_HIP(hipMemsetAsync(v.w_v, 0, U * S * r * d * es, st), "memset w_v");
  RSKV_HIP(hipMemsetAsync(v.log_len, 0, c->B * S * sizeof(float), st), "memset log_len");
  RSKV_HIP(hipMemsetAsync(v.expanded, 0, U * S, st), "memset expanded");
  RSKV_HIP(hipMemsetAsync(v.n_sel, 0, U * sizeof(int32_t), st), "memset n_sel");
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

int finish_sizes(rskv_cache* c, const rskv_build_opts* o) {
  int s_max = 0, f_max = 0, n_max = 0;
  for (int b = 0; b < c->B; ++b) {
    s_max = std::max(s_max, c->h_n_spans[b]);
    f_max = std::max(f_max, c->h_n_full0[b]);
    n_max = std::max(n_max, c->h_n_span_tokens[b]);
  }
  c->S = std::max(1, s_max);
  c->F = std::max(1, f_max + c->tail_cap);
  c->N = std::max(1, n_max);
  c->k_max_cap = o->k_max_cap > 0 ? o->k_max_cap : 0x7fffffff;  // <= 0: no limit
  return RSKV_OK;
}

}  // namespace

extern "C" {

const char* rskv_last_error(void) { return g_err.c_str(); }

const char* rskv_version(void) { return "rskv 0.1.0 (gfx950)"; }

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
    const double na_d = floor(opts->anchor_frac * static_cast<double>(T));
    const int n_anchor = static_cast<int>(na_d);

    // ---- segmentation into temporaries of pitch T
    rc = dev_alloc(c, &c->dev.span_id, static_cast<size_t>(B) * T, "span_id");
    if (rc != RSKV_OK) return rc;
    int32_t *start_tmp = nullptr, *len_tmp = nullptr, *tokoff_tmp = nullptr,
            *full_tmp = nullptr, *counts = nullptr;
    std::vector<void*> tmps;
    auto tmp_alloc = [&](int32_t** p, size_t n) -> int {
      void* q = nullptr;
      if (hipMalloc(&q, std::max<size_t>(n, 1) * sizeof(int32_t)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(RSKV_ENOMEM, "device allocation failed: segmentation temporaries");
      }
      tmps.push_back(q);
      *p = static_cast<int32_t*>(q);
      return RSKV_OK;
    };
    struct TmpFree {
      std::vector<void*>* v;
      hipStream_t st;
      ~TmpFree() {
        if (!v->empty()) (void)hipStreamSynchronize(st);
        for (void* p : *v) (void)hipFree(p);
      }
    } tmp_free{&tmps, st};
    const size_t BT = static_cast<size_t>(B) * T;
    if ((rc = tmp_alloc(&start_tmp, BT)) != RSKV_OK) return rc;
    if ((rc = tmp_alloc(&len_tmp, BT)) != RSKV_OK) return rc;
    if ((rc = tmp_alloc(&tokoff_tmp, static_cast<size_t>(B) * (T + 1))) != RSKV_OK) return rc;
    if ((rc = tmp_alloc(&full_tmp, BT)) != RSKV_OK) return rc;
    if ((rc = tmp_alloc(&counts, static_cast<size_t>(B) * 4)) != RSKV_OK) return rc;
    RSKV_HIP(rskv::launch_segment(surprisal, B, T, n_anchor, c->dev.span_id, start_tmp, len_tmp,
                                  tokoff_tmp, full_tmp, counts, st),
             "segment kernel");
    std::vector<int32_t> hc(static_cast<size_t>(B) * 4);
    RSKV_HIP(hipMemcpyAsync(hc.data(), counts, hc.size() * sizeof(int32_t),
                            hipMemcpyDeviceToHost, st),
             "copy counts");
    RSKV_HIP(hipStreamSynchronize(st), "segment kernel");
    c->h_n_anchor.resize(B);
    c->h_n_spans.resize(B);
    c->h_n_full0.resize(B);
    c->h_n_span_tokens.resize(B);
    for (int b = 0; b < B; ++b) {
      if (hc[4 * b] < 0) return fail(RSKV_EINVAL, "surprisal holds NaN");
      c->h_n_anchor[b] = hc[4 * b];
      c->h_n_spans[b] = hc[4 * b + 1];
      c->h_n_full0[b] = hc[4 * b + 2];
      c->h_n_span_tokens[b] = hc[4 * b + 3];
    }
    finish_sizes(c, opts);
    if ((rc = alloc_arrays(c, st)) != RSKV_OK) return rc;
    if ((rc = copy_proj(c, opts, st, false)) != RSKV_OK) return rc;
    auto& v = c->dev;
    RSKV_HIP(rskv::launch_copy_rows(v.span_start, c->S, start_tmp, T, counts, 4, 1, 0, 0, B, st),
             "copy span_start");
    RSKV_HIP(rskv::launch_copy_rows(v.span_len, c->S, len_tmp, T, counts, 4, 1, 0, 0, B, st),
             "copy span_len");
    RSKV_HIP(rskv::launch_copy_rows(v.tok_off, c->S + 1, tokoff_tmp, T + 1, counts, 4, 1, 1, 0,
                                    B, st),
             "copy tok_off");
    RSKV_HIP(rskv::launch_copy_rows(v.full_pos, c->F, full_tmp, T, counts, 4, 2, 0, -1, B, st),
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
    RSKV_HIP(rskv::launch_pack(c, K, V, st), "pack kernel");
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
    if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
    if (q == nullptr || out == nullptr) return fail(RSKV_EINVAL, "q and out must be non-NULL");
    if (tau != tau) return fail(RSKV_EINVAL, "tau is NaN");
    if (k_max < 0) return fail(RSKV_EINVAL, "k_max must be >= 0");
    if (k_max > c->k_max_cap) return fail(RSKV_ECAPACITY, "k_max exceeds k_max_cap");
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    const int nsplit = rskv::decode_nsplit(c, k_max);
    hipEvent_t ev[5] = {};
    const bool prof = c->prof.on;
    if (prof) {
      for (int i = 0; i < 5; ++i) {
        if (c->prof.pool.empty()) {
          hipEvent_t e;
          RSKV_HIP(hipEventCreate(&e), "event create");
          c->prof.pool.push_back(e);
        }
        ev[i] = c->prof.pool.back();
        c->prof.pool.pop_back();
      }
      RSKV_HIP(hipEventRecord(ev[0], st), "event record");
    }
    RSKV_HIP(rskv::launch_route(c, q, st), "route kernel");
    if (prof) RSKV_HIP(hipEventRecord(ev[1], st), "event record");
    RSKV_HIP(rskv::launch_topk(c, tau, k_max, sel, n_sel, st), "topk kernel");
    if (prof) RSKV_HIP(hipEventRecord(ev[2], st), "event record");
    RSKV_HIP(rskv::launch_attend(c, q, k_max, nsplit, st), "attend kernel");
    if (prof) RSKV_HIP(hipEventRecord(ev[3], st), "event record");
    RSKV_HIP(rskv::launch_merge(c, nsplit, out, st), "merge kernel");
    if (prof) {
      RSKV_HIP(hipEventRecord(ev[4], st), "event record");
      for (int i = 0; i < 5; ++i) c->prof.pending.push_back(ev[i]);
    }
    return RSKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(RSKV_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(RSKV_EINVAL, "unexpected error in rskv_decode_step");
  }
}

int rskv_append_kv(rskv_cache* c, const void* k, const void* v, void* stream) {
  if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
  if (k == nullptr || v == nullptr) return fail(RSKV_EINVAL, "k and v must be non-NULL");
  if (c->appended >= c->tail_cap) return fail(RSKV_ECAPACITY, "tail capacity exhausted");
  hipStream_t st = static_cast<hipStream_t>(stream);
  c->last_stream = st;
  RSKV_HIP(rskv::launch_append(c, k, v, st), "append kernel");
  c->appended += 1;
  return RSKV_OK;
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
  return RSKV_OK;
}

int rskv_cache_export(const rskv_cache* c, rskv_host_arrays* a) {
  try {
    if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
    if (a == nullptr) return fail(RSKV_EINVAL, "arrays is NULL");
    RSKV_HIP(hipDeviceSynchronize(), "export sync");
    const int B = c->B;
    const size_t U = static_cast<size_t>(B) * c->Hkv;
    const size_t es = elem_size(c->dtype);
    const size_t d = c->d, S = c->S, F = c->F, N = c->N, r = c->rank;
    for (int b = 0; b < B; ++b) {
      if (a->n_anchor) a->n_anchor[b] = c->h_n_anchor[b];
      if (a->n_spans) a->n_spans[b] = c->h_n_spans[b];
      if (a->n_full) a->n_full[b] = c->h_n_full0[b] + c->appended;
      if (a->n_span_tokens) a->n_span_tokens[b] = c->h_n_span_tokens[b];
    }
    auto cp = [&](void* dst, const void* src, size_t bytes, const char* what) -> int {
      if (dst == nullptr) return RSKV_OK;
      hipError_t e = hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(e, what);
      return RSKV_OK;
    };
    int rc;
#define CP(dst, src, bytes) \
  if ((rc = cp(dst, src, bytes, "export " #dst)) != RSKV_OK) return rc
    const auto& v = c->dev;
    CP(a->span_id, v.span_id, static_cast<size_t>(B) * c->T * 4);
    CP(a->span_start, v.span_start, B * S * 4);
    CP(a->span_len, v.span_len, B * S * 4);
    CP(a->full_pos, v.full_pos, B * F * 4);
    CP(a->summary, v.summary, U * S * d * es);
    CP(a->vmean, v.vmean, U * S * d * es);
    CP(a->log_len, v.log_len, B * S * 4);
    CP(a->k_full, v.k_full, U * F * d * es);
    CP(a->v_full, v.v_full, U * F * d * es);
    CP(a->a_k, v.a_k, U * N * r * es);
    CP(a->a_v, v.a_v, U * N * r * es);
    CP(a->w_k, v.w_k, U * S * r * d * es);
    CP(a->w_v, v.w_v, U * S * r * d * es);
#undef CP
    return RSKV_OK;
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
    for (int b = 0; b < B; ++b) {
      const int ns = a->n_spans[b], nf = a->n_full[b], nt = a->n_span_tokens[b];
      if (ns < 0 || ns > S_in || nf < 0 || nf > F_in || nt < 0 || nt > N_in)
        return fail(RSKV_EINVAL, "counts exceed the padded dimensions");
      long long sum = 0;
      for (int j = 0; j < ns; ++j) {
        const int len = a->span_len[static_cast<size_t>(b) * S_in + j];
        if (len < 1) return fail(RSKV_EINVAL, "span lengths must be >= 1");
        sum += len;
      }
      if (sum != nt) return fail(RSKV_EINVAL, "n_span_tokens differs from the sum of lengths");
      c->h_n_anchor[b] = a->n_anchor ? a->n_anchor[b] : 0;
      c->h_n_spans[b] = ns;
      c->h_n_full0[b] = nf;
      c->h_n_span_tokens[b] = nt;
    }
    finish_sizes(c, opts);
    if ((rc = alloc_arrays(c, st)) != RSKV_OK) return rc;
    rc = dev_alloc(c, &c->dev.span_id, static_cast<size_t>(B) * c->T, "span_id");
    if (rc != RSKV_OK) return rc;
    if ((rc = copy_proj(c, opts, st, true)) != RSKV_OK) return rc;
    auto& v = c->dev;
    const size_t U = static_cast<size_t>(B) * c->Hkv;
    const size_t es = elem_size(c->dtype);
    const size_t d = c->d, r = c->rank;
    // tok_off on the host from the lengths
    std::vector<int32_t> tok(static_cast<size_t>(B) * (c->S + 1), 0);
    for (int b = 0; b < B; ++b) {
      int acc = 0;
      for (int j = 0; j < c->h_n_spans[b]; ++j) {
        tok[static_cast<size_t>(b) * (c->S + 1) + j] = acc;
        acc += a->span_len[static_cast<size_t>(b) * S_in + j];
      }
      tok[static_cast<size_t>(b) * (c->S + 1) + c->h_n_spans[b]] = acc;
    }
    RSKV_HIP(hipMemcpy(v.tok_off, tok.data(), tok.size() * 4, hipMemcpyHostToDevice), "tok_off");
    auto cp2d = [&](void* dst, size_t dpitch, const void* src, size_t spitch, size_t width,
                    size_t rows, const char* what) -> int {
      hipError_t e = hipMemcpy2D(dst, dpitch, src, spitch, width, rows, hipMemcpyHostToDevice);
      if (e != hipSuccess) return hip_fail(e, what);
      return RSKV_OK;
    };
    const size_t Sd = c->S, Fd = c->F, Nd = c->N;
    const size_t sw = std::min<size_t>(S_in, Sd), fw = std::min<size_t>(F_in, Fd),
                 nw = std::min<size_t>(N_in, Nd);
    if ((rc = cp2d(v.span_start, Sd * 4, a->span_start, S_in * 4ul, sw * 4, B, "span_start")))
      return rc;
    if ((rc = cp2d(v.span_len, Sd * 4, a->span_len, S_in * 4ul, sw * 4, B, "span_len"))) return rc;
    if ((rc = cp2d(v.log_len, Sd * 4, a->log_len, S_in * 4ul, sw * 4, B, "log_len"))) return rc;
    // full_pos: pad -1
    std::vector<int32_t> fp(static_cast<size_t>(B) * Fd, -1);
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < c->h_n_full0[b]; ++i)
        fp[static_cast<size_t>(b) * Fd + i] = a->full_pos[static_cast<size_t>(b) * F_in + i];
    RSKV_HIP(hipMemcpy(v.full_pos, fp.data(), fp.size() * 4, hipMemcpyHostToDevice), "full_pos");
    if (a->span_id != nullptr)
      RSKV_HIP(hipMemcpy(v.span_id, a->span_id, static_cast<size_t>(B) * c->T * 4,
                         hipMemcpyHostToDevice),
               "span_id");
    if ((rc = cp2d(v.summary, Sd * d * es, a->summary, S_in * d * es, sw * d * es, U, "summary")))
      return rc;
    if ((rc = cp2d(v.vmean, Sd * d * es, a->vmean, S_in * d * es, sw * d * es, U, "vmean")))
      return rc;
    if ((rc = cp2d(v.k_full, Fd * d * es, a->k_full, F_in * d * es, fw * d * es, U, "k_full")))
      return rc;
    if ((rc = cp2d(v.v_full, Fd * d * es, a->v_full, F_in * d * es, fw * d * es, U, "v_full")))
      return rc;
    if ((rc = cp2d(v.a_k, Nd * r * es, a->a_k, N_in * r * es, nw * r * es, U, "a_k"))) return rc;
    if ((rc = cp2d(v.a_v, Nd * r * es, a->a_v, N_in * r * es, nw * r * es, U, "a_v"))) return rc;
    if ((rc = cp2d(v.w_k, Sd * r * d * es, a->w_k, S_in * r * d * es, sw * r * d * es, U, "w_k")))
      return rc;
    if ((rc = cp2d(v.w_v, Sd * r * d * es, a->w_v, S_in * r * d * es, sw * r * d * es, U, "w_v")))
      return rc;
    RSKV_HIP(hipMemcpy(v.n_spans, c->h_n_spans.data(), B * 4, hipMemcpyHostToDevice), "n_spans");
    RSKV_HIP(hipMemcpy(v.n_full, c->h_n_full0.data(), B * 4, hipMemcpyHostToDevice), "n_full");
    RSKV_HIP(hipMemcpy(v.n_full0, c->h_n_full0.data(), B * 4, hipMemcpyHostToDevice), "n_full0");
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
  for (hipEvent_t e : c->prof.pending) c->prof.pool.push_back(e);
  c->prof.pending.clear();
  c->prof.on = on != 0;
  c->prof.steps = 0;
  for (double& m : c->prof.ms) m = 0.0;
  return RSKV_OK;
}

int rskv_profile_read(rskv_cache* c, rskv_profile* p) {
  if (!valid_cache(c)) return fail(RSKV_ESTATE, "invalid cache handle");
  if (p == nullptr) return fail(RSKV_EINVAL, "profile is NULL");
  auto& pr = c->prof;
  for (size_t i = 0; i + 5 <= pr.pending.size(); i += 5) {
    RSKV_HIP(hipEventSynchronize(pr.pending[i + 4]), "event sync");
    for (int k = 0; k < 4; ++k) {
      float ms = 0.f;
      RSKV_HIP(hipEventElapsedTime(&ms, pr.pending[i + k], pr.pending[i + k + 1]), "elapsed");
      pr.ms[k] += ms;
    }
    pr.steps += 1;
  }
  for (hipEvent_t e : pr.pending) pr.pool.push_back(e);
  pr.pending.clear();
  p->steps = pr.steps;
  p->route_ms = pr.ms[0];
  p->topk_ms = pr.ms[1];
  p->attend_ms = pr.ms[2];
  p->merge_ms = pr.ms[3];
  return RSKV_OK;
}

}  // extern "C"
