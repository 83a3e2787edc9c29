// C ABI of the token-retrieval router (rskv_retrieval.h): option checks,
// the codebook, allocation, build and decode orchestration, export, trace
// and per-kernel timing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "retrieval.h"

namespace {

using rskv::report_error;
namespace R = rskv::ret;

int hip_fail(hipError_t e, const char* what) {
  return report_error(RSKV_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define RET_HIP(expr, what)                          \
  do {                                               \
    hipError_t e_ = (expr);                          \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool valid(const rskv_retrieval* r) { return r != nullptr && r->magic == R::kMagic; }

size_t esize(int dtype) { return dtype == RSKV_BF16 ? 2 : 4; }

// ------------------------------------------------------------- codebook
//
// Octiles and bin means of |y|, y one coordinate of a uniform unit vector of
// R^m.  |y| has density proportional to (1 - t^2)^((m-3)/2) on [0, 1]; with
// t = sin(th) this is cos^(m-2)(th) dth, whose integral from 0 follows the
// reduction I_n = cos^(n-1) sin / n + (n-1)/n I_(n-2) (I_0 = th, I_1 =
// sin th).  The first moment integrates to (1 - (1-t^2)^((m-1)/2)) / (m-1).
// The octiles come from bisection on the closed-form CDF.

double cos_power_integral(int n, double th) {
  const double c = cos(th), s = sin(th);
  double a = (n % 2 == 0) ? th : s;
  for (int k = (n % 2 == 0) ? 2 : 3; k <= n; k += 2)
    a = pow(c, k - 1) * s / k + static_cast<double>(k - 1) / k * a;
  return a;
}

void make_codebook(int m, R::Codebook* cb) {
  const int n = m - 2;
  const double Z = cos_power_integral(n, M_PI / 2);
  auto mass = [&](double t) { return cos_power_integral(n, asin(t)); };
  auto moment = [&](double t) { return (1.0 - pow(1.0 - t * t, 0.5 * (m - 1))) / (m - 1); };
  double beta[9];
  beta[0] = 0.0;
  beta[8] = 1.0;
  for (int j = 1; j < 8; ++j) {
    double lo = 0.0, hi = 1.0;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (!(mid > lo && mid < hi)) break;
      if (mass(mid) < Z * j / 8.0)
        lo = mid;
      else
        hi = mid;
    }
    beta[j] = 0.5 * (lo + hi);
  }
  for (int j = 0; j < 8; ++j) {
    cb->beta[j] = beta[j];
    cb->lam[j] = (moment(beta[j + 1]) - moment(beta[j])) / (mass(beta[j + 1]) - mass(beta[j]));
  }
}

// ------------------------------------------------------------- memory

int dev_alloc(rskv_retrieval* r, void** p, size_t bytes, const char* what) {
  *p = nullptr;
  bytes = std::max<size_t>(bytes, 16);
  void* q = r->mem.alloc(bytes, r->last_stream);
  if (q == nullptr)
    return report_error(RSKV_ENOMEM, std::string("device allocation failed: ") + what);
  r->allocs.push_back(q);
  r->bytes += bytes;
  *p = q;
  return RSKV_OK;
}

int host_alloc(rskv_retrieval* r, void** p, size_t bytes, const char* what) {
  *p = nullptr;
  bytes = std::max<size_t>(bytes, 16);
  void* q = nullptr;
  hipError_t e = hipHostMalloc(&q, bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return report_error(RSKV_ENOMEM, std::string("pinned host allocation failed: ") + what);
  }
  r->host_allocs.push_back(q);
  r->host_bytes += bytes;
  *p = q;
  return RSKV_OK;
}

template <typename T>
int dev_array(rskv_retrieval* r, T** p, size_t count, const char* what) {
  void* q = nullptr;
  int rc = dev_alloc(r, &q, count * sizeof(T), what);
  *p = static_cast<T*>(q);
  return rc;
}

void free_index(rskv_retrieval* r) {
  if (r == nullptr) return;
  // the last stream only; then every block goes back to the allocator
  (void)hipStreamSynchronize(r->last_stream);
  for (void* p : r->allocs) r->mem.release(p, r->last_stream);
  for (void* p : r->host_allocs) (void)hipHostFree(p);
  for (hipEvent_t e : r->pending)
    if (e != nullptr) (void)hipEventDestroy(e);
  for (hipEvent_t e : r->pool) (void)hipEventDestroy(e);
  r->magic = 0;
  delete r;
}

struct Guard {
  rskv_retrieval* r;
  ~Guard() {
    if (r) free_index(r);
  }
};

int check_opts(const rskv_retrieval_opts* o) {
  if (o == nullptr) return report_error(RSKV_EINVAL, "opts is NULL");
  if (o->dtype != RSKV_F32 && o->dtype != RSKV_BF16)
    return report_error(RSKV_EDTYPE, "dtype must be RSKV_F32 or RSKV_BF16");
  if (o->batch < 1 || o->n_q_heads < 1 || o->n_kv_heads < 1 || o->context_len < 1)
    return report_error(RSKV_EINVAL, "batch, heads and context_len must be >= 1");
  if (o->n_q_heads % o->n_kv_heads)
    return report_error(RSKV_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
  if (o->n_q_heads / o->n_kv_heads > 8)
    return report_error(RSKV_EINVAL, "query group size above 8 is not supported");
  if (o->head_dim != 64 && o->head_dim != 128)
    return report_error(RSKV_EINVAL, "head_dim must be 64 or 128");
  if (o->m != 8) return report_error(RSKV_EINVAL, "subspace width m must be 8");
  if (o->rho < 1 || o->rho > R::kMaxRho) return report_error(RSKV_EINVAL, "rho must lie in [1, 16]");
  if (!(o->cand_frac >= 0.0 && o->cand_frac <= 1.0))
    return report_error(RSKV_EINVAL, "cand_frac must lie in [0, 1]");
  if (o->k_ret < 0 || o->n_sink < 0 || o->n_local < 0)
    return report_error(RSKV_EINVAL, "k_ret, n_sink and n_local must be >= 0");
  if (!rskv::valid_hook(o->allocator))
    return report_error(RSKV_EINVAL, "allocator needs both alloc and free, or neither");
  if (o->kv_tier != RSKV_TIER_HBM && o->kv_tier != RSKV_TIER_HOST)
    return report_error(RSKV_EINVAL, "kv_tier must be RSKV_TIER_HBM or RSKV_TIER_HOST");
  if (static_cast<long long>(o->batch) * o->n_kv_heads * o->context_len > (1ll << 31) - 1)
    return report_error(RSKV_EINVAL, "batch * n_kv_heads * context_len must be < 2^31");
  return RSKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int copy_rows(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
              hipStream_t st) {
  if (width == 0 || height == 0) return RSKV_OK;
  RET_HIP(hipMemcpy2DAsync(dst, dpitch, src, spitch, width, height, hipMemcpyDefault, st),
          "row copy");
  return RSKV_OK;
}

}  // namespace

extern "C" {

int rskv_retrieval_build(const void* K, const void* V, const int8_t* signs,
                         const rskv_retrieval_opts* o, void* stream, rskv_retrieval** out) {
  try {
    if (out == nullptr) return report_error(RSKV_EINVAL, "out is NULL");
    *out = nullptr;
    int rc = check_opts(o);
    if (rc != RSKV_OK) return rc;
    if (K == nullptr || V == nullptr || signs == nullptr)
      return report_error(RSKV_EINVAL, "K, V and signs must be non-NULL");
    if (!aligned16(K) || !aligned16(V))
      return report_error(RSKV_EINVAL, "K and V must be 16-byte aligned");
    const int d = o->head_dim;
    rskv_retrieval* r = new rskv_retrieval();
    Guard guard{r};
    for (int c = 0; c < d; ++c) {
      if (signs[c] != 1 && signs[c] != -1)
        return report_error(RSKV_EINVAL, "signs must be +1 or -1");
      if (signs[c] < 0) r->signs.w[c >> 5] |= 1u << (c & 31);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    r->last_stream = st;
    r->mem.hook = o->allocator;
    r->B = o->batch;
    r->Hq = o->n_q_heads;
    r->Hkv = o->n_kv_heads;
    r->G = r->Hq / r->Hkv;
    r->d = d;
    r->T = o->context_len;
    r->dtype = o->dtype;
    r->m = o->m;
    r->Bs = d / o->m;
    r->rho = o->rho;
    r->k_ret = o->k_ret;
    r->kv_tier = o->kv_tier;
    r->cand_frac = o->cand_frac;
    r->ns = std::min(o->n_sink, r->T);
    r->l0 = std::max(r->ns, r->T - std::min(o->n_local, r->T));
    r->nl = r->T - r->l0;
    r->N = r->l0 - r->ns;
    r->C = std::min(r->N, static_cast<int>(ceil(o->cand_frac * static_cast<double>(r->N))));
    r->n_sel = std::min(r->k_ret, r->C);
    r->n_att = r->ns + r->n_sel + r->nl;
    r->n_near = r->ns + r->nl;
    if (r->n_att == 0)
      return report_error(RSKV_EINVAL, "nothing to attend: no Sink, no Local and no retrieval");
    r->rec_bytes = d;  // d/2 bytes of codes + d/8 fp32 calibrations
    r->nchunk = (r->N + R::kChunk - 1) / R::kChunk;
    r->npad = static_cast<size_t>(r->nchunk) * R::kChunk;
    r->nbins = r->Bs * r->rho + 1;
    r->nsplit = (r->n_att + R::kRows - 1) / R::kRows;
    r->nsb = (r->C + R::kSelBlock - 1) / R::kSelBlock;
    r->nrwg = (r->C + 255) / 256;
    if (r->nsb > R::kSelMaxBlocks)
      return report_error(RSKV_EINVAL, "too many candidates: ceil(cand_frac * N) must be <= " +
                                           std::to_string(R::kSelBlock * R::kSelMaxBlocks));
    make_codebook(r->m, &r->cb);

    const size_t U = static_cast<size_t>(r->B) * r->Hkv;
    const size_t row = static_cast<size_t>(d) * esize(r->dtype);
    const size_t N = static_cast<size_t>(r->N);
    if ((rc = dev_alloc(r, &r->k_near, U * r->n_near * row, "Sink/Local keys")) ||
        (rc = dev_alloc(r, &r->v_near, U * r->n_near * row, "Sink/Local values")))
      return rc;
    if (r->kv_tier == RSKV_TIER_HOST) {
      if ((rc = host_alloc(r, &r->k_far, U * N * row, "retrieval keys")) ||
          (rc = host_alloc(r, &r->v_far, U * N * row, "retrieval values")))
        return rc;
    } else {
      if ((rc = dev_alloc(r, &r->k_far, U * N * row, "retrieval keys")) ||
          (rc = dev_alloc(r, &r->v_far, U * N * row, "retrieval values")))
        return rc;
    }
    if ((rc = dev_array(r, &r->buckets, U * N * r->Bs, "buckets")) ||
        (rc = dev_array(r, &r->rec, U * N * r->rec_bytes, "codes")) ||
        (rc = dev_array(r, &r->qt, U * d, "rotated queries")) ||
        (rc = dev_array(r, &r->qn, U, "query norms")) ||
        (rc = dev_array(r, &r->votes, U * r->Bs * 256, "vote tables")) ||
        (rc = dev_array(r, &r->tot, U * R::kMaxBins, "vote histograms")) ||
        (rc = dev_array(r, &r->scores, U * r->npad, "vote totals")) ||
        (rc = dev_array(r, &r->chist, U * r->nchunk * R::kMaxBins, "chunk histograms")) ||
        (rc = dev_array(r, &r->thr, U * 2, "thresholds")) ||
        (rc = dev_array(r, &r->cand, U * r->C, "candidates")) ||
        (rc = dev_array(r, &r->est, U * r->C, "estimates")) ||
        (rc = dev_array(r, &r->rmm, U * r->nrwg * 2, "estimate ranges")) ||
        (rc = dev_array(r, &r->rng, U * 2, "estimate ranges")) ||
        (rc = dev_array(r, &r->ehtot, U * R::kSelBins, "estimate histograms")) ||
        (rc = dev_array(r, &r->gtb, U * r->nsb, "top-k block counts")) ||
        (rc = dev_array(r, &r->lval, U * r->C, "top-k members")) ||
        (rc = dev_array(r, &r->lidx, U * r->C, "top-k members")) ||
        (rc = dev_array(r, &r->lcnt, U, "top-k member counts")) ||
        (rc = dev_array(r, &r->soff, U * r->nsb, "top-k offsets")) ||
        (rc = dev_array(r, &r->selp, U * 2, "top-k thresholds")) ||
        (rc = dev_array(r, &r->sel, U * r->n_sel, "retrieved")) ||
        (rc = dev_array(r, &r->part, U * r->nsplit * r->G * (d + 2), "partials")))
      return rc;

    // K/V rows: Sink then Local into the near arrays, the retrieval region
    // into the far arrays (device or pinned host memory).
    const char* Kc = static_cast<const char*>(K);
    const char* Vc = static_cast<const char*>(V);
    const size_t sp = static_cast<size_t>(r->T) * row;
    for (int kv = 0; kv < 2; ++kv) {
      const char* src = kv ? Vc : Kc;
      char* near = static_cast<char*>(kv ? r->v_near : r->k_near);
      char* far = static_cast<char*>(kv ? r->v_far : r->k_far);
      const size_t np = static_cast<size_t>(r->n_near) * row;
      if ((rc = copy_rows(near, np, src, sp, r->ns * row, U, st)) ||
          (rc = copy_rows(near + r->ns * row, np, src + r->l0 * row, sp, r->nl * row, U, st)) ||
          (rc = copy_rows(far, N * row, src + r->ns * row, sp, N * row, U, st)))
        return rc;
    }
    RET_HIP(R::launch_encode(r, K, st), "encode launch");
    RET_HIP(hipStreamSynchronize(st), "build synchronize");
    r->magic = R::kMagic;
    *out = r;
    guard.r = nullptr;
    return RSKV_OK;
  } catch (const std::bad_alloc&) {
    return report_error(RSKV_ENOMEM, "host allocation failed");
  } catch (...) {
    return report_error(RSKV_EINVAL, "unexpected error in rskv_retrieval_build");
  }
}

int rskv_retrieval_decode(rskv_retrieval* r, const void* q, float* out, int32_t* retrieved,
                          void* stream) {
  try {
    if (!valid(r)) return report_error(RSKV_ESTATE, "invalid retrieval handle");
    if (q == nullptr || out == nullptr) return report_error(RSKV_EINVAL, "q and out must be non-NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    r->last_stream = st;
    if (!r->prof_on) {
      RET_HIP(R::launch_decode(r, q, out, retrieved, st, nullptr, nullptr), "decode launch");
      return RSKV_OK;
    }
    rskv::KernelEvents ev[R::kKernels];
    for (auto& k : ev)
      for (hipEvent_t* e : {&k.start, &k.stop}) {
        if (r->pool.empty()) {
          hipEvent_t n;
          RET_HIP(hipEventCreate(&n), "event create");
          r->pool.push_back(n);
        }
        *e = r->pool.back();
        r->pool.pop_back();
      }
    bool rec[R::kKernels];
    hipError_t e = R::launch_decode(r, q, out, retrieved, st, ev, rec);
    for (int k = 0; k < R::kKernels; ++k) {
      if (rec[k] && e == hipSuccess) {
        r->pending.push_back(ev[k].start);
        r->pending.push_back(ev[k].stop);
      } else {
        r->pending.push_back(nullptr);
        r->pending.push_back(nullptr);
        r->pool.push_back(ev[k].start);
        r->pool.push_back(ev[k].stop);
      }
    }
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return RSKV_OK;
  } catch (const std::bad_alloc&) {
    return report_error(RSKV_ENOMEM, "host allocation failed");
  } catch (...) {
    return report_error(RSKV_EINVAL, "unexpected error in rskv_retrieval_decode");
  }
}

int rskv_retrieval_info_get(const rskv_retrieval* r, rskv_retrieval_info* i) {
  if (!valid(r)) return report_error(RSKV_ESTATE, "invalid retrieval handle");
  if (i == nullptr) return report_error(RSKV_EINVAL, "info is NULL");
  i->batch = r->B;
  i->n_q_heads = r->Hq;
  i->n_kv_heads = r->Hkv;
  i->head_dim = r->d;
  i->context_len = r->T;
  i->dtype = r->dtype;
  i->m = r->m;
  i->rho = r->rho;
  i->k_ret = r->k_ret;
  i->n_sink = r->ns;
  i->local_start = r->l0;
  i->n_retrieval = r->N;
  i->n_cand = r->C;
  i->n_sel = r->n_sel;
  i->n_attend = r->n_att;
  i->record_bytes = r->rec_bytes;
  i->kv_tier = r->kv_tier;
  i->cand_frac = r->cand_frac;
  i->device_bytes = r->bytes;
  i->host_bytes = r->host_bytes;
  return RSKV_OK;
}

int rskv_retrieval_export(const rskv_retrieval* r, rskv_retrieval_host* a) {
  try {
    if (!valid(r)) return report_error(RSKV_ESTATE, "invalid retrieval handle");
    if (a == nullptr) return report_error(RSKV_EINVAL, "arrays is NULL");
    RET_HIP(hipStreamSynchronize(r->last_stream), "export synchronize");
    const size_t rows = static_cast<size_t>(r->B) * r->Hkv * r->N;
    if (a->buckets && rows)
      RET_HIP(hipMemcpy(a->buckets, r->buckets, rows * r->Bs, hipMemcpyDeviceToHost), "export");
    if ((a->codes || a->w) && rows) {
      std::vector<uint8_t> rec(rows * r->rec_bytes);
      RET_HIP(hipMemcpy(rec.data(), r->rec, rec.size(), hipMemcpyDeviceToHost), "export");
      const size_t half = r->d / 2;
      for (size_t i = 0; i < rows; ++i) {
        if (a->codes) memcpy(a->codes + i * half, rec.data() + i * r->rec_bytes, half);
        if (a->w) memcpy(a->w + i * r->Bs, rec.data() + i * r->rec_bytes + half, r->Bs * 4);
      }
    }
    if (a->beta) {
      for (int j = 0; j < 8; ++j) a->beta[j] = r->cb.beta[j];
      a->beta[8] = 1.0;
    }
    if (a->lambda)
      for (int j = 0; j < 8; ++j) a->lambda[j] = r->cb.lam[j];
    return RSKV_OK;
  } catch (const std::bad_alloc&) {
    return report_error(RSKV_ENOMEM, "host allocation failed");
  }
}

int rskv_retrieval_trace_get(const rskv_retrieval* r, rskv_retrieval_trace* t) {
  if (!valid(r)) return report_error(RSKV_ESTATE, "invalid retrieval handle");
  if (t == nullptr) return report_error(RSKV_EINVAL, "trace is NULL");
  RET_HIP(hipStreamSynchronize(r->last_stream), "trace synchronize");
  const size_t U = static_cast<size_t>(r->B) * r->Hkv;
  auto cp = [&](void* dst, const void* src, size_t bytes) -> hipError_t {
    if (dst == nullptr || bytes == 0) return hipSuccess;
    return hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
  };
  RET_HIP(cp(t->q_rot, r->qt, U * r->d * sizeof(double)), "trace");
  RET_HIP(cp(t->q_norm, r->qn, U * sizeof(double)), "trace");
  RET_HIP(cp(t->votes, r->votes, U * r->Bs * 256), "trace");
  if (t->scores && r->N > 0)
    RET_HIP(hipMemcpy2D(t->scores, r->N * sizeof(uint16_t), r->scores, r->npad * sizeof(uint16_t),
                        r->N * sizeof(uint16_t), U, hipMemcpyDeviceToHost),
            "trace");
  RET_HIP(cp(t->threshold, r->thr, U * 2 * sizeof(int32_t)), "trace");
  RET_HIP(cp(t->cand, r->cand, U * r->C * sizeof(int32_t)), "trace");
  RET_HIP(cp(t->est, r->est, U * r->C * sizeof(float)), "trace");
  RET_HIP(cp(t->retrieved, r->sel, U * r->n_sel * sizeof(int32_t)), "trace");
  return RSKV_OK;
}

int rskv_retrieval_profile_enable(rskv_retrieval* r, int32_t on) {
  if (!valid(r)) return report_error(RSKV_ESTATE, "invalid retrieval handle");
  r->prof_on = on != 0;
  return RSKV_OK;
}

int rskv_retrieval_profile_read(rskv_retrieval* r, rskv_retrieval_profile* p) {
  if (!valid(r)) return report_error(RSKV_ESTATE, "invalid retrieval handle");
  if (p == nullptr) return report_error(RSKV_EINVAL, "prof is NULL");
  constexpr int kEv = 2 * R::kKernels;
  for (size_t s = 0; s + kEv <= r->pending.size(); s += kEv) {
    for (int k = 0; k < R::kKernels; ++k) {
      hipEvent_t a = r->pending[s + 2 * k], b = r->pending[s + 2 * k + 1];
      if (a == nullptr) continue;
      RET_HIP(hipEventSynchronize(b), "event synchronize");
      float ms = 0.f;
      RET_HIP(hipEventElapsedTime(&ms, a, b), "event elapsed");
      r->prof_ms[k] += ms;
    }
    ++r->prof_steps;
  }
  for (hipEvent_t e : r->pending)
    if (e != nullptr) r->pool.push_back(e);
  r->pending.clear();
  p->steps = r->prof_steps;
  for (int k = 0; k < R::kKernels; ++k) p->ms[k] = r->prof_ms[k];
  return RSKV_OK;
}

void rskv_retrieval_destroy(rskv_retrieval* r) {
  if (valid(r)) free_index(r);
}

}  // extern "C"
