// Host runtime of libsekv: argument checks, span planning and building,
// workspace layout and the launch sequence of one decode step.
//
// Pages (by title and section): gist.science German explainer of "SeKV:
// Resolution-Adaptive KV Cache with Hierarchical Semantic Memory for
// Long-Context LLM Inference", "Technisches Resümee" > "Methodik" parts 1-3,
// and its Chinese counterpart "技术摘要" > "方法论" parts 1-3; the authors'
// abstract (GPU summaries, CPU low-rank SVD basis, on-demand reconstruction).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdio>
#include <cstdarg>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/sekv.h"
#include "sekv_factor_cache.h"
#include "sekv_internal.h"

using namespace sekv;

namespace {

thread_local std::string g_err;

sekv_status fail(sekv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sekv_status fail(sekv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_OR_FAIL(call)                                                                  \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) return fail(SEKV_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// ---------------------------------------------------------------- thread pool
class ThreadPool {
 public:
  explicit ThreadPool(int n) {
    for (int i = 0; i < n; ++i) workers_.emplace_back([this] { loop(); });
  }
  ~ThreadPool() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_ = true;
      ++gen_;
    }
    cv_.notify_all();
    for (auto& t : workers_) t.join();
  }
  int size() const { return (int)workers_.size() + 1; }
  // fn(i) for i in [0, n), spread over the workers and the calling thread.
  void parallel_for(int64_t n, const std::function<void(int64_t)>& fn) {
    if (n <= 0) return;
    if (workers_.empty() || n == 1) {
      for (int64_t i = 0; i < n; ++i) fn(i);
      return;
    }
    std::unique_lock<std::mutex> lk(mu_);
    job_ = &fn;
    n_ = n;
    next_.store(0);
    active_ = (int)workers_.size();
    ++gen_;
    lk.unlock();
    cv_.notify_all();
    run();
    lk.lock();
    done_cv_.wait(lk, [this] { return active_ == 0; });
    job_ = nullptr;
  }

 private:
  void run() {
    for (;;) {
      const int64_t i = next_.fetch_add(1);
      if (i >= n_) break;
      (*job_)(i);
    }
  }
  void loop() {
    uint64_t seen = 0;
    for (;;) {
      std::unique_lock<std::mutex> lk(mu_);
      cv_.wait(lk, [&] { return gen_ != seen; });
      seen = gen_;
      if (stop_) return;
      lk.unlock();
      run();
      lk.lock();
      if (--active_ == 0) done_cv_.notify_all();
    }
  }
  std::vector<std::thread> workers_;
  std::mutex mu_;
  std::condition_variable cv_, done_cv_;
  const std::function<void(int64_t)>* job_ = nullptr;
  int64_t n_ = 0;
  std::atomic<int64_t> next_{0};
  int active_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

int default_threads() {
  const char* env = std::getenv("SEKV_THREADS");
  if (env && std::atoi(env) > 0) return std::atoi(env);
  const unsigned hc = std::thread::hardware_concurrency();
  return (int)std::max(1u, std::min(hc == 0 ? 8u : hc, 16u));
}

}  // namespace

constexpr int kRing = 3;
constexpr int kCacheParts = 8;    // default partitions of a device factor cache
constexpr int kCacheChunks = 4;   // fill launches (chunks of partitions) of one cached decode
constexpr size_t kRingBytes = 8u << 20;

struct EventPairs {
  std::vector<hipEvent_t> ev;  // start, stop, start, stop, ...
  size_t used = 0;             // events recorded since the last read
};

struct sekv_ctx {
  int device = 0;
  hipEvent_t ev_list = nullptr, ev_copy = nullptr;
  hipEvent_t ev_ring[kRing] = {};
  ThreadPool* pool = nullptr;
  bool profile = false;
  EventPairs prof_route, prof_attend, prof_expand, prof_overlap, prof_fill;
  hipStream_t aux = nullptr;                          // second stream of sekv_decode_step (default priority)
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;    // its fork / join points
  int32_t split_entries = 0;      // full-resolution entries per split-K chunk (0: automatic)
  int32_t fetch_mode = SEKV_FETCH_DIRECT;
  int32_t build_mode = SEKV_BUILD_DEVICE;
  int32_t fault = SEKV_FAULT_NONE;  // injected failure of the next host-resident decode
  void* route_scratch = nullptr;      // this device's static route state (sekv_route_noalloc)
  int route_resident[2][2][4][2] = {};  // route workgroups resident at once, by dtype, d == 128, log2 G, fold
  // host phases of host-resident decode calls since the last read
  double host_wait_ms = 0, host_gather_ms = 0, host_call_ms = 0;
  int64_t host_calls = 0;
};

namespace {
// Start/stop events of one timed launch (both null while timing is off).
hipError_t prof_pair(sekv_ctx* c, EventPairs& p, hipEvent_t* e0, hipEvent_t* e1) {
  *e0 = *e1 = nullptr;
  if (!c->profile) return hipSuccess;
  while (p.used + 2 > p.ev.size()) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return err;
    p.ev.push_back(e);
  }
  *e0 = p.ev[p.used++];
  *e1 = p.ev[p.used++];
  return hipSuccess;
}
hipError_t prof_sum(EventPairs& p, double* ms, int64_t* n) {
  double tot = 0;
  for (size_t i = 0; i + 1 < p.used; i += 2) {
    hipError_t err = hipEventSynchronize(p.ev[i + 1]);
    if (err != hipSuccess) return err;
    float t = 0;
    err = hipEventElapsedTime(&t, p.ev[i], p.ev[i + 1]);
    if (err != hipSuccess) return err;
    tot += t;
  }
  *ms = tot;
  *n = (int64_t)(p.used / 2);
  p.used = 0;
  return hipSuccess;
}
}  // namespace

namespace {

int elem_size(int dtype) { return dtype == SEKV_BF16 ? 2 : 4; }

// Factor block of one span: Vh_K [r][d] | U [L][rp] | W_V; rp = r rounded up
// to 8, padding zero.  Vh_K row k holds its d/8 groups of 8 elements rotated
// by k (group u at position (u + k) mod d/8).  W_V is the value part of Vh
// transposed, cut into 16-rank column blocks g, each [d][min(16, rp - 16 g)].
// In this order the expanded-span pass consumes the block front to back.
// With separate bases (sep) a second U [L][rp] (the value basis) follows U.
int64_t fac_block_elems(int L, int r, int rp, int D, bool sep = false) {
  return (int64_t)r * D + (int64_t)L * rp * (sep ? 2 : 1) + (int64_t)D * rp;
}
int64_t fac_vk_index(int D, int k, int col) {
  const int ng = D / 8;
  return (int64_t)k * D + (int64_t)(((col / 8) + k) % ng) * 8 + (col % 8);
}
int64_t fac_u_index(int r, int rp, int D, int t, int j) { return (int64_t)r * D + (int64_t)t * rp + j; }
int64_t fac_uv_index(int L, int r, int rp, int D, int t, int j) { return (int64_t)r * D + (int64_t)L * rp + (int64_t)t * rp + j; }
int64_t fac_wv_index(int L, int r, int rp, int D, int col, int j, bool sep = false) {
  const int g = j / 16, wk = std::min(16, rp - 16 * g);
  return (int64_t)r * D + (int64_t)L * rp * (sep ? 2 : 1) + (int64_t)g * 16 * D + (int64_t)col * wk + (j % 16);
}
// sigma|gate entry of one span: sigma [rq] | gate [rq], rq = r rounded up to 4;
// with separate bases sigma_K | gate | sigma_V | gate.
int64_t sg_entry_elems(int r, bool sep = false) { return (sep ? 4 : 2) * (((int64_t)r + 3) & ~(int64_t)3); }

sekv_status check_config(const sekv_config* c) {
  if (!c) return fail(SEKV_EINVAL, "config is NULL");
  if (c->dtype != SEKV_F32 && c->dtype != SEKV_BF16) return fail(SEKV_EINVAL, "dtype %d is not SEKV_F32 or SEKV_BF16", c->dtype);
  if (c->batch < 1 || c->batch > kMaxBatch) return fail(SEKV_ESHAPE, "batch %d outside [1, %d]", c->batch, kMaxBatch);
  if (c->n_ctx < 1) return fail(SEKV_ESHAPE, "n_ctx %d < 1", c->n_ctx);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(SEKV_ESHAPE, "head_dim %d is not 64 or 128", c->head_dim);
  if (c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads != 0)
    return fail(SEKV_ESHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d", c->n_q_heads, c->n_kv_heads);
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(SEKV_ESHAPE, "group size %d is not 1, 2, 4 or 8 (head mask is 8 bits)", G);
  if ((int64_t)c->batch * c->n_kv_heads > kMaxGroups)
    return fail(SEKV_ESHAPE, "batch * n_kv_heads = %d exceeds %d", c->batch * c->n_kv_heads, kMaxGroups);
  if (c->n_sink < 0 || c->n_recent < 0) return fail(SEKV_EINVAL, "n_sink/n_recent must be >= 0");
  if (c->n_sink + c->n_recent < 1) return fail(SEKV_EINVAL, "n_sink + n_recent must be >= 1 (full-resolution set never empty)");
  if ((int64_t)c->n_sink + c->n_recent > c->n_ctx) return fail(SEKV_ESHAPE, "n_sink + n_recent = %d exceeds n_ctx %d", c->n_sink + c->n_recent, c->n_ctx);
  if (c->min_span < 1) return fail(SEKV_EINVAL, "min_span %d < 1", c->min_span);
  if (c->min_span > c->max_span) return fail(SEKV_EINVAL, "min_span %d > max_span %d", c->min_span, c->max_span);
  if (c->max_span > kMaxSpan) return fail(SEKV_ESHAPE, "max_span %d exceeds %d", c->max_span, kMaxSpan);
  if (c->factors_on_host != 0 && c->factors_on_host != 1) return fail(SEKV_EINVAL, "factors_on_host must be 0 or 1");
  if (c->rank_cap != 0 && c->rank_cap != 1) return fail(SEKV_EINVAL, "rank_cap must be 0 or 1");
  if (c->basis != 0 && c->basis != 1) return fail(SEKV_EINVAL, "basis must be 0 or 1");
  if (c->route_keys != 0 && c->route_keys != 1) return fail(SEKV_EINVAL, "route_keys must be 0 or 1");
  if (c->sealed != 0 && c->sealed != 1) return fail(SEKV_EINVAL, "sealed must be 0 or 1");
  if (c->n_ctx_max < 0) return fail(SEKV_EINVAL, "n_ctx_max %d < 0", c->n_ctx_max);
  return SEKV_OK;
}

int32_t cap_ctx(const sekv_config* c) { return std::max(c->n_ctx, c->n_ctx_max); }
int32_t seg_cap_of(const sekv_config* c) {
  return std::max(0, (cap_ctx(c) - c->n_sink - c->n_recent) / (c->min_span + 1)) + 1;
}
// The sealed layout's tail also holds the undecided tokens (min_span + 1) and
// the open span's body (at most max_span) before the recent window.
int32_t full_cap_of(const sekv_config* c) {
  const int64_t extra = c->sealed ? (int64_t)c->min_span + c->max_span : 0;
  return std::min<int64_t>(cap_ctx(c), (int64_t)c->n_sink + seg_cap_of(c) + c->n_recent + 1 + extra);
}

const void* device_address(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return attr.devicePointer;
}

bool is_pinned_host(const void* p) {
  hipPointerAttribute_t attr;
  const hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeHost;
}

sekv_status check_spans(const sekv_config* c, const sekv_spans* s, bool need_factors) {
  if (!s) return fail(SEKV_EINVAL, "spans is NULL");
  if (s->seg_cap != seg_cap_of(c) || s->full_cap != full_cap_of(c))
    return fail(SEKV_ESHAPE, "spans capacities (%d, %d) differ from the configuration's (%d, %d)", s->seg_cap,
                s->full_cap, seg_cap_of(c), full_cap_of(c));
  if (!s->n_seg_host || !s->n_full_host) return fail(SEKV_EINVAL, "n_seg_host / n_full_host is NULL");
  if (!s->seg_off || !s->rank || !s->full_k || !s->full_v || !s->sum_k || !s->sum_v)
    return fail(SEKV_EINVAL, "a span-cache device array is NULL");
  if (c->route_keys == 0 && !s->rho) return fail(SEKV_EINVAL, "route_keys = 0 needs rho");
  if (c->route_keys == 1 && (!s->key_scale || !s->fold)) return fail(SEKV_EINVAL, "route_keys = 1 needs key_scale and fold");
  for (int b = 0; b < c->batch; ++b) {
    if (s->n_seg_host[b] < 0 || s->n_seg_host[b] > s->seg_cap)
      return fail(SEKV_ESHAPE, "n_seg[%d] = %d outside [0, seg_cap=%d]", b, s->n_seg_host[b], s->seg_cap);
    if (s->n_full_host[b] < 1 || s->n_full_host[b] > s->full_cap)
      return fail(SEKV_ESHAPE, "n_full[%d] = %d outside [1, full_cap=%d]", b, s->n_full_host[b], s->full_cap);
  }
  if (need_factors) {
    if (!s->fac_off || !s->sg_off || !s->fac || !s->sg) return fail(SEKV_EINVAL, "factor offsets or pools are NULL");
    if (c->factors_on_host) {
      if (!s->seg_off_host || !s->rank_host || !s->fac_off_host || !s->sg_off_host)
        return fail(SEKV_EINVAL, "host-resident factors need the *_host plan arrays");
      if (!is_pinned_host(s->fac) || !is_pinned_host(s->sg))
        return fail(SEKV_EINVAL, "factors_on_host = 1 needs pinned host pools (hipHostMalloc), got pageable or device memory");
    }
  }
  return SEKV_OK;
}

size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Store an fp64 value in the cache element type: fp64 -> f32 (nearest even) -> bf16 (nearest even).
void store(void* base, int dtype, int64_t i, double x) {
  const float f = (float)x;
  if (dtype == SEKV_BF16) static_cast<uint16_t*>(base)[i] = to_bf16(f);
  else static_cast<float*>(base)[i] = f;
}
double fetch(const void* base, int dtype, int64_t i) {
  return dtype == SEKV_BF16 ? (double)from_bf16(static_cast<const uint16_t*>(base)[i])
                            : (double)static_cast<const float*>(base)[i];
}

// Greedy segmentation of one sequence (see sekv_plan_spans in sekv.h).
int segment_one(const float* s, float thr, const sekv_config* c, int32_t* seg_off, int32_t cap) {
  const int a = c->n_sink, e = c->n_ctx - c->n_recent, lo = c->min_span, hi = c->max_span;
  int n = 0;
  if (e - a < 2) {
    seg_off[0] = a;
    return 0;
  }
  seg_off[n++] = a;
  int h = a;
  for (int t = a + 1; t < e; ++t) {
    const int body = t - h - 1;
    const bool forced = body == hi;
    const bool data = s[t] > thr && body >= lo && (e - t - 1) >= lo;
    if (forced || data) {
      seg_off[n++] = t;
      h = t;
    }
  }
  int tail = e;
  if (h == e - 1) {
    --n;
    tail = h;
  }
  (void)cap;
  seg_off[n] = tail;
  if (c->sealed) {
    // decode-time layout: only the decided heads (t <= e - 1 - lo) stay
    // heads; the last of them starts the tail
    int k = 0;
    while (k < n && seg_off[k] <= e - 1 - lo) ++k;
    if (k == 0) {
      seg_off[0] = a;
      return 0;
    }
    return k - 1;
  }
  return n;
}

// M = P^T P for a d x d row-major P: M[i][j] = sum over rows a of P[a][i] *
// P[a][j], accumulated in row order with every product and sum rounded in fp64.
void fold_matrix(const float* P, int D, double* M) {
#pragma clang fp contract(off)
  for (int i = 0; i < D * D; ++i) M[i] = 0.0;
  for (int a = 0; a < D; ++a)
    for (int i = 0; i < D; ++i) {
      const double pi = (double)P[(size_t)a * D + i];
      for (int j = 0; j < D; ++j) {
        const double prod = pi * (double)P[(size_t)a * D + j];
        M[(size_t)i * D + j] = M[(size_t)i * D + j] + prod;
      }
    }
}

// One-sided Jacobi SVD of an L x n matrix M given by its rows (row-major,
// overwritten).  On return sig[i] (descending), u[t*L + i] = U[t][i] and the
// rows of M hold the right singular vectors' directions scaled by sig (order
// given by perm: output component i is input row perm[i]).
void jacobi_svd(int L, int n, double* M, double* Vc, double* sig, int* perm) {
  for (int i = 0; i < L * L; ++i) Vc[i] = 0.0;
  for (int i = 0; i < L; ++i) Vc[i * L + i] = 1.0;
  const double eps = 1e-15;
  for (int sweep = 0; sweep < 60; ++sweep) {
    bool rotated = false;
    for (int p = 0; p < L - 1; ++p) {
      double* ap = M + (size_t)p * n;
      for (int q = p + 1; q < L; ++q) {
        double* aq = M + (size_t)q * n;
        double al = 0, be = 0, ga = 0;
        for (int k = 0; k < n; ++k) {
          al += ap[k] * ap[k];
          be += aq[k] * aq[k];
          ga += ap[k] * aq[k];
        }
        if (ga == 0.0 || std::fabs(ga) <= eps * std::sqrt(al * be)) continue;
        rotated = true;
        const double zeta = (be - al) / (2.0 * ga);
        const double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        const double cs = 1.0 / std::sqrt(1.0 + t * t), sn = cs * t;
        for (int k = 0; k < n; ++k) {
          const double x = ap[k], y = aq[k];
          ap[k] = cs * x - sn * y;
          aq[k] = sn * x + cs * y;
        }
        double* vp = Vc + (size_t)p * L;
        double* vq = Vc + (size_t)q * L;
        for (int k = 0; k < L; ++k) {
          const double x = vp[k], y = vq[k];
          vp[k] = cs * x - sn * y;
          vq[k] = sn * x + cs * y;
        }
      }
    }
    if (!rotated) break;
  }
  std::vector<double> nrm(L);
  for (int i = 0; i < L; ++i) {
    double acc = 0;
    const double* ai = M + (size_t)i * n;
    for (int k = 0; k < n; ++k) acc += ai[k] * ai[k];
    nrm[i] = std::sqrt(acc);
    perm[i] = i;
  }
  std::stable_sort(perm, perm + L, [&](int x, int y) { return nrm[x] > nrm[y]; });
  for (int i = 0; i < L; ++i) sig[i] = nrm[perm[i]];
}

}  // namespace

// =================================================================== ABI
extern "C" {

const char* sekv_last_error(void) { return g_err.c_str(); }

sekv_status sekv_ctx_create(int device, sekv_ctx** out) {
  if (!out) return fail(SEKV_EINVAL, "out is NULL");
  *out = nullptr;
  int n = 0;
  HIP_OR_FAIL(hipGetDeviceCount(&n));
  if (device < 0 || device >= n) return fail(SEKV_EHIP, "device %d outside [0, %d)", device, n);
  HIP_OR_FAIL(hipSetDevice(device));
  sekv_ctx* c = new (std::nothrow) sekv_ctx();
  if (!c) return fail(SEKV_ENOMEM, "cannot allocate the context");
  c->device = device;
  hipError_t e = hipEventCreateWithFlags(&c->ev_list, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_copy, hipEventDisableTiming);
  for (int i = 0; i < kRing && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&c->ev_ring[i], hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking);
  if (e != hipSuccess) {
    sekv_ctx_destroy(c);
    return fail(SEKV_EHIP, "context setup failed: %s", hipGetErrorString(e));
  }
  e = route_scratch_address(device, &c->route_scratch);
  if (e != hipSuccess) {
    sekv_ctx_destroy(c);
    return fail(SEKV_EHIP, "route scratch setup failed: %s", hipGetErrorString(e));
  }
  c->pool = new ThreadPool(default_threads() - 1);
  *out = c;
  return SEKV_OK;
}

void sekv_ctx_destroy(sekv_ctx* c) {
  if (!c) return;
  for (hipEvent_t e : c->prof_route.ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->prof_attend.ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->prof_expand.ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->prof_overlap.ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->prof_fill.ev) (void)hipEventDestroy(e);
  if (c->aux) (void)hipStreamDestroy(c->aux);
  if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
  if (c->ev_join) (void)hipEventDestroy(c->ev_join);
  if (c->ev_list) (void)hipEventDestroy(c->ev_list);
  if (c->ev_copy) (void)hipEventDestroy(c->ev_copy);
  for (int i = 0; i < kRing; ++i)
    if (c->ev_ring[i]) (void)hipEventDestroy(c->ev_ring[i]);
  delete c->pool;
  delete c;
}

sekv_status sekv_capacities(const sekv_config* cfg, int32_t* seg_cap, int32_t* full_cap) {
  sekv_status st = check_config(cfg);
  if (st != SEKV_OK) return st;
  if (!seg_cap || !full_cap) return fail(SEKV_EINVAL, "seg_cap/full_cap output is NULL");
  *seg_cap = seg_cap_of(cfg);
  *full_cap = full_cap_of(cfg);
  return SEKV_OK;
}

sekv_status sekv_plan_spans(const sekv_config* c, const float* surprisal, const float* thr, const int32_t* rank_req,
                            int32_t* n_seg, int32_t* n_full, int32_t* seg_off, int32_t* rank, int64_t* fac_off,
                            int64_t* sg_off, int64_t* fac_elems, int64_t* sg_elems) {
  sekv_status st = check_config(c);
  if (st != SEKV_OK) return st;
  if (!surprisal || !thr || !rank_req || !n_seg || !n_full || !seg_off || !rank || !fac_off || !sg_off || !fac_elems ||
      !sg_elems)
    return fail(SEKV_EINVAL, "sekv_plan_spans: a pointer argument is NULL");
  const int B = c->batch, T = c->n_ctx, Hkv = c->n_kv_heads, D = c->head_dim;
  const int32_t cap = seg_cap_of(c);
  for (int b = 0; b < B; ++b) {
    if (!std::isfinite(thr[b])) return fail(SEKV_EINVAL, "boundary_thr[%d] is not finite", b);
    for (int t = 0; t < T; ++t)
      if (!std::isfinite(surprisal[(size_t)b * T + t])) return fail(SEKV_EINVAL, "surprisal[%d][%d] is not finite", b, t);
  }
  std::vector<int32_t> so((size_t)B * (cap + 1));
  std::vector<int32_t> ns(B), nf(B);
  for (int b = 0; b < B; ++b) {
    int32_t* sob = so.data() + (size_t)b * (cap + 1);
    const int n = segment_one(surprisal + (size_t)b * T, thr[b], c, sob, cap);
    for (int i = n + 1; i <= cap; ++i) sob[i] = sob[n];
    ns[b] = n;
    nf[b] = c->n_sink + n + (T - sob[n]);
    for (int i = 0; i < n; ++i)
      if (rank_req[(size_t)b * cap + i] < 1) return fail(SEKV_EINVAL, "rank_req[%d][%d] = %d < 1", b, i, rank_req[(size_t)b * cap + i]);
  }
  int64_t fo = 0, go = 0;
  for (int b = 0; b < B; ++b) {
    const int32_t* sob = so.data() + (size_t)b * (cap + 1);
    for (int i = 0; i < cap; ++i) {
      int32_t r = 0;
      if (i < ns[b]) {
        const int L = sob[i + 1] - sob[i] - 1;
        const int Lc = c->rank_cap ? (L + 1) / 2 : L;
        r = std::min(std::min(rank_req[(size_t)b * cap + i], Lc), c->basis ? D : 2 * D);
      }
      rank[(size_t)b * cap + i] = r;
    }
    for (int kv = 0; kv < Hkv; ++kv) {
      for (int i = 0; i < cap; ++i) {
        const size_t o = ((size_t)b * Hkv + kv) * cap + i;
        if (i < ns[b]) {
          const int L = sob[i + 1] - sob[i] - 1;
          const int r = rank[(size_t)b * cap + i];
          const int rp = (r + 7) & ~7;
          fac_off[o] = fo;
          sg_off[o] = go;
          fo += fac_block_elems(L, r, rp, D, c->basis != 0);
          go += sg_entry_elems(r, c->basis != 0);
        } else {
          fac_off[o] = 0;
          sg_off[o] = 0;
        }
      }
    }
  }
  std::memcpy(seg_off, so.data(), so.size() * sizeof(int32_t));
  std::memcpy(n_seg, ns.data(), B * sizeof(int32_t));
  std::memcpy(n_full, nf.data(), B * sizeof(int32_t));
  *fac_elems = fo;
  *sg_elems = go;
  return SEKV_OK;
}

namespace {
size_t seal_lds_bytes(int L);
constexpr int kBuildVldsMax = 90;   // longest span whose eigenvectors stay in LDS beside its Gram matrix

// Device arrays a call allocates for itself and frees on every return path.
struct DevBuffers {
  std::vector<void*> p;
  ~DevBuffers() {
    for (void* x : p) (void)hipFree(x);
  }
  hipError_t alloc(void** out, size_t bytes) {
    *out = nullptr;
    if (bytes == 0) return hipSuccess;
    const hipError_t e = hipMalloc(out, bytes);
    if (e == hipSuccess) p.push_back(*out);
    return e;
  }
};

// sekv_build_spans on the GPU (joint basis): the plan's offsets, per-token
// surprisal weights, projections and gates go up; the full-resolution rows
// are gathered and every span built by kernels; the fold matrices stay host
// work.
sekv_status build_on_device(sekv_ctx* ctx, const sekv_config* c, const void* k, const void* v, const float* surprisal,
                            const float* route_proj, const float* gate, int32_t gate_stride, const sekv_spans* s,
                            int64_t need_f, int64_t need_g, hipStream_t stream) {
  const int B = c->batch, T = c->n_ctx, Hkv = c->n_kv_heads, D = c->head_dim, dt = c->dtype;
  const int es = elem_size(dt);
  const int32_t cap = s->seg_cap, fcap = s->full_cap;
  // surprisal weight of every body token within its span (as the host build)
  std::vector<double> wts((size_t)B * T, 0.0);
  int n_items = 0;
  BuildArgs ba{};
  for (int b = 0; b < B; ++b) {
    const int32_t* so = s->seg_off_host + (size_t)b * (cap + 1);
    const float* sb = surprisal + (size_t)b * T;
    const int ns = s->n_seg_host[b];
    for (int i = 0; i < ns; ++i) {
      const int t0 = so[i] + 1, t1 = so[i + 1], L = t1 - t0;
      double tot = 0;
      for (int t = t0; t < t1; ++t) tot += (double)sb[t];
      for (int t = t0; t < t1; ++t) wts[(size_t)b * T + t] = tot > 0 ? (double)sb[t] / tot : 1.0 / L;
    }
    ba.item_base[b] = n_items;
    ba.n_seg[b] = ns;
    ba.n_full[b] = s->n_full_host[b];
    n_items += Hkv * ns;
  }
  const size_t lds = std::max(seal_lds_bytes(std::min(c->max_span, kBuildVldsMax)), seal_lds_bytes(c->max_span));
  ba.dtype = dt; ba.B = B; ba.Hkv = Hkv; ba.D = D; ba.T = T; ba.seg_cap = cap; ba.full_cap = fcap;
  ba.n_sink = c->n_sink; ba.gate_stride = gate_stride; ba.vlds_max = kBuildVldsMax; ba.n_items = n_items;
  int resident = 0;
  HIP_OR_FAIL(build_resident_blocks(ba, lds, ctx->device, &resident));
  if (resident <= 0) return fail(SEKV_EHIP, "the span build kernel does not fit on the device");
  const int grid = std::max(1, std::min(n_items, resident));
  DevBuffers buf;
  void *d_w, *d_p, *d_g, *d_vs;
  HIP_OR_FAIL(buf.alloc(&d_w, wts.size() * sizeof(double)));
  HIP_OR_FAIL(buf.alloc(&d_p, (size_t)Hkv * D * D * sizeof(float)));
  HIP_OR_FAIL(buf.alloc(&d_g, (size_t)B * Hkv * cap * gate_stride * sizeof(float)));
  HIP_OR_FAIL(buf.alloc(&d_vs, c->max_span > kBuildVldsMax ? (size_t)grid * kMaxSpan * kMaxSpan * sizeof(double) : 0));
  auto up = [&](const void* dst, const void* src, size_t bytes) -> hipError_t {
    return hipMemcpyAsync(const_cast<void*>(dst), src, bytes, hipMemcpyHostToDevice, stream);
  };
  HIP_OR_FAIL(up(d_w, wts.data(), wts.size() * sizeof(double)));
  HIP_OR_FAIL(up(d_p, route_proj, (size_t)Hkv * D * D * sizeof(float)));
  HIP_OR_FAIL(up(d_g, gate, (size_t)B * Hkv * cap * gate_stride * sizeof(float)));
  HIP_OR_FAIL(up(s->seg_off, s->seg_off_host, (size_t)B * (cap + 1) * sizeof(int32_t)));
  HIP_OR_FAIL(up(s->rank, s->rank_host, (size_t)B * cap * sizeof(int32_t)));
  HIP_OR_FAIL(up(s->fac_off, s->fac_off_host, (size_t)B * Hkv * cap * sizeof(int64_t)));
  HIP_OR_FAIL(up(s->sg_off, s->sg_off_host, (size_t)B * Hkv * cap * sizeof(int64_t)));
  // every output starts at zero (padding rows and entries stay zero, as in the host build)
  const int ftiles = (fcap + 31) / 32, stiles = (cap + 31) / 32;
  const size_t BG = (size_t)B * Hkv;
  HIP_OR_FAIL(hipMemsetAsync(const_cast<void*>(s->full_k), 0, BG * fcap * D * es, stream));
  HIP_OR_FAIL(hipMemsetAsync(const_cast<void*>(s->full_v), 0, BG * ftiles * 32 * D * es, stream));
  HIP_OR_FAIL(hipMemsetAsync(const_cast<void*>(s->sum_k), 0, BG * cap * D * es, stream));
  HIP_OR_FAIL(hipMemsetAsync(const_cast<void*>(s->sum_v), 0, BG * stiles * 32 * D * es, stream));
  if (s->rho) HIP_OR_FAIL(hipMemsetAsync(const_cast<void*>(s->rho), 0, BG * cap * D * es, stream));
  if (s->key_scale) HIP_OR_FAIL(hipMemsetAsync(const_cast<float*>(s->key_scale), 0, BG * cap * sizeof(float), stream));
  void* fac = const_cast<void*>(s->fac);
  float* sg = const_cast<float*>(s->sg);
  if (c->factors_on_host) {
    HIP_OR_FAIL(hipStreamSynchronize(stream));
    std::memset(fac, 0, (size_t)need_f * es);
    std::memset(sg, 0, (size_t)need_g * sizeof(float));
    fac = const_cast<void*>(device_address(s->fac));
    sg = static_cast<float*>(const_cast<void*>(device_address(s->sg)));
    if (!fac || !sg) return fail(SEKV_EHIP, "pinned factor pools have no device address");
  } else {
    HIP_OR_FAIL(hipMemsetAsync(fac, 0, (size_t)need_f * es, stream));
    HIP_OR_FAIL(hipMemsetAsync(sg, 0, (size_t)need_g * sizeof(float), stream));
  }
  ba.seg_off = s->seg_off; ba.rank = s->rank; ba.fac_off = s->fac_off; ba.sg_off = s->sg_off;
  ba.weights = static_cast<const double*>(d_w);
  ba.route_proj = static_cast<const float*>(d_p);
  ba.gates = static_cast<const float*>(d_g);
  ba.k = k; ba.v = v;
  ba.full_k = const_cast<void*>(s->full_k); ba.full_v = const_cast<void*>(s->full_v);
  ba.sum_k = const_cast<void*>(s->sum_k); ba.sum_v = const_cast<void*>(s->sum_v);
  ba.rho = const_cast<void*>(s->rho); ba.key_scale = const_cast<float*>(s->key_scale);
  ba.fac = fac; ba.sg = sg;
  ba.vscratch = static_cast<double*>(d_vs);
  HIP_OR_FAIL(launch_build(ba, grid, lds, stream));
  if (s->fold) {
    std::vector<double> fold((size_t)Hkv * D * D, 0.0);
    for (int kv = 0; kv < Hkv; ++kv) fold_matrix(route_proj + (size_t)kv * D * D, D, fold.data() + (size_t)kv * D * D);
    HIP_OR_FAIL(up(s->fold, fold.data(), fold.size() * sizeof(double)));
  }
  HIP_OR_FAIL(hipStreamSynchronize(stream));
  return SEKV_OK;
}
}  // namespace

sekv_status sekv_build_spans(sekv_ctx* ctx, const sekv_config* c, const void* k, const void* v, const float* surprisal,
                             const float* route_proj, const float* gate, int32_t gate_stride, const sekv_spans* s,
                             hipStream_t stream) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  sekv_status st = check_config(c);
  if (st != SEKV_OK) return st;
  if (!k || !v || !surprisal || !route_proj || !gate) return fail(SEKV_EINVAL, "sekv_build_spans: an input is NULL");
  st = check_spans(c, s, true);
  if (st != SEKV_OK) return st;
  if (!s->seg_off_host || !s->rank_host || !s->fac_off_host || !s->sg_off_host)
    return fail(SEKV_EINVAL, "sekv_build_spans needs the plan's host arrays in spans");
  const int B = c->batch, T = c->n_ctx, Hkv = c->n_kv_heads, D = c->head_dim, dt = c->dtype;
  const int es = elem_size(dt);
  const int32_t cap = s->seg_cap, fcap = s->full_cap;
  // pool sizes implied by the plan
  int64_t need_f = 0, need_g = 0;
  for (int b = 0; b < B; ++b)
    for (int kv = 0; kv < Hkv; ++kv)
      for (int i = 0; i < s->n_seg_host[b]; ++i) {
        const size_t o = ((size_t)b * Hkv + kv) * cap + i;
        const int L = s->seg_off_host[(size_t)b * (cap + 1) + i + 1] - s->seg_off_host[(size_t)b * (cap + 1) + i] - 1;
        const int r = s->rank_host[(size_t)b * cap + i];
        const int rmax = std::min(c->rank_cap ? (L + 1) / 2 : L, c->basis ? D : 2 * D);
        if (r < 1 || r > rmax) return fail(SEKV_EINVAL, "rank[%d][%d] = %d outside [1, %d] (L = %d)", b, i, r, rmax, L);
        if (r > gate_stride) return fail(SEKV_ESHAPE, "gate_stride %d < rank %d", gate_stride, r);
        const int rp = (r + 7) & ~7;
        need_f = std::max<int64_t>(need_f, s->fac_off_host[o] + fac_block_elems(L, r, rp, D, c->basis != 0));
        need_g = std::max<int64_t>(need_g, s->sg_off_host[o] + sg_entry_elems(r, c->basis != 0));
        if (s->fac_off_host[o] % 8 != 0 || s->sg_off_host[o] % 4 != 0)
          return fail(SEKV_EINVAL, "pool offsets of span (%d, %d, %d) are not 8- and 4-element aligned", b, kv, i);
      }
  if (need_f > s->fac_elems || need_g > s->sg_elems)
    return fail(SEKV_ECAPACITY, "factor pools hold (%lld, %lld) elements, plan needs (%lld, %lld)", (long long)s->fac_elems,
                (long long)s->sg_elems, (long long)need_f, (long long)need_g);
  HIP_OR_FAIL(hipSetDevice(ctx->device));
  if (ctx->build_mode == SEKV_BUILD_DEVICE && c->basis == 0)
    return build_on_device(ctx, c, k, v, surprisal, route_proj, gate, gate_stride, s, need_f, need_g, stream);

  const size_t kv_elems = (size_t)B * Hkv * T * D;
  std::vector<char> hk(kv_elems * es), hv(kv_elems * es);
  HIP_OR_FAIL(hipMemcpyAsync(hk.data(), k, hk.size(), hipMemcpyDeviceToHost, stream));
  HIP_OR_FAIL(hipMemcpyAsync(hv.data(), v, hv.size(), hipMemcpyDeviceToHost, stream));
  HIP_OR_FAIL(hipStreamSynchronize(stream));

  const int ftiles = (fcap + 31) / 32, stiles = (cap + 31) / 32;
  std::vector<char> full_k((size_t)B * Hkv * fcap * D * es, 0), full_v((size_t)B * Hkv * ftiles * 32 * D * es, 0);
  std::vector<char> sum_k((size_t)B * Hkv * cap * D * es, 0), rho(sum_k.size(), 0);
  std::vector<char> sum_v((size_t)B * Hkv * stiles * 32 * D * es, 0);
  std::vector<float> key_scale((size_t)B * Hkv * cap, 0.0f);
  // value rows live in 32-entry tiles, each stored transposed: (e, j) -> ((e/32)*D + j)*32 + e%32
  auto vt_index = [D](int64_t e, int j) { return ((e / 32) * D + j) * 32 + e % 32; };
  const bool on_host = c->factors_on_host != 0;
  std::vector<char> fac_tmp;
  std::vector<float> sg_tmp;
  char* fac_dst;
  float* sg_dst;
  if (on_host) {
    fac_dst = static_cast<char*>(const_cast<void*>(s->fac));
    sg_dst = const_cast<float*>(s->sg);
  } else {
    fac_tmp.assign((size_t)need_f * es, 0);
    sg_tmp.assign((size_t)need_g, 0.0f);
    fac_dst = fac_tmp.data();
    sg_dst = sg_tmp.data();
  }

  // work items: (b, kv, block of spans)
  constexpr int kSpansPerItem = 64;
  struct Item { int b, kv, i0, i1; };
  std::vector<Item> items;
  for (int b = 0; b < B; ++b)
    for (int kv = 0; kv < Hkv; ++kv) {
      for (int i0 = 0; i0 < s->n_seg_host[b]; i0 += kSpansPerItem)
        items.push_back({b, kv, i0, std::min(s->n_seg_host[b], i0 + kSpansPerItem)});
      if (s->n_seg_host[b] == 0) items.push_back({b, kv, 0, 0});
    }

  ctx->pool->parallel_for((int64_t)items.size(), [&](int64_t it) {
    const Item w = items[it];
    const int b = w.b, kv = w.kv;
    const int32_t* so = s->seg_off_host + (size_t)b * (cap + 1);
    const size_t g = (size_t)b * Hkv + kv;
    const char* kb = hk.data() + g * T * D * es;
    const char* vb = hv.data() + g * T * D * es;
    const float* sb = surprisal + (size_t)b * T;
    const float* P = route_proj + (size_t)kv * D * D;
    // full-resolution rows (once per (b, kv)): sink, anchors, tail
    if (w.i0 == 0) {
      int row = 0;
      const int ns = s->n_seg_host[b];
      char* fvb = full_v.data() + g * ftiles * 32 * D * es;
      auto copy_row = [&](int t) {
        std::memcpy(full_k.data() + (g * fcap + row) * D * es, kb + (size_t)t * D * es, (size_t)D * es);
        for (int j = 0; j < D; ++j)
          std::memcpy(fvb + vt_index(row, j) * es, vb + ((size_t)t * D + j) * es, es);
        ++row;
      };
      for (int t = 0; t < c->n_sink; ++t) copy_row(t);
      for (int i = 0; i < ns; ++i) copy_row(so[i]);
      for (int t = so[ns]; t < T; ++t) copy_row(t);
    }
    std::vector<double> M, Vc, sig, kbar(D), vbar(D), r(D), rh(D);
    std::vector<int> perm;
    for (int i = w.i0; i < w.i1; ++i) {
      const int t0 = so[i] + 1, t1 = so[i + 1], L = t1 - t0;
      // surprisal-weighted summaries
      double tot = 0;
      for (int t = t0; t < t1; ++t) tot += (double)sb[t];
      std::fill(kbar.begin(), kbar.end(), 0.0);
      std::fill(vbar.begin(), vbar.end(), 0.0);
      for (int t = t0; t < t1; ++t) {
        const double wt = tot > 0 ? (double)sb[t] / tot : 1.0 / L;
        for (int j = 0; j < D; ++j) {
          kbar[j] += wt * fetch(kb, dt, (int64_t)t * D + j);
          vbar[j] += wt * fetch(vb, dt, (int64_t)t * D + j);
        }
      }
      // routing key rho = P^T (P kbar / |P kbar|)
      double nn = 0;
      for (int a = 0; a < D; ++a) {
        double acc = 0;
        for (int j = 0; j < D; ++j) acc += (double)P[(size_t)a * D + j] * kbar[j];
        r[a] = acc;
        nn += acc * acc;
      }
      nn = std::sqrt(nn);
      for (int a = 0; a < D; ++a) rh[a] = nn > 0 ? r[a] / nn : 0.0;
      const size_t srow = (g * cap + i) * D;
      const int64_t svbase = (int64_t)g * stiles * 32 * D;
      for (int j = 0; j < D; ++j) {
        double acc = 0;
        for (int a = 0; a < D; ++a) acc += (double)P[(size_t)a * D + j] * rh[a];
        store(rho.data(), dt, (int64_t)srow + j, acc);
        store(sum_k.data(), dt, (int64_t)srow + j, kbar[j]);
        store(sum_v.data(), dt, svbase + vt_index(i, j), vbar[j]);
      }
      key_scale[g * cap + i] = nn > 0 ? (float)(1.0 / nn) : 0.0f;
      // rank-r factors: one basis of [K_body | V_body], or separate bases of
      // K_body (part 0) and V_body (part 1)
      const bool sep = c->basis != 0;
      const int rk = s->rank_host[(size_t)b * cap + i];
      const int rp = (rk + 7) & ~7, rq = (rk + 3) & ~3;
      const size_t o = g * cap + i;
      const int64_t fbase = s->fac_off_host[o];
      const int64_t gbase = s->sg_off_host[o];
      const float* gt = gate + (g * cap + i) * (size_t)gate_stride;
      for (int part = 0; part < (sep ? 2 : 1); ++part) {
        const int n = sep ? D : 2 * D;
        M.assign((size_t)L * n, 0.0);
        for (int t = 0; t < L; ++t)
          for (int j = 0; j < D; ++j) {
            const double kx = fetch(kb, dt, (int64_t)(t0 + t) * D + j), vx = fetch(vb, dt, (int64_t)(t0 + t) * D + j);
            if (sep) {
              M[(size_t)t * n + j] = part == 0 ? kx : vx;
            } else {
              M[(size_t)t * n + j] = kx;
              M[(size_t)t * n + D + j] = vx;
            }
          }
        Vc.resize((size_t)L * L);
        sig.resize(L);
        perm.resize(L);
        jacobi_svd(L, n, M.data(), Vc.data(), sig.data(), perm.data());
        auto u_at = [&](int t, int j) {
          return part == 0 ? fac_u_index(rk, rp, D, t, j) : fac_uv_index(L, rk, rp, D, t, j);
        };
        for (int j = 0; j < rk; ++j) {
          const int src = perm[j];
          const double* u = Vc.data() + (size_t)src * L;  // column src of U
          int imax = 0;
          for (int t = 1; t < L; ++t)
            if (std::fabs(u[t]) > std::fabs(u[imax])) imax = t;
          const double sgn = u[imax] < 0 ? -1.0 : 1.0;
          for (int t = 0; t < L; ++t) store(fac_dst, dt, fbase + u_at(t, j), sgn * u[t]);
          const double sj = sig[j];
          const double inv = sj > 0 ? sgn / sj : 0.0;
          const double* wrow = M.data() + (size_t)src * n;
          for (int col = 0; col < D; ++col) {
            if (!sep || part == 0) store(fac_dst, dt, fbase + fac_vk_index(D, j, col), wrow[col] * inv);
            if (!sep) store(fac_dst, dt, fbase + fac_wv_index(L, rk, rp, D, col, j), wrow[D + col] * inv);
            if (sep && part == 1) store(fac_dst, dt, fbase + fac_wv_index(L, rk, rp, D, col, j, true), wrow[col] * inv);
          }
          sg_dst[gbase + 2 * part * rq + j] = (float)sj;
          sg_dst[gbase + 2 * part * rq + rq + j] = gt[j];
        }
        for (int j = rk; j < rp; ++j) {
          for (int t = 0; t < L; ++t) store(fac_dst, dt, fbase + u_at(t, j), 0.0);
          if (!sep || part == 1)
            for (int col = 0; col < D; ++col) store(fac_dst, dt, fbase + fac_wv_index(L, rk, rp, D, col, j, sep), 0.0);
        }
        for (int j = rk; j < rq; ++j) {
          sg_dst[gbase + 2 * part * rq + j] = 0.0f;
          sg_dst[gbase + 2 * part * rq + rq + j] = 0.0f;
        }
      }
    }
  });

  // fold matrices M = P^T P of the folded routing, accumulated over the rows
  // of P in order (each product and sum rounded in fp64)
  std::vector<double> fold;
  if (s->fold) {
    fold.assign((size_t)Hkv * D * D, 0.0);
    for (int kv = 0; kv < Hkv; ++kv) fold_matrix(route_proj + (size_t)kv * D * D, D, fold.data() + (size_t)kv * D * D);
  }

  auto up = [&](const void* dst, const void* src, size_t bytes) -> hipError_t {
    return hipMemcpyAsync(const_cast<void*>(dst), src, bytes, hipMemcpyHostToDevice, stream);
  };
  HIP_OR_FAIL(up(s->seg_off, s->seg_off_host, (size_t)B * (cap + 1) * sizeof(int32_t)));
  HIP_OR_FAIL(up(s->rank, s->rank_host, (size_t)B * cap * sizeof(int32_t)));
  HIP_OR_FAIL(up(s->fac_off, s->fac_off_host, (size_t)B * Hkv * cap * sizeof(int64_t)));
  HIP_OR_FAIL(up(s->sg_off, s->sg_off_host, (size_t)B * Hkv * cap * sizeof(int64_t)));
  HIP_OR_FAIL(up(s->full_k, full_k.data(), full_k.size()));
  HIP_OR_FAIL(up(s->full_v, full_v.data(), full_v.size()));
  HIP_OR_FAIL(up(s->sum_k, sum_k.data(), sum_k.size()));
  HIP_OR_FAIL(up(s->sum_v, sum_v.data(), sum_v.size()));
  if (s->rho) HIP_OR_FAIL(up(s->rho, rho.data(), rho.size()));
  if (s->key_scale) HIP_OR_FAIL(up(s->key_scale, key_scale.data(), key_scale.size() * sizeof(float)));
  if (s->fold) HIP_OR_FAIL(up(s->fold, fold.data(), fold.size() * sizeof(double)));
  if (!on_host) {
    HIP_OR_FAIL(up(s->fac, fac_tmp.data(), fac_tmp.size()));
    HIP_OR_FAIL(up(s->sg, sg_tmp.data(), sg_tmp.size() * sizeof(float)));
  }
  HIP_OR_FAIL(hipStreamSynchronize(stream));
  return SEKV_OK;
}

// Route workspace: per group a ticket, then per group one status word per
// 256-span tile (all uint32, zero between calls).
static int32_t route_tiles_cap(const sekv_spans* s) { return std::max(1, (s->seg_cap + kRouteThreads - 1) / kRouteThreads); }

// Folded routing adds the folded queries [B][Hq][d] f32 after them.
static size_t route_words_bytes(const sekv_config* c, const sekv_spans* s) {
  const size_t BG = (size_t)c->batch * c->n_kv_heads;
  return align_up(BG * (1 + (size_t)route_tiles_cap(s)) * sizeof(uint32_t));
}

size_t sekv_route_workspace_bytes(const sekv_config* c, const sekv_spans* s) {
  if (check_config(c) != SEKV_OK || !s) return 0;
  size_t n = route_words_bytes(c, s);
  if (c->route_keys) n += align_up((size_t)c->batch * c->n_q_heads * c->head_dim * sizeof(float));
  return n;
}

namespace {
sekv_status route_checked(sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s, const void* q, const float* theta,
                          int32_t* exp_list, uint8_t* exp_mask, int32_t* exp_count) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  sekv_status st = check_config(c);
  if (st != SEKV_OK) return st;
  st = check_spans(c, s, false);
  if (st != SEKV_OK) return st;
  if (!q || !theta || !exp_list || !exp_mask || !exp_count) return fail(SEKV_EINVAL, "sekv_route: a pointer argument is NULL");
  return SEKV_OK;
}

sekv_status route_launch(sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s, const void* q, const float* theta,
                         int32_t* exp_list, uint8_t* exp_mask, int32_t* exp_count, void* ws, bool timed,
                         hipStream_t stream) {
  RouteArgs a{};
  a.dtype = c->dtype;
  a.B = c->batch; a.Hq = c->n_q_heads; a.Hkv = c->n_kv_heads; a.D = c->head_dim; a.seg_cap = s->seg_cap;
  int mx = 0;
  for (int b = 0; b < c->batch; ++b) { a.n_seg[b] = s->n_seg_host[b]; mx = std::max(mx, s->n_seg_host[b]); }
  a.nblk = std::max(1, (mx + kRouteThreads - 1) / kRouteThreads);
  a.nblk_cap = route_tiles_cap(s);
  a.q = q; a.theta = theta; a.rho = c->route_keys ? s->sum_k : s->rho;
  const size_t BG = (size_t)c->batch * c->n_kv_heads;
  a.ticket = static_cast<uint32_t*>(ws);
  a.status = a.ticket + BG;
  a.fold = c->route_keys;
  a.key_scale = s->key_scale;
  a.foldm = s->fold;
  a.qfold = c->route_keys ? reinterpret_cast<float*>(static_cast<char*>(ws) + route_words_bytes(c, s)) : nullptr;
  a.exp_list = exp_list; a.exp_mask = exp_mask; a.exp_count = exp_count;
  HIP_OR_FAIL(hipSetDevice(ctx->device));
  // tiles in dispatch order when the whole grid is resident at once, tickets otherwise
  const int G = c->n_q_heads / c->n_kv_heads;
  int& resident =
      ctx->route_resident[c->dtype == SEKV_BF16][c->head_dim == 128][G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3][c->route_keys];
  if (resident == 0) HIP_OR_FAIL(route_resident_blocks(a, ctx->device, &resident));
  a.use_ticket = (int64_t)a.nblk * c->n_kv_heads * c->batch > resident ? 1 : 0;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (timed) HIP_OR_FAIL(prof_pair(ctx, ctx->prof_route, &e0, &e1));
  HIP_OR_FAIL(launch_route(a, stream, e0, e1));
  return SEKV_OK;
}
}  // namespace

sekv_status sekv_route(sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s, const void* q, const float* theta,
                       int32_t* exp_list, uint8_t* exp_mask, int32_t* exp_count, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  sekv_status st = route_checked(ctx, c, s, q, theta, exp_list, exp_mask, exp_count);
  if (st != SEKV_OK) return st;
  if (!ws) return fail(SEKV_EINVAL, "sekv_route: ws is NULL");
  if (ws_bytes < sekv_route_workspace_bytes(c, s))
    return fail(SEKV_ECAPACITY, "route workspace %zu bytes < %zu needed", ws_bytes, sekv_route_workspace_bytes(c, s));
  return route_launch(ctx, c, s, q, theta, exp_list, exp_mask, exp_count, ws, true, stream);
}

sekv_status sekv_route_noalloc(sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s, const void* q,
                               const float* theta, int32_t* exp_list, uint8_t* exp_mask, int32_t* exp_count,
                               hipStream_t stream) {
  sekv_status st = route_checked(ctx, c, s, q, theta, exp_list, exp_mask, exp_count);
  if (st != SEKV_OK) return st;
  const size_t need = sekv_route_workspace_bytes(c, s);
  if (need > kRouteScratchBytes)
    return fail(SEKV_ECAPACITY, "route state of %zu bytes exceeds the %zu-byte static scratch of sekv_route_noalloc",
                need, kRouteScratchBytes);
  if (!ctx->route_scratch) return fail(SEKV_EHIP, "the context has no route scratch address");
  return route_launch(ctx, c, s, q, theta, exp_list, exp_mask, exp_count, ctx->route_scratch, false, stream);
}

sekv_status sekv_reconstruct(sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s, const int32_t* exp_list,
                             const int32_t* exp_count, int32_t* tok_off, float* k_out, float* v_out, hipStream_t stream) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  sekv_status st = check_config(c);
  if (st != SEKV_OK) return st;
  st = check_spans(c, s, true);
  if (st != SEKV_OK) return st;
  if (!exp_list || !exp_count || !tok_off || !k_out || !v_out) return fail(SEKV_EINVAL, "sekv_reconstruct: a pointer argument is NULL");
  ReconArgs a{};
  a.dtype = c->dtype; a.B = c->batch; a.Hkv = c->n_kv_heads; a.D = c->head_dim; a.seg_cap = s->seg_cap; a.T = c->n_ctx;
  a.sep = c->basis;
  a.seg_off = s->seg_off; a.rank = s->rank; a.fac_off = s->fac_off; a.sg_off = s->sg_off; a.fac = s->fac; a.sg = s->sg;
  a.exp_list = exp_list; a.exp_count = exp_count; a.tok_off = tok_off; a.k_out = k_out; a.v_out = v_out;
  HIP_OR_FAIL(hipSetDevice(ctx->device));
  HIP_OR_FAIL(launch_reconstruct(a, stream));
  return SEKV_OK;
}

namespace {

struct DecodePlan {
  AttendArgs a{};
  size_t off_ml = 0, off_o = 0, off_stage_off = 0, off_stage_fac = 0, off_stage_sg = 0, dev_bytes = 0;
  size_t h_list = 0, h_count = 0, h_stage_off = 0, h_sg = 0, h_ring = 0, h_fill = 0, host_bytes = 0;
};

// How the expanded-span pass reaches the factors: device pools or the direct
// host fetch (no staging), the staged host fetch, or the device factor cache.
enum PlanFetch { kPlanDirect = 0, kPlanStaged = 1, kPlanCached = 2 };

void make_plan(const sekv_config* c, const sekv_spans* s, int32_t split_entries, int fetch, DecodePlan& p) {
  const bool staged = fetch == kPlanStaged, cached = fetch == kPlanCached;
  const int B = c->batch, Hkv = c->n_kv_heads, D = c->head_dim, G = c->n_q_heads / Hkv;
  const int BG = B * Hkv;
  AttendArgs& a = p.a;
  a.dtype = c->dtype; a.B = B; a.Hq = c->n_q_heads; a.Hkv = Hkv; a.D = D;
  a.seg_cap = s->seg_cap; a.full_cap = s->full_cap;
  a.sep = c->basis;
  // 32-entry tiles of the longest (b, kv) full-resolution and summary streams
  int nft = 1, nst = 0;
  for (int b = 0; b < B; ++b) {
    a.n_full[b] = s->n_full_host[b];
    a.n_seg[b] = s->n_seg_host[b];
    nft = std::max(nft, (a.n_full[b] + 31) / 32);
    nst = std::max(nst, (a.n_seg[b] + 31) / 32);
  }
  // about four full-res/summary workgroups per compute unit
  const int64_t target = 1024;
  int64_t tc = ((int64_t)BG * (nft + nst) + target - 1) / target;
  tc = std::max<int64_t>(4, std::min<int64_t>(64, tc));
  if (split_entries > 0) tc = std::max<int64_t>(1, std::min<int64_t>(64, (split_entries + 31) / 32));
  a.tiles_a4 = (int)tc;
  // full-resolution chunks first, then summary chunks; no chunk mixes the two
  a.nch_full = (int)((nft + tc - 1) / tc);
  a.nch_a4 = a.nch_full + (int)((nst + tc - 1) / tc);
  a.a4_lo = 0;
  a.a4_n = a.nch_a4;
  a.chunk_major = 1;
  const int64_t max_items = (int64_t)BG * ((s->seg_cap + kExpChunkMin - 1) / kExpChunkMin);
  a.n_a5_wg = (int)std::max<int64_t>(1, std::min<int64_t>(kExpWaves, max_items));
  // Items of one group: ceil(count / c), where the expanded-span pass takes
  // c = kExpChunk, or max(kExpChunkMin, ceil(listed / waves)).  With
  // c = kExpChunk that is at most ceil(seg_cap / kExpChunk); otherwise either
  // c >= listed / waves >= count / waves, so at most `waves`, or
  // c = kExpChunkMin, so at most ceil(seg_cap / kExpChunkMin).
  a.P_max = a.nch_a4 + (int)std::min<int64_t>((s->seg_cap + kExpChunkMin - 1) / kExpChunkMin,
                                              std::max<int64_t>(a.n_a5_wg, (s->seg_cap + kExpChunk - 1) / kExpChunk));
  a.n_fx_wg = (a.n_a5_wg + 3) / 4;
  a.n_a4_wg = BG * a.nch_a4;
  int mr = 0;
  for (int b = 0; b < B; ++b) {
    const int32_t* rk = s->rank_host + (size_t)b * s->seg_cap;
    for (int i = 0; i < a.n_seg[b]; ++i) mr = std::max(mr, rk[i]);
  }
  a.max_rank = mr;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)D));
  size_t off = 0;
  p.off_ml = off; off = align_up(off + (size_t)BG * a.P_max * G * 2 * sizeof(float));
  p.off_o = off; off = align_up(off + (size_t)BG * a.P_max * G * D * sizeof(float));
  if (staged) {
    p.off_stage_off = off; off = align_up(off + (size_t)BG * (2 * (size_t)s->seg_cap + 1) * sizeof(int64_t));
    p.off_stage_fac = off; off = align_up(off + (size_t)s->fac_elems * elem_size(c->dtype));
    p.off_stage_sg = off; off = align_up(off + (size_t)s->sg_elems * sizeof(float));
  }
  if (cached) {
    p.off_stage_off = off; off = align_up(off + (size_t)BG * (2 * (size_t)s->seg_cap + 1) * sizeof(int64_t));
  }
  p.dev_bytes = off;
  size_t h = 0;
  if (staged) {
    p.h_count = h; h = align_up(h + (size_t)BG * sizeof(int32_t));
    p.h_list = h; h = align_up(h + (size_t)BG * s->seg_cap * sizeof(int32_t));
    p.h_stage_off = h; h = align_up(h + (size_t)BG * (2 * (size_t)s->seg_cap + 1) * sizeof(int64_t));
    p.h_sg = h; h = align_up(h + (size_t)s->sg_elems * sizeof(float));
    p.h_ring = h; h = align_up(h + (size_t)kRing * kRingBytes);
  }
  if (cached) {
    p.h_count = h; h = align_up(h + (size_t)BG * sizeof(int32_t));
    p.h_list = h; h = align_up(h + (size_t)BG * s->seg_cap * sizeof(int32_t));
    p.h_stage_off = h; h = align_up(h + (size_t)BG * (2 * (size_t)s->seg_cap + 1) * sizeof(int64_t));
    p.h_fill = h; h = align_up(h + (size_t)BG * s->seg_cap * sizeof(FillItem));
  }
  p.host_bytes = h;
}

bool staged_fetch(const sekv_ctx* ctx, const sekv_config* c) {
  return c->factors_on_host && ctx && ctx->fetch_mode == SEKV_FETCH_STAGED;
}

}  // namespace

size_t sekv_decode_workspace_bytes(const sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s) {
  if (check_config(c) != SEKV_OK || !s) return 0;
  DecodePlan p;
  make_plan(c, s, ctx ? ctx->split_entries : 0, staged_fetch(ctx, c) ? kPlanStaged : kPlanDirect, p);
  return p.dev_bytes;
}

size_t sekv_decode_host_workspace_bytes(const sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s) {
  if (check_config(c) != SEKV_OK || !s) return 0;
  DecodePlan p;
  make_plan(c, s, ctx ? ctx->split_entries : 0, staged_fetch(ctx, c) ? kPlanStaged : kPlanDirect, p);
  return p.host_bytes;
}

namespace {
// Checks shared by the decode entry points, and the attention arguments of
// one call (all chunks of the full-resolution + summary pass).
sekv_status decode_setup(sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s, const void* q,
                         const int32_t* exp_list, const uint8_t* exp_mask, const int32_t* exp_count, float* out,
                         void* dev_ws, size_t dev_ws_bytes, int fetch, const char* who, DecodePlan& p,
                         AttendArgs& a) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  sekv_status st = check_config(c);
  if (st != SEKV_OK) return st;
  st = check_spans(c, s, true);
  if (st != SEKV_OK) return st;
  if (!q || !exp_list || !exp_mask || !exp_count || !out || !dev_ws)
    return fail(SEKV_EINVAL, "%s: a pointer argument is NULL", who);
  make_plan(c, s, ctx->split_entries, fetch, p);
  if (dev_ws_bytes < p.dev_bytes) return fail(SEKV_ECAPACITY, "device workspace %zu bytes < %zu needed", dev_ws_bytes, p.dev_bytes);
  if (p.a.tiles_a4 * 32 > 2048) return fail(SEKV_ESHAPE, "internal chunk size too large");
  a = p.a;
  char* dws = static_cast<char*>(dev_ws);
  a.q = q; a.full_k = s->full_k; a.full_v = s->full_v; a.sum_k = s->sum_k; a.sum_v = s->sum_v;
  a.seg_off = s->seg_off; a.rank = s->rank; a.fac_off = s->fac_off; a.sg_off = s->sg_off; a.fac = s->fac; a.sg = s->sg;
  a.exp_list = exp_list; a.exp_mask = exp_mask; a.exp_count = exp_count;
  a.part_ml = reinterpret_cast<float*>(dws + p.off_ml);
  a.part_o = reinterpret_cast<float*>(dws + p.off_o);
  a.out = out;
  a.stage_off = nullptr;
  if (c->factors_on_host && fetch == kPlanDirect) {
    // direct fetch: the kernels read the listed spans' factor blocks from the
    // pinned host pools over the bus, through the pools' device addresses
    a.fac = device_address(s->fac);
    a.sg = static_cast<const float*>(device_address(s->sg));
    if (!a.fac || !a.sg) return fail(SEKV_EHIP, "pinned factor pools have no device address");
  }
  return SEKV_OK;
}

// The attention launches on device-visible factors for the role-A chunks
// a.a4_lo .. a.a4_lo + a.a4_n - 1 of each (b, kv), then the combine.
hipError_t launch_attention(sekv_ctx* ctx, AttendArgs a, hipStream_t stream) {
  const int BG = a.B * a.Hkv;
  a.n_a4_wg = BG * a.a4_n;
  hipEvent_t e0, e1;
  if (a.max_rank <= 64) {
    // both passes in one launch on the caller's stream
    hipError_t e = prof_pair(ctx, ctx->prof_attend, &e0, &e1);
    if (e == hipSuccess) e = launch_attend_fused(a, stream, e0, e1);
    if (e != hipSuccess) return e;
  } else {
    hipError_t e = prof_pair(ctx, ctx->prof_expand, &e0, &e1);
    if (e == hipSuccess) e = launch_attend_expanded(a, stream, e0, e1);
    if (e == hipSuccess) e = prof_pair(ctx, ctx->prof_attend, &e0, &e1);
    if (e == hipSuccess) e = launch_attend_full(a, stream, e0, e1);
    if (e != hipSuccess) return e;
  }
  return launch_combine(a, stream);
}
}  // namespace

sekv_status sekv_mixed_attention_decode(sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s, const void* q,
                                        const int32_t* exp_list, const uint8_t* exp_mask, const int32_t* exp_count,
                                        float* out, void* dev_ws, size_t dev_ws_bytes, void* host_ws,
                                        size_t host_ws_bytes, hipStream_t stream, hipStream_t copy_stream) {
  const bool staged = ctx && c && staged_fetch(ctx, c);
  DecodePlan p;
  AttendArgs a;
  sekv_status st = decode_setup(ctx, c, s, q, exp_list, exp_mask, exp_count, out, dev_ws, dev_ws_bytes,
                                staged ? kPlanStaged : kPlanDirect,
                                "sekv_mixed_attention_decode", p, a);
  if (st != SEKV_OK) return st;
  if (staged) {
    if (!host_ws) return fail(SEKV_EINVAL, "host-resident factors need a pinned host workspace");
    if (host_ws_bytes < p.host_bytes) return fail(SEKV_ECAPACITY, "host workspace %zu bytes < %zu needed", host_ws_bytes, p.host_bytes);
    if (!is_pinned_host(host_ws)) return fail(SEKV_EINVAL, "host workspace must be pinned (hipHostMalloc)");
  }
  if (!copy_stream) copy_stream = stream;
  HIP_OR_FAIL(hipSetDevice(ctx->device));
  char* dws = static_cast<char*>(dev_ws);

  if (!staged) {
    HIP_OR_FAIL(launch_attention(ctx, a, stream));
    return SEKV_OK;
  }

  // ---- host-resident factors
  const int B = c->batch, Hkv = c->n_kv_heads, D = c->head_dim, BG = B * Hkv;
  const int es = elem_size(c->dtype);
  const int32_t cap = s->seg_cap;
  char* hws = static_cast<char*>(host_ws);
  int32_t* h_count = reinterpret_cast<int32_t*>(hws + p.h_count);
  int32_t* h_list = reinterpret_cast<int32_t*>(hws + p.h_list);
  int64_t* h_soff = reinterpret_cast<int64_t*>(hws + p.h_stage_off);
  float* h_sg = reinterpret_cast<float*>(hws + p.h_sg);
  char* h_ring = hws + p.h_ring;
  const auto t_call = std::chrono::steady_clock::now();
  // previous call's copies must be done before the pinned buffers are reused
  HIP_OR_FAIL(hipEventSynchronize(ctx->ev_copy));
  HIP_OR_FAIL(hipMemcpyAsync(h_count, exp_count, BG * sizeof(int32_t), hipMemcpyDeviceToHost, stream));
  HIP_OR_FAIL(hipMemcpyAsync(h_list, exp_list, (size_t)BG * cap * sizeof(int32_t), hipMemcpyDeviceToHost, stream));
  HIP_OR_FAIL(hipEventRecord(ctx->ev_list, stream));
  // full-resolution + summary pass runs while the host gathers
  hipEvent_t t0, t1;
  HIP_OR_FAIL(prof_pair(ctx, ctx->prof_attend, &t0, &t1));
  HIP_OR_FAIL(launch_attend_full(a, stream, t0, t1));
  const auto t_wait = std::chrono::steady_clock::now();
  HIP_OR_FAIL(hipEventSynchronize(ctx->ev_list));
  const auto t_listed = std::chrono::steady_clock::now();
  if (ctx->fault == SEKV_FAULT_GATHER) {
    ctx->fault = SEKV_FAULT_NONE;
    return fail(SEKV_EHIP, "factor gather failed (injected by sekv_ctx_inject_fault); out was not written");
  }

  // staging layout in list order; the offset table is [BG] per-group bases
  // (in list entries) followed by one (fac, sg) offset pair per listed entry
  struct Ent { const char* src; int64_t bytes; int64_t dst; };
  std::vector<Ent> ents;
  int64_t fo = 0, go = 0, ne = 0;
  for (int g = 0; g < BG; ++g) {
    const int b = g / Hkv;
    const int cnt = h_count[g];
    if (cnt < 0 || cnt > s->n_seg_host[b])
      return fail(SEKV_EHIP, "route count %d for group %d is out of range; out was not written", cnt, g);
    h_soff[g] = ne;
    const int32_t* so = s->seg_off_host + (size_t)b * (cap + 1);
    for (int j = 0; j < cnt; ++j) {
      const int S = h_list[(size_t)g * cap + j];
      if (S < 0 || S >= s->n_seg_host[b])
        return fail(SEKV_EHIP, "route list entry %d out of range; out was not written", S);
      const int L = so[S + 1] - so[S] - 1;
      const int r = s->rank_host[(size_t)b * cap + S];
      const int rp = (r + 7) & ~7;
      const int64_t fe = fac_block_elems(L, r, rp, D, c->basis != 0);
      const size_t o = (size_t)g * cap + S;
      ents.push_back({static_cast<const char*>(s->fac) + s->fac_off_host[o] * es, fe * es, fo});
      h_soff[BG + 2 * (ne + j)] = fo;
      h_soff[BG + 2 * (ne + j) + 1] = go;
      std::memcpy(h_sg + go, s->sg + s->sg_off_host[o], sg_entry_elems(r, c->basis != 0) * sizeof(float));
      fo += fe;
      go += sg_entry_elems(r, c->basis != 0);
    }
    ne += cnt;
  }
  char* d_stage_fac = dws + p.off_stage_fac;
  HIP_OR_FAIL(hipMemcpyAsync(dws + p.off_stage_off, h_soff, (size_t)(BG + 2 * ne) * sizeof(int64_t), hipMemcpyHostToDevice, copy_stream));
  HIP_OR_FAIL(hipMemcpyAsync(dws + p.off_stage_sg, h_sg, (size_t)go * sizeof(float), hipMemcpyHostToDevice, copy_stream));
  // gather factor blocks into pinned ring buffers, copy each as it fills
  size_t e0 = 0;
  int slot = 0;
  double gather_ms = 0;
  std::vector<int> used(kRing, 0);
  while (e0 < ents.size()) {
    size_t e1 = e0;
    int64_t bytes = 0;
    while (e1 < ents.size() && bytes + ents[e1].bytes <= (int64_t)kRingBytes) bytes += ents[e1++].bytes;
    if (used[slot]) HIP_OR_FAIL(hipEventSynchronize(ctx->ev_ring[slot]));
    char* buf = h_ring + (size_t)slot * kRingBytes;
    const int64_t base = ents[e0].dst;
    const auto t_g0 = std::chrono::steady_clock::now();
    ctx->pool->parallel_for((int64_t)(e1 - e0), [&](int64_t i) {
      const Ent& en = ents[e0 + i];
      std::memcpy(buf + (en.dst - base) * es, en.src, en.bytes);
    });
    gather_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t_g0).count();
    HIP_OR_FAIL(hipMemcpyAsync(d_stage_fac + base * es, buf, bytes, hipMemcpyHostToDevice, copy_stream));
    HIP_OR_FAIL(hipEventRecord(ctx->ev_ring[slot], copy_stream));
    used[slot] = 1;
    slot = (slot + 1) % kRing;
    e0 = e1;
  }
  HIP_OR_FAIL(hipEventRecord(ctx->ev_copy, copy_stream));
  if (copy_stream != stream) HIP_OR_FAIL(hipStreamWaitEvent(stream, ctx->ev_copy, 0));
  AttendArgs a5 = a;
  a5.stage_off = reinterpret_cast<const int64_t*>(dws + p.off_stage_off);
  a5.stage_fac = d_stage_fac;
  a5.stage_sg = reinterpret_cast<const float*>(dws + p.off_stage_sg);
  HIP_OR_FAIL(prof_pair(ctx, ctx->prof_expand, &t0, &t1));
  HIP_OR_FAIL(launch_attend_expanded(a5, stream, t0, t1));
  HIP_OR_FAIL(launch_combine(a, stream));
  const auto t_end = std::chrono::steady_clock::now();
  ctx->host_wait_ms += std::chrono::duration<double, std::milli>(t_listed - t_wait).count();
  ctx->host_gather_ms += gather_ms;
  ctx->host_call_ms += std::chrono::duration<double, std::milli>(t_end - t_call).count();
  ctx->host_calls += 1;
  return SEKV_OK;
}

// ---------------------------------------------------------------- device factor cache
extern "C++" {
namespace {
// One listed entry of a cache batch, prepared by cache_prepare.
struct CacheItem {
  uint64_t key;
  int64_t bytes, tag;    // block bytes (factor block + sigma|gate entry), host address of the block
  int64_t fac, sg;       // pool element offsets of the factor block and the sigma|gate entry
  int32_t fb, g;         // factor block bytes, group
};
}  // namespace
}  // extern "C++"

struct sekv_factor_cache {
  sekv_factor_cache(int64_t bytes, int parts) : book(bytes, parts) {}
  FactorCacheBook book;
  int device = -1;
  char* arena = nullptr;          // device memory of book.arena_bytes() (null: bookkeeping only)
  hipEvent_t ev_read = nullptr;   // end of the last expanded-span pass that read the arena
  bool read_recorded = false;
  std::vector<CacheItem> items;   // the current call's listed entries
};

extern "C++" {
namespace {
// Host arrays a cache lookup reads, checked.
sekv_status check_cache_spans(const sekv_config* c, const sekv_spans* s) {
  sekv_status st = check_config(c);
  if (st != SEKV_OK) return st;
  if (!s) return fail(SEKV_EINVAL, "spans is NULL");
  if (s->seg_cap != seg_cap_of(c)) return fail(SEKV_ESHAPE, "spans seg_cap %d differs from the configuration's %d", s->seg_cap, seg_cap_of(c));
  if (!s->n_seg_host || !s->seg_off_host || !s->rank_host || !s->fac_off_host || !s->sg_off_host)
    return fail(SEKV_EINVAL, "the factor cache needs n_seg_host, seg_off_host, rank_host, fac_off_host and sg_off_host");
  for (int b = 0; b < c->batch; ++b)
    if (s->n_seg_host[b] < 0 || s->n_seg_host[b] > s->seg_cap)
      return fail(SEKV_ESHAPE, "n_seg[%d] = %d outside [0, seg_cap=%d]", b, s->n_seg_host[b], s->seg_cap);
  return SEKV_OK;
}

// Checks a route list (host copies h_count [B*Hkv], h_list [B*Hkv][seg_cap]):
// counts, span indices, span shapes and pool bounds of every listed entry,
// so that a bad list leaves the cache untouched; and prepares the entries in
// list order (group-major) for cache_lookup_items.
sekv_status cache_prepare(int32_t layer, const sekv_config* c, const sekv_spans* s, const int32_t* h_count,
                          const int32_t* h_list, std::vector<CacheItem>& items) {
  const int Hkv = c->n_kv_heads, D = c->head_dim, BG = c->batch * Hkv;
  const int es = elem_size(c->dtype);
  const bool sep = c->basis != 0;
  const int32_t cap = s->seg_cap;
  items.clear();
  for (int g = 0; g < BG; ++g) {
    const int b = g / Hkv, cnt = h_count[g];
    if (cnt < 0 || cnt > s->n_seg_host[b])
      return fail(SEKV_EHIP, "route count %d for group %d is out of range; out was not written", cnt, g);
    const int32_t* so = s->seg_off_host + (size_t)b * (cap + 1);
    const int32_t* rk = s->rank_host + (size_t)b * cap;
    const int64_t* fo = s->fac_off_host + (size_t)g * cap;
    const int64_t* go = s->sg_off_host + (size_t)g * cap;
    const int32_t* lst = h_list + (size_t)g * cap;
    for (int j = 0; j < cnt; ++j) {
      const int S = lst[j];
      if (S < 0 || S >= s->n_seg_host[b])
        return fail(SEKV_EHIP, "route list entry %d out of range; out was not written", S);
      const int L = so[S + 1] - so[S] - 1, r = rk[S];
      if (L < 1 || L > kMaxSpan || r < 1 || r > L) return fail(SEKV_ESHAPE, "span %d of sequence %d has L = %d, r = %d", S, b, L, r);
      const int64_t fe = fac_block_elems(L, r, (r + 7) & ~7, D, sep), ge = sg_entry_elems(r, sep);
      if (fo[S] < 0 || fo[S] + fe > s->fac_elems || go[S] < 0 || go[S] + ge > s->sg_elems)
        return fail(SEKV_ESHAPE, "factor block of span %d (group %d) lies outside the pools", S, g);
      // tag: the block's host address, so a different pool under the same key refills
      items.push_back(CacheItem{FactorCacheBook::key(layer, g, S), fe * es + ge * 4,
                                (int64_t)((uintptr_t)s->fac + (uintptr_t)(fo[S] * es)), fo[S], go[S],
                                (int32_t)(fe * es), g});
    }
  }
  return SEKV_OK;
}

}  // namespace
}  // extern "C++"

sekv_status sekv_factor_cache_create(sekv_ctx* ctx, size_t bytes, int32_t partitions, sekv_factor_cache** out) {
  if (!out) return fail(SEKV_EINVAL, "out is NULL");
  *out = nullptr;
  if (partitions == 0) partitions = kCacheParts;
  if (partitions < 1 || partitions > 256) return fail(SEKV_EINVAL, "partitions %d outside [1, 256]", partitions);
  if ((int64_t)bytes < FactorCacheBook::kPageBytes * partitions)
    return fail(SEKV_ESHAPE, "a factor cache of %zu bytes has less than one %lld-byte page per partition (%d)",
                bytes, (long long)FactorCacheBook::kPageBytes, partitions);
  sekv_factor_cache* fc = new (std::nothrow) sekv_factor_cache((int64_t)bytes, partitions);
  if (!fc) return fail(SEKV_ENOMEM, "cannot allocate the factor cache");
  if (ctx) {
    fc->device = ctx->device;
    hipError_t e = hipSetDevice(ctx->device);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&fc->arena), (size_t)fc->book.arena_bytes());
    if (e == hipSuccess) e = hipEventCreateWithFlags(&fc->ev_read, hipEventDisableTiming);
    if (e != hipSuccess) {
      sekv_factor_cache_destroy(fc);
      return fail(SEKV_EHIP, "factor cache arena of %lld bytes: %s", (long long)fc->book.arena_bytes(), hipGetErrorString(e));
    }
  }
  *out = fc;
  return SEKV_OK;
}

void sekv_factor_cache_destroy(sekv_factor_cache* fc) {
  if (!fc) return;
  if (fc->ev_read) {
    (void)hipEventSynchronize(fc->ev_read);
    (void)hipEventDestroy(fc->ev_read);
  }
  if (fc->arena) (void)hipFree(fc->arena);
  delete fc;
}

sekv_status sekv_factor_cache_invalidate(sekv_factor_cache* fc, int32_t layer) {
  if (!fc) return fail(SEKV_EINVAL, "cache is NULL");
  if (layer < -1 || layer > 65535) return fail(SEKV_EINVAL, "layer %d outside [-1, 65535]", layer);
  if (layer < 0) fc->book.clear();
  else fc->book.invalidate(layer);
  return SEKV_OK;
}

sekv_status sekv_factor_cache_stats(sekv_factor_cache* fc, sekv_cache_stats* out, int32_t reset) {
  if (!fc || !out) return fail(SEKV_EINVAL, "cache or out is NULL");
  const FactorCacheBook::Stats& st = fc->book.stats();
  out->lookups = st.lookups;
  out->hits = st.hits;
  out->fills = st.fills;
  out->bypasses = st.bypasses;
  out->evictions = st.evictions;
  out->bytes_hit = st.bytes_hit;
  out->bytes_filled = st.bytes_filled;
  out->bytes_bypassed = st.bytes_bypassed;
  out->resident_blocks = fc->book.resident_blocks();
  out->resident_bytes = fc->book.resident_bytes();
  out->pages_used = fc->book.pages_used();
  out->pages_total = fc->book.pages();
  if (reset) fc->book.reset_stats();
  return SEKV_OK;
}

sekv_status sekv_factor_cache_lookup(sekv_factor_cache* fc, int32_t layer, const sekv_config* c, const sekv_spans* s,
                                     const int32_t* exp_list, const int32_t* exp_count, int32_t* status,
                                     int64_t* offset) {
  if (!fc) return fail(SEKV_EINVAL, "cache is NULL");
  if (layer < 0 || layer > 65535) return fail(SEKV_EINVAL, "layer %d outside [0, 65535]", layer);
  sekv_status st = check_cache_spans(c, s);
  if (st != SEKV_OK) return st;
  if (!exp_list || !exp_count || !status || !offset) return fail(SEKV_EINVAL, "a pointer argument is NULL");
  const int32_t cap = s->seg_cap;
  st = cache_prepare(layer, c, s, exp_count, exp_list, fc->items);
  if (st != SEKV_OK) return st;
  fc->book.begin();
  int g = 0, j = 0;
  for (const CacheItem& it : fc->items) {
    if (it.g != g) {
      g = it.g;
      j = 0;
    }
    int64_t off = -1;
    status[(size_t)g * cap + j] = fc->book.part(fc->book.part_of_group(g)).lookup(it.key, it.bytes, it.tag, &off);
    offset[(size_t)g * cap + j] = off;
    ++j;
  }
  return SEKV_OK;
}

size_t sekv_cached_decode_workspace_bytes(const sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s) {
  if (check_config(c) != SEKV_OK || !s) return 0;
  DecodePlan p;
  make_plan(c, s, ctx ? ctx->split_entries : 0, kPlanCached, p);
  return p.dev_bytes;
}

size_t sekv_cached_decode_host_workspace_bytes(const sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s) {
  if (check_config(c) != SEKV_OK || !s) return 0;
  DecodePlan p;
  make_plan(c, s, ctx ? ctx->split_entries : 0, kPlanCached, p);
  return p.host_bytes;
}

sekv_status sekv_cached_attention_decode(sekv_ctx* ctx, sekv_factor_cache* fc, int32_t layer, const sekv_config* c,
                                         const sekv_spans* s, const void* q, const int32_t* exp_list,
                                         const uint8_t* exp_mask, const int32_t* exp_count, float* out,
                                         void* dev_ws, size_t dev_ws_bytes, void* host_ws, size_t host_ws_bytes,
                                         hipStream_t stream, hipStream_t copy_stream) {
  if (!fc) return fail(SEKV_EINVAL, "cache is NULL");
  if (!fc->arena) return fail(SEKV_EINVAL, "the cache has no device arena (it was created without a context)");
  if (ctx && fc->device != ctx->device) return fail(SEKV_EINVAL, "the cache lives on device %d, the context on %d", fc->device, ctx->device);
  if (layer < 0 || layer > 65535) return fail(SEKV_EINVAL, "layer %d outside [0, 65535]", layer);
  if (c && c->factors_on_host != 1) return fail(SEKV_EINVAL, "the factor cache serves host-resident factors (factors_on_host = 1)");
  DecodePlan p;
  AttendArgs a;
  sekv_status st = decode_setup(ctx, c, s, q, exp_list, exp_mask, exp_count, out, dev_ws, dev_ws_bytes, kPlanCached,
                                "sekv_cached_attention_decode", p, a);
  if (st != SEKV_OK) return st;
  if (!host_ws) return fail(SEKV_EINVAL, "the cached decode needs a pinned host workspace");
  if (host_ws_bytes < p.host_bytes) return fail(SEKV_ECAPACITY, "host workspace %zu bytes < %zu needed", host_ws_bytes, p.host_bytes);
  if (!is_pinned_host(host_ws)) return fail(SEKV_EINVAL, "host workspace must be pinned (hipHostMalloc)");
  const char* fac_dev = static_cast<const char*>(device_address(s->fac));
  const char* sg_dev = static_cast<const char*>(device_address(s->sg));
  if (!fac_dev || !sg_dev) return fail(SEKV_EHIP, "pinned factor pools have no device address");
  if (!copy_stream) copy_stream = stream;
  HIP_OR_FAIL(hipSetDevice(ctx->device));

  const int BG = c->batch * c->n_kv_heads;
  const int es = elem_size(c->dtype);
  const int32_t cap = s->seg_cap;
  char* dws = static_cast<char*>(dev_ws);
  char* hws = static_cast<char*>(host_ws);
  int32_t* h_count = reinterpret_cast<int32_t*>(hws + p.h_count);
  int32_t* h_list = reinterpret_cast<int32_t*>(hws + p.h_list);
  int64_t* h_soff = reinterpret_cast<int64_t*>(hws + p.h_stage_off);
  FillItem* h_fill = reinterpret_cast<FillItem*>(hws + p.h_fill);
  const auto t_call = std::chrono::steady_clock::now();
  // the previous host-resident call's uploads from pinned staging must be done
  HIP_OR_FAIL(hipEventSynchronize(ctx->ev_copy));
  HIP_OR_FAIL(hipMemcpyAsync(h_count, exp_count, BG * sizeof(int32_t), hipMemcpyDeviceToHost, stream));
  HIP_OR_FAIL(hipMemcpyAsync(h_list, exp_list, (size_t)BG * cap * sizeof(int32_t), hipMemcpyDeviceToHost, stream));
  HIP_OR_FAIL(hipEventRecord(ctx->ev_list, stream));
  // the full-resolution + summary pass runs while the host does the bookkeeping and the fills run
  hipEvent_t t0, t1;
  HIP_OR_FAIL(prof_pair(ctx, ctx->prof_attend, &t0, &t1));
  HIP_OR_FAIL(launch_attend_full(a, stream, t0, t1));
  const auto t_wait = std::chrono::steady_clock::now();
  HIP_OR_FAIL(hipEventSynchronize(ctx->ev_list));
  const auto t_listed = std::chrono::steady_clock::now();

  // stage table: per group the first list entry, then (factor, sigma|gate)
  // offsets per entry, in elements from the arena base (also for bypassed
  // blocks, which are read from the pinned pools through their device address)
  st = cache_prepare(layer, c, s, h_count, h_list, fc->items);
  if (st != SEKV_OK) return st;
  const std::vector<CacheItem>& items = fc->items;
  const size_t ne = items.size();
  {
    int64_t base = 0;
    for (int g = 0; g < BG; ++g) {
      h_soff[g] = base;
      base += h_count[g];
    }
  }
  const FillItem* d_fill = static_cast<const FillItem*>(device_address(h_fill));
  if (!d_fill) return fail(SEKV_EHIP, "the pinned host workspace has no device address");
  int64_t* d_soff = reinterpret_cast<int64_t*>(dws + p.off_stage_off);
  // slots being refilled may still be read by the previous cached call's expanded pass
  if (fc->read_recorded) HIP_OR_FAIL(hipStreamWaitEvent(copy_stream, fc->ev_read, 0));
  // bookkeeping partition by partition (each over its groups' entries in list
  // order); after every chunk of partitions its fills start on the copy
  // stream while the host works on the next chunk
  fc->book.begin();
  const int P = std::min(fc->book.parts(), BG);
  const int per = (P + kCacheChunks - 1) / kCacheChunks;
  const intptr_t arena = (intptr_t)fc->arena;
  const int64_t arena_bytes = fc->book.arena_bytes();
  int64_t* ent = h_soff + BG;   // (factor, sigma|gate) offsets per entry, list order
  bool bad_slot = false;
  int n_fill = 0;
  for (int p0 = 0; p0 < P && !bad_slot; p0 += per) {
    const int f0 = n_fill;
    for (int pi = p0; pi < std::min(P, p0 + per) && !bad_slot; ++pi) {
      CachePart& part = fc->book.part(pi);
      for (int g = pi; g < BG && !bad_slot; g += fc->book.parts()) {
        for (int64_t i = h_soff[g], i1 = h_soff[g] + h_count[g]; i < i1; ++i) {
          const CacheItem& it = items[i];
          int64_t off = -1;
          const int32_t stt = part.lookup(it.key, it.bytes, it.tag, &off);
          int64_t* e = ent + 2 * i;
          const intptr_t fsrc = (intptr_t)(fac_dev + it.fac * es);
          const intptr_t gsrc = (intptr_t)(sg_dev + it.sg * 4);
          if (stt == CachePart::kBypass) {
            e[0] = (int64_t)(fsrc - arena) / es;
            e[1] = (int64_t)(gsrc - arena) / 4;
            continue;
          }
          if (off < 0 || off + it.bytes > arena_bytes) {
            bad_slot = true;
            break;
          }
          e[0] = off / es;
          e[1] = (off + it.fb) / 4;
          if (stt == CachePart::kFill)
            h_fill[n_fill++] = FillItem{(uint64_t)fsrc, (uint64_t)gsrc, (uint64_t)off, (uint32_t)it.fb,
                                        (uint32_t)(it.bytes - it.fb)};
        }
      }
    }
    if (n_fill > f0 && !bad_slot) {
      // the kernel reads its items from the pinned workspace (written above)
      HIP_OR_FAIL(prof_pair(ctx, ctx->prof_fill, &t0, &t1));
      HIP_OR_FAIL(launch_cache_fill(d_fill + f0, n_fill - f0, fc->arena, copy_stream, t0, t1));
    }
  }
  const auto t_booked = std::chrono::steady_clock::now();
  HIP_OR_FAIL(hipMemcpyAsync(d_soff, h_soff, (size_t)(BG + 2 * ne) * sizeof(int64_t), hipMemcpyHostToDevice, copy_stream));
  HIP_OR_FAIL(hipEventRecord(ctx->ev_copy, copy_stream));
  if (copy_stream != stream) HIP_OR_FAIL(hipStreamWaitEvent(stream, ctx->ev_copy, 0));
  if (bad_slot) {
    // nothing reads the arena: the expanded pass and the merge are not launched
    return fail(SEKV_EHIP, "factor cache slot outside the arena (internal error); out was not written");
  }
  AttendArgs a5 = a;
  a5.stage_off = d_soff;
  a5.stage_fac = fc->arena;
  a5.stage_sg = reinterpret_cast<const float*>(fc->arena);
  HIP_OR_FAIL(prof_pair(ctx, ctx->prof_expand, &t0, &t1));
  HIP_OR_FAIL(launch_attend_expanded(a5, stream, t0, t1));
  HIP_OR_FAIL(hipEventRecord(fc->ev_read, stream));
  fc->read_recorded = true;
  HIP_OR_FAIL(launch_combine(a, stream));
  const auto t_end = std::chrono::steady_clock::now();
  ctx->host_wait_ms += std::chrono::duration<double, std::milli>(t_listed - t_wait).count();
  ctx->host_gather_ms += std::chrono::duration<double, std::milli>(t_booked - t_listed).count();
  ctx->host_call_ms += std::chrono::duration<double, std::milli>(t_end - t_call).count();
  ctx->host_calls += 1;
  return SEKV_OK;
}

// ---------------------------------------------------------------- online sealing
namespace {
constexpr int kSealVldsMax = 90;   // longest span whose eigenvectors stay in LDS beside its Gram matrix
size_t seal_lds_bytes(int L) {
  const size_t n2 = (size_t)((L + 1) & ~1);
  return n2 * n2 * sizeof(double) * (L <= kSealVldsMax ? 2 : 1) + (n2 / 2) * 4 * sizeof(double);
}
struct SealLayout {
  size_t desc, weights, gates, vscratch, bytes;
};
SealLayout seal_layout(const sekv_config* c) {
  const size_t B = c->batch, Hkv = c->n_kv_heads;
  SealLayout l;
  size_t off = 0;
  l.desc = off; off = align_up(off + B * sizeof(SealDesc));
  l.weights = off; off = align_up(off + B * kMaxSpan * sizeof(double));
  l.gates = off; off = align_up(off + B * Hkv * kMaxSpan * sizeof(float));
  l.vscratch = off;
  if (c->max_span > kSealVldsMax) off = align_up(off + B * Hkv * (size_t)kMaxSpan * kMaxSpan * sizeof(double));
  l.bytes = off;
  return l;
}
}  // namespace

size_t sekv_append_workspace_bytes(const sekv_config* c, const sekv_spans* s) {
  if (check_config(c) != SEKV_OK || !s) return 0;
  return seal_layout(c).bytes;
}

sekv_status sekv_append_token(sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s, const void* k_new,
                              const void* v_new, const float* surprisal, int32_t s_stride, const float* boundary_thr,
                              const float* route_proj, const float* gate, int32_t gate_stride,
                              const int32_t* rank_req, int64_t* fac_used, int64_t* sg_used, int32_t* sealed_out,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  sekv_status st = check_config(c);
  if (st != SEKV_OK) return st;
  if (c->sealed != 1) return fail(SEKV_EINVAL, "sekv_append_token needs the decode-time layout (cfg->sealed = 1)");
  if (c->basis != 0) return fail(SEKV_EINVAL, "sekv_append_token supports the joint basis (cfg->basis = 0)");
  st = check_spans(c, s, true);
  if (st != SEKV_OK) return st;
  if (!k_new || !v_new || !surprisal || !boundary_thr || !route_proj || !gate || !rank_req || !fac_used || !sg_used ||
      !ws)
    return fail(SEKV_EINVAL, "sekv_append_token: a pointer argument is NULL");
  if (!s->seg_off_host || !s->rank_host || !s->fac_off_host || !s->sg_off_host)
    return fail(SEKV_EINVAL, "sekv_append_token needs the host arrays of spans");
  const SealLayout lay = seal_layout(c);
  if (ws_bytes < lay.bytes) return fail(SEKV_ECAPACITY, "append workspace %zu bytes < %zu needed", ws_bytes, lay.bytes);
  const int B = c->batch, Hkv = c->n_kv_heads, D = c->head_dim, a = c->n_sink, lo = c->min_span, hi = c->max_span;
  const int T = c->n_ctx, Tn = T + 1;
  const int32_t cap = s->seg_cap;
  if (Tn > cap_ctx(c)) return fail(SEKV_ECAPACITY, "context %d exceeds the capacities' %d", Tn, cap_ctx(c));
  if (s_stride < Tn) return fail(SEKV_ESHAPE, "s_stride %d < n_ctx + 1 = %d", s_stride, Tn);
  // decide this step's token of every sequence and lay out the sealed spans
  std::vector<SealDesc> desc(B);
  std::vector<double> wts;
  std::vector<float> gts;
  int64_t fu = (*fac_used + 7) & ~(int64_t)7, gu = (*sg_used + 3) & ~(int64_t)3;
  size_t lds = 0;
  for (int b = 0; b < B; ++b) {
    SealDesc& d = desc[b];
    d = SealDesc{};
    const int ns = s->n_seg_host[b];
    d.n_full_old = s->n_full_host[b];
    d.n_seg_old = ns;
    if (d.n_full_old + 1 > s->full_cap)
      return fail(SEKV_ECAPACITY, "sequence %d: %d full-resolution rows exceed full_cap %d", b, d.n_full_old + 1, s->full_cap);
    if (!std::isfinite(boundary_thr[b])) return fail(SEKV_EINVAL, "boundary_thr[%d] is not finite", b);
    const int t = Tn - c->n_recent - 1 - lo;   // the token decided by this step
    if (t < a + 1) continue;
    const float* sb = surprisal + (size_t)b * s_stride;
    const int h = s->seg_off_host[(size_t)b * (cap + 1) + ns];
    const int body = t - h - 1;
    if (body < 0 || body > hi) return fail(SEKV_EINVAL, "sequence %d: span state (tail at %d, token %d) is not the sealed layout of %d tokens", b, h, t, T);
    if (!std::isfinite(sb[t])) return fail(SEKV_EINVAL, "surprisal[%d][%d] is not finite", b, t);
    if (!(body == hi || (sb[t] > boundary_thr[b] && body >= lo))) continue;
    if (ns + 1 > cap) return fail(SEKV_ECAPACITY, "sequence %d: span %d exceeds seg_cap %d", b, ns + 1, cap);
    const int L = body;
    const int req = rank_req[(size_t)b * cap + ns];
    if (req < 1) return fail(SEKV_EINVAL, "rank_req[%d][%d] = %d < 1", b, ns, req);
    const int r = std::min(std::min(req, c->rank_cap ? (L + 1) / 2 : L), 2 * D);
    if (r > gate_stride) return fail(SEKV_ESHAPE, "gate_stride %d < rank %d", gate_stride, r);
    const int rp = (r + 7) & ~7;
    d.sealed = 1;
    d.h_old = h;
    d.h_new = t;
    d.L = L;
    d.r = r;
    d.row0 = a + ns + 1;
    d.fac_stride = fac_block_elems(L, r, rp, D);
    d.sg_stride = sg_entry_elems(r);
    d.fac_base = fu;
    d.sg_base = gu;
    fu += (int64_t)Hkv * d.fac_stride;
    gu += (int64_t)Hkv * d.sg_stride;
    if (fu > s->fac_elems || gu > s->sg_elems)
      return fail(SEKV_ECAPACITY, "factor pools hold (%lld, %lld) elements, the sealed spans need (%lld, %lld)",
                  (long long)s->fac_elems, (long long)s->sg_elems, (long long)fu, (long long)gu);
    // surprisal weights of the body, as in the prefill build
    double tot = 0;
    for (int u = h + 1; u < t; ++u) tot += (double)sb[u];
    d.w_off = (int)wts.size();
    for (int u = h + 1; u < t; ++u) wts.push_back(tot > 0 ? (double)sb[u] / tot : 1.0 / L);
    d.g_off = (int)gts.size();
    for (int kv = 0; kv < Hkv; ++kv)
      for (int j = 0; j < r; ++j) gts.push_back(gate[(((size_t)b * Hkv + kv) * cap + ns) * (size_t)gate_stride + j]);
    lds = std::max(lds, seal_lds_bytes(L));
  }
  HIP_OR_FAIL(hipSetDevice(ctx->device));
  char* w8 = static_cast<char*>(ws);
  // one upload: descriptors, weights and gates at their workspace offsets
  const size_t up_bytes = gts.empty() ? (wts.empty() ? B * sizeof(SealDesc) : lay.weights + wts.size() * sizeof(double))
                                      : lay.gates + gts.size() * sizeof(float);
  std::vector<char> up(up_bytes, 0);
  std::memcpy(up.data() + lay.desc, desc.data(), B * sizeof(SealDesc));
  if (!wts.empty()) std::memcpy(up.data() + lay.weights, wts.data(), wts.size() * sizeof(double));
  if (!gts.empty()) std::memcpy(up.data() + lay.gates, gts.data(), gts.size() * sizeof(float));
  HIP_OR_FAIL(hipMemcpyAsync(w8, up.data(), up_bytes, hipMemcpyHostToDevice, stream));
  SealArgs sa{};
  sa.dtype = c->dtype; sa.B = B; sa.Hkv = Hkv; sa.D = D; sa.seg_cap = cap; sa.full_cap = s->full_cap;
  sa.vlds_max = kSealVldsMax;
  sa.desc = reinterpret_cast<const SealDesc*>(w8 + lay.desc);
  sa.weights = reinterpret_cast<const double*>(w8 + lay.weights);
  sa.gates = reinterpret_cast<const float*>(w8 + lay.gates);
  sa.vscratch = reinterpret_cast<double*>(w8 + lay.vscratch);
  sa.k_new = k_new; sa.v_new = v_new; sa.route_proj = route_proj;
  sa.full_k = const_cast<void*>(s->full_k); sa.full_v = const_cast<void*>(s->full_v);
  sa.sum_k = const_cast<void*>(s->sum_k); sa.sum_v = const_cast<void*>(s->sum_v);
  sa.rho = const_cast<void*>(s->rho); sa.key_scale = const_cast<float*>(s->key_scale);
  sa.seg_off = const_cast<int32_t*>(s->seg_off); sa.rank = const_cast<int32_t*>(s->rank);
  sa.fac_off = const_cast<int64_t*>(s->fac_off); sa.sg_off = const_cast<int64_t*>(s->sg_off);
  if (c->factors_on_host) {
    sa.fac = const_cast<void*>(device_address(s->fac));
    sa.sg = static_cast<float*>(const_cast<void*>(device_address(s->sg)));
    if (!sa.fac || !sa.sg) return fail(SEKV_EHIP, "pinned factor pools have no device address");
  } else {
    sa.fac = const_cast<void*>(s->fac);
    sa.sg = const_cast<float*>(s->sg);
  }
  HIP_OR_FAIL(launch_seal(sa, lds, stream));
  // the host mirrors follow
  int32_t* n_seg_h = const_cast<int32_t*>(s->n_seg_host);
  int32_t* n_full_h = const_cast<int32_t*>(s->n_full_host);
  int32_t* so_h = const_cast<int32_t*>(s->seg_off_host);
  int32_t* rank_h = const_cast<int32_t*>(s->rank_host);
  int64_t* fo_h = const_cast<int64_t*>(s->fac_off_host);
  int64_t* go_h = const_cast<int64_t*>(s->sg_off_host);
  for (int b = 0; b < B; ++b) {
    const SealDesc& d = desc[b];
    if (sealed_out) sealed_out[b] = d.sealed;
    n_full_h[b] = d.n_full_old + 1 - (d.sealed ? d.L : 0);
    if (!d.sealed) continue;
    const int ns = d.n_seg_old;
    n_seg_h[b] = ns + 1;
    so_h[(size_t)b * (cap + 1) + ns + 1] = d.h_new;
    rank_h[(size_t)b * cap + ns] = d.r;
    for (int kv = 0; kv < Hkv; ++kv) {
      fo_h[((size_t)b * Hkv + kv) * cap + ns] = d.fac_base + kv * d.fac_stride;
      go_h[((size_t)b * Hkv + kv) * cap + ns] = d.sg_base + kv * d.sg_stride;
    }
  }
  *fac_used = fu;
  *sg_used = gu;
  return SEKV_OK;
}

// ---------------------------------------------------------------- decode step
sekv_status sekv_decode_step(sekv_ctx* ctx, const sekv_config* c, const sekv_spans* s, const void* q,
                             const float* theta, int32_t* exp_list, uint8_t* exp_mask, int32_t* exp_count, float* out,
                             void* route_ws, size_t route_ws_bytes, void* dev_ws, size_t dev_ws_bytes,
                             hipStream_t stream) {
  sekv_status st = route_checked(ctx, c, s, q, theta, exp_list, exp_mask, exp_count);
  if (st != SEKV_OK) return st;
  if (!route_ws) return fail(SEKV_EINVAL, "sekv_decode_step: route_ws is NULL");
  if (route_ws_bytes < sekv_route_workspace_bytes(c, s))
    return fail(SEKV_ECAPACITY, "route workspace %zu bytes < %zu needed", route_ws_bytes, sekv_route_workspace_bytes(c, s));
  if (staged_fetch(ctx, c))
    return fail(SEKV_EINVAL, "sekv_decode_step: staged host-resident fetch runs through sekv_route and "
                             "sekv_mixed_attention_decode");
  DecodePlan p;
  AttendArgs a;
  st = decode_setup(ctx, c, s, q, exp_list, exp_mask, exp_count, out, dev_ws, dev_ws_bytes, kPlanDirect,
                    "sekv_decode_step", p, a);
  if (st != SEKV_OK) return st;
  HIP_OR_FAIL(hipSetDevice(ctx->device));
  // the full-resolution chunks read neither the route's outputs nor anything
  // it writes: they run on the second stream while the route runs here
  AttendArgs af = a;
  af.a4_lo = 0;
  af.a4_n = a.nch_full;
  af.n_a4_wg = c->batch * c->n_kv_heads * a.nch_full;
  HIP_OR_FAIL(hipEventRecord(ctx->ev_fork, stream));
  HIP_OR_FAIL(hipStreamWaitEvent(ctx->aux, ctx->ev_fork, 0));
  hipEvent_t e0, e1;
  hipError_t he = prof_pair(ctx, ctx->prof_overlap, &e0, &e1);
  if (he == hipSuccess) he = launch_attend_full(af, ctx->aux, e0, e1);
  const hipError_t hj = hipEventRecord(ctx->ev_join, ctx->aux);
  if (he != hipSuccess || hj != hipSuccess) {
    (void)hipStreamWaitEvent(stream, ctx->ev_join, 0);
    return fail(SEKV_EHIP, "sekv_decode_step: %s", hipGetErrorString(he != hipSuccess ? he : hj));
  }
  st = route_launch(ctx, c, s, q, theta, exp_list, exp_mask, exp_count, route_ws, true, stream);
  HIP_OR_FAIL(hipStreamWaitEvent(stream, ctx->ev_join, 0));   // joined on every path
  if (st != SEKV_OK) return st;
  AttendArgs ar = a;
  ar.a4_lo = a.nch_full;
  ar.a4_n = a.nch_a4 - a.nch_full;
  HIP_OR_FAIL(launch_attention(ctx, ar, stream));
  return SEKV_OK;
}

// ---------------------------------------------------------------- dense baseline
namespace {
// Dense decode: the full-resolution pass over all T tokens of every (b, kv),
// split into chunks of tiles_a4 32-token tiles, then the combine.
void make_dense_plan(const sekv_config* c, int32_t split_entries, AttendArgs& a, size_t& off_ml, size_t& off_o,
                     size_t& bytes) {
  const int B = c->batch, Hkv = c->n_kv_heads, D = c->head_dim, G = c->n_q_heads / Hkv, T = c->n_ctx;
  const int BG = B * Hkv;
  a = AttendArgs{};
  a.dtype = c->dtype; a.B = B; a.Hq = c->n_q_heads; a.Hkv = Hkv; a.D = D;
  a.seg_cap = 1; a.full_cap = T;
  for (int b = 0; b < B; ++b) { a.n_full[b] = T; a.n_seg[b] = 0; }
  const int ntiles = (T + 31) / 32;
  int64_t tc = ((int64_t)BG * ntiles + 1023) / 1024;
  tc = std::max<int64_t>(4, std::min<int64_t>(64, tc));
  if (split_entries > 0) tc = std::max<int64_t>(1, std::min<int64_t>(64, (split_entries + 31) / 32));
  a.tiles_a4 = (int)tc;
  a.nch_a4 = (ntiles + a.tiles_a4 - 1) / a.tiles_a4;
  a.nch_full = a.nch_a4;
  a.a4_lo = 0;
  a.a4_n = a.nch_a4;
  a.P_max = a.nch_a4;
  a.n_a4_wg = BG * a.nch_a4;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)D));
  off_ml = 0;
  off_o = align_up((size_t)BG * a.P_max * G * 2 * sizeof(float));
  bytes = align_up(off_o + (size_t)BG * a.P_max * G * D * sizeof(float));
}
}  // namespace

size_t sekv_dense_workspace_bytes(const sekv_ctx* ctx, const sekv_config* c) {
  if (check_config(c) != SEKV_OK) return 0;
  AttendArgs a;
  size_t ml, o, bytes;
  make_dense_plan(c, ctx ? ctx->split_entries : 0, a, ml, o, bytes);
  return bytes;
}

sekv_status sekv_dense_attention_decode(sekv_ctx* ctx, const sekv_config* c, const void* k, const void* v,
                                        const void* q, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  sekv_status st = check_config(c);
  if (st != SEKV_OK) return st;
  if (!k || !v || !q || !out || !ws) return fail(SEKV_EINVAL, "sekv_dense_attention_decode: a pointer argument is NULL");
  AttendArgs a;
  size_t off_ml, off_o, bytes;
  make_dense_plan(c, ctx->split_entries, a, off_ml, off_o, bytes);
  if (ws_bytes < bytes) return fail(SEKV_ECAPACITY, "dense workspace %zu bytes < %zu needed", ws_bytes, bytes);
  char* w = static_cast<char*>(ws);
  a.q = q; a.full_k = k; a.full_v = v; a.sum_k = k; a.sum_v = v;
  a.exp_count = nullptr;
  a.part_ml = reinterpret_cast<float*>(w + off_ml);
  a.part_o = reinterpret_cast<float*>(w + off_o);
  a.out = out;
  HIP_OR_FAIL(hipSetDevice(ctx->device));
  hipEvent_t e0, e1;
  HIP_OR_FAIL(prof_pair(ctx, ctx->prof_attend, &e0, &e1));
  HIP_OR_FAIL(launch_attend_full(a, stream, e0, e1));
  HIP_OR_FAIL(launch_combine(a, stream));
  return SEKV_OK;
}

sekv_status sekv_ctx_set_split(sekv_ctx* ctx, int32_t entries) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  if (entries < 0 || entries > 2048) return fail(SEKV_EINVAL, "split of %d entries outside [0, 2048]", entries);
  ctx->split_entries = entries;
  return SEKV_OK;
}

sekv_status sekv_ctx_set_fetch_mode(sekv_ctx* ctx, int32_t mode) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  if (mode != SEKV_FETCH_STAGED && mode != SEKV_FETCH_DIRECT) return fail(SEKV_EINVAL, "fetch mode %d is not SEKV_FETCH_STAGED or SEKV_FETCH_DIRECT", mode);
  ctx->fetch_mode = mode;
  return SEKV_OK;
}

sekv_status sekv_ctx_set_build_mode(sekv_ctx* ctx, int32_t mode) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  if (mode != SEKV_BUILD_DEVICE && mode != SEKV_BUILD_HOST) return fail(SEKV_EINVAL, "build mode %d is not SEKV_BUILD_DEVICE or SEKV_BUILD_HOST", mode);
  ctx->build_mode = mode;
  return SEKV_OK;
}

sekv_status sekv_ctx_inject_fault(sekv_ctx* ctx, int32_t fault) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  if (fault != SEKV_FAULT_NONE && fault != SEKV_FAULT_GATHER) return fail(SEKV_EINVAL, "fault %d is not SEKV_FAULT_NONE or SEKV_FAULT_GATHER", fault);
  ctx->fault = fault;
  return SEKV_OK;
}

sekv_status sekv_profile_read_host(sekv_ctx* ctx, double* wait_ms, double* gather_ms, double* call_ms, int64_t* calls) {
  if (!ctx || !wait_ms || !gather_ms || !call_ms || !calls) return fail(SEKV_EINVAL, "sekv_profile_read_host: NULL argument");
  *wait_ms = ctx->host_wait_ms;
  *gather_ms = ctx->host_gather_ms;
  *call_ms = ctx->host_call_ms;
  *calls = ctx->host_calls;
  ctx->host_wait_ms = ctx->host_gather_ms = ctx->host_call_ms = 0;
  ctx->host_calls = 0;
  return SEKV_OK;
}

sekv_status sekv_profile_enable(sekv_ctx* ctx, int32_t enable) {
  if (!ctx) return fail(SEKV_EINVAL, "ctx is NULL");
  ctx->profile = enable != 0;
  ctx->prof_route.used = ctx->prof_attend.used = ctx->prof_expand.used = ctx->prof_overlap.used = 0;
  return SEKV_OK;
}

sekv_status sekv_profile_read(sekv_ctx* ctx, double* route_ms, int64_t* route_n, double* full_ms, int64_t* full_n,
                              double* expand_ms, int64_t* expand_n) {
  if (!ctx || !route_ms || !route_n || !full_ms || !full_n || !expand_ms || !expand_n)
    return fail(SEKV_EINVAL, "sekv_profile_read: NULL argument");
  HIP_OR_FAIL(hipSetDevice(ctx->device));
  HIP_OR_FAIL(prof_sum(ctx->prof_route, route_ms, route_n));
  HIP_OR_FAIL(prof_sum(ctx->prof_attend, full_ms, full_n));
  HIP_OR_FAIL(prof_sum(ctx->prof_expand, expand_ms, expand_n));
  return SEKV_OK;
}

sekv_status sekv_profile_read_overlap(sekv_ctx* ctx, double* ms, int64_t* launches) {
  if (!ctx || !ms || !launches) return fail(SEKV_EINVAL, "sekv_profile_read_overlap: NULL argument");
  HIP_OR_FAIL(hipSetDevice(ctx->device));
  HIP_OR_FAIL(prof_sum(ctx->prof_overlap, ms, launches));
  return SEKV_OK;
}

sekv_status sekv_profile_read_fill(sekv_ctx* ctx, double* ms, int64_t* launches) {
  if (!ctx || !ms || !launches) return fail(SEKV_EINVAL, "sekv_profile_read_fill: NULL argument");
  HIP_OR_FAIL(hipSetDevice(ctx->device));
  HIP_OR_FAIL(prof_sum(ctx->prof_fill, ms, launches));
  return SEKV_OK;
}

}  // extern "C"
