// Host-only exercise of libsekv's runtime for the address and undefined-behaviour
// sanitizers: capacities, span planning over random configurations (all
// reading variants), argument errors, workspace sizing, and the device factor
// cache's bookkeeping (a cache without a device arena) over random route
// lists.  No GPU call is made.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "sekv.h"

static int failures = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      std::fprintf(stderr, "FAILED %s (line %d)\n", #c, __LINE__);  \
      ++failures;                                                   \
    }                                                               \
  } while (0)

int main() {
  std::mt19937 rng(7);
  int planned = 0;
  for (int trial = 0; trial < 400; ++trial) {
    sekv_config c{};
    c.batch = 1 + (int)(rng() % 4);
    c.n_ctx = 2 + (int)(rng() % 3000);
    c.n_kv_heads = 1 + (int)(rng() % 3);
    const int G = 1 << (rng() % 4);
    c.n_q_heads = c.n_kv_heads * G;
    c.head_dim = (rng() % 2) ? 64 : 128;
    c.n_sink = (int)(rng() % 6);
    c.n_recent = (int)(rng() % 40);
    c.min_span = 1 + (int)(rng() % 9);
    c.max_span = c.min_span + (int)(rng() % 120);
    if (c.max_span > 128) c.max_span = 128;
    c.dtype = (int)(rng() % 2);
    c.rank_cap = (int)(rng() % 2);
    c.basis = (int)(rng() % 2);
    c.route_keys = (int)(rng() % 2);
    int32_t seg_cap = 0, full_cap = 0;
    const sekv_status st = sekv_capacities(&c, &seg_cap, &full_cap);
    if (c.n_sink + c.n_recent < 1 || c.n_sink + c.n_recent > c.n_ctx) {
      EXPECT(st != SEKV_OK);
      continue;
    }
    EXPECT(st == SEKV_OK);
    const int B = c.batch, T = c.n_ctx, Hkv = c.n_kv_heads;
    std::vector<float> s((size_t)B * T), thr(B);
    std::lognormal_distribution<float> ln(0.f, 1.f);
    for (auto& x : s) x = ln(rng);
    for (int b = 0; b < B; ++b) thr[b] = 1.5f;
    std::vector<int32_t> req((size_t)B * seg_cap), n_seg(B), n_full(B), seg_off((size_t)B * (seg_cap + 1)),
        rank((size_t)B * seg_cap);
    for (auto& r : req) r = 1 + (int)(rng() % 200);
    std::vector<int64_t> fac_off((size_t)B * Hkv * seg_cap), sg_off((size_t)B * Hkv * seg_cap);
    int64_t fe = 0, ge = 0;
    EXPECT(sekv_plan_spans(&c, s.data(), thr.data(), req.data(), n_seg.data(), n_full.data(), seg_off.data(),
                           rank.data(), fac_off.data(), sg_off.data(), &fe, &ge) == SEKV_OK);
    for (int b = 0; b < B; ++b) {
      EXPECT(n_seg[b] >= 0 && n_seg[b] <= seg_cap);
      EXPECT(n_full[b] >= 1 && n_full[b] <= full_cap);
      for (int i = 0; i < n_seg[b]; ++i) {
        const int L = seg_off[(size_t)b * (seg_cap + 1) + i + 1] - seg_off[(size_t)b * (seg_cap + 1) + i] - 1;
        const int r = rank[(size_t)b * seg_cap + i];
        EXPECT(L >= 1 && L <= c.max_span);
        EXPECT(r >= 1 && r <= L && (!c.rank_cap || r <= (L + 1) / 2) && r <= (c.basis ? c.head_dim : 2 * c.head_dim));
      }
    }
    // workspace sizes of a span cache with these capacities (no device memory is touched)
    sekv_spans sp{};
    sp.seg_cap = seg_cap;
    sp.full_cap = full_cap;
    sp.n_seg_host = n_seg.data();
    sp.n_full_host = n_full.data();
    sp.rank_host = rank.data();
    EXPECT(sekv_route_workspace_bytes(&c, &sp) > 0);
    EXPECT(sekv_decode_workspace_bytes(nullptr, &c, &sp) > 0);
    EXPECT(sekv_dense_workspace_bytes(nullptr, &c) > 0);
    EXPECT(sekv_cached_decode_workspace_bytes(nullptr, &c, &sp) > 0);
    // factor cache bookkeeping over random lists (a tiny cache: evictions and bypasses)
    sp.seg_off_host = seg_off.data();
    sp.fac_off_host = fac_off.data();
    sp.sg_off_host = sg_off.data();
    sp.fac = reinterpret_cast<const void*>(uintptr_t(1) << 40);
    sp.fac_elems = fe;
    sp.sg_elems = ge;
    sekv_factor_cache* fc = nullptr;
    const int parts = 1 + (int)(rng() % 3);
    EXPECT(sekv_factor_cache_create(nullptr, (size_t(2) << 20) * parts * (1 + rng() % 2), parts, &fc) == SEKV_OK);
    std::vector<int32_t> lst((size_t)B * Hkv * seg_cap), cnt((size_t)B * Hkv), stt(lst.size());
    std::vector<int64_t> off(lst.size());
    for (int call = 0; call < 6 && fc; ++call) {
      for (int g = 0; g < B * Hkv; ++g) {
        const int ns = n_seg[g / Hkv];
        int n = 0;
        for (int i = 0; i < ns; ++i)
          if (rng() % 3 == 0) lst[(size_t)g * seg_cap + n++] = i;
        cnt[g] = n;
      }
      EXPECT(sekv_factor_cache_lookup(fc, call % 3, &c, &sp, lst.data(), cnt.data(), stt.data(), off.data()) ==
             SEKV_OK);
      for (int g = 0; g < B * Hkv; ++g)
        for (int j = 0; j < cnt[g]; ++j) {
          const size_t k = (size_t)g * seg_cap + j;
          EXPECT(stt[k] >= 0 && stt[k] <= 2 && (stt[k] == 2) == (off[k] < 0));
        }
    }
    sekv_cache_stats cs{};
    if (fc) {
      EXPECT(sekv_factor_cache_stats(fc, &cs, 1) == SEKV_OK);
      EXPECT(cs.lookups == cs.hits + cs.fills + cs.bypasses);
      EXPECT(sekv_factor_cache_invalidate(fc, 1) == SEKV_OK);
      EXPECT(sekv_factor_cache_invalidate(fc, -1) == SEKV_OK);
      sekv_factor_cache_destroy(fc);
    }
    ++planned;
  }
  // argument errors
  sekv_config bad{};
  int32_t a = 0, b = 0;
  EXPECT(sekv_capacities(nullptr, &a, &b) == SEKV_EINVAL);
  EXPECT(sekv_capacities(&bad, &a, &b) != SEKV_OK);
  EXPECT(sekv_last_error()[0] != '\0');
  EXPECT(sekv_route(nullptr, &bad, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
         SEKV_EINVAL);
  EXPECT(sekv_ctx_set_split(nullptr, 32) == SEKV_EINVAL);
  std::printf("host sanitize driver: %d plans, %d failures\n", planned, failures);
  return failures == 0 ? 0 : 1;
}
