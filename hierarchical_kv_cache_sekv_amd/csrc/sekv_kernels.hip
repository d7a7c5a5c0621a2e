// gfx950 (CDNA4) kernels of the SeKV mixed-resolution decode path.
//
// Pages (by title and section): gist.science German explainer of "SeKV:
// Resolution-Adaptive KV Cache with Hierarchical Semantic Memory for
// Long-Context LLM Inference", "Technisches Resümee" > "Methodik" part 3
// (Routing, Expansion, Mixed-Resolution Attention); the Chinese explainer,
// "技术摘要" > "方法论" part 3; the authors' abstract (low-rank SVD basis per
// span, on-demand token-level reconstruction).
//
// Kernels
//   route_decide_kernel   one lane per span, the G heads of a KV group per
//                   lane: canonical float32 score and decision bits.
//   route_compact_kernel  one workgroup per (b, kv): ascending list, head
//                   masks and count.
//   attend_full_kernel  (role A) full-resolution entries + size-corrected
//                   summaries: streams K/V rows with 16 lanes per row (8
//                   elements per lane, 16-byte loads), one online-softmax state
//                   per row subgroup.
//   attend_expanded_kernel  (role E) expanded spans, never materialising the
//                   rebuilt K/V: it applies the factors to the query
//                   (y = sigma~ .* (Vh_K q)), scores the tokens with U y, and
//                   applies the weights back through U and Vh_V, reading every
//                   factor byte once.
//   combine_kernel  log-sum-exp merge of all partials of a query head.
//   recon_*         standalone token-level K/V rebuild (tests, unfused use).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sekv_internal.h"

namespace sekv {
namespace {

using bf16raw = uint16_t;

// ---------------------------------------------------------------- loads
__device__ __forceinline__ void load8(const float* p, float (&f)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__device__ __forceinline__ void load8(const bf16raw* p, float (&f)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
  f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xffff0000u);
  f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xffff0000u);
}

__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const bf16raw* p) { return __uint_as_float(uint32_t(*p) << 16); }

// Eight consecutive elements kept in their storage form (16 B of bf16 or 32 B
// of float), so loads can be issued early and unpacked when used.
template <typename T> struct Vec8;
template <> struct Vec8<bf16raw> { uint4 v; };
template <> struct Vec8<float> { float4 a, b; };

__device__ __forceinline__ Vec8<bf16raw> ld8(const bf16raw* p) { return {*reinterpret_cast<const uint4*>(p)}; }
__device__ __forceinline__ Vec8<float> ld8(const float* p) {
  return {*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
}
__device__ __forceinline__ void st8(bf16raw* p, const Vec8<bf16raw>& x) { *reinterpret_cast<uint4*>(p) = x.v; }
__device__ __forceinline__ void st8(float* p, const Vec8<float>& x) {
  *reinterpret_cast<float4*>(p) = x.a;
  *reinterpret_cast<float4*>(p + 4) = x.b;
}
__device__ __forceinline__ void zero8(Vec8<bf16raw>& x) { x.v = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void zero8(Vec8<float>& x) { x.a = x.b = make_float4(0, 0, 0, 0); }
__device__ __forceinline__ void unpack(const Vec8<bf16raw>& x, float (&f)[8]) {
  const uint4 u = x.v;
  f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
  f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xffff0000u);
  f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xffff0000u);
}
__device__ __forceinline__ void unpack(const Vec8<float>& x, float (&f)[8]) {
  f[0] = x.a.x; f[1] = x.a.y; f[2] = x.a.z; f[3] = x.a.w;
  f[4] = x.b.x; f[5] = x.b.y; f[6] = x.b.z; f[7] = x.b.w;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
// 8-term dot product of two stored vectors (bf16: four packed dot2 steps).
__device__ __forceinline__ float dot8(const Vec8<bf16raw>& x, const Vec8<bf16raw>& y) {
  float acc = dot2bf(x.v.x, y.v.x, 0.0f);
  acc = dot2bf(x.v.y, y.v.y, acc);
  acc = dot2bf(x.v.z, y.v.z, acc);
  return dot2bf(x.v.w, y.v.w, acc);
}
__device__ __forceinline__ float dot8(const Vec8<float>& x, const Vec8<float>& y) {
  float acc = x.a.x * y.a.x;
  acc += x.a.y * y.a.y; acc += x.a.z * y.a.z; acc += x.a.w * y.a.w;
  acc += x.b.x * y.b.x; acc += x.b.y * y.b.y; acc += x.b.z * y.b.z; acc += x.b.w * y.b.w;
  return acc;
}

// ---------------------------------------------------------------- lane reductions
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of LPR (8 or 16) lanes; every lane gets the group sum.
// quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_half_mirror, row_mirror.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  if constexpr (LPR == 16) x += dpp<0x140>(x);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// LDS written and read by different lanes of the same wave.  The LDS unit
// executes one wave's ds instructions in order, so only the compiler must be
// kept from reordering; no wait on outstanding global loads is wanted here.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

constexpr float kNegInf = -__builtin_inff();

// ================================================================ route
// Canonical score: z = 0; for i in 0..D-1: z = fl32(z + fl32(q_i * rho_i)).
// Contraction into FMA is switched off for exactly these two operations, so
// each product is rounded to float32 before it is added.
//
// Two kernels: route_decide_kernel (one lane per span, many workgroups) writes
// the per-span head mask; route_compact_kernel (one workgroup per (b, kv))
// turns it into the ascending list.  The kernel boundary makes the masks
// visible across XCDs; no device-scope fence is needed inside either kernel.
template <typename T, int D, int G>
__global__ __launch_bounds__(kRouteThreads) void route_decide_kernel(const RouteArgs a) {
  __shared__ float qs[G * D];
  const int blk = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int g = b * a.Hkv + kv;
  const int ns = a.n_seg[b];
  if (blk * kRouteThreads >= ns) return;
  const T* q = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)kv * G) * D;
  for (int i = tid; i < G * D; i += kRouteThreads) qs[i] = load1(q + i);
  float th[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) th[gi] = a.theta[(size_t)b * a.Hq + kv * G + gi];
  __syncthreads();

  const int S = blk * kRouteThreads + tid;
  if (S >= ns) return;
  const T* r = static_cast<const T*>(a.rho) + ((size_t)g * a.seg_cap + S) * D;
  float z[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) z[gi] = 0.0f;
#pragma unroll 2
  for (int c = 0; c < D; c += 8) {
    float rv[8];
    load8(r + c, rv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
#pragma clang fp contract(off)
        const float prod = qs[gi * D + c + i] * rv[i];
        z[gi] = z[gi] + prod;
      }
    }
  }
  uint32_t bits = 0;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) bits |= (z[gi] > th[gi] ? 1u : 0u) << gi;
  a.dmask[(size_t)g * a.seg_cap + S] = (uint8_t)bits;
}

// One workgroup per (b, kv).  The masks are staged in LDS by tiles with
// coalesced loads; each thread then takes a contiguous run of spans, counts the
// expanded ones, one block-wide exclusive scan gives its output position.
constexpr int kCompactTile = 16384;
__global__ __launch_bounds__(kRouteThreads) void route_compact_kernel(const RouteArgs a) {
  __shared__ int wsum[kRouteThreads / 64];
  __shared__ uint8_t tile[kCompactTile];
  const int kv = blockIdx.x, b = blockIdx.y;
  const int g = b * a.Hkv + kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.n_seg[b];
  const uint8_t* dm = a.dmask + (size_t)g * a.seg_cap;
  int32_t* lst = a.exp_list + (size_t)g * a.seg_cap;
  uint8_t* msk = a.exp_mask + (size_t)g * a.seg_cap;
  int base = 0;
  for (int t0 = 0; t0 < ns; t0 += kCompactTile) {
    const int n = min(kCompactTile, ns - t0);
#pragma unroll 8
    for (int i = tid; i < n; i += kRouteThreads) tile[i] = dm[t0 + i];
    __syncthreads();
    const int per = (n + kRouteThreads - 1) / kRouteThreads;
    const int s0 = min(n, tid * per), s1 = min(n, s0 + per);
    int c = 0;
    for (int S = s0; S < s1; ++S) c += tile[S] != 0;
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int wbase = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kRouteThreads / 64; ++w) {
      const int v = wsum[w];
      if (w < wave) wbase += v;
      total += v;
    }
    int pos = base + wbase + incl - c;
    for (int S = s0; S < s1; ++S) {
      const uint8_t m = tile[S];
      if (m) {
        lst[pos] = t0 + S;
        msk[pos] = m;
        ++pos;
      }
    }
    base += total;
    __syncthreads();
  }
  if (tid == 0) a.exp_count[g] = base;
}

// ================================================================ attention
template <int D, int G>
struct AttnLds {
  // role A: per-chunk summary masks and log2 span lengths, cross-wave merge
  static constexpr int kMaskBytes = 2048;  // >= chunk_a4 (host checks)
  static constexpr int kMergeFloats = 4 * G * (D + 2);
  static constexpr int kRoleA = kMaskBytes + kMaskBytes * 4 + kMergeFloats * 4;
  // role E, per wave: y/b [kMaxSpan][G], p [kMaxSpan][G], sigma*gate [kMaxSpan],
  // and a slot for the span's U block
  static constexpr int kUBytes = 4096;
  static constexpr int kWaveBytes = (2 * kMaxSpan * G + kMaxSpan) * 4 + kUBytes;
  static constexpr int kRoleE = 4 * kWaveBytes + (kMaxGroups + 1) * 4 * 2;
  static constexpr int kBytes = kRoleA > kRoleE ? kRoleA : kRoleE;
};

template <int D, int G>
__device__ __forceinline__ void write_partial_merged(const AttendArgs& a, int g, int slot, float (&m)[G],
                                                     float (&l)[G], float (&o)[G][8], float* merge) {
  // Merge the states of the row-subgroups of this wave, then of the 4 waves.
  constexpr int LPR = D / 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = lane % LPR, sub = lane / LPR;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    float M = m[gi];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float f = (m[gi] == kNegInf) ? 0.0f : exp2f(m[gi] - M);
    float lv = l[gi] * f;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) lv += __shfl_xor(lv, off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float ov = o[gi][i] * f;
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) ov += __shfl_xor(ov, off);
      o[gi][i] = ov;
    }
    m[gi] = M;
    l[gi] = lv;
  }
  float* mm = merge;                 // [4][G]
  float* ll = merge + 4 * G;         // [4][G]
  float* oo = merge + 8 * G;         // [4][G][D]
  if (lane == 0) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) { mm[wave * G + gi] = m[gi]; ll[wave * G + gi] = l[gi]; }
  }
  if (sub == 0) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int i = 0; i < 8; ++i) oo[(wave * G + gi) * D + part * 8 + i] = o[gi][i];
  }
  __syncthreads();
  float* pml = a.part_ml + ((size_t)g * a.P_max + slot) * G * 2;
  float* po = a.part_o + ((size_t)g * a.P_max + slot) * G * D;
  for (int idx = tid; idx < G * D; idx += kAttnThreads) {
    const int gi = idx / D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mm[w * G + gi]);
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = mm[w * G + gi];
      const float f = (mw == kNegInf) ? 0.0f : exp2f(mw - M);
      acc += f * oo[(w * G + gi) * D + (idx % D)];
    }
    po[idx] = acc;
  }
  if (tid < G) {
    const int gi = tid;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mm[w * G + gi]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = mm[w * G + gi];
      L += (mw == kNegInf) ? 0.0f : exp2f(mw - M) * ll[w * G + gi];
    }
    pml[gi * 2] = M;
    pml[gi * 2 + 1] = L;
  }
}

// Role A: one workgroup = one chunk of the (b, kv) memory stream
// [full-res entries 0..n_full) ++ [span summaries 0..n_seg).
template <typename T, int D, int G>
__device__ void role_full_summary(const AttendArgs& a, int idx, char* lds) {
  constexpr int LPR = D / 8, RPW = 64 / LPR, U = 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPR, part = lane % LPR;
  const int g = idx / a.nch_a4, chunk = idx % a.nch_a4;
  const int b = g / a.Hkv, kv = g % a.Hkv;
  const int nf = a.n_full[b], ns = a.n_seg[b];
  const int ntot = nf + ns;
  const int e0 = min(ntot, chunk * a.chunk_a4), e1 = min(ntot, e0 + a.chunk_a4);
  const int S0 = max(e0, nf) - nf, S1 = max(e1, nf) - nf;

  uint8_t* smask = reinterpret_cast<uint8_t*>(lds);
  float* slog = reinterpret_cast<float*>(lds + AttnLds<D, G>::kMaskBytes);
  float* merge = reinterpret_cast<float*>(lds + AttnLds<D, G>::kMaskBytes * 5);

  const int32_t* so = a.seg_off + (size_t)b * (a.seg_cap + 1);
  for (int i = tid; i < S1 - S0; i += kAttnThreads) {
    const int S = S0 + i;
    smask[i] = 0;
    slog[i] = log2f((float)(so[S + 1] - so[S] - 1));
  }
  __syncthreads();
  if (S1 > S0) {
    const int cnt = a.exp_count[g];
    const int32_t* lst = a.exp_list + (size_t)g * a.seg_cap;
    int lo = 0, hi = cnt;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (lst[mid] < S0) lo = mid + 1; else hi = mid;
    }
    for (int j = lo + tid; j < cnt; j += kAttnThreads) {
      const int S = lst[j];
      if (S >= S1) break;
      smask[S - S0] = a.exp_mask[(size_t)g * a.seg_cap + j];
    }
  }
  __syncthreads();

  Vec8<T> qv[G];
  const T* qb = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)kv * G) * D;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) qv[gi] = ld8(qb + (size_t)gi * D + part * 8);
  const float qscale = a.qscale;
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    m[gi] = kNegInf; l[gi] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[gi][i] = 0.0f;
  }

  const int per_wave = (a.chunk_a4 + 3) / 4;
  const int wb = min(e1, e0 + wave * per_wave), we = min(e1, wb + per_wave);
  const T* fk = static_cast<const T*>(a.full_k) + (size_t)g * a.full_cap * D;
  const T* fv = static_cast<const T*>(a.full_v) + (size_t)g * a.full_cap * D;
  const T* sk = static_cast<const T*>(a.sum_k) + (size_t)g * a.seg_cap * D;
  const T* sv = static_cast<const T*>(a.sum_v) + (size_t)g * a.seg_cap * D;

  for (int base = wb; base < we; base += RPW * U) {
    Vec8<T> kr[U], vr[U];
    int ev[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = base + u * RPW + sub;
      ev[u] = e;
      const int ec = e < we ? e : wb;  // clamp: an in-range row, weight forced to 0 below
      const T* kp = ec < nf ? fk + (size_t)ec * D : sk + (size_t)(ec - nf) * D;
      const T* vp = ec < nf ? fv + (size_t)ec * D : sv + (size_t)(ec - nf) * D;
      kr[u] = ld8(kp + part * 8);
      vr[u] = ld8(vp + part * 8);
    }
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = ev[u];
      uint32_t bits = 0;
      float adj = 0.0f;
      if (e >= nf && e < we) {
        bits = smask[e - nf - S0];
        adj = slog[e - nf - S0];
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float acc = group_sum<LPR>(dot8(kr[u], qv[gi]));
        s[u][gi] = (e >= we || ((bits >> gi) & 1u)) ? kNegInf : acc * qscale + adj;
      }
    }
    float vf[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) unpack(vr[u], vf[u]);
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float mt = s[0][gi];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][gi]);
      const float mn = fmaxf(m[gi], mt);
      if (mn == kNegInf) continue;
      const float alpha = exp2f(m[gi] - mn);
      float p[U], ps = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u) { p[u] = exp2f(s[u][gi] - mn); ps += p[u]; }
      l[gi] = l[gi] * alpha + ps;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float acc = o[gi][i] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) acc += p[u] * vf[u][i];
        o[gi][i] = acc;
      }
      m[gi] = mn;
    }
  }
  write_partial_merged<D, G>(a, g, chunk, m, l, o, merge);
}

// Role E: each wave takes work items of up to kExpChunk listed spans of one
// (b, kv); a wave keeps one online-softmax state per head of the group.
// Latency hiding: the metadata of the item's spans is fetched once, one lane
// per span; the key-part rank rows, U block and sigma*gate of span i+1 are
// issued into the registers step 1 of span i has just released, so they are
// in flight while steps 2-5 of span i run; the value-part rows of span i are
// issued after its step 1.  U is staged in LDS for the two passes over it.
template <typename T>
struct SpanMeta {
  int L, r, rp;
  uint32_t bits;
  const T* U;
  const float* sg;
};

__device__ __forceinline__ int64_t readlane64(int64_t x, int i) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), i);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(x & 0xffffffff), i);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <typename T>
__device__ __forceinline__ SpanMeta<T> span_meta(int i, int mL, int mr, int mbits, int64_t mfo, int64_t mgo,
                                                 const T* fac_base, const float* sg_base) {
  SpanMeta<T> sm;
  sm.L = __builtin_amdgcn_readlane(mL, i);
  sm.r = __builtin_amdgcn_readlane(mr, i);
  sm.rp = (sm.r + 7) & ~7;
  sm.bits = (uint32_t)__builtin_amdgcn_readlane(mbits, i);
  sm.U = fac_base + readlane64(mfo, i);
  sm.sg = sg_base + readlane64(mgo, i);
  return sm;
}

// Every load here is unconditional with a clamped, in-range address (rank rows
// past r repeat row r-1, U pieces past the block repeat its last piece): a
// predicated load whose value is used inside the branch would force a wait on
// all loads in flight.  Lanes past r are masked where the values are used.
template <typename T, int D, int G>
__device__ __forceinline__ void issue_span_loads(const SpanMeta<T>& sm, int sub, int part, int lane, int ucap,
                                                 Vec8<T> (&vk)[4], Vec8<T> (&ureg)[2], float (&sgr)[4]) {
  constexpr int RPW = 64 / (D / 8);
  const int r1 = sm.r - 1;
  sgr[0] = sm.sg[min(lane, r1)];
  sgr[1] = sm.sg[sm.r + min(lane, r1)];
  sgr[2] = sm.sg[min(lane + 64, r1)];
  sgr[3] = sm.sg[sm.r + min(lane + 64, r1)];
  const int nU = min(sm.L, ucap / sm.rp) * sm.rp;  // first token tile of U
  const int lastp = nU / 8 - 1;
#pragma unroll
  for (int i = 0; i < 2; ++i) ureg[i] = ld8(sm.U + min(lane + 64 * i, lastp) * 8);
  const T* Vb = sm.U + (size_t)sm.L * sm.rp;
#pragma unroll
  for (int u = 0; u < 4; ++u) vk[u] = ld8(Vb + (size_t)min(u * RPW + sub, r1) * 2 * D + part * 8);
}

// The first token tile of U and sigma*gate of a span go to LDS once its loads
// have landed.
template <typename T>
__device__ __forceinline__ void stage_span(const SpanMeta<T>& sm, int lane, int ucap, const Vec8<T> (&ureg)[2],
                                           const float (&sgr)[4], T* ub, float* stl, float& c0, float& c1) {
  const int nU = min(sm.L, ucap / sm.rp) * sm.rp;
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int piece = lane + 64 * q2;
    if (piece * 8 < nU) st8(ub + piece * 8, ureg[q2]);
  }
  for (int piece = lane + 128; piece * 8 < nU; piece += 64) st8(ub + piece * 8, ld8(sm.U + piece * 8));
  c0 = lane < sm.r ? sgr[0] * sgr[1] : 0.0f;
  c1 = lane + 64 < sm.r ? sgr[2] * sgr[3] : 0.0f;
  if (lane < sm.r) stl[lane] = c0;
  if (lane + 64 < sm.r) stl[lane + 64] = c1;
}

template <typename T, int D, int G>
__device__ void role_expanded(const AttendArgs& a, int wg, char* lds) {
  using L_ = AttnLds<D, G>;
  constexpr int LPR = D / 8, RPW = 64 / LPR, UK = 4;
  constexpr int RREG = UK * RPW;                      // rank rows per register pass
  constexpr int UCAP = L_::kUBytes / (int)sizeof(T);  // U elements that fit the LDS slot
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPR, part = lane % LPR;
  const int BG = a.B * a.Hkv;
  int* pre = reinterpret_cast<int*>(lds + 4 * L_::kWaveBytes);  // [BG+1] chunk prefix
  {
    int* tmp = pre + (kMaxGroups + 1);
    for (int i = tid; i < BG; i += kAttnThreads) tmp[i] = (a.exp_count[i] + kExpChunk - 1) / kExpChunk;
    __syncthreads();
    if (wave == 0) {
      int run = 0;
      for (int c0 = 0; c0 < BG; c0 += 64) {
        const int i = c0 + lane;
        const int v = i < BG ? tmp[i] : 0;
        int incl = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int t = __shfl_up(incl, off);
          if (lane >= off) incl += t;
        }
        if (i < BG) pre[i] = run + incl - v;
        run += __shfl(incl, 63);
      }
      if (lane == 0) pre[BG] = run;
    }
    __syncthreads();
  }
  const int total = pre[BG];
  char* wl = lds + wave * L_::kWaveBytes;
  float* yb = reinterpret_cast<float*>(wl);   // [kMaxSpan][G]: y, later b
  float* pb = yb + kMaxSpan * G;              // [kMaxSpan][G]: softmax weights
  float* stl = pb + kMaxSpan * G;             // [kMaxSpan]: sigma * gate
  T* ub = reinterpret_cast<T*>(stl + kMaxSpan);
  const int nwaves = a.n_a5_wg * 4;
  const bool staged = a.stage_off != nullptr;
  const float qscale = a.qscale;

  for (int c = wg * 4 + wave; c < total; c += nwaves) {
    int lo = 0, hi = BG;  // g with pre[g] <= c < pre[g+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= c) lo = mid; else hi = mid;
    }
    const int g = lo, lc = c - pre[g];
    const int b = g / a.Hkv, kv = g % a.Hkv;
    const int cnt = a.exp_count[g];
    const int j0 = lc * kExpChunk, n = min(cnt, j0 + kExpChunk) - j0;

    // metadata of the item's spans, lane i holds span j0 + i
    const int32_t* so = a.seg_off + (size_t)b * (a.seg_cap + 1);
    const int jl = j0 + min(lane, n - 1);
    const int mS = a.exp_list[(size_t)g * a.seg_cap + jl];
    const int mbits = a.exp_mask[(size_t)g * a.seg_cap + jl];
    int64_t mfo, mgo;
    if (staged) {
      const int64_t* st = a.stage_off + ((size_t)g * a.seg_cap + jl) * 2;
      mfo = st[0];
      mgo = st[1];
    } else {
      mfo = a.fac_off[(size_t)g * a.seg_cap + mS];
      mgo = a.sg_off[(size_t)g * a.seg_cap + mS];
    }
    const int mL = so[mS + 1] - so[mS] - 1;
    const int mr = a.rank[(size_t)b * a.seg_cap + mS];
    const T* fac_base = staged ? static_cast<const T*>(a.stage_fac) : static_cast<const T*>(a.fac);
    const float* sg_base = staged ? a.stage_sg : a.sg;
    Vec8<T> qv[G];
    const T* qb = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)kv * G) * D;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) qv[gi] = ld8(qb + (size_t)gi * D + part * 8);
    float m[G], l[G], o[G][8];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      m[gi] = kNegInf; l[gi] = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[gi][i] = 0.0f;
    }

    Vec8<T> vk[UK], ureg[2];
    float sgr[4];
    SpanMeta<T> cur = span_meta<T>(0, mL, mr, mbits, mfo, mgo, fac_base, sg_base);
    issue_span_loads<T, D, G>(cur, sub, part, lane, UCAP, vk, ureg, sgr);
    // span i+1 is staged at the end of span i, so no load is pending across
    // the loop back-edge.
    float cst0, cst1;
    stage_span<T>(cur, lane, UCAP, ureg, sgr, ub, stl, cst0, cst1);
    wave_lds_sync();
    for (int i = 0; i < n; ++i) {
      const int L = cur.L, r = cur.r, rp = cur.rp;
      const uint32_t bits = cur.bits;
      const T* Ub = cur.U;
      const T* Vb = Ub + (size_t)L * rp;
      const int TT = min(L, UCAP / rp);  // tokens per U tile held in LDS
      // ---- step 1: y[k][gi] = sigma_k gate_k (Vh_K[k] . q_gi) * log2(e)/sqrt(d)
#pragma unroll
      for (int u = 0; u < UK; ++u) {
        if (u * RPW < r) {
          const int k = u * RPW + sub;
#pragma unroll
          for (int gi = 0; gi < G; ++gi) {
            const float acc = group_sum<LPR>(dot8(vk[u], qv[gi]));
            if (part == 0 && k < r) yb[k * G + gi] = acc * qscale * stl[k];
          }
        }
      }
      for (int k0 = RREG; k0 < r; k0 += RREG) {  // ranks beyond the register pass
#pragma unroll
        for (int u = 0; u < UK; ++u) vk[u] = ld8(Vb + (size_t)min(k0 + u * RPW + sub, r - 1) * 2 * D + part * 8);
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          if (k0 + u * RPW < r) {
            const int k = k0 + u * RPW + sub;
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
              const float acc = group_sum<LPR>(dot8(vk[u], qv[gi]));
              if (part == 0 && k < r) yb[k * G + gi] = acc * qscale * stl[k];
            }
          }
        }
      }
      // value-part rank rows of this span, then the next span's key rows, U, sigma*gate
      Vec8<T> vv[UK];
#pragma unroll
      for (int u = 0; u < UK; ++u) vv[u] = ld8(Vb + (size_t)min(u * RPW + sub, r - 1) * 2 * D + D + part * 8);
      // (unconditional: the last span re-issues its own loads, which keeps the
      // load state the same on every path)
      const SpanMeta<T> nxt = span_meta<T>(min(i + 1, n - 1), mL, mr, mbits, mfo, mgo, fac_base, sg_base);
      issue_span_loads<T, D, G>(nxt, sub, part, lane, UCAP, vk, ureg, sgr);
      wave_lds_sync();
      // ---- steps 2-4 over token tiles of U (one tile unless L*rp exceeds the slot)
      float am[2][G];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int gi = 0; gi < G; ++gi) am[kk][gi] = 0.0f;
      for (int t0 = 0; t0 < L; t0 += TT) {
        const int tn = min(TT, L - t0);
        if (t0 > 0) {
          for (int piece = lane; piece * 8 < tn * rp; piece += 64)
            st8(ub + piece * 8, ld8(Ub + (size_t)t0 * rp + piece * 8));
          wave_lds_sync();
        }
        // step 2: token scores s_t = U[t] . y
        float s[2][G];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = lane + 64 * tt;
#pragma unroll
          for (int gi = 0; gi < G; ++gi) s[tt][gi] = kNegInf;
          if (t < tn) {
            float acc[G];
#pragma unroll
            for (int gi = 0; gi < G; ++gi) acc[gi] = 0.0f;
            for (int k8 = 0; k8 < rp; k8 += 8) {
              float u8[8];
              unpack(ld8(ub + t * rp + k8), u8);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                if (k8 + e < r) {
#pragma unroll
                  for (int gi = 0; gi < G; ++gi) acc[gi] += u8[e] * yb[(k8 + e) * G + gi];
                }
              }
            }
#pragma unroll
            for (int gi = 0; gi < G; ++gi) s[tt][gi] = ((bits >> gi) & 1u) ? acc[gi] : kNegInf;
          }
        }
        // step 3: online softmax; the span's partial U^T p is rescaled with o
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          const float ms = wave_max(fmaxf(s[0][gi], s[1][gi]));
          const float mn = fmaxf(m[gi], ms);
          float p0 = 0.0f, p1 = 0.0f;
          if (mn != kNegInf) {
            const float alpha = exp2f(m[gi] - mn);
            p0 = exp2f(s[0][gi] - mn);
            p1 = exp2f(s[1][gi] - mn);
            l[gi] = l[gi] * alpha + wave_sum(p0 + p1);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[gi][e] *= alpha;
            am[0][gi] *= alpha;
            am[1][gi] *= alpha;
            m[gi] = mn;
          }
          if (lane < tn) pb[lane * G + gi] = p0;
          if (lane + 64 < tn) pb[(lane + 64) * G + gi] = p1;
        }
        wave_lds_sync();
        // step 4: a[k] += sum_t U[t][k] p_t
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int k = lane + 64 * kk;
          if (k < r) {
#pragma unroll 4
            for (int t = 0; t < tn; ++t) {
              const float u = load1(ub + t * rp + k);
#pragma unroll
              for (int gi = 0; gi < G; ++gi) am[kk][gi] += u * pb[t * G + gi];
            }
          }
        }
        wave_lds_sync();
      }
      // b[k] = sigma_k gate_k a[k]  (into yb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k = lane + 64 * kk;
        if (k < r) {
          const float st = kk == 0 ? cst0 : cst1;
#pragma unroll
          for (int gi = 0; gi < G; ++gi) yb[k * G + gi] = am[kk][gi] * st;
        }
      }
      wave_lds_sync();
      // ---- step 5: o += Vh_V^T b
#pragma unroll
      for (int u = 0; u < UK; ++u) {
        if (u * RPW < r) {
          const int k = u * RPW + sub;
          if (k < r) {
            float v8[8];
            unpack(vv[u], v8);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
              const float bk = yb[k * G + gi];
#pragma unroll
              for (int e = 0; e < 8; ++e) o[gi][e] += bk * v8[e];
            }
          }
        }
      }
      for (int k0 = RREG; k0 < r; k0 += RREG) {
#pragma unroll
        for (int u = 0; u < UK; ++u) vv[u] = ld8(Vb + (size_t)min(k0 + u * RPW + sub, r - 1) * 2 * D + D + part * 8);
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          const int k = k0 + u * RPW + sub;
          if (k0 + u * RPW < r && k < r) {
            float v8[8];
            unpack(vv[u], v8);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
              const float bk = yb[k * G + gi];
#pragma unroll
              for (int e = 0; e < 8; ++e) o[gi][e] += bk * v8[e];
            }
          }
        }
      }
      wave_lds_sync();
      cur = nxt;
      stage_span<T>(cur, lane, UCAP, ureg, sgr, ub, stl, cst0, cst1);
      wave_lds_sync();
    }
    // merge the row-subgroups of this wave (states share m, l) and write the partial
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float ov = o[gi][e];
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) ov += __shfl_xor(ov, off);
        o[gi][e] = ov;
      }
    const int slot = a.nch_a4 + lc;
    float* pml = a.part_ml + ((size_t)g * a.P_max + slot) * G * 2;
    float* po = a.part_o + ((size_t)g * a.P_max + slot) * G * D;
    if (sub == 0) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int e = 0; e < 8; ++e) po[gi * D + part * 8 + e] = o[gi][e];
    }
    if (lane < G) {
      float mv = m[0], lv = l[0];
#pragma unroll
      for (int gi = 1; gi < G; ++gi) if (lane == gi) { mv = m[gi]; lv = l[gi]; }
      pml[lane * 2] = mv;
      pml[lane * 2 + 1] = lv;
    }
  }
}

// Full-resolution + summary pass (role A) and expanded-span pass (role E) are
// separate kernels so each gets its own register budget; the host runs them
// concurrently on two streams.
template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnThreads) void attend_full_kernel(const AttendArgs a) {
  extern __shared__ __align__(16) char lds[];
  role_full_summary<T, D, G>(a, blockIdx.x, lds);
}
template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnThreads) void attend_expanded_kernel(const AttendArgs a) {
  extern __shared__ __align__(16) char lds[];
  role_expanded<T, D, G>(a, blockIdx.x, lds);
}

// ================================================================ combine
// One workgroup per (b, h).  Pass 1: the maximum over partials (strided over
// threads).  Pass 2: kCombineSplit thread groups each accumulate a strided
// share of the partials for all D outputs; the groups are summed in LDS.
constexpr int kCombineThreads = 256;
template <int D, int G>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const AttendArgs a) {
  constexpr int SPLIT = kCombineThreads / D;   // 2 (D=128) or 4 (D=64)
  __shared__ float red[kCombineThreads];
  __shared__ float acc_s[SPLIT][D];
  __shared__ float l_s[SPLIT];
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int g = b * a.Hkv + h / G, gi = h % G;
  const int tid = threadIdx.x;
  const int np = a.nch_a4 + (a.exp_count[g] + kExpChunk - 1) / kExpChunk;
  const float* ml = a.part_ml + (size_t)g * a.P_max * G * 2;
  const float* po = a.part_o + (size_t)g * a.P_max * G * D;
  float M = kNegInf;
  for (int p = tid; p < np; p += kCombineThreads) M = fmaxf(M, ml[(p * G + gi) * 2]);
  red[tid] = M;
  __syncthreads();
  for (int off = kCombineThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
    __syncthreads();
  }
  M = red[0];
  const int j = tid % D, part = tid / D;
  float acc = 0.0f, L = 0.0f;
#pragma unroll 4
  for (int p = part; p < np; p += SPLIT) {
    const float mp = ml[(p * G + gi) * 2];
    const float lp = ml[(p * G + gi) * 2 + 1];
    const float ov = po[((size_t)p * G + gi) * D + j];
    const float f = (mp == kNegInf) ? 0.0f : exp2f(mp - M);
    L += f * lp;
    acc += f * ov;
  }
  acc_s[part][j] = acc;
  if (j == 0) l_s[part] = L;
  __syncthreads();
  if (tid < D) {
    float o = 0.0f, Lt = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < SPLIT; ++s2) { o += acc_s[s2][tid]; Lt += l_s[s2]; }
    a.out[(size_t)bh * D + tid] = o / Lt;
  }
}

// ================================================================ reconstruct
__global__ __launch_bounds__(64) void recon_scan_kernel(const ReconArgs a) {
  const int g = blockIdx.x, b = g / a.Hkv;
  const int lane = threadIdx.x;
  const int cnt = a.exp_count[g];
  const int32_t* lst = a.exp_list + (size_t)g * a.seg_cap;
  const int32_t* so = a.seg_off + (size_t)b * (a.seg_cap + 1);
  int32_t* to = a.tok_off + (size_t)g * (a.seg_cap + 1);
  int run = 0;
  for (int j0 = 0; j0 < cnt; j0 += 64) {
    const int j = j0 + lane;
    int v = 0;
    if (j < cnt) {
      const int S = lst[j];
      v = so[S + 1] - so[S] - 1;
    }
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    if (j < cnt) to[j] = run + incl - v;
    run += __shfl(incl, 63);
  }
  if (lane == 0) to[cnt] = run;
}

template <typename T, int D>
__global__ __launch_bounds__(64) void recon_kernel(const ReconArgs a) {
  const int kv = blockIdx.y, b = blockIdx.z, g = b * a.Hkv + kv;
  const int lane = threadIdx.x;
  const int cnt = a.exp_count[g];
  const int32_t* so = a.seg_off + (size_t)b * (a.seg_cap + 1);
  constexpr int CPL = 2 * D / 64;  // output columns per lane
  for (int j = blockIdx.x; j < cnt; j += gridDim.x) {
    const int S = a.exp_list[(size_t)g * a.seg_cap + j];
    const int L = so[S + 1] - so[S] - 1;
    const int r = a.rank[(size_t)b * a.seg_cap + S];
    const int rp = (r + 7) & ~7;
    const T* Ub = static_cast<const T*>(a.fac) + a.fac_off[(size_t)g * a.seg_cap + S];
    const T* Vb = Ub + (size_t)L * rp;
    const float* sgp = a.sg + a.sg_off[(size_t)g * a.seg_cap + S];
    const int row0 = a.tok_off[(size_t)g * (a.seg_cap + 1) + j];
    for (int t = 0; t < L; ++t) {
      float acc[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
      for (int k = 0; k < r; ++k) {
        const float w = load1(Ub + (size_t)t * rp + k) * (sgp[k] * sgp[r + k]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] += w * load1(Vb + (size_t)k * 2 * D + lane + 64 * c);
      }
      const size_t orow = ((size_t)g * a.T + row0 + t) * D;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int col = lane + 64 * c;
        if (col < D) a.k_out[orow + col] = acc[c];
        else a.v_out[orow + col - D] = acc[c];
      }
    }
  }
}

// ---------------------------------------------------------------- dispatch
#define SEKV_DISPATCH(DT, DIM, GRP, BODY)                                   \
  do {                                                                      \
    if ((DT) == 0) {                                                        \
      using TT = float;                                                     \
      SEKV_DISPATCH_D(DIM, GRP, BODY);                                      \
    } else {                                                                \
      using TT = bf16raw;                                                   \
      SEKV_DISPATCH_D(DIM, GRP, BODY);                                      \
    }                                                                       \
  } while (0)
#define SEKV_DISPATCH_D(DIM, GRP, BODY)                                     \
  do {                                                                      \
    if ((DIM) == 64) {                                                      \
      constexpr int DD = 64;                                                \
      SEKV_DISPATCH_G(GRP, BODY);                                           \
    } else {                                                                \
      constexpr int DD = 128;                                               \
      SEKV_DISPATCH_G(GRP, BODY);                                           \
    }                                                                       \
  } while (0)
#define SEKV_DISPATCH_G(GRP, BODY)                                          \
  do {                                                                      \
    switch (GRP) {                                                          \
      case 1: { constexpr int GG = 1; BODY; } break;                        \
      case 2: { constexpr int GG = 2; BODY; } break;                        \
      case 4: { constexpr int GG = 4; BODY; } break;                        \
      default: { constexpr int GG = 8; BODY; } break;                       \
    }                                                                       \
  } while (0)

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  dim3 grid(a.nblk, a.Hkv, a.B);
  SEKV_DISPATCH(a.dtype, a.D, G, (route_decide_kernel<TT, DD, GG><<<grid, kRouteThreads, 0, s>>>(a)));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  route_compact_kernel<<<dim3(a.Hkv, a.B), kRouteThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_attend_full(const AttendArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (a.n_a4_wg == 0) return hipSuccess;
  SEKV_DISPATCH(a.dtype, a.D, G,
                (attend_full_kernel<TT, DD, GG><<<a.n_a4_wg, kAttnThreads, AttnLds<DD, GG>::kRoleA, s>>>(a)));
  return hipGetLastError();
}

hipError_t launch_attend_expanded(const AttendArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (a.n_a5_wg == 0) return hipSuccess;
  SEKV_DISPATCH(a.dtype, a.D, G,
                (attend_expanded_kernel<TT, DD, GG><<<a.n_a5_wg, kAttnThreads, AttnLds<DD, GG>::kRoleE, s>>>(a)));
  return hipGetLastError();
}

hipError_t launch_combine(const AttendArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  SEKV_DISPATCH_D(a.D, G, (combine_kernel<DD, GG><<<a.B * a.Hq, kCombineThreads, 0, s>>>(a)));
  return hipGetLastError();
}

hipError_t launch_reconstruct(const ReconArgs& a, hipStream_t s) {
  recon_scan_kernel<<<a.B * a.Hkv, 64, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(256, a.Hkv, a.B);
  if (a.dtype == 0) {
    if (a.D == 64) recon_kernel<float, 64><<<grid, 64, 0, s>>>(a);
    else recon_kernel<float, 128><<<grid, 64, 0, s>>>(a);
  } else {
    if (a.D == 64) recon_kernel<bf16raw, 64><<<grid, 64, 0, s>>>(a);
    else recon_kernel<bf16raw, 128><<<grid, 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace sekv
