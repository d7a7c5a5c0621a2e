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
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One MFMA accumulation over 32 contraction positions, 8 per lane class
// (class = lane / 16): C[i][j] += sum over classes c and t < 8 of
// A_lane(i, c)[t] * B_lane(j, c)[t], where lane 16c + i supplies row i of A and
// lane 16c + j column j of B; lane 16c + j holds C[4c + v][j], v = 0..3.
// bf16: one v_mfma_f32_16x16x32_bf16; float: eight v_mfma_f32_16x16x4f32.
__device__ __forceinline__ f32x4_t mma8(const Vec8<bf16raw>& x, const Vec8<bf16raw>& y, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.v), __builtin_bit_cast(bf16x8_t, y.v),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma8(const Vec8<float>& x, const Vec8<float>& y, f32x4_t c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.a.x, y.a.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.a.y, y.a.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.a.z, y.a.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.a.w, y.a.w, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.b.x, y.b.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.b.y, y.b.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.b.z, y.b.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.b.w, y.b.w, c, 0, 0, 0);
  return c;
}
// Eight floats as an MFMA operand of the storage type (bf16: round to nearest even).
__device__ __forceinline__ void pack8(const float (&p)[8], Vec8<bf16raw>& out) {
  bf16x8_t v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)p[i];
  out.v = __builtin_bit_cast(uint4, v);
}
__device__ __forceinline__ void pack8(const float (&p)[8], Vec8<float>& out) {
  out.a = make_float4(p[0], p[1], p[2], p[3]);
  out.b = make_float4(p[4], p[5], p[6], p[7]);
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
  static constexpr int kMaskBytes = 2048;  // >= 32 * tiles_a4 (host checks)
  static constexpr int kMergeFloats = 4 * G * (D + 2);
  static constexpr int kRoleA = kMaskBytes + kMaskBytes * 4 + kMergeFloats * 4;
  // role E, per wave: one 32-token x 32-rank tile of U as float, row-major and
  // transposed (row stride 36), y [16 heads][kMaxSpan], sigma*gate [kMaxSpan]
  static constexpr int kTileStride = 36;
  static constexpr int kWaveBytes = (2 * 32 * kTileStride + G * kMaxSpan + kMaxSpan) * 4;
  static constexpr int kRoleE = 4 * kWaveBytes + (kMaxGroups + 1) * 4 * 2;
  static constexpr int kBytes = kRoleA > kRoleE ? kRoleA : kRoleE;
};

// Role A: one workgroup = a chunk of tiles_a4 32-entry tiles of the (b, kv)
// memory stream [full-resolution tiles ++ summary tiles]; wave w takes tiles
// w, w+4, ... of the chunk.  Per tile, q.K and P.V run on the matrix cores:
//   scores  S^T[entry][head] = K rows (A operand) x q (B operand), two MFMA
//           halves; lane 16c + h ends up holding the 8 scores of head h for
//           entries 8c..8c+7 of the tile;
//   output  O^T[j][head] += V^T (A operand, from the transposed value tile)
//           x P (B operand = exactly those 8 softmax weights of the lane).
// Each lane therefore keeps the online-softmax state of head (lane % 16) and
// rescales only its own accumulators.
template <typename T, int D, int G>
__device__ void role_full_summary(const AttendArgs& a, int idx, char* lds) {
  constexpr int NC = D / 32, NJ = D / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, cls = lane >> 4;
  const int g = idx / a.nch_a4, chunk = idx % a.nch_a4;
  const int b = g / a.Hkv, kv = g % a.Hkv;
  const int nf = a.n_full[b], ns = a.n_seg[b];
  const int nft = (nf + 31) / 32, nst = (ns + 31) / 32;
  const int t0 = min(nft + nst, chunk * a.tiles_a4), t1 = min(nft + nst, t0 + a.tiles_a4);
  const int S0 = (max(t0, nft) - nft) * 32, S1 = min(ns, (max(t1, nft) - nft) * 32);

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

  // q as the B operand: column = head (zero for columns >= G)
  Vec8<T> qB[NC];
  const T* qrow = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)kv * G + min(col, G - 1)) * D;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qB[c] = ld8(qrow + 32 * c + 8 * cls);
    if (col >= G) zero8(qB[c]);
  }
  const float qscale = a.qscale;
  float m = kNegInf, lsum = 0.0f;
  f32x4_t acc[NJ];
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt) acc[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int ftiles = (a.full_cap + 31) / 32, stiles = (a.seg_cap + 31) / 32;
  const T* fk = static_cast<const T*>(a.full_k) + (size_t)g * a.full_cap * D;
  const T* fvt = static_cast<const T*>(a.full_v) + (size_t)g * ftiles * 32 * D;
  const T* sk = static_cast<const T*>(a.sum_k) + (size_t)g * a.seg_cap * D;
  const T* svt = static_cast<const T*>(a.sum_v) + (size_t)g * stiles * 32 * D;

  for (int t = t0 + wave; t < t1; t += 4) {
    const bool summ = t >= nft;
    const int tt = summ ? t - nft : t;
    const int base = tt * 32;
    const int npart = summ ? ns : nf;
    const T* krows = summ ? sk : fk;
    const T* vt = (summ ? svt : fvt) + (size_t)tt * 32 * D;
    // K operands: MFMA half h, row (col) = entry 8*(col/4) + 4h + col%4 of the tile
    Vec8<T> kop[2][NC];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = min(base + 8 * (col >> 2) + 4 * h + (col & 3), npart - 1);
#pragma unroll
      for (int c = 0; c < NC; ++c) kop[h][c] = ld8(krows + (size_t)e * D + 32 * c + 8 * cls);
    }
    Vec8<T> vop[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) vop[jt] = ld8(vt + (16 * jt + col) * 32 + 8 * cls);
    f32x4_t sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sc[h] = mma8(kop[h][c], qB[c], sc[h]);
    }
    // this lane: head col, tile entries 8*cls + 4h + v
    float sv[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int e = base + 8 * cls + 4 * h + v;
        float val = sc[h][v] * qscale;
        if (e >= npart) {
          val = kNegInf;
        } else if (summ) {
          const uint32_t bits = smask[e - S0];
          val = ((bits >> col) & 1u) ? kNegInf : val + slog[e - S0];
        }
        sv[4 * h + v] = val;
      }
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    float p[8];
    if (mn != kNegInf) {
      const float alpha = exp2f(m - mn);
      float ps = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { p[i] = exp2f(sv[i] - mn); ps += p[i]; }
      lsum = lsum * alpha + ps;
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) acc[jt] *= alpha;
      m = mn;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = 0.0f;
    }
    Vec8<T> pB;
    pack8(p, pB);
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) acc[jt] = mma8(vop[jt], pB, acc[jt]);
  }

  // this wave's state of head col: lsum summed over the four lane classes
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  float* mm = merge;                 // [4][G]
  float* ll = merge + 4 * G;         // [4][G]
  float* oo = merge + 8 * G;         // [4][G][D]
  if (cls == 0 && col < G) {
    mm[wave * G + col] = m;
    ll[wave * G + col] = lsum;
  }
  if (col < G) {
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) oo[(wave * G + col) * D + 16 * jt + 4 * cls + v] = acc[jt][v];
  }
  __syncthreads();
  float* pml = a.part_ml + ((size_t)g * a.P_max + chunk) * G * 2;
  float* po = a.part_o + ((size_t)g * a.P_max + chunk) * G * D;
  for (int i = tid; i < G * D; i += kAttnThreads) {
    const int gi = i / D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mm[w * G + gi]);
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = mm[w * G + gi];
      o += (mw == kNegInf) ? 0.0f : exp2f(mw - M) * oo[(w * G + gi) * D + (i % D)];
    }
    po[i] = o;
  }
  if (tid < G) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mm[w * G + tid]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = mm[w * G + tid];
      L += (mw == kNegInf) ? 0.0f : exp2f(mw - M) * ll[w * G + tid];
    }
    pml[tid * 2] = M;
    pml[tid * 2 + 1] = L;
  }
}

// Role E: each wave takes work items of up to kExpChunk listed spans of one
// (b, kv) and keeps, like role A, the online-softmax state of head (lane % 16).
// Per span every contraction runs on the matrix cores (ranks and tokens in
// blocks of 32; one block each for almost every span):
//   step 1  y[k][h] = sigma_k gate_k (Vh_K[k] . q_h) / sqrt(d)   A = Vh_K rows, B = q
//   step 2  s[t][h] = U[t] . y[:, h]                               A = U rows,    B = y
//   step 3  online softmax over the span's tokens
//   step 4  a[k][h] = sum_t U[t][k] p[t][h]                        A = U^T rows,  B = p
//   step 5  o[j][h] += sum_k W_V[j][k] sigma_k gate_k a[k][h]      A = W_V rows,  B = b
// Rows of each A operand are permuted so that lane 16c + h ends up holding the
// 8 values (ranks or tokens 8c..8c+7) of head h that the next step takes as its
// B operand: nothing moves between lanes from step to step.  Steps 2 and 4 run
// in float32 (scores and weights unrounded); step 1 and 5 take the stored
// element type (step 5's b is rounded to it).  U tiles are staged in LDS as
// float, row-major and transposed.  The first tile, the first 32 key-part rank
// rows and sigma/gate of span i+1 are loaded while span i is processed.
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

// Row of the A operand that MFMA half h gives to lane row i: the 4-row groups
// interleave so output row 4c + v of half h is block position 8c + 4h + v.
__device__ __forceinline__ int half_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// One 16-byte piece of U tile (tb, kb): piece p -> token p/4, ranks 8(p%4)..+8.
// Clamped to an in-range address; pieces outside the span are zeroed when staged.
template <typename T>
__device__ __forceinline__ Vec8<T> ld_upiece(const SpanMeta<T>& sm, int tb, int kb, int p) {
  const int t = min(tb * 32 + (p >> 2), sm.L - 1);
  const int k8 = min(kb * 32 + 8 * (p & 3), sm.rp - 8);
  return ld8(sm.U + (size_t)t * sm.rp + k8);
}

template <typename T, int NC>
__device__ __forceinline__ void ld_vk(const SpanMeta<T>& sm, int kb, int col, int cls, int D, Vec8<T> (&vk)[2][NC]) {
  const T* Vk = sm.U + (size_t)sm.L * sm.rp;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = min(kb * 32 + half_row(col, h), sm.r - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) vk[h][c] = ld8(Vk + (size_t)k * D + 32 * c + 8 * cls);
  }
}

template <typename T, int D>
__device__ __forceinline__ void issue_span_loads(const SpanMeta<T>& sm, int col, int cls, int lane,
                                                 Vec8<T> (&vk)[2][D / 32], Vec8<T> (&ureg)[2], float (&sgr)[4]) {
  const int r1 = sm.r - 1;
  sgr[0] = sm.sg[min(lane, r1)];
  sgr[1] = sm.sg[sm.r + min(lane, r1)];
  sgr[2] = sm.sg[min(lane + 64, r1)];
  sgr[3] = sm.sg[sm.r + min(lane + 64, r1)];
#pragma unroll
  for (int i = 0; i < 2; ++i) ureg[i] = ld_upiece(sm, 0, 0, lane + 64 * i);
  ld_vk<T, D / 32>(sm, 0, col, cls, D, vk);
}

// Stage U tile (tb, kb) from its two pieces per lane into LDS (float),
// row-major ut[t][k] and transposed utt[k][t]; zero outside the span.
template <typename T>
__device__ __forceinline__ void stage_tile(const SpanMeta<T>& sm, int tb, int kb, int lane, const Vec8<T> (&ureg)[2],
                                           float* ut, float* utt) {
  constexpr int S = 36;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = lane + 64 * i;
    const int t = p >> 2, c8 = 8 * (p & 3);
    const bool ok = tb * 32 + t < sm.L && kb * 32 + c8 < sm.rp;
    float f[8];
    unpack(ureg[i], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = ok ? f[e] : 0.0f;
    *reinterpret_cast<float4*>(ut + t * S + c8) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(ut + t * S + c8 + 4) = make_float4(f[4], f[5], f[6], f[7]);
#pragma unroll
    for (int e = 0; e < 8; ++e) utt[(c8 + e) * S + t] = f[e];
  }
}

__device__ __forceinline__ Vec8<float> lds8f(const float* p) {
  return {*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
}

// Load and stage U tile (tb, kb) (synchronous; multi-block spans only).
template <typename T>
__device__ __forceinline__ void restage_tile(const SpanMeta<T>& sm, int tb, int kb, int lane, float* ut, float* utt) {
  Vec8<T> up[2];
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) up[q2] = ld_upiece(sm, tb, kb, lane + 64 * q2);
  wave_lds_sync();
  stage_tile(sm, tb, kb, lane, up, ut, utt);
  wave_lds_sync();
}

// Step 2 for token block tb: scores of tokens tb*32 + 8*cls + 4h + v for head
// (lane % 16), summed over the RB rank blocks; y is read from LDS.  With
// restage, each (tb, kb) tile is loaded first; otherwise tile (0, 0) is in LDS.
template <typename T, int G>
__device__ __forceinline__ void tile_scores(const SpanMeta<T>& sm, int tb, int RB, int col, int cls, int lane,
                                            const float* yb, float* ut, float* utt, bool restage, f32x4_t (&sc)[2]) {
  constexpr int TS = 36;
  sc[0] = sc[1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const float* yrow = yb + min(col, G - 1) * kMaxSpan;
  for (int kb = 0; kb < RB; ++kb) {
    if (restage) restage_tile(sm, tb, kb, lane, ut, utt);
    const Vec8<float> yk = lds8f(yrow + kb * 32 + 8 * cls);
#pragma unroll
    for (int h = 0; h < 2; ++h) sc[h] = mma8(lds8f(ut + half_row(col, h) * TS + 8 * cls), yk, sc[h]);
  }
}

template <typename T, int D, int G>
__device__ void role_expanded(const AttendArgs& a, int wg, char* lds) {
  using L_ = AttnLds<D, G>;
  constexpr int NC = D / 32, NJ = D / 16, TS = L_::kTileStride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, cls = lane >> 4;
  const int BG = a.B * a.Hkv;
  int* pre = reinterpret_cast<int*>(lds + 4 * L_::kWaveBytes);  // [BG+1] item prefix
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
  float* ut = reinterpret_cast<float*>(lds + wave * L_::kWaveBytes);  // [32][TS]
  float* utt = ut + 32 * TS;                                           // [32][TS]
  float* yb = utt + 32 * TS;                                           // [G][kMaxSpan]
  float* stl = yb + G * kMaxSpan;                                      // [kMaxSpan]
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

    // q as the B operand of step 1: column = head (zero for columns >= G)
    Vec8<T> qB[NC];
    const T* qrow = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)kv * G + min(col, G - 1)) * D;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      qB[cc] = ld8(qrow + 32 * cc + 8 * cls);
      if (col >= G) zero8(qB[cc]);
    }
    float m = kNegInf, lsum = 0.0f;
    f32x4_t acc[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) acc[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    Vec8<T> vk[2][NC], ureg[2];
    float sgr[4];
    SpanMeta<T> cur = span_meta<T>(0, mL, mr, mbits, mfo, mgo, fac_base, sg_base);
    issue_span_loads<T, D>(cur, col, cls, lane, vk, ureg, sgr);
    for (int i = 0; i < n; ++i) {
      const int L = cur.L, r = cur.r, rp = cur.rp;
      const int RB = (r + 31) >> 5, TB = (L + 31) >> 5;
      const bool head_on = (cur.bits >> col) & 1u;
      const T* Wv = cur.U + (size_t)L * rp + (size_t)r * D;
      // ---- sigma*gate (zero past r) and the first U tile into LDS
      {
        const float c0 = lane < r ? sgr[0] * sgr[1] : 0.0f;
        const float c1 = lane + 64 < r ? sgr[2] * sgr[3] : 0.0f;
        stl[lane] = c0;
        stl[lane + 64] = c1;
      }
      stage_tile(cur, 0, 0, lane, ureg, ut, utt);
      wave_lds_sync();
      // ---- step 1, rank blocks of 32 (block 0 was prefetched)
      for (int kb = 0; kb < RB; ++kb) {
        if (kb > 0) ld_vk<T, NC>(cur, kb, col, cls, D, vk);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4_t yc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) yc = mma8(vk[h][cc], qB[cc], yc);
          if (col < G) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int k = kb * 32 + 8 * cls + 4 * h + v;
              yb[col * kMaxSpan + k] = yc[v] * qscale * stl[k];
            }
          }
        }
      }
      // value-part rows (W_V, rank block 0) for step 5, then span i+1's loads
      Vec8<T> wv[NJ];
      {
        const int k8 = min(8 * cls, rp - 8);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) wv[jt] = ld8(Wv + (size_t)(16 * jt + col) * rp + k8);
      }
      const SpanMeta<T> nxt = span_meta<T>(min(i + 1, n - 1), mL, mr, mbits, mfo, mgo, fac_base, sg_base);
      issue_span_loads<T, D>(nxt, col, cls, lane, vk, ureg, sgr);
      wave_lds_sync();

      // ---- steps 2-5.  r <= L, so a span with one token block (L <= 32, almost
      // all) has one rank block and its single U tile is already staged.  Longer
      // spans take two passes: the span maximum first, then per rank block the
      // weights and U^T p, re-staging tiles as needed.
      float sv0[8];
      float mt = kNegInf;
      for (int tb = 0; tb < TB; ++tb) {
        f32x4_t sc[2];
        tile_scores<T, G>(cur, tb, RB, col, cls, lane, yb, ut, utt, TB > 1 || RB > 1, sc);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int t = tb * 32 + 8 * cls + 4 * h + v;
            const float x = (head_on && t < L) ? sc[h][v] : kNegInf;
            sv0[4 * h + v] = x;
            mt = fmaxf(mt, x);
          }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m, mt);
      if (mn != kNegInf) {
        const float alpha = exp2f(m - mn);
        lsum *= alpha;
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) acc[jt] *= alpha;
        m = mn;
      }
      for (int kb = 0; kb < RB; ++kb) {
        f32x4_t am[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
        for (int tb = 0; tb < TB; ++tb) {
          float sv[8];
          if (TB == 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sv[e] = sv0[e];
          } else {
            f32x4_t sc[2];
            tile_scores<T, G>(cur, tb, RB, col, cls, lane, yb, ut, utt, true, sc);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int t = tb * 32 + 8 * cls + 4 * h + v;
                sv[4 * h + v] = (head_on && t < L) ? sc[h][v] : kNegInf;
              }
            restage_tile(cur, tb, kb, lane, ut, utt);
          }
          float pr[8];
          float ps = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pr[e] = (m == kNegInf) ? 0.0f : exp2f(sv[e] - m);
            ps += pr[e];
          }
          if (kb == 0) lsum += ps;
          Vec8<float> pv;
          pack8(pr, pv);
          // step 4: a[k][h] += sum_t U[t][k] p[t][h]
#pragma unroll
          for (int h = 0; h < 2; ++h) am[h] = mma8(lds8f(utt + half_row(col, h) * TS + 8 * cls), pv, am[h]);
        }
        // step 5: o[j][h] += sum_k W_V[j][k] b[k][h],  b = sigma*gate * a
        if (kb > 0) {
          const int k8 = min(kb * 32 + 8 * cls, rp - 8);
#pragma unroll
          for (int jt = 0; jt < NJ; ++jt) wv[jt] = ld8(Wv + (size_t)(16 * jt + col) * rp + k8);
        }
        float bv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int v = 0; v < 4; ++v) bv[4 * h + v] = am[h][v] * stl[kb * 32 + 8 * cls + 4 * h + v];
        Vec8<T> bp;
        pack8(bv, bp);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) acc[jt] = mma8(wv[jt], bp, acc[jt]);
      }
      wave_lds_sync();
      cur = nxt;
    }
    // partial of this item: head col, summed over the four lane classes
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const int slot = a.nch_a4 + lc;
    float* pml = a.part_ml + ((size_t)g * a.P_max + slot) * G * 2;
    float* po = a.part_o + ((size_t)g * a.P_max + slot) * G * D;
    if (col < G) {
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int v = 0; v < 4; ++v) po[col * D + 16 * jt + 4 * cls + v] = acc[jt][v];
      if (cls == 0) {
        pml[col * 2] = m;
        pml[col * 2 + 1] = lsum;
      }
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
// Two waves per SIMD: the span steps are latency-bound, and a second resident wave hides
// more of it than the few registers spilled to reach 256 VGPRs cost.
template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attend_expanded_kernel(const AttendArgs a) {
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
    const T* Vk = Ub + (size_t)L * rp;            // key part   [r][D]
    const T* Wv = Vk + (size_t)r * D;             // value part [D][rp]
    const float* sgp = a.sg + a.sg_off[(size_t)g * a.seg_cap + S];
    const int row0 = a.tok_off[(size_t)g * (a.seg_cap + 1) + j];
    for (int t = 0; t < L; ++t) {
      float acc[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
      for (int k = 0; k < r; ++k) {
        const float w = load1(Ub + (size_t)t * rp + k) * (sgp[k] * sgp[r + k]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int colj = lane + 64 * c;
          acc[c] += w * (colj < D ? load1(Vk + (size_t)k * D + colj) : load1(Wv + (size_t)(colj - D) * rp + k));
        }
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
