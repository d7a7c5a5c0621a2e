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
//   route_kernel    one lane per span, the G heads of a KV group per lane:
//                   canonical float32 score, decision bits, and the
//                   ascending list, head masks and count of each (b, kv).
//   attend_fused_kernel  both attention passes in one launch (every rank
//                   <= 64): expanded-span waves first, then full-resolution
//                   chunks.
//   attend_full_kernel  (role A) full-resolution entries + size-corrected
//                   summaries in 32-entry tiles, q.K and P.V on the matrix
//                   cores, one online-softmax state per head.
//   attend_expanded_kernel  (role E) expanded spans, never materialising the
//                   rebuilt K/V: it applies the factors to the query
//                   (y = sigma~ .* (Vh_K q)), scores the tokens with U y, and
//                   applies the weights back through U and Vh_V.
//   combine_kernel  log-sum-exp merge of all partials of a query head.
//   recon_*         standalone token-level K/V rebuild (tests, unfused use).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

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
//
// One launch per call.  A workgroup scores 256 consecutive spans of one
// (b, kv) (one lane per span, the G heads of the group per lane), compacts
// its own expanded spans and writes them at their final list positions.  A
// position needs the number of expanded spans in the group's earlier tiles:
// every workgroup but the group's last publishes its own count in a status
// word as soon as it has it, then takes the counts of all earlier tiles from
// their status words (one lane per tile).  Only these counts cross
// workgroups, through relaxed device-scope atomics, so no fence has to order
// any other memory (a fenced variant, in which the last workgroup of a group
// compacted masks written by the others, ran about five times slower).  A
// workgroup only ever waits for tiles that come before its own, and those
// publish without waiting:
//   - when the whole grid fits on the GPU at once (the host checks the
//     occupancy), tile = blockIdx.x: every earlier workgroup is resident or
//     done, since workgroups are dispatched in index order;
//   - otherwise a per-group ticket drawn at the start gives the tile, so the
//     tiles waited for belong to workgroups that are already running (the
//     ticket's atomic round trip costs about 5 us per call, hence the first
//     form when it is safe).
// Every wait therefore ends; it is also bounded, and a workgroup that gives up
// reports exp_count = -1.
//
// The workspace is all zero between calls, and each of its words is returned
// to zero by operations on that word alone (so no ordering between different
// words is assumed): the workgroup drawing a group's last ticket stores 0 to
// the ticket; a status word holds (count + 1) in its low 16 bits, published
// by a store, and in its high 16 bits the number of later tiles that have
// read it, counted by their atomic adds once they see it published; the
// reader that completes the count stores 0.
//
// Fused multiply-adds were tried twice for the score chain (exact when every
// bf16 product is exact in float32): with per-product range checks (1.5 us
// slower per call), and with a per-tile bound on min/max |q| and |rho| plus
// the query in scalar registers (24 against 22 us at 128K batch 4).  The call
// is bound by its memory phase: without the chain it still takes 18 us, and
// streaming the keys alone 12 us.
//
// 16 bytes from global memory as a vector value (keeps the staging array in
// registers; an aggregate copy into it leaves the array in scratch memory).
typedef unsigned int route_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 route_ld16(const char* p) {
  const route_u32x4 x = *reinterpret_cast<const route_u32x4*>(p);
  return make_uint4(x[0], x[1], x[2], x[3]);
}
constexpr int kRouteRowBytes = 128;
constexpr int kRouteRowStride = 144;
constexpr int kRouteSpinLimit = 1 << 20;

__device__ __forceinline__ uint32_t atomic_add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_load_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Routing keys are staged through LDS 128 bytes of each row at a time
// (coalesced 16-byte loads, 8 lanes per row), padded to a 144-byte row stride
// so that each lane then reads its own row without bank conflicts; every
// pass's loads are issued up front.
// Folded routing (route_keys = 1): the query is folded once per call,
// q'[b][h][j] = fl32(sum over m of fold[kv][j][m] * q[b][h][m]), a sequential
// fp64 chain in m with every product and sum rounded separately (one thread
// per output element).  The operands of 16 products are requested at a time
// (the head dimension is a template parameter, so the loop unrolls); a loop
// over a run-time length waited for each product's two loads in turn.
template <typename T, int D>
__global__ __launch_bounds__(256) void fold_query_kernel(const RouteArgs a) {
#pragma clang fp contract(off)
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int G = a.Hq / a.Hkv;
  if (idx >= a.B * a.Hq * D) return;
  const int j = idx % D, bh = idx / D, h = bh % a.Hq;
  const double* M = a.foldm + ((size_t)(h / G) * D + j) * D;
  const T* q = static_cast<const T*>(a.q) + (size_t)bh * D;
  double acc = 0.0;
#pragma unroll
  for (int m0 = 0; m0 < D; m0 += 16) {
    double mv[16];
    float qv[16];
#pragma unroll
    for (int u = 0; u < 16; u += 2) {
      const double2 x = *reinterpret_cast<const double2*>(M + m0 + u);
      mv[u] = x.x;
      mv[u + 1] = x.y;
    }
    float f0[8], f1[8];
    load8(q + m0, f0);
    load8(q + m0 + 8, f1);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      qv[u] = f0[u];
      qv[u + 8] = f1[u];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const double prod = mv[u] * (double)qv[u];
      acc = acc + prod;
    }
  }
  a.qfold[idx] = (float)acc;
}

// FOLD: the keys are the attention summary keys kbar and the query the folded
// one; the chain's result is then scaled by the span's key scale,
// z' = fl32(z * key_scale).
template <typename T, int D, int G, bool FOLD>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const RouteArgs a) {
  constexpr int EPP = kRouteRowBytes / (int)sizeof(T);   // elements of a row per pass
  constexpr int NP = D / EPP;
  __shared__ float qs[G * D];
  __shared__ __align__(16) char tile[kRouteThreads * kRouteRowStride];
  __shared__ int s_ticket, s_prefix, s_fail;
  __shared__ int s_wcnt[kRouteThreads / 64];
  const int kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = b * a.Hkv + kv;
  const int ns = a.n_seg[b];
  const int nb = (ns + kRouteThreads - 1) / kRouteThreads;
  if (ns == 0) {
    if (blockIdx.x == 0 && tid == 0) a.exp_count[g] = 0;
    return;
  }
  if ((int)blockIdx.x >= nb) return;
  if (tid == 0) s_ticket = a.use_ticket ? (int)atomic_add_dev(a.ticket + g, 1u) : (int)blockIdx.x;
  // Every load before the row stream is unconditional, with its index clamped
  // into range: a load under a condition becomes a branch, and the compiler
  // then waits for it inside the branch before the next load is issued.  The
  // query rows are requested first and stored to LDS after the key rows are
  // requested, so the row stream does not wait for them.
  constexpr int QPT = (G * D + kRouteThreads - 1) / kRouteThreads;
  float qv[QPT];
  if constexpr (FOLD) {
    const float* qf = a.qfold + ((size_t)b * a.Hq + (size_t)kv * G) * D;
#pragma unroll
    for (int k = 0; k < QPT; ++k) qv[k] = qf[min(tid + kRouteThreads * k, G * D - 1)];
  } else {
    const T* q = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)kv * G) * D;
#pragma unroll
    for (int k = 0; k < QPT; ++k) qv[k] = load1(q + min(tid + kRouteThreads * k, G * D - 1));
  }
  float th[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) th[gi] = a.theta[(size_t)b * a.Hq + kv * G + gi];
  __syncthreads();
  const int vb = s_ticket;
  if (a.use_ticket && tid == 0 && vb == nb - 1) atomic_store_dev(a.ticket + g, 0u);   // every ticket of this call is drawn
  const int S0 = vb * kRouteThreads;
  const int nrow = min(kRouteThreads, ns - S0);
  const char* rbase = static_cast<const char*>(a.rho) + ((size_t)g * a.seg_cap + S0) * D * sizeof(T);

  float z[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) z[gi] = 0.0f;
  const float ksc = FOLD ? a.key_scale[(size_t)g * a.seg_cap + S0 + min(tid, nrow - 1)] : 0.0f;
  uint4 v[NP][8];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // rows past the tile's last span repeat that span's row; no lane reads them
      const int piece = tid + kRouteThreads * j, row = min(piece >> 3, nrow - 1), c = piece & 7;
      v[p][j] = route_ld16(rbase + (size_t)row * D * sizeof(T) + p * kRouteRowBytes + c * 16);
      // keep the passes' loads in pass order: the first pass's data then lands
      // first, and its chain runs while the later passes' rows are in flight
      if (j == 7) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
  for (int k = 0; k < QPT; ++k)
    if (tid + kRouteThreads * k < G * D) qs[tid + kRouteThreads * k] = qv[k];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    __syncthreads();  // the previous pass's row reads are done (first pass: the query rows are staged)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int piece = tid + kRouteThreads * j, row = piece >> 3, c = piece & 7;
      *reinterpret_cast<uint4*>(tile + row * kRouteRowStride + c * 16) = v[p][j];
    }
    __syncthreads();
    if (tid < nrow) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float rv[16 / sizeof(T)];
        const uint4 u = *reinterpret_cast<const uint4*>(tile + tid * kRouteRowStride + c * 16);
        if constexpr (sizeof(T) == 2) {
          rv[0] = __uint_as_float(u.x << 16); rv[1] = __uint_as_float(u.x & 0xffff0000u);
          rv[2] = __uint_as_float(u.y << 16); rv[3] = __uint_as_float(u.y & 0xffff0000u);
          rv[4] = __uint_as_float(u.z << 16); rv[5] = __uint_as_float(u.z & 0xffff0000u);
          rv[6] = __uint_as_float(u.w << 16); rv[7] = __uint_as_float(u.w & 0xffff0000u);
        } else {
          rv[0] = __uint_as_float(u.x); rv[1] = __uint_as_float(u.y);
          rv[2] = __uint_as_float(u.z); rv[3] = __uint_as_float(u.w);
        }
        const int i0 = p * EPP + c * (int)(16 / sizeof(T));
#pragma unroll
        for (int e = 0; e < (int)(16 / sizeof(T)); ++e) {
#pragma unroll
          for (int gi = 0; gi < G; ++gi) {
#pragma clang fp contract(off)
            const float prod = qs[gi * D + i0 + e] * rv[e];
            z[gi] = z[gi] + prod;
          }
        }
      }
    }
  }
  if constexpr (FOLD) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
#pragma clang fp contract(off)
      z[gi] = z[gi] * ksc;
    }
  }
  // this tile's expanded spans, their order within the tile, and the tile count
  uint32_t bits = 0;
  if (tid < nrow) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) bits |= (z[gi] > th[gi] ? 1u : 0u) << gi;
  }
  const uint64_t bal = __ballot(bits != 0);
  const int wexcl = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) s_wcnt[wave] = __popcll(bal);
  __syncthreads();
  int woff = 0, cnt = 0;
#pragma unroll
  for (int w = 0; w < kRouteThreads / 64; ++w) {
    const int c = s_wcnt[w];
    if (w < wave) woff += c;
    cnt += c;
  }
  uint32_t* status = a.status + (size_t)g * a.nblk_cap;
  if (tid == 0 && vb < nb - 1) atomic_store_dev(status + vb, (uint32_t)cnt + 1u);   // count + 1 (0 = not yet)
  if (wave == 0) {
    int acc = 0, fail = 0;
    for (int i = lane; i < vb; i += 64) {
      uint32_t st = atomic_load_dev(status + i);
      for (int spin = 0; (st & 0xFFFFu) == 0u; ++spin) {
        if (spin == kRouteSpinLimit) break;
        __builtin_amdgcn_s_sleep(2);
        st = atomic_load_dev(status + i);
      }
      if ((st & 0xFFFFu) == 0u) {
        fail = 1;
        continue;
      }
      const uint32_t old = atomic_add_dev(status + i, 1u << 16);   // this tile has read tile i
      acc += (int)(old & 0xFFFFu) - 1;
      if ((old >> 16) + 1u == (uint32_t)(nb - 1 - i)) atomic_store_dev(status + i, 0u);   // its last reader
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      acc += __shfl_xor(acc, off);
      fail |= __shfl_xor(fail, off);
    }
    if (lane == 0) {
      s_prefix = acc;
      s_fail = fail;
    }
  }
  __syncthreads();
  const int prefix = s_prefix;
  if (s_fail) {
    if (tid == 0) a.exp_count[g] = -1;
    return;
  }
  if (bits != 0) {
    const int pos = prefix + woff + wexcl;
    a.exp_list[(size_t)g * a.seg_cap + pos] = S0 + tid;
    a.exp_mask[(size_t)g * a.seg_cap + pos] = (uint8_t)bits;
  }
  if (tid == 0 && vb == nb - 1) a.exp_count[g] = prefix + cnt;
}

// ================================================================ attention
template <int D, int G>
struct AttnLds {
  // role A: per-chunk summary masks and log2 span lengths, cross-wave merge
  static constexpr int kMaskBytes = 2048;  // >= 32 * tiles_a4 (host checks)
  static constexpr int kMergeFloats = 4 * G * (D + 2);
  static constexpr int kRoleA = kMaskBytes + kMaskBytes * 4 + kMergeFloats * 4;
};

// Maximum and sum over the four 16-lane rows, same position in each row
// (lanes h, h + 16, h + 32, h + 48): row swaps on the VALU, no LDS.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Operands of one 32-entry tile of the full-resolution + summary stream.
template <typename T, int D>
struct TileOps {
  Vec8<T> k[2][D / 32];   // K rows, MFMA halves: row (col) = entry 8*(col/4) + 4h + col%4
  Vec8<T> v[D / 16];      // V^T rows 16 jt + col, entries 8 cls .. 8 cls + 7
};
template <typename T>
struct TileSrc {
  const T *fk, *fvt, *sk, *svt;   // full-res keys / value tiles, summary keys / value tiles
  int nft, nf, ns;                // full-res tiles, full-res entries, summaries
};

template <typename T, int D>
__device__ __forceinline__ void tile_load_k(TileOps<T, D>& o, const TileSrc<T>& s, int t, int col, int cls) {
  constexpr int NC = D / 32;
  const bool summ = t >= s.nft;
  const int base = (summ ? t - s.nft : t) * 32;
  const int npart = summ ? s.ns : s.nf;
  const T* krows = summ ? s.sk : s.fk;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = min(base + 8 * (col >> 2) + 4 * h + (col & 3), npart - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) o.k[h][c] = ld8(krows + (size_t)e * D + 32 * c + 8 * cls);
  }
}
template <typename T, int D>
__device__ __forceinline__ void tile_load_v(TileOps<T, D>& o, const TileSrc<T>& s, int t, int col, int cls) {
  constexpr int NJ = D / 16;
  const bool summ = t >= s.nft;
  const int tt = summ ? t - s.nft : t;
  const T* vt = (summ ? s.svt : s.fvt) + (size_t)tt * 32 * D;
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt) o.v[jt] = ld8(vt + (16 * jt + col) * 32 + 8 * cls);
}
template <typename T, int D>
__device__ __forceinline__ void tile_load(TileOps<T, D>& o, const TileSrc<T>& s, int t, int col, int cls) {
  tile_load_k<T, D>(o, s, t, col, cls);
  tile_load_v<T, D>(o, s, t, col, cls);
}

// Scores, online softmax and P.V of one tile for head `col` of this lane.
template <typename T, int D, int G>
__device__ __forceinline__ void tile_step(TileOps<T, D>& o, const TileSrc<T>& s, int t, int tn, int S0,
                                          const uint8_t* smask, const float* slog, const Vec8<T> (&qB)[D / 32],
                                          float qscale, int col, int cls, float& m, float& lsum,
                                          f32x4_t (&acc)[D / 16]) {
  constexpr int NC = D / 32, NJ = D / 16;
  const bool summ = t >= s.nft;
  const int base = (summ ? t - s.nft : t) * 32;
  const int npart = summ ? s.ns : s.nf;
  f32x4_t sc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    sc[h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < NC; ++c) sc[h] = mma8(o.k[h][c], qB[c], sc[h]);
  }
  // the next tile's keys go in flight as soon as the scores have used these
  // registers, its values after P.V (fused attention at 128K batch 4: 78.0
  // against 79.2 us; with no expansion 48.9 against 50.3 us)
  if (tn >= 0) tile_load_k<T, D>(o, s, tn, col, cls);
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
  mt = rows_max(mt);
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
  for (int jt = 0; jt < NJ; ++jt) acc[jt] = mma8(o.v[jt], pB, acc[jt]);
  if (tn >= 0) tile_load_v<T, D>(o, s, tn, col, cls);
}

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
__device__ __forceinline__ void role_full_summary(const AttendArgs& a, int idx, char* lds) {
  constexpr int NC = D / 32, NJ = D / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, cls = lane >> 4;
  // Chunk-major order (mixed decode): chunk k of every (b, kv) before chunk
  // k + 1 of any, so the ragged last chunks are dispatched last, a shorter
  // tail (79.3 against 81.0 us at 128K batch 4).  Group-major (dense decode,
  // 64 chunks per group): 353-355 against 359-361 us.
  const int BGn = a.B * a.Hkv;
  const int g = a.chunk_major ? idx % BGn : idx / a.a4_n;
  const int chunk = a.a4_lo + (a.chunk_major ? idx / BGn : idx % a.a4_n);
  const int b = g / a.Hkv, kv = g % a.Hkv;
  const int nf = a.n_full[b], ns = a.n_seg[b];
  const int nft = (nf + 31) / 32, nst = (ns + 31) / 32;
  // chunks [0, nch_full) hold full-resolution tiles only, the rest summary
  // tiles only (a full-resolution chunk never reads the route's outputs, so
  // it may run while the route does); tiles numbered full first, then summary
  int t0, t1;
  if (chunk < a.nch_full) {
    t0 = min(nft, chunk * a.tiles_a4);
    t1 = min(nft, t0 + a.tiles_a4);
  } else {
    const int cs = (chunk - a.nch_full) * a.tiles_a4;
    t0 = nft + min(nst, cs);
    t1 = nft + min(nst, cs + a.tiles_a4);
  }
  const int S0 = (max(t0, nft) - nft) * 32, S1 = min(ns, (max(t1, nft) - nft) * 32);

  uint8_t* smask = reinterpret_cast<uint8_t*>(lds);
  float* slog = reinterpret_cast<float*>(lds + AttnLds<D, G>::kMaskBytes);
  float* merge = reinterpret_cast<float*>(lds + AttnLds<D, G>::kMaskBytes * 5);

  const int ftiles = (a.full_cap + 31) / 32, stiles = (a.seg_cap + 31) / 32;
  const T* fk = static_cast<const T*>(a.full_k) + (size_t)g * a.full_cap * D;
  const T* fvt = static_cast<const T*>(a.full_v) + (size_t)g * ftiles * 32 * D;
  const T* sk = static_cast<const T*>(a.sum_k) + (size_t)g * a.seg_cap * D;
  const T* svt = static_cast<const T*>(a.sum_v) + (size_t)g * stiles * 32 * D;

  // This wave's first tile (t0 + wave) and q are put in flight before the
  // summary masks are gathered, so the gather's memory round trips overlap
  // the tile loads.
  TileOps<T, D> opA;
  const TileSrc<T> src{fk, fvt, sk, svt, nft, nf, ns};
  int t = t0 + wave;
  if (t < t1) tile_load<T, D>(opA, src, t, col, cls);
  // q as the B operand: column = head (zero for columns >= G)
  Vec8<T> qB[NC];
  const T* qrow = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)kv * G + min(col, G - 1)) * D;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qB[c] = ld8(qrow + 32 * c + 8 * cls);
    if (col >= G) zero8(qB[c]);
  }

  // Summaries of this chunk: log2 of the span length, and the head mask of
  // spans in the expanded list (0 for the others).  The list is ascending, so
  // its entries in [S0, S1) are one run starting at lo = the number of entries
  // below S0, found in two rounds of parallel probes.
  const int32_t* so = a.seg_off + (size_t)b * (a.seg_cap + 1);
  for (int i = tid; i < S1 - S0; i += kAttnThreads) {
    const int S = S0 + i;
    smask[i] = 0;
    slog[i] = log2f((float)(so[S + 1] - so[S] - 1));
  }
  if (S1 > S0) {
    const int cnt = a.exp_count[g];
    const int32_t* lst = a.exp_list + (size_t)g * a.seg_cap;
    // round 1: probe entries 0, step, 2 step, ...; the probes below S0 are a prefix
    const int step = (cnt + kAttnThreads - 1) / kAttnThreads;
    const int pj = tid * step;
    const int nb = __syncthreads_count(pj < cnt && lst[pj] < S0);
    int lo = 0;
    if (nb > 0) {
      // lo lies in ((nb - 1) step, nb step]: count the unknown entries between
      const int base = (nb - 1) * step + 1, end = min(nb * step, cnt);
      lo = base;
      for (int k0 = 0; k0 < end - base; k0 += kAttnThreads) {
        const int j = base + k0 + tid;
        lo += __syncthreads_count(j < end && lst[j] < S0);
      }
    }
    for (int j = lo + tid; j < cnt; j += kAttnThreads) {
      const int S = lst[j];
      if (S >= S1) break;
      smask[S - S0] = a.exp_mask[(size_t)g * a.seg_cap + j];
    }
  }
  __syncthreads();

  const float qscale = a.qscale;
  float m = kNegInf, lsum = 0.0f;
  f32x4_t acc[NJ];
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt) acc[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // This wave's tiles t, t + 4, ...: one operand set, refilled with the next
  // tile inside tile_step as soon as each half has been used.  A single set
  // keeps the fused launch at three waves per SIMD; the other waves of the
  // SIMD cover the load latency.
  while (t < t1) {
    tile_step<T, D, G>(opA, src, t, t + 4 < t1 ? t + 4 : -1, S0, smask, slog, qB, qscale, col, cls, m, lsum, acc);
    t += 4;
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

// Spans per work item of the expanded-span pass, given the spans listed over
// all groups and the pass's waves.  One item's chain of memory round trips
// sets the length of the pass, so while few spans are listed (at most
// kExpAdaptMax per wave) items are as short as lets every wave take at most
// one, and no shorter than kExpChunkMin; with more listed spans they are
// kExpChunk long: fewer items leave expanded-span waves idle early, and their
// slots go to the full-resolution chunks of the fused launch.  Measured at
// 128K batch 4: 1% listed, attention 67.3 -> 58.6 us; 2%, 70.8 -> 66.0 us;
// 5% (5.7 spans per wave), 79.6 us with 8-span items against 81.0 us with 6;
// 32K batch 1 at 10%: 38.5 -> 19.2 us.  The merge recomputes the same size
// from the same counts.
constexpr int kExpAdaptMax = 4;
__device__ __forceinline__ int item_spans(int listed, int waves) {
  const int c = (listed + waves - 1) / waves;
  return c > kExpAdaptMax ? kExpChunk : max(kExpChunkMin, c);
}

// Role E (expanded spans): one wave per workgroup.  A work item is up to
// item_spans consecutive entries of one (b, kv) expanded list, processed one
// span at a time in two passes:
//   pass 1: y[k][h] = sigma_k gate_k (Vh_K[k] . q_h) log2(e)/sqrt(d)
//           (A = Vh_K rows, B = q) and the token scores s[t][h] = U[t] . y[:, h]
//           (A = U rows, B = y), kept in LDS; the span's maximum per head.
//   pass 2: p = exp2(s - m), a[k][h] = sum_t U[t][k] p[t][h]
//           (A = U^T rows, B = p) and o[j][h] += sum_k W_V[j][k] sigma_k gate_k a[k][h]
//           (A = W_V rows, B = b).
// Between the passes the output accumulators are rescaled once to the new
// maximum; the two passes keep different registers live.  Head h = lane % 16
// (columns >= G unused); ranks and tokens in groups of 16.  The products of
// scores, U^T p and W_V b are 16x16x16: the result of each (lane 16c + h
// holds rows 4c..4c+3 of column h) is exactly the B operand the next one
// takes, so nothing moves between lanes.  bf16: y enters the score product as
// a two-term bf16 split (hi + lo, about 16 significant bits), p and b are
// rounded to bf16; float: every product in float32.
//
// Factor data streams through a per-wave LDS ring in 1 KB chunks (16 bytes
// per lane), loaded into registers one granule (ExpCfg::K chunks) ahead of
// the consumer and written to the ring a granule at a time.  The stream is a
// sequence of regions, each starting on a chunk boundary; per span:
//   read once (one basis, U at most RING - 1024 K bytes): the sigma|gate
//     entry, then the whole block Vh_K | U | W_V; pass 2 reads U where pass 1
//     left it in the ring and sigma * gate from LDS;
//   one basis, larger U: the entry, Vh_K | U, then U | W_V;
//   separate bases: the entry's key half, Vh_K | U_K, its value half,
//     U_V | W_V.
// Factor block of a span: Vh_K [r][d] (8-element groups rotated by the row) |
// U [L][rp] | W_V in 16-rank column blocks [d][min(16, rp - 16 g)].  Lanes
// past the end of a region re-read its last 16 bytes (no extra memory lines).
template <typename T, int RGM> struct ExpCfg;
// K: 1 KB chunks per granule in flight.  The ring holds a granule in flight
// plus the largest piece read at once (16 rows of Vh_K or U, or one 16-rank
// W_V block: 16 x 128 elements).  The four waves of a workgroup stay within
// 64 KB of LDS: more than that per workgroup halves the workgroups a compute
// unit holds.
template <int RGM> struct ExpCfg<bf16raw, RGM> { static constexpr int K = 4; static constexpr int kRing = 8192; };
template <int RGM> struct ExpCfg<float, RGM> { static constexpr int K = 8; static constexpr int kRing = 16384; };
constexpr int kExpTok = kMaxSpan;   // tokens of one span (score buffer)

// Byte positions in a per-wave ring of RING bytes (a multiple of 1 KB, not
// necessarily a power of two).
template <uint32_t RING>
struct RingPos {
  static constexpr bool kPow2 = (RING & (RING - 1)) == 0;
  // stream offset x -> ring position
  __device__ static __forceinline__ uint32_t of(uint32_t x) {
    if constexpr (kPow2) return x & (RING - 1);
    else return x % RING;
  }
  // (p + o) mod RING for a ring position p and an offset o < RING
  __device__ static __forceinline__ uint32_t add(uint32_t p, uint32_t o) {
    if constexpr (kPow2) {
      return (p + o) & (RING - 1);
    } else {
      const uint32_t x = p + o;
      return x >= RING ? x - RING : x;
    }
  }
};

template <typename T, int G, int RGM>
struct ExpLds {
  static constexpr int kRing = ExpCfg<T, RGM>::kRing;
  static_assert(kRing % 1024 == 0, "ring size is a whole number of 1 KB chunks");
  static_assert(kRing >= ExpCfg<T, RGM>::K * 1024 + 16 * kMaxSpan * (int)sizeof(T), "ring holds a granule and a piece");
  static constexpr int kS = kRing;                          // scores [token group][class][G] float4
  static constexpr int kQ = kS + (kExpTok / 16) * 4 * G * 16;   // q of the item's G heads [G][kMaxD]
  static constexpr int kStl = kQ + G * 128 * (int)sizeof(T);    // sigma*gate of the current span [kMaxSpan]
  static constexpr int kBytes = kStl + kMaxSpan * 4;
};

// Four elements of the storage type as an MFMA operand of a 16x16x16 product.
template <typename T> struct Vec4;
template <> struct Vec4<bf16raw> { uint2 v; };
template <> struct Vec4<float> { float4 v; };
typedef short s16x4_t __attribute__((ext_vector_type(4)));
// C[i][j] += sum over classes c and m < 4 of A_lane(16c+i)[m] * B_lane(16c+j)[m];
// lane 16c + j holds C[4c + v][j].
__device__ __forceinline__ f32x4_t mma4(const Vec4<bf16raw>& x, const Vec4<bf16raw>& y, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, x.v), __builtin_bit_cast(s16x4_t, y.v),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma4(const Vec4<float>& x, const Vec4<float>& y, f32x4_t c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.v.x, y.v.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.v.y, y.v.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.v.z, y.v.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(x.v.w, y.v.w, c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void pack4(const float (&p)[4], Vec4<bf16raw>& o) {
  o.v = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
}
__device__ __forceinline__ void pack4(const float (&p)[4], Vec4<float>& o) { o.v = make_float4(p[0], p[1], p[2], p[3]); }

// Ring reads at ring byte offsets (already reduced modulo the ring size).
template <typename T>
__device__ __forceinline__ Vec4<T> rd4(const char* ring, uint32_t ob) {
  Vec4<T> x;
  if constexpr (sizeof(T) == 2) x.v = *reinterpret_cast<const uint2*>(ring + ob);
  else x.v = *reinterpret_cast<const float4*>(ring + ob);
  return x;
}
template <typename T, uint32_t RING>
__device__ __forceinline__ Vec8<T> rd8(const char* ring, uint32_t ob) {
  Vec8<T> x;
  if constexpr (sizeof(T) == 2) {
    x.v = *reinterpret_cast<const uint4*>(ring + ob);
  } else {
    x.a = *reinterpret_cast<const float4*>(ring + ob);
    x.b = *reinterpret_cast<const float4*>(ring + RingPos<RING>::add(ob, 16u));
  }
  return x;
}

// 16 bytes from a global byte address (address space 1: a global load, not a
// flat one that would also count against the LDS counter).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t g_u32x4;
__device__ __forceinline__ uint4 gload16(uint64_t addr) {
  const u32x4_t v = *reinterpret_cast<g_u32x4*>(addr);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t x, int i) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), i);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(x & 0xffffffffu), i);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t kb_round(uint32_t x) { return (x + 1023u) & ~1023u; }

// Per-lane metadata of an item (lane i < n: span i of the item).
struct ItemMeta {
  int L, r, bits;
  uint64_t sga, fa;   // global addresses of the sg entry and the factor block
};
// A span is read once (sigma|gate, then its whole factor block) when its U
// stays in the ring from the score pass to the weight pass: nothing is
// written to the ring between the two, and after the score pass the ring
// holds at least RING - 1024 K bytes before the end of U.  Otherwise (and
// with separate bases) the weight pass streams U | W_V again.
template <typename T, int K, uint32_t RING>
__device__ __forceinline__ bool read_once(int L, int r, bool sep) {
  return !sep && (uint32_t)(L * ((r + 7) & ~7)) * (uint32_t)sizeof(T) <= RING - 1024u * K;
}

// Region `kind` of span i: 0 / 2 sigma|gate, 1 Vh_K | U (the whole block
// Vh_K | U | W_V for a span read once), 3 U | W_V.  With separate key and
// value bases (sep) the block is Vh_K | U_K | U_V | W_V and the sigma|gate
// entry sigma_K | gate | sigma_V | gate: region 2 is the second half of the
// entry and region 3 is U_V | W_V.
template <typename T, int D, int K, uint32_t RING>
__device__ __forceinline__ void region_of(const ItemMeta& m, int i, int kind, bool sep, uint64_t& base, uint32_t& size) {
  constexpr uint32_t ES = sizeof(T);
  const int L = __builtin_amdgcn_readlane(m.L, i), r = __builtin_amdgcn_readlane(m.r, i);
  const uint32_t rp = (uint32_t)((r + 7) & ~7), rq = (uint32_t)((r + 3) & ~3);
  if ((kind & 1) == 0) {
    base = readlane64(m.sga, i) + (kind == 2 && sep ? 8u * rq : 0u);
    size = 8u * rq;
  } else if (kind == 1) {
    base = readlane64(m.fa, i);
    size = ES * ((uint32_t)r * D + (uint32_t)L * rp + (read_once<T, K, RING>(L, r, sep) ? D * rp : 0u));
  } else {
    base = readlane64(m.fa, i) + ES * (uint64_t)((uint32_t)r * D + (sep ? (uint32_t)L * rp : 0u));
    size = ES * ((uint32_t)L * rp + D * rp);
  }
}

// Wave-uniform walk over the regions of an item, span by span: span i,
// region kind, byte `off` of a region of `size` bytes at `base`.  Per span the
// regions are 0, 1 (read once); 0, 1, 3 (one basis); 0, 1, 2, 3 (separate
// bases).  Past the last region the last 1 KB is repeated (never read from
// the ring).
struct RegionCursor {
  int i, kind, n;
  bool sep;
  uint32_t off, size;
  uint64_t base;
};

template <typename T, int D, int K, uint32_t RING>
__device__ __forceinline__ void cursor_next(RegionCursor& c, const ItemMeta& m) {
  c.off += 1024u;
  if (c.off < c.size) return;
  const bool once = c.kind == 1 && read_once<T, K, RING>(__builtin_amdgcn_readlane(m.L, c.i),
                                                          __builtin_amdgcn_readlane(m.r, c.i), c.sep);
  if (c.kind == 0 || c.kind == 2) {
    c.kind += 1;
  } else if (c.kind == 1 && !once) {
    c.kind = c.sep ? 2 : 3;
  } else if (c.i + 1 < c.n) {
    c.i += 1;
    c.kind = 0;
  } else {
    c.off -= 1024u;
    return;
  }
  region_of<T, D, K, RING>(m, c.i, c.kind, c.sep, c.base, c.size);
  c.off = 0;
}
__device__ __forceinline__ uint64_t cursor_addr(const RegionCursor& c, int lane) {
  return c.base + min(c.off + 16u * (uint32_t)lane, c.size - 16u);
}

// Make stream bytes [.., e) readable from the ring: write staged granules and
// stage the following ones until the ring holds everything before e.
// `written` counts the stream bytes already in the ring (a multiple of 1024 K).
// The staging registers hold kExpStages granules in flight, oldest first: the
// oldest is written to the ring, the others move up, and the next granule of
// the stream is requested into the last stage.  One stage: two (8 KB in
// flight per wave) took the fused kernel to 168 registers with spills and
// ran slower (fused attention 98 against 80 us at 128K batch 4).
constexpr int kExpStages = 1;
template <typename T, int D, int K, int RING>
__device__ __forceinline__ void advance(uint4 (&stg)[K * kExpStages], uint32_t& written, uint32_t e, RegionCursor& c,
                                        const ItemMeta& m, int lane, char* ring) {
  while (written < e) {
    const uint32_t w0 = RingPos<RING>::of(written);
#pragma unroll
    for (int jj = 0; jj < K; ++jj)
      *reinterpret_cast<uint4*>(ring + RingPos<RING>::add(w0, 1024u * jj) + 16u * (uint32_t)lane) = stg[jj];
#pragma unroll
    for (int jj = 0; jj < K * (kExpStages - 1); ++jj) stg[jj] = stg[jj + K];
#pragma unroll
    for (int jj = 0; jj < K; ++jj) {
      stg[K * (kExpStages - 1) + jj] = gload16(cursor_addr(c, lane));
      cursor_next<T, D, K, RING>(c, m);
    }
    written += 1024u * K;
  }
  wave_lds_sync();
}

// `wid`: this wave's index among the `nwaves` waves running the pass; `lds`:
// the wave's own LDS area (ExpLds::kBytes).
template <typename T, int D, int G, int RGM>
__device__ __forceinline__ void role_expanded(const AttendArgs& a, int wid, int nwaves, char* lds) {
  using X = ExpLds<T, G, RGM>;
  constexpr int K = ExpCfg<T, RGM>::K;
  constexpr uint32_t RING = X::kRing;
  using RP = RingPos<RING>;
  constexpr int NC = D / 32, NJ = D / 16, ES = (int)sizeof(T), DG = D / 8;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, cls = lane >> 4;
  const int hc = min(col, G - 1);
  char* ring = lds;
  float4* sbuf = reinterpret_cast<float4*>(lds + X::kS);
  float* stl = reinterpret_cast<float*>(lds + X::kStl);
  const int BG = a.B * a.Hkv;
  const bool staged = a.stage_off != nullptr;
  const float qscale = a.qscale;

  // work items per group: lane holds groups 4 lane .. 4 lane + 3
  int cg[4];
  int listed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * lane + i;
    cg[i] = g < BG ? a.exp_count[g] : 0;
    listed += cg[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) listed += __shfl_xor(listed, off);
  const int chunk = item_spans(listed, a.n_a5_wg);
  int ip[4];
  int own = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ip[i] = own;
    own += (cg[i] + chunk - 1) / chunk;
  }
  int incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  const int excl = incl - own;
  const int total = __builtin_amdgcn_readlane(incl, 63);

  for (int c = wid; c < total; c += nwaves) {
    // group of item c: the last lane, then the last of its groups, starting at or before c
    const uint64_t lm = __ballot(excl <= c);
    const int ln = 63 - __builtin_clzll(lm);
    const int lbase = __builtin_amdgcn_readlane(excl, ln);
    int gi = 0, gstart = lbase;
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      const int st = lbase + __builtin_amdgcn_readlane(ip[i], ln);
      if (st <= c) { gi = i; gstart = st; }
    }
    const int g = 4 * ln + gi, lc = c - gstart;
    const int b = g / a.Hkv, kv = g % a.Hkv;
    const int cnt = a.exp_count[g];
    const int j0 = lc * chunk, n = min(cnt, j0 + chunk) - j0;

    // metadata of the item's spans: lane i holds span j0 + i
    ItemMeta im;
    {
      const int32_t* so = a.seg_off + (size_t)b * (a.seg_cap + 1);
      const int jl = j0 + min(lane, n - 1);
      const int mS = a.exp_list[(size_t)g * a.seg_cap + jl];
      im.bits = a.exp_mask[(size_t)g * a.seg_cap + jl];
      int64_t mfo, mgo;
      if (staged) {
        const int64_t* st = a.stage_off + BG + (a.stage_off[g] + jl) * 2;
        mfo = st[0];
        mgo = st[1];
      } else {
        mfo = a.fac_off[(size_t)g * a.seg_cap + mS];
        mgo = a.sg_off[(size_t)g * a.seg_cap + mS];
      }
      im.L = so[mS + 1] - so[mS] - 1;
      im.r = a.rank[(size_t)b * a.seg_cap + mS];
      const char* fb = static_cast<const char*>(staged ? a.stage_fac : a.fac);
      const char* gb = reinterpret_cast<const char*>(staged ? a.stage_sg : a.sg);
      im.sga = reinterpret_cast<uint64_t>(gb + mgo * 4);
      im.fa = reinterpret_cast<uint64_t>(fb + mfo * ES);
    }
    RegionCursor cur;
    cur.n = n;
    cur.sep = a.sep != 0;
    cur.i = 0;
    cur.kind = 0;
    cur.off = 0;
    region_of<T, D, K, RING>(im, 0, 0, cur.sep, cur.base, cur.size);
    uint4 stg[K * kExpStages];
#pragma unroll
    for (int jj = 0; jj < K * kExpStages; ++jj) {
      stg[jj] = gload16(cursor_addr(cur, lane));
      cursor_next<T, D, K, RING>(cur, im);
    }
    uint32_t written = 0, spos = 0;

    // the item's G query rows, kept in LDS (read as the B operand of y)
    T* qs = reinterpret_cast<T*>(lds + X::kQ);
    {
      const T* q0 = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)kv * G) * D;
      for (int i = 8 * lane; i < G * D; i += 8 * 64) st8(qs + i, ld8(q0 + i));
    }
    float m = kNegInf, lsum = 0.0f;
    f32x4_t acc[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) acc[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // one span at a time: its score pass, one rescale, its weight pass
    for (int ca = 0; ca < n; ++ca) {
      const int cb = ca + 1;
      // ---------------- pass 1: scores of the span's tokens
      float cmax = kNegInf;
      int tgb = 0;
      uint32_t s_u1 = 0;   // U of the span read once: the weight pass reads it where this pass left it
      for (int i = ca; i < cb; ++i) {
        const int L = __builtin_amdgcn_readlane(im.L, i), r = __builtin_amdgcn_readlane(im.r, i);
        const int rp = (r + 7) & ~7, rq = (r + 3) & ~3;
        const bool head_on = ((uint32_t)__builtin_amdgcn_readlane(im.bits, i) >> col) & 1u;
        const int RG = (r + 15) >> 4, TG = (L + 15) >> 4;
        const bool once = read_once<T, K, RING>(L, r, cur.sep);
        const uint32_t s_sg = spos;
        const uint32_t s_vk = s_sg + kb_round(8u * (uint32_t)rq);
        const uint32_t s_u = s_vk + (uint32_t)(r * D * ES);
        s_u1 = s_u;
        spos = s_vk + kb_round((uint32_t)((r * D + L * rp + (once ? D * rp : 0)) * ES));
        advance<T, D, K, RING>(stg, written, s_sg + 8u * (uint32_t)rq, cur, im, lane, ring);
        // sigma * gate (zero past r), staged in LDS: the ring holds the entry
        // only until the next advance
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int k = lane + 64 * q2;
          const int kc = min(k, r - 1);
          const float sv = *reinterpret_cast<const float*>(ring + RP::add(RP::of(s_sg), 4u * kc));
          const float gv = *reinterpret_cast<const float*>(ring + RP::add(RP::of(s_sg), 4u * (rq + kc)));
          stl[k] = k < r ? sv * gv : 0.0f;
        }
        // y of rank groups rg, as the B operand of the score product
        Vec4<T> yhi[RGM], ylo[RGM];
#pragma unroll
        for (int rg = 0; rg < RGM; ++rg) {
          if (rg < RG) {
            advance<T, D, K, RING>(stg, written, s_vk + (uint32_t)(min(r, 16 * rg + 16) * D * ES), cur, im, lane, ring);
            const int k = min(16 * rg + col, r - 1);
            const uint32_t b_vk = RP::of(s_vk + (uint32_t)(16 * rg * D * ES));   // this rank group's 16 rows
            f32x4_t yc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) {
              const int pg = (4 * cc + cls + k) & (DG - 1);   // rotated 8-element group
              Vec8<T> qop = ld8(qs + hc * D + 32 * cc + 8 * cls);
              if (col >= G) zero8(qop);
              yc = mma8(rd8<T, RING>(ring, RP::add(b_vk, (uint32_t)(((k - 16 * rg) * D + 8 * pg) * ES))), qop, yc);
            }
            // sigma * gate of ranks 16 rg + 4 cls + v
            const float4 sgv = *reinterpret_cast<const float4*>(stl + 16 * rg + 4 * cls);
            float y[4] = {yc[0] * qscale * sgv.x, yc[1] * qscale * sgv.y, yc[2] * qscale * sgv.z,
                          yc[3] * qscale * sgv.w};
            pack4(y, yhi[rg]);
            if constexpr (ES == 2) {
              float rem[4] = {y[0] - __uint_as_float(yhi[rg].v.x << 16), y[1] - __uint_as_float(yhi[rg].v.x & 0xffff0000u),
                              y[2] - __uint_as_float(yhi[rg].v.y << 16), y[3] - __uint_as_float(yhi[rg].v.y & 0xffff0000u)};
              pack4(rem, ylo[rg]);
            }
          }
        }
        // scores, one token group at a time
        for (int tg = 0; tg < TG; ++tg) {
          advance<T, D, K, RING>(stg, written, s_u + (uint32_t)(min(L, 16 * tg + 16) * rp * ES), cur, im, lane, ring);
          const int trow = min(16 * tg + col, L - 1);
          const uint32_t b_tg = RP::of(s_u + (uint32_t)(16 * tg * rp * ES));   // this token group's 16 rows
          f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int rg = 0; rg < RGM; ++rg) {
            if (rg < RG) {
              const int k0 = min(16 * rg + 4 * cls, rp - 4);
              const Vec4<T> uop = rd4<T>(ring, RP::add(b_tg, (uint32_t)(((trow - 16 * tg) * rp + k0) * ES)));
              sc = mma4(uop, yhi[rg], sc);
              if constexpr (ES == 2) sc = mma4(uop, ylo[rg], sc);
            }
          }
          float4 sv;
          {
            const int t0 = 16 * tg + 4 * cls;
            sv.x = (head_on && t0 + 0 < L) ? sc[0] : kNegInf;
            sv.y = (head_on && t0 + 1 < L) ? sc[1] : kNegInf;
            sv.z = (head_on && t0 + 2 < L) ? sc[2] : kNegInf;
            sv.w = (head_on && t0 + 3 < L) ? sc[3] : kNegInf;
          }
          cmax = fmaxf(cmax, fmaxf(fmaxf(sv.x, sv.y), fmaxf(sv.z, sv.w)));
          if (col < G) sbuf[((tgb + tg) * 4 + cls) * G + col] = sv;
        }
        tgb += TG;
      }
      // chunk maximum per head; rescale the accumulators once
      cmax = rows_max(cmax);
      const float mn = fmaxf(m, cmax);
      if (mn != kNegInf && mn != m) {
        const float alpha = exp2f(m - mn);
        lsum *= alpha;
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) acc[jt] *= alpha;
        m = mn;
      }
      wave_lds_sync();
      // ---------------- pass 2: weights through U^T and W_V
      tgb = 0;
      for (int i = ca; i < cb; ++i) {
        const int L = __builtin_amdgcn_readlane(im.L, i), r = __builtin_amdgcn_readlane(im.r, i);
        const int rp = (r + 7) & ~7, rq = (r + 3) & ~3;
        const int RG = (r + 15) >> 4, TG = (L + 15) >> 4;
        uint32_t s_u;
        if (read_once<T, K, RING>(L, r, cur.sep)) {
          s_u = s_u1;                       // still in the ring; sigma * gate still in LDS
        } else if (!cur.sep) {
          s_u = spos;                       // U | W_V again; sigma * gate still in LDS
          spos = s_u + kb_round((uint32_t)((L * rp + D * rp) * ES));
        } else {
          // separate bases: sigma_V * gate of the value basis, then U_V | W_V
          const uint32_t s_sg = spos;
          s_u = s_sg + kb_round(8u * (uint32_t)rq);
          spos = s_u + kb_round((uint32_t)((L * rp + D * rp) * ES));
          advance<T, D, K, RING>(stg, written, s_sg + 8u * (uint32_t)rq, cur, im, lane, ring);
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) {
            const int k = lane + 64 * q2;
            const int kc = min(k, r - 1);
            const float sv = *reinterpret_cast<const float*>(ring + RP::add(RP::of(s_sg), 4u * kc));
            const float gv = *reinterpret_cast<const float*>(ring + RP::add(RP::of(s_sg), 4u * (rq + kc)));
            stl[k] = k < r ? sv * gv : 0.0f;
          }
        }
        const uint32_t s_w = s_u + (uint32_t)(L * rp * ES);
        f32x4_t am[RGM];
#pragma unroll
        for (int rg = 0; rg < RGM; ++rg) am[rg] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int tg = 0; tg < TG; ++tg) {
          advance<T, D, K, RING>(stg, written, s_u + (uint32_t)(min(L, 16 * tg + 16) * rp * ES), cur, im, lane, ring);
          const float4 sv = sbuf[((tgb + tg) * 4 + cls) * G + hc];
          const uint32_t b_tg = RP::of(s_u + (uint32_t)(16 * tg * rp * ES));   // this token group's 16 rows
          float pr[4];
          pr[0] = (m == kNegInf) ? 0.0f : exp2f(sv.x - m);
          pr[1] = (m == kNegInf) ? 0.0f : exp2f(sv.y - m);
          pr[2] = (m == kNegInf) ? 0.0f : exp2f(sv.z - m);
          pr[3] = (m == kNegInf) ? 0.0f : exp2f(sv.w - m);
          lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
          Vec4<T> pB;
          pack4(pr, pB);
#pragma unroll
          for (int rg = 0; rg < RGM; ++rg) {
            if (rg < RG) {
              const int kc = min(16 * rg + col, rp - 1);
              uint32_t ev[4];
#pragma unroll
              for (int e4 = 0; e4 < 4; ++e4) {
                const int t = min(16 * tg + 4 * cls + e4, L - 1);
                const uint32_t ob = RP::add(b_tg, (uint32_t)(((t - 16 * tg) * rp + kc) * ES));
                if constexpr (ES == 2) ev[e4] = *reinterpret_cast<const uint16_t*>(ring + ob);
                else ev[e4] = *reinterpret_cast<const uint32_t*>(ring + ob);
              }
              Vec4<T> uop;
              if constexpr (ES == 2) uop.v = make_uint2(ev[0] | (ev[1] << 16), ev[2] | (ev[3] << 16));
              else uop.v = make_float4(__uint_as_float(ev[0]), __uint_as_float(ev[1]), __uint_as_float(ev[2]),
                                       __uint_as_float(ev[3]));
              am[rg] = mma4(uop, pB, am[rg]);
            }
          }
        }
        tgb += TG;
#pragma unroll
        for (int rg = 0; rg < RGM; ++rg) {
          if (rg < RG) {
            const int wk = min(16, rp - 16 * rg);
            const uint32_t s_wg = s_w + (uint32_t)(16 * rg * D * ES);
            advance<T, D, K, RING>(stg, written, s_wg + (uint32_t)(D * wk * ES), cur, im, lane, ring);
            const float4 sg4 = *reinterpret_cast<const float4*>(stl + 16 * rg + 4 * cls);
            const float bv[4] = {am[rg][0] * sg4.x, am[rg][1] * sg4.y, am[rg][2] * sg4.z, am[rg][3] * sg4.w};
            Vec4<T> bB;
            pack4(bv, bB);
            const int k0 = min(4 * cls, wk - 4);
            const uint32_t b_wg = RP::of(s_wg);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
              acc[jt] = mma4(rd4<T>(ring, RP::add(b_wg, (uint32_t)(((16 * jt + col) * wk + k0) * ES))), bB, acc[jt]);
          }
        }
      }
      wave_lds_sync();
    }
    // partial of this item: head col, summed over the four lane classes
    lsum = rows_sum(lsum);
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
    wave_lds_sync();
  }
}

// Full-resolution + summary pass (role A) and expanded-span pass (role E).
// With every rank at most 64 both run in one launch: the first n_fx_wg
// workgroups are four independent expanded-span waves each, the rest are
// full-resolution chunks, so the two passes share the machine without a
// second stream; otherwise (wider ranks, or host-resident factors that
// arrive after the full-resolution pass starts) they are separate kernels.
// Three waves per SIMD: with every slot taken by a wave at the start, the
// expanded-span waves leave a third of the slots to full-resolution chunks.
// Waves per SIMD the attention kernels ask for: three for bf16 caches (166
// VGPRs); float32 operands take twice the registers, and a cap of three waves
// would spill them, so float32 kernels take no cap.
template <typename T> struct AttnOcc { static constexpr int kWaves = sizeof(T) == 2 ? 3 : 1; };

template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(AttnOcc<T>::kWaves)))
void attend_fused_kernel(const AttendArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int nx = a.n_fx_wg;
  if ((int)blockIdx.x < nx) {
    const int wave = threadIdx.x >> 6;
    role_expanded<T, D, G, 4>(a, blockIdx.x * 4 + wave, nx * 4, lds + wave * ExpLds<T, G, 4>::kBytes);
  } else {
    role_full_summary<T, D, G>(a, blockIdx.x - nx, lds);
  }
}
template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(AttnOcc<T>::kWaves)))
void attend_full_kernel(const AttendArgs a) {
  extern __shared__ __align__(16) char lds[];
  role_full_summary<T, D, G>(a, blockIdx.x, lds);
}
// Ranks up to 64 (four rank groups in registers): three waves per SIMD.
template <typename T, int D, int G>
__global__ __launch_bounds__(kExpThreads) __attribute__((amdgpu_waves_per_eu(AttnOcc<T>::kWaves)))
void attend_expanded_kernel(const AttendArgs a) {
  extern __shared__ __align__(16) char lds[];
  role_expanded<T, D, G, 4>(a, blockIdx.x, a.n_a5_wg, lds);
}
// Any rank up to kMaxSpan.
template <typename T, int D, int G>
__global__ __launch_bounds__(kExpThreads) void attend_expanded_wide_kernel(const AttendArgs a) {
  extern __shared__ __align__(16) char lds[];
  role_expanded<T, D, G, kMaxSpan / 16>(a, blockIdx.x, a.n_a5_wg, lds);
}

// ================================================================ combine
// One workgroup per (b, h, slice of 32 output elements): D/32 workgroups per
// head, so a launch has B * Hq * D/32 of them.  The 256 threads form 32 rows
// of 8; row r merges partials r, r + 32, ... (four loads in flight per step,
// branch-free online log-sum-exp), each thread owning four of the slice's
// elements.  The 32 row states then merge pairwise in LDS in five halving
// steps.
constexpr int kCombineThreads = 256;
constexpr int kCombineRows = kCombineThreads / 8;
template <int D, int G>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const AttendArgs a) {
  constexpr int NSL = D / 32;
  __shared__ float m_s[kCombineRows], l_s[kCombineRows];
  __shared__ float4 o_s[kCombineRows][8];
  const int bh = blockIdx.x / NSL, sl = blockIdx.x % NSL;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int g = b * a.Hkv + h / G, gi = h % G;
  const int tid = threadIdx.x, row = tid >> 3, c4 = tid & 7;
  int np = a.nch_a4;
  if (a.exp_count) {
    // the item size of the expanded-span pass, from all groups' counts
    __shared__ int red_s[kCombineThreads / 64];
    const int BG = a.B * a.Hkv;
    int listed = tid < BG ? a.exp_count[tid] : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) listed += __shfl_xor(listed, off);
    if ((tid & 63) == 0) red_s[tid >> 6] = listed;
    __syncthreads();
    listed = 0;
#pragma unroll
    for (int w = 0; w < kCombineThreads / 64; ++w) listed += red_s[w];
    const int chunk = item_spans(listed, a.n_a5_wg);
    np += (a.exp_count[g] + chunk - 1) / chunk;
  }
  const float* ml = a.part_ml + (size_t)g * a.P_max * G * 2;
  const float* po = a.part_o + (size_t)g * a.P_max * G * D + 32 * sl + 4 * c4;
  float M = kNegInf, L = 0.0f;
  float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int p0 = row; p0 < np; p0 += 4 * kCombineRows) {
    float2 mlp[4];
    float4 ov[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = min(p0 + u * kCombineRows, np - 1);
      mlp[u] = *reinterpret_cast<const float2*>(ml + (p * G + gi) * 2);
      ov[u] = *reinterpret_cast<const float4*>(po + ((size_t)p * G + gi) * D);
      if (p0 + u * kCombineRows >= np) mlp[u].x = kNegInf;
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < 4; ++u) Mn = fmaxf(Mn, mlp[u].x);
    if (Mn == kNegInf) continue;
    const float sc = exp2f(M - Mn);   // 0 while M is -inf
    L *= sc;
    O = make_float4(O.x * sc, O.y * sc, O.z * sc, O.w * sc);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float f = exp2f(mlp[u].x - Mn);   // 0 for -inf partials
      L += f * mlp[u].y;
      O = make_float4(O.x + f * ov[u].x, O.y + f * ov[u].y, O.z + f * ov[u].z, O.w + f * ov[u].w);
    }
    M = Mn;
  }
  // rows [s, 2s) fold into rows [0, s): reads and writes of one step touch
  // disjoint rows, so one barrier per step orders them
  if (c4 == 0) {
    m_s[row] = M;
    l_s[row] = L;
  }
  o_s[row][c4] = O;
#pragma unroll
  for (int s = kCombineRows / 2; s >= 1; s >>= 1) {
    __syncthreads();
    if (row < s) {
      const float m2 = m_s[row + s], l2 = l_s[row + s];
      const float4 o2 = o_s[row + s][c4];
      const float Mn = fmaxf(M, m2);
      if (Mn != kNegInf) {
        const float f1 = exp2f(M - Mn), f2 = exp2f(m2 - Mn);
        L = L * f1 + l2 * f2;
        O = make_float4(O.x * f1 + o2.x * f2, O.y * f1 + o2.y * f2, O.z * f1 + o2.z * f2, O.w * f1 + o2.w * f2);
        M = Mn;
      }
      if (c4 == 0) {
        m_s[row] = M;
        l_s[row] = L;
      }
      o_s[row][c4] = O;
    }
  }
  if (row == 0) {
    const float inv = 1.0f / L;
    *reinterpret_cast<float4*>(a.out + (size_t)bh * D + 32 * sl + 4 * c4) =
        make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv);
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
    const T* Vk = static_cast<const T*>(a.fac) + a.fac_off[(size_t)g * a.seg_cap + S];  // key part [r][D], rotated groups
    const T* Ub = Vk + (size_t)r * D;             // U [L][rp] (the key basis U_K with separate bases)
    const T* Uv = a.sep ? Ub + (size_t)L * rp : Ub;   // U of the values
    const T* Wv = Uv + (size_t)L * rp;            // value part, 16-rank column blocks [D][wk]
    const int rq = (r + 3) & ~3;
    const float* sgp = a.sg + a.sg_off[(size_t)g * a.seg_cap + S];
    const int row0 = a.tok_off[(size_t)g * (a.seg_cap + 1) + j];
    for (int t = 0; t < L; ++t) {
      float acc[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
      for (int k = 0; k < r; ++k) {
        const float wkey = load1(Ub + (size_t)t * rp + k) * (sgp[k] * sgp[rq + k]);
        const float wval = a.sep ? load1(Uv + (size_t)t * rp + k) * (sgp[2 * rq + k] * sgp[3 * rq + k]) : wkey;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int colj = lane + 64 * c;
          const int kg = k >> 4, wk = min(16, rp - 16 * kg);
          acc[c] += colj < D ? wkey * load1(Vk + (size_t)k * D + (((colj >> 3) + k) % (D / 8)) * 8 + (colj & 7))
                             : wval * load1(Wv + (size_t)kg * 16 * D + (size_t)(colj - D) * wk + (k & 15));
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
#define SEKV_DISPATCH_T(DT, BODY) \
  do {                              \
    if ((DT) == 0) {                \
      using TT = float;             \
      BODY;                         \
    } else {                        \
      using TT = bf16raw;           \
      BODY;                         \
    }                               \
  } while (0)
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

// ================================================================ online sealing
// Pages: German explainer, "Methodik" parts 1 (boundaries at high surprisal,
// spans between anchors) and 2 (per-span summary and low-rank basis); the
// Chinese explainer, "方法论" parts 1 and 2.  During decode the newest token
// is appended to the full-resolution tail, and when the token that just got
// decided closes a span, that span is summarised and factored in place.
//
// Build kernel: one workgroup per (b, kv) (256 threads).  Every workgroup
// appends its new key/value row; a workgroup whose sequence seals a span also
//   - summarises it: kbar, vbar = sum_t w_t k_t, w_t v_t in fp64, t in order
//     (the weights w_t = s_t / sum s come from the host), stored rounded;
//   - computes its routing key rho = P^T (r / |r|), r = P kbar (fp64, index
//     order), or the key scale 1 / |r|;
//   - factors M = [K_body | V_body] (L x 2d): the Gram matrix G = M M^T in
//     fp64, its eigenvectors by cyclic two-sided Jacobi with all L/2 disjoint
//     rotations of a round-robin step applied at once (rows, then columns and
//     the eigenvector matrix), then for the r largest eigenvalues
//     u_j = the eigenvector, w_j = M^T u_j, sigma_j = |w_j|, W column w_j /
//     sigma_j; each column pair's sign makes u's largest-magnitude entry
//     positive (first on ties);
//   - writes the factor block, the sigma|gate entry and its CSR entries.
// Arithmetic whose result the host builder also produces (summaries, routing
// key, key scale) follows the builder's operation order with contraction off,
// so both give the same stored bits.
template <typename T>
__device__ __forceinline__ double ld_el(const void* p, size_t i) {
  if constexpr (sizeof(T) == 2) return (double)__uint_as_float(uint32_t(static_cast<const bf16raw*>(p)[i]) << 16);
  else return (double)static_cast<const float*>(p)[i];
}
// fp64 -> f32 (nearest even) -> storage type (bf16: nearest even on the upper 16 bits)
template <typename T>
__device__ __forceinline__ void st_el(void* p, size_t i, double x) {
  const float f = (float)x;
  if constexpr (sizeof(T) == 2) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    static_cast<bf16raw*>(p)[i] = (bf16raw)(u >> 16);
  } else {
    static_cast<float*>(p)[i] = f;
  }
}
// value (entry e, dim j) of a (b, kv) block of 32-entry transposed tiles
__device__ __forceinline__ size_t vt_at(size_t e, int j, int D) { return ((e / 32) * D + j) * 32 + e % 32; }

constexpr int kSealThreads = 256;
constexpr int kJacobiSweeps = 40;
constexpr double kJacobiTol = 1e-24;   // (off-diagonal / diagonal Frobenius norm)^2 at convergence

// What one span's build needs and where it goes.
struct SpanJob {
  int L, r, S;            // body length, rank, span index
  size_t g;               // (b, kv) group
  const double* w;        // body weights [L]
  const float* P;         // routing projection of the KV head [D][D]
  const float* gt;        // gates [r]
  int64_t fb, gb;         // factor block and sigma|gate entry (pool element offsets)
  double* vscr;           // [kMaxSpan][kMaxSpan] eigenvectors when L > vlds_max
};
struct SpanDst {
  int seg_cap, vlds_max;
  void* sum_k; void* sum_v; void* rho; float* key_scale;
  void* fac; float* sg;
};
// Body rows in the full-resolution rows of a (b, kv) (keys row-major, values
// in transposed 32-entry tiles), from row row0 on.
template <typename T, int D>
struct RowsFull {
  const T* fk; const T* fv; int row0;
  __device__ double k(int t, int c) const { return ld_el<T>(fk, (size_t)(row0 + t) * D + c); }
  __device__ double v(int t, int c) const { return ld_el<T>(fv, vt_at(row0 + t, c, D)); }
};
// Body rows in the prefill keys and values [T][D] of a (b, kv), from token t0 on.
template <typename T, int D>
struct RowsRaw {
  const T* kp; const T* vp; int t0;
  __device__ double k(int t, int c) const { return ld_el<T>(kp, (size_t)(t0 + t) * D + c); }
  __device__ double v(int t, int c) const { return ld_el<T>(vp, (size_t)(t0 + t) * D + c); }
};

// One span: summaries, routing key or key scale, factors and sigma|gate entry
// (all threads of the workgroup; lds: seal_lds_bytes(L) bytes).
template <typename T, int D, class Rows>
__device__ void build_span(const Rows& rows, const SpanJob& j, const SpanDst& o, char* lds, double* s_kbar,
                           double* s_vbar, double* s_r, double (*s_red)[2]) {
#pragma clang fp contract(off)
  const int L = j.L, r = j.r, S = j.S;
  const size_t g = j.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int stiles = (o.seg_cap + 31) / 32;
  __syncthreads();   // LDS of the previous span is no longer read
  const int rp = (r + 7) & ~7, rq = (r + 3) & ~3;
  const double* w = j.w;
  // ---- summaries (thread j: one dimension, tokens in order)
  for (int jj = tid; jj < D; jj += kSealThreads) {
    double kb = 0.0, vb = 0.0;
    for (int t = 0; t < L; ++t) {
      kb += w[t] * rows.k(t, jj);
      vb += w[t] * rows.v(t, jj);
    }
    s_kbar[jj] = kb;
    s_vbar[jj] = vb;
    st_el<T>(o.sum_k, (g * o.seg_cap + S) * D + jj, kb);
    st_el<T>(static_cast<T*>(o.sum_v) + g * stiles * 32 * D, vt_at(S, jj, D), vb);
  }
  __syncthreads();
  // ---- routing key
  const float* P = j.P;
  for (int i = tid; i < D; i += kSealThreads) {
    double acc = 0.0;
    for (int j = 0; j < D; ++j) acc += (double)P[(size_t)i * D + j] * s_kbar[j];
    s_r[i] = acc;
  }
  __syncthreads();
  if (tid == 0) {
    double nn = 0.0;
    for (int i = 0; i < D; ++i) nn += s_r[i] * s_r[i];
    s_red[0][0] = sqrt(nn);
  }
  __syncthreads();
  const double nrm = s_red[0][0];
  __syncthreads();
  if (o.rho) {
    for (int jj = tid; jj < D; jj += kSealThreads) {
      double acc = 0.0;
      for (int i = 0; i < D; ++i) acc += (double)P[(size_t)i * D + jj] * (nrm > 0 ? s_r[i] / nrm : 0.0);
      st_el<T>(o.rho, (g * o.seg_cap + S) * D + jj, acc);
    }
  }
  if (o.key_scale && tid == 0) o.key_scale[g * o.seg_cap + S] = nrm > 0 ? (float)(1.0 / nrm) : 0.0f;

  // ---- factors: Gram matrix and Jacobi
  const int n2 = (L + 1) & ~1;                    // even order (a dummy index past L when L is odd)
  const bool vlds = L <= o.vlds_max;
  double* G = reinterpret_cast<double*>(lds);     // [n2][n2]
  double* V = vlds ? G + (size_t)n2 * n2 : j.vscr;   // [n2][n2]
  double* rot = G + (size_t)n2 * n2 * (vlds ? 2 : 1);                             // [n2/2]: c, s, (p, q)
  auto mval = [&](int t, int c) -> double { return c < D ? rows.k(t, c) : rows.v(t, c - D); };
  for (int e = tid; e < n2 * n2; e += kSealThreads) {
    const int i = e / n2, j = e % n2;
    double acc = 0.0;
    if (i < L && j < L && i <= j)
      for (int c = 0; c < 2 * D; ++c) acc += mval(i, c) * mval(j, c);
    if (i <= j) {
      G[(size_t)i * n2 + j] = acc;
      G[(size_t)j * n2 + i] = acc;
    }
    V[(size_t)i * n2 + j] = i == j ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
    // stop once the off-diagonal mass is negligible against the diagonal's
    double off = 0.0, dia = 0.0;
    for (int e = tid; e < n2 * n2; e += kSealThreads) {
      const double x = G[e];
      if (e / n2 == e % n2) dia += x * x;
      else off += x * x;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      off += __shfl_xor(off, o);
      dia += __shfl_xor(dia, o);
    }
    if (lane == 0) {
      s_red[wave][0] = off;
      s_red[wave][1] = dia;
    }
    __syncthreads();
    double offt = 0.0, diat = 0.0;
    for (int w2 = 0; w2 < kSealThreads / 64; ++w2) {
      offt += s_red[w2][0];
      diat += s_red[w2][1];
    }
    __syncthreads();   // s_red is rewritten by the next sweep
    if (!(offt > kJacobiTol * diat)) break;
    for (int st = 0; st < n2 - 1; ++st) {
      // round-robin step st: pair k joins (n2 - 1, st) for k = 0, else
      // ((st + k) mod (n2 - 1), (st - k) mod (n2 - 1))
      for (int k = tid; k < n2 / 2; k += kSealThreads) {
        int p = k == 0 ? n2 - 1 : (st + k) % (n2 - 1);
        int q = k == 0 ? st : (st - k + n2 - 1) % (n2 - 1);
        if (p > q) { const int x = p; p = q; q = x; }
        double c = 1.0, s = 0.0;
        const double apq = G[(size_t)p * n2 + q];
        if (q < L && apq != 0.0) {
          const double tau = (G[(size_t)q * n2 + q] - G[(size_t)p * n2 + p]) / (2.0 * apq);
          const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        rot[4 * k + 0] = c;
        rot[4 * k + 1] = s;
        reinterpret_cast<int*>(rot + 4 * k + 2)[0] = p;
        reinterpret_cast<int*>(rot + 4 * k + 2)[1] = q;
      }
      __syncthreads();
      // rows p, q of G  (G <- J^T G)
      for (int e = tid; e < (n2 / 2) * n2; e += kSealThreads) {
        const int k = e / n2, col = e % n2;
        const double c = rot[4 * k], s = rot[4 * k + 1];
        const int p = reinterpret_cast<const int*>(rot + 4 * k + 2)[0], q = reinterpret_cast<const int*>(rot + 4 * k + 2)[1];
        const double gp = G[(size_t)p * n2 + col], gq = G[(size_t)q * n2 + col];
        G[(size_t)p * n2 + col] = c * gp - s * gq;
        G[(size_t)q * n2 + col] = s * gp + c * gq;
      }
      __syncthreads();
      // columns p, q of G and of V  (G <- G J, V <- V J)
      for (int e = tid; e < (n2 / 2) * n2; e += kSealThreads) {
        const int k = e / n2, row = e % n2;
        const double c = rot[4 * k], s = rot[4 * k + 1];
        const int p = reinterpret_cast<const int*>(rot + 4 * k + 2)[0], q = reinterpret_cast<const int*>(rot + 4 * k + 2)[1];
        const double gp = G[(size_t)row * n2 + p], gq = G[(size_t)row * n2 + q];
        G[(size_t)row * n2 + p] = c * gp - s * gq;
        G[(size_t)row * n2 + q] = s * gp + c * gq;
        const double vp = V[(size_t)row * n2 + p], vq = V[(size_t)row * n2 + q];
        V[(size_t)row * n2 + p] = c * vp - s * vq;
        V[(size_t)row * n2 + q] = s * vp + c * vq;
      }
      __syncthreads();
    }
  }
  // ---- the r largest eigenvalues: position of eigenvalue i in descending order
  int* perm = reinterpret_cast<int*>(s_r);         // D doubles hold kMaxSpan ints; s_r is no longer read
  __syncthreads();
  for (int i = tid; i < L; i += kSealThreads) {
    const double li = G[(size_t)i * n2 + i];
    int pos = 0;
    for (int j = 0; j < L; ++j) {
      const double lj = G[(size_t)j * n2 + j];
      pos += (lj > li || (lj == li && j < i)) ? 1 : 0;
    }
    if (pos < r) perm[pos] = i;
  }
  __syncthreads();
  void* fac = o.fac;
  const int64_t fb = j.fb, gb = j.gb;
  const float* gt = j.gt;
  // one wave per factor column jc: sign, U column, W column, sigma
  for (int jc = wave; jc < rp; jc += kSealThreads / 64) {
    if (jc >= r) {
      for (int t = lane; t < L; t += 64) st_el<T>(fac, fb + (int64_t)r * D + (int64_t)t * rp + jc, 0.0);
      for (int col = lane; col < D; col += 64) {
        const int gg = jc / 16, wk = min(16, rp - 16 * gg);
        st_el<T>(fac, fb + (int64_t)r * D + (int64_t)L * rp + (int64_t)gg * 16 * D + (int64_t)col * wk + (jc % 16), 0.0);
      }
      continue;
    }
    const int src = perm[jc];
    // sign: largest |u_t|, first on ties
    double best = -1.0;
    int bi = 0;
    for (int t = lane; t < L; t += 64) {
      const double x = fabs(V[(size_t)t * n2 + src]);
      if (x > best) { best = x; bi = t; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int oi = __shfl_xor(bi, o);
      if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    const double sgn = V[(size_t)bi * n2 + src] < 0.0 ? -1.0 : 1.0;
    for (int t = lane; t < L; t += 64) st_el<T>(fac, fb + (int64_t)r * D + (int64_t)t * rp + jc, sgn * V[(size_t)t * n2 + src]);
    // w = M^T u (2d entries, 4 per lane for d = 128), sigma = |w|
    double wv[2 * D / 64];
    double ss = 0.0;
#pragma unroll
    for (int m = 0; m < 2 * D / 64; ++m) {
      const int col = lane + 64 * m;
      double acc = 0.0;
      for (int t = 0; t < L; ++t) acc += mval(t, col) * (sgn * V[(size_t)t * n2 + src]);
      wv[m] = acc;
      ss += acc * acc;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const double sig = sqrt(ss);
    const double inv = sig > 0.0 ? 1.0 / sig : 0.0;
#pragma unroll
    for (int m = 0; m < 2 * D / 64; ++m) {
      const int col = lane + 64 * m;
      if (col < D) {
        const int ng = D / 8;
        st_el<T>(fac, fb + (int64_t)jc * D + (int64_t)(((col / 8) + jc) % ng) * 8 + (col % 8), wv[m] * inv);
      } else {
        const int cv = col - D, gg = jc / 16, wk = min(16, rp - 16 * gg);
        st_el<T>(fac, fb + (int64_t)r * D + (int64_t)L * rp + (int64_t)gg * 16 * D + (int64_t)cv * wk + (jc % 16),
                 wv[m] * inv);
      }
    }
    if (lane == 0) {
      o.sg[gb + jc] = (float)sig;
      o.sg[gb + rq + jc] = gt[jc];
    }
  }
  for (int jc = r + tid; jc < rq; jc += kSealThreads) {
    o.sg[gb + jc] = 0.0f;
    o.sg[gb + rq + jc] = 0.0f;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kSealThreads) void seal_build_kernel(const SealArgs a) {
  extern __shared__ __align__(16) char lds[];
  __shared__ double s_kbar[D], s_vbar[D], s_r[D];
  __shared__ double s_red[kSealThreads / 64][2];
  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t g = (size_t)b * a.Hkv + kv;
  const SealDesc& ds = a.desc[b];
  const int ftiles = (a.full_cap + 31) / 32;
  T* fk = static_cast<T*>(a.full_k) + g * a.full_cap * D;
  T* fv = static_cast<T*>(a.full_v) + g * ftiles * 32 * D;
  // the new token at full-resolution row n_full_old
  for (int j = tid; j < D; j += kSealThreads) {
    fk[(size_t)ds.n_full_old * D + j] = static_cast<const T*>(a.k_new)[g * D + j];
    fv[vt_at(ds.n_full_old, j, D)] = static_cast<const T*>(a.v_new)[g * D + j];
  }
  if (!ds.sealed) return;
  const int S = ds.n_seg_old;
  SpanJob job;
  job.L = ds.L; job.r = ds.r; job.S = S; job.g = g;
  job.w = a.weights + ds.w_off;
  job.P = a.route_proj + (size_t)kv * D * D;
  job.gt = a.gates + ds.g_off + (size_t)kv * ds.r;
  job.fb = ds.fac_base + (int64_t)kv * ds.fac_stride;
  job.gb = ds.sg_base + (int64_t)kv * ds.sg_stride;
  job.vscr = a.vscratch + g * kMaxSpan * kMaxSpan;
  SpanDst dst{a.seg_cap, a.vlds_max, a.sum_k, a.sum_v, a.rho, a.key_scale, a.fac, a.sg};
  build_span<T, D>(RowsFull<T, D>{fk, fv, ds.row0}, job, dst, lds, s_kbar, s_vbar, s_r, s_red);
  // ---- CSR entries of the new span
  if (tid == 0) {
    a.fac_off[g * a.seg_cap + S] = job.fb;
    a.sg_off[g * a.seg_cap + S] = job.gb;
    if (kv == 0) {
      a.seg_off[(size_t)b * (a.seg_cap + 1) + S + 1] = ds.h_new;
      a.rank[(size_t)b * a.seg_cap + S] = ds.r;
    }
  }
}

// Prefill build (every span of every (b, kv)): a persistent grid, workgroup w
// taking spans w, w + grid, ... of the list (b, then kv, then span), each
// with its own eigenvector scratch; the plan's offsets are already on the
// device.
template <typename T, int D>
__global__ __launch_bounds__(kSealThreads) void build_spans_kernel(const BuildArgs a) {
  extern __shared__ __align__(16) char lds[];
  __shared__ double s_kbar[D], s_vbar[D], s_r[D];
  __shared__ double s_red[kSealThreads / 64][2];
  const SpanDst dst{a.seg_cap, a.vlds_max, a.sum_k, a.sum_v, a.rho, a.key_scale, a.fac, a.sg};
  for (int it = blockIdx.x; it < a.n_items; it += gridDim.x) {
    int b = 0;
    while (b + 1 < a.B && a.item_base[b + 1] <= it) ++b;
    const int ns = a.n_seg[b];
    const int rel = it - a.item_base[b];
    const int kv = rel / ns, S = rel % ns;
    const size_t g = (size_t)b * a.Hkv + kv;
    const int32_t* so = a.seg_off + (size_t)b * (a.seg_cap + 1);
    const int t0 = so[S] + 1;
    SpanJob job;
    job.L = so[S + 1] - t0;
    job.r = a.rank[(size_t)b * a.seg_cap + S];
    job.S = S;
    job.g = g;
    job.w = a.weights + (size_t)b * a.T + t0;
    job.P = a.route_proj + (size_t)kv * D * D;
    job.gt = a.gates + (g * a.seg_cap + S) * (size_t)a.gate_stride;
    job.fb = a.fac_off[g * a.seg_cap + S];
    job.gb = a.sg_off[g * a.seg_cap + S];
    job.vscr = a.vscratch + (size_t)blockIdx.x * kMaxSpan * kMaxSpan;
    const T* kp = static_cast<const T*>(a.k) + g * a.T * D;
    const T* vp = static_cast<const T*>(a.v) + g * a.T * D;
    build_span<T, D>(RowsRaw<T, D>{kp, vp, t0}, job, dst, lds, s_kbar, s_vbar, s_r, s_red);
  }
}

// Full-resolution rows of the prefill (sink, anchors, tail) of a (b, kv).
template <typename T, int D>
__global__ __launch_bounds__(kSealThreads) void build_full_kernel(const BuildArgs a) {
  const int kv = blockIdx.x % a.Hkv, b = blockIdx.x / a.Hkv;
  const size_t g = (size_t)b * a.Hkv + kv;
  const int ns = a.n_seg[b], nf = a.n_full[b], sink = a.n_sink;
  const int32_t* so = a.seg_off + (size_t)b * (a.seg_cap + 1);
  const int ftiles = (a.full_cap + 31) / 32;
  T* fk = static_cast<T*>(a.full_k) + g * a.full_cap * D;
  T* fv = static_cast<T*>(a.full_v) + g * ftiles * 32 * D;
  const T* kp = static_cast<const T*>(a.k) + g * a.T * D;
  const T* vp = static_cast<const T*>(a.v) + g * a.T * D;
  for (int e = threadIdx.x + blockIdx.y * kSealThreads; e < nf * D; e += kSealThreads * gridDim.y) {
    const int row = e / D, c = e % D;
    const int t = row < sink ? row : row < sink + ns ? so[row - sink] : so[ns] + (row - sink - ns);
    fk[(size_t)row * D + c] = kp[(size_t)t * D + c];
    fv[vt_at(row, c, D)] = vp[(size_t)t * D + c];
  }
}

// Compaction of a sealing sequence's full-resolution rows: the body rows
// [row0, row0 + L) leave, rows [row0 + L, n_full_old + 1) move down by L.
// Destinations lie below sources, so ascending chunks staged through LDS
// (all of a chunk read before any of it is written) never overwrite a row
// still to be read.
constexpr int kSealChunk = 64;
template <typename T, int D>
__global__ __launch_bounds__(kSealThreads) void seal_compact_kernel(const SealArgs a) {
  __shared__ T buf[kSealChunk * D];
  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const SealDesc& ds = a.desc[b];
  if (!ds.sealed) return;
  const size_t g = (size_t)b * a.Hkv + kv;
  const int ftiles = (a.full_cap + 31) / 32;
  T* fk = static_cast<T*>(a.full_k) + g * a.full_cap * D;
  T* fv = static_cast<T*>(a.full_v) + g * ftiles * 32 * D;
  const int L = ds.L, s0 = ds.row0 + L, s1 = ds.n_full_old + 1;
  for (int c0 = s0; c0 < s1; c0 += kSealChunk) {
    const int nrow = min(kSealChunk, s1 - c0);
    for (int e = tid; e < nrow * D; e += kSealThreads) buf[e] = fk[(size_t)(c0 + e / D) * D + e % D];
    __syncthreads();
    for (int e = tid; e < nrow * D; e += kSealThreads) fk[(size_t)(c0 - L + e / D) * D + e % D] = buf[e];
    __syncthreads();
    for (int e = tid; e < nrow * D; e += kSealThreads) buf[e] = fv[vt_at(c0 + e / D, e % D, D)];
    __syncthreads();
    for (int e = tid; e < nrow * D; e += kSealThreads) fv[vt_at(c0 - L + e / D, e % D, D)] = buf[e];
    __syncthreads();
  }
  // the vacated rows past the new end hold zeros (padding stays finite)
  for (int e = tid; e < L * D; e += kSealThreads) {
    const int row = s1 - L + e / D, j = e % D;
    fk[(size_t)row * D + j] = T(0);
    fv[vt_at(row, j, D)] = T(0);
  }
}

// ---------------------------------------------------------------- route scratch
// State of sekv_route_noalloc: the route workspace (tickets and status words)
// held in a file-scope device array.  Every GPU the library runs on holds its
// own copy until the process ends, and every call on that GPU shares it.  In
// host code the array's name is only a stand-in: its device address comes
// from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) uint32_t scratch[kRouteScratchBytes / sizeof(uint32_t)];

}  // namespace

hipError_t route_scratch_address(int device, void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[device]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // the route state must start at zero; every route call leaves it zero
    e = hipMemset(p, 0, kRouteScratchBytes);
    if (e != hipSuccess) return e;
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

// Timed launches: a non-null start (stop) event is recorded at the start (the
// end) of the kernel's own execution.
#define SEKV_LAUNCH(KERNEL, GRID, BLOCK, SHMEM, S, EV0, EV1, ARG)                                  \
  do {                                                                                             \
    if ((EV0) || (EV1)) hipExtLaunchKernelGGL(KERNEL, dim3(GRID), dim3(BLOCK), SHMEM, S, EV0, EV1, 0, ARG); \
    else KERNEL<<<dim3(GRID), dim3(BLOCK), SHMEM, S>>>(ARG);                                       \
  } while (0)

hipError_t launch_route(const RouteArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int G = a.Hq / a.Hkv;
  dim3 grid(a.nblk, a.Hkv, a.B);
  if (a.fold) {
    const int n = a.B * a.Hq * a.D;
    hipEvent_t none = nullptr;
    SEKV_DISPATCH_T(a.dtype, ({
      if (a.D == 64) SEKV_LAUNCH((fold_query_kernel<TT, 64>), (n + 255) / 256, 256, 0, s, ev0, none, a);
      else SEKV_LAUNCH((fold_query_kernel<TT, 128>), (n + 255) / 256, 256, 0, s, ev0, none, a);
    }));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    SEKV_DISPATCH(a.dtype, a.D, G,
                  ({ SEKV_LAUNCH((route_kernel<TT, DD, GG, true>), grid, kRouteThreads, 0, s, none, ev1, a); }));
  } else {
    SEKV_DISPATCH(a.dtype, a.D, G,
                  ({ SEKV_LAUNCH((route_kernel<TT, DD, GG, false>), grid, kRouteThreads, 0, s, ev0, ev1, a); }));
  }
  return hipGetLastError();
}

hipError_t route_resident_blocks(const RouteArgs& a, int device, int* blocks) {
  const int G = a.Hq / a.Hkv;
  int per_cu = 0;
  hipError_t e = hipSuccess;
  SEKV_DISPATCH(a.dtype, a.D, G,
                (e = a.fold ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, route_kernel<TT, DD, GG, true>,
                                                                            kRouteThreads, 0)
                            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, route_kernel<TT, DD, GG, false>,
                                                                            kRouteThreads, 0)));
  if (e != hipSuccess) return e;
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return e;
  *blocks = per_cu * cus;
  return hipSuccess;
}

hipError_t launch_attend_full(const AttendArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int G = a.Hq / a.Hkv;
  if (a.n_a4_wg == 0) return hipSuccess;
  SEKV_DISPATCH(a.dtype, a.D, G,
                ({ SEKV_LAUNCH((attend_full_kernel<TT, DD, GG>), a.n_a4_wg, kAttnThreads, (AttnLds<DD, GG>::kRoleA), s,
                               ev0, ev1, a); }));
  return hipGetLastError();
}

hipError_t launch_attend_expanded(const AttendArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int G = a.Hq / a.Hkv;
  if (a.n_a5_wg == 0) return hipSuccess;
  SEKV_DISPATCH(a.dtype, a.D, G, ({
                  if (a.max_rank <= 64)
                    SEKV_LAUNCH((attend_expanded_kernel<TT, DD, GG>), a.n_a5_wg, kExpThreads, (ExpLds<TT, GG, 4>::kBytes),
                                s, ev0, ev1, a);
                  else
                    SEKV_LAUNCH((attend_expanded_wide_kernel<TT, DD, GG>), a.n_a5_wg, kExpThreads,
                                (ExpLds<TT, GG, kMaxSpan / 16>::kBytes), s, ev0, ev1, a);
                }));
  return hipGetLastError();
}

hipError_t launch_attend_fused(const AttendArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int G = a.Hq / a.Hkv;
  if (a.n_fx_wg + a.n_a4_wg == 0) return hipSuccess;
  SEKV_DISPATCH(a.dtype, a.D, G,
                ({ SEKV_LAUNCH((attend_fused_kernel<TT, DD, GG>), a.n_fx_wg + a.n_a4_wg, kAttnThreads,
                               (AttnLds<DD, GG>::kRoleA > 4 * ExpLds<TT, GG, 4>::kBytes ? AttnLds<DD, GG>::kRoleA
                                                                                        : 4 * ExpLds<TT, GG, 4>::kBytes),
                               s, ev0, ev1, a); }));
  return hipGetLastError();
}

hipError_t launch_combine(const AttendArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  SEKV_DISPATCH_D(a.D, G, (combine_kernel<DD, GG><<<a.B * a.Hq * (DD / 32), kCombineThreads, 0, s>>>(a)));
  return hipGetLastError();
}

hipError_t launch_seal(const SealArgs& a, size_t lds_bytes, hipStream_t s) {
  const dim3 grid(a.Hkv, a.B);
  hipError_t e = hipSuccess;
  if (a.dtype == 0) {
    if (a.D == 64) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&seal_build_kernel<float, 64>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
      if (e == hipSuccess) seal_build_kernel<float, 64><<<grid, kSealThreads, lds_bytes, s>>>(a);
    } else {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&seal_build_kernel<float, 128>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
      if (e == hipSuccess) seal_build_kernel<float, 128><<<grid, kSealThreads, lds_bytes, s>>>(a);
    }
  } else {
    if (a.D == 64) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&seal_build_kernel<bf16raw, 64>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
      if (e == hipSuccess) seal_build_kernel<bf16raw, 64><<<grid, kSealThreads, lds_bytes, s>>>(a);
    } else {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&seal_build_kernel<bf16raw, 128>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
      if (e == hipSuccess) seal_build_kernel<bf16raw, 128><<<grid, kSealThreads, lds_bytes, s>>>(a);
    }
  }
  if (e != hipSuccess) return e;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.dtype == 0) {
    if (a.D == 64) seal_compact_kernel<float, 64><<<grid, kSealThreads, 0, s>>>(a);
    else seal_compact_kernel<float, 128><<<grid, kSealThreads, 0, s>>>(a);
  } else {
    if (a.D == 64) seal_compact_kernel<bf16raw, 64><<<grid, kSealThreads, 0, s>>>(a);
    else seal_compact_kernel<bf16raw, 128><<<grid, kSealThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

#define SEKV_DISPATCH_TD(DT, DIM, BODY)                                     \
  do {                                                                      \
    if ((DT) == 0) {                                                        \
      using TT = float;                                                     \
      if ((DIM) == 64) { constexpr int DD = 64; BODY; }                     \
      else { constexpr int DD = 128; BODY; }                                \
    } else {                                                                \
      using TT = bf16raw;                                                   \
      if ((DIM) == 64) { constexpr int DD = 64; BODY; }                     \
      else { constexpr int DD = 128; BODY; }                                \
    }                                                                       \
  } while (0)

hipError_t launch_build(const BuildArgs& a, int grid, size_t lds_bytes, hipStream_t s) {
  hipError_t e = hipSuccess;
  SEKV_DISPATCH_TD(a.dtype, a.D, ({
                     build_full_kernel<TT, DD><<<dim3(a.B * a.Hkv, 8), kSealThreads, 0, s>>>(a);
                     e = hipGetLastError();
                     if (e == hipSuccess && a.n_items > 0) {
                       e = hipFuncSetAttribute(reinterpret_cast<const void*>(&build_spans_kernel<TT, DD>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
                       if (e == hipSuccess) build_spans_kernel<TT, DD><<<grid, kSealThreads, lds_bytes, s>>>(a);
                     }
                   }));
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t build_resident_blocks(const BuildArgs& a, size_t lds_bytes, int device, int* blocks) {
  int per_cu = 0;
  hipError_t e = hipSuccess;
  SEKV_DISPATCH_TD(a.dtype, a.D, ({
                     e = hipFuncSetAttribute(reinterpret_cast<const void*>(&build_spans_kernel<TT, DD>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
                     if (e == hipSuccess)
                       e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, build_spans_kernel<TT, DD>,
                                                                        kSealThreads, lds_bytes);
                   }));
  if (e != hipSuccess) return e;
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return e;
  *blocks = per_cu * cus;
  return hipSuccess;
}

// ---------------------------------------------------------------- device factor cache fill
// Each workgroup copies whole items (grid-strided over the list): 16 bytes per
// lane, four loads in flight per lane before their stores, so that many reads
// of the pinned host pools are outstanding on the bus at once.
constexpr int kFillThreads = 256;
constexpr int kFillGrid = 2048;
__global__ __launch_bounds__(kFillThreads) void cache_fill_kernel(const FillItem* items, int n, char* arena) {
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const FillItem it = items[i];
    const int nf = (int)(it.fac_bytes >> 4), tot = nf + (int)(it.sg_bytes >> 4);
    const uint4* sf = reinterpret_cast<const uint4*>(it.src_fac);
    const uint4* sg = reinterpret_cast<const uint4*>(it.src_sg);
    uint4* dst = reinterpret_cast<uint4*>(arena + it.dst);
    for (int k0 = 0; k0 < tot; k0 += 4 * kFillThreads) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + u * kFillThreads + (int)threadIdx.x;
        if (k < tot) v[u] = k < nf ? sf[k] : sg[k - nf];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + u * kFillThreads + (int)threadIdx.x;
        if (k < tot) dst[k] = v[u];
      }
    }
  }
}

hipError_t launch_cache_fill(const FillItem* items, int n, char* arena, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (n <= 0) return hipSuccess;
  const int grid = std::min(n, kFillGrid);
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(cache_fill_kernel, dim3(grid), dim3(kFillThreads), 0, s, ev0, ev1, 0, items, n, arena);
  else
    cache_fill_kernel<<<grid, kFillThreads, 0, s>>>(items, n, arena);
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
