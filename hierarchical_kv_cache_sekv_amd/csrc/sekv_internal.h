// Internal launch interface between the host runtime (sekv_host.cpp) and the
// gfx950 kernels (sekv_kernels.hip).  Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace sekv {

constexpr int kMaxBatch = 64;        // per-sequence sizes travel in kernel arguments
constexpr int kMaxGroups = 256;      // batch * kv heads handled by one decode launch
constexpr int kMaxSpan = 128;        // longest span body / highest rank the kernels hold
constexpr int kRouteThreads = 256;   // spans per route workgroup (one lane per span)
constexpr int kAttnThreads = 256;    // four waves per attention workgroup
constexpr int kExpChunk = 8;         // most expanded spans per work item of the expanded-span kernel
constexpr int kExpChunkMin = 2;      // fewest (the item size adapts to the listed count, see item_spans)
constexpr int kExpThreads = 64;      // one wave per expanded-span workgroup
constexpr int kExpWaves = 2048;      // most waves (workgroups) of one expanded-span launch
constexpr int kMaxDevices = 64;      // devices with a route scratch address
constexpr size_t kRouteScratchBytes = size_t(1) << 20;  // static route state of sekv_route_noalloc

struct RouteArgs {
  int dtype;                 // 0 f32, 1 bf16
  int B, Hq, Hkv, D, seg_cap, nblk;
  int nblk_cap;              // status words per group: ceil(seg_cap / kRouteThreads)
  int use_ticket;            // 1: tiles by per-group tickets (grid larger than the GPU holds at once)
  int n_seg[kMaxBatch];
  const void* q;             // [B][Hq][D]
  const float* theta;        // [B][Hq]
  const void* rho;           // [B][Hkv][seg_cap][D]
  uint32_t* ticket;          // [B*Hkv] workspace, zero between calls
  uint32_t* status;          // [B*Hkv][nblk_cap] workspace, zero between calls
  int fold;                  // 1: folded routing (keys = kbar in `rho`, scaled by key_scale)
  const float* key_scale;    // [B][Hkv][seg_cap]
  const double* foldm;       // [Hkv][D][D]
  float* qfold;              // [B][Hq][D] workspace: folded queries
  int32_t* exp_list;         // [B][Hkv][seg_cap]
  uint8_t* exp_mask;         // [B][Hkv][seg_cap]
  int32_t* exp_count;        // [B][Hkv]
};

struct AttendArgs {
  int dtype;
  int B, Hq, Hkv, D, seg_cap, full_cap;
  int n_full[kMaxBatch];
  int n_seg[kMaxBatch];
  int tiles_a4;              // 32-entry tiles per full-res/summary workgroup
  int nch_a4;                // chunks (workgroups) per (b, kv) for that pass: nch_full full-res, then summary
  int nch_full;              // chunks of full-resolution tiles per (b, kv)
  int a4_lo, a4_n;           // this launch's chunks of each (b, kv): [a4_lo, a4_lo + a4_n); n_a4_wg = B*Hkv*a4_n
  int chunk_major;           // 1: workgroups in chunk-major order over the groups, 0: group-major
  int P_max;                 // partial slots per (b, kv)
  int n_a5_wg;               // workgroups (one wave each) of the expanded-span kernel
  int n_fx_wg;               // workgroups (four expanded-span waves each) of the fused launch
  int max_rank;              // largest span rank (selects the expanded-span kernel's register tiling)
  int sep;                   // 1: separate key and value bases (factor block and sigma|gate layout)
  int n_a4_wg;               // workgroups of the full-res/summary kernel
  float qscale;              // log2(e) / sqrt(D)
  const void* q;
  const void* full_k; const void* full_v;
  const void* sum_k; const void* sum_v;
  const int32_t* seg_off; const int32_t* rank;
  const int64_t* fac_off; const int64_t* sg_off;   // device pools (staged == nullptr)
  const void* fac; const float* sg;
  const int64_t* stage_off;  // staged host-resident mode: [B*Hkv] first entry of each group, then (fac, sg) offsets per listed entry
  const void* stage_fac; const float* stage_sg;
  const int32_t* exp_list; const uint8_t* exp_mask;
  const int32_t* exp_count;  // nullptr: no expanded spans (dense decode)
  float* part_ml;            // [B*Hkv][P_max][G][2]
  float* part_o;             // [B*Hkv][P_max][G][D]
  float* out;                // [B][Hq][D]
};

struct ReconArgs {
  int dtype;
  int sep;                   // 1: separate key and value bases
  int B, Hkv, D, seg_cap;
  const int32_t* seg_off; const int32_t* rank;
  const int64_t* fac_off; const int64_t* sg_off;
  const void* fac; const float* sg;
  const int32_t* exp_list; const int32_t* exp_count;
  int32_t* tok_off;          // [B][Hkv][seg_cap+1]
  float* k_out; float* v_out;
  int T;
};

// One decode step of online sealing, per sequence b (written by the host).
struct SealDesc {
  int sealed;          // 1: the newly decided token closes a span this step
  int n_full_old;      // full-resolution rows before the new token is appended
  int n_seg_old;       // sealed spans before this step (the new span's index)
  int h_old, h_new;    // its anchor and its closing head (tokens)
  int L, r;            // body length and rank of the new span
  int row0;            // full-resolution row of the first body token
  int w_off, g_off;    // offsets of its weights (doubles) and gates (floats, [Hkv][r])
  int64_t fac_base, fac_stride;   // factor block of KV head kv at fac_base + kv * fac_stride
  int64_t sg_base, sg_stride;     // sigma|gate entry of KV head kv at sg_base + kv * sg_stride
};

struct SealArgs {
  int dtype;
  int B, Hkv, D, seg_cap, full_cap;
  int rank_cap_unused;
  int vlds_max;        // largest L whose eigenvector matrix fits in LDS next to the Gram matrix
  const SealDesc* desc;        // [B] device
  const double* weights;       // device
  const float* gates;          // device
  const void* k_new; const void* v_new;   // [B][Hkv][D]
  const float* route_proj;     // [Hkv][D][D] device
  void* full_k; void* full_v; void* sum_k; void* sum_v; void* rho; float* key_scale;
  void* fac; float* sg;
  int32_t* seg_off; int32_t* rank; int64_t* fac_off; int64_t* sg_off;
  double* vscratch;            // [B][Hkv][kMaxSpan][kMaxSpan] eigenvectors of spans longer than vlds_max
};

// Prefill build on the GPU (every span of the plan).
struct BuildArgs {
  int dtype;
  int B, Hkv, D, T, seg_cap, full_cap, n_sink, gate_stride, vlds_max;
  int n_items;                 // spans of all (b, kv)
  int item_base[kMaxBatch];    // first item of sequence b (its Hkv groups' spans follow in kv order)
  int n_seg[kMaxBatch], n_full[kMaxBatch];
  const int32_t* seg_off; const int32_t* rank; const int64_t* fac_off; const int64_t* sg_off;   // device
  const double* weights;       // [B][T] surprisal weight of each body token within its span
  const float* route_proj;     // [Hkv][D][D]
  const float* gates;          // [B][Hkv][seg_cap][gate_stride]
  const void* k; const void* v;   // [B][Hkv][T][D]
  void* full_k; void* full_v; void* sum_k; void* sum_v; void* rho; float* key_scale;
  void* fac; float* sg;
  double* vscratch;            // [grid][kMaxSpan][kMaxSpan]
};

// One factor block copied into the device factor cache: the span's factor
// block (fac_bytes) and its sigma|gate entry (sg_bytes) go to the cache slot
// at arena byte offset dst, the entry right after the block.  Sources are
// device-visible addresses (pinned host pools); every size and address is a
// multiple of 16 bytes.
struct FillItem {
  uint64_t src_fac, src_sg;
  uint64_t dst;
  uint32_t fac_bytes, sg_bytes;
};

// ev0/ev1: optional start/stop events of the kernel itself (both or neither)
hipError_t launch_route(const RouteArgs& a, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// Route workgroups the device holds at once (occupancy x compute units).
hipError_t route_resident_blocks(const RouteArgs& a, int device, int* blocks);
// Device address of the static route state on `device` (must be current);
// taken and zero-filled on the first call per device.
hipError_t route_scratch_address(int device, void** ptr);
hipError_t launch_attend_full(const AttendArgs& a, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_attend_expanded(const AttendArgs& a, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_attend_fused(const AttendArgs& a, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_combine(const AttendArgs& a, hipStream_t s);
hipError_t launch_reconstruct(const ReconArgs& a, hipStream_t s);
// Online sealing: append the new token, build the sealed spans (summaries,
// routing keys, factors, CSR entries), then compact the full-resolution tails.
// lds_bytes: dynamic LDS of the build kernel.
hipError_t launch_seal(const SealArgs& a, size_t lds_bytes, hipStream_t s);
// Prefill build: full-resolution rows, then every span (persistent grid of
// `grid` workgroups, dynamic LDS lds_bytes).
hipError_t launch_build(const BuildArgs& a, int grid, size_t lds_bytes, hipStream_t s);
// Workgroups of the span build kernel resident at once with lds_bytes of dynamic LDS.
hipError_t build_resident_blocks(const BuildArgs& a, size_t lds_bytes, int device, int* blocks);
// Copy n cache fills into the arena; `items` is a device-visible address (the
// pinned host workspace); the arena must hold every dst + fac_bytes +
// sg_bytes (checked by the caller).
hipError_t launch_cache_fill(const FillItem* items, int n, char* arena, hipStream_t s, hipEvent_t ev0 = nullptr,
                             hipEvent_t ev1 = nullptr);

}  // namespace sekv
