// common.hpp -- types, bf16 helpers and MFMA wrappers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row keys of the plan: a row that takes no delta, and a row that is not
// written at all (outside every segment / an expert id out of range).
constexpr int kSkip = -1;
constexpr int kDrop = -2;

enum Mode : int { kModeDecode = 0, kModeSegmented = 1, kModeMoe = 2, kModeMoeGrouped = 3 };

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// f32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ u16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u16)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A(16x32) * B(32x16) + C.  Lane l holds A row l%16, B column l%16, each
// with k = 8*(l/16) .. +7; D column l%16, rows 4*(l/16) .. +3.
__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 z4() { return make_uint4(0u, 0u, 0u, 0u); }

// 16 bytes from device memory.  The global address space is explicit (set
// through an integer: a direct pointer cast is folded back to a generic
// pointer): a pointer read from a route table would otherwise give a flat
// load, which may reach LDS, and the compiler then waits for it before every
// LDS access.
typedef unsigned int u32x4n __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16(const void *p) {
  const u32x4n v = *(const __attribute__((address_space(1))) u32x4n *)(uintptr_t)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t pack2(u16 lo, u16 hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// s_waitcnt with only the vector-memory counter constrained (<= n).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Waits until at most `stages_younger` stages of `PER` DMA instructions each
// (0 <= stages_younger <= MAXS), plus X other vector-memory operations
// issued after the stage waited for, are still in flight.
template <int PER, int MAXS, int X = 0>
__device__ __forceinline__ void wait_stages(int stages_younger) {
  if constexpr (MAXS >= 6) { if (stages_younger >= 6) { wait_vmcnt<6 * PER + X>(); return; } }
  if constexpr (MAXS >= 5) { if (stages_younger == 5) { wait_vmcnt<5 * PER + X>(); return; } }
  if constexpr (MAXS >= 4) { if (stages_younger == 4) { wait_vmcnt<4 * PER + X>(); return; } }
  if constexpr (MAXS >= 3) { if (stages_younger == 3) { wait_vmcnt<3 * PER + X>(); return; } }
  if constexpr (MAXS >= 2) { if (stages_younger == 2) { wait_vmcnt<2 * PER + X>(); return; } }
  if constexpr (MAXS >= 1) { if (stages_younger == 1) { wait_vmcnt<PER + X>(); return; } }
  wait_vmcnt<X>();
}

// One LDS-DMA instruction: 16 bytes per lane from `g` into the wave's 1 KB
// LDS block at byte address `lds` (lane l lands at lds + 16 l).  Issued as
// assembly so that the compiler adds no waits of its own around the LDS
// reads that follow; every wait on these transfers is explicit.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory");
}

// Device-coherent 16-byte accesses (cache policy sc1) through a buffer
// resource over [base, base + bytes): stores write through to the memory
// side that every XCD shares and loads read from there, so results pass
// between workgroups on different XCDs without an L2-wide writeback or
// invalidate.  A wave's consecutive lanes at consecutive 16-byte offsets
// make whole-line transfers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
constexpr int kCachePolicySc1 = 16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// The byte offset is voff (per lane) + soff (the same for the whole wave).
__device__ __forceinline__ void st16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)voff, (int)soff,
                                         kCachePolicySc1);
}
__device__ __forceinline__ f32x4 ld16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCachePolicySc1));
}

// The same with 4 bytes per lane (lane l lands at lds + 4 l).
__device__ __forceinline__ void dma4(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// Workgroup barrier that the compiler may not move memory accesses across.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The route-resolve rule of every entry point: slot in range, both table
// entries non-NULL, scale non-zero.  Returns the table index or kSkip.  The
// three entries of an in-range slot are read together, one round trip, and
// the rule applied to what they hold.
__device__ __forceinline__ int resolve_slot(int slot, int expert, int max_loras, int n_experts,
                                            const void *const *a_table,
                                            const void *const *b_table,
                                            const float *scale_table) {
  if (slot < 0 || slot >= max_loras) return kSkip;
  const int idx = slot * n_experts + expert;
  const void *ae = a_table[idx], *be = b_table[idx];
  const float sc = scale_table[slot];
  __builtin_amdgcn_sched_barrier(0);  // all three loads out before the first compare
  return ((ae == nullptr) | (be == nullptr) | (sc == 0.0f)) ? kSkip : idx;
}

// Routing inputs of one call, in the form the caller handed them over.
struct Routing {
  int mode;                 // Mode
  const int32_t *seq_slot;  // decode, moe grouped: [n]
  const int32_t *seg_indptr;  // segmented: [n_seg+1]
  const int32_t *seg_slot;    // segmented: [n_seg]
  int n_seg;
  const int32_t *indices;     // moe: [n]
  const int32_t *token_slot;  // moe: [n / top_k]
  int top_k;
  int n_experts;              // 1 unless moe
  const int32_t *expert_offsets;  // moe grouped: [n_experts+1], rows sorted by expert
};

struct RouteDev {
  const void *const *a_table;
  const void *const *b_table;
  const float *scale_table;
  int max_loras;
  int n_experts;
  int R;  // max_rank
};

// resolve_slot on a one-expert table (index = slot), handing back the
// entries it read: A, B and the scale of a resolved slot.
__device__ __forceinline__ int resolve_slot_entries(int slot, const RouteDev &rd, const void *&ae, const void *&be,
                                                    float &sc) {
  ae = be = nullptr;
  sc = 0.f;
  if (slot < 0 || slot >= rd.max_loras) return kSkip;
  ae = rd.a_table[slot];
  be = rd.b_table[slot];
  sc = rd.scale_table[slot];
  __builtin_amdgcn_sched_barrier(0);  // all three loads out before the first compare
  return ((ae == nullptr) | (be == nullptr) | (sc == 0.0f)) ? kSkip : slot;
}

// Segment of row r (binary search over seg_indptr), or -1.
__device__ __forceinline__ int segment_of(const int32_t *indptr, int n_seg, int r) {
  if (n_seg <= 0 || r < indptr[0] || r >= indptr[n_seg]) return -1;
  int lo = 0, hi = n_seg - 1;  // find last g with indptr[g] <= r
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (indptr[mid] <= r) lo = mid; else hi = mid - 1;
  }
  // empty segments share a start; the last one with indptr[g] <= r and r <
  // indptr[g+1] is the owner
  return lo;
}

// Per-row routing: the W group (expert) and the pair table index, or
// kSkip (base only) / kDrop (row not written).  `scale_idx` gets the scale
// table index (the adapter).
__device__ __forceinline__ int row_route(const Routing &rt, const RouteDev &rd, bool has_lora,
                                         int r, int *group, int *scale_idx) {
  *group = 0;
  *scale_idx = 0;
  int slot = -1, expert = 0;
  if (rt.mode == kModeDecode) {
    slot = rt.seq_slot ? rt.seq_slot[r] : -1;
  } else if (rt.mode == kModeSegmented) {
    int g = segment_of(rt.seg_indptr, rt.n_seg, r);
    if (g < 0) return kDrop;
    slot = rt.seg_slot[g];
  } else if (rt.mode == kModeMoeGrouped) {
    expert = segment_of(rt.expert_offsets, rt.n_experts, r);
    if (expert < 0) return kDrop;
    *group = expert;
    if (!has_lora) return kSkip;  // seq_slot may be NULL for a base-only call
    slot = rt.seq_slot[r];
  } else {
    expert = rt.indices[r];
    if (expert < 0 || expert >= rt.n_experts) return kDrop;
    *group = expert;
    if (!has_lora) return kSkip;  // token_slot may be NULL for a base-only call
    slot = rt.token_slot[r / rt.top_k];
  }
  if (!has_lora) return kSkip;
  *scale_idx = slot;
  return resolve_slot(slot, expert, rd.max_loras, rd.n_experts, rd.a_table, rd.b_table,
                      rd.scale_table);
}

}  // namespace lora
