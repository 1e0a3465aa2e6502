// k_decode.hip -- the decode-shaped apply (n <= 64 rows): base contraction,
// split-K reduction, expand and fold in one launch, after the shrink.
//
//     y_i = W x_i + s_q B_q (A_q x_i),   q = the slot row i resolves to
//
// (ferrox-core "weight_matrix/lora.rs", module doc; atlas "lora_delta.rs",
// apply_lora_bgmv doc: the shrink t = A x, then the expand-and-fold).  At
// decode sizes the cost is reading W once; on this chip a stream of W runs
// fastest as loads of whole 128-byte lines into registers, all of a
// workgroup's share requested early.  The layout:
//
//  * workgroup (g, z) owns output tile g (TO = 16 NSW outputs) over k range z
//    (kKR = 512 columns; S = ceil(k_in / 512) ranges).  Its x rows over the
//    range go to LDS once (LDS-DMA, whole lines, XOR-swizzled), requested by
//    its first four waves, which count themselves in on an LDS word once
//    theirs have landed.  Each of its W waves owns SPW slices of 16 outputs
//    (two on 128-output tiles): it requests their W rows x 512 columns
//    (sixteen 16-byte loads per lane and slice, whole lines, through buffer
//    resources: half of them, then, once x has landed, the other half),
//    then, one 64-column stage at a time as the loads land, lays
//    the stage out in a wave-private LDS buffer and runs the MFMAs of its
//    outputs against every row block of x, each x fragment read from LDS
//    serving all its slices (LDS traffic, not the MFMAs, bounds this phase).
//    No block-wide barrier sits in the stream.
//  * split-K: every slice's f32 partial [16 outputs x rows] goes to the
//    workspace through device-coherent stores; contributor z finalizes the
//    slices z, z + S, ... of its tile once all S contributors of the tile have
//    stored theirs (a bounded wait on the tile's arrival count; the
//    contributors of a tile are consecutive workgroups, so in-order dispatch
//    always runs them together).  Finalizing sums the S partials in range
//    order, adds s_q B_q t_i in f32 (ranks in order), an adapter stack's
//    further levels, and rounds y once.
//  * the shrink: when the pool's units (slot x 16-rank block) fit, wave 0
//    of the workgroups of the first few tiles ("carriers") takes one unit
//    over its k range.  The unit's 16 A rows are requested
//    into MFMA operand layout before the workgroup's W (the W waves wait at
//    a block barrier until then: on this chip a request made behind a CU's
//    W stream waits for most of it), then contracted with the x rows of the
//    slot's rows only, gathered from LDS 16 at a time: a piece of t for
//    those rows (pieces by pool slot, so no route is needed to place them),
//    stored while W still streams.  A range's last unit counts the range
//    into every tile's arrival word, and every tile waits for its S
//    contributors and the S ranges before it finalizes.  Carriers never wait
//    before they count themselves in; the carrier workgroups are the first
//    of the launch and at most half the device's CUs, so they all run
//    whatever else is resident.  A larger pool takes a prep launch (k_prep.hip) that leaves
//    t in the workspace first.
//
// Skipped rows (slot < 0 or past the pool, NULL table entry, zero scale) get
// no delta arithmetic: their y is the sum of the same partials in the same
// order as a base-only call's.  Every output element's reduction order is a
// function of k_in alone (ranges of 512 columns, stages of 64, two 32-column
// MFMA steps per stage), so it does not depend on n_out, on the batch's other
// rows or on the routing.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

namespace {

constexpr int kKR = kDecodeKR;       // columns per k range
constexpr int kNSt = kKR / 64;       // 64-column stages per range
// s_waitcnt with only the vector-memory counter constrained: at most n
// operations still in flight (0 <= n <= 32).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define LORA_W(N) case N: wait_vmcnt<N>(); break;
    LORA_W(1) LORA_W(2) LORA_W(3) LORA_W(4) LORA_W(5) LORA_W(6) LORA_W(7) LORA_W(8)
    LORA_W(9) LORA_W(10) LORA_W(11) LORA_W(12) LORA_W(13) LORA_W(14) LORA_W(15) LORA_W(16)
    LORA_W(17) LORA_W(18) LORA_W(19) LORA_W(20) LORA_W(21) LORA_W(22) LORA_W(23) LORA_W(24)
    LORA_W(25) LORA_W(26) LORA_W(27) LORA_W(28) LORA_W(29) LORA_W(30) LORA_W(31) LORA_W(32)
#undef LORA_W
    default: wait_vmcnt<0>(); break;
  }
}

// The wait for a tile's contributors gives up after this many ticks of the
// 100 MHz real-time counter (0.5 s: only a fault elsewhere gets there), so
// every wave reaches the end of the kernel; the tile's outputs are then NaN.
constexpr uint64_t kTileWaitTicks = 50000000ull;

// A tile's partials when its contributors all run on one XCD
// (DecodeArgs::xcd_local), cache policy sc0: a store lands in that XCD's L2
// and a load misses the CU's L1 and reads the L2.
constexpr int kCachePolicySc0 = 1;
__device__ __forceinline__ void st16_l2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)voff, (int)soff, kCachePolicySc0);
}
__device__ __forceinline__ f32x4 ld16_l2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCachePolicySc0));
}

// Polls a counter until it reaches `target` or `ticks` pass.  Each poll is
// a device-scope atomic load, which reads past this XCD's L2.
__device__ __forceinline__ unsigned poll(unsigned *ctr) {
  return __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned spin_until(unsigned *ctr, unsigned target, uint64_t ticks) {
  unsigned v = poll(ctr);
  if (v < target) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (v < target && __builtin_amdgcn_s_memrealtime() - t0 < ticks) {
      __builtin_amdgcn_s_sleep(4);
      v = poll(ctr);
    }
  }
  asm volatile("" ::: "memory");
  return v;
}

// The compiler barriers keep every memory access on its side of the atomic:
// the stores before it have completed (the caller waited for them) and the
// loads after it depend on what it returned.
__device__ __forceinline__ unsigned wave_atomic_add(unsigned *p, unsigned v) {
  unsigned old = 0;
  asm volatile("" ::: "memory");
  if ((threadIdx.x & 63) == 0) old = __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = (unsigned)__builtin_amdgcn_readfirstlane((int)old);
  asm volatile("" ::: "memory");
  return old;
}
__device__ __forceinline__ void wave_store0(unsigned *p) {
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A slice: 16 rows of a row-major matrix (W's outputs, or A's ranks) over
// the k range [kb, ke), as sixteen whole-line loads per lane: load 2 st + h
// carries rows 8 h .. 8 h + 7 (lane l: row 8 h + l / 8, 16-byte chunk l % 8)
// of stage st.  The loads go through a buffer resource over the slice's
// rows (scalar) with one 32-bit offset per lane and row group; rows past the
// matrix read its last row instead.
struct Slice {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off[2];  // byte offset of this lane's chunk at column kb, rows 8 h + l / 8
};
__device__ __forceinline__ Slice make_slice(const u16 *base, int row_stride, int row0, int rows, int kb) {
  const int lane = threadIdx.x & 63;
  Slice sl;
  // every argument is uniform over the wave; readfirstlane lets the compiler
  // see that, so the resource lives in scalar registers (a per-lane resource
  // would turn every load into a loop over the distinct values)
  const uint64_t b64 = (uint64_t)(uintptr_t)(base + (size_t)__builtin_amdgcn_readfirstlane(row0) * row_stride);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b64), hi = __builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  sl.rs = __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)(((uint64_t)hi << 32) | lo), 0, 0x7ffffff0, 0x00020000);
  const int last = rows - 1 - row0;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    sl.off[h] = (uint32_t)((min(8 * h + (lane >> 3), last) * row_stride + kb + (lane & 7) * 8) * 2);
  return sl;
}
__device__ __forceinline__ uint4 buf_ld16(const __amdgpu_buffer_rsrc_t &rs, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
}
// A W wave's SPW slices (consecutive 16-row blocks) over a range, stage by
// stage: load (st SPW + s) 2 + h is slice s's rows 8 h .. 8 h + 7 of stage
// st, so the stages land in order.  A whole range (512 columns): stages
// [ST0, ST1), the stage step in the instruction's immediate offset.
template <int SPW, int ST0, int ST1>
__device__ __forceinline__ void issue_full(const Slice (&sl)[SPW], uint4 (&v)[2 * SPW * kNSt]) {
#pragma unroll
  for (int st = ST0; st < ST1; ++st)
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) v[(st * SPW + s) * 2 + h] = buf_ld16(sl[s].rs, sl[s].off[h] + st * 128);
}
// The last, shorter range: its nst stages; a chunk past ke reads column kb
// and is zeroed once it lands.
template <int SPW>
__device__ __forceinline__ void issue_part(const Slice (&sl)[SPW], int kb, int ke, int nst,
                                           uint4 (&v)[2 * SPW * kNSt]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int st = 0; st < kNSt; ++st) {
    if (st < nst) {
      const bool past = kb + st * 64 + (lane & 7) * 8 >= ke;
#pragma unroll
      for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          v[(st * SPW + s) * 2 + h] =
              buf_ld16(sl[s].rs, past ? sl[s].off[h] - (lane & 7) * 16 : sl[s].off[h] + st * 128);
    }
  }
}

// The MFMAs of a W wave's slices against the x rows in LDS, stage by stage
// as its loads land (on a shorter range `extra` more vector-memory
// operations were issued after all of them).  Each x fragment read from LDS
// serves the wave's SPW slices.  acc[s][b] = D[16 rows of slice s][16 x rows
// of row block b]: lane l holds slice rows 4 (l / 16) .. +3 of x row
// 16 b + l % 16; every element accumulates stage by stage, two 32-column
// steps each.  On a whole range every wait is a constant: a wait whose count
// is known only at run time leaves the compiler unsure which loads have
// landed, and it then waits for all of them before the first stage.
template <int NB, int SPW, bool FULL>
__device__ __forceinline__ void slice_mma(uint4 (&v)[2 * SPW * kNSt], const uint4 *xs, uint4 *wb, int kb, int ke,
                                          int nst, f32x4 (&acc)[SPW][NB], int extra = 0) {
  const int lane = threadIdx.x & 63;
  constexpr int XR = 16 * NB;
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[s][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < kNSt; ++st) {
    if (FULL || st < nst) {
      if (FULL) {  // a constant once the loop is unrolled
        wait_vm(2 * SPW * (kNSt - 1 - st));
      } else {
        wait_vm(2 * SPW * (nst - 1 - st) + extra);
        if (kb + st * 64 + (lane & 7) * 8 >= ke) {
#pragma unroll
          for (int q = 0; q < 2 * SPW; ++q) v[st * 2 * SPW + q] = z4();
        }
      }
      uint4 *buf = wb + (st & 1) * 128 * SPW;
#pragma unroll
      for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 8 * h + (lane >> 3);
          buf[s * 128 + r * 8 + ((lane & 7) ^ ((r >> 1) & 7))] = v[(st * SPW + s) * 2 + h];
        }
      const uint4 *xst = xs + st * XR * 8;
      uint4 af[SPW][2], xf[2][NB];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 4 * h + (lane >> 4);
        const int r = lane & 15;
#pragma unroll
        for (int s = 0; s < SPW; ++s) af[s][h] = buf[s * 128 + r * 8 + (c ^ ((r >> 1) & 7))];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int rx = 16 * b + (lane & 15);
          xf[h][b] = xst[rx * 8 + (c ^ ((rx >> 1) & 7))];
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int s = 0; s < SPW; ++s) acc[s][b] = mfma16(af[s][h], xf[h][b], acc[s][b]);
    }
  }
}

// A W wave that requested x rows counts itself in on an LDS word once they
// have landed (NAFTER vector memory operations were issued after them); every
// W wave waits there for the NXW waves that request x before its first
// stage reads x.
template <int NAFTER, int NXW>
__device__ __forceinline__ void x_ready(int wv, int *ctr) {
  if (wv < NXW) {
    wait_vmcnt<NAFTER>();
    asm volatile("" ::: "memory");
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < NXW) __builtin_amdgcn_s_sleep(1);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float *slice_partial(const DecodeArgs &p, int g, int z, int j) {
  return p.partials + ((size_t)(g * p.S + z) * kDecodeSlices + j) * kDecodeSliceFloats;
}

// A row's route by the rule of every entry point: slot in the pool, both
// table entries non-NULL, scale non-zero; otherwise *bq = NULL.
struct RowRoute {
  const u16 *bq;
  float sig;
  int slot;
};
__device__ __forceinline__ RowRoute row_route_decode(const DecodeArgs &p, int i) {
  RowRoute r{nullptr, 0.f, kSkip};
  const int slot = p.has_lora && i < p.n ? p.seq_slot[i] : -1;
  const bool in = slot >= 0 && slot < p.rd.max_loras;
  const void *a = in ? p.rd.a_table[slot] : nullptr;
  const void *b = in ? p.rd.b_table[slot] : nullptr;
  const float sc = in ? p.rd.scale_table[slot] : 0.f;
  if (a != nullptr && b != nullptr && sc != 0.0f) {
    r.bq = (const u16 *)b;
    r.sig = sc;
    r.slot = slot;
  }
  return r;
}

// A table entry read through the scalar cache: the vector memory path of a
// CU is queued behind its share of W, the scalar one is not.  `idx` is
// uniform over the wave; the read goes through the constant address space,
// so the compiler issues it as a scalar load and waits for it where the
// value is first used.
__device__ __forceinline__ uint64_t scalar_entry(const void *const *tab, int idx) {
  const __attribute__((address_space(4))) uint64_t *t =
      (const __attribute__((address_space(4))) uint64_t *)(uintptr_t)tab;
  return t[__builtin_amdgcn_readfirstlane(idx)];
}

// One finalization item, by one wave: slice j of tile g, row block b.  Every
// contributor's partial (and, with the shrink in this launch, every piece
// of t) has been stored; rr is the route of this lane's row.  Every load the
// item needs goes out before any arithmetic: the S partials and B over the
// first 16 ranks (PRE: a wave's first item's were requested before the wait
// for the tile's arrivals, in bpre).  t comes from the workgroup's LDS copy
// (tsh, rows from r0 on, summed from the pieces by the unit waves; they count
// themselves in on *tready), or as a prep launch left it.
template <bool PRE, bool XL>
__device__ __forceinline__ void finalize_item(const DecodeArgs &p, const StackFold &f, const RowRoute &rr, int g, int j,
                                              int b, const float *tsh, int r0, const int *tready,
                                              const uint4 (&bpre)[4][2]) {
  const int lane = threadIdx.x & 63;
  const int i = 16 * b + (lane & 15);
  const int ic = min(i, p.n - 1);
  const int o = g * p.tile_out + 16 * j + 4 * (lane >> 4);
  const bool routed = rr.bq != nullptr;
  const int R = p.R;
  // the S partials in range order, eight in flight at a time
  constexpr int kG = 8;
  f32x4 part[kG];
  auto load_parts = [&](int z0) {
#pragma unroll
    for (int zz = 0; zz < kG; ++zz)
      part[zz] = z0 + zz >= p.S ? f32x4{0.f, 0.f, 0.f, 0.f}
                 : XL ? ld16_l2(coherent_rsrc(slice_partial(p, g, z0 + zz, j), kDecodeSliceFloats * 4),
                                         (uint32_t)(b * 64 + lane) * 16, 0)
                               : ld16_coherent(coherent_rsrc(slice_partial(p, g, z0 + zz, j), kDecodeSliceFloats * 4),
                                               (uint32_t)(b * 64 + lane) * 16, 0);
  };
  load_parts(0);
  // B_q[o .. o+3] over the first 16 ranks: it goes out with the partials
  const bool expand = routed && i < p.n && o < p.n_out;
  const u16 *bq = expand ? rr.bq + (size_t)o * R : nullptr;
  uint4 b0[4][2];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) b0[c][h] = PRE ? bpre[c][h] : expand ? ldg16(bq + (size_t)c * R + 8 * h) : z4();
  if (p.unit_tiles > 0) {  // the unit waves' sums of t are in LDS
    while (__hip_atomic_load(tready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < 2) __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
  }
  if (i >= p.n || o >= p.n_out) return;
  float d[4] = {0.f, 0.f, 0.f, 0.f};
  if (routed) {  // B_q[o .. o+3] t_i, ranks in order, 16 at a time
    const float *ti = p.unit_tiles > 0 ? tsh + (i - r0) * R : p.t + (size_t)i * R;
    for (int r0 = 0; r0 < R; r0 += 16) {  // 16 ranks: every B load of the step in flight together
      uint4 bb[4][2];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) bb[c][h] = r0 == 0 ? b0[c][h] : ldg16(bq + (size_t)c * R + r0 + 8 * h);
      float tr[16];
#pragma unroll
      for (int e = 0; e < 16; e += 4) {
        const f32x4 t4 = *(const f32x4 *)(ti + r0 + e);
        tr[e] = t4[0];
        tr[e + 1] = t4[1];
        tr[e + 2] = t4[2];
        tr[e + 3] = t4[3];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w[4] = {bb[c][h].x, bb[c][h].y, bb[c][h].z, bb[c][h].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d[c] += bf2f((u16)(w[e] & 0xffffu)) * tr[8 * h + 2 * e];
            d[c] += bf2f((u16)(w[e] >> 16)) * tr[8 * h + 2 * e + 1];
          }
        }
    }
  }
  f32x4 v = part[0];
#pragma unroll
  for (int zz = 1; zz < kG; ++zz)
    if (zz < p.S) v += part[zz];
  for (int z0 = kG; z0 < p.S; z0 += kG) {  // k_in past 4096: more ranges, in order
    load_parts(z0);
#pragma unroll
    for (int zz = 0; zz < kG; ++zz)
      if (z0 + zz < p.S) v += part[zz];
  }
  if (routed) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = v[c] + rr.sig * d[c];
  }
  // an adapter stack's further levels, in level order, from their final t
  if (f.n_levels > 0 && p.has_lora) {
    for (int l = 0; l < f.n_levels; ++l) {
      const StackLevel &L = f.lv[l];
      const int sl = L.seq_slot[i];
      const bool in = sl >= 0 && sl < L.max_loras;
      const void *ta = in ? L.a_table[sl] : nullptr;
      const void *tb2 = in ? L.b_table[sl] : nullptr;
      const float sc = in ? L.scale_table[sl] : 0.f;
      if (ta == nullptr || tb2 == nullptr || sc == 0.0f) continue;
      const u16 *bl = (const u16 *)tb2 + (size_t)o * L.R;
      const float *tl = L.t + (size_t)i * L.R;
      float e4[4] = {0.f, 0.f, 0.f, 0.f};
      for (int r0 = 0; r0 < L.R; r0 += 8) {
        float tr[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) tr[c] = tl[r0 + c];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 bb = ldg16(bl + (size_t)c * L.R + r0);
          const uint32_t w[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            e4[c] += bf2f((u16)(w[e] & 0xffffu)) * tr[2 * e];
            e4[c] += bf2f((u16)(w[e] >> 16)) * tr[2 * e + 1];
          }
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = v[c] + sc * e4[c];
    }
  }
  *(uint2 *)(p.y + (size_t)i * p.y_row_stride + o) =
      make_uint2(pack2(f2bf(v[0]), f2bf(v[1])), pack2(f2bf(v[2]), f2bf(v[3])));
}

}  // namespace

// NB: 16-row blocks of the batch (n <= 16 NB); NSW: slices of 16 outputs
// per tile (TO = 16 NSW outputs), two per W wave on 128-output tiles (each x
// fragment read from LDS then serves two slices) and one on 64-output tiles
// (their launches are small: more waves keep more loads in flight); XL: the
// tile's contributors on one XCD, their partials through its L2
// (DecodeArgs::xcd_local; its own instantiation, so that the other keeps the
// code it had).  A
// workgroup's waves by role (a SIMD issues the requests of its older waves
// first):
//  * waves 0 and 1, the unit waves: wave 0 carries a unit of the shrink on
//    the first unit_tiles tiles; after the tile's wait both sum the pieces
//    of t for the workgroup's finalization rows;
//  * waves 2 .. NSW / SPW + 1, the W waves, stream W;
//  * waves 0 .. 3 also request the range's x rows into LDS; each of them,
//    once its own have landed, counts itself in on an LDS word that the W
//    waves watch before their first stage reads x (no block barrier between
//    the W loads and the first MFMAs).
template <int NB, int NSW, bool XL>
__global__ __launch_bounds__((NSW / (NSW >= 8 ? 2 : 1) + 2) * 64) void decode_kernel(DecodeArgs p, StackFold f) {
  constexpr int XR = 16 * NB;
  constexpr int NSL = NSW;      // slices per tile
  constexpr int SPW = NSW >= 8 ? 2 : 1;  // slices per W wave
  constexpr int NWW = NSW / SPW;         // W waves
  constexpr int NXW = 4;        // waves that request x
  __shared__ __attribute__((aligned(16))) uint4 xs[kNSt * XR * 8];
  __shared__ __attribute__((aligned(16))) uint4 wb[NWW][2 * 128 * SPW];
  __shared__ int s_rows[2][64];
  __shared__ int s_done, s_ready, s_xready, s_tready;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int b8 = blockIdx.x >> 3;
  const int g = XL ? (b8 / p.S) * 8 + (blockIdx.x & 7) : blockIdx.x / p.S;
  const int z = XL ? b8 % p.S : blockIdx.x % p.S;
  const int kb = z * kKR, ke = min(kb + kKR, p.k_in);
  const int nst = (ke - kb + 63) / 64;
  const int o0 = g * p.tile_out;
  const bool full = ke - kb == kKR;  // eight whole stages
  const int RB = p.R / 16;
  if (tid == 0) {
    s_done = 0;
    s_ready = 0;
    s_xready = 0;
    s_tready = 0;
  }
  __syncthreads();
  // Finalization items of the tile: (row block b, slice j), item m = b NSL + j
  // over the batch's row blocks; contributor z takes items [it_lo, it_hi), so
  // its items share one or two row blocks (rows r0 ..), whose t the unit
  // waves sum from the pieces once for the workgroup.
  const int T = max(1, (p.n + 15) / 16) * NSL;
  const int it_lo = z * T / p.S, it_hi = (z + 1) * T / p.S;
  const int r0 = 16 * (it_lo / NSL);

  // x rows over the range: stages st = wave, wave + NXW, ... (2 NB DMAs each)
  for (int st = wave; wave < NXW && st < nst; st += NXW) {
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) {
      const int r = 8 * i + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int k = kb + st * 64 + c * 8;
      dma16(p.x + (size_t)min(r, p.n - 1) * p.x_row_stride + (k < ke ? k : kb), lds_addr(&xs[(st * XR + 8 * i) * 8]));
    }
  }
  // On the last, shorter range the chunks of x past ke are zeroed once they
  // have landed (by the wave that requested them), and a block barrier
  // publishes x.
  auto zero_tail = [&]() {
    for (int st = wave; wave < NXW && st < nst; st += NXW) {
      if (kb + st * 64 + 64 <= ke) continue;
#pragma unroll
      for (int i = 0; i < 2 * NB; ++i) {
        const int r = 8 * i + (lane >> 3);
        if (kb + st * 64 + ((lane & 7) ^ ((r >> 1) & 7)) * 8 >= ke) xs[(st * XR + 8 * i) * 8 + lane] = z4();
      }
    }
  };

  // The shrink rides this launch on the first unit_tiles tiles (the carrier
  // workgroups): wave 0 of tile g's workgroups takes unit g (pool slot x
  // 16-rank block) over the workgroup's range.  Its slot's 16 A rows
  // are requested straight into MFMA operand layout before any W load of the
  // workgroup (a block barrier holds the W waves until then: a request made
  // behind the W stream would wait for most of it); it then contracts them
  // with the x rows of its slot's rows only, gathered 16 at a time from LDS,
  // and stores and counts its piece of t while W still streams.
  const bool carrier = p.unit_tiles > 0 && g < p.unit_tiles;
  // A unit wave, its shrink work done: once the tile's arrivals are in (the
  // pieces are all stored), t of the workgroup's finalization rows, each
  // row's pieces summed in range order, into LDS over x (no wave reads x
  // any more); then it counts itself in on s_tready.
  auto t_sums = [&]() {
    if (p.unit_tiles == 0 || it_lo >= it_hi) return;
    // (row, 4-rank quad) pairs w = lane + 64 wv + 128 k: at most 64 rows of
    // at most 16 quads (R <= 64 whenever the shrink rides this launch), so
    // k < 8.  Their rows' routes depend on nothing this launch stores: they
    // are looked up before the wait.
    const int nrow = min(16 * ((it_hi - 1) / NSL + 1), p.n) - r0;
    const int R = p.R, nq = R / 4, P = p.rd.max_loras;
    int sl[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int w = lane + 64 * wv + 128 * k;
      sl[k] = -1;
      if (w < nrow * nq) {
        const RowRoute rr = row_route_decode(p, r0 + w / nq);
        if (rr.bq != nullptr) sl[k] = rr.slot;
      }
    }
    while (__hip_atomic_load(&s_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
      __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
    if (__hip_atomic_load(&s_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 1) {
      const auto tall = coherent_rsrc(p.t_part, (uint32_t)((size_t)p.S * P * p.n * R * 4));
      const uint32_t zstep = (uint32_t)(P * p.n * R) * 4;
      float *tsh = (float *)xs;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int w = lane + 64 * wv + 128 * k;
        if (w >= nrow * nq || sl[k] < 0) continue;
        const int i = r0 + w / nq, qd = w % nq;
        const uint32_t off = (uint32_t)((sl[k] * p.n + i) * R + 4 * qd) * 4;
        f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int z0 = 0; z0 < p.S; z0 += 8) {
          f32x4 pz[8];
#pragma unroll
          for (int zz = 0; zz < 8; ++zz)
            pz[zz] = z0 + zz < p.S ? ld16_coherent(tall, off, (z0 + zz) * zstep) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int zz = 0; zz < 8; ++zz)
            if (z0 + zz < p.S) sum = z0 + zz == 0 ? pz[zz] : sum + pz[zz];
        }
        *(f32x4 *)(tsh + (i - r0) * R + 4 * qd) = sum;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the sums are in LDS
    asm volatile("" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(&s_tready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  if (wv < 2) {
    const int n_units = p.rd.max_loras * RB;
    const int uk = g;
    const bool unit = carrier && wv == 0 && uk < n_units;
    const uint64_t aentry = unit ? scalar_entry(p.rd.a_table, uk / RB) : 0;
    const bool ua = unit && aentry != 0;  // a unit with A rows to contract
    const int uslot = uk / RB, urb = uk % RB;
    // lane l's k chunk in stage st, step h: columns kb + 64 st + 8 (4 h + l / 16) ..
    // (A through a buffer resource, the step in the immediate offset; a chunk
    // past ke is zeroed once it lands, and one past the buffer reads 0)
    const int cl = lane >> 4;
    auto kcol = [&](int st, int h) { return kb + st * 64 + 8 * (4 * h + cl); };
    int rslot = -1;
    uint4 af[2 * kNSt];
    if (ua) {
      rslot = lane < p.n ? p.seq_slot[lane] : -1;
      const auto ars = __builtin_amdgcn_make_buffer_rsrc(
          (void *)((const u16 *)aentry + (size_t)urb * 16 * p.k_in), 0, 16 * p.k_in * 2, 0x00020000);
      const uint32_t aoff = ((uint32_t)(lane & 15) * p.k_in + kb + 8 * cl) * 2;
#pragma unroll
      for (int st = 0; st < kNSt; ++st)
#pragma unroll
        for (int h = 0; h < 2; ++h) af[2 * st + h] = buf_ld16(ars, aoff + st * 128 + h * 64);
    }
    if (carrier) block_barrier();  // the W waves may start
    if (ua) wait_vmcnt<2 * kNSt + 1>();  // this wave's x requests have landed
    else wait_vmcnt<0>();
    if (full) {
      asm volatile("" ::: "memory");
      if (lane == 0) __hip_atomic_fetch_add(&s_xready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      zero_tail();
      __syncthreads();
    }
    if (!unit) {
      t_sums();
      return;
    }
    auto count_unit = [&]() {
      unsigned *ccnt = p.tile_cnt + (size_t)(p.n_tiles + z) * kDecodeCtrStride;
      if (wave_atomic_add(ccnt, 1u) == (unsigned)n_units - 1) {  // the range's last unit
        wave_store0(ccnt);
        for (int t = lane; t < p.n_tiles; t += 64)
          __hip_atomic_fetch_add(p.tile_cnt + (size_t)t * kDecodeCtrStride, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    };
    if (!ua) {  // no A: no row reads this slot's pieces
      count_unit();
      t_sums();
      return;
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int st = 0; st < kNSt; ++st)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (kcol(st, h) >= ke) af[2 * st + h] = z4();
    // the rows on the slot, in row order
    const uint64_t mine = __ballot(rslot == uslot);
    const int cnt = __popcll(mine);
    if (rslot == uslot) s_rows[wv][__popcll(mine & ((1ull << lane) - 1))] = lane;
    if (full) {  // every x stage has landed
      while (__hip_atomic_load(&s_xready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < NXW)
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    const int P = p.rd.max_loras;
    const auto ts = coherent_rsrc(p.t_part, (uint32_t)((size_t)p.S * P * p.n * p.R * 4));
    for (int j0 = 0; j0 < cnt; j0 += 16) {
      // lane l: gathered row j0 + l % 16 (the block's first row past cnt);
      // D[16 ranks][16 gathered rows], stages and steps in the order of a W
      // slice: lane l holds ranks 4 (l / 16) .. +3 of gathered row l % 16
      const int j = j0 + (lane & 15);
      const int row = s_rows[wv][j < cnt ? j : j0];
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < kNSt; ++st) {
        if (full || st < nst) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int c = 4 * h + cl;
            const uint4 xx = xs[(st * XR + row) * 8 + (c ^ ((row >> 1) & 7))];
            acc = mfma16(af[2 * st + h], xx, acc);
          }
        }
      }
      if (j < cnt)
        st16_coherent(ts, (uint32_t)(((z * P + uslot) * p.n + row) * p.R + urb * 16 + 4 * cl) * 4, 0, acc);
    }
    wait_vmcnt<0>();
    count_unit();
    t_sums();
    return;
  }
  if (carrier) block_barrier();  // the unit waves' requests are out

  // a W wave: slices SPW ww .. SPW ww + SPW - 1, outputs o0 + 16 SPW ww ..
  const int ww = wv - 2;
  uint4 v[2 * SPW * kNSt];
  f32x4 acc[SPW][NB];
  Slice wsl[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) wsl[s] = make_slice(p.W, p.w_row_stride, o0 + 16 * (SPW * ww + s), p.n_out, kb);
  if (full) {
    // half of the range's W, then the wait for x, then the other half: x
    // comes from HBM behind whatever W the chip has asked for, so holding
    // half of it back until x is in lets x land sooner while the first half
    // keeps the stream going; the MFMAs then follow the second half's loads
    // (all of W before the wait, or none, measured slower)
    issue_full<SPW, 0, kNSt / 2>(wsl, v);
    x_ready<2 * SPW * (kNSt / 2), NXW>(wv, &s_xready);
    issue_full<SPW, kNSt / 2, kNSt>(wsl, v);
    slice_mma<NB, SPW, true>(v, xs, wb[ww], kb, ke, nst, acc);
  } else {
    issue_part<SPW>(wsl, kb, ke, nst, v);
    wait_vm(2 * SPW * nst);  // this wave's x requests have landed
    zero_tail();
    __syncthreads();
    slice_mma<NB, SPW, false>(v, xs, wb[ww], kb, ke, nst, acc, 0);
  }
  wait_vmcnt<0>();
  if (p.S == 1 && !p.has_lora && f.n_levels == 0) {  // nothing to sum: y directly
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int i = 16 * b + (lane & 15), o = o0 + 16 * (SPW * ww + s) + 4 * (lane >> 4);
        if (i < p.n && o < p.n_out)
          *(uint2 *)(p.y + (size_t)i * p.y_row_stride + o) = make_uint2(pack2(f2bf(acc[s][b][0]), f2bf(acc[s][b][1])),
                                                                        pack2(f2bf(acc[s][b][2]), f2bf(acc[s][b][3])));
      }
    return;
  }
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const auto rs = coherent_rsrc(slice_partial(p, g, z, SPW * ww + s), kDecodeSliceFloats * 4);
    if constexpr (XL) {
#pragma unroll
      for (int b = 0; b < NB; ++b) st16_l2(rs, (uint32_t)(b * 64 + lane) * 16, 0, acc[s][b]);
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b) st16_coherent(rs, (uint32_t)(b * 64 + lane) * 16, 0, acc[s][b]);
    }
  }
  wait_vmcnt<0>();
  // the last W wave of the workgroup to have stored counts the workgroup in;
  // each tile's words sit on a cache line of their own
  unsigned *tcnt = p.tile_cnt + (size_t)g * kDecodeCtrStride;
  unsigned *tpass = tcnt + 1;
  int last = 0;
  if (lane == 0) last = atomicAdd(&s_done, 1) == NWW - 1;
  if (__builtin_amdgcn_readfirstlane(last)) (void)wave_atomic_add(tcnt, 1u);
  // this contributor's finalization items it_lo + ww, it_lo + ww + NWW, ... < it_hi
  const int m0 = it_lo + ww;
  if (m0 >= it_hi) return;
  // W wave 0 alone polls the tile's arrival count (few pollers keep the
  // line free for the arrivals); the workgroup's other item waves wait on LDS
  const RowRoute rr0 = row_route_decode(p, 16 * (m0 / NSL) + (lane & 15));  // in flight during the wait
  // the first item's B rows depend on nothing this launch stores: they are
  // in flight during the wait too
  uint4 bpre[4][2];
  {
    const int j = m0 % NSL, i = 16 * (m0 / NSL) + (lane & 15), o = g * p.tile_out + 16 * j + 4 * (lane >> 4);
    const bool expand = rr0.bq != nullptr && i < p.n && o < p.n_out;
    const u16 *bq = expand ? rr0.bq + (size_t)o * p.R : nullptr;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) bpre[c][h] = expand ? ldg16(bq + (size_t)c * p.R + 8 * h) : z4();
  }
  // s_ready: 1 once every arrival is in (the S contributors, and with the
  // shrink in this launch the S ranges whose units are all counted), 2 if
  // the wait gave up (then the tile's outputs are written as NaN: a loud
  // failure, never partial sums)
  if (ww == 0) {
    const unsigned need = (unsigned)(p.unit_tiles > 0 ? 2 * p.S : p.S);
    const unsigned got = spin_until(tcnt, need, kTileWaitTicks);
    if (lane == 0) __hip_atomic_store(&s_ready, got >= need ? 1 : 2, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    while (__hip_atomic_load(&s_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
      __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
  const bool gave_up = __hip_atomic_load(&s_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 2;
  const unsigned items_per_tile = (unsigned)T;
  for (int it = m0; it < it_hi; it += NWW) {
    const int j = it % NSL, b = it / NSL;
    const RowRoute rr = it == m0 ? rr0 : row_route_decode(p, 16 * b + (lane & 15));
    if (gave_up) {
      const int i = 16 * b + (lane & 15), o = g * p.tile_out + 16 * j + 4 * (lane >> 4);
      if (i < p.n && o < p.n_out) *(uint2 *)(p.y + (size_t)i * p.y_row_stride + o) = make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
    } else {
      if (it == m0) finalize_item<true, XL>(p, f, rr, g, j, b, (const float *)xs, r0, &s_tready, bpre);
      else finalize_item<false, XL>(p, f, rr, g, j, b, (const float *)xs, r0, &s_tready, bpre);
    }
    if (wave_atomic_add(tpass, 1u) == items_per_tile - 1) {  // every item is past the wait
      wave_store0(tcnt);
      wave_store0(tpass);
    }
  }
}

hipError_t launch_decode(const DecodeArgs &a, const StackFold *stack, hipStream_t st) {
  const int grid = a.n_tiles * a.S;
  if (grid == 0) return hipSuccess;
  StackFold f{};
  if (stack) f = *stack;
  const int nb = (a.n + 15) / 16;
  const int nsw = a.tile_out / 16;
#define LORA_DECODE(NB, NSW)                                                                                     \
  do {                                                                                                           \
    if (a.xcd_local)                                                                                             \
      hipLaunchKernelGGL((decode_kernel<NB, NSW, true>), dim3(grid), dim3((NSW / (NSW >= 8 ? 2 : 1) + 2) * 64), 0, \
                         st, a, f);                                                                              \
    else                                                                                                         \
      hipLaunchKernelGGL((decode_kernel<NB, NSW, false>), dim3(grid), dim3((NSW / (NSW >= 8 ? 2 : 1) + 2) * 64),   \
                         0, st, a, f);                                                                           \
  } while (0)
  if (nsw == 8) {
    if (nb <= 1) LORA_DECODE(1, 8);
    else if (nb == 2) LORA_DECODE(2, 8);
    else if (nb <= 4) LORA_DECODE(4, 8);
    else return hipErrorInvalidValue;
  } else if (nsw == 4) {
    if (nb <= 1) LORA_DECODE(1, 4);
    else if (nb == 2) LORA_DECODE(2, 4);
    else if (nb <= 4) LORA_DECODE(4, 4);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
#undef LORA_DECODE
  return hipGetLastError();
}

}  // namespace lora
