// k_decode.hip -- the decode-shaped apply (n <= 64 rows): a main launch and an
// epilogue launch.
//
//     y_i = W x_i + s_q B_q (A_q x_i),   q = the slot row i resolves to
//
// (ferrox lora.rs module doc; atlas lora_delta.rs apply_lora_bgmv: shrink,
// then expand-and-fold).  At decode sizes the cost is streaming W once, and
// what limits that on this chip is how fast the bytes reach the CUs: whole
// 128-byte lines move far faster than the 64-byte half lines of MFMA
// fragments loaded straight into registers.  So:
//
//  * decode_main_kernel: a workgroup owns a tile of 128 output features
//    (64 for small projections) x all rows x one k range of at most 512
//    columns (k is split S ways; S depends on k_in only).  Each 64-column
//    stage of the tile's W rows and of the batch's x rows goes to LDS by
//    LDS-DMA, whole lines, stored XOR-swizzled so the MFMA fragment reads
//    hit distinct banks; a ring of stages keeps 120 KB in flight per CU.
//    The waves own disjoint (output block, row block) pairs over the whole
//    range, so they need no reduction; the f32 partial tile goes to the
//    workspace.  The shrink t = A_q x rides along: a workgroup runs shrink
//    units (touched slot, 16-rank block) of its k range, each staging A_q's
//    rows and the slot's x rows the same way, so each A_q is read once per
//    call; on a full k range the first unit's stages go out mid-stream into
//    ring slots the W stream has finished with.  Nothing in this launch
//    waits for another workgroup;
//  * decode_epilogue_kernel: y = bf16(sum_z partial_z + s_q sum_r B_q[o, r]
//    t_i[r]), the S partials in split order, t summed over the k ranges in
//    range order, the rank sum in f32 in rank order, one rounding.
// With no adapters and no k split the main launch stores y itself.
// Skipped rows (slot < 0 or past the pool, NULL table entry, zero scale) get
// no delta arithmetic, so they equal the base-only launch bit for bit.
// Every output element is reduced in an order that does not depend on the
// batch's other rows or on n_out.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace lora {

namespace {

constexpr int kNW = 8;                               // waves per workgroup
constexpr int kNS = 6;                               // ring depth: 6 stages of TO + 64 rows

struct Rows {  // the batch's routes, resolved once per workgroup
  int raw[64];        // seq_slot, as the caller gave it (LDS-DMA)
  int q[64];          // slot or kSkip
  const u16 *bq[64];  // the row's B (rows that resolve)
  float sig[64];      // the row's scale
  int list[64];       // rows grouped by slot (row order within one)
  int start[65];      // list offsets per touched slot
  int slot[64];       // touched slots in order of first appearance
  const u16 *aq[64];  // the touched slot's A (its table entry, read once)
  int T;              // touched slots
  uint32_t ea[2][64], eb[2][64];  // the row's A and B table entries (low, high words; LDS-DMA)
  float esc[64];                  // the row's scale table entry (LDS-DMA)
};

// Routes, in three steps that keep their latency off the stream of W:
// at the start wave 0 sends seq_slot to LDS by LDS-DMA (issued before the
// first stage, so it has landed once that stage has); once it has, the
// table entries each row needs go to LDS the same way (five 4-byte DMAs:
// the halves of A's and B's pointers, the scale), counted by the explicit
// waits like the stages; later, when they have landed, wave 0 resolves the
// rows by the rule of resolve_slot and groups them by slot, slots numbered
// in order of first appearance: one round of ballots per touched slot.
constexpr int kEnt = 5;  // DMAs of fetch_entries

__device__ __forceinline__ void fetch_slots(const DecodeArgs &p, Rows &s) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64 && p.has_lora)
    dma4(p.seq_slot + min(lane, p.n - 1), lds_addr(&s.raw[0]));
}

__device__ __forceinline__ bool row_in_pool(const DecodeArgs &p, const Rows &s, int lane, int *slot) {
  *slot = lane < p.n ? s.raw[lane] : -1;
  return *slot >= 0 && *slot < p.rd.max_loras;
}

// Wave 0, once seq_slot has landed.  Every lane issues all five DMAs (a row
// that does not index the pool reads its seq_slot word again), so the count
// in flight is the same for every wave 0.
__device__ __forceinline__ void fetch_entries(const DecodeArgs &p, Rows &s) {
  const int lane = threadIdx.x & 63;
  int slot;
  const bool in = row_in_pool(p, s, lane, &slot);
  const uint32_t *dummy = (const uint32_t *)(p.seq_slot + min(lane, p.n - 1));
  const uint32_t *pa = in ? (const uint32_t *)(p.rd.a_table + slot) : dummy;
  const uint32_t *pb = in ? (const uint32_t *)(p.rd.b_table + slot) : dummy;
  dma4(pa, lds_addr(&s.ea[0][0]));
  dma4(in ? pa + 1 : dummy, lds_addr(&s.ea[1][0]));
  dma4(pb, lds_addr(&s.eb[0][0]));
  dma4(in ? pb + 1 : dummy, lds_addr(&s.eb[1][0]));
  dma4(in ? (const uint32_t *)(p.rd.scale_table + slot) : dummy, lds_addr(&s.esc[0]));
}

// Wave 0, once the entries have landed.
__device__ void resolve_rows(const DecodeArgs &p, Rows &s) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x >= 64) return;
  int slot;
  const bool in = row_in_pool(p, s, lane, &slot);
  const uint64_t a = in ? ((uint64_t)s.ea[1][lane] << 32) | s.ea[0][lane] : 0;
  const uint64_t b = in ? ((uint64_t)s.eb[1][lane] << 32) | s.eb[0][lane] : 0;
  const float sc = in ? s.esc[lane] : 0.f;
  const int q = in && a != 0 && b != 0 && sc != 0.f ? slot : kSkip;
  s.q[lane] = q;
  s.bq[lane] = q >= 0 ? (const u16 *)b : nullptr;
  s.sig[lane] = q >= 0 ? sc : 0.f;
  const uint64_t below = (1ull << lane) - 1ull;
  uint64_t todo = __ballot(q >= 0);
  int T = 0, pos = 0;
  while (todo) {  // uniform: the lowest row not yet grouped names the next slot
    const int first = __ffsll((unsigned long long)todo) - 1;
    const int v = __builtin_amdgcn_readlane(q, first);
    const uint64_t av = ((uint64_t)__builtin_amdgcn_readlane((int)(a >> 32), first) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)a, first);
    const uint64_t m = __ballot(q == v);
    if (q == v) s.list[pos + __popcll(m & below)] = lane;
    if (lane == 0) {
      s.slot[T] = v;
      s.aq[T] = (const u16 *)av;
      s.start[T] = pos;
    }
    pos += __popcll(m);
    ++T;
    todo &= ~m;
  }
  if (lane == 0) {
    s.T = T;
    s.start[T] = pos;
  }
}

// Zeroes, after its stage has landed, each 16-byte chunk this lane fetched
// from past the k range (it fetched column 0 of its row instead).
__device__ __forceinline__ void zero_past(uint4 *slot, int k0, int ke, int chunk) {
  if (k0 + chunk >= ke) *slot = z4();
}

// One shrink unit (touched slot u, rank block rb) of this workgroup's k
// range: the range's partial of t for the rows of slot u, ranks 16 rb .. +15.
// The range's stages of A_u's 16 rows and of the slot's x rows (gathered, up
// to 64, in groups of 16) go to LDS in one go; wave g then takes row group g
// through every stage.
__device__ __forceinline__ int unit_groups(const Rows &s, int R, int uidx) {
  const int u = uidx / (R / 16);
  return (s.start[u + 1] - s.start[u] + 15) / 16;  // groups of 16 gathered rows (<= 4)
}

// LDS bytes a unit of G row groups stages over ns 64-column stages.
__device__ __forceinline__ int unit_bytes(int G, int ns) { return ns * (16 + 16 * G) * 128; }

// Issues the unit's DMAs: wave w takes instructions w, w + 8, ...
__device__ void unit_issue(const DecodeArgs &p, const Rows &s, int uidx, int k0, int k1, uint4 *lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = p.R, RB = R / 16;
  const int rb = uidx % RB, u = uidx / RB;
  const u16 *A = s.aq[u];
  const int m = s.start[u + 1] - s.start[u];
  const int G = (m + 15) / 16;
  const int ns = (k1 - k0 + 63) / 64;
  const int RU = 16 + 16 * G;   // rows of a unit stage: A's 16, then the x rows
  const int per = RU / 8;       // DMA instructions per unit stage
  for (int ii = wave; ii < ns * per; ii += kNW) {
    const int st = ii / per, k8 = ii % per;
    const int rr = k8 * 8 + (lane >> 3);  // row of the unit stage
    const u16 *rowp;
    if (rr < 16) {
      rowp = A + (size_t)(rb * 16 + rr) * p.k_in;
    } else {
      const int j = min(rr - 16, m - 1);
      rowp = p.x + (size_t)s.list[s.start[u] + j] * p.x_row_stride;
    }
    const int kk = k0 + st * 64 + ((lane & 7) ^ ((rr >> 1) & 7)) * 8;
    dma16(rowp + (kk < k1 ? kk : k0), lds_addr(lds + (st * RU + k8 * 8) * 8));
  }
}

// Zeroes what the unit fetched past the k range; then the unit's MFMAs (wave
// g takes row group g) and its partial of t.  The unit's stages have landed
// for every wave before this is called.
__device__ void unit_compute(const DecodeArgs &p, const Rows &s, int uidx, int k0, int k1, uint4 *lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = p.R, RB = R / 16;
  const int rb = uidx % RB, u = uidx / RB;
  const int c = blockIdx.x % p.S;  // the k range: the partial's index
  const int m = s.start[u + 1] - s.start[u];
  const int G = (m + 15) / 16;
  const int ns = (k1 - k0 + 63) / 64;
  const int RU = 16 + 16 * G;
  const int per = RU / 8;
  if (k0 + ns * 64 > k1) {  // the last stage runs past the chunk
    for (int ii = wave; ii < ns * per; ii += kNW) {
      const int st = ii / per, k8 = ii % per;
      const int rr = k8 * 8 + (lane >> 3);
      zero_past(lds + (st * RU + k8 * 8) * 8 + lane, k0 + st * 64, k1, ((lane & 7) ^ ((rr >> 1) & 7)) * 8);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __syncthreads();
  }
  if (wave < G) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ra = lane & 15, rx = 16 + wave * 16 + (lane & 15);
    for (int st = 0; st < ns; ++st) {
      const uint4 *sl = lds + st * RU * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ch = 4 * h + (lane >> 4);
        acc = mfma16(sl[ra * 8 + (ch ^ ((ra >> 1) & 7))], sl[rx * 8 + (ch ^ ((rx >> 1) & 7))], acc);
      }
    }
    // D: ranks 4 (l/16) .. +3 of gathered row 16 g + l%16
    const int j = wave * 16 + (lane & 15);
    if (j < m) {
      const int row = s.list[s.start[u] + j];
      *(f32x4 *)(p.t_part + ((size_t)c * p.n + row) * R + rb * 16 + (lane >> 4) * 4) = acc;
    }
  }
}

__device__ void shrink_unit(const DecodeArgs &p, const Rows &s, int uidx, int k0, int k1, uint4 *lds) {
  unit_issue(p, s, uidx, k0, k1, lds);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unit_compute(p, s, uidx, k0, k1, lds);
  __syncthreads();  // the ring is reused by the next unit
}

}  // namespace

// NB: 16-row blocks of the batch that hold rows (n <= 16 NB); TO: output
// features per tile.  Wave w owns
// output blocks OBW (w % OWAVES) .. +OBW-1 and row blocks RBW (w / OWAVES) ..
template <int NB, int TO>
__global__ __launch_bounds__(kNW * 64) void decode_main_kernel(DecodeArgs p) {
  constexpr int kTO = TO;
  constexpr int kRS = kTO + kDecodeMaxRows;  // rows of a stage: W rows, then x rows
  constexpr int kLPW = kRS / 8 / kNW;        // DMA instructions per wave per stage
  static_assert(kLPW * 8 * kNW == kRS, "stage rows must split evenly over the waves");
  constexpr int RWAVES = NB >= 2 ? 2 : 1;  // waves across the row blocks
  constexpr int OWAVES = kNW / RWAVES;     // waves across the output blocks
  constexpr int OBW = kTO / 16 / OWAVES;   // output blocks per wave
  constexpr int RBW = NB / RWAVES;         // row blocks per wave
  static_assert(OWAVES * OBW * 16 == kTO && RWAVES * RBW == NB, "wave tiling");
  __shared__ __attribute__((aligned(16))) uint4 ring[kNS][kRS * 8];
  __shared__ Rows s;

  // every argument the first DMAs need comes in with the first batch of
  // scalar loads (the route pointer too, which the compiler would otherwise
  // load behind a branch, one more round trip before the first stage)
  asm volatile("" ::"s"(p.seq_slot), "s"(p.has_lora));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.k_in;
  const int tl = blockIdx.x / p.S, z = blockIdx.x % p.S;
  const int o0 = tl * kTO;
  const int kb = min(z * p.k_per_split, K), ke = min(kb + p.k_per_split, K);
  const int nstage = (ke - kb + 63) / 64;
  // Each DMA instruction moves 8 whole 128-byte row segments: lane l takes
  // row 8i + l/8 of the stage and the chunk that belongs at slot l%8 of it.
  // Rows past n_out or past the batch read a valid row instead; their
  // outputs are never stored.
  const u16 *src[kLPW];
  int sch[kLPW];
#pragma unroll
  for (int j = 0; j < kLPW; ++j) {
    const int rr = (wave + kNW * j) * 8 + (lane >> 3);
    src[j] = rr < kTO ? p.W + (size_t)min(o0 + rr, p.n_out - 1) * p.w_row_stride
                      : p.x + (size_t)min(rr - kTO, p.n - 1) * p.x_row_stride;
    sch[j] = ((lane & 7) ^ ((rr >> 1) & 7)) * 8;
  }
  auto issue = [&](int st) {
    const int k0 = kb + st * 64;
#pragma unroll
    for (int j = 0; j < kLPW; ++j) {
      const int kk = k0 + sch[j] < ke ? k0 + sch[j] : kb;
      dma16(src[j] + kk, lds_addr(&ring[st % kNS][(wave + kNW * j) * 64]));
    }
  };
  fetch_slots(p, s);
  const int npro = min(kNS - 1, nstage);  // stages issued before the loop
  for (int st = 0; st < npro; ++st) issue(st);
  // wave 0: once seq_slot has landed (older than every stage), the table
  // entries go out; they are younger than the first npro stages, so wave 0
  // allows for them (kEnt more operations in flight) when it waits for those
  const bool ents = p.has_lora && wave == 0;
  if (ents) {
    wait_stages<kLPW, kNS - 1>(npro);
    fetch_entries(p, s);
  }

  const int ob0 = (wave % OWAVES) * OBW, rb0 = (wave / OWAVES) * RBW;
  f32x4 acc[OBW][RBW];
#pragma unroll
  for (int a = 0; a < OBW; ++a)
#pragma unroll
    for (int b = 0; b < RBW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // On a full k range the routes are resolved at stage kEarly, once the table
  // entries are sure to have landed (they went out before stage kEarly), and
  // this workgroup's first shrink unit sends its stages into the ring slots
  // of stages 2 .. 4, which no later stage takes; its MFMAs then run right
  // after the loop instead of behind a round trip of their own.  Each wave
  // issues exactly xw of those DMAs, which the later stage waits allow for.
  constexpr int kEarly = kNS - 1;
  static_assert(kEarly + 1 < kDecodeMaxStages && kDecodeMaxStages - kNS == 2, "free slots 2 .. kEarly - 1");
  const bool early_ok = p.has_lora && nstage == kDecodeMaxStages && ke - kb == 64 * kDecodeMaxStages;
  bool early = false;
  // one stage: wait until it has landed (at most kNS - 2 younger stages, and
  // X more operations issued after them, in flight), zero what lies past the
  // k range, `mid` before the barrier, the barrier, refill the ring, `post`,
  // then the stage's fragments and MFMAs
  auto stage = [&](int st, auto xc, auto mid, auto post) {
    constexpr int X = decltype(xc)::value;
    const int younger = min(kNS - 2, nstage - 1 - st);
    if (ents && st < npro)
      wait_stages<kLPW, kNS - 2, kEnt>(younger);
    else
      wait_stages<kLPW, kNS - 2, X>(younger);
    if (kb + st * 64 + 64 > ke) {
#pragma unroll
      for (int j = 0; j < kLPW; ++j)
        zero_past(&ring[st % kNS][(wave + kNW * j) * 64 + lane], kb + st * 64, ke, sch[j]);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    }
    mid();
    block_barrier();
    // every wave is done with stage st - 1: its slot takes stage st + kNS - 1
    if (st + kNS - 1 < nstage) issue(st + kNS - 1);
    post();
    const uint4 *sl = ring[st % kNS];
    uint4 af[2][OBW], bf[2][RBW];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 4 * h + (lane >> 4);
#pragma unroll
      for (int a = 0; a < OBW; ++a) {
        const int r = (ob0 + a) * 16 + (lane & 15);
        af[h][a] = sl[r * 8 + (c ^ ((r >> 1) & 7))];
      }
#pragma unroll
      for (int b = 0; b < RBW; ++b) {
        const int r = kTO + (rb0 + b) * 16 + (lane & 15);
        bf[h][b] = sl[r * 8 + (c ^ ((r >> 1) & 7))];
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int a = 0; a < OBW; ++a)
#pragma unroll
        for (int b = 0; b < RBW; ++b) acc[a][b] = mfma16(af[h][a], bf[h][b], acc[a][b]);
  };
  using X0 = std::integral_constant<int, 0>;
  auto none = [] {};
  const int st1 = early_ok ? kEarly : nstage;
  for (int st = 0; st < st1; ++st) stage(st, X0{}, none, none);
  int xw = 0;
  if (early_ok) {
    stage(kEarly, X0{},
          [&] {
            if (wave == 0) {  // its LDS writes land before the barrier
              resolve_rows(p, s);
              __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
            }
          },
          [&] {
            if (tl < s.T * (p.R / 16)) {
              const int G = unit_groups(s, p.R, tl);
              if (unit_bytes(G, kDecodeMaxStages) <= 3 * (int)sizeof(ring[0])) {
                unit_issue(p, s, tl, kb, ke, &ring[2][0]);
                xw = 2 + 2 * G;  // (16 + 16 G) / 8 instructions per unit stage, 8 stages over 8 waves
                early = true;
              }
            }
          });
    for (int st = kEarly + 1; st < nstage; ++st) {
      if (xw == 0) stage(st, X0{}, none, none);
      else if (xw == 4) stage(st, std::integral_constant<int, 4>{}, none, none);
      else if (xw == 6) stage(st, std::integral_constant<int, 6>{}, none, none);
      else stage(st, std::integral_constant<int, 8>{}, none, none);
    }
  }

  // the routes first (the table entries arrived long ago; no store is
  // outstanding yet that the wait for them would include)
  if (p.has_lora && !early_ok) {
    if (wave == 0) __builtin_amdgcn_s_waitcnt(0);  // the entries (the last stage's wait may allow them)
    resolve_rows(p, s);
  }
  if (early) {  // the early unit: only its DMAs are in flight
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    unit_compute(p, s, tl, kb, ke, &ring[2][0]);
  }
  // D layout: column (row) l%16 of the row block, outputs 4 (l/16) .. +3 of
  // the output block
  const bool direct = p.S == 1 && !p.has_lora;  // nothing left for an epilogue: store y now
  float *part = p.partials + ((size_t)tl * p.S + z) * (kDecodeMaxRows * kTO);
#pragma unroll
  for (int a = 0; a < OBW; ++a)
#pragma unroll
    for (int b = 0; b < RBW; ++b) {
      const int i = (rb0 + b) * 16 + (lane & 15), oo = (ob0 + a) * 16 + (lane >> 4) * 4;
      if (i >= p.n) continue;
      const f32x4 v = acc[a][b];
      if (direct) {
        if (o0 + oo < p.n_out)
          *(uint2 *)(p.y + (size_t)i * p.y_row_stride + o0 + oo) =
              make_uint2(pack2(f2bf(v[0]), f2bf(v[1])), pack2(f2bf(v[2]), f2bf(v[3])));
      } else {
        *(f32x4 *)(part + i * kTO + oo) = v;
      }
    }
  if (!p.has_lora) return;
  __syncthreads();  // the routes are resolved and the ring is free
  if (blockIdx.x == 0 && tid < 64) {  // the epilogue's per-row routes
    p.row_q[tid] = s.q[tid];
    p.row_sig[tid] = s.sig[tid];
    p.row_b[tid] = s.bq[tid];
  }
  const int units = s.T * (p.R / 16);  // of this k range
  for (int uidx = tl + (early ? p.n_tiles : 0); uidx < units; uidx += p.n_tiles)
    shrink_unit(p, s, uidx, kb, ke, &ring[0][0]);
}

// y for 16 rows x 64 output features per workgroup, one thread per (row,
// four features): t is then needed for 16 rows only.  Every load that does
// not depend on another goes out first: the row's route, the S partials, t.
constexpr int kEpiOut = 64;  // output features per epilogue workgroup
__global__ __launch_bounds__(256) void decode_epilogue_kernel(DecodeArgs p, StackFold f) {
  __shared__ __attribute__((aligned(16))) float st[16 * 256];  // t of the 16 rows, 16 x R
  const int tid = threadIdx.x;
  const int R = p.R;
  const int kTO = p.tile_out;
  const int OPT = kTO / kEpiOut;  // output groups per tile
  const int rg = blockIdx.x % 4, og = blockIdx.x / 4;  // row group, output group
  const int tl = og / OPT;
  const int i = rg * 16 + (tid >> 4), oo = (og % OPT) * kEpiOut + (tid & 15) * 4, o = tl * kTO + oo;
  if (rg * 16 >= p.n) return;  // no rows in this group
  const bool live = i < p.n && o < p.n_out;
  const bool lora = p.has_lora;
  // the row's route: slot, B and scale load together
  const int q = live && lora ? p.row_q[i] : kSkip;
  const u16 *rb_ = live && lora ? p.row_b[i] : nullptr;
  const float sig = live && lora ? p.row_sig[i] : 0.f;
  f32x4 a[kDecodeMaxSplit];
  const float *pp = p.partials + (size_t)tl * p.S * (kDecodeMaxRows * kTO) + i * kTO + oo;
#pragma unroll
  for (int z = 0; z < kDecodeMaxSplit; ++z)
    a[z] = live && z < p.S ? *(const f32x4 *)(pp + (size_t)z * (kDecodeMaxRows * kTO)) : f32x4{0.f, 0.f, 0.f, 0.f};
  const int nr = min(16, p.n - rg * 16);  // rows of this group
  if (lora)  // stage t of the group's rows in LDS: the k ranges' partials summed in range order
    for (int e = tid * 4; e < nr * R; e += 256 * 4) {
      const float *tp = p.t_part + (size_t)rg * 16 * R + e;
      f32x4 w[kDecodeMaxSplit];
#pragma unroll
      for (int c = 0; c < kDecodeMaxSplit; ++c)
        w[c] = c < p.n_chunks ? *(const f32x4 *)(tp + (size_t)c * p.n * R) : f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 v = w[0];
#pragma unroll
      for (int c = 1; c < kDecodeMaxSplit; ++c)
        if (c < p.n_chunks) v += w[c];
      *(f32x4 *)(st + e) = v;
    }
  const u16 *Bq = q >= 0 ? rb_ + (size_t)o * R : nullptr;
  uint4 b[2][4];  // ranks 0..15 of the thread's four B rows
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) b[h][j] = Bq && h * 8 < R ? ldg16(Bq + (size_t)j * R + h * 8) : z4();
  __syncthreads();
  if (!live) return;
  f32x4 v = a[0];
#pragma unroll
  for (int z = 1; z < kDecodeMaxSplit; ++z)  // split order
    if (z < p.S) v += a[z];
  if (q >= 0) {
    const float *ti = st + (i - rg * 16) * R;
    float d[4] = {0.f, 0.f, 0.f, 0.f};
    auto fma8 = [&](const uint4 *bb, int r0) {
      float tr[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) tr[c] = ti[r0 + c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w[4] = {bb[j].x, bb[j].y, bb[j].z, bb[j].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          d[j] += bf2f((u16)(w[c] & 0xffffu)) * tr[2 * c];
          d[j] += bf2f((u16)(w[c] >> 16)) * tr[2 * c + 1];
        }
      }
    };
    fma8(b[0], 0);
    if (R > 8) fma8(b[1], 8);
    for (int r0 = 16; r0 < R; r0 += 8) {  // ranks past 16, in order
      uint4 bb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = ldg16(Bq + (size_t)j * R + r0);
      fma8(bb, r0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = v[j] + sig * d[j];
  }
  // an adapter stack's further levels, in level order, from their final t:
  // every level's slot, then its table entries, go out together, so the
  // levels cost one chain of round trips, not one each
  if (f.n_levels > 0) {
    int sl[kMaxStackLevels];
#pragma unroll
    for (int l = 0; l < kMaxStackLevels; ++l) sl[l] = l < f.n_levels ? f.lv[l].seq_slot[i] : -1;
    const u16 *bl[kMaxStackLevels];
    float sc[kMaxStackLevels];
#pragma unroll
    for (int l = 0; l < kMaxStackLevels; ++l) {
      const StackLevel &L = f.lv[l];
      const bool in = l < f.n_levels && sl[l] >= 0 && sl[l] < L.max_loras;
      const void *ta = in ? L.a_table[sl[l]] : nullptr;
      const void *tb = in ? L.b_table[sl[l]] : nullptr;
      const float s = in ? L.scale_table[sl[l]] : 0.f;
      const bool ok = ta != nullptr && tb != nullptr && s != 0.0f;
      bl[l] = ok ? (const u16 *)tb + (size_t)o * L.R : nullptr;
      sc[l] = s;
    }
#pragma unroll
    for (int l = 0; l < kMaxStackLevels; ++l) {
      if (bl[l] == nullptr) continue;
      const StackLevel &L = f.lv[l];
      const float *tl = L.t + (size_t)i * L.R;
      float d[4] = {0.f, 0.f, 0.f, 0.f};
      for (int r0 = 0; r0 < L.R; r0 += 8) {  // ranks in order, 8 at a time
        float tr[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) tr[c] = tl[r0 + c];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 bb = ldg16(bl[l] + (size_t)j * L.R + r0);
          const uint32_t w[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            d[j] += bf2f((u16)(w[c] & 0xffffu)) * tr[2 * c];
            d[j] += bf2f((u16)(w[c] >> 16)) * tr[2 * c + 1];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = v[j] + sc[l] * d[j];
    }
  }
  *(uint2 *)(p.y + (size_t)i * p.y_row_stride + o) =
      make_uint2(pack2(f2bf(v[0]), f2bf(v[1])), pack2(f2bf(v[2]), f2bf(v[3])));
}

hipError_t launch_decode_main(const DecodeArgs &a, hipStream_t st) {
  const int grid = a.n_tiles * a.S;
  if (grid == 0) return hipSuccess;
  const int nb = (a.n + 15) / 16;
#define LORA_DECODE(NB, TO) hipLaunchKernelGGL((decode_main_kernel<NB, TO>), dim3(grid), dim3(kNW * 64), 0, st, a)
  const bool small = a.tile_out == kDecodeTileOutSmall;
  if (!small && a.tile_out != kDecodeTileOut) return hipErrorInvalidValue;
  if (nb <= 1) {  // one row block: the small tile leaves waves without output blocks
    if (small) return hipErrorInvalidValue;
    LORA_DECODE(1, kDecodeTileOut);
  } else if (nb == 2) {
    if (small) LORA_DECODE(2, kDecodeTileOutSmall); else LORA_DECODE(2, kDecodeTileOut);
  } else if (nb <= 4) {
    if (small) LORA_DECODE(4, kDecodeTileOutSmall); else LORA_DECODE(4, kDecodeTileOut);
  } else {
    return hipErrorInvalidValue;
  }
#undef LORA_DECODE
  return hipGetLastError();
}

hipError_t launch_decode_epilogue(const DecodeArgs &a, const StackFold *stack, hipStream_t st) {
  StackFold f{};
  if (stack) f = *stack;
  if (a.S == 1 && !a.has_lora)  // the main launch stored y; a stack always has a routed first level
    return f.n_levels ? hipErrorInvalidValue : hipSuccess;
  hipLaunchKernelGGL(decode_epilogue_kernel, dim3(a.n_tiles * (a.tile_out / kEpiOut) * 4), dim3(256), 0, st, a, f);
  return hipGetLastError();
}

}  // namespace lora
