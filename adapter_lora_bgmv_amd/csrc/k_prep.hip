// k_prep.hip -- route resolve, the row plan, and the grouped MFMA shrink (bf16).
//
// route_kernel resolves every row's route once (slot -> pair or skip, atlas
// apply_lora_bgmv doc), counts each pair's rows and ranks every row within
// its pair; a segmented call of up to 4096 rows over at most 64 segments does
// without it, since every row of a segment routes alike.  Then one launch of
// prep_kernel does two independent jobs:
//  * workgroup plan_at groups the rows by (W group, adapter) -- a counting
//    sort in LDS, or for a segmented call whole segments sorted by key --
//    and cuts each W group into the main kernel's row tiles.  Within a key
//    the order is whatever the LDS atomics give: no output value depends on
//    it, because every output element is reduced row-locally with the same
//    instruction sequence.
//  * every other workgroup is one shrink unit: up to 64 rows that share one
//    pair over one k chunk, t[rows] = x[rows] . A_pair^T (ferrox
//    LoraDelta::project), on bf16 MFMA with f32 accumulation.  A unit finds
//    its pair and rows from the pair counts (the route kernel's, the
//    segments', or its own histogram), so the shrink does not wait for the
//    plan; its waves' sums meet in a fixed order, and the k chunks' partials
//    are summed in chunk order by the pair's last unit to arrive.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

// Exclusive scan of a[0..L) in LDS by the 256 threads; returns the total.
// Deterministic: sequential per thread, fixed shuffle tree across lanes.
__device__ int block_exscan(int *a, int L, int *wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (L + 255) / 256;
  const int b = min(tid * per, L), e = min(b + per, L);
  int s = 0;
  for (int i = b; i < e; ++i) s += a[i];
  int v = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  int run = pre + v - s;
  for (int i = b; i < e; ++i) {
    int c = a[i];
    a[i] = run;
    run += c;
  }
  __syncthreads();
  return total;
}

// ------------------------------------------------------------------ routing
// Every row's route is computed once per workgroup into a packed LDS word:
// (key + 1) << 13 | (pair + 2), key = the plan's sort key (-1: row not
// written), pair = table index, kSkip or kDrop.  Keys and pairs are below
// kMaxKeys = 4096.
__device__ __forceinline__ int pk_key(int w) { return (w >> 13) - 1; }
__device__ __forceinline__ int pk_pair(int w) { return (w & 0x1fff) - 2; }

// A wave's 64 rows split into runs of equal keys (a new run where the key
// changes from the lane before).  `bnds` has a bit per run start; a run
// start's run ends at the next start (or lane 64); a lane's run starts at
// the highest start at or below it.  Sorted rows (a prefill segment, an
// expert's range) make a few long runs, unsorted rows runs of one.
__device__ __forceinline__ uint64_t run_starts(int k, int lane) {
  const int kp = __shfl_up(k, 1, 64);
  return __ballot(lane == 0 || kp != k);
}
__device__ __forceinline__ int run_end(uint64_t bnds, int lane) {
  const uint64_t later = bnds & ~((2ull << lane) - 1ull);
  return later ? __ffsll((unsigned long long)later) - 1 : 64;
}
__device__ __forceinline__ int run_start(uint64_t bnds, int lane) {
  return 63 - __clzll((unsigned long long)(bnds & ((2ull << lane) - 1ull)));
}

// Row ranges of a call: the segments of a segmented call, the experts of a
// grouped MoE call ([n+1] non-decreasing starts); tables up to kSegLds
// entries are copied to LDS for the routing.
constexpr int kSegLds = 4096;
// Pairs a wave's rows are grouped by before the rest go by runs of equal pairs.
constexpr int kRankGroups = 8;
// Segments a shrink unit looks through for its adapter's first one.
constexpr int kSegScan = 64;

__device__ __forceinline__ bool has_ranges(const Routing &rt) {
  return rt.mode == kModeSegmented || rt.mode == kModeMoeGrouped;
}
__device__ __forceinline__ const int32_t *range_starts(const Routing &rt) {
  return rt.mode == kModeSegmented ? rt.seg_indptr : rt.expert_offsets;
}
__device__ __forceinline__ int range_count(const Routing &rt) {
  return rt.mode == kModeSegmented ? rt.n_seg : rt.n_experts;
}
__device__ __forceinline__ bool seg_in_lds(const Routing &rt) {
  return has_ranges(rt) && range_count(rt) + 1 <= kSegLds;
}

// The segment of row r from an LDS copy of seg_indptr (binary search).
__device__ __forceinline__ int segment_lds(const int *ip, int n_seg, int r) {
  if (n_seg <= 0 || r < ip[0] || r >= ip[n_seg]) return -1;
  int lo = 0, hi = n_seg - 1;  // last g with ip[g] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ip[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Routes rows row0 + tid + 256 j (j < J) into pk[]: every load of the batch
// (the slot inputs, then the three route tables) in flight together.  `seg`
// is an LDS copy of the row ranges (segmented and grouped MoE calls), or null.
template <int J = 8>
__device__ __forceinline__ void route_all(const PrepArgs &a, int *pk, const int *seg, int row0,
                                          bool ranked = false) {
  const int ml = a.has_lora ? a.rd.max_loras : 0;
  const RouteDev &rd = a.rd;
  const Routing &rt = a.rt;
  {
    const int r0 = row0 + (int)threadIdx.x;
    int slot[J], expert[J], drop[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int r = r0 + 256 * j;
      const bool live = r < a.n;
      int sl = -1, ex = 0, dr = !live;
      if (live && rt.mode == kModeDecode) {
        sl = rt.seq_slot ? rt.seq_slot[r] : -1;
      } else if (live && rt.mode == kModeSegmented) {
        const int g = seg ? segment_lds(seg, rt.n_seg, r) : segment_of(rt.seg_indptr, rt.n_seg, r);
        dr = g < 0;
        sl = g < 0 ? -1 : rt.seg_slot[g];
      } else if (live && rt.mode == kModeMoeGrouped) {
        const int e = seg ? segment_lds(seg, rt.n_experts, r) : segment_of(rt.expert_offsets, rt.n_experts, r);
        dr = e < 0;
        ex = dr ? 0 : e;
        sl = a.has_lora && !dr ? rt.seq_slot[r] : -1;
      } else if (live) {
        const int e = rt.indices[r];
        dr = e < 0 || e >= rt.n_experts;
        ex = dr ? 0 : e;
        sl = a.has_lora && !dr ? rt.token_slot[r / rt.top_k] : -1;
      }
      slot[j] = sl;
      expert[j] = ex;
      drop[j] = dr;
    }
    uint64_t ta[J], tb[J];
    float sc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {  // the three tables, index 0 standing in for rows without a slot
      const bool in = a.has_lora && !drop[j] && slot[j] >= 0 && slot[j] < rd.max_loras;
      const int idx = in ? slot[j] * rd.n_experts + expert[j] : 0;
      ta[j] = in ? (uint64_t)(uintptr_t)rd.a_table[idx] : 0ull;
      tb[j] = in ? (uint64_t)(uintptr_t)rd.b_table[idx] : 0ull;
      sc[j] = in ? rd.scale_table[slot[j]] : 0.f;
    }
    int qv[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int r = r0 + 256 * j;
      const bool ok = ta[j] != 0ull && tb[j] != 0ull && sc[j] != 0.0f;
      const int q = drop[j] ? kDrop : (ok ? slot[j] * rd.n_experts + expert[j] : kSkip);
      const int key = drop[j] ? -1 : expert[j] * (ml + 1) + (q >= 0 ? slot[j] : ml);
      if (r < a.n) pk[r] = ((key + 1) << 13) | (q + 2);
      qv[j] = r < a.n ? q : kSkip;
    }
    if (ranked) {  // each row's rank within its pair: the rows of one pair in a wave take their ranks with one atomic
      const int lane = threadIdx.x & 63;
      const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int q = qv[j];
        // group the wave's rows by pair (one round of ballots per pair, the
        // lowest lane of a pair leading it) for up to kRankGroups pairs; the
        // rows of a wave with more pairs go by runs of equal pairs; then
        // every leader's atomic goes out in one instruction
        uint64_t todo = __ballot(q >= 0);
        int lead = lane, off = 0, cnt = 0;
        for (int it = 0; todo && it < kRankGroups; ++it) {  // uniform
          const int l0 = __ffsll((unsigned long long)todo) - 1;
          const int v = __builtin_amdgcn_readlane(q, l0);
          const uint64_t m = __ballot(q == v);
          if (q == v) {
            lead = l0;
            off = (int)__popcll(m & below);
          }
          if (lane == l0) cnt = (int)__popcll(m);
          todo &= ~m;
        }
        if (todo) {  // uniform
          const bool left = (todo >> lane) & 1ull;
          const uint64_t bnds = run_starts(left ? q : -2 - lane, lane);  // other lanes end every run
          if (left) {
            lead = run_start(bnds, lane);
            off = lane - lead;
            if (lane == lead) cnt = run_end(bnds, lane) - lane;
          }
        }
        unsigned got = 0;
        if (q >= 0 && lane == lead) got = atomicAdd(&a.pair_cnt[q], (unsigned)cnt);
        const int base = __shfl((int)got, lead, 64);
        const int r = r0 + 256 * j;
        if (r < a.n) {
          a.ranks[r] = q >= 0 ? base + off : -1;
          // the pair's first kShrinkRows rows, by rank, in its bucket
          if (a.bucket != nullptr && q >= 0 && q < a.bucket_pairs && base + off < kShrinkRows)
            a.bucket[q * kShrinkRows + base + off] = r;
        }
      }
    }
  }
}

// Adds to cnt[k] the number of rows with k = f(pk[r]) >= 0: each wave takes
// 64 rows at a time and adds every run of equal keys with one atomic.
template <typename F>
__device__ __forceinline__ void count_rows(const int *pk, int n, int *cnt, F f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r0 = wave * 64; r0 < n; r0 += 256) {
    const int r = r0 + lane;
    const int k = r < n ? f(pk[r]) : -1;
    const uint64_t bnds = run_starts(k, lane);
    if (k >= 0 && ((bnds >> lane) & 1ull)) atomicAdd(&cnt[k], run_end(bnds, lane) - lane);
  }
}

// The plan of a segmented call over at most 64 segments whose bounds never
// decrease: every row of a segment routes alike (its slot is the segment's),
// so the rows sorted by key are the segments sorted by key (stably, by
// segment index), each segment's rows in row order.  Segment g owns the rows
// [indptr[g], indptr[g + 1]) clamped to the batch, which are the rows
// segment_of assigns it when the bounds never decrease.  No per-row counting:
// one round trip for the bounds and slots, then every row placed directly.
// Returns false (uniform) where the call does not have that form.
__device__ __forceinline__ bool plan_segments(const PrepArgs &a, int *lds) {
  const Routing &rt = a.rt;
  if (rt.mode != kModeSegmented || rt.n_seg > 64 || rt.n_experts != 1) return false;
  const int tid = threadIdx.x, lane = tid & 63, ns = rt.n_seg;
  int *s_off = lds, *s_lo = lds + 64, *s_len = lds + 128, *s_q = lds + 192, *s_ok = lds + 256;
  if (tid < 64) {
    const bool in = lane < ns;
    const int ilo = in ? rt.seg_indptr[lane] : 0, ihi = in ? rt.seg_indptr[lane + 1] : 0;
    const int slot = in ? rt.seg_slot[lane] : -1;
    const int ml = a.has_lora ? a.rd.max_loras : 0;
    const int q = in && a.has_lora ? resolve_slot(slot, 0, ml, a.rd.n_experts, a.rd.a_table, a.rd.b_table, a.rd.scale_table)
                                   : kSkip;
    const int key = q >= 0 ? slot : ml;
    const int lo = min(max(ilo, 0), a.n), hi = min(max(ihi, 0), a.n);
    const int len = in ? max(hi - lo, 0) : 0;
    int off = 0;
    for (int g = 0; g < ns; ++g) {  // uniform: the segments before this one in (key, index) order
      const int kg = __builtin_amdgcn_readlane(key, g), lg = __builtin_amdgcn_readlane(len, g);
      if (kg < key || (kg == key && g < lane)) off += lg;
    }
    if (in) {
      s_off[lane] = off;
      s_lo[lane] = lo;
      s_len[lane] = len;
      s_q[lane] = q;
    }
    const uint64_t bad = __ballot(in && ilo > ihi);
    if (lane == 0) s_ok[0] = bad == 0ull;
  }
  __syncthreads();
  if (!s_ok[0]) {  // uniform: the general plan, which may reuse this LDS
    __syncthreads();
    return false;
  }
  int total = 0;
  for (int g = 0; g < ns; ++g) {  // uniform
    const int off = s_off[g], lo = s_lo[g], len = s_len[g], q = s_q[g];
    for (int i = tid; i < len; i += 256) {
      a.plan.pos_row[off + i] = lo + i;
      a.plan.pos_pair[off + i] = q;
    }
    total += len;
  }
  const int ntiles = (total + a.tile_rows - 1) / a.tile_rows;
  for (int t = tid; t < ntiles; t += 256)
    a.plan.tiles[t] = make_int4(0, t * a.tile_rows, min(a.tile_rows, total - t * a.tile_rows), 0);
  if (tid == 0) *a.plan.n_tiles = ntiles;
  return true;
}

__device__ __forceinline__ void plan_block(const PrepArgs &a, int *lds) {
  if (plan_segments(a, lds)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ml = a.has_lora ? a.rd.max_loras : 0;
  const int NG = a.rt.n_experts;
  const int NK = NG * (ml + 1);
  int *cnt = lds;            // [NK+1] counts, then starts
  int *fill = cnt + NK + 1;  // [NK]
  int *gt = fill + NK;       // [NG+1] tiles per group, then tile starts
  int *wsum = gt + NG + 1;   // [4]
  int *pk = wsum + 4;        // [n] the rows' packed routes
  for (int k = tid; k < NK + 1; k += 256) cnt[k] = 0;
  for (int k = tid; k < NK; k += 256) fill[k] = 0;
  if (a.routes) {  // eight loads per thread in flight at a time
    for (int r0 = tid; r0 < a.n; r0 += 256 * 8) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = r0 + 256 * j < a.n ? a.routes[r0 + 256 * j] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (r0 + 256 * j < a.n) pk[r0 + 256 * j] = v[j];
    }
  } else {  // no route buffer (the standalone shrink): route here
    for (int r0 = 0; r0 < a.n; r0 += 256 * 8) route_all(a, pk, nullptr, r0);
  }
  __syncthreads();
  count_rows(pk, a.n, cnt, [](int w) { return pk_key(w); });
  __syncthreads();
  const int total = block_exscan(cnt, NK, wsum);
  if (tid == 0) cnt[NK] = total;
  __syncthreads();
  // scatter: each run of equal keys in a wave's 64 rows takes its places
  // with one atomic (its rows keep their order)
  for (int r0 = wave * 64; r0 < a.n; r0 += 256) {
    const int r = r0 + lane;
    const int w = r < a.n ? pk[r] : 0;
    const int k = r < a.n ? pk_key(w) : -1;
    const uint64_t bnds = run_starts(k, lane);
    int base = 0;
    if (k >= 0 && ((bnds >> lane) & 1ull)) base = atomicAdd(&fill[k], run_end(bnds, lane) - lane);
    const int rs = run_start(bnds, lane);
    base = __shfl(base, rs, 64);
    if (k >= 0) {
      const int pos = cnt[k] + base + (lane - rs);
      a.plan.pos_row[pos] = r;
      a.plan.pos_pair[pos] = pk_pair(w);
    }
  }
  __syncthreads();
  // row tiles: group g owns sorted positions [cnt[g*(ml+1)], cnt[(g+1)*(ml+1)])
  for (int g = tid; g < NG; g += 256) {
    const int len = cnt[(g + 1) * (ml + 1)] - cnt[g * (ml + 1)];
    gt[g] = (len + a.tile_rows - 1) / a.tile_rows;
  }
  __syncthreads();
  const int ntiles = block_exscan(gt, NG, wsum);
  for (int g = tid; g < NG; g += 256) {
    const int s0 = cnt[g * (ml + 1)];
    const int len = cnt[(g + 1) * (ml + 1)] - s0;
    for (int j = 0, t0 = gt[g]; j * a.tile_rows < len; ++j)
      a.plan.tiles[t0 + j] = make_int4(g, s0 + j * a.tile_rows, min(a.tile_rows, len - j * a.tile_rows), 0);
  }
  if (tid == 0) *a.plan.n_tiles = ntiles;
}

// Pair of row r (or kSkip / kDrop), from the LDS cache when the batch fits it.

// One shrink unit: up to 16 rows sharing one pair, over one k chunk.
// t_part[kz][row][0:R] = x[row, chunk] . A_pair[:, chunk]^T; the consumer sums
// the k_splits partials in kz order.

// The GEMM's copy of t: s * t split into a bf16 high part and the bf16
// rounding of what it leaves over (hi + lo carries s * t to ~16 bits).
__device__ __forceinline__ void store_tt(u16 *tt, int R, int row, int r, float s, const float *v, int nv) {
  u16 *dst = tt + (size_t)row * 2 * R;
  for (int e = 0; e < nv; ++e) {
    const float w = s * v[e];
    const u16 hi = f2bf(w);
    dst[r + e] = hi;
    dst[R + r + e] = f2bf(w - bf2f(hi));
  }
}

// REG: the unit's operands go straight into registers, all of a 512-column
// chunk's in flight at once (fewer round trips on large units; 236
// registers, two workgroups per CU); otherwise by LDS-DMA in batches of
// kShrinkStages stages (three workgroups per CU).
template <bool REG>
__device__ __forceinline__ void shrink_unit(const PrepArgs &a, int u, int *lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.n_pairs;
  const int KS = a.k_splits;
  const int kz = u % KS;
  u /= KS;
  int *cnt = lds;             // [P]
  int *wsum = cnt + P;        // [4]
  int *info = wsum + 4;       // [4]
  int *rows = info + 4;       // [kShrinkRows]
  // [kShrinkStages][128 rows][8] stages, or (REG) the waves' sums
  uint4 *stg = (uint4 *)(lds + ((P + 8 + kShrinkRows + 3) & ~3));
  int *pk = (int *)(stg + kShrinkLdsBytes / 16);  // [n] the rows' packed routes (standalone shrink)

  // the pairs' row counts, read once, wait in the staging space until the
  // unit's own count has been taken from them
  int *raw = (int *)stg;
  static_assert(kMaxKeys * 4 <= kShrinkLdsBytes, "every pair's count fits the staging space");
  const bool ranked = a.ranks != nullptr;  // the route kernel counted and ranked the rows
  // A segmented call over at most 64 segments whose bounds never decrease,
  // without the route kernel: a pair's rows are its segments' rows in
  // segment order, so the counts and each unit's rows follow from the
  // segments alone (segment g: rows [lo, hi) clamped to the batch, the rows
  // segment_of assigns it when the bounds never decrease).
  int *s_lo = raw + kMaxKeys, *s_len = s_lo + 64, *s_q = s_len + 64, *s_ok = s_q + 64;
  static_assert((kMaxKeys + 3 * 64 + 1) * 4 <= kShrinkLdsBytes, "the segment table fits beside the counts");
  bool seg_ok = false;
  if (!ranked && a.seg_units) {
    for (int p = tid; p < P; p += 256) raw[p] = 0;
    __syncthreads();
    if (tid < 64) {
      const Routing &rt = a.rt;
      const bool in = lane < rt.n_seg;
      const int ilo = in ? rt.seg_indptr[lane] : 0, ihi = in ? rt.seg_indptr[lane + 1] : 0;
      const int slot = in ? rt.seg_slot[lane] : -1;
      const int q = in && a.has_lora ? resolve_slot(slot, 0, a.rd.max_loras, a.rd.n_experts, a.rd.a_table,
                                                    a.rd.b_table, a.rd.scale_table)
                                     : kSkip;
      const int lo = min(max(ilo, 0), a.n), hi = min(max(ihi, 0), a.n);
      const int len = in ? max(hi - lo, 0) : 0;
      s_lo[lane] = lo;
      s_len[lane] = len;
      s_q[lane] = q;
      const uint64_t bad = __ballot(in && ilo > ihi);
      if (lane == 0) s_ok[0] = bad == 0ull;
      if (bad == 0ull && q >= 0 && len > 0) atomicAdd(&raw[q], len);
    }
    __syncthreads();
    seg_ok = s_ok[0] != 0;  // uniform
  }
  if (ranked) {
    for (int p = tid; p < P; p += 256) {
      const int c = (int)a.pair_cnt[p];
      raw[p] = c;
      cnt[p] = (c + kShrinkRows - 1) / kShrinkRows;
    }
  } else if (seg_ok) {
    for (int p = tid; p < P; p += 256) cnt[p] = (raw[p] + kShrinkRows - 1) / kShrinkRows;
  } else {  // the standalone shrink: route and count here
    for (int p = tid; p < P; p += 256) cnt[p] = 0;
    for (int r0 = 0; r0 < a.n; r0 += 256 * 8) route_all(a, pk, nullptr, r0);
    __syncthreads();
    count_rows(pk, a.n, cnt, [](int w) { return pk_pair(w); });
    __syncthreads();
    for (int p = tid; p < P; p += 256) cnt[p] = (cnt[p] + kShrinkRows - 1) / kShrinkRows;
  }
  __syncthreads();
  const int n_units = block_exscan(cnt, P, wsum);
  if (u >= n_units) return;  // uniform: every thread saw the same total
  if (tid == 0) {
    int lo = 0, hi = P - 1;  // last pair whose first unit is <= u
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cnt[mid] <= u) lo = mid; else hi = mid - 1;
    }
    info[0] = lo;
    info[1] = u - cnt[lo];
  }
  // every slot of rows[] holds a row index or -1 before anyone looks for rows:
  // a count that disagrees with the rows found (a workspace that was not
  // zeroed, a call cut short between the route and prep launches) then
  // leaves -1 entries, which read row 0 and store nothing, never an address
  // outside the operands
  if (tid < kShrinkRows) rows[tid] = -1;
  __syncthreads();
  const int pstar = info[0];
  const int first = info[1] * kShrinkRows;
  // the pair's table entry and scale go out now, beside the row lookups
  const u16 *A = (const u16 *)a.rd.a_table[pstar];
  const float sig = a.rd.scale_table[pstar / a.rd.n_experts];

  if (ranked) {  // the rows of pstar whose rank falls in [first, first + kShrinkRows)
    const int total = raw[pstar];
    const int want = min(kShrinkRows, total - first);
    // a grouped call's pair lives in its expert's row range, a segmented
    // call's usually in the first segment bound to its adapter: scan only
    // that, and the whole batch if the range does not hold every wanted row
    // (offsets that are not non-decreasing, an adapter on several segments)
    int r_lo = 0, r_hi = a.n;
    bool direct = false;  // pstar's rows are exactly one segment's rows
    if (a.rt.mode == kModeMoeGrouped) {
      const int e = pstar % a.rd.n_experts;
      r_lo = min(max(a.rt.expert_offsets[e], 0), a.n);
      r_hi = min(max(a.rt.expert_offsets[e + 1], r_lo), a.n);
    } else if (a.rt.mode == kModeSegmented && a.rt.n_seg <= kSegScan) {
      // pairs of a segmented call are pool slots (one W group); the first
      // segment bound to pstar: lane g of every wave reads segment g's slot
      // and bounds, all in one round trip
      const bool in = lane < a.rt.n_seg;
      const int gs = in ? a.rt.seg_slot[lane] : -1;
      const int glo = in ? a.rt.seg_indptr[lane] : 0, ghi = in ? a.rt.seg_indptr[lane + 1] : 0;
      const uint64_t hit = __ballot(gs == pstar);
      if (hit) {  // uniform
        const int g = __ffsll((unsigned long long)hit) - 1;
        r_lo = min(max(__builtin_amdgcn_readlane(glo, g), 0), a.n);
        r_hi = min(max(__builtin_amdgcn_readlane(ghi, g), r_lo), a.n);
      }
      // every row of a segment routes alike, so when the pair's row count is
      // the segment's, its rows are that segment's: this unit takes the
      // positions [first, first + want) of the segment (a partition of the
      // pair's rows like the ranks', and each row's t is its own)
      direct = r_hi - r_lo == total;
    }
    if (direct) {
      if (tid < want) rows[tid] = r_lo + first + tid;
      if (tid == 0) info[3] = total;
    } else if (a.bucket != nullptr && pstar < a.bucket_pairs && first == 0 && total <= kShrinkRows) {
      // every row of the pair is in its bucket (the route kernel's, by
      // rank); an entry outside the batch (a stale workspace) reads row 0
      // and stores nothing
      if (tid < want) {
        const int r = a.bucket[pstar * kShrinkRows + tid];
        rows[tid] = r >= 0 && r < a.n ? r : -1;
      }
      if (tid == 0) info[3] = total;
      direct = true;
    }
    for (int pass = 0; pass < 2 && !direct; ++pass) {
      __syncthreads();  // every thread has read the last pass's count
      if (tid == 0) info[2] = 0;
      __syncthreads();
      int found = 0;
      for (int r0 = r_lo + tid; r0 < r_hi; r0 += 256 * 8) {
        int rk[8], w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool in = r0 + 256 * j < r_hi;
          rk[j] = in ? a.ranks[r0 + 256 * j] : -1;
          w[j] = in ? a.routes[r0 + 256 * j] : 0;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (rk[j] >= first && rk[j] < first + kShrinkRows && pk_pair(w[j]) == pstar) {
            rows[rk[j] - first] = r0 + 256 * j;
            ++found;
          }
      }
      if (found) atomicAdd(&info[2], found);
      __syncthreads();
      if (info[2] == want || (r_lo == 0 && r_hi == a.n)) break;  // uniform
      r_lo = 0;
      r_hi = a.n;
    }
    if (tid == 0 && !direct) info[3] = total;
  } else if (seg_ok) {
    // segment g holds the pair's positions [pre, pre + len) (an exclusive
    // scan over the pair's segments in order); this unit takes [first,
    // first + kShrinkRows)
    if (tid < 64) {
      const int len = s_len[lane], lo = s_lo[lane];
      const int v = s_q[lane] == pstar && len > 0 ? len : 0;
      int pre = v;
  #pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(pre, off, 64);
        if (lane >= off) pre += t;
      }
      const int total = __shfl(pre, 63, 64);
      pre -= v;
      const int b0 = max(first, pre), b1 = min(first + kShrinkRows, pre + v);
      for (int pos = b0; pos < b1; ++pos) rows[pos - first] = lo + (pos - pre);
      if (lane == 0) info[3] = total;
    }
  } else {
    // rows of pstar in row order, ranks [first, first + kShrinkRows): thread t
    // counts them in its 16-row span, an exclusive scan gives its first rank
    constexpr int SPAN = 16;
    int c = 0;
    // every thread runs the same number of rounds (the barriers inside)
    for (int base = 0; base < a.n; base += 256 * SPAN) {
      const int r0 = base + tid * SPAN;
      int mine = 0;
#pragma unroll
      for (int j = 0; j < SPAN; ++j) mine += r0 + j < a.n && pk_pair(pk[r0 + j]) == pstar;
      int pre = mine;  // inclusive scan over the block, then over earlier spans
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(pre, off, 64);
        if (lane >= off) pre += t;
      }
      if (lane == 63) wsum[wave] = pre;
      __syncthreads();
      int wpre = 0;
      for (int w = 0; w < wave; ++w) wpre += wsum[w];
      const int round_total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
      int k = c + wpre + pre - mine;  // rank of this span's first match
      for (int j = 0; j < SPAN && mine; ++j) {
        if (r0 + j < a.n && pk_pair(pk[r0 + j]) == pstar) {
          if (k >= first && k < first + kShrinkRows) rows[k - first] = r0 + j;
          ++k;
        }
      }
      c += round_total;
      __syncthreads();
    }
    if (tid == 0) info[3] = c;
  }
  __syncthreads();
  const int nrows = max(0, min(kShrinkRows, info[3] - first));

  // a stale count may name a pair that has no table entry: nothing to shrink
  // (uniform over the workgroup)
  if (A == nullptr || nrows == 0) return;
  const int R = a.rd.R, K = a.k_in;
  const int G = (nrows + 15) / 16;  // row groups of 16 (<= kShrinkRows / 16)
  // this unit's k chunk, in 64-wide stages
  const int chunk = ((K + KS - 1) / KS + 127) / 128 * 128;
  const int kc0 = min(kz * chunk, K), kc1 = min(kc0 + chunk, K);
  const int nst = (kc1 - kc0 + 63) / 64;
  // k_splits == 1: this unit writes the final t.  Otherwise it writes its
  // partial through device-coherent stores and the last of the unit's
  // k_splits workgroups to arrive sums them in chunk order.
  float *tout = KS == 1 ? a.t_final : a.t + (size_t)kz * a.n * R;
  const auto prs = coherent_rsrc(a.t, (uint32_t)((size_t)KS * a.n * R * 4));  // the k-chunk partials

  if constexpr (REG) {
    // 64 ranks at a time.  The chunk's 32-column steps are shared out over the
    // four waves (wave w: steps w, w + 4, ...).  Per step a wave loads, straight
    // into MFMA operand layout, the group's rank rows of A (one 16-byte load
    // per 16-rank block: lane l holds rank 16 rb + l % 16, columns 8 (l / 16)
    // .. + 7 of the step) and the unit's gathered x rows (one per 16-row
    // group, the same way), kShrinkSteps steps' loads in flight together, and
    // accumulates D[16 ranks][16 rows] per (rank block, row group).  Wave w
    // then adds rank block w's sums of the four waves in wave order: its own
    // from registers, the other three's from LDS (block (w', rb), w' != rb, at
    // slot 3 rb + w' - (w' > rb)).
    const int nstep = (kc1 - kc0 + 31) / 32;
    f32x4 *red = (f32x4 *)stg;  // [12 blocks][4 row groups][64 lanes]
    int xrow[kShrinkRows / 16];  // this lane's x row per group (row 0 where none: never stored)
  #pragma unroll
    for (int g = 0; g < kShrinkRows / 16; ++g) {
      const int i = g * 16 + (lane & 15);
      const int r = i < nrows ? rows[i] : -1;
      xrow[g] = r < 0 ? 0 : r;
    }
    for (int rg = 0; rg * 64 < R; ++rg) {
      const int RB = min(64, R - rg * 64) / 16;  // rank blocks of the group
      f32x4 acc[4][kShrinkRows / 16];
  #pragma unroll
      for (int rb = 0; rb < 4; ++rb)
  #pragma unroll
        for (int g = 0; g < kShrinkRows / 16; ++g) acc[rb][g] = f32x4{0.f, 0.f, 0.f, 0.f};
      const u16 *Ag = A + (size_t)(rg * 64 + (lane & 15)) * K;
      for (int j0 = 0; wave + 4 * j0 < nstep; j0 += kShrinkSteps) {
        uint4 af[kShrinkSteps][4], xf[kShrinkSteps][kShrinkRows / 16];
  #pragma unroll
        for (int d = 0; d < kShrinkSteps; ++d) {
          const int st = wave + 4 * (j0 + d);
          const bool live = st < nstep;  // uniform over the wave
          const int k = kc0 + st * 32 + (lane >> 4) * 8;
          const bool in = live && k < kc1;  // k_in is a multiple of 8: a lane's 8 columns are all in or all out
          const int kk = in ? k : kc0;
  #pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            af[d][rb] = live && rb < RB ? ldg16(Ag + (size_t)rb * 16 * K + kk) : z4();
            if (!in) af[d][rb] = z4();
          }
  #pragma unroll
          for (int g = 0; g < kShrinkRows / 16; ++g) {
            xf[d][g] = live && g < G ? ldg16(a.x + (size_t)xrow[g] * a.x_stride + kk) : z4();
            if (!in) xf[d][g] = z4();
          }
        }
  #pragma unroll
        for (int d = 0; d < kShrinkSteps; ++d) {
          if (wave + 4 * (j0 + d) >= nstep) break;
  #pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            if (rb >= RB) break;
  #pragma unroll
            for (int g = 0; g < kShrinkRows / 16; ++g) {
              if (g >= G) break;
              acc[rb][g] = mfma16(af[d][rb], xf[d][g], acc[rb][g]);
            }
          }
        }
      }
      __syncthreads();  // the last rank group's sums are read
  #pragma unroll
      for (int rb = 0; rb < 4; ++rb)
  #pragma unroll
        for (int g = 0; g < kShrinkRows / 16; ++g)
          if (rb != wave && rb < RB && g < G)
            red[((3 * rb + wave - (wave > rb)) * 4 + g) * 64 + lane] = acc[rb][g];
      __syncthreads();
      if (wave < RB) {  // wave w: rank block w, every row group, the four waves' sums in order
  #pragma unroll
        for (int g = 0; g < kShrinkRows / 16; ++g) {
          const int i = g * 16 + (lane & 15);
          if (g >= G || i >= nrows || rows[i] < 0) continue;
          const f32x4 own = wave == 0 ? acc[0][g] : wave == 1 ? acc[1][g] : wave == 2 ? acc[2][g] : acc[3][g];
          f32x4 v = wave == 0 ? own : red[((3 * wave + 0) * 4 + g) * 64 + lane];
  #pragma unroll
          for (int w = 1; w < 4; ++w) v += w == wave ? own : red[((3 * wave + w - (w > wave)) * 4 + g) * 64 + lane];
          // D column = lane%16 (the row), D rows = ranks 4*(lane/16) .. +3 of the wave's block
          const int rk = rg * 64 + wave * 16 + (lane >> 4) * 4;
          float *dst = tout + (size_t)rows[i] * R + rk;
          if (KS == 1) {
            *(f32x4 *)dst = v;
            if (a.tt) {
              const float vv[4] = {v[0], v[1], v[2], v[3]};
              store_tt(a.tt, R, rows[i], rk, sig, vv, 4);
            }
          } else {  // 16-byte device-coherent store into this chunk's partial
            st16_coherent(prs, (uint32_t)((dst - a.t) * 4), 0, v);
          }
        }
      }
    }
  } else {
    // 64 ranks at a time.  A stage is 64 k columns of the group's rank rows of
    // A, then of the unit's x rows (gathered, 16 G of them), in whole 128-byte
    // lines by LDS-DMA (chunk c of row r at slot c ^ ((r >> 1) & 7)); a batch
    // of stages (as many as the staging space holds) goes out together, then
    // wave w takes rank block w through them, every row group, in k order.
    for (int rg = 0; rg * 64 < R; ++rg) {
      const int RA = min(64, R - rg * 64);  // rank rows of the group
      const int RU = RA + 16 * G;           // rows of a stage
      const int per = RU / 8;               // DMA instructions per stage
      f32x4 acc[kShrinkRows / 16];
  #pragma unroll
      for (int g = 0; g < kShrinkRows / 16; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      // as many stages to a batch as the staging space holds (at least
      // kShrinkStages): a unit of few rows and ranks takes its chunk in one
      const int SB = max(kShrinkStages, kShrinkLdsBytes / (RU * 128));
      for (int sb = 0; sb < nst; sb += SB) {
        const int nsn = min(SB, nst - sb), kb0 = kc0 + sb * 64;
        __syncthreads();  // the previous batch is read
        for (int ii = wave; ii < nsn * per; ii += 4) {
          const int st = ii / per, k8 = ii % per;
          const int rr = k8 * 8 + (lane >> 3);  // row of the stage
          const u16 *rowp = rr < RA ? A + (size_t)(rg * 64 + rr) * K
                                    : a.x + (size_t)max(rows[min(rr - RA, nrows - 1)], 0) * a.x_stride;
          const int kk = kb0 + st * 64 + ((lane & 7) ^ ((rr >> 1) & 7)) * 8;
          dma16(rowp + (kk < kc1 ? kk : kc0), lds_addr(stg + (st * RU + k8 * 8) * 8));
        }
        __builtin_amdgcn_s_waitcnt(0);
        if (kb0 + nsn * 64 > kc1) {  // zero what the last stage fetched past the chunk
          for (int ii = wave; ii < nsn * per; ii += 4) {
            const int st = ii / per, k8 = ii % per;
            const int rr = k8 * 8 + (lane >> 3);
            if (kb0 + st * 64 + ((lane & 7) ^ ((rr >> 1) & 7)) * 8 >= kc1) stg[(st * RU + k8 * 8) * 8 + lane] = z4();
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        }
        __syncthreads();
        if (wave * 16 < RA) {
          const int ra = wave * 16 + (lane & 15);
          for (int st = 0; st < nsn; ++st) {
            const uint4 *sl = stg + st * RU * 8;
  #pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int c = 4 * h + (lane >> 4);
              const uint4 av = sl[ra * 8 + (c ^ ((ra >> 1) & 7))];
  #pragma unroll
              for (int g = 0; g < kShrinkRows / 16; ++g) {
                if (g >= G) break;
                const int rx = RA + g * 16 + (lane & 15);
                acc[g] = mfma16(av, sl[rx * 8 + (c ^ ((rx >> 1) & 7))], acc[g]);
              }
            }
          }
        }
      }
      if (wave * 16 < RA) {
  #pragma unroll
        for (int g = 0; g < kShrinkRows / 16; ++g) {
          const int i = g * 16 + (lane & 15);
          if (g >= G || i >= nrows || rows[i] < 0) continue;
          // D column = lane%16 (the row), D rows = ranks 4*(lane/16) .. +3 of the wave's block
          const int rk = rg * 64 + wave * 16 + (lane >> 4) * 4;
          float *dst = tout + (size_t)rows[i] * R + rk;
          const f32x4 v = acc[g];
          if (KS == 1) {
            *(f32x4 *)dst = v;
            if (a.tt) {
              const float vv[4] = {v[0], v[1], v[2], v[3]};
              store_tt(a.tt, R, rows[i], rk, sig, vv, 4);
            }
          } else {  // 16-byte device-coherent store into this chunk's partial
            st16_coherent(prs, (uint32_t)((dst - a.t) * 4), 0, v);
          }
        }
      }
    }
  }
  if (KS == 1) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    info[2] = __hip_atomic_fetch_add(&a.counters[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(KS - 1);
  __syncthreads();
  if (!info[2]) return;
  // the last of the unit's workgroups: t = sum of the k-chunk partials in
  // chunk order; a thread's pieces (kSumIt at a time: with REG all of a
  // 64-row unit's at rank 64, within the registers that path has anyway)
  // have every chunk's 16-byte load in flight together before any is summed
  constexpr int kSumIt = REG ? 4 : 2;
  for (int e0 = tid * 4; e0 < nrows * R; e0 += 256 * 4 * kSumIt) {
    f32x4 v[kSumIt][kMaxShrinkSplits];
    size_t off[kSumIt];
    bool ok[kSumIt];
#pragma unroll
    for (int it = 0; it < kSumIt; ++it) {
      const int e = e0 + it * 256 * 4;
      const int i = min(e / R, nrows - 1), r = e - (e / R) * R;
      ok[it] = e < nrows * R && rows[i] >= 0;
      off[it] = ok[it] ? (size_t)rows[i] * R + r : 0;
#pragma unroll
      for (int z = 0; z < kMaxShrinkSplits; ++z)
        v[it][z] = ok[it] && z < KS
                       ? ld16_coherent(prs, (uint32_t)(off[it] * 4), (uint32_t)((size_t)z * a.n * R * 4))
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int it = 0; it < kSumIt; ++it) {
      if (!ok[it]) continue;
      f32x4 sum = v[it][0];
#pragma unroll
      for (int z = 1; z < kMaxShrinkSplits; ++z)
        if (z < KS) sum += v[it][z];
      *(f32x4 *)(a.t_final + off[it]) = sum;
      if (a.tt) {
        const int e = e0 + it * 256 * 4;
        const float vv[4] = {sum[0], sum[1], sum[2], sum[3]};
        store_tt(a.tt, R, rows[e / R], e - (e / R) * R, sig, vv, 4);
      }
    }
  }
  if (tid == 0) __hip_atomic_store(&a.counters[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Every row's packed route, once per call (the plan and the shrink units read
// it instead of routing all rows again in each workgroup): one row per
// thread, so that each thread's chain of dependent loads and rank atomics is
// as short as it can be.
__global__ __launch_bounds__(256) void route_kernel(PrepArgs a) {
  __shared__ int seg[kSegLds];
  const bool sl = seg_in_lds(a.rt);
  if (sl) {
    const int32_t *starts = range_starts(a.rt);
    for (int g = threadIdx.x; g <= range_count(a.rt); g += 256) seg[g] = starts[g];
  }
  __syncthreads();
  route_all<1>(a, a.routes, sl ? seg : nullptr, (int)blockIdx.x * 256, a.ranks != nullptr);
}

// The plan is workgroup plan_at: the first, or after the units that fill
// the device's first round (with two units per CU those then all run in the
// first round, and the plan takes the first slot a unit frees, ahead of any
// unit slots past the batch's actual units).
template <bool REG>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  extern __shared__ int lds[];
  const int pb = a.plan_at;
  if (a.do_plan && (int)blockIdx.x == pb)
    plan_block(a, lds);
  else
    shrink_unit<REG>(a, (int)blockIdx.x - (a.do_plan && (int)blockIdx.x > pb ? 1 : 0), lds);
  if (a.ranks == nullptr) return;
  // every workgroup has read the pair counts once all have arrived: the last
  // one zeroes them (and the arrival count) for the next call
  __syncthreads();
  __shared__ int last;
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(a.prep_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  for (int p = threadIdx.x; p < a.n_pairs; p += 256) a.pair_cnt[p] = 0u;
  if (threadIdx.x == 0) *a.prep_done = 0u;
}

// A stack's further levels: every level's shrink units in one grid.
__global__ __launch_bounds__(256) void shrink_levels_kernel(ShrinkLevels s) {
  extern __shared__ int lds[];
  const int l = (int)blockIdx.x / s.blocks_per_level;
  shrink_unit<false>(s.lv[l], (int)blockIdx.x - l * s.blocks_per_level, lds);
}

size_t prep_lds_bytes(const PrepArgs &a) {
  const int ml = a.has_lora ? a.rd.max_loras : 0;
  const int NG = a.rt.n_experts;
  const int NK = NG * (ml + 1);
  // (the segmented plan's five 64-entry arrays fit beside any n)
  size_t plan = a.do_plan ? (size_t)(2 * NK + NG + 8 + std::max(a.n, 5 * 64)) * 4 : 0;
  size_t shr = a.n_units ? (size_t)((a.n_pairs + 8 + kShrinkRows + 3) & ~3) * 4 + (size_t)kShrinkLdsBytes +
                               (a.ranks ? 0 : (size_t)a.n * 4)
                         : 0;
  return plan > shr ? plan : shr;
}

hipError_t launch_shrink_levels(const ShrinkLevels &s, hipStream_t st) {
  if (s.n_levels <= 0 || s.blocks_per_level <= 0) return hipSuccess;
  size_t lds = 0;
  for (int l = 0; l < s.n_levels; ++l) {
    const size_t b = prep_lds_bytes(s.lv[l]);
    lds = b > lds ? b : lds;
  }
  hipLaunchKernelGGL(shrink_levels_kernel, dim3(s.n_levels * s.blocks_per_level), dim3(256), lds, st, s);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs &a, hipStream_t st) {
  const int grid = a.do_plan + a.n_units * a.k_splits;
  if (grid == 0) return hipSuccess;
  if (a.routes) hipLaunchKernelGGL(route_kernel, dim3((a.n + 255) / 256), dim3(256), 0, st, a);
  if (a.reg_units)
    hipLaunchKernelGGL(prep_kernel<true>, dim3(grid), dim3(256), prep_lds_bytes(a), st, a);
  else
    hipLaunchKernelGGL(prep_kernel<false>, dim3(grid), dim3(256), prep_lds_bytes(a), st, a);
  return hipGetLastError();
}

}  // namespace lora
