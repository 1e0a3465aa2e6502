// k_prep.hip -- route resolve, the row plan, and the grouped MFMA shrink (bf16).
//
// One launch does two independent jobs:
//  * block 0 (when a plan is wanted) resolves every row's route (slot ->
//    pair or skip, atlas apply_lora_bgmv doc) and groups the rows by
//    (W group, adapter) with a counting sort in LDS, then cuts each W group
//    into the main kernel's row tiles.  Within a key the order is whatever
//    the LDS atomics give: no output value depends on it, because every
//    output element is reduced row-locally with the same instruction sequence.
//  * every other block is one shrink unit: up to 16 rows that share one
//    pair, t[rows] = x[rows] . A_pair^T (ferrox LoraDelta::project), on bf16
//    MFMA with f32 accumulation.  Each block finds its unit by histogramming
//    the pairs itself, so the shrink does not wait for the plan.  The four
//    waves split k_in; their partial sums meet in LDS in a fixed order.
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

// Exclusive prefix of one int per thread across the block; *total gets the sum.
__device__ int block_exclusive(int v0, int *wsum, int *total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v = v0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return pre + v - v0;
}

// Sort key of a row: W group major, then adapter, the skip bucket last in
// its group.  -1 for a row that is not written.
__device__ __forceinline__ int row_key(const PrepArgs &a, int r, int *pair) {
  int g, ad;
  const int q = row_route(a.rt, a.rd, a.has_lora, r, &g, &ad);
  *pair = q;
  if (q == kDrop) return -1;
  const int ml = a.has_lora ? a.rd.max_loras : 0;
  return g * (ml + 1) + (q >= 0 ? ad : ml);
}

__device__ void plan_block(const PrepArgs &a, int *lds) {
  const int tid = threadIdx.x;
  const int ml = a.has_lora ? a.rd.max_loras : 0;
  const int NG = a.rt.n_experts;
  const int NK = NG * (ml + 1);
  int *cnt = lds;            // [NK+1] counts, then starts
  int *fill = cnt + NK + 1;  // [NK]
  int *gt = fill + NK;       // [NG+1] tiles per group, then tile starts
  int *wsum = gt + NG + 1;   // [4]
  for (int k = tid; k < NK + 1; k += 256) cnt[k] = 0;
  for (int k = tid; k < NK; k += 256) fill[k] = 0;
  __syncthreads();
  for (int r = tid; r < a.n; r += 256) {
    int q;
    const int key = row_key(a, r, &q);
    if (key >= 0) atomicAdd(&cnt[key], 1);
  }
  __syncthreads();
  const int total = block_exscan(cnt, NK, wsum);
  if (tid == 0) cnt[NK] = total;
  __syncthreads();
  for (int r = tid; r < a.n; r += 256) {
    int q;
    const int key = row_key(a, r, &q);
    if (key < 0) continue;
    const int pos = cnt[key] + atomicAdd(&fill[key], 1);
    a.plan.pos_row[pos] = r;
    a.plan.pos_pair[pos] = q;
  }
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
__device__ __forceinline__ int cached_route(const PrepArgs &a, const int *qv, int r) {
  if (qv) return qv[r];
  int g, ad;
  return row_route(a.rt, a.rd, true, r, &g, &ad);
}

// One shrink unit: up to 16 rows sharing one pair, over one k chunk.
// t_part[kz][row][0:R] = x[row, chunk] . A_pair[:, chunk]^T; the consumer sums
// the k_splits partials in kz order.
__device__ void shrink_unit(const PrepArgs &a, int u, int *lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.n_pairs;
  const int KS = a.k_splits;
  const int kz = u % KS;
  u /= KS;
  int *cnt = lds;             // [P]
  int *wsum = cnt + P;        // [4]
  int *info = wsum + 4;       // [4]
  int *rows = info + 4;       // [16]
  f32x4 *red = (f32x4 *)(lds + ((P + 24 + 3) & ~3));  // [3][4][64]
  int *qv = a.n <= kRowCache ? (int *)(red + 3 * 4 * 64) : nullptr;  // [n]

  for (int p = tid; p < P; p += 256) cnt[p] = 0;
  __syncthreads();
  for (int r = tid; r < a.n; r += 256) {
    int g, ad;
    const int q = row_route(a.rt, a.rd, true, r, &g, &ad);
    if (qv) qv[r] = q;
    if (q >= 0) atomicAdd(&cnt[q], 1);
  }
  __syncthreads();
  for (int p = tid; p < P; p += 256) cnt[p] = (cnt[p] + kShrinkRows - 1) / kShrinkRows;
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
  __syncthreads();
  const int pstar = info[0];
  const int first = info[1] * kShrinkRows;

  // rows of pstar, in row order, ranks [first, first + 16)
  const int m = (a.n + 255) / 256;
  const int rb = min(tid * m, a.n), re = min(rb + m, a.n);
  int c = 0;
  for (int r = rb; r < re; ++r) c += cached_route(a, qv, r) == pstar;
  int total_rows;
  int k = block_exclusive(c, wsum, &total_rows);
  for (int r = rb; r < re && k < first + kShrinkRows; ++r) {
    if (cached_route(a, qv, r) != pstar) continue;
    if (k >= first) rows[k - first] = r;
    ++k;
  }
  __syncthreads();
  const int nrows = min(kShrinkRows, total_rows - first);

  const u16 *A = (const u16 *)a.rd.a_table[pstar];
  const int R = a.rd.R, nrb = R / 16, K = a.k_in;
  const int myrow = (lane & 15) < nrows ? rows[lane & 15] : -1;
  const u16 *xr = myrow >= 0 ? a.x + (size_t)myrow * a.x_stride : nullptr;
  // this unit's k chunk, cut in 32-wide steps; wave w takes steps w, w+4, ...
  const int chunk = ((K + KS - 1) / KS + 127) / 128 * 128;
  const int kc0 = min(kz * chunk, K), kc1 = min(kc0 + chunk, K);
  const int nsteps = (kc1 - kc0 + 31) / 32;
  const int koff = (lane >> 4) * 8;
  // k_splits == 1: this unit writes the final t.  Otherwise it writes its
  // partial through device-coherent (sc1) stores and the last of the unit's
  // k_splits workgroups to arrive sums them in chunk order.
  float *tout = KS == 1 ? a.t_final : a.t + (size_t)kz * a.n * R;

  for (int rb0 = 0; rb0 < nrb; rb0 += 4) {
    const int nb = min(4, nrb - rb0);
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const u16 *Ab = A + (size_t)(rb0 * 16 + (lane & 15)) * K;
    for (int s0 = wave; s0 < nsteps; s0 += 4 * 8) {
      uint4 xv[8], av[8][4];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int kk = kc0 + (s0 + 4 * s) * 32 + koff;
        const bool in = kk < kc1;
        xv[s] = (xr && in) ? ldg16(xr + kk) : z4();
#pragma unroll
        for (int j = 0; j < 4; ++j)
          av[s][j] = (in && j < nb) ? ldg16(Ab + (size_t)j * 16 * K + kk) : z4();
      }
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j < nb) acc[j] = mfma16(av[s][j], xv[s], acc[j]);
    }
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) red[((wave - 1) * 4 + j) * 64 + lane] = acc[j];
    }
    __syncthreads();
    if (wave == 0 && myrow >= 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j >= nb) continue;
        f32x4 v = acc[j];
        v += red[(0 * 4 + j) * 64 + lane];
        v += red[(1 * 4 + j) * 64 + lane];
        v += red[(2 * 4 + j) * 64 + lane];
        // D column = lane%16 (the row), D rows = ranks 4*(lane/16) .. +3 of block rb0+j
        float *dst = tout + (size_t)myrow * R + (rb0 + j) * 16 + (lane >> 4) * 4;
        if (KS == 1) {
          *(f32x4 *)dst = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __hip_atomic_store(dst + e, v[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();
  }
  if (KS == 1) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    info[2] = __hip_atomic_fetch_add(&a.counters[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(KS - 1);
  __syncthreads();
  if (!info[2]) return;
  for (int e = tid; e < nrows * R; e += 256) {
    const int i = e / R, r = e - i * R;
    const size_t off = (size_t)rows[i] * R + r;
    float v = 0.f;
    for (int z = 0; z < KS; ++z)
      v += __hip_atomic_load(a.t + (size_t)z * a.n * R + off, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.t_final[off] = v;
  }
  if (tid == 0) __hip_atomic_store(&a.counters[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  extern __shared__ int lds[];
  if (a.do_plan && blockIdx.x == 0) {
    plan_block(a, lds);
    return;
  }
  shrink_unit(a, (int)blockIdx.x - a.do_plan, lds);
}

size_t prep_lds_bytes(const PrepArgs &a) {
  const int ml = a.has_lora ? a.rd.max_loras : 0;
  const int NG = a.rt.n_experts;
  const int NK = NG * (ml + 1);
  size_t plan = a.do_plan ? (size_t)(2 * NK + NG + 8) * 4 : 0;
  size_t shr = a.n_units ? (size_t)((a.n_pairs + 24 + 3) & ~3) * 4 + 3 * 4 * 64 * 16 +
                               (a.n <= kRowCache ? (size_t)a.n * 4 : 0)
                         : 0;
  return plan > shr ? plan : shr;
}

hipError_t launch_prep(const PrepArgs &a, hipStream_t st) {
  const int grid = a.do_plan + a.n_units * a.k_splits;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(prep_kernel, dim3(grid), dim3(256), prep_lds_bytes(a), st, a);
  return hipGetLastError();
}

}  // namespace lora
