// k_bgmv.hip -- the standalone two-step delta for decode-sized batches:
//
//   shrink:       t_i = A_s x_i                     (lora_shrink)
//   expand+fold:  y_i = y_i + s_s (B_s t_i)         (lora_expand_fold)
//
// for every row i whose slot s resolves (ferrox-core "weight_matrix/lora.rs",
// module doc, the project and accumulate steps; atlas "lora_delta.rs",
// apply_lora_bgmv doc: kernel 1 the shrink, kernel 2 the expand-and-fold).
//
// Both kernels take their work by pool slot, not by row: a workgroup owns
// one slot, gathers the rows that resolve to it (a scan of seq_slot with
// ballots, which suits batches of up to a few hundred rows), and reads
// that slot's A or B once for all of them.  Every global access is a
// 16-byte load or store of consecutive elements.
//
//  * shrink: workgroup (s, r) = rank r of slot s, four waves that split
//    k_in into 512-column steps; lane l takes columns 8 l of each step of
//    A's row and of each row of x, so a wave reads whole 1 KiB stretches.
//    A's row goes out before the slot's rows are known, then x for eight
//    rows at a time (four in the levels kernel).  A lane sums its columns in k order (bf16 pair dot
//    products into f32), the wave adds its 64 sums with a butterfly of lane
//    shuffles and wave 0 adds the four waves' in order.
//  * expand+fold: workgroup (c, s) = 512 outputs of slot s; lane l of each
//    wave owns outputs 8 l .. 8 l + 7 of the chunk, whose B rows (8 x R
//    contiguous elements) it reads with 16-byte loads before the rows are
//    known, holding them in registers for every row when R <= 16; wave w
//    takes the slot's rows w, w + 4, ..., two at a time with their y and t
//    loads together.  The rank sum runs in f32, ranks ascending; y is read,
//    s times the sum added in f32 and rounded once.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

namespace {

constexpr int kExpandOut = 512;

// The rows i < n with seq_slot[i] == s, in index order, into rows[]; one
// wave.  v0 is this lane's seq_slot[lane] (or -1 past n), loaded by the
// caller ahead of everything else.  Returns their count.
__device__ __forceinline__ int gather_rows(const int32_t *seq_slot, int n, int s, int *rows, int v0) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  int cnt = 0;
  for (int b = 0; b < n; b += 64) {
    const int i = b + lane;
    const bool hit = i < n && (b == 0 ? v0 : seq_slot[i]) == s;
    const uint64_t m = __ballot(hit);
    if (hit) rows[cnt + (int)__popcll(m & below)] = i;
    cnt += (int)__popcll(m);
  }
  return cnt;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum over the 8 bf16 pairs of a and b, in f32, added to acc in pairs
// (v_dot2: each pair's two products, exact in f32, and acc)
__device__ __forceinline__ float dot8(uint4 a, uint4 b, float acc) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, av[e]), __builtin_bit_cast(bf16x2, bv[e]), acc,
                                          false);
  return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// The slot's table entries by the resolve rule, or false.
__device__ __forceinline__ bool slot_live(const RouteDev &rd, int s) {
  return rd.a_table[s] != nullptr && rd.b_table[s] != nullptr && rd.scale_table[s] != 0.0f;
}

constexpr int kShrinkWaves = 4;

// Workgroup (s, r): rank r of slot s.  Wave w takes the 512-column k steps
// w, w + 4, ...; lane l the 8 columns 8 l of each step.  A lane's sum over
// its columns (k order), the wave's butterfly, then the four waves in order.
template <int RC>  // rows of the slot at a time
__device__ __forceinline__ void shrink_slot_rank(const RouteDev &rd, const int32_t *seq_slot, int n, const u16 *x,
                                                 int x_stride, int k_in, float *t, int s, int r) {
  __shared__ int rows[kBgmvMaxRows];
  __shared__ int s_cnt;
  __shared__ float part[kShrinkWaves][RC];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int v0 = wave == 0 && lane < n ? seq_slot[lane] : -1;  // in flight with the table reads
  if (!slot_live(rd, s)) return;  // the same for the whole workgroup
  const u16 *Ar = (const u16 *)rd.a_table[s] + (size_t)r * k_in;
  // A's row goes out before the rows are known: this wave's steps, KS at a time
  constexpr int KS = 4;  // k steps held
  const int kstep = 512 * kShrinkWaves;
  uint4 a[KS];
  auto load_a = [&](int kc) {
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      const int k0 = kc + q * kstep + wave * 512 + lane * 8;
      a[q] = k0 < k_in ? ldg16(Ar + k0) : z4();
    }
  };
  load_a(0);
  if (wave == 0) {
    const int c = gather_rows(seq_slot, n, s, rows, v0);
    if (lane == 0) s_cnt = c;
  }
  __syncthreads();
  const int cnt = s_cnt;
  for (int j0 = 0; j0 < cnt; j0 += RC) {
    const u16 *xr[RC];
#pragma unroll
    for (int c = 0; c < RC; ++c) xr[c] = x + (size_t)rows[min(j0 + c, cnt - 1)] * x_stride;
    float acc[RC] = {};
    for (int kc = 0; kc < k_in; kc += KS * kstep) {
      if (kc > 0 || j0 > 0) load_a(kc);
      uint4 xv[RC][KS];
#pragma unroll
      for (int c = 0; c < RC; ++c)
#pragma unroll
        for (int q = 0; q < KS; ++q) {
          const int k0 = kc + q * kstep + wave * 512 + lane * 8;
          xv[c][q] = k0 < k_in ? ldg16(xr[c] + k0) : z4();
        }
#pragma unroll
      for (int c = 0; c < RC; ++c)
#pragma unroll
        for (int q = 0; q < KS; ++q) acc[c] = dot8(a[q], xv[c][q], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < RC; ++c) {
      const float v = wave_sum(acc[c]);
      if (lane == 0) part[wave][c] = v;
    }
    __syncthreads();
    if (wave == 0 && lane < RC && j0 + lane < cnt) {
      float v = part[0][lane];
#pragma unroll
      for (int w = 1; w < kShrinkWaves; ++w) v += part[w][lane];
      t[(size_t)rows[j0 + lane] * rd.R + r] = v;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(64 * kShrinkWaves) void bgmv_shrink_kernel(RouteDev rd, const int32_t *seq_slot, int n,
                                                                         const u16 *x, int x_stride, int k_in,
                                                                         float *t) {
  shrink_slot_rank<8>(rd, seq_slot, n, x, x_stride, k_in, t, blockIdx.x / rd.R, blockIdx.x % rd.R);
}

// An adapter stack's further levels: level l takes workgroups
// [l blocks_per_level, (l + 1) blocks_per_level), (slot, rank) as above.
__global__ __launch_bounds__(64 * kShrinkWaves) void bgmv_shrink_levels_kernel(BgmvLevels L, const u16 *x,
                                                                                int x_stride, int k_in, int n) {
  const int l = blockIdx.x / L.blocks_per_level, b = blockIdx.x % L.blocks_per_level;
  const RouteDev &rd = L.rd[l];
  if (b >= rd.max_loras * rd.R) return;  // the same for the whole workgroup
  // four rows at a time here: eight measured slower on the stack's levels
  shrink_slot_rank<4>(rd, L.seq_slot[l], n, x, x_stride, k_in, L.t[l], b / rd.R, b % rd.R);
}

constexpr int kExpandWaves = 4;

// Workgroup (c, s): outputs 512 c .. 512 c + 511 of slot s; lane l of every
// wave owns outputs 8 l .. 8 l + 7 of them, and wave w the slot's rows
// w, w + 4, ...  KR ranks at a time; KEEP: B's 8 x R elements of the lane
// stay in registers over the rows (R <= KR); otherwise each row reads them
// again (from the cache).  Rows go RB at a time, their y and t loads
// together.
template <int KR, bool KEEP>
__global__ __launch_bounds__(64 * kExpandWaves) void bgmv_expand_kernel(RouteDev rd, const int32_t *seq_slot, int n,
                                                                         const float *t, u16 *y, int y_stride,
                                                                         int n_out) {
  __shared__ int rows[kBgmvMaxRows];
  __shared__ int s_cnt;
  const int s = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int v0 = wave == 0 && lane < n ? seq_slot[lane] : -1;  // in flight with the table reads
  if (!slot_live(rd, s)) return;
  const int o0 = blockIdx.x * kExpandOut + lane * 8;
  const bool live = o0 < n_out;
  const int R = rd.R;
  const u16 *Bl = (const u16 *)rd.b_table[s] + (size_t)(live ? o0 : 0) * R;  // outputs o0 .. o0 + 7, contiguous
  const float sc = rd.scale_table[s];
  uint4 bk[8][KR / 8];
  auto load_b = [&](int r0) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int h = 0; h < KR / 8; ++h)
        bk[j][h] = live && r0 + 8 * h < R ? ldg16(Bl + (size_t)j * R + r0 + 8 * h) : z4();
  };
  if (KEEP) load_b(0);  // before the rows are known
  if (wave == 0) {
    const int c = gather_rows(seq_slot, n, s, rows, v0);
    if (lane == 0) s_cnt = c;
  }
  __syncthreads();
  const int cnt = s_cnt;
  constexpr int RB = 2;
  for (int j0 = wave * RB; j0 < cnt; j0 += kExpandWaves * RB) {
    int ii[RB];
    uint4 yv[RB];
#pragma unroll
    for (int c = 0; c < RB; ++c) {
      ii[c] = __builtin_amdgcn_readfirstlane(rows[min(j0 + c, cnt - 1)]);
      yv[c] = live ? ldg16(y + (size_t)ii[c] * y_stride + o0) : z4();
    }
    float d[RB][8];
#pragma unroll
    for (int c = 0; c < RB; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) d[c][j] = 0.f;
    for (int r0 = 0; r0 < R; r0 += KR) {
      if (!KEEP) load_b(r0);
#pragma unroll
      for (int c = 0; c < RB; ++c) {
        const float *ti = t + (size_t)ii[c] * R + r0;
        float tr[KR];
#pragma unroll
        for (int e = 0; e < KR; e += 4) {
          const f32x4 t4 = r0 + e < R ? *(const f32x4 *)(ti + e) : f32x4{0.f, 0.f, 0.f, 0.f};
          tr[e] = t4[0];
          tr[e + 1] = t4[1];
          tr[e + 2] = t4[2];
          tr[e + 3] = t4[3];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int h = 0; h < KR / 8; ++h) {
            const uint32_t w[4] = {bk[j][h].x, bk[j][h].y, bk[j][h].z, bk[j][h].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              d[c][j] += bf2f((u16)(w[e] & 0xffffu)) * tr[8 * h + 2 * e];
              d[c][j] += bf2f((u16)(w[e] >> 16)) * tr[8 * h + 2 * e + 1];
            }
          }
      }
    }
#pragma unroll
    for (int c = 0; c < RB; ++c) {
      if (!live || j0 + c >= cnt) continue;
      const uint32_t yw[4] = {yv[c].x, yv[c].y, yv[c].z, yv[c].w};
      uint32_t ow[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf2f((u16)(yw[e] & 0xffffu)) + sc * d[c][2 * e];
        const float hi = bf2f((u16)(yw[e] >> 16)) + sc * d[c][2 * e + 1];
        ow[e] = pack2(f2bf(lo), f2bf(hi));
      }
      *(uint4 *)(y + (size_t)ii[c] * y_stride + o0) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
  }
}

}  // namespace

hipError_t launch_bgmv_shrink(const RouteDev &rd, const int32_t *seq_slot, int n, const u16 *x, int x_stride,
                              int k_in, float *t, hipStream_t st) {
  const int grid = rd.max_loras * rd.R;
  if (grid == 0 || n == 0) return hipSuccess;
  hipLaunchKernelGGL(bgmv_shrink_kernel, dim3(grid), dim3(64 * kShrinkWaves), 0, st, rd, seq_slot, n, x, x_stride,
                     k_in, t);
  return hipGetLastError();
}

hipError_t launch_bgmv_shrink_levels(const BgmvLevels &L, const u16 *x, int x_stride, int k_in, int n,
                                     hipStream_t st) {
  const int grid = L.n_levels * L.blocks_per_level;
  if (grid == 0 || n == 0) return hipSuccess;
  hipLaunchKernelGGL(bgmv_shrink_levels_kernel, dim3(grid), dim3(64 * kShrinkWaves), 0, st, L, x, x_stride, k_in, n);
  return hipGetLastError();
}

hipError_t launch_bgmv_expand(const RouteDev &rd, const int32_t *seq_slot, int n, const float *t, u16 *y,
                              int y_stride, int n_out, hipStream_t st) {
  const dim3 grid((n_out + kExpandOut - 1) / kExpandOut, rd.max_loras);
  if (rd.max_loras == 0 || n == 0) return hipSuccess;
  if (rd.R <= 16)
    hipLaunchKernelGGL((bgmv_expand_kernel<16, true>), grid, dim3(64 * kExpandWaves), 0, st, rd, seq_slot, n, t, y, y_stride, n_out);
  else
    hipLaunchKernelGGL((bgmv_expand_kernel<16, false>), grid, dim3(64 * kExpandWaves), 0, st, rd, seq_slot, n, t, y,
                       y_stride, n_out);
  return hipGetLastError();
}

}  // namespace lora
