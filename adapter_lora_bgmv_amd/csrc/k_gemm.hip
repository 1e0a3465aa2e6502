// k_gemm.hip -- the fused apply: y = W x + s B (A x), bf16 MFMA, f32 accumulate.
//
// A workgroup owns an output tile of TO output features x TR rows (rows in
// the plan's grouped order, gathered from x and scattered to y).  The
// contraction over k_in runs on v_mfma_f32_16x16x32_bf16 with W as the A
// operand (output features) and the gathered x rows as the B operand; both
// tiles are staged through LDS in double-buffered 64-wide k slabs.
//
// The low-rank term rides the same accumulators as a k-extension that runs
// FIRST, before the base contraction (ferrox lora.rs "expand + fold"; atlas
// lora_delta.rs dense_gemm_tc_scaled_acc folds the scaled expand into the
// output the same way):
//     acc[o, i] += sum_kappa B_q[o, kappa] * T[i, kappa]
// where T holds s_q * t_i split into a bf16 high and low part (so the f32
// intermediate t is carried at ~16 mantissa bits), and rows of another pair,
// or skipped rows, contribute exact zeros.  Starting from +0, a skipped row's
// accumulator is still +0 when the base contraction begins, so its output is
// bit-identical to the base-only launch of the same shape.
//
// Split-K: `splits` workgroups share a tile, each over its own k range; the
// last to arrive (a device-scope counter) sums the partial tiles in split
// order and writes y, so results do not depend on arrival order.  The
// extension always runs in split 0.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

// The bf16 high part of v, or (part != 0) the bf16 rounding of what the
// high part leaves over; hi + lo carries v to about 16 significant bits.
__device__ __forceinline__ u16 hilo(float v, int part) {
  const u16 hi = f2bf(v);
  return part ? f2bf(v - bf2f(hi)) : hi;
}

template <int TO, int TR>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int BK = 64, PITCH = BK + 8;  // u16 per LDS row; +16 B breaks bank aliasing
  constexpr int WO = TO / 2, WR = TR / 2;
  constexpr int NBO = WO / 16, NBR = WR / 16;
  constexpr int NW = TO * 8 / 256, NX = TR * 8 / 256;  // 16-byte chunks per thread per slab
  static_assert(NW >= 1 && NX >= 1, "tile too small for 256 threads");
  __shared__ __attribute__((aligned(16))) u16 Ws[2][TO * PITCH];
  __shared__ __attribute__((aligned(16))) u16 Xs[2][TR * PITCH];
  __shared__ int s_row[TR], s_pair[TR];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wo = wave & 1, wr = wave >> 1;
  int bid = blockIdx.x;
  const int z = bid % p.splits;
  bid /= p.splits;
  const int nt = bid % p.n_ntiles;
  const int mt = bid / p.n_ntiles;
  if (mt >= *p.plan.n_tiles) return;
  const int4 tile = p.plan.tiles[mt];
  const int o0 = nt * TO;
  for (int i = tid; i < TR; i += 256) {
    const bool in = i < tile.z;
    s_row[i] = in ? p.plan.pos_row[tile.y + i] : -1;
    s_pair[i] = in ? p.plan.pos_pair[tile.y + i] : kSkip;
  }
  __syncthreads();

  f32x4 acc[NBO][NBR];
#pragma unroll
  for (int a = 0; a < NBO; ++a)
#pragma unroll
    for (int b = 0; b < NBR; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};


  // ---------------------------------------------------------- k-extension
  if (p.has_lora && z == 0) {
    const int R = p.R, nks = 2 * R / 32;
#pragma unroll
    for (int br = 0; br < NBR; ++br) {
      const int l0 = wr * WR + br * 16;
      const int myr = lane & 15;
      const int grow = s_row[l0 + myr];
      int i = 0;
      while (i < 16) {
        const int q = s_pair[l0 + i];
        int j = i + 1;
        while (j < 16 && s_pair[l0 + j] == q) ++j;
        if (q >= 0) {
          const u16 *Bq = (const u16 *)p.b_table[q];
          const float sig = p.scale_table[q / p.n_experts];
          const bool mine = myr >= i && myr < j && grow >= 0;
          for (int ks = 0; ks < nks; ++ks) {
            const int kap = ks * 32 + (lane >> 4) * 8;
            const int part = kap >= R;
            const int r0 = kap - part * R;
            uint4 tv = z4();
            if (mine) {
              const f32x4 t0 = *(const f32x4 *)(p.t + (size_t)grow * R + r0);
              const f32x4 t1 = *(const f32x4 *)(p.t + (size_t)grow * R + r0 + 4);
              tv = make_uint4(pack2(hilo(sig * t0[0], part), hilo(sig * t0[1], part)),
                              pack2(hilo(sig * t0[2], part), hilo(sig * t0[3], part)),
                              pack2(hilo(sig * t1[0], part), hilo(sig * t1[1], part)),
                              pack2(hilo(sig * t1[2], part), hilo(sig * t1[3], part)));
            }
#pragma unroll
            for (int bo = 0; bo < NBO; ++bo) {
              const int o = o0 + wo * WO + bo * 16 + (lane & 15);
              const uint4 bv = o < p.n_out ? ldg16(Bq + (size_t)o * R + r0) : z4();
              acc[bo][br] = mfma16(bv, tv, acc[bo][br]);
            }
          }
        }
        i = j;
      }
    }
  }

  // ---------------------------------------------------------- base contraction
  const int kb = min(z * p.k_per_split, p.k_in);
  const int ke = min(kb + p.k_per_split, p.k_in);
  const u16 *Wg = p.W + (size_t)tile.x * (size_t)p.w_group_stride;
  if (kb < ke) {
    uint4 wreg[NW], xreg[NX];
    auto gload = [&](int k0) {
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const int c = tid + 256 * j, r = c >> 3, kk = k0 + (c & 7) * 8;
        const int o = o0 + r;
        wreg[j] = (o < p.n_out && kk < ke) ? ldg16(Wg + (size_t)o * p.w_row_stride + kk) : z4();
      }
#pragma unroll
      for (int j = 0; j < NX; ++j) {
        const int c = tid + 256 * j, r = c >> 3, kk = k0 + (c & 7) * 8;
        const int row = s_row[r];
        xreg[j] = (row >= 0 && kk < ke) ? ldg16(p.x + (size_t)row * p.x_row_stride + kk) : z4();
      }
    };
    auto swrite = [&](int buf) {
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const int c = tid + 256 * j;
        *(uint4 *)&Ws[buf][(c >> 3) * PITCH + (c & 7) * 8] = wreg[j];
      }
#pragma unroll
      for (int j = 0; j < NX; ++j) {
        const int c = tid + 256 * j;
        *(uint4 *)&Xs[buf][(c >> 3) * PITCH + (c & 7) * 8] = xreg[j];
      }
    };
    gload(kb);
    swrite(0);
    __syncthreads();
    int cur = 0;
    for (int k0 = kb; k0 < ke; k0 += BK) {
      const bool more = k0 + BK < ke;
      if (more) gload(k0 + BK);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int col = ks * 32 + (lane >> 4) * 8;
        uint4 af[NBO], bf[NBR];
#pragma unroll
        for (int bo = 0; bo < NBO; ++bo)
          af[bo] = *(const uint4 *)&Ws[cur][(wo * WO + bo * 16 + (lane & 15)) * PITCH + col];
#pragma unroll
        for (int br = 0; br < NBR; ++br)
          bf[br] = *(const uint4 *)&Xs[cur][(wr * WR + br * 16 + (lane & 15)) * PITCH + col];
#pragma unroll
        for (int bo = 0; bo < NBO; ++bo)
#pragma unroll
          for (int br = 0; br < NBR; ++br) acc[bo][br] = mfma16(af[bo], bf[br], acc[bo][br]);
      }
      if (more) swrite(cur ^ 1);
      __syncthreads();
      cur ^= 1;
    }
  }

  // ---------------------------------------------------------- split-K fixup
  if (p.splits > 1) {
    constexpr int TT = TO * TR;
    const int tl = mt * p.n_ntiles + nt;
    float *part = p.partials + (size_t)tl * p.splits * TT;
#pragma unroll
    for (int bo = 0; bo < NBO; ++bo)
#pragma unroll
      for (int br = 0; br < NBR; ++br) {
        const int idx = ((wave * NBO + bo) * NBR + br) * 64 + lane;
        *(f32x4 *)(part + (size_t)z * TT + idx * 4) = acc[bo][br];
      }
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&p.counters[tl], 1u) == (unsigned)(p.splits - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int bo = 0; bo < NBO; ++bo)
#pragma unroll
      for (int br = 0; br < NBR; ++br) {
        const int idx = ((wave * NBO + bo) * NBR + br) * 64 + lane;
        f32x4 s = *(const f32x4 *)(part + idx * 4);
        for (int zz = 1; zz < p.splits; ++zz) s += *(const f32x4 *)(part + (size_t)zz * TT + idx * 4);
        acc[bo][br] = s;
      }
    if (tid == 0) p.counters[tl] = 0u;
  }

  // ---------------------------------------------------------- epilogue
#pragma unroll
  for (int bo = 0; bo < NBO; ++bo) {
    const int o = o0 + wo * WO + bo * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int br = 0; br < NBR; ++br) {
      const int lr = wr * WR + br * 16 + (lane & 15);
      const int grow = s_row[lr];
      if (grow < 0 || o >= p.n_out) continue;
      const f32x4 v = acc[bo][br];
      uint2 pk = make_uint2(pack2(f2bf(v[0]), f2bf(v[1])), pack2(f2bf(v[2]), f2bf(v[3])));
      *(uint2 *)(p.y + (size_t)grow * p.y_row_stride + o) = pk;
    }
  }
}

hipError_t launch_gemm(const GemmArgs &a, int to, int tr, hipStream_t st) {
  const int grid = a.max_mtiles * a.n_ntiles * a.splits;
  if (grid == 0) return hipSuccess;
  if (to == 64 && tr == 64)
    hipLaunchKernelGGL((gemm_bf16_kernel<64, 64>), dim3(grid), dim3(256), 0, st, a);
  else if (to == 128 && tr == 64)
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 64>), dim3(grid), dim3(256), 0, st, a);
  else if (to == 128 && tr == 128)
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128>), dim3(grid), dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lora
