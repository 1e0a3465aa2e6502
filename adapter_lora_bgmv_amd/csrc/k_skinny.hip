// k_skinny.hip -- the fused apply for decode-shaped batches (n <= 64 rows).
//
// y_i = W x_i + s B_s (A_s x_i) when the whole batch is a few MFMA column
// blocks wide.  The cost is streaming W from HBM once, so the layout is
// chosen for that:
//  * one workgroup owns 16 output features (one MFMA row block of W) for
//    every row of the batch and the WHOLE k range -- no split-K, so there is
//    no partial tile, no cross-workgroup traffic and no counter;
//  * its 8 waves take interleaved 64-wide k steps (each reads whole 128-byte
//    lines of its rows) and keep two batches of two steps in flight, W
//    fragments loaded straight into MFMA registers;
//  * the 8 per-wave accumulators meet in LDS in a fixed order;
//  * the rank-sized delta, sum_r B_s[o, r] t_i[r], is a handful of f32 FMAs per
//    output and runs on the VALU in the epilogue, added to the base in f32
//    only for rows that resolve to a slot (skipped rows are stored from the
//    base accumulator untouched), then one rounding to bf16.
// The batch keeps its order (no plan kernel runs before this one); each
// workgroup resolves the batch's routes itself (n <= 64 loads) while its
// first W and x loads are in flight.  Only the shrink (t) must precede it.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

template <int NB>  // batch column blocks of 16 rows: n <= 16 * NB
__global__ __launch_bounds__(512) void skinny_bf16_kernel(SkinnyArgs p) {
  constexpr int NWAVE = 8, D = 4;
  constexpr int NR = 16 * NB;
  constexpr int TPT = (NR * kSkinnyMaxRank + 511) / 512;  // t values per thread
  constexpr int RB = kSkinnyMaxRank / 8;                   // 16-byte pieces of a B row
  __shared__ int s_pair[NR], s_sidx[NR];
  __shared__ f32x4 red[NWAVE][NB][64];
  __shared__ float s_base[NR][17];  // reduced base tile [row][o], padded
  __shared__ float s_t[NR * kSkinnyMaxRank];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int o0 = blockIdx.x * 16;
  const int K = p.k_in, R = p.R;
  // Lane group g = lane/16 owns k elements 16g .. 16g+15 of each 64-wide
  // double step and feeds them to two MFMAs (8 each); W and x use the same
  // assignment, so the product is unchanged, and the four groups together
  // read whole 128-byte lines of every row.
  const int koff = (lane >> 4) * 16;
  const int orow = o0 + (lane & 15);
  const u16 *wr = orow < p.n_out ? p.W + (size_t)orow * p.w_row_stride : nullptr;
  const int nsteps = (K + 63) / 64;  // 64-wide double steps
  // on this path the batch keeps its order: MFMA column i is row i
  const u16 *xr[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int r = b * 16 + (lane & 15);
    xr[b] = r < p.n ? p.x + (size_t)r * p.x_row_stride : nullptr;
  }

  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // wave w takes double steps w, w+8, w+16, ...; two batches in flight
  uint4 wa[D], xa[D][NB], wb[D], xb[D][NB];
#define SKINNY_LOAD(WV, XV, J0)                                                  \
  _Pragma("unroll") for (int d = 0; d < D; ++d) {                                \
    const int kk = (wave + NWAVE * ((J0) + d / 2)) * 64 + koff + (d & 1) * 8;    \
    const bool in = kk < K;                                                      \
    WV[d] = (wr && in) ? ldg16(wr + kk) : z4();                                  \
    _Pragma("unroll") for (int b = 0; b < NB; ++b)                               \
      XV[d][b] = (xr[b] && in) ? ldg16(xr[b] + kk) : z4();                       \
  }
#define SKINNY_MMA(WV, XV)                                                       \
  _Pragma("unroll") for (int d = 0; d < D; ++d)                                  \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) acc[b] = mfma16(WV[d], XV[d][b], acc[b]);

  constexpr int DS = D / 2;                            // double steps per batch
  const int nj = (nsteps - wave + NWAVE - 1) / NWAVE;  // double steps of this wave
  if (nj > 0) { SKINNY_LOAD(wa, xa, 0) }
  if (DS < nj) { SKINNY_LOAD(wb, xb, DS) }

  // routes and t, fetched while the first loads are in flight
  if (tid < NR) {
    int q = kSkip, sidx = 0;
    if (tid < p.n) {
      int g;
      q = row_route(p.rt, p.rd, p.has_lora, tid, &g, &sidx);
    }
    s_pair[tid] = q;
    s_sidx[tid] = sidx;
  }
  float tv[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int e = tid + 512 * j;
    tv[j] = (p.has_lora && e < p.n * R) ? p.t[e] : 0.f;  // [n][R] is flat in e
  }

  for (int j = 0; j < nj;) {
    SKINNY_MMA(wa, xa)
    j += DS;
    if (j >= nj) break;
    if (j + DS < nj) { SKINNY_LOAD(wa, xa, j + DS) }
    SKINNY_MMA(wb, xb)
    j += DS;
    if (j >= nj) break;
    if (j + DS < nj) { SKINNY_LOAD(wb, xb, j + DS) }
  }
#undef SKINNY_LOAD
#undef SKINNY_MMA

#pragma unroll
  for (int b = 0; b < NB; ++b) red[wave][b][lane] = acc[b];
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int e = tid + 512 * j;
    if (e < NR * R) s_t[e] = tv[j];
  }
  __syncthreads();

  // epilogue element of this thread: (row i, outputs o, o+1); its B rows are
  // fetched now so the loads overlap the reduction
  const int i = tid >> 3, oc = (tid & 7) * 2, o = o0 + oc;
  const bool live = i < p.n && o < p.n_out;
  const int q = live ? s_pair[i] : kSkip;
  uint4 bq0[RB], bq1[RB];
  if (q >= 0) {
    const u16 *Bq = (const u16 *)p.rd.b_table[q] + (size_t)o * R;
#pragma unroll
    for (int h = 0; h < RB; ++h) {
      bq0[h] = h * 8 < R ? ldg16(Bq + h * 8) : z4();
      bq1[h] = h * 8 < R ? ldg16(Bq + R + h * 8) : z4();
    }
  }

  if (wave < NB) {  // fixed-order reduction of the 8 waves' accumulators
    const int b = wave;
    f32x4 v = red[0][b][lane];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) v += red[w][b][lane];
    // D layout: column (row) = lane%16, rows (outputs) 4*(lane/16) .. +3
    const int ii = b * 16 + (lane & 15), oq = (lane >> 4) * 4;
    s_base[ii][oq + 0] = v[0];
    s_base[ii][oq + 1] = v[1];
    s_base[ii][oq + 2] = v[2];
    s_base[ii][oq + 3] = v[3];
  }
  __syncthreads();

  if (!live) return;
  float v0 = s_base[i][oc], v1 = s_base[i][oc + 1];
  if (q >= 0) {
    const float *ti = s_t + i * R;
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int h = 0; h < RB; ++h) {
      if (h * 8 >= R) break;
      const uint32_t w0[4] = {bq0[h].x, bq0[h].y, bq0[h].z, bq0[h].w};
      const uint32_t w1[4] = {bq1[h].x, bq1[h].y, bq1[h].z, bq1[h].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float ta = ti[h * 8 + 2 * c], tb = ti[h * 8 + 2 * c + 1];
        d0 += bf2f((u16)(w0[c] & 0xffffu)) * ta;
        d0 += bf2f((u16)(w0[c] >> 16)) * tb;
        d1 += bf2f((u16)(w1[c] & 0xffffu)) * ta;
        d1 += bf2f((u16)(w1[c] >> 16)) * tb;
      }
    }
    const float sig = p.rd.scale_table[s_sidx[i]];
    v0 = v0 + sig * d0;
    v1 = v1 + sig * d1;
  }
  *(uint32_t *)(p.y + (size_t)i * p.y_row_stride + o) = pack2(f2bf(v0), f2bf(v1));
}

hipError_t launch_skinny(const SkinnyArgs &a, hipStream_t st) {
  const int grid = (a.n_out + 15) / 16;
  const int nb = (a.n + 15) / 16;
  if (nb <= 1)
    hipLaunchKernelGGL(skinny_bf16_kernel<1>, dim3(grid), dim3(512), 0, st, a);
  else if (nb == 2)
    hipLaunchKernelGGL(skinny_bf16_kernel<2>, dim3(grid), dim3(512), 0, st, a);
  else if (nb <= 4)
    hipLaunchKernelGGL(skinny_bf16_kernel<4>, dim3(grid), dim3(512), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lora
