// k_decode.hip -- the decode-shaped apply (n <= 64 rows): a main launch and an
// epilogue launch.
//
//     y_i = W x_i + s_q B_q (A_q x_i),   q = the slot row i resolves to
//
// (ferrox lora.rs module doc; atlas lora_delta.rs apply_lora_bgmv: shrink,
// then expand-and-fold).  At decode sizes the cost is streaming W once, and
// what limits that on this chip is how many bytes each CU must take in: its
// share of W plus the x columns its k range needs.  So:
//
//  * decode_main_kernel: a workgroup owns a tile of 64 output features x all
//    rows x one k range (k is split S ways; S depends on k_in only).  Each CU
//    then takes in 128 KB of W and only 1/S of x.  The 8 waves take
//    interleaved 32-wide k steps (W rows as the MFMA A operand, x rows as B,
//    fragments loaded straight into registers, all of a wave's loads in
//    flight together) and meet in LDS in a fixed order; the f32 partial tile
//    goes to the workspace.  The shrink t = A_q x rides along: once its tile
//    is stored, a workgroup runs one shrink unit (touched slot, 16-rank
//    block, k chunk), which gathers the rows of its slot into MFMA columns,
//    so each A_q is read once per call.  Nothing in this launch waits for
//    another workgroup;
//  * decode_epilogue_kernel: y = bf16(sum_z partial_z + s_q sum_r B_q[o, r]
//    t_i[r]), the S partials in split order, t summed over its k chunks in
//    chunk order, the rank sum in f32 in rank order, one rounding.
// The shrink's k chunks are the base contraction's S k ranges.
// With no adapters and no k split the main launch stores y itself.
// Skipped rows (slot < 0 or past the pool, NULL table entry, zero scale) get
// no delta arithmetic, so they equal the base-only launch bit for bit.
// Every output element is reduced in an order that does not depend on the
// batch's other rows or on n_out.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

namespace {

constexpr int kNW = 8;                    // waves per workgroup
constexpr int kMB = kDecodeTileOut / 16;  // W row blocks per tile

struct Rows {  // the batch's routes, resolved once per workgroup
  int q[64];          // slot or kSkip
  const u16 *bq[64];  // the row's B (rows that resolve)
  float sig[64];      // the row's scale
  int list[64];       // rows grouped by slot (row order within one)
  int start[65];      // list offsets per touched slot
  int slot[64];       // touched slots in order of first appearance
  int T;              // touched slots
};

// Resolves every row (wave 0; n <= 64, one row per lane) and groups the rows
// by slot, slots numbered in order of first appearance: one round of
// ballots per touched slot, no LDS round trips.
__device__ void resolve_rows(const DecodeArgs &p, Rows &s) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x >= 64) return;
  int q = kSkip;
  if (p.has_lora && lane < p.n)
    q = resolve_slot(p.seq_slot[lane], 0, p.rd.max_loras, 1, p.rd.a_table, p.rd.b_table, p.rd.scale_table);
  s.q[lane] = q;
  s.bq[lane] = q >= 0 ? (const u16 *)p.rd.b_table[q] : nullptr;
  s.sig[lane] = q >= 0 ? p.rd.scale_table[q] : 0.f;
  const uint64_t below = (1ull << lane) - 1ull;
  uint64_t todo = __ballot(q >= 0);
  int T = 0, pos = 0;
  while (todo) {  // uniform: the lowest row not yet grouped names the next slot
    const int v = __builtin_amdgcn_readlane(q, __ffsll((unsigned long long)todo) - 1);
    const uint64_t m = __ballot(q == v);
    if (q == v) s.list[pos + __popcll(m & below)] = lane;
    if (lane == 0) {
      s.slot[T] = v;
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

// One shrink unit (touched slot u, rank block rb, k chunk c): the chunk's
// partial of t for the rows of slot u, ranks 16 rb .. 16 rb + 15.  The 8 waves
// take the chunk's 32-wide steps in turn, four at a time with every load out
// before their MFMAs, and meet in LDS (`red`, 32 KB) in a fixed order.
__device__ void shrink_unit(const DecodeArgs &p, const Rows &s, int uidx, f32x4 (*red)[64]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.k_in, R = p.R, RB = R / 16, nchunks = p.n_chunks;
  const int c = uidx % nchunks, rb = (uidx / nchunks) % RB, u = uidx / (nchunks * RB);
  const u16 *A = (const u16 *)p.rd.a_table[s.slot[u]];
  const int m = s.start[u + 1] - s.start[u];
  const int G = (m + 15) / 16;  // groups of 16 gathered rows (<= 4)
  const int kb = c * p.chunk, ke = min(kb + p.chunk, K);
  const int nsteps = (ke - kb + 31) / 32;
  const int koff = (lane >> 4) * 8;
  const u16 *ap = A + (size_t)(rb * 16 + (lane & 15)) * K + kb + koff;
  const u16 *xp[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int j = g * 16 + (lane & 15);
    xp[g] = g < G && j < m ? p.x + (size_t)s.list[s.start[u] + j] * p.x_row_stride + kb + koff : nullptr;
  }
  f32x4 acc[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; wave + kNW * i0 < nsteps; i0 += 4) {
    uint4 av[4], xv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int st = wave + kNW * (i0 + i);
      const bool in = st < nsteps && kb + st * 32 + koff < ke;
      av[i] = in ? ldg16(ap + st * 32) : z4();
#pragma unroll
      for (int g = 0; g < 4; ++g) xv[i][g] = in && xp[g] ? ldg16(xp[g] + st * 32) : z4();
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[g] = mfma16(av[i], xv[i][g], acc[g]);
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) red[wave * 4 + g][lane] = acc[g];
  __syncthreads();
  // D holds ranks 4*(l/16)..+3 of gathered column l%16
  for (int e = tid; e < G * 64; e += kNW * 64) {
    const int g = e >> 6, l = e & 63, j = g * 16 + (l & 15);
    if (j >= m) continue;
    f32x4 v = red[g][l];
#pragma unroll
    for (int w = 1; w < kNW; ++w) v += red[w * 4 + g][l];
    const int row = s.list[s.start[u] + j];
    *(f32x4 *)(p.t_part + ((size_t)c * p.n + row) * R + rb * 16 + (l >> 4) * 4) = v;
  }
  __syncthreads();  // red is reused by the next unit
}

}  // namespace

template <int NB>  // 16-row column blocks of the batch: n <= 16 * NB
__global__ __launch_bounds__(kNW * 64, 2) void decode_main_kernel(DecodeArgs p) {
  constexpr int NF = kMB * NB;  // accumulator fragments per wave
  static_assert(kNW * kMB * 4 * 1024 <= kDecodeLds, "LDS scratch holds the reduction");
  __shared__ __attribute__((aligned(16))) f32x4 red[kDecodeLds / 1024][64];
  __shared__ Rows s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.k_in;
  const int tl = blockIdx.x / p.S, z = blockIdx.x % p.S;
  const int o0 = tl * kDecodeTileOut;
  const int kb = min(z * p.k_per_split, K), ke = min(kb + p.k_per_split, K);
  const int nsteps = (ke - kb + 31) / 32;
  const int nj = (nsteps - wave + kNW - 1) / kNW;  // this wave's steps: wave, wave + 8, ...
  const int koff = (lane >> 4) * 8;
  // rows past n_out read the last row instead; their outputs are never stored
  const u16 *wr = p.W + kb + koff;
  int wrow[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) wrow[mb] = min(o0 + mb * 16 + (lane & 15), p.n_out - 1);
  const u16 *xr = p.x + (size_t)(lane & 15) * p.x_row_stride + kb + koff;
  const size_t xstep = (size_t)16 * p.x_row_stride;
  f32x4 acc[kMB][NB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[mb][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A wave's steps go out in batches of kDecodeBatch (all of them when k_in
  // <= 1024 * S): every load of the batch is in flight before the first
  // MFMA waits, so the loop costs one memory latency per batch.
  uint4 wv[kDecodeBatch][kMB], xv[kDecodeBatch][NB];
  auto load = [&](int d, int j) {
    const int s0 = (wave + kNW * j) * 32;
    const bool in = j < nj && kb + s0 + koff < ke;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) wv[d][mb] = in ? ldg16(wr + (size_t)wrow[mb] * p.w_row_stride + s0) : z4();
#pragma unroll
    for (int b = 0; b < NB; ++b)
      xv[d][b] = (in && b * 16 + (lane & 15) < p.n) ? ldg16(xr + b * xstep + s0) : z4();
  };
  for (int j0 = 0; j0 < nj; j0 += kDecodeBatch) {
#pragma unroll
    for (int d = 0; d < kDecodeBatch; ++d) load(d, j0 + d);
    if (j0 == 0) resolve_rows(p, s);  // wave 0, while its first loads are in flight
#pragma unroll
    for (int d = 0; d < kDecodeBatch; ++d)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[mb][b] = mfma16(wv[d][mb], xv[d][b], acc[mb][b]);
  }
  if (nj <= 0) resolve_rows(p, s);

  // fixed-order reduction of the 8 waves through LDS
#pragma unroll
  for (int f = 0; f < NF; ++f) red[wave * NF + f][lane] = acc[f / NB][f % NB];
  __syncthreads();
  const bool direct = p.S == 1 && !p.has_lora;  // nothing left for an epilogue: store y now
  float *part = p.partials + ((size_t)tl * p.S + z) * (64 * kDecodeTileOut);
  for (int e = tid; e < NF * 64; e += kNW * 64) {
    const int f = e >> 6, l = e & 63;
    f32x4 v = red[f][l];
#pragma unroll
    for (int w = 1; w < kNW; ++w) v += red[w * NF + f][l];
    // D layout: column (row) l%16 of block b, outputs 4*(l/16)..+3 of block mb
    const int mb = f / NB, b = f % NB;
    const int i = b * 16 + (l & 15), oo = mb * 16 + (l >> 4) * 4;
    if (direct) {
      if (i < p.n && o0 + oo < p.n_out)
        *(uint2 *)(p.y + (size_t)i * p.y_row_stride + o0 + oo) =
            make_uint2(pack2(f2bf(v[0]), f2bf(v[1])), pack2(f2bf(v[2]), f2bf(v[3])));
    } else {
      *(f32x4 *)(part + i * kDecodeTileOut + oo) = v;
    }
  }
  if (!p.has_lora) return;
  __syncthreads();  // the routes are resolved and red is free
  if (blockIdx.x == 0 && tid < 64) {  // the epilogue's per-row routes
    p.row_q[tid] = s.q[tid];
    p.row_sig[tid] = s.sig[tid];
    p.row_b[tid] = s.bq[tid];
  }
  const int units = s.T * (p.R / 16) * p.n_chunks;
  for (int uidx = blockIdx.x; uidx < units; uidx += gridDim.x) shrink_unit(p, s, uidx, red);
}

// y for 16 output features x all rows per workgroup, one thread per (row,
// four features).  Every load that does not depend on another goes out
// first: the row's route, the S partials, t's chunk partials.
__global__ __launch_bounds__(256) void decode_epilogue_kernel(DecodeArgs p) {
  __shared__ __attribute__((aligned(16))) float st[64 * 256];  // t rows, n x R
  const int tid = threadIdx.x;
  const int R = p.R;
  const int tl = blockIdx.x / 4;
  const int i = tid >> 2, oo = (blockIdx.x % 4) * 16 + (tid & 3) * 4, o = tl * kDecodeTileOut + oo;
  const bool live = i < p.n && o < p.n_out;
  const bool lora = p.has_lora;
  const int q = live && lora ? p.row_q[i] : kSkip;
  f32x4 a[kDecodeMaxSplit];
  const float *pp = p.partials + (size_t)tl * p.S * (64 * kDecodeTileOut) + i * kDecodeTileOut + oo;
#pragma unroll
  for (int z = 0; z < kDecodeMaxSplit; ++z)
    a[z] = live && z < p.S ? *(const f32x4 *)(pp + (size_t)z * (64 * kDecodeTileOut)) : f32x4{0.f, 0.f, 0.f, 0.f};
  if (lora)  // stage t in LDS: the chunk partials summed in chunk order
    for (int e = tid * 4; e < p.n * R; e += 256 * 4) {
      f32x4 v[kDecodeMaxChunks];
#pragma unroll
      for (int c = 0; c < kDecodeMaxChunks; ++c)
        v[c] = c < p.n_chunks ? *(const f32x4 *)(p.t_part + (size_t)c * p.n * R + e) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 1; c < kDecodeMaxChunks; ++c)
        if (c < p.n_chunks) v[0] += v[c];
      *(f32x4 *)(st + e) = v[0];
    }
  const u16 *Bq = q >= 0 ? p.row_b[i] + (size_t)o * R : nullptr;
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
    const float *ti = st + i * R;
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
    const float sig = p.row_sig[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = v[j] + sig * d[j];
  }
  *(uint2 *)(p.y + (size_t)i * p.y_row_stride + o) =
      make_uint2(pack2(f2bf(v[0]), f2bf(v[1])), pack2(f2bf(v[2]), f2bf(v[3])));
}

hipError_t launch_decode_main(const DecodeArgs &a, hipStream_t st) {
  const int grid = a.n_tiles * a.S;
  if (grid == 0) return hipSuccess;
  const int nb = (a.n + 15) / 16;
  if (nb <= 1)
    hipLaunchKernelGGL(decode_main_kernel<1>, dim3(grid), dim3(kNW * 64), 0, st, a);
  else if (nb == 2)
    hipLaunchKernelGGL(decode_main_kernel<2>, dim3(grid), dim3(kNW * 64), 0, st, a);
  else if (nb <= 4)
    hipLaunchKernelGGL(decode_main_kernel<4>, dim3(grid), dim3(kNW * 64), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_epilogue(const DecodeArgs &a, hipStream_t st) {
  if (a.S == 1 && !a.has_lora) return hipSuccess;  // the main launch stored y
  hipLaunchKernelGGL(decode_epilogue_kernel, dim3(a.n_tiles * 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lora
