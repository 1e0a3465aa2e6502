// k_embed.hip -- the token-embedding row gather with the routed delta.
//
// y[i, :] = E[t, :] + s * (B[t, :] A), t = token_ids[i]: the delta of one row
// of the adapted matrix (ferrox lora.rs LoraDelta::add_row_to), with the
// embedding pair in the one layout (A [rank][n_embd], B [n_vocab][rank]).
// Memory-bound: a gathered row of E, one row of B per row, and each touched
// slot's A, which every row on that slot shares.  A workgroup takes 64 rows
// and 256 columns (wave w 16 of the rows, 4 columns per lane).  bf16 tables
// of rank 16 take embed_rows_bf16_kernel (rows sorted by pair, A in
// registers per run, two ranks per v_dot2); every other call the general
// kernel: for every 8 ranks the A rows of the workgroup's pairs go to LDS
// once (bf16: by LDS-DMA, every piece of the pass in flight at once) and all
// four waves read them there, the rank sum k ascending in f32.  y is rounded
// once.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

constexpr int kEmbedRows = 64;               // rows per workgroup, 16 per wave
constexpr int kEmbedVec = 4;                 // columns per lane
constexpr int kEmbedCols = 64 * kEmbedVec;   // columns per workgroup (every wave takes all of them)
constexpr int kEmbedKC = 8;                  // ranks per pass
constexpr int kEmbedLds = 32 * 1024;         // bytes of staged A per pass

typedef __bf16 bf16x2e __attribute__((ext_vector_type(2)));
typedef float f32x2e __attribute__((ext_vector_type(2)));

template <typename T> struct Vec4;
// bf16 rows are multiples of 8 long, 16-byte aligned: whole 8-byte pieces
template <> struct Vec4<u16> {
  static __device__ __forceinline__ void load(const u16 *p, float *v, int) {
    const uint2 w = *(const uint2 *)p;
    v[0] = bf2f((u16)(w.x & 0xffffu));
    v[1] = bf2f((u16)(w.x >> 16));
    v[2] = bf2f((u16)(w.y & 0xffffu));
    v[3] = bf2f((u16)(w.y >> 16));
  }
  static __device__ __forceinline__ void copy(const u16 *src, u16 *dst, int) { *(uint2 *)dst = *(const uint2 *)src; }
  static __device__ __forceinline__ void store(u16 *p, const float *v, int) {
    uint2 w;
    w.x = pack2(f2bf(v[0]), f2bf(v[1]));
    w.y = pack2(f2bf(v[2]), f2bf(v[3]));
    *(uint2 *)p = w;
  }
  static __device__ __forceinline__ float one(const u16 *p) { return bf2f(*p); }
  // the same 4 columns held packed (so that many k rows stay in flight)
  typedef uint2 raw;
  static __device__ __forceinline__ raw load_raw(const u16 *p, int) { return *(const uint2 *)p; }
  static __device__ __forceinline__ void store_raw(u16 *p, raw w, int) { *(uint2 *)p = w; }
  static __device__ __forceinline__ float at(raw w, int j) {
    const uint32_t u = j < 2 ? w.x : w.y;
    return bf2f((u16)((j & 1) ? (u >> 16) : (u & 0xffffu)));
  }
};
// f32 rows take any length and stride: element by element, up to `valid`
template <> struct Vec4<float> {
  static __device__ __forceinline__ void load(const float *p, float *v, int valid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = j < valid ? p[j] : 0.f;
  }
  static __device__ __forceinline__ void copy(const float *src, float *dst, int valid) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < valid) dst[j] = src[j];
  }
  static __device__ __forceinline__ void store(float *p, const float *v, int valid) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < valid) p[j] = v[j];
  }
  static __device__ __forceinline__ float one(const float *p) { return *p; }
  typedef float4 raw;
  static __device__ __forceinline__ raw load_raw(const float *p, int valid) {
    float v[4];
    load(p, v, valid);
    return make_float4(v[0], v[1], v[2], v[3]);
  }
  static __device__ __forceinline__ float at(raw w, int j) { return j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w; }
  static __device__ __forceinline__ void store_raw(float *p, raw w, int valid) {
    const float v[4] = {w.x, w.y, w.z, w.w};
    store(p, v, valid);
  }
};

template <typename T>
__global__ __launch_bounds__(256) void embed_rows_kernel(EmbedArgs a) {
  constexpr int PG = kEmbedLds / (kEmbedKC * kEmbedCols * (int)sizeof(T));  // pairs staged per pass
  __shared__ __attribute__((aligned(16))) T ash[PG][kEmbedKC][kEmbedCols];   // A rows of PG pairs
  __shared__ float bsh[kEmbedRows][kEmbedKC];  // B[t, kc .. kc + KC) of each row, f32
  __shared__ int r_tok[kEmbedRows], r_q[kEmbedRows], r_d[kEmbedRows];  // token, pair, place in d_pair
  __shared__ float r_sig[kEmbedRows];
  __shared__ const T *r_b[kEmbedRows];  // the row's B row
  __shared__ int d_pair[kEmbedRows];    // the workgroup's pairs, in order of first appearance
  __shared__ const T *d_a[kEmbedRows];  // their A
  __shared__ int n_d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = blockIdx.y * kEmbedRows;
  const RouteDev &rd = a.rd;
  const int R = rd.R;
  if (tid < kEmbedRows) {  // one row per lane of wave 0
    const int i = i0 + tid;
    int tok = -1, q = kSkip;
    float sig = 0.f;
    const T *brow = nullptr;
    if (i < a.n) {
      tok = a.token_ids[i];
      if (tok < 0 || tok >= a.n_vocab) {
        tok = -1;  // past the vocabulary: the row is not written
      } else if (a.has_lora) {
        const int s = a.seq_slot[i];
        q = resolve_slot(s, 0, rd.max_loras, 1, rd.a_table, rd.b_table, rd.scale_table);
        if (q >= 0) {
          sig = rd.scale_table[s];
          brow = (const T *)rd.b_table[q] + (size_t)tok * R;
        }
      }
    }
    r_tok[tid] = tok;
    r_q[tid] = q;
    r_sig[tid] = sig;
    r_b[tid] = brow;
    // the distinct pairs, in order of first appearance: one round of
    // ballots per pair, then their A entries in one round trip
    uint64_t todo = __ballot(q >= 0);
    int nd = 0, mine = -1;
    while (todo) {  // uniform
      const int l0 = __ffsll((unsigned long long)todo) - 1;
      const int v = __builtin_amdgcn_readlane(q, l0);
      const uint64_t m = __ballot(q == v);
      if (q == v) mine = nd;
      if (lane == l0) d_pair[nd] = v;
      ++nd;
      todo &= ~m;
    }
    r_d[tid] = mine;
    if (lane < nd) d_a[lane] = (const T *)rd.a_table[d_pair[lane]];
    if (lane == 0) n_d = nd;
  }
  __syncthreads();
  const int nd = n_d;
  const int c0 = blockIdx.x * kEmbedCols + lane * kEmbedVec;
  const int valid = c0 < a.n_embd ? min(kEmbedVec, a.n_embd - c0) : 0;
  // every row's piece of E goes out first and is in flight during the rank
  // sums (the stores to y below could otherwise hold each load back)
  typename Vec4<T>::raw e_raw[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int tok = r_tok[wave * 16 + j];
    if (tok >= 0 && valid > 0) e_raw[j] = Vec4<T>::load_raw((const T *)a.E + (size_t)tok * a.e_row_stride + c0, valid);
  }
  float acc[16][kEmbedVec];
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int v = 0; v < kEmbedVec; ++v) acc[j][v] = 0.f;
  for (int kc = 0; kc < R && nd > 0; kc += kEmbedKC) {
    __syncthreads();  // every wave is done with the last pass's B
    for (int e = tid; e < kEmbedRows * kEmbedKC; e += 256) {
      const int r = e / kEmbedKC, kk = e % kEmbedKC;
      const T *brow = r_b[r];
      bsh[r][kk] = brow != nullptr && kc + kk < R ? Vec4<T>::one(brow + kc + kk) : 0.f;
    }
    for (int g0 = 0; g0 < nd; g0 += PG) {
      __syncthreads();  // every wave is done with the last pass's A (and this pass's B has landed)
      const int np = min(PG, nd - g0);
      if constexpr (sizeof(T) == 2) {
        // LDS-DMA: instruction m carries the 512-byte rows 2 m and 2 m + 1
        // (row = (pair ps, rank kk); lane l: row 2 m + l / 32, 8 columns from
        // (l % 32) 8); a piece outside the pass reads the first pair's row 0
        const int nrow = np * kEmbedKC;
        for (int m = wave; 2 * m < nrow; m += 4) {
          const int row = 2 * m + (lane >> 5), ps = row / kEmbedKC, kk = row % kEmbedKC;
          const int cc = blockIdx.x * kEmbedCols + (lane & 31) * 8;
          const bool in = kc + kk < R && cc < a.n_embd;
          dma16(in ? d_a[g0 + ps] + (size_t)(kc + kk) * a.n_embd + cc : d_a[g0],
                lds_addr(&ash[0][0][0] + (size_t)m * 512));
        }
        wait_vmcnt<0>();
      } else {
        for (int e = tid; e < np * kEmbedKC * 64; e += 256) {
          const int ps = e / (kEmbedKC * 64), kk = (e / 64) % kEmbedKC, cl = e % 64;
          const int cc = blockIdx.x * kEmbedCols + cl * kEmbedVec;
          const int vv = cc < a.n_embd ? min(kEmbedVec, a.n_embd - cc) : 0;
          T *dst = &ash[ps][kk][cl * kEmbedVec];
          if (kc + kk < R && vv > 0)
            Vec4<T>::store_raw(dst, Vec4<T>::load_raw(d_a[g0 + ps] + (size_t)(kc + kk) * a.n_embd + cc, vv), kEmbedVec);
        }
      }
      __syncthreads();
      if (valid > 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = wave * 16 + j;
          const int d = r_d[r] - g0;  // uniform over the wave
          if (d < 0 || d >= np) continue;
#pragma unroll
          for (int kk = 0; kk < kEmbedKC; ++kk) {
            if (kc + kk >= R) break;
            const float b = bsh[r][kk];
            const typename Vec4<T>::raw av = *(const typename Vec4<T>::raw *)&ash[d][kk][lane * kEmbedVec];
#pragma unroll
            for (int v = 0; v < kEmbedVec; ++v) acc[j][v] += b * Vec4<T>::at(av, v);
          }
        }
      }
    }
  }
  if (valid == 0) return;
  // every load has landed: the stores below then need no waits of their
  // own (a wait for a load would also wait for every store before it)
  wait_vmcnt<0>();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = wave * 16 + j;
    if (r_tok[r] < 0) continue;
    T *yr = (T *)a.y + (size_t)(i0 + r) * a.y_row_stride + c0;
    if (r_q[r] < 0) {  // base only: the table row, bit for bit
      Vec4<T>::store_raw(yr, e_raw[j], valid);
      continue;
    }
    float ev[kEmbedVec];
#pragma unroll
    for (int v = 0; v < kEmbedVec; ++v) ev[v] = Vec4<T>::at(e_raw[j], v) + r_sig[r] * acc[j][v];
    Vec4<T>::store(yr, ev, valid);
  }
}

// bf16 tables of rank 16 (and calls without a route): the workgroup's
// 64 rows are sorted by pair before any work, so a wave meets its 16 rows'
// pairs in runs.  A lane holds the current run's A for its 4 columns in
// registers, two ranks packed per register, and takes a row's rank sum two
// ranks per v_dot2 (both bf16 products exact in f32), rank pairs ascending;
// the next run's A is in flight while the current one is used.  The packing
// is done once per run, not once per row.  Each row's E piece stays in
// LDS (by LDS-DMA), is overwritten there by the row's result, and every row
// is stored after the last load has landed; a row whose slot skips keeps the
// table row bit for bit.
constexpr int kEmbedSortRows = 64;  // rows per workgroup, 16 per wave

template <int RK>
__global__ __launch_bounds__(256) void embed_rows_bf16_kernel(EmbedArgs a) {
  constexpr int kBase = kEmbedSortRows;  // s_d of a row written with its table row alone
  constexpr int kNone = -2;              // s_d of a row that is not written
  __shared__ int s_row[kEmbedSortRows], s_tok[kEmbedSortRows], s_d[kEmbedSortRows];
  __shared__ float s_sig[kEmbedSortRows];
  __shared__ const u16 *s_bp[kEmbedSortRows];  // the row's B row
  __shared__ const u16 *s_a[kEmbedSortRows];   // A of the workgroup's pairs, in order of first appearance
  __shared__ __attribute__((aligned(16))) u16 s_b[kEmbedSortRows][RK];
  __shared__ __attribute__((aligned(16))) u16 s_e[4][16][kEmbedCols];  // each wave's rows' E pieces
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  if (wave == 0) {  // one row per lane: resolve, then sort by pair
    const RouteDev &rd = a.rd;
    const int i = blockIdx.y * kEmbedSortRows + lane;
    int tok = -1, q = kSkip;
    float sig = 0.f;
    const u16 *brow = nullptr, *arow = nullptr;
    if (i < a.n) {  // the token and the slot are read together
      tok = a.token_ids[i];
      const int s = a.has_lora ? a.seq_slot[i] : -1;
      if (tok < 0 || tok >= a.n_vocab) {
        tok = -1;
      } else if (a.has_lora) {
        const void *ae, *be;
        float sc;
        q = resolve_slot_entries(s, rd, ae, be, sc);
        if (q >= 0) {
          sig = sc;
          arow = (const u16 *)ae;
          brow = (const u16 *)be + (size_t)tok * RK;
        }
      }
    }
    uint64_t todo = __ballot(q >= 0);
    int nd = 0, mine = -1;
    const uint64_t a64 = (uint64_t)(uintptr_t)arow;
    uint32_t alo = 0, ahi = 0;  // lane d: A of the d-th pair
    while (todo) {  // uniform: one round of ballots per distinct pair
      const int l0 = __ffsll((unsigned long long)todo) - 1;
      const int v = __builtin_amdgcn_readlane(q, l0);
      const uint32_t vlo = __builtin_amdgcn_readlane((uint32_t)a64, l0), vhi = __builtin_amdgcn_readlane((uint32_t)(a64 >> 32), l0);
      const uint64_t m = __ballot(q == v);
      if (q == v) mine = nd;
      if (lane == nd) {
        alo = vlo;
        ahi = vhi;
      }
      ++nd;
      todo &= ~m;
    }
    if (lane < nd) s_a[lane] = (const u16 *)(uintptr_t)(((uint64_t)ahi << 32) | alo);
    // place in the sorted order: pairs first (by first appearance), then the
    // rows written with the table row alone, then the rows not written
    const int cls = tok < 0 ? nd + 1 : (q < 0 ? nd : mine);
    int pos = 0, start = 0;
    for (int c = 0; c <= nd + 1; ++c) {  // uniform
      const uint64_t m = __ballot(cls == c);
      if (cls == c) pos = start + (int)__popcll(m & below);
      start += (int)__popcll(m);
    }
    s_row[pos] = i;
    s_tok[pos] = tok;
    s_sig[pos] = sig;
    s_bp[pos] = brow;
    s_d[pos] = tok < 0 ? kNone : (q < 0 ? kBase : mine);
  }
  __syncthreads();
  const int c0 = blockIdx.x * kEmbedCols + lane * kEmbedVec;
  const bool colv = c0 < a.n_embd;  // n_embd is a multiple of 8: a piece is whole or absent
  const int wb = wave * 16;
  // the runs of equal pairs among the wave's rows: lane j < 16 looks at row wb + j
  const int dj = lane < 16 ? s_d[wb + lane] : kNone;
  const int dp = lane > 0 && lane < 16 ? s_d[wb + lane - 1] : kNone;
  const bool mine_ad = dj >= 0 && dj < kBase;
  // the wave's rows, sorted: [0, n_ad) adapted, in runs of equal pairs that
  // begin at the bits of `starts`, then [n_ad, n_wr) base only
  const uint64_t starts = __ballot(mine_ad && dj != dp);
  const int n_ad = (int)__popcll(__ballot(mine_ad));
  const int n_wr = (int)__popcll(__ballot(lane < 16 && dj != kNone));
  // loads, oldest first: the rows' B, the first run's A, E
  uint4 bl[RK / 8];
  if (mine_ad) {
    const uint4 *bp = (const uint4 *)s_bp[wb + lane];
#pragma unroll
    for (int e = 0; e < RK / 8; ++e) bl[e] = bp[e];
  }
  // A by buffer loads: one offset register for every rank (a lane past the
  // columns reads column 0 and drops it)
  uint2 an[RK];
  const uint32_t a_off = colv ? 2u * (uint32_t)c0 : 0u, a_pitch = 2u * (uint32_t)a.n_embd;
  auto load_run = [&](int d) {
    const uint64_t ab = (uint64_t)(uintptr_t)s_a[d];
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)ab), hi = __builtin_amdgcn_readfirstlane((uint32_t)(ab >> 32));
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)(((uint64_t)hi << 32) | lo), 0, 0x7ffffff0, 0x00020000);
#pragma unroll
    for (int r = 0; r < RK; ++r)
      an[r] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)a_off, (int)(r * a_pitch), 0));
  };
  if (n_ad > 0) load_run(__builtin_amdgcn_readfirstlane(s_d[wb]));
  {  // the rows' E pieces by LDS-DMA: instruction m carries the wave's rows 2 m
     // and 2 m + 1, lane l row 2 m + l / 32 and 8 columns from (l % 32) 8; a
     // piece that is not needed reads the table's first element instead
    const int cc = blockIdx.x * kEmbedCols + (lane & 31) * 8;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int tok = s_tok[wb + 2 * m + (lane >> 5)];
      const bool in = tok >= 0 && cc < a.n_embd;
      dma16(in ? (const u16 *)a.E + (size_t)tok * a.e_row_stride + cc : (const u16 *)a.E,
            lds_addr(&s_e[wave][2 * m][0]));
    }
  }
  wait_vmcnt<0>();  // B, the first run's A and E have landed
  if (mine_ad) {
#pragma unroll
    for (int e = 0; e < RK / 8; ++e) *(uint4 *)&s_b[wb + lane][8 * e] = bl[e];
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own B rows, read back below
  u16 *const yb = (u16 *)a.y + c0;
  for (int j = 0; j < n_ad;) {  // one run per pass
    uint32_t pk[RK / 2][4];     // (rank 2 p, rank 2 p + 1) of column c0 + c
#pragma unroll
    for (int p = 0; p < RK / 2; ++p) {
      const uint2 lo = an[2 * p], hi = an[2 * p + 1];
      pk[p][0] = (lo.x & 0xffffu) | (hi.x << 16);
      pk[p][1] = (lo.x >> 16) | (hi.x & 0xffff0000u);
      pk[p][2] = (lo.y & 0xffffu) | (hi.y << 16);
      pk[p][3] = (lo.y >> 16) | (hi.y & 0xffff0000u);
    }
    const uint64_t later = starts & ~((2ull << j) - 1ull);
    const int jend = later ? __ffsll((unsigned long long)later) - 1 : n_ad;
    if (jend < n_ad) load_run(__builtin_amdgcn_readfirstlane(s_d[wb + jend]));  // in flight during this run
    for (; j < jend; ++j) {
      const uint4 *brow = (const uint4 *)&s_b[wb + j][0];
      uint32_t bw[RK / 2];
#pragma unroll
      for (int e = 0; e < RK / 8; ++e) {
        const uint4 t = brow[e];
        bw[4 * e] = t.x;
        bw[4 * e + 1] = t.y;
        bw[4 * e + 2] = t.z;
        bw[4 * e + 3] = t.w;
      }
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < RK / 2; ++p)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2e, pk[p][c]),
                                                   __builtin_bit_cast(bf16x2e, bw[p]), acc[c], false);
      const float sig = s_sig[wb + j];
      const uint2 ev = *(const uint2 *)&s_e[wave][j][lane * kEmbedVec];
      f32x2e y01, y23;
      y01.x = Vec4<u16>::at(ev, 0) + sig * acc[0];
      y01.y = Vec4<u16>::at(ev, 1) + sig * acc[1];
      y23.x = Vec4<u16>::at(ev, 2) + sig * acc[2];
      y23.y = Vec4<u16>::at(ev, 3) + sig * acc[3];
      // round to nearest even (v_cvt_pk_bf16_f32)
      const uint2 out = make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(y01, bf16x2e)),
                                   __builtin_bit_cast(uint32_t, __builtin_convertvector(y23, bf16x2e)));
      *(uint2 *)&s_e[wave][j][lane * kEmbedVec] = out;  // in place of the row's E
    }
  }
  // the stores go out once no load is left to wait for (a wait for a load
  // also waits for every store issued before it); base-only rows store the
  // table row, bit for bit
  if (!colv) return;
  for (int j = 0; j < n_wr; ++j)
    *(uint2 *)(yb + (size_t)s_row[wb + j] * a.y_row_stride) = *(const uint2 *)&s_e[wave][j][lane * kEmbedVec];
}

hipError_t launch_embed_rows(const EmbedArgs &a, int dtype, hipStream_t st) {
  dim3 grid((a.n_embd + kEmbedCols - 1) / kEmbedCols, (a.n + kEmbedRows - 1) / kEmbedRows);
  static_assert(kEmbedSortRows == kEmbedRows, "the two kernels share the grid");
  // the sorted kernel's buffer loads address A by 32-bit offsets
  const bool sorted = dtype != 0 && (size_t)32 * a.n_embd < 0x7ffffff0u;
  if (sorted && (!a.has_lora || a.rd.R == 16))  // bf16 pools pad max_rank to a multiple of 16
    hipLaunchKernelGGL(embed_rows_bf16_kernel<16>, grid, dim3(256), 0, st, a);
  else if (dtype == 0)
    hipLaunchKernelGGL(embed_rows_kernel<float>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(embed_rows_kernel<u16>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lora
