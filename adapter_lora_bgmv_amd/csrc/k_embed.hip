// k_embed.hip -- the token-embedding row gather with the routed delta.
//
// y[i, :] = E[t, :] + s * (B[t, :] A), t = token_ids[i]: the delta of one row
// of the adapted matrix (ferrox lora.rs LoraDelta::add_row_to), with the
// embedding pair in the one layout (A [rank][n_embd], B [n_vocab][rank]).
// Memory-bound: a gathered row of E, one row of B per row, and each touched
// slot's A, which every row on that slot shares.  A workgroup takes 64 rows
// and 256 columns (wave w its rows 16 w .. +15, 4 columns per lane); for
// every 8 ranks the A rows of the workgroup's pairs go to LDS once (bf16:
// by LDS-DMA, every piece of the pass in flight at once) and all four waves
// read them there, so each pair's A is read once per workgroup.
// The rank sum runs k ascending in f32; y is rounded once.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

constexpr int kEmbedRows = 64;               // rows per workgroup, 16 per wave
constexpr int kEmbedVec = 4;                 // columns per lane
constexpr int kEmbedCols = 64 * kEmbedVec;   // columns per workgroup (every wave takes all of them)
constexpr int kEmbedKC = 8;                  // ranks per pass
constexpr int kEmbedLds = 32 * 1024;         // bytes of staged A per pass

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

hipError_t launch_embed_rows(const EmbedArgs &a, int dtype, hipStream_t st) {
  dim3 grid((a.n_embd + kEmbedCols - 1) / kEmbedCols, (a.n + kEmbedRows - 1) / kEmbedRows);
  if (dtype == 0)
    hipLaunchKernelGGL(embed_rows_kernel<float>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(embed_rows_kernel<u16>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lora
