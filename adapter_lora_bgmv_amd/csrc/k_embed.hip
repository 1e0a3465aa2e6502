// k_embed.hip -- the token-embedding row gather with the routed delta.
//
// y[i, :] = E[t, :] + s * (B[t, :] A), t = token_ids[i]: the delta of one row
// of the adapted matrix (ferrox lora.rs LoraDelta::add_row_to), with the
// embedding pair in the one layout (A [rank][n_embd], B [n_vocab][rank]).
// Memory-bound: a gathered row of E, one row of B per row, and each touched
// slot's A, which every row on that slot shares.  A workgroup takes 16 rows
// and 1024 columns, 4 columns per thread, its rows ordered by pair; the
// rows' B entries go to LDS and each pair's A rows are read once for all
// of its rows.  The rank sum runs k ascending in f32; y is rounded once.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

constexpr int kEmbedRows = 16;
constexpr int kEmbedVec = 4;                  // columns per thread
constexpr int kEmbedCols = 256 * kEmbedVec;   // columns per workgroup

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

// A workgroup takes 16 rows and 1024 columns (4 per thread).  It orders its
// rows by pair in LDS, so that walking them in that order each pair's A rows
// are loaded once (when the pair changes) and shared by all of its rows; the
// accumulators are indexed by that order, which keeps them in registers.
template <typename T>
__global__ __launch_bounds__(256) void embed_rows_kernel(EmbedArgs a) {
  __shared__ float bsh[kEmbedRows][256];  // B[t, 0:R] of the row at each sorted place, f32
  __shared__ int r_tok[kEmbedRows], r_q[kEmbedRows];
  __shared__ float r_sig[kEmbedRows];
  __shared__ int p_row[kEmbedRows], p_q[kEmbedRows];  // by sorted place: row (in the block), pair
  const int tid = threadIdx.x;
  const int i0 = blockIdx.y * kEmbedRows;
  const RouteDev &rd = a.rd;
  if (tid < kEmbedRows) {
    const int i = i0 + tid;
    int tok = -1, q = kSkip;
    float sig = 0.f;
    if (i < a.n) {
      tok = a.token_ids[i];
      if (tok < 0 || tok >= a.n_vocab) {
        tok = -1;  // past the vocabulary: the row is not written
      } else if (a.has_lora) {
        const int s = a.seq_slot[i];
        q = resolve_slot(s, 0, rd.max_loras, 1, rd.a_table, rd.b_table, rd.scale_table);
        if (q >= 0) sig = rd.scale_table[s];
      }
    }
    r_tok[tid] = tok;
    r_q[tid] = q;
    r_sig[tid] = sig;
  }
  __syncthreads();
  if (tid < kEmbedRows) {  // place of this row in (pair, row) order
    const int q = r_q[tid];
    int place = 0;
    for (int r = 0; r < kEmbedRows; ++r) {
      const int qr = r_q[r];
      place += qr < q || (qr == q && r < tid);
    }
    p_row[place] = tid;
    p_q[place] = q;
  }
  __syncthreads();
  for (int e = tid; e < kEmbedRows * rd.R; e += 256) {
    const int p = e / rd.R, k = e % rd.R;
    const int q = p_q[p];
    if (q >= 0) bsh[p][k] = Vec4<T>::one((const T *)rd.b_table[q] + (size_t)r_tok[p_row[p]] * rd.R + k);
  }
  __syncthreads();
  const int c0 = blockIdx.x * kEmbedCols + tid * kEmbedVec;
  if (c0 >= a.n_embd) return;
  const int valid = min(kEmbedVec, a.n_embd - c0);
  // every row's piece of E goes out first and is in flight during the rank
  // sums (the stores to y below could otherwise hold each load back)
  typename Vec4<T>::raw e_raw[kEmbedRows];
#pragma unroll
  for (int p = 0; p < kEmbedRows; ++p) {
    const int tok = r_tok[p_row[p]];
    if (tok >= 0) e_raw[p] = Vec4<T>::load_raw((const T *)a.E + (size_t)tok * a.e_row_stride + c0, valid);
  }
  float acc[kEmbedRows][kEmbedVec];
#pragma unroll
  for (int p = 0; p < kEmbedRows; ++p)
#pragma unroll
    for (int j = 0; j < kEmbedVec; ++j) acc[p][j] = 0.f;
  // k in blocks of 8: at each change of pair along the sorted rows, the
  // block's 8 rows of that pair's A go out together, then every row of the
  // pair takes them
  constexpr int KC = 8;
  for (int kc = 0; kc < rd.R; kc += KC) {
    typename Vec4<T>::raw ar[KC];
    int cur = kSkip;
#pragma unroll
    for (int p = 0; p < kEmbedRows; ++p) {
      const int q = p_q[p];
      if (q < 0) continue;
      if (q != cur) {
        cur = q;
        const T *Aq = (const T *)rd.a_table[q] + (size_t)kc * a.n_embd + c0;
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
          if (kc + kk < rd.R) ar[kk] = Vec4<T>::load_raw(Aq + (size_t)kk * a.n_embd, valid);
      }
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        if (kc + kk >= rd.R) break;
        const float b = bsh[p][kc + kk];
#pragma unroll
        for (int j = 0; j < kEmbedVec; ++j) acc[p][j] += b * Vec4<T>::at(ar[kk], j);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < kEmbedRows; ++p) {
    const int r = p_row[p];
    if (r_tok[r] < 0) continue;
    T *yr = (T *)a.y + (size_t)(i0 + r) * a.y_row_stride + c0;
    if (p_q[p] < 0) {  // base only: the table row, bit for bit
      Vec4<T>::store_raw(yr, e_raw[p], valid);
      continue;
    }
    float ev[kEmbedVec];
#pragma unroll
    for (int j = 0; j < kEmbedVec; ++j) ev[j] = Vec4<T>::at(e_raw[p], j) + r_sig[r] * acc[p][j];
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
