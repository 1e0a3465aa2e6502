// k_embed.hip -- the token-embedding row gather with the routed delta.
//
// y[i, :] = E[t, :] + s * (B[t, :] A), t = token_ids[i]: the delta of one row
// of the adapted matrix (ferrox lora.rs LoraDelta::add_row_to), with the
// embedding pair in the one layout (A [rank][n_embd], B [n_vocab][rank]).
// Memory-bound: a gathered row of E, one row of B per row, and each touched
// slot's A, which every row on that slot shares.  A workgroup takes 8 rows
// and 2048 columns, 8 columns per thread; the rows' B entries go to LDS and
// each distinct slot among the 8 rows reads its A rows once for all of its
// rows.  The rank sum runs k ascending in f32; y is rounded once.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

constexpr int kEmbedRows = 8;
constexpr int kEmbedCols = 256 * 8;

template <typename T> struct Vec8;
template <> struct Vec8<u16> {
  static __device__ __forceinline__ void load(const u16 *p, int valid, float *v) {
    if (valid >= 8) {
      const uint4 w = *(const uint4 *)p;
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf2f((u16)(u[j] & 0xffffu));
        v[2 * j + 1] = bf2f((u16)(u[j] >> 16));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = j < valid ? bf2f(p[j]) : 0.f;
    }
  }
  static __device__ __forceinline__ void copy(const u16 *src, u16 *dst, int valid) {
    if (valid >= 8) {
      *(uint4 *)dst = *(const uint4 *)src;
    } else {
      for (int j = 0; j < valid; ++j) dst[j] = src[j];
    }
  }
  static __device__ __forceinline__ void store(u16 *p, int valid, const float *v) {
    if (valid >= 8) {
      uint4 w;
      w.x = pack2(f2bf(v[0]), f2bf(v[1]));
      w.y = pack2(f2bf(v[2]), f2bf(v[3]));
      w.z = pack2(f2bf(v[4]), f2bf(v[5]));
      w.w = pack2(f2bf(v[6]), f2bf(v[7]));
      *(uint4 *)p = w;
    } else {
      for (int j = 0; j < valid; ++j) p[j] = f2bf(v[j]);
    }
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float *p, int valid, float *v) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = j < valid ? p[j] : 0.f;
  }
  static __device__ __forceinline__ void copy(const float *src, float *dst, int valid) {
    for (int j = 0; j < valid && j < 8; ++j) dst[j] = src[j];
  }
  static __device__ __forceinline__ void store(float *p, int valid, const float *v) {
    for (int j = 0; j < valid && j < 8; ++j) p[j] = v[j];
  }
};

template <typename T>
__global__ __launch_bounds__(256) void embed_rows_kernel(EmbedArgs a) {
  __shared__ float bsh[kEmbedRows][256];  // B[t, 0:R] of each row, f32
  __shared__ int s_tok[kEmbedRows], s_q[kEmbedRows];
  __shared__ float s_sig[kEmbedRows];
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
    s_tok[tid] = tok;
    s_q[tid] = q;
    s_sig[tid] = sig;
  }
  __syncthreads();
  for (int e = tid; e < kEmbedRows * rd.R; e += 256) {
    const int r = e / rd.R, k = e % rd.R;
    if (s_q[r] >= 0) {
      const T *Bq = (const T *)rd.b_table[s_q[r]];
      float v[8];
      Vec8<T>::load(Bq + (size_t)s_tok[r] * rd.R + k, 1, v);
      bsh[r][k] = v[0];
    }
  }
  __syncthreads();
  const int c0 = blockIdx.x * kEmbedCols + tid * 8;
  if (c0 >= a.n_embd) return;
  const int valid = min(8, a.n_embd - c0);
  float acc[kEmbedRows][8];
#pragma unroll
  for (int r = 0; r < kEmbedRows; ++r)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[r][j] = 0.f;
  // every distinct slot of the workgroup's rows once: its A rows against
  // the B entries of all of its rows
#pragma unroll
  for (int lead = 0; lead < kEmbedRows; ++lead) {
    const int q = s_q[lead];
    if (q < 0) continue;
    bool first = true;
#pragma unroll
    for (int r = 0; r < lead; ++r) first = first && s_q[r] != q;
    if (!first) continue;
    const T *Aq = (const T *)rd.a_table[q] + c0;
    for (int k = 0; k < rd.R; ++k) {
      float av[8];
      Vec8<T>::load(Aq + (size_t)k * a.n_embd, valid, av);
#pragma unroll
      for (int r = 0; r < kEmbedRows; ++r) {
        if (s_q[r] != q) continue;
        const float b = bsh[r][k];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[r][j] += b * av[j];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kEmbedRows; ++r) {
    const int tok = s_tok[r];
    if (tok < 0) continue;
    const T *er = (const T *)a.E + (size_t)tok * a.e_row_stride + c0;
    T *yr = (T *)a.y + (size_t)(i0 + r) * a.y_row_stride + c0;
    if (s_q[r] < 0) {  // base only: the table row, bit for bit
      Vec8<T>::copy(er, yr, valid);
      continue;
    }
    float ev[8];
    Vec8<T>::load(er, valid, ev);
#pragma unroll
    for (int j = 0; j < 8; ++j) ev[j] = ev[j] + s_sig[r] * acc[r][j];
    Vec8<T>::store(yr, valid, ev);
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
