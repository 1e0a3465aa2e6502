// k_small.hip -- the f32 path (all entry points) and the standalone expand-and-fold.
//
// The f32 path is the single-projection workload (a 256x256 f32 matrix, rank
// 8): a handful of rows, launch-latency bound.  One workgroup handles one row
// and a block of outputs; lanes stride along the contraction and a fixed
// xor-butterfly reduces each dot, so every result is reproducible.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <typename T> __device__ __forceinline__ float ld(const T *p, size_t i);
template <> __device__ __forceinline__ float ld<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<u16>(const u16 *p, size_t i) { return bf2f(p[i]); }

template <typename T> __device__ __forceinline__ void st(T *p, size_t i, float v);
template <> __device__ __forceinline__ void st<float>(float *p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st<u16>(u16 *p, size_t i, float v) { p[i] = f2bf(v); }

// ---------------------------------------------------------------- f32 shrink
// t[i, k] = A_s[k, :] . x_i  (ferrox LoraDelta::project), rows that skip untouched.
__global__ __launch_bounds__(256) void shrink_f32_kernel(RouteDev rd, Routing rt, const float *x,
                                                         int x_stride, int k_in, float *t) {
  const int i = blockIdx.x;
  int group, sidx;
  const int q = row_route(rt, rd, true, i, &group, &sidx);
  if (q < 0) return;
  const float *A = (const float *)rd.a_table[q];
  const float *xi = x + (size_t)i * x_stride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int k = wave; k < rd.R; k += 4) {
    float acc = 0.f;
    for (int c = lane; c < k_in; c += 64) acc += A[(size_t)k * k_in + c] * xi[c];
    acc = wave_sum(acc);
    if (lane == 0) t[(size_t)i * rd.R + k] = acc;
  }
}

// ---------------------------------------------------------------- f32 apply
// y_i = W x_i + s B_s (A_s x_i), one row per blockIdx.y, 16 outputs per
// block: each wave takes 4 outputs at once, their loads in flight together
// (a wave per output one after another would be a chain of memory round
// trips).  Each dot runs lanes-strided over k, then a fixed butterfly.
constexpr int kF32Out = 16;

__global__ __launch_bounds__(256) void apply_f32_kernel(RouteDev rd, Routing rt, bool has_lora,
                                                        const float *W, long long w_group_stride,
                                                        int w_stride, const float *x,
                                                        int x_stride, int k_in, int n_out,
                                                        float *y, int y_stride) {
  __shared__ float tsh[256];
  const int i = blockIdx.y;
  int group, sidx;
  const int q = row_route(rt, rd, has_lora, i, &group, &sidx);
  if (q == kDrop) return;
  const float *xi = x + (size_t)i * x_stride;
  const float *Wg = W + (size_t)group * (size_t)w_group_stride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (q >= 0) {
    const float *A = (const float *)rd.a_table[q];
    for (int k = wave; k < rd.R; k += 4) {
      float acc = 0.f;
      for (int c = lane; c < k_in; c += 64) acc += A[(size_t)k * k_in + c] * xi[c];
      acc = wave_sum(acc);
      if (lane == 0) tsh[k] = acc;
    }
  }
  __syncthreads();
  const int o0 = blockIdx.x * kF32Out + wave * 4;
  int oo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) oo[j] = min(o0 + j, n_out - 1);  // a clamped duplicate is not written
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c = lane; c < k_in; c += 64) {
    const float xv = xi[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += Wg[(size_t)oo[j] * w_stride + c] * xv;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = wave_sum(acc[j]);
  if (q >= 0) {
    const float *B = (const float *)rd.b_table[q];
    float d[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = lane; k < rd.R; k += 64) {
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] += B[(size_t)oo[j] * rd.R + k] * tsh[k];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = acc[j] + rd.scale_table[sidx] * wave_sum(d[j]);
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (o0 + j < n_out) y[(size_t)i * y_stride + o0 + j] = acc[j];
  }
}

// ---------------------------------------------------------------- expand + fold
// y[i, o] = y[i, o] + s * (B_pair t_i)[o] for rows that resolve; others untouched
// (rows outside every range too).  One thread per output; t_i staged in LDS;
// the rank sum runs k ascending.
template <typename T>
__global__ __launch_bounds__(256) void expand_fold_kernel(RouteDev rd, Routing rt, const float *t,
                                                          T *y, int y_stride, int n_out) {
  __shared__ float tsh[256];
  const int i = blockIdx.y;
  int group, sidx;
  const int q = row_route(rt, rd, true, i, &group, &sidx);
  if (q < 0) return;
  for (int k = threadIdx.x; k < rd.R; k += 256) tsh[k] = t[(size_t)i * rd.R + k];
  __syncthreads();
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= n_out) return;
  const T *B = (const T *)rd.b_table[q];
  float d = 0.f;
  for (int k = 0; k < rd.R; ++k) d += ld(B, (size_t)o * rd.R + k) * tsh[k];
  const size_t yi = (size_t)i * y_stride + o;
  st(y, yi, ld((const T *)y, yi) + rd.scale_table[sidx] * d);
}

// ---------------------------------------------------------------- stack fold
// The extra levels of an adapter stack (ferrox LoraStack: every adapter a
// term of the sum, in order): y[i, o] = y[i, o] + sum over levels of
// s_l * (B_l t_l[i])[o], the level sum in f32 and y rounded once.  A row no
// level resolves is untouched.  One thread per output; each resolved
// level's t row staged in LDS.
template <typename T>
__global__ __launch_bounds__(256) void expand_fold_stack_kernel(StackFold f, T *y, int y_stride, int n_out) {
  __shared__ float tsh[kMaxStackLevels][256];
  __shared__ int q_of[kMaxStackLevels];
  const int i = blockIdx.y;
  if (threadIdx.x < f.n_levels) {
    const StackLevel &L = f.lv[threadIdx.x];
    q_of[threadIdx.x] = resolve_slot(L.seq_slot[i], 0, L.max_loras, 1, L.a_table, L.b_table, L.scale_table);
  }
  __syncthreads();
  bool any = false;
  for (int l = 0; l < f.n_levels; ++l) {
    if (q_of[l] < 0) continue;
    any = true;
    for (int k = threadIdx.x; k < f.lv[l].R; k += 256) tsh[l][k] = f.lv[l].t[(size_t)i * f.lv[l].R + k];
  }
  if (!any) return;  // uniform: q_of is the same for every thread
  __syncthreads();
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= n_out) return;
  float acc = 0.f;
  for (int l = 0; l < f.n_levels; ++l) {
    const int q = q_of[l];
    if (q < 0) continue;
    const StackLevel &L = f.lv[l];
    const T *B = (const T *)L.b_table[q];
    float d = 0.f;
    for (int k = 0; k < L.R; ++k) d += ld(B, (size_t)o * L.R + k) * tsh[l][k];
    acc += L.scale_table[L.seq_slot[i]] * d;
  }
  const size_t yi = (size_t)i * y_stride + o;
  st(y, yi, ld((const T *)y, yi) + acc);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_shrink_f32(const RouteDev &rd, const Routing &rt, const float *x, int x_stride,
                             int k_in, int n, float *t, hipStream_t st) {
  hipLaunchKernelGGL(shrink_f32_kernel, dim3(n), dim3(256), 0, st, rd, rt, x, x_stride, k_in, t);
  return hipGetLastError();
}

hipError_t launch_apply_f32(const RouteDev &rd, const Routing &rt, bool has_lora, const float *W,
                            long long w_group_stride, int w_stride, const float *x, int x_stride,
                            int k_in, int n_out, int n, float *y, int y_stride, hipStream_t st) {
  dim3 grid((n_out + kF32Out - 1) / kF32Out, n);
  hipLaunchKernelGGL(apply_f32_kernel, grid, dim3(256), 0, st, rd, rt, has_lora, W,
                     w_group_stride, w_stride, x, x_stride, k_in, n_out, y, y_stride);
  return hipGetLastError();
}

hipError_t launch_expand_fold(const RouteDev &rd, int dtype, const Routing &rt, const float *t,
                              void *y, int y_stride, int n_out, int n, hipStream_t st) {
  dim3 grid((n_out + 255) / 256, n);
  if (dtype == 0)
    hipLaunchKernelGGL(expand_fold_kernel<float>, grid, dim3(256), 0, st, rd, rt, t, (float *)y,
                       y_stride, n_out);
  else
    hipLaunchKernelGGL(expand_fold_kernel<u16>, grid, dim3(256), 0, st, rd, rt, t, (u16 *)y,
                       y_stride, n_out);
  return hipGetLastError();
}

hipError_t launch_expand_fold_stack(const StackFold &f, int dtype, void *y, int y_stride, int n_out, int n,
                                    hipStream_t st) {
  dim3 grid((n_out + 255) / 256, n);
  if (dtype == 0)
    hipLaunchKernelGGL(expand_fold_stack_kernel<float>, grid, dim3(256), 0, st, f, (float *)y, y_stride, n_out);
  else
    hipLaunchKernelGGL(expand_fold_stack_kernel<u16>, grid, dim3(256), 0, st, f, (u16 *)y, y_stride, n_out);
  return hipGetLastError();
}

}  // namespace lora
