// The fused op's last two steps as separate launches: the minimum over one
// spatial axis of a stored conv result, then the softmax over channels. This is
// the unfused form the fused kernel replaces (POPCORNBENCH "Kimi-K2.6" page
// l2_p24, opening turns: torch.min over the chosen axis of the Conv3d output,
// then torch.softmax over the channel axis; the page also weighs keeping the
// library conv and writing only these two steps as custom kernels). The library
// runs them to measure that chain beside the fused kernel.
//
// Both are bound by HBM bandwidth: each reads its input once and writes its
// output once, with every wave's loads covering whole contiguous runs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/convhip.h"

namespace convhip_unfused {

typedef float v4f __attribute__((ext_vector_type(4)));

// NaN-propagating minimum and maximum (v_minimum_f32 / v_maximum_f32): a NaN
// operand gives NaN, as torch.min and torch.softmax's row maximum do.
__device__ __forceinline__ float min_nan(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

constexpr int kThreads = 256;

// y viewed as [outer, R, inner]: out[o][i] = min over r of y[(o R + r) inner + i].
// One thread per 4 consecutive i (16-byte loads and stores), so a wave reads
// 1 KiB of one row of the reduced axis per step.
__global__ __launch_bounds__(kThreads) void min_axis_vec4_kernel(const float* __restrict__ y,
                                                                 float* __restrict__ out, int64_t outer, int R,
                                                                 int64_t inner4) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= outer * inner4) return;
  const int64_t o = t / inner4, i4 = t - o * inner4;
  const v4f* p = reinterpret_cast<const v4f*>(y) + o * R * inner4 + i4;
  v4f m = p[0];
#pragma unroll 4
  for (int r = 1; r < R; r++) {
    const v4f u = p[int64_t(r) * inner4];
    m = v4f{min_nan(m.x, u.x), min_nan(m.y, u.y), min_nan(m.z, u.z), min_nan(m.w, u.w)};
  }
  reinterpret_cast<v4f*>(out)[t] = m;
}

// Any inner size (the minimum over the last axis has inner = 1): one thread per
// output; adjacent threads read adjacent runs, so each wave's loads stay within
// the lines of its own contiguous block of the input.
__global__ __launch_bounds__(kThreads) void min_axis_kernel(const float* __restrict__ y, float* __restrict__ out,
                                                            int64_t outer, int R, int64_t inner) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= outer * inner) return;
  const int64_t o = t / inner, i = t - o * inner;
  const float* p = y + o * R * inner + i;
  float m = p[0];
#pragma unroll 8
  for (int r = 1; r < R; r++) m = min_nan(m, p[int64_t(r) * inner]);
  out[t] = m;
}

// z [N, C, S]: out[n, c, s] = exp(z[n,c,s] - M) / sum over c' of exp(z[n,c',s] - M),
// M = max over c of z[n,c,s]. One thread per (n, s); consecutive threads take
// consecutive s, so every channel's loads and stores are contiguous per wave.
// Up to CR channels stay in registers (one read of z); more take three passes,
// the second and third reading the wave's lines again from cache.
template <int CR>
__global__ __launch_bounds__(kThreads) void softmax_channels_kernel(const float* __restrict__ z,
                                                                    float* __restrict__ out, int64_t N, int C,
                                                                    int64_t S) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= N * S) return;
  const int64_t n = t / S, s = t - n * S;
  const float* p = z + n * C * S + s;
  float* q = out + n * C * S + s;
  if (C <= CR) {
    float v[CR];
#pragma unroll
    for (int c = 0; c < CR; c++) v[c] = c < C ? p[int64_t(c) * S] : 0.0f;
    float m = v[0];
#pragma unroll
    for (int c = 1; c < CR; c++)
      if (c < C) m = max_nan(m, v[c]);
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < CR; c++)
      if (c < C) {
        v[c] = expf(v[c] - m);
        sum += v[c];
      }
#pragma unroll
    for (int c = 0; c < CR; c++)
      if (c < C) q[int64_t(c) * S] = v[c] / sum;
    return;
  }
  float m = p[0];
  for (int c = 1; c < C; c++) m = max_nan(m, p[int64_t(c) * S]);
  float sum = 0.0f;
  for (int c = 0; c < C; c++) sum += expf(p[int64_t(c) * S] - m);
  for (int c = 0; c < C; c++) q[int64_t(c) * S] = expf(p[int64_t(c) * S] - m) / sum;
}

constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1;

}  // namespace convhip_unfused

using namespace convhip_unfused;

extern "C" {

int min_over_axis(const float* y, const int64_t* y_shape, int dim, float* out, convhip_stream_t stream) {
  if (!y_shape) return CONV_ERR_NULL;
  for (int a = 0; a < 5; a++)
    if (y_shape[a] < 1) return CONV_ERR_SHAPE;
  if (dim < 2 || dim > 4) return CONV_ERR_PARAM;
  if (!y || !out) return CONV_ERR_NULL;
  int64_t outer = 1, inner = 1;
  for (int a = 0; a < dim; a++) outer *= y_shape[a];
  for (int a = dim + 1; a < 5; a++) inner *= y_shape[a];
  const int64_t R = y_shape[dim];
  // Sizes: the element count must fit int64 comfortably and R an int.
  if (R > (int64_t(1) << 30) || outer > (int64_t(1) << 40) / R || inner > (int64_t(1) << 40) / (outer * R))
    return CONV_ERR_OVERFLOW;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool vec = inner % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  const int64_t items = vec ? outer * (inner / 4) : outer * inner;
  const int64_t blocks = (items + kThreads - 1) / kThreads;
  if (blocks > kMaxBlocks) return CONV_ERR_OVERFLOW;
  if (vec)
    hipLaunchKernelGGL(min_axis_vec4_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, y, out, outer, int(R),
                       inner / 4);
  else
    hipLaunchKernelGGL(min_axis_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, y, out, outer, int(R), inner);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

int softmax_over_channels(const float* z, const int64_t* z_shape, float* out, convhip_stream_t stream) {
  if (!z_shape) return CONV_ERR_NULL;
  for (int a = 0; a < 3; a++)
    if (z_shape[a] < 1) return CONV_ERR_SHAPE;
  if (!z || !out) return CONV_ERR_NULL;
  const int64_t N = z_shape[0], C = z_shape[1], S = z_shape[2];
  if (C > (int64_t(1) << 30) || N > (int64_t(1) << 40) / C || S > (int64_t(1) << 40) / (N * C))
    return CONV_ERR_OVERFLOW;
  const int64_t blocks = (N * S + kThreads - 1) / kThreads;
  if (blocks > kMaxBlocks) return CONV_ERR_OVERFLOW;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(softmax_channels_kernel<32>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, z, out, N, int(C),
                     S);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

}  // extern "C"
