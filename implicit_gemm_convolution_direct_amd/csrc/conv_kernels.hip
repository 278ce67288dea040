// fp32 convolution kernels for gfx950 (MI355X) and the C-ABI entry points.
//
// conv_mfma16: implicit-GEMM direct convolution. Per workgroup, an output tile
//   of BM channels x BN positions is a GEMM  Y[m][n] = sum_k W[m][k] * Xhat[k][n]
//   with k = (input channel, kernel tap). Xhat is never formed: the input halo
//   box of a chunk of input channels is staged in LDS once, and each matrix-core
//   operand is gathered from it through a per-k offset table (koff) plus a
//   per-position offset (noff), so one LDS copy of every input element serves
//   all taps and all BM output channels. The contraction runs on
//   v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate).
//
// fused_min_softmax_mfma4: Conv3d -> min over depth -> softmax over channels.
//   One lane owns one output column (n, oh, ow) and all its channels, using the
//   4x4x1 matrix-core form with the weight operand broadcast from one 4-lane
//   block (cbsz=4): each instruction updates 4 channels x 64 columns. The
//   running minimum over output depth and the softmax over channels both stay
//   in the lane's registers; only the final [N, C_out, H_out, W_out] is stored.
//
// Problem statements: POPCORNBENCH "Kimi-K2.6" pages l1_p60 (Conv3d), l1_p76
// (Conv1d), l2_p24 (Conv3d + min + softmax), opening turns.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <utility>

#include "../../include/convhip.h"
#include "convhip_plan.h"

namespace convhip {

typedef float v4f __attribute__((ext_vector_type(4)));

struct ConvArgs {
  const float* __restrict__ x;
  const float* __restrict__ w;
  const float* __restrict__ bias;
  float* __restrict__ y;
  int Cin, Cout, Cg, Coutg;
  int L0, L1, L2;
  int K0, K1, K2;
  int S0, S1, S2;
  int D0, D1, D2;
  int P0, P1, P2;
  int O0, O1, O2;
  int kvol, kfull;
  int mode, Cc, kc_pad, ldw, kdspan, rows, bw, boxc;
  int row_tiles, ctiles;
  int plane_out;
};

// ---------------------------------------------------------------------------
// conv_mfma16
// ---------------------------------------------------------------------------
template <int MT, int NT, int WM, int WN>
__global__ __launch_bounds__(256) void conv_mfma16_kernel(ConvArgs a) {
  constexpr int BM = 16 * MT * WM;
  constexpr int BN = 16 * NT * WN;
  extern __shared__ float smem[];
  float* Xs = smem;
  const int zero_idx = a.Cc * a.boxc;
  int* koff = reinterpret_cast<int*>(smem + zero_idx + 4);
  float* Ws = smem + zero_idx + 4 + a.kc_pad;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave - wm * WN;
  const int kg = lane >> 4;   // k row of this lane inside a 4-deep MFMA step
  const int li = lane & 15;   // m (A operand) or n (B operand) index of this lane

  // Workgroup coordinates: position tile, (n, od) plane, (group, channel tile).
  const int tile = blockIdx.x;
  const int plane = blockIdx.y;
  const int n = plane / a.O0;
  const int od = plane - n * a.O0;
  const int gz = blockIdx.z;
  const int g = gz / a.ctiles;
  const int m0 = (gz - g * a.ctiles) * BM;

  int oh_first, oh_last, ow0 = 0, p0 = 0;
  if (a.mode == TILE_FLAT) {
    p0 = tile * BN;
    const int p_last = min(p0 + BN, a.plane_out) - 1;
    oh_first = p0 / a.O2;
    oh_last = p_last / a.O2;
  } else {
    oh_first = oh_last = tile / a.row_tiles;
    ow0 = (tile - oh_first * a.row_tiles) * BN;
  }
  const int iwb = ow0 * a.S2;  // box column 0 is input column iwb - P2
  const int rows_needed = (oh_last - oh_first) * a.S1 + (a.K1 - 1) * a.D1 + 1;
  const int id0 = od * a.S0 - a.P0;
  const int ih0 = oh_first * a.S1 - a.P1;
  const int iw0 = iwb - a.P2;
  const int plane_stride = a.rows * a.bw;

  // Offset of every (channel, tap) of a chunk inside the staged box. Padding taps
  // (k >= Cc*kvol) carry zero weights and point at the box start, so the value
  // they multiply is a staged, finite input element.
  for (int k = tid; k < a.kc_pad; k += 256) {
    int off = 0;
    if (k < a.Cc * a.kvol) {
      const int c = k / a.kvol;
      const int r = k - c * a.kvol;
      const int td = r / (a.K1 * a.K2);
      const int r2 = r - td * a.K1 * a.K2;
      const int th = r2 / a.K2;
      const int tw = r2 - th * a.K2;
      off = c * a.boxc + td * a.D0 * plane_stride + th * a.D1 * a.bw + tw * a.D2;
    }
    koff[k] = off;
  }

  // Per-lane output positions of this wave's NT sub-tiles.
  int noff[NT];
  int pidx[NT];
#pragma unroll
  for (int ni = 0; ni < NT; ni++) {
    const int q = wn * (16 * NT) + 16 * ni + li;
    int oh, ow, valid;
    if (a.mode == TILE_FLAT) {
      const int p = p0 + q;
      valid = p < a.plane_out;
      oh = p / a.O2;
      ow = p - oh * a.O2;
    } else {
      oh = oh_first;
      ow = ow0 + q;
      valid = ow < a.O2;
    }
    noff[ni] = valid ? (oh - oh_first) * a.S1 * a.bw + ow * a.S2 - iwb : 0;
    pidx[ni] = valid ? oh * a.O2 + ow : -1;
  }

  v4f acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; mi++)
#pragma unroll
    for (int ni = 0; ni < NT; ni++) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t x_n = (int64_t(n) * a.Cin + int64_t(g) * a.Cg) * a.L0;
  const int wrow = wm * 16 * MT + li;

  for (int c0 = 0; c0 < a.Cg; c0 += a.Cc) {
    const int cc_count = min(a.Cc, a.Cg - c0);
    __syncthreads();  // previous chunk's reads are complete (and the koff table is written)

    // Stage the input box of this chunk: rows of bw contiguous input columns.
    const int rows_per_c = a.kdspan * rows_needed;
    const int nrows = a.Cc * rows_per_c;
    for (int r = wave; r < nrows; r += 4) {
      const int c = r / rows_per_c;
      const int rem = r - c * rows_per_c;
      const int zd = rem / rows_needed;
      const int zr = rem - zd * rows_needed;
      const int id = id0 + zd;
      const int ih = ih0 + zr;
      const bool rv = (c < cc_count) && (id >= 0) && (id < a.L0) && (ih >= 0) && (ih < a.L1);
      const float* src = a.x + ((x_n + int64_t(c0 + c) * a.L0 + (rv ? id : 0)) * a.L1 + (rv ? ih : 0)) * a.L2;
      float* dst = Xs + c * a.boxc + zd * plane_stride + zr * a.bw;
      for (int col = lane; col < a.bw; col += 64) {
        const int iw = iw0 + col;
        float v = 0.0f;
        if (rv && iw >= 0 && iw < a.L2) v = src[iw];
        dst[col] = v;
      }
    }
    // Stage the weight chunk transposed to [k][m] (zero beyond the valid k and m).
    const int kvalid = cc_count * a.kvol;
    for (int idx = tid; idx < a.kc_pad * BM; idx += 256) {
      const int m = idx / a.kc_pad;
      const int k = idx - m * a.kc_pad;
      const int co = m0 + m;
      float v = 0.0f;
      if (k < kvalid && co < a.Coutg) v = a.w[int64_t(g * a.Coutg + co) * a.kfull + c0 * a.kvol + k];
      Ws[k * a.ldw + m] = v;
    }
    __syncthreads();

    const int nsteps = a.kc_pad >> 2;
    for (int s = 0; s < nsteps; s++) {
      const int kk = 4 * s + kg;
      const int ko = koff[kk];
      float av[MT], bv[NT];
#pragma unroll
      for (int mi = 0; mi < MT; mi++) av[mi] = Ws[kk * a.ldw + wrow + 16 * mi];
#pragma unroll
      for (int ni = 0; ni < NT; ni++) bv[ni] = Xs[ko + noff[ni]];
#pragma unroll
      for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    }
  }

  // Epilogue: D[m][n] sits in lane n + 16*(m/4), register m%4.
  const int64_t out_plane = int64_t(a.O1) * a.O2;
#pragma unroll
  for (int mi = 0; mi < MT; mi++) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int ch = m0 + wm * 16 * MT + 16 * mi + 4 * kg + r;
      if (ch < a.Coutg) {
        const int co = g * a.Coutg + ch;
        const float b = a.bias ? a.bias[co] : 0.0f;
        float* yp = a.y + ((int64_t(n) * a.Cout + co) * a.O0 + od) * out_plane;
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
          if (pidx[ni] >= 0) yp[pidx[ni]] = acc[mi][ni][r] + b;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fused_min_softmax_mfma4
// ---------------------------------------------------------------------------
struct FusedArgs {
  const float* __restrict__ x;
  const float* __restrict__ w;
  const float* __restrict__ bias;
  float* __restrict__ y;
  int Cin, Cout;
  int L0, L1, L2;
  int K0, K1, K2;
  int S0, S1, S2;
  int D0, D1, D2;
  int P0, P1, P2;
  int O0, O1, O2;
  int kvol, kfull, cpad;
  int mode, dspan, rows, bw, boxc, row_tiles;
  int plane_out;
};

template <int A>
__device__ __forceinline__ void mfma4_bcast(float av, float bv, v4f* acc) {
  acc[A] = __builtin_amdgcn_mfma_f32_4x4x1f32(av, bv, acc[A], 4, A, 0);
}

template <int NG, int... I>
__device__ __forceinline__ void mfma4_all(float av, float bv, v4f* acc, std::integer_sequence<int, I...>) {
  (mfma4_bcast<I>(av, bv, acc), ...);
}

template <int NG>
__global__ __launch_bounds__(256) void fused_min_softmax_mfma4_kernel(FusedArgs a) {
  extern __shared__ float smem[];
  float* Xs = smem;
  const int box = a.Cin * a.boxc;
  const int red_floats = 4 * a.cpad * 64;
  const int region = max(box + 4, red_floats);
  int* koff = reinterpret_cast<int*>(smem + region);
  float* Wt = smem + region + a.kfull;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tile = blockIdx.x;
  const int n = blockIdx.y;

  int oh_first, oh_last, ow0 = 0, p0 = 0;
  if (a.mode == TILE_FLAT) {
    p0 = tile * 64;
    const int p_last = min(p0 + 64, a.plane_out) - 1;
    oh_first = p0 / a.O2;
    oh_last = p_last / a.O2;
  } else {
    oh_first = oh_last = tile / a.row_tiles;
    ow0 = (tile - oh_first * a.row_tiles) * 64;
  }
  const int iwb = ow0 * a.S2;
  const int rows_needed = (oh_last - oh_first) * a.S1 + (a.K1 - 1) * a.D1 + 1;
  const int ih0 = oh_first * a.S1 - a.P1;
  const int iw0 = iwb - a.P2;
  const int plane_stride = a.rows * a.bw;

  for (int k = tid; k < a.kfull; k += 256) {
    const int c = k / a.kvol;
    const int r = k - c * a.kvol;
    const int td = r / (a.K1 * a.K2);
    const int r2 = r - td * a.K1 * a.K2;
    const int th = r2 / a.K2;
    const int tw = r2 - th * a.K2;
    koff[k] = c * a.boxc + td * a.D0 * plane_stride + th * a.D1 * a.bw + tw * a.D2;
  }
  // Weights transposed to [k][c_out] so lane c reads channel c of tap k.
  for (int idx = tid; idx < a.kfull * a.cpad; idx += 256) {
    const int c = idx / a.kfull;
    const int k = idx - c * a.kfull;
    Wt[k * a.cpad + c] = (c < a.Cout) ? a.w[int64_t(c) * a.kfull + k] : 0.0f;
  }
  // Input box: all input planes the output depths read, rows of this tile.
  const int rows_per_c = a.dspan * rows_needed;
  const int nrows = a.Cin * rows_per_c;
  const int64_t x_n = int64_t(n) * a.Cin * a.L0;
  for (int r = wave; r < nrows; r += 4) {
    const int c = r / rows_per_c;
    const int rem = r - c * rows_per_c;
    const int zd = rem / rows_needed;
    const int zr = rem - zd * rows_needed;
    const int id = zd - a.P0;
    const int ih = ih0 + zr;
    const bool rv = (id >= 0) && (id < a.L0) && (ih >= 0) && (ih < a.L1);
    const float* src = a.x + ((x_n + int64_t(c) * a.L0 + (rv ? id : 0)) * a.L1 + (rv ? ih : 0)) * a.L2;
    float* dst = Xs + c * a.boxc + zd * plane_stride + zr * a.bw;
    for (int col = lane; col < a.bw; col += 64) {
      const int iw = iw0 + col;
      float v = 0.0f;
      if (rv && iw >= 0 && iw < a.L2) v = src[iw];
      dst[col] = v;
    }
  }
  __syncthreads();

  // This lane's output column.
  int oh, ow, valid;
  if (a.mode == TILE_FLAT) {
    const int p = p0 + lane;
    valid = p < a.plane_out;
    oh = p / a.O2;
    ow = p - oh * a.O2;
  } else {
    oh = oh_first;
    ow = ow0 + lane;
    valid = ow < a.O2;
  }
  const int noff = valid ? (oh - oh_first) * a.S1 * a.bw + ow * a.S2 - iwb : 0;
  const int wlane = min(lane, a.cpad - 1);

  v4f mn[NG];
#pragma unroll
  for (int i = 0; i < NG; i++) mn[i] = v4f{INFINITY, INFINITY, INFINITY, INFINITY};

  for (int od = wave; od < a.O0; od += 4) {
    const int base = od * a.S0 * plane_stride + noff;
    v4f acc[NG];
#pragma unroll
    for (int i = 0; i < NG; i++) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < a.kfull; k++) {
      const float bv = Xs[koff[k] + base];
      const float av = Wt[k * a.cpad + wlane];
      mfma4_all<NG>(av, bv, acc, std::make_integer_sequence<int, NG>{});
    }
#pragma unroll
    for (int i = 0; i < NG; i++) {
      mn[i][0] = fminf(mn[i][0], acc[i][0]);
      mn[i][1] = fminf(mn[i][1], acc[i][1]);
      mn[i][2] = fminf(mn[i][2], acc[i][2]);
      mn[i][3] = fminf(mn[i][3], acc[i][3]);
    }
  }

  // Merge the four waves' minima through LDS (the box is no longer needed).
  __syncthreads();
  float* red = smem;
#pragma unroll
  for (int i = 0; i < NG; i++)
#pragma unroll
    for (int r = 0; r < 4; r++) red[(wave * a.cpad + 4 * i + r) * 64 + lane] = mn[i][r];
  __syncthreads();
  if (wave == 0 && valid) {
    float m[4 * NG];
#pragma unroll
    for (int c = 0; c < 4 * NG; c++) {
      float v = red[c * 64 + lane];
      v = fminf(v, red[(a.cpad + c) * 64 + lane]);
      v = fminf(v, red[(2 * a.cpad + c) * 64 + lane]);
      v = fminf(v, red[(3 * a.cpad + c) * 64 + lane]);
      // fp32 addition is monotone, so min(v_i) + b == min(v_i + b) exactly.
      m[c] = (c < a.Cout) ? v + (a.bias ? a.bias[c] : 0.0f) : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4 * NG; c++) mx = fmaxf(mx, m[c]);
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < 4 * NG; c++) {
      const float e = (c < a.Cout) ? expf(m[c] - mx) : 0.0f;
      m[c] = e;
      sum += e;
    }
    const float inv_den = 1.0f / sum;
    const int64_t out_plane = int64_t(a.O1) * a.O2;
    float* yp = a.y + int64_t(n) * a.Cout * out_plane + int64_t(oh) * a.O2 + ow;
#pragma unroll
    for (int c = 0; c < 4 * NG; c++)
      if (c < a.Cout) yp[int64_t(c) * out_plane] = m[c] * inv_den;
  }
}

// ---------------------------------------------------------------------------
// Device-side synthetic input generator (SplitMix64, one output per element).
// ---------------------------------------------------------------------------
__global__ void synth_fill_kernel(float* __restrict__ dst, int64_t count, uint64_t seed, uint64_t start,
                                  int kind, float bound, int lo, int span) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) {
    uint64_t z = seed + (start + uint64_t(i) + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z = z ^ (z >> 31);
    const uint64_t m = z >> 40;
    float v;
    if (kind == 0) {
      v = float(uint32_t(m)) * 0x1p-24f;
    } else if (kind == 1) {
      const float u = float(uint32_t(m)) * 0x1p-24f;
      const float t = 2.0f * u - 1.0f;  // exact
      v = __fmul_rn(t, bound);
    } else {
      v = float(int64_t(lo) + int64_t((m * uint64_t(span)) >> 24));
    }
    dst[i] = v;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
typedef void (*ConvKernelFn)(ConvArgs);

template <int MT, int NT, int WM, int WN>
static int launch_conv_cfg(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  auto fn = conv_mfma16_kernel<MT, NT, WM, WN>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsLimit));
  });
  if (attr_err != hipSuccess) return CONV_ERR_HIP;
  dim3 grid(unsigned(p.grid[0]), unsigned(p.grid[1]), unsigned(p.grid[2]));
  hipLaunchKernelGGL(fn, grid, dim3(256), size_t(p.lds_bytes), stream, args);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

template <int NG>
static int launch_fused_ng(const FusedArgs& args, const FusedPlan& p, hipStream_t stream) {
  auto fn = fused_min_softmax_mfma4_kernel<NG>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsLimit));
  });
  if (attr_err != hipSuccess) return CONV_ERR_HIP;
  dim3 grid(unsigned(p.grid[0]), unsigned(p.grid[1]), unsigned(p.grid[2]));
  hipLaunchKernelGGL(fn, grid, dim3(256), size_t(p.lds_bytes), stream, args);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

static ConvArgs conv_args(const Geom& g, const ConvPlan& p, const float* x, const float* w, const float* bias,
                          float* y) {
  ConvArgs a;
  a.x = x; a.w = w; a.bias = bias; a.y = y;
  a.Cin = int(g.Cin); a.Cout = int(g.Cout); a.Cg = int(g.Cg); a.Coutg = int(g.Coutg);
  a.L0 = int(g.L[0]); a.L1 = int(g.L[1]); a.L2 = int(g.L[2]);
  a.K0 = int(g.K[0]); a.K1 = int(g.K[1]); a.K2 = int(g.K[2]);
  a.S0 = int(g.S[0]); a.S1 = int(g.S[1]); a.S2 = int(g.S[2]);
  a.D0 = int(g.Dl[0]); a.D1 = int(g.Dl[1]); a.D2 = int(g.Dl[2]);
  a.P0 = int(g.P[0]); a.P1 = int(g.P[1]); a.P2 = int(g.P[2]);
  a.O0 = int(g.O[0]); a.O1 = int(g.O[1]); a.O2 = int(g.O[2]);
  a.kvol = int(g.kvol()); a.kfull = int(g.kred());
  a.mode = p.mode; a.Cc = p.Cc; a.kc_pad = p.kc_pad; a.ldw = p.ldw; a.kdspan = p.kdspan;
  a.rows = p.rows; a.bw = p.bw; a.boxc = p.boxc; a.row_tiles = p.row_tiles; a.ctiles = p.ctiles;
  a.plane_out = int(g.plane_out());
  return a;
}

}  // namespace convhip

using namespace convhip;

extern "C" {

int conv_out_shape(int nd, const int64_t* in_spatial, const int64_t* k_spatial, const int* stride,
                   const int* dilation, const int* padding, int64_t* out_spatial) {
  if (nd < 1 || nd > 3) return CONV_ERR_RANK;
  if (!in_spatial || !k_spatial || !stride || !dilation || !padding || !out_spatial) return CONV_ERR_NULL;
  for (int a = 0; a < nd; a++)
    if (stride[a] < 1 || dilation[a] < 1 || padding[a] < 0 || k_spatial[a] < 1 || in_spatial[a] < 1)
      return CONV_ERR_PARAM;
  int rc = CONV_OK;
  for (int a = 0; a < nd; a++) {
    out_spatial[a] = out_len(in_spatial[a], k_spatial[a], stride[a], dilation[a], padding[a]);
    if (out_spatial[a] < 1) rc = CONV_ERR_EMPTY_OUTPUT;
  }
  return rc;
}

const char* conv_status_string(int status) {
  switch (status) {
    case CONV_OK: return "CONV_OK";
    case CONV_ERR_NULL: return "CONV_ERR_NULL: a required pointer is NULL";
    case CONV_ERR_RANK: return "CONV_ERR_RANK: nd must be 1 or 3";
    case CONV_ERR_SHAPE: return "CONV_ERR_SHAPE: bad dimension or weight shape";
    case CONV_ERR_GROUPS: return "CONV_ERR_GROUPS: groups < 1 or channels not divisible by groups";
    case CONV_ERR_PARAM: return "CONV_ERR_PARAM: stride/dilation < 1 or padding < 0";
    case CONV_ERR_EMPTY_OUTPUT: return "CONV_ERR_EMPTY_OUTPUT: an output length is <= 0";
    case CONV_ERR_UNSUPPORTED: return "CONV_ERR_UNSUPPORTED: valid arguments this build does not handle";
    case CONV_ERR_OVERFLOW: return "CONV_ERR_OVERFLOW: a size exceeds the index arithmetic";
    case CONV_ERR_HIP: return "CONV_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown conv_status";
  }
}

int conv_plan_describe(int nd, const int64_t* x_shape, const int64_t* w_shape, const int* stride,
                       const int* dilation, const int* padding, int groups, int fused, char* buf, int buflen) {
  if (!buf || buflen < 1) return CONV_ERR_NULL;
  buf[0] = 0;
  Geom g;
  int rc = make_geom(nd, x_shape, w_shape, stride, dilation, padding, groups, &g);
  if (rc != CONV_OK) return rc;
  std::string s;
  if (fused) {
    FusedPlan p;
    rc = plan_fused(g, 2, &p);
    if (rc != CONV_OK) return rc;
    s = describe(g, p);
  } else {
    ConvPlan p;
    rc = plan_conv(g, &p);
    if (rc != CONV_OK) return rc;
    s = describe(g, p);
  }
  std::snprintf(buf, size_t(buflen), "%s", s.c_str());
  return CONV_OK;
}

int conv_fwd(int nd, const float* x, const int64_t* x_shape, const float* w, const int64_t* w_shape,
             const float* bias, const int* stride, const int* dilation, const int* padding, int groups, float* y,
             convhip_stream_t stream) {
  Geom g;
  int rc = make_geom(nd, x_shape, w_shape, stride, dilation, padding, groups, &g);
  if (rc != CONV_OK) return rc;
  if (!x || !w || !y) return CONV_ERR_NULL;
  ConvPlan p;
  rc = plan_conv(g, &p);
  if (rc != CONV_OK) return rc;
  ConvArgs a = conv_args(g, p, x, w, bias, y);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (p.cfg) {
    case CFG_M16: return launch_conv_cfg<1, 4, 1, 4>(a, p, s);
    case CFG_M32: return launch_conv_cfg<2, 4, 1, 4>(a, p, s);
    case CFG_M64: return launch_conv_cfg<4, 4, 1, 4>(a, p, s);
    default: return launch_conv_cfg<4, 4, 2, 2>(a, p, s);
  }
}

int conv3d_min_softmax(const float* x, const int64_t* x_shape, const float* w, const int64_t* w_shape,
                       const float* bias, const int* stride, const int* dilation, const int* padding, int groups,
                       int min_dim, float* y, convhip_stream_t stream) {
  Geom g;
  int rc = make_geom(3, x_shape, w_shape, stride, dilation, padding, groups, &g);
  if (rc != CONV_OK) return rc;
  if (!x || !w || !y) return CONV_ERR_NULL;
  if (min_dim < 2 || min_dim > 4) return CONV_ERR_PARAM;
  FusedPlan p;
  rc = plan_fused(g, min_dim, &p);
  if (rc != CONV_OK) return rc;
  FusedArgs a;
  a.x = x; a.w = w; a.bias = bias; a.y = y;
  a.Cin = int(g.Cin); a.Cout = int(g.Cout);
  a.L0 = int(g.L[0]); a.L1 = int(g.L[1]); a.L2 = int(g.L[2]);
  a.K0 = int(g.K[0]); a.K1 = int(g.K[1]); a.K2 = int(g.K[2]);
  a.S0 = int(g.S[0]); a.S1 = int(g.S[1]); a.S2 = int(g.S[2]);
  a.D0 = int(g.Dl[0]); a.D1 = int(g.Dl[1]); a.D2 = int(g.Dl[2]);
  a.P0 = int(g.P[0]); a.P1 = int(g.P[1]); a.P2 = int(g.P[2]);
  a.O0 = int(g.O[0]); a.O1 = int(g.O[1]); a.O2 = int(g.O[2]);
  a.kvol = int(g.kvol()); a.kfull = p.kfull; a.cpad = p.cpad;
  a.mode = p.mode; a.dspan = p.dspan; a.rows = p.rows; a.bw = p.bw; a.boxc = p.boxc; a.row_tiles = p.row_tiles;
  a.plane_out = int(g.plane_out());
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (p.ng) {
    case 1: return launch_fused_ng<1>(a, p, s);
    case 2: return launch_fused_ng<2>(a, p, s);
    case 3: return launch_fused_ng<3>(a, p, s);
    case 4: return launch_fused_ng<4>(a, p, s);
    case 5: return launch_fused_ng<5>(a, p, s);
    case 6: return launch_fused_ng<6>(a, p, s);
    case 7: return launch_fused_ng<7>(a, p, s);
    case 8: return launch_fused_ng<8>(a, p, s);
    case 9: return launch_fused_ng<9>(a, p, s);
    case 10: return launch_fused_ng<10>(a, p, s);
    case 11: return launch_fused_ng<11>(a, p, s);
    case 12: return launch_fused_ng<12>(a, p, s);
    case 13: return launch_fused_ng<13>(a, p, s);
    case 14: return launch_fused_ng<14>(a, p, s);
    case 15: return launch_fused_ng<15>(a, p, s);
    default: return launch_fused_ng<16>(a, p, s);
  }
}

int convhip_synth_fill(float* dst, int64_t count, uint64_t seed, uint64_t start, int kind, float bound, int lo,
                       int span, convhip_stream_t stream) {
  if (!dst) return CONV_ERR_NULL;
  if (kind < 0 || kind > 2 || span < 1 || count < 0) return CONV_ERR_PARAM;
  if (count == 0) return CONV_OK;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(synth_fill_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), dst, count, seed, start, kind, bound, lo, span);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

}  // extern "C"
