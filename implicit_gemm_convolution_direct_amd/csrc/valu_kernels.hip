// Direct convolution on the vector ALU (plain fp32 FMA, no matrix cores): the
// thread-per-output kernel design of POPCORNBENCH "Kimi-K2.6" page l1_p60
// (design monologue: each thread owns output positions, loops over input
// channels and kernel taps, weights staged in shared memory next to the
// input) and page l1_p76 turn 2 (several output channels per thread from one
// input load), recast for a 64-wide wavefront: every lane of a workgroup
// computes the same CO output channels of one group at PP output positions, so
// the weights of a (channel, tap) are one broadcast LDS read for the whole
// wave and each input value loaded feeds CO FMAs.
//
// It serves the geometries the matrix-core kernels cannot stage (large kernels
// over many channels), and, forced, measures per shape which unit the
// convolution should run on.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>

#include "../../include/convhip.h"
#include "convhip_plan.h"

namespace convhip {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

struct ValuArgs {
  const float* x;
  const float* w;
  const float* bias;
  float* y;
  int Cin, Cg, Cout, Coutg;
  int L0, L1, L2;  // input D, H, W
  int K0, K1, K2;  // kernel
  int S0, S1, S2;
  int D0, D1, D2;
  int P0, P1, P2;
  int O0, O1, O2;  // output D, H, W
  int npos;        // N * O0 * O1 * O2
  int ncob;        // channel blocks of CO per group
  int pps;         // (input channel, depth tap) pairs staged per LDS buffer
};

// acc[pp][4q..4q+3] += xv[pp] * w4 for every position pp.
template <int CO, int PP>
__device__ __forceinline__ void fma_tap(float (&acc)[PP][CO], const float (&xv)[PP], const v4f* wr) {
#pragma unroll
  for (int q = 0; q < CO / 4; q++) {
    const v4f wv = wr[q];
#pragma unroll
    for (int pp = 0; pp < PP; pp++) {
      acc[pp][4 * q + 0] = __builtin_fmaf(xv[pp], wv.x, acc[pp][4 * q + 0]);
      acc[pp][4 * q + 1] = __builtin_fmaf(xv[pp], wv.y, acc[pp][4 * q + 1]);
      acc[pp][4 * q + 2] = __builtin_fmaf(xv[pp], wv.z, acc[pp][4 * q + 2]);
      acc[pp][4 * q + 3] = __builtin_fmaf(xv[pp], wv.w, acc[pp][4 * q + 3]);
    }
  }
}

// One workgroup: T lanes x PP positions (position p = block base + pp * T +
// lane) times CO output channels of one group. The reduction runs over
// (input channel, depth tap) pairs; the weights of `pps` consecutive pairs,
// CO x kH x kW each, are staged transposed, [pair][tap][CO], in one of two LDS
// buffers, one barrier per stage (a buffer is rewritten two stages later,
// after every lane has passed the barrier that follows its use).
// CL: channels-last tensors, x [N, D, H, W, C_in] and y [N, D_out, H_out,
// W_out, C_out]; otherwise NCDHW.
template <int CO, int PP, int T, bool CL>
__global__ __launch_bounds__(T) void conv_valu_kernel(ValuArgs a) {
  extern __shared__ float wl[];
  const int tid = threadIdx.x;
  const int g = int(blockIdx.y) / a.ncob;
  const int co0 = (int(blockIdx.y) - g * a.ncob) * CO;  // first channel of the block within the group
  const int khw = a.K1 * a.K2;
  const int kvol = a.K0 * khw;
  const int64_t plane_in = int64_t(a.L0) * a.L1 * a.L2;
  const int64_t plane_out = int64_t(a.O0) * a.O1 * a.O2;
  // Element strides of x: between input channels and between sites (W steps).
  const int64_t cstride = CL ? 1 : plane_in;
  const int site = CL ? a.Cin : 1;
  const int wstep = a.D2 * site;  // between a row's taps

  // This lane's positions: sample, window origin and input base (clamped into
  // range for invalid lanes; their stores are skipped).
  int id0[PP], ih0[PP], iw0[PP];
  int64_t sp[PP], nn[PP];
  bool valid[PP];
  const float* xb[PP];
#pragma unroll
  for (int pp = 0; pp < PP; pp++) {
    const int p0 = int(blockIdx.x) * (T * PP) + pp * T + tid;
    valid[pp] = p0 < a.npos;
    const int p = valid[pp] ? p0 : a.npos - 1;
    const int ow = p % a.O2;
    const int r1 = p / a.O2;
    const int oh = r1 % a.O1;
    const int r2 = r1 / a.O1;
    const int od = r2 % a.O0;
    const int n = r2 / a.O0;
    id0[pp] = od * a.S0 - a.P0;
    ih0[pp] = oh * a.S1 - a.P1;
    iw0[pp] = ow * a.S2 - a.P2;
    sp[pp] = (int64_t(od) * a.O1 + oh) * a.O2 + ow;
    nn[pp] = n;
    xb[pp] = a.x + int64_t(n) * a.Cin * plane_in + int64_t(g) * a.Cg * cstride;
  }

  float acc[PP][CO];
#pragma unroll
  for (int pp = 0; pp < PP; pp++)
#pragma unroll
    for (int j = 0; j < CO; j++) acc[pp][j] = 0.0f;

  const int npairs = a.Cg * a.K0;
  const int psz = khw * CO;  // floats per staged pair
  const float* wgrp = a.w + int64_t(g) * a.Coutg * a.Cg * kvol;
  int stage = 0;
  for (int pair0 = 0; pair0 < npairs; pair0 += a.pps, stage++) {
    const int np = min(a.pps, npairs - pair0);
    float* wb = wl + (stage & 1) * (a.pps * psz);
    // Pairs run in w's (c, td) order, so a stage is the contiguous run
    // [pair0 * khw, (pair0 + np) * khw) of every output channel's weights.
    for (int i = tid; i < np * psz; i += T) {
      const int t = i / CO, j = i - t * CO;
      const int co = co0 + j;
      wb[i] = co < a.Coutg ? wgrp[int64_t(co) * a.Cg * kvol + int64_t(pair0) * khw + t] : 0.0f;
    }
    __syncthreads();
    for (int pr = 0; pr < np; pr++) {
      const int c = (pair0 + pr) / a.K0, td = (pair0 + pr) - c * a.K0;
      const float* wpair = wb + pr * psz;
      for (int th = 0; th < a.K1; th++) {
        const float* xrow[PP];
        bool rowok[PP];
#pragma unroll
        for (int pp = 0; pp < PP; pp++) {
          const int zd = id0[pp] + td * a.D0, zh = ih0[pp] + th * a.D1;
          rowok[pp] = zd >= 0 && zd < a.L0 && zh >= 0 && zh < a.L1;
          // The row's first tap; dereferenced only where the tap is in range.
          xrow[pp] = xb[pp] + int64_t(c) * cstride + ((int64_t(zd) * a.L1 + zh) * a.L2 + iw0[pp]) * int64_t(site);
        }
        const v4f* wr0 = reinterpret_cast<const v4f*>(wpair + th * a.K2 * CO);
        // Out-of-range taps load the plane's first element (always in range)
        // and use 0: no branch around the loads, so unrolled taps issue their
        // loads together.
#pragma unroll 4
        for (int tw = 0; tw < a.K2; tw++) {
          float xv[PP];
#pragma unroll
          for (int pp = 0; pp < PP; pp++) {
            const int zw = iw0[pp] + tw * a.D2;
            const bool ok = rowok[pp] && zw >= 0 && zw < a.L2;
            const float v = *(ok ? xrow[pp] + tw * wstep : xb[pp]);
            xv[pp] = ok ? v : 0.0f;
          }
          fma_tap<CO, PP>(acc, xv, wr0 + tw * (CO / 4));
        }
      }
    }
  }

#pragma unroll
  for (int j = 0; j < CO; j++) {
    const int co = co0 + j;
    if (co >= a.Coutg) break;
    const int cg = g * a.Coutg + co;
    const float b = a.bias ? a.bias[cg] : 0.0f;
#pragma unroll
    for (int pp = 0; pp < PP; pp++)
      if (valid[pp]) {
        const int64_t yi = CL ? (nn[pp] * plane_out + sp[pp]) * a.Cout + cg : (nn[pp] * a.Cout + cg) * plane_out + sp[pp];
        a.y[yi] = acc[pp][j] + b;
      }
  }
}

// Floats of staged pairs per LDS buffer for 256-lane workgroups (a quarter for
// single-wave ones; at least one pair), and the LDS cap.
constexpr int kStageFloats = 4096;
constexpr int kMaxLdsBytes = 64 * 1024;

}  // namespace

int plan_valu(const Geom& g, ValuPlan* p) {
  const int co = g.Coutg <= 8 ? 8 : 16;
  const int64_t psz = g.K[1] * g.K[2] * co;
  if (2 * psz * 4 > kMaxLdsBytes) return CONV_ERR_UNSUPPORTED;
  const int64_t npos = g.N * g.O[0] * g.O[1] * g.O[2];
  if (npos >= (int64_t(1) << 30)) return CONV_ERR_OVERFLOW;
  for (int i = 0; i < 3; i++)
    if (g.L[i] >= (int64_t(1) << 30) || g.O[i] >= (int64_t(1) << 30)) return CONV_ERR_OVERFLOW;
  const int64_t npairs = g.Cg * g.K[0];
  if (g.Cin >= (int64_t(1) << 30) || g.Cout >= (int64_t(1) << 30) || npairs >= (int64_t(1) << 30))
    return CONV_ERR_OVERFLOW;
  // The kernel steps along a row's taps in 32-bit element offsets.
  if (g.K[2] * g.Dl[2] * (g.cl ? g.Cin : 1) >= (int64_t(1) << 31)) return CONV_ERR_OVERFLOW;
  p->co = co;
  p->ncob = int((g.Coutg + co - 1) / co);
  // 256 lanes x 2 positions per workgroup where that still gives 4 workgroups
  // per compute unit, else single-wave workgroups of 64 positions (and a
  // smaller weight stage, so that LDS does not limit their occupancy).
  const bool big = (npos + 511) / 512 * g.G * p->ncob >= 1024;
  p->threads = big ? 256 : 64;
  p->pp = big ? 2 : 1;
  p->pps = int(std::max<int64_t>(1, std::min<int64_t>(npairs, (big ? kStageFloats : kStageFloats / 4) / psz)));
  const int64_t per = int64_t(p->threads) * p->pp;
  p->grid[0] = (npos + per - 1) / per;
  p->grid[1] = g.G * p->ncob;
  if (p->grid[1] > 65535) return CONV_ERR_UNSUPPORTED;
  p->lds_bytes = int(2 * p->pps * psz * 4);
  return CONV_OK;
}

int launch_valu(const Geom& g, const ValuPlan& p, const float* x, const float* w, const float* bias, float* y,
                void* stream) {
  ValuArgs a;
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.y = y;
  a.Cin = int(g.Cin);
  a.Cg = int(g.Cg);
  a.Cout = int(g.Cout);
  a.Coutg = int(g.Coutg);
  a.L0 = int(g.L[0]), a.L1 = int(g.L[1]), a.L2 = int(g.L[2]);
  a.K0 = int(g.K[0]), a.K1 = int(g.K[1]), a.K2 = int(g.K[2]);
  a.S0 = int(g.S[0]), a.S1 = int(g.S[1]), a.S2 = int(g.S[2]);
  a.D0 = int(g.Dl[0]), a.D1 = int(g.Dl[1]), a.D2 = int(g.Dl[2]);
  a.P0 = int(g.P[0]), a.P1 = int(g.P[1]), a.P2 = int(g.P[2]);
  a.O0 = int(g.O[0]), a.O1 = int(g.O[1]), a.O2 = int(g.O[2]);
  a.npos = int(g.N * g.O[0] * g.O[1] * g.O[2]);
  a.ncob = p.ncob;
  a.pps = p.pps;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(p.grid[0]), unsigned(p.grid[1]));
#define CONVHIP_VALU_CASE(CO, PP, T, CL)                                                     \
  if (p.co == CO && p.pp == PP && p.threads == T && g.cl == CL) {                            \
    hipLaunchKernelGGL((conv_valu_kernel<CO, PP, T, CL>), grid, dim3(T), p.lds_bytes, s, a); \
    return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;                         \
  }
  CONVHIP_VALU_CASE(8, 2, 256, false)
  CONVHIP_VALU_CASE(16, 2, 256, false)
  CONVHIP_VALU_CASE(8, 1, 64, false)
  CONVHIP_VALU_CASE(16, 1, 64, false)
  CONVHIP_VALU_CASE(8, 2, 256, true)
  CONVHIP_VALU_CASE(16, 2, 256, true)
  CONVHIP_VALU_CASE(8, 1, 64, true)
  CONVHIP_VALU_CASE(16, 1, 64, true)
#undef CONVHIP_VALU_CASE
  return CONV_ERR_UNSUPPORTED;
}

}  // namespace convhip
