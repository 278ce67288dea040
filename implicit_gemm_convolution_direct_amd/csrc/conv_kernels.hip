// fp32 convolution kernels for gfx950 (MI355X) and the C-ABI entry points.
//
// Every conv kernel here is an implicit GEMM  Y[m][n] = sum_k W[m][k] * Xhat[k][n]
// with m = output channel, n = output position and k = (input channel, kernel
// tap). Xhat is never formed: the input halo box is copied into LDS once (by the
// LDS DMA path, global_load_lds) and each matrix-core B operand is read from it
// at (position offset + tap offset), so one LDS copy of every input element
// serves all taps and all output channels. Products run on the fp32 matrix
// cores (fp32 in, fp32 accumulate).
//
// conv_mfma16       any geometry: tile of BM channels x BN positions per
//                   workgroup, chunks of input channels double-buffered, tap
//                   offsets from an LDS table; v_mfma_f32_16x16x4_f32.
// conv_tap          build-time specialised geometries (every tap offset an
//                   immediate), persistent grid, weights resident in LDS.
// conv_tap_split    build-time specialised, few output channels per group: one
//                   wave per input channel of the group, partial tiles summed in
//                   LDS; the whole (n, od) output plane per workgroup.
// conv_tap_split_pipe  the same split for planes of 8+ tiles, with per-wave
//                   weights staged one depth tap at a time and held in VGPRs,
//                   and the first tile batch's sum overlapped with the second
//                   batch's products.
// conv_tap_kstream  build-time specialised, few output channels per group: one
//                   workgroup per (n, od) plane and group, whole tiles per
//                   compute wave plus the remainder tiles split over the
//                   waves by reduction blocks (stream-K inside the
//                   workgroup), copy waves issuing every LDS DMA copy.
// conv_direct16     small convolutions: one wave per 16 positions, operands
//                   read from global memory straight into registers.
// fused_stream      Conv3d -> min over depth -> softmax over channels for a
//                   build-time geometry: depth planes streamed through a 4-slot
//                   LDS ring, 4x4x1 MFMA with the weight operand broadcast.
// fused_min_softmax_mfma4  the same fused op for any geometry, min axis and
//                   number of groups.
//
// Problem statements: POPCORNBENCH "Kimi-K2.6" pages l1_p60 (Conv3d), l1_p76
// (Conv1d), l2_p24 (Conv3d + min + softmax), opening turns. The tiled direct
// convolution with the input halo staged on chip and the weights cached next
// to it follows the design monologue of l1_p60; the depth-streamed fused op
// with its running minimum, turns 2 and 7 of l2_p24.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <utility>

#include "../../include/convhip.h"
#include "convhip_plan.h"

namespace convhip {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const float GlobalF;  // a float in global memory
typedef float v16f __attribute__((ext_vector_type(16)));

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>): loops whose
// index must be a compile-time constant (immediate offsets, register indices).
template <int N, class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

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
  int mode, Cc, kc_pad, kdspan, rows, bw, boxc;
  int xs_floats, koff_ints, ws_floats;
  int row_tiles, ctiles, tiles_per_plane;
  int plane_out;
  int nchunks;
  int items;  // persistent kernel: (tile, plane) work items
  int ccp;        // channels-last box: LDS floats per (plane, row, column) site
  int cl_vec;     // channels-last box copied in 16-byte channel quads (ccp, Cc, C_in/groups multiples of 4)
  int vec_store;  // channels-last output: 4 consecutive channels stored as one 16-byte write
  int spin_cap;   // conv_tap_split_pipe: polls of the batch-1 counter before a wave gives up
};

// q = n / d and r = n % d for 0 <= n < 2^24, d >= 1, from a float reciprocal
// with one correction step (the product is within one of the true quotient).
__device__ __forceinline__ int divmod_small(int n, int d, float inv, int& r) {
  int q = int(float(n) * inv);
  r = n - q * d;
  if (r < 0) { q -= 1; r += d; }
  if (r >= d) { q += 1; r -= d; }
  return q;
}

// Minimum that propagates NaN, as torch.min does (IEEE 754-2019 minimum: one
// v_minimum / v_minimum3 instruction on gfx950; the C library's fmin would
// drop the NaN).
__device__ __forceinline__ float min_nan(float a, float b) { return __builtin_elementwise_minimum(a, b); }

template <int MT>
struct AFrag;
template <>
struct AFrag<1> {
  float v[1];
  __device__ __forceinline__ void load(const float* __restrict__ p) { v[0] = p[0]; }
};
template <>
struct AFrag<2> {
  float v[2];
  __device__ __forceinline__ void load(const float* __restrict__ p) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x; v[1] = t.y;
  }
};
template <>
struct AFrag<3> {
  float v[3];
  __device__ __forceinline__ void load(const float* __restrict__ p) { v[0] = p[0]; v[1] = p[1]; v[2] = p[2]; }
};
template <>
struct AFrag<4> {
  float v[4];
  __device__ __forceinline__ void load(const float* __restrict__ p) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
};

// A zero word in device memory: global->LDS copies of padding elements read it.
__device__ __align__(16) const float kZeroWord[4] = {0.0f, 0.0f, 0.0f, 0.0f};

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima), emitted through the
// builtin so the compiler's own wait-count tracking sees it.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Asynchronous copy of one float per lane from global memory into LDS: lane l
// of the wave writes dst[l] (dst is the same for the whole wave).
__device__ __forceinline__ void lds_dma_f32(const float* src, float* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

// s_waitcnt vmcnt(V) with expcnt and lgkmcnt left at their maxima (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int V>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(V >= 0 && V < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Keeps a wave-uniform value in scalar registers from here on: the compiler may
// not re-read it from the kernel-argument segment later (such a scalar load
// inside a loop costs a wait that also drains the LDS reads in flight).
__device__ __forceinline__ void pin_sgpr(int& v) {
  v = __builtin_amdgcn_readfirstlane(v);
  asm volatile("" : "+s"(v));
}
__device__ __forceinline__ void pin_sgpr(int64_t& v) {
  int lo = int(uint64_t(v)), hi = int(uint64_t(v) >> 32);
  pin_sgpr(lo);
  pin_sgpr(hi);
  v = int64_t((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo));
}
template <class T>
__device__ __forceinline__ void pin_sgpr(T*& p) {
  int64_t v = int64_t(reinterpret_cast<uintptr_t>(p));
  pin_sgpr(v);
  p = reinterpret_cast<T*>(uintptr_t(v));
}

// Asynchronous 16-byte copy per lane: lane l writes dst[4l .. 4l+3].
__device__ __forceinline__ void lds_dma_f32x4(const float* src, float* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}


// Geometry of one output tile: BN positions of the (n, od) plane, BM channels
// of group g starting at m0.
struct TileGeo {
  int n, od, g, m0;
  int oh_first, ow0, p0, iwb;
  int id0, ih0, iw0;
  int rows_ld;  // input rows per plane in the staged box
};

__device__ __forceinline__ TileGeo tile_geo(const ConvArgs& a, int tile, int plane, int gz, int BM, int BN,
                                            bool fixed_rows) {
  TileGeo t;
  t.n = plane / a.O0;
  t.od = plane - t.n * a.O0;
  t.g = gz / a.ctiles;
  t.m0 = (gz - t.g * a.ctiles) * BM;
  int oh_last;
  if (a.mode == TILE_FLAT) {
    t.p0 = tile * BN;
    t.ow0 = 0;
    const int p_last = min(t.p0 + BN, a.plane_out) - 1;
    t.oh_first = t.p0 / a.O2;
    oh_last = p_last / a.O2;
  } else {
    t.p0 = 0;
    t.oh_first = oh_last = tile / a.row_tiles;
    t.ow0 = (tile - t.oh_first * a.row_tiles) * BN;
  }
  t.iwb = t.ow0 * a.S2;  // box column 0 is input column iwb - P2
  t.id0 = t.od * a.S0 - a.P0;
  t.ih0 = t.oh_first * a.S1 - a.P1;
  t.iw0 = t.iwb - a.P2;
  t.rows_ld = fixed_rows ? a.rows : (oh_last - t.oh_first) * a.S1 + (a.K1 - 1) * a.D1 + 1;
  return t;
}

// Offset of every (channel, tap) of a chunk inside a box with rows_ld rows per
// plane. Padding taps (k >= Cc*kvol) carry zero weights and point at the box
// start, a staged finite element; entries past kc_pad serve the prefetch.
// Channels-last boxes (CL) hold the channels of a site contiguously, so a tap
// moves by whole sites of ccp floats and a channel by one float.
template <bool CL = false>
__device__ __forceinline__ void build_koff(const ConvArgs& a, int rows_ld, int* koff, int tid) {
  const int plane_stride = rows_ld * a.bw;
  const int boxc_t = a.kdspan * plane_stride;
  for (int k = tid; k < a.koff_ints; k += 256) {
    int off = 0;
    if (k < a.Cc * a.kvol) {
      const int c = k / a.kvol;
      const int r = k - c * a.kvol;
      const int td = r / (a.K1 * a.K2);
      const int r2 = r - td * a.K1 * a.K2;
      const int th = r2 / a.K2;
      const int tw = r2 - th * a.K2;
      const int site = td * a.D0 * plane_stride + th * a.D1 * a.bw + tw * a.D2;
      off = CL ? c + site * a.ccp : c * boxc_t + site;
    }
    koff[k] = off;
  }
}

// Copy the box of channels [c0, c0+Cc) of a tile into dst, dense layout
// [c][zd][zr < rows_ld][col]. Rows are spread over the waves; a row's channel,
// plane and input row are wave-uniform (scalar arithmetic) and its lanes copy
// consecutive columns, so each copy instruction moves up to 64 contiguous
// floats. Slots whose source lies outside the input (zero padding, channels
// past C_in/groups) read the zero word.
template <int NWAVES = 4>
__device__ __forceinline__ void stage_box(const ConvArgs& a, const TileGeo& t, int c0, float* dst, int wave,
                                          int lane) {
  const int cc_count = min(a.Cc, a.Cg - c0);
  const int rows_total = a.Cc * a.kdspan * t.rows_ld;
  const int64_t x_c0 = (int64_t(t.n) * a.Cin + int64_t(t.g) * a.Cg + c0) * a.L0;
  // (c, zd, zr) of row r = wave, advanced by NWAVES rows per iteration.
  int c = 0, zd = 0, zr = wave;
  while (zr >= t.rows_ld) { zr -= t.rows_ld; zd++; }
  while (zd >= a.kdspan) { zd -= a.kdspan; c++; }
  for (int r = wave; r < rows_total; r += NWAVES) {
    const int id = t.id0 + zd, ih = t.ih0 + zr;
    const bool row_ok = (c < cc_count) && (unsigned(id) < unsigned(a.L0)) && (unsigned(ih) < unsigned(a.L1));
    const float* srow = a.x + ((x_c0 + int64_t(c) * a.L0 + (row_ok ? id : 0)) * a.L1 + (row_ok ? ih : 0)) * a.L2;
    float* drow = dst + r * a.bw;
    for (int j = 0; j < a.bw; j += 64) {
      const int col = j + lane;
      if (col < a.bw) {
        const int iw = t.iw0 + col;
        const bool ok = row_ok && (unsigned(iw) < unsigned(a.L2));
        lds_dma_f32(ok ? srow + iw : kZeroWord, drow + j);
      }
    }
    zr += NWAVES;
    while (zr >= t.rows_ld) { zr -= t.rows_ld; zd++; }
    while (zd >= a.kdspan) { zd -= a.kdspan; c++; }
  }
}

// Channels-last input x [N, D, H, W, C_in]: copy the box of channels [c0, c0+Cc)
// of a tile into dst, layout [zd][zr < rows_ld][col][c < ccp]. The LDS slots are
// walked in order, 64 per copy instruction, so consecutive lanes read the
// consecutive channels of a site and then the next site along W: runs of Cc
// contiguous input floats. Slots outside the input (zero padding, channels past
// the chunk, the pitch padding c >= Cc) read the zero word.
template <int NWAVES = 4>
__device__ __forceinline__ void stage_box_cl(const ConvArgs& a, const TileGeo& t, int c0, float* dst, int wave,
                                             int lane) {
  const int cc_count = min(a.Cc, a.Cg - c0);
  const float inv_bw = 1.0f / float(a.bw);
  const float inv_rows = 1.0f / float(t.rows_ld);
  const float* xn = a.x + int64_t(t.n) * a.L0 * a.L1 * a.L2 * a.Cin + (int64_t(t.g) * a.Cg + c0);
  if (a.cl_vec) {
    // 16-byte units: a site holds ccp/4 channel quads, 64 quads per copy instruction.
    const int q = a.ccp >> 2, q_valid = cc_count >> 2;
    const float inv_q = 1.0f / float(q);
    const int total4 = a.kdspan * t.rows_ld * a.bw * q;
    for (int r = wave; r * 64 < total4; r += NWAVES) {
      const int s = r * 64 + lane;
      if (s < total4) {
        int cq, col, zr;
        const int site = divmod_small(s, q, inv_q, cq);
        const int zz = divmod_small(site, a.bw, inv_bw, col);
        const int zd = divmod_small(zz, t.rows_ld, inv_rows, zr);
        const int id = t.id0 + zd, ih = t.ih0 + zr, iw = t.iw0 + col;
        const bool ok = (cq < q_valid) && (unsigned(id) < unsigned(a.L0)) && (unsigned(ih) < unsigned(a.L1)) &&
                        (unsigned(iw) < unsigned(a.L2));
        const float* src = ok ? xn + ((int64_t(id) * a.L1 + ih) * a.L2 + iw) * a.Cin + 4 * cq : kZeroWord;
        lds_dma_f32x4(src, dst + r * 256);
      }
    }
    return;
  }
  const int total = a.kdspan * t.rows_ld * a.bw * a.ccp;
  const float inv_ccp = 1.0f / float(a.ccp);
  for (int r = wave; r * 64 < total; r += NWAVES) {
    const int s = r * 64 + lane;
    if (s < total) {
      int c, col, zr;
      const int site = divmod_small(s, a.ccp, inv_ccp, c);
      const int zz = divmod_small(site, a.bw, inv_bw, col);
      const int zd = divmod_small(zz, t.rows_ld, inv_rows, zr);
      const int id = t.id0 + zd, ih = t.ih0 + zr, iw = t.iw0 + col;
      const bool ok = (c < cc_count) && (unsigned(id) < unsigned(a.L0)) && (unsigned(ih) < unsigned(a.L1)) &&
                      (unsigned(iw) < unsigned(a.L2));
      const float* src = ok ? xn + ((int64_t(id) * a.L1 + ih) * a.L2 + iw) * a.Cin + c : kZeroWord;
      lds_dma_f32(src, dst + r * 64);
    }
  }
}

// Copy the weight fragments of channels [c0, c0+Cc) (k-steps 0..nsteps-1 of a
// chunk) into dst, in the order the matrix core consumes them: for k-step s and
// wave row wm, lane l holds W[m = wm*16*MT + 16*mi + (l%16)][k = 4s + l/16] for
// mi = 0..MT-1 contiguously, so one vector LDS read delivers a lane's A operands.
// TAPMAJOR: the chunk's reduction index runs k = tap * Cc + c (channels-last
// specialisations) instead of k = c * kvol + tap.
template <int MT, int WM, int NWAVES = 4, bool TAPMAJOR = false>
__device__ __forceinline__ void stage_wfrag(const ConvArgs& a, int g, int m0, int c0, int nsteps, float* dst,
                                            int wave, int lane) {
  const int cc_count = min(a.Cc, a.Cg - c0);
  const int kvalid = cc_count * a.kvol;
  const int64_t w_g = int64_t(g * a.Coutg + m0) * a.kfull + int64_t(c0) * a.kvol;
  const int w_waves = (nsteps * WM * 64 * MT) >> 6;
  for (int wi = wave; wi < w_waves; wi += NWAVES) {
    const int f = wi * 64 + lane;
    const int mi = f % MT;
    const int q = f / MT;  // (s*WM + fwm)*64 + fl
    const int fl = q & 63;
    const int sw = q >> 6;
    const int s = sw / WM;
    const int fwm = sw - s * WM;
    const int k = 4 * s + (fl >> 4);
    const int m = fwm * 16 * MT + 16 * mi + (fl & 15);
    const bool ok = (k < kvalid) && (m0 + m < a.Coutg);
    const int kw = TAPMAJOR ? (k % a.Cc) * a.kvol + k / a.Cc : k;
    const float* src = ok ? a.w + (w_g + int64_t(m) * a.kfull + kw) : kZeroWord;
    lds_dma_f32(src, dst + wi * 64);
  }
}

// Row and column of flattened plane positions p, p + 16, p + 32, ... in a plane
// `width` wide: one division for the first, then steps of 16 = q16 rows plus
// r16 columns (r16 < width, so a step wraps at most once). This replaces a
// division per tile, which sat on the path to the first product.
struct PosStep {
  int oh, ow, q16, r16, width;
  __device__ __forceinline__ PosStep(int p, int w) : width(w) {
    oh = p / w;
    ow = p - oh * w;
    q16 = 16 / w;
    r16 = 16 - q16 * w;
  }
  __device__ __forceinline__ void next() {
    ow += r16;
    oh += q16;
    const bool wrap = ow >= width;
    ow -= wrap ? width : 0;
    oh += wrap ? 1 : 0;
  }
};

// Box offsets base + (p / width) * row + (p % width) * col of positions p,
// p + 16, p + 32, ..., stepped by additions only.
struct OffStep {
  int ow, off, r16, width, d16, dwrap;
  __device__ __forceinline__ OffStep(int p, int w, int base, int row, int col) : width(w) {
    const int oh = p / w;
    ow = p - oh * w;
    off = base + oh * row + ow * col;
    const int q16 = 16 / w;
    r16 = 16 - q16 * w;
    d16 = q16 * row + r16 * col;
    dwrap = row - w * col;
  }
  __device__ __forceinline__ void next() {
    ow += r16;
    off += d16;
    const bool wrap = ow >= width;
    ow -= wrap ? width : 0;
    off += wrap ? dwrap : 0;
  }
};

// Per-lane output positions of a wave's NT sub-tiles: LDS offset inside the box
// (row stride bw) and flattened index in the (n, co, od) output plane (-1: none).
template <int NT, bool CL = false>
__device__ __forceinline__ void tile_positions(const ConvArgs& a, const TileGeo& t, int wn, int li, int noff[NT],
                                               int pidx[NT]) {
  PosStep ps(t.p0 + wn * (16 * NT) + li, a.O2);
#pragma unroll
  for (int ni = 0; ni < NT; ni++) {
    const int q = wn * (16 * NT) + 16 * ni + li;
    int oh, ow, valid;
    if (a.mode == TILE_FLAT) {
      valid = t.p0 + q < a.plane_out;
      oh = ps.oh;
      ow = ps.ow;
      ps.next();
    } else {
      oh = t.oh_first;
      ow = t.ow0 + q;
      valid = ow < a.O2;
    }
    const int site = (oh - t.oh_first) * a.S1 * a.bw + ow * a.S2 - t.iwb;
    noff[ni] = valid ? (CL ? site * a.ccp : site) : 0;
    pidx[ni] = valid ? oh * a.O2 + ow : -1;
  }
}

// Reduction of one staged chunk: this wave takes k-steps ks, ks+KS, ... < nsteps,
// software-pipelined (tap offsets two steps ahead, operands one step ahead of
// the matrix-core instructions that use them).
template <int MT, int NT, int WM, int KS>
__device__ __forceinline__ void mma_chunk(const float* __restrict__ Xs, const float* __restrict__ Ws,
                                          const int* __restrict__ koff, int nsteps, int ks, int wfrag_base,
                                          const int (&noff)[NT], v4f (&acc)[MT][NT], int kg) {
  constexpr int SSTRIDE = WM * 64 * MT;
  int s = ks;
  int ko_next = koff[4 * (s + KS) + kg];
  AFrag<MT> af;
  float bv[NT];
  {
    const int ko = koff[4 * s + kg];
    af.load(Ws + s * SSTRIDE + wfrag_base);
#pragma unroll
    for (int ni = 0; ni < NT; ni++) bv[ni] = Xs[ko + noff[ni]];
  }
  for (; s < nsteps; s += KS) {
    AFrag<MT> af_n;
    float bv_n[NT];
    const int ko = ko_next;
    ko_next = koff[4 * (s + 2 * KS) + kg];
    af_n.load(Ws + (s + KS) * SSTRIDE + wfrag_base);
#pragma unroll
    for (int ni = 0; ni < NT; ni++) bv_n[ni] = Xs[ko + noff[ni]];
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
      for (int ni = 0; ni < NT; ni++)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(af.v[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    af = af_n;
#pragma unroll
    for (int ni = 0; ni < NT; ni++) bv[ni] = bv_n[ni];
  }
}

// Bias of the channels this lane stores: register r of sub-tile mi holds channel
// m0 + wm*16*MT + 16*mi + 4*kg + r. Loaded once, so no global load sits between
// the output stores.
template <int MT>
__device__ __forceinline__ void load_bias(const ConvArgs& a, const TileGeo& t, int wm, int kg, float (&bias)[MT][4]) {
#pragma unroll
  for (int mi = 0; mi < MT; mi++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int ch = t.m0 + wm * 16 * MT + 16 * mi + 4 * kg + r;
      bias[mi][r] = (a.bias && ch < a.Coutg) ? a.bias[t.g * a.Coutg + ch] : 0.0f;
    }
}

// Non-temporal output stores, for the channels-last tap kernel when it reads
// each input site's channels in several chunks, one after the other: the
// output it writes meanwhile (as large as the input for the long Conv1d) would
// otherwise push those sites' lines out of L2 before the later chunks read
// them. Elsewhere outputs keep plain stores: non-temporal ones add write
// traffic (partly written lines reach HBM separately), measured at 1.26x to
// 1.42x of the output size.
__device__ __forceinline__ void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt4(float* p, v4f v) { __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p)); }

// Store a wave tile (+ bias). D[m][n] of the matrix core sits in lane
// n + 16*(m/4), register m%4: a lane holds 4 consecutive channels of one
// position, which channels-last output y [N, D_out, H_out, W_out, C_out] takes
// as one 16-byte store.
template <int MT, int NT, bool CL = false, bool NTSTORE = false>
__device__ __forceinline__ void store_tile(const ConvArgs& a, const TileGeo& t, int wm, int kg,
                                           const int (&pidx)[NT], const v4f (&acc)[MT][NT],
                                           const float (&bias)[MT][4]) {
  const int64_t out_plane = int64_t(a.O1) * a.O2;
  if constexpr (CL) {
    float* yplane = a.y + (int64_t(t.n) * a.O0 + t.od) * out_plane * a.Cout + int64_t(t.g) * a.Coutg;
#pragma unroll
    for (int mi = 0; mi < MT; mi++) {
      const int ch0 = t.m0 + wm * 16 * MT + 16 * mi + 4 * kg;
#pragma unroll
      for (int ni = 0; ni < NT; ni++) {
        if (pidx[ni] < 0 || ch0 >= a.Coutg) continue;
        float* yp = yplane + int64_t(pidx[ni]) * a.Cout + ch0;
        if (a.vec_store) {
          const v4f v = v4f{acc[mi][ni][0] + bias[mi][0], acc[mi][ni][1] + bias[mi][1], acc[mi][ni][2] + bias[mi][2],
                            acc[mi][ni][3] + bias[mi][3]};
          if constexpr (NTSTORE) store_nt4(yp, v);
          else *reinterpret_cast<v4f*>(yp) = v;
        } else {
#pragma unroll
          for (int r = 0; r < 4; r++) {
            if (ch0 + r >= a.Coutg) continue;
            if constexpr (NTSTORE) store_nt(yp + r, acc[mi][ni][r] + bias[mi][r]);
            else yp[r] = acc[mi][ni][r] + bias[mi][r];
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < MT; mi++) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int ch = t.m0 + wm * 16 * MT + 16 * mi + 4 * kg + r;
      if (ch < a.Coutg) {
        const int co = t.g * a.Coutg + ch;
        float* yp = a.y + ((int64_t(t.n) * a.Cout + co) * a.O0 + t.od) * out_plane;
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
          if (pidx[ni] >= 0) yp[pidx[ni]] = acc[mi][ni][r] + bias[mi][r];
      }
    }
  }
}

// One pipeline stage of the streamed kernel: start the copies of the next chunk
// into `nxt`, then reduce the chunk in `cur`. The buffers are distinct; the
// restrict qualifiers let the compiler keep the copies in flight across the
// reduction instead of waiting for them before every LDS read.
template <int MT, int NT, int WM, int KS, bool CL>
__device__ __forceinline__ void stream_stage(const ConvArgs& a, const TileGeo& t, bool has_next, int c0_next,
                                             const float* __restrict__ cur, float* __restrict__ nxt,
                                             const int* __restrict__ koff, int nsteps, int ks, int wfrag_base,
                                             const int (&noff)[NT], v4f (&acc)[MT][NT], int kg, int wave, int lane) {
  if (has_next) {
    if constexpr (CL) stage_box_cl(a, t, c0_next, nxt, wave, lane);
    else stage_box(a, t, c0_next, nxt, wave, lane);
    stage_wfrag<MT, WM>(a, t.g, t.m0, c0_next, nsteps, nxt + a.xs_floats, wave, lane);
  }
  __builtin_amdgcn_sched_barrier(0);
  mma_chunk<MT, NT, WM, KS>(cur, cur + a.xs_floats, koff, nsteps, ks, wfrag_base, noff, acc, kg);
}

// ---------------------------------------------------------------------------
// conv_mfma16 (streamed): one tile per workgroup; chunks of input channels
// (box + weight fragments) are double-buffered in LDS.
// LDS (floats): [ koff | buffer 0 | buffer 1 ], buffer = [ box | weights ].
// ---------------------------------------------------------------------------
template <int MT, int NT, int WM, int WN, int KS, bool CL>
__global__ __launch_bounds__(256) void conv_mfma16_kernel(ConvArgs a) {
  constexpr int BM = 16 * MT * WM;
  constexpr int BN = 16 * NT * WN;
  extern __shared__ __align__(16) float smem[];
  int* koff = reinterpret_cast<int*>(smem);
  float* buf0 = smem + a.koff_ints;
  float* buf1 = buf0 + a.xs_floats + a.ws_floats;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = wave % KS;
  const int wt = wave / KS;
  const int wm = wt / WN;
  const int wn = wt - wm * WN;
  const int kg = lane >> 4;
  const int li = lane & 15;

  const TileGeo t = tile_geo(a, blockIdx.x, blockIdx.y, blockIdx.z, BM, BN, false);
  const int nsteps = a.kc_pad >> 2;
  build_koff<CL>(a, t.rows_ld, koff, tid);
  int noff[NT], pidx[NT];
  tile_positions<NT, CL>(a, t, wn, li, noff, pidx);
  v4f acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; mi++)
#pragma unroll
    for (int ni = 0; ni < NT; ni++) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};
  const int wfrag_base = wm * 64 * MT + lane * MT;
  float bias[MT][4];
  load_bias<MT>(a, t, wm, kg, bias);

  if constexpr (CL) stage_box_cl(a, t, 0, buf0, wave, lane);
  else stage_box(a, t, 0, buf0, wave, lane);
  stage_wfrag<MT, WM>(a, t.g, t.m0, 0, nsteps, buf0 + a.xs_floats, wave, lane);
  wait_vmem();
  __syncthreads();
  for (int ci = 0; ci < a.nchunks; ci++) {
    const bool has_next = ci + 1 < a.nchunks;
    if (ci & 1)
      stream_stage<MT, NT, WM, KS, CL>(a, t, has_next, (ci + 1) * a.Cc, buf1, buf0, koff, nsteps, ks, wfrag_base,
                                   noff, acc, kg, wave, lane);
    else
      stream_stage<MT, NT, WM, KS, CL>(a, t, has_next, (ci + 1) * a.Cc, buf0, buf1, koff, nsteps, ks, wfrag_base,
                                   noff, acc, kg, wave, lane);
    wait_vmem();       // this thread's copies of the next chunk have landed
    __syncthreads();   // everyone's copies have landed; everyone is done with the current buffer
  }

  if constexpr (KS > 1) {
    // Add the split-reduction partial sums through LDS (the buffers are free).
    constexpr int TILE_F = MT * NT * 4 * 64;
    float* red = buf0;
    if (ks > 0) {
      float* dstp = red + ((ks - 1) * (WM * WN) + wt) * TILE_F;
#pragma unroll
      for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
#pragma unroll
          for (int r = 0; r < 4; r++) dstp[((mi * NT + ni) * 4 + r) * 64 + lane] = acc[mi][ni][r];
    }
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int j = 1; j < KS; j++) {
      const float* srcp = red + ((j - 1) * (WM * WN) + wt) * TILE_F;
#pragma unroll
      for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
#pragma unroll
          for (int r = 0; r < 4; r++) acc[mi][ni][r] += srcp[((mi * NT + ni) * 4 + r) * 64 + lane];
    }
  }
  store_tile<MT, NT, CL>(a, t, wm, kg, pidx, acc, bias);
}

// ---------------------------------------------------------------------------
// conv_tap: the implicit GEMM specialised at build time for one geometry
// (channel chunk, kernel taps, dilations, strides, staged box shape, tiling).
// Every tap offset is a compile-time constant, so each matrix-core B operand is
// one LDS read at (per-lane register + immediate offset): the register holds the
// lane's output-position offset plus the lane's share of the 4-deep k-step, and
// the few distinct per-step lane patterns are precomputed once per tile.
// The kernel is persistent: each workgroup keeps the whole weight matrix in LDS
// and walks work items (tile, plane) blockIdx.x, blockIdx.x + gridDim.x, ...;
// chunks of the input box are double-buffered and copied by the DMA engine while
// the previous chunk is reduced.
// LDS (floats): [ box 0 | box 1 | weight fragments of all chunks (+1 step) ].
// ---------------------------------------------------------------------------
template <int KD, int KH, int KW, int DD, int DH, int DW, int CC, int KDSPAN, int ROWS, int BW>
struct TapGeo {
  static constexpr int CCH = CC;
  static constexpr int KVOL = KD * KH * KW;
  static constexpr int K = CC * KVOL;
  static constexpr int NS = (K + 3) / 4;  // 4-deep k-steps per chunk
  static constexpr int PLANE = ROWS * BW;
  static constexpr int BOXC = KDSPAN * PLANE;
  static constexpr int XS = (CC * BOXC + 255) / 256 * 256;  // floats per box buffer
  // Box rows a multiple of 4 floats long: copied in 16-byte chunks (the planner
  // checks the alignment of the rows' first input column).
  static constexpr bool ROWCOPY = BW % 4 == 0;
  static constexpr bool CL = false;       // channel-major box (NCDHW input)
  static constexpr bool TAPMAJOR = false; // reduction index k = c * KVOL + tap
  static constexpr int BW_ = BW, ROWS_ = ROWS, KDSPAN_ = KDSPAN;
  template <int NCH, int WM, int MT>
  static constexpr int lds_floats() { return 2 * XS + (NCH * NS + 1) * WM * 64 * MT; }
  // LDS offset (floats) of reduction index k = (channel, td, th, tw) of a chunk;
  // padding indices (zero weights) point at the box start.
  static constexpr int koff(int k) {
    if (k >= K) return 0;
    const int c = k / KVOL, r = k % KVOL, td = r / (KH * KW), r2 = r % (KH * KW), th = r2 / KW, tw = r2 % KW;
    return c * BOXC + td * DD * PLANE + th * DH * BW + tw * DW;
  }
};

// The same specialisation for channels-last input x [N, D, H, W, C_in]: the box
// holds CCP floats per (plane, row, column) site, channels innermost, and the
// reduction index runs tap-major, k = tap * CC + c (with CC a multiple of 4 each
// 4-deep k-step reads 4 consecutive channels of one tap). CC and CCP multiples
// of 4: the box is copied in 16-byte channel quads, else float by float.
template <int KD, int KH, int KW, int DD, int DH, int DW, int CC, int KDSPAN, int ROWS, int BW, int CCP>
struct TapGeoCL {
  static_assert(CCP >= CC, "site pitch");
  static constexpr bool QUADS = CC % 4 == 0 && CCP % 4 == 0;
  static constexpr int CCH = CC;
  static constexpr int KVOL = KD * KH * KW;
  static constexpr int K = CC * KVOL;
  static constexpr int NS = (K + 3) / 4;
  static constexpr int PLANE = ROWS * BW;     // sites per box plane
  static constexpr int BOXC = KDSPAN * PLANE; // sites in the box
  static constexpr int XS = (CCP * BOXC + 255) / 256 * 256;
  static constexpr bool ROWCOPY = false;
  static constexpr bool CL = true;
  static constexpr bool TAPMAJOR = true;
  static constexpr int CCP_ = CCP;
  static constexpr int BW_ = BW, ROWS_ = ROWS, KDSPAN_ = KDSPAN;
  template <int NCH, int WM, int MT>
  static constexpr int lds_floats() { return 2 * XS + (NCH * NS + 1) * WM * 64 * MT; }
  static constexpr int koff(int k) {
    if (k >= K) return 0;
    const int c = k % CC, tap = k / CC, td = tap / (KH * KW), r2 = tap % (KH * KW), th = r2 / KW, tw = r2 % KW;
    return c + (td * DD * PLANE + th * DH * BW + tw * DW) * CCP;
  }
};

// Distinct per-step lane patterns koff(4s + j) - koff(4s), j = 0..3.
template <class G>
struct TapPatterns {
  int np = 0;
  int pid[G::NS] = {};
  int pat[G::NS][4] = {};
  constexpr TapPatterns() {
    for (int s = 0; s < G::NS; s++) {
      int d[4] = {};
      for (int j = 0; j < 4; j++) d[j] = G::koff(4 * s + j) - G::koff(4 * s);
      int found = -1;
      for (int q = 0; q < np && found < 0; q++) {
        bool eq = true;
        for (int j = 0; j < 4; j++) eq = eq && pat[q][j] == d[j];
        if (eq) found = q;
      }
      if (found < 0) {
        for (int j = 0; j < 4; j++) pat[np][j] = d[j];
        found = np++;
      }
      pid[s] = found;
    }
  }
};

// Lane kg's share of distinct step pattern Q, from compile-time constants (no
// table in memory), computed from the two bits of kg (a chain of selects was
// compiled to exec-mask branches).
template <class G, int Q>
__device__ __forceinline__ int pat_delta(int kg) {
  constexpr TapPatterns<G> P{};
  constexpr int d0 = P.pat[Q][0], d1 = P.pat[Q][1], d2 = P.pat[Q][2], d3 = P.pat[Q][3];
  const int b0 = kg & 1, b1 = (kg >> 1) & 1;
  return d0 + b0 * (d1 - d0) + b1 * (d2 - d0) + (b0 & b1) * (d3 - d2 - d1 + d0);
}
template <class G, int... Q>
__device__ __forceinline__ void fill_pat_deltas(int* dp, int kg, std::integer_sequence<int, Q...>) {
  ((dp[Q] = pat_delta<G, Q>(kg)), ...);
}

// Box of one chunk as whole 16-byte chunks (ROWCOPY). The box is CC*KDSPAN*ROWS
// rows of BW floats, row (c, zd, zr) <- input row (c0 + c, id0 + zd, ih0 + zr),
// columns iw0 .. iw0 + BW - 1. The rows are contiguous in LDS, so copy i of wave
// w moves box chunks u = (i*NWAVES + w)*64 + lane as one contiguous 1 KB run.
// iw0, the input row length and the input pointer are multiples of 4 floats
// (the planner checks), so a chunk lies wholly inside or wholly outside a row.
template <class G, int NWAVES>
__device__ __forceinline__ void stage_rows16(const ConvArgs& a, const TileGeo& t, int c0, float* dst, int wave,
                                             int lane) {
  constexpr int Q = G::BW_ / 4;                                  // chunks per row
  constexpr int NROWS = G::CCH * G::KDSPAN_ * G::ROWS_;
  constexpr int NCHUNK = NROWS * Q;
  constexpr int NI = (NCHUNK + 64 * NWAVES - 1) / (64 * NWAVES);  // copies per wave
  const int64_t chan0 = int64_t(t.n) * a.Cin + int64_t(t.g) * a.Cg + c0;
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int u0 = (i * NWAVES + wave) * 64;
    const int u = u0 + lane;
    if (u < NCHUNK) {
      const int row = u / Q, q = u - row * Q;
      const int c = row / (G::KDSPAN_ * G::ROWS_), rr = row - c * (G::KDSPAN_ * G::ROWS_);
      const int zd = rr / G::ROWS_, zr = rr - zd * G::ROWS_;
      const int id = t.id0 + zd, ih = t.ih0 + zr, iw = t.iw0 + 4 * q;
      const bool ok = unsigned(id) < unsigned(a.L0) && unsigned(ih) < unsigned(a.L1) && unsigned(iw) < unsigned(a.L2);
      const float* src = a.x + (((chan0 + c) * a.L0 + id) * a.L1 + ih) * a.L2 + iw;
      lds_dma_f32x4(ok ? src : kZeroWord, dst + 4 * u0);
    }
  }
}

// Channels-last box of one chunk (TapGeoCL) as 16-byte channel quads: box quad u
// = (site, cq) <- channels c0 + 4cq .. c0 + 4cq + 3 of input site (id0 + zd,
// ih0 + zr, iw0 + col); quads past the chunk's channels and sites outside the
// input read the zero word. Copy i of wave w moves quads (i*NWAVES + w)*64 + lane.
// Float-by-float form (TapGeoCL without quads): box slot u = (site, c).
template <class G, int NWAVES>
__device__ __forceinline__ void stage_cl_floats(const ConvArgs& a, const TileGeo& t, int c0, float* dst, int wave,
                                                int lane) {
  constexpr int NU = G::BOXC * G::CCP_;
  constexpr int NI = (NU + 64 * NWAVES - 1) / (64 * NWAVES);
  const float* xn = a.x + int64_t(t.n) * a.L0 * a.L1 * a.L2 * a.Cin + (int64_t(t.g) * a.Cg + c0);
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int u0 = (i * NWAVES + wave) * 64;
    const int u = u0 + lane;
    if (u < NU) {
      const int site = u / G::CCP_, c = u - site * G::CCP_;
      const int zz = site / G::BW_, col = site - zz * G::BW_;
      const int zd = zz / G::ROWS_, zr = zz - zd * G::ROWS_;
      const int id = t.id0 + zd, ih = t.ih0 + zr, iw = t.iw0 + col;
      const bool ok = c < G::CCH && unsigned(id) < unsigned(a.L0) && unsigned(ih) < unsigned(a.L1) &&
                      unsigned(iw) < unsigned(a.L2);
      const float* src = xn + ((int64_t(id) * a.L1 + ih) * a.L2 + iw) * a.Cin + c;
      lds_dma_f32(ok ? src : kZeroWord, dst + u0);
    }
  }
}

template <class G, int NWAVES>
__device__ __forceinline__ void stage_cl_quads(const ConvArgs& a, const TileGeo& t, int c0, float* dst, int wave,
                                               int lane) {
  constexpr int Q = G::CCP_ / 4, QV = G::CCH / 4;
  constexpr int NQ = G::BOXC * Q;
  constexpr int NI = (NQ + 64 * NWAVES - 1) / (64 * NWAVES);
  const float* xn = a.x + int64_t(t.n) * a.L0 * a.L1 * a.L2 * a.Cin + (int64_t(t.g) * a.Cg + c0);
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int u0 = (i * NWAVES + wave) * 64;
    const int u = u0 + lane;
    if (u < NQ) {
      const int site = u / Q, cq = u - site * Q;
      const int zz = site / G::BW_, col = site - zz * G::BW_;
      const int zd = zz / G::ROWS_, zr = zz - zd * G::ROWS_;
      const int id = t.id0 + zd, ih = t.ih0 + zr, iw = t.iw0 + col;
      const bool ok = cq < QV && unsigned(id) < unsigned(a.L0) && unsigned(ih) < unsigned(a.L1) &&
                      unsigned(iw) < unsigned(a.L2);
      const float* src = xn + ((int64_t(id) * a.L1 + ih) * a.L2 + iw) * a.Cin + 4 * cq;
      lds_dma_f32x4(ok ? src : kZeroWord, dst + 4 * u0);
    }
  }
}

template <class G, int NWAVES>
__device__ __forceinline__ void stage_tap_box(const ConvArgs& a, const TileGeo& t, int c0, float* dst, int wave,
                                              int lane) {
  if constexpr (G::CL) {
    if constexpr (G::QUADS) stage_cl_quads<G, NWAVES>(a, t, c0, dst, wave, lane);
    else stage_cl_floats<G, NWAVES>(a, t, c0, dst, wave, lane);
  } else if constexpr (G::ROWCOPY) stage_rows16<G, NWAVES>(a, t, c0, dst, wave, lane);
  else stage_box<NWAVES>(a, t, c0, dst, wave, lane);
}

// Reduce one staged chunk: all k-steps unrolled, B operands read at
// (lane register + immediate), A operands from the resident weight fragments
// (wchunk already includes this lane's and wave row's offset).
template <int MT, int NT, int WM, class G, int NP>
__device__ __forceinline__ void tap_chunk(const float* __restrict__ box, const float* __restrict__ wchunk,
                                          const int (&addr)[NP][NT], v4f (&acc)[MT][NT]) {
  constexpr TapPatterns<G> P{};
  const char* bb = reinterpret_cast<const char*>(box);
  // Operands of step s+1 are read while the matrix core works on step s.
  AFrag<MT> af[2];
  float bv[2][NT];
  af[0].load(wchunk);
#pragma unroll
  for (int ni = 0; ni < NT; ni++) bv[0][ni] = *reinterpret_cast<const float*>(bb + addr[P.pid[0]][ni]);
#pragma unroll
  for (int s = 0; s < G::NS; s++) {
    const int cu = s & 1, nx = cu ^ 1;
    if (s + 1 < G::NS) {
      af[nx].load(wchunk + (s + 1) * (WM * 64 * MT));
#pragma unroll
      for (int ni = 0; ni < NT; ni++)
        bv[nx][ni] = *reinterpret_cast<const float*>(bb + addr[P.pid[s + 1]][ni] + 4 * G::koff(4 * (s + 1)));
    }
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
      for (int ni = 0; ni < NT; ni++)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[cu].v[mi], bv[cu][ni], acc[mi][ni], 0, 0, 0);
    // Interleave the next step's LDS reads with this step's matrix-core work.
#pragma unroll
    for (int i = 0; i < NT + 1; i++) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MT * NT / (NT + 1) > 0 ? MT * NT / (NT + 1) : 1, 0);
    }
  }
}

// One pipeline stage: start the copy of the next box into `nxt`, then reduce the
// box in `cur` (distinct buffers; see stream_stage).
template <int MT, int NT, int WM, int NWAVES, class G, int NP>
__device__ __forceinline__ void tap_stage(const ConvArgs& a, const TileGeo& tn, bool has_next, int c0_next,
                                          const float* __restrict__ cur, float* __restrict__ nxt,
                                          const float* __restrict__ wchunk, const int (&addr)[NP][NT],
                                          v4f (&acc)[MT][NT], int wave, int lane) {
  if (has_next) stage_tap_box<G, NWAVES>(a, tn, c0_next, nxt, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  tap_chunk<MT, NT, WM, G, NP>(cur, wchunk, addr, acc);
}

template <int MT, int NT, int WM, int WN, int NCH, class G>
__global__ __launch_bounds__(64 * WM * WN) void conv_tap_kernel(ConvArgs a) {
  constexpr int NWAVES = WM * WN;
  constexpr int BM = 16 * MT * WM;
  constexpr int BN = 16 * NT * WN;
  constexpr int SSTRIDE = WM * 64 * MT;  // floats per k-step of the weight fragments
  constexpr TapPatterns<G> P{};
  constexpr int NP = P.np;
  // Static LDS: its address is known when compiling, so box offsets fold into
  // the LDS read's immediate.
  __shared__ __align__(16) float smem[G::template lds_floats<NCH, WM, MT>()];
  float* box0 = smem;
  float* box1 = smem + G::XS;
  float* Wres = smem + 2 * G::XS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave - wm * WN;
  const int kg = lane >> 4;
  const int li = lane & 15;

  // Workgroups are dispatched round-robin over the 8 XCDs. Each XCD takes a
  // contiguous eighth of the items and its workgroups stride through it, so
  // the items in flight on one XCD are neighbours (the same tile of adjacent
  // output depths, adjacent tiles) whose input rows its L2 serves once.
  int item = blockIdx.x, item_step = gridDim.x, item_end = a.items;
  if ((gridDim.x & 7) == 0) {
    const int xcd = blockIdx.x & 7;
    item_step = gridDim.x >> 3;
    item = int(int64_t(a.items) * xcd / 8) + (blockIdx.x >> 3);
    item_end = int(int64_t(a.items) * (xcd + 1) / 8);
  }
  if (item >= item_end) return;
#pragma unroll
  for (int c = 0; c < NCH; c++)
    stage_wfrag<MT, WM, NWAVES, G::TAPMAJOR>(a, 0, 0, c * G::CCH, G::NS, Wres + c * G::NS * SSTRIDE, wave, lane);
  TileGeo t = tile_geo(a, item % a.tiles_per_plane, item / a.tiles_per_plane, 0, BM, BN, true);
  stage_tap_box<G, NWAVES>(a, t, 0, box0, wave, lane);
  wait_vmem();
  __syncthreads();

  // This lane's share of each distinct k-step pattern (row kg of the step).
  int dpat[NP];
  fill_pat_deltas<G>(dpat, kg, std::make_integer_sequence<int, NP>{});
  const float* wlane = Wres + wm * 64 * MT + lane * MT;
  float bias[MT][4];
  load_bias<MT>(a, t, wm, kg, bias);  // one channel tile: the same for every item

  v4f acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; mi++)
#pragma unroll
    for (int ni = 0; ni < NT; ni++) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

  int parity = 0;  // buffer holding chunk 0 of the current item
  for (;;) {
    int noff[NT], pidx[NT];
    tile_positions<NT, G::CL>(a, t, wn, li, noff, pidx);
    int addr[NP][NT];
#pragma unroll
    for (int q = 0; q < NP; q++)
#pragma unroll
      for (int ni = 0; ni < NT; ni++) addr[q][ni] = 4 * (noff[ni] + dpat[q]);
    const int next_item = item + item_step;
    const bool more = next_item < item_end;
    TileGeo tn = t;
    if (more) tn = tile_geo(a, next_item % a.tiles_per_plane, next_item / a.tiles_per_plane, 0, BM, BN, true);
#pragma unroll
    for (int c = 0; c < NCH; c++) {
      const bool last = c + 1 == NCH;
      const bool has_next = !last || more;
      const int c0n = last ? 0 : (c + 1) * G::CCH;
      const bool odd = ((c & 1) != 0) != (parity != 0);
      const float* wchunk = wlane + c * G::NS * SSTRIDE;
      if (odd)
        tap_stage<MT, NT, WM, NWAVES, G, NP>(a, last ? tn : t, has_next, c0n, box1, box0, wchunk, addr, acc, wave,
                                             lane);
      else
        tap_stage<MT, NT, WM, NWAVES, G, NP>(a, last ? tn : t, has_next, c0n, box0, box1, wchunk, addr, acc, wave,
                                             lane);
      auto store_and_clear = [&] {
        store_tile<MT, NT, G::CL, G::CL && (NCH > 1)>(a, t, wm, kg, pidx, acc, bias);
#pragma unroll
        for (int mi = 0; mi < MT; mi++)
#pragma unroll
          for (int ni = 0; ni < NT; ni++) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};
      };
      // With several chunks per item, the item's stores go out after the
      // barrier below: they complete while the next item's first chunk is
      // reduced, instead of inside the wait. With one chunk per item they would
      // sit in front of the next item's copies, so they go out before the wait.
      if constexpr (NCH == 1) store_and_clear();
      // The next chunk's copies have landed in every wave and no wave still
      // reads this chunk's buffer.
      wait_vmem();
      __syncthreads();
      if constexpr (NCH > 1) {
        if (last) store_and_clear();
      }
    }
    if (!more) break;
    if (NCH & 1) parity ^= 1;
    item = next_item;
    t = tn;
  }
}

// ---------------------------------------------------------------------------
// conv_tap_split: one workgroup per (n, od) plane and group, for few output
// channels (<= 16) and small planes (<= 16*NT positions). Each of the NW waves
// owns one input channel of the group and reduces it against the group's
// weights; the NW partial tiles are summed through LDS at the end.
// - The group's weight matrix (C_out/g rows of C_in/g * kvol floats) is copied
//   once per workgroup with 16-byte DMA copies into a shared LDS region.
// - Each wave copies its channel's input box into its own LDS region, one kernel
//   depth tap (input plane) at a time, so the reduction of the first taps starts
//   while the rest is in flight. The box keeps every F-th input column: with
//   stride and dilation along W both multiples of F no other column is read.
// ---------------------------------------------------------------------------
template <int KD, int KH, int KW, int DD, int DH, int DW, int F, int ROWS, int BW, int NW>
struct SplitGeo {
  static constexpr int FF = F;
  static constexpr int NROWS = ROWS;
  static constexpr int BWC = BW;
  static constexpr int KVOL = KD * KH * KW;
  static constexpr int K = KVOL;          // one channel per wave
  static constexpr int NS = (K + 3) / 4;
  static constexpr int KDT = KD;          // depth taps: staged one at a time
  static constexpr int KPP = KH * KW;     // reduction indices per depth tap
  static constexpr int PLANE = ROWS * BW;
  static constexpr int BOX = KD * PLANE;  // only the planes the depth taps read
  static constexpr int XSW = (BOX + 3) / 4 * 4;           // floats of a wave's box region
  static constexpr int PLANE_INSTR = (PLANE + 63) / 64;   // copies per box plane
  // Shared weights: 16 rows of WROW = NW * KVOL floats (the group's reduction
  // length), stored contiguously (the LDS copy writes consecutive addresses per
  // lane), plus a tail read by the last row's padding taps.
  static constexpr int WROW = NW * KVOL;
  static constexpr bool W4 = WROW % 4 == 0;               // 16-byte copies, else 4-byte
  static constexpr int WCW = W4 ? 4 : 1;                   // floats per copy per lane
  static constexpr int WCH = 16 * WROW / WCW;              // copies of the weight block
  // 16-byte copies go row by row into rows of WLD floats, with WLD/4 odd so the
  // 16 rows of one A-operand read fall on distinct bank groups; 4-byte copies
  // fill the block contiguously (WLD = WROW).
  static constexpr int WQ = WROW / 4;                      // 16-byte chunks per row
  static constexpr int WLD = W4 ? ((WQ % 2) ? WROW : WROW + 4) : WROW;
  static constexpr int WRI = (WQ + 63) / 64;               // copies per row (16-byte path)
  static constexpr int WSH = (16 * WLD + 4 + 3) / 4 * 4;
  static constexpr int W_INSTR = W4 ? (16 * WRI + NW - 1) / NW : (WCH + 64 * NW - 1) / (64 * NW);
  static_assert((KDT - 1) * PLANE_INSTR < 64, "vmcnt range");
  // Highest depth tap read by k-step s (its 4 reduction indices).
  static constexpr int td_of(int s) { return (4 * s + 3 < K ? 4 * s + 3 : K - 1) / KPP; }
  // First k-step that reads depth tap 1.
  static constexpr int first_td1() {
    for (int s = 0; s < NS; s++)
      if (td_of(s) >= 1) return s;
    return NS;
  }
  static constexpr int FIRST_TD1 = first_td1();
  // LDS offset (floats) of reduction index k = (td, th, tw) of the box; padding
  // indices (zero weights) point at the box start.
  static constexpr int koff(int k) {
    if (k >= K) return 0;
    const int td = k / (KH * KW), r2 = k % (KH * KW), th = r2 / KW, tw = r2 % KW;
    return td * PLANE + th * DH * BW + tw * (DW / F);
  }
};

// CL: channels-last x [N, D, H, W, C_in] and y [N, D_out, H_out, W_out, C_out];
// the LDS box keeps the same per-channel layout, only the copies' sources (input
// sites C_in floats apart) and the output addresses change.
template <int NT, int NW, class G, bool CL = false>
__global__ __launch_bounds__(64 * NW) void conv_tap_split_kernel(ConvArgs a) {
  constexpr TapPatterns<G> P{};
  constexpr int NP = P.np;
  constexpr int RED = NW * NT * 4 * 64;
  constexpr int STAGE = G::WSH + NW * G::XSW;
  constexpr int LDS = (STAGE > RED) ? STAGE : RED;
  __shared__ __align__(16) float smem[LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4;
  const int li = lane & 15;
  // Every kernel argument used is read here, in one batch of scalar loads (one
  // memory round trip), and pinned in scalar registers.
  const float* k_x = a.x;
  const float* k_w = a.w;
  const float* k_bias = a.bias;
  float* k_y = a.y;
  int k_Cin = a.Cin;
  int k_Cout = a.Cout;
  int k_Cg = a.Cg;
  int k_Coutg = a.Coutg;
  int k_L0 = a.L0;
  int k_L1 = a.L1;
  int k_L2 = a.L2;
  int k_S0 = a.S0;
  int k_S1 = a.S1;
  int k_S2 = a.S2;
  int k_D0 = a.D0;
  int k_P0 = a.P0;
  int k_P1 = a.P1;
  int k_P2 = a.P2;
  int k_O0 = a.O0;
  int k_O1 = a.O1;
  int k_O2 = a.O2;
  int k_plane_out = a.plane_out;
  int gx = gridDim.x, gy = gridDim.y;
  asm volatile(""
               : "+s"(k_x), "+s"(k_w), "+s"(k_bias), "+s"(k_y), "+s"(k_Cin), "+s"(k_Cout), "+s"(k_Cg), "+s"(k_Coutg),
                 "+s"(k_L0), "+s"(k_L1), "+s"(k_L2), "+s"(k_S0), "+s"(k_S1), "+s"(k_S2), "+s"(k_D0), "+s"(k_P0),
                 "+s"(k_P1), "+s"(k_P2), "+s"(k_O0), "+s"(k_O1), "+s"(k_O2), "+s"(k_plane_out), "+s"(gx), "+s"(gy));
  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous run of (plane, group) items so the input planes that
  // neighbouring output depths share stay in that XCD's L2.
  int item = blockIdx.x + gx * blockIdx.y;
  const int items = gx * gy;
  if ((items & 7) == 0) item = (item & 7) * (items >> 3) + (item >> 3);
  const int plane = item % gx;
  const int g = item / gx;
  const int n = plane / k_O0;
  const int od = plane - n * k_O0;
  const int c = wave;  // this wave's input channel within the group
  float* wsh = smem;
  float* box = smem + G::WSH + wave * G::XSW;

  float b4[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int ch = 4 * kg + r;
    b4[r] = (k_bias && ch < k_Coutg) ? k_bias[g * k_Coutg + ch] : 0.0f;
  }
  {
    // The group's weights, 16 rows (rows past C_out/g read as zero).
    const float* wg = k_w + int64_t(g) * k_Coutg * G::WROW;
    if constexpr (G::W4) {
      // Copy (m, i) moves chunks 64i .. 64i+63 of row m into row m of stride WLD.
#pragma unroll
      for (int it = 0; it < G::W_INSTR; it++) {
        const int ci = it * NW + wave;  // = m * WRI + i
        if (ci < 16 * G::WRI) {
          const int m = ci / G::WRI, i = ci - m * G::WRI;
          const int q = 64 * i + lane;
          const bool ok = m < k_Coutg;
          if (q < G::WQ) lds_dma_f32x4(ok ? wg + m * G::WROW + 4 * q : kZeroWord, wsh + m * G::WLD + 256 * i);
        }
      }
    } else {
      // Copy j moves float j of the contiguous [16][WROW] block.
#pragma unroll
      for (int i = 0; i < G::W_INSTR; i++) {
        const int j0 = (i * NW + wave) * 64;
        const int j = j0 + lane;
        if (j < G::WCH) {
          const bool ok = j / G::WROW < k_Coutg;
          lds_dma_f32(ok ? wg + j : kZeroWord, wsh + j0);
        }
      }
    }
  }
  // Box: element e = ((td * ROWS) + zr) * BW + j <- input
  // (od*S0 - P0 + td*DD, zr - P1, F*j - P2) of channel g*Cg + c. Copy i of a
  // plane moves elements 64i .. 64i + 63; the in-plane part of each lane's
  // source is the same for every plane.
  const int64_t vol_in = int64_t(k_L0) * k_L1 * k_L2;
  const float* xc = CL ? k_x + int64_t(n) * vol_in * k_Cin + (int64_t(g) * k_Cg + c)
                       : k_x + (int64_t(n) * k_Cin + int64_t(g) * k_Cg + c) * vol_in;
  const int site = CL ? k_Cin : 1;  // floats between neighbouring input sites
  int soff[G::PLANE_INSTR];
  uint32_t sok = 0;
#pragma unroll
  for (int i = 0; i < G::PLANE_INSTR; i++) {
    const int e = i * 64 + lane;
    const int zr = e / G::BWC, j = e - zr * G::BWC;
    const int ih = zr - k_P1, iw = G::FF * j - k_P2;
    const bool ok = e < G::PLANE && unsigned(ih) < unsigned(k_L1) && unsigned(iw) < unsigned(k_L2);
    soff[i] = ok ? (ih * k_L2 + iw) * site : 0;
    sok |= uint32_t(ok) << i;
  }
  auto stage_copy = [&](int td, int i) {
    const int id = od * k_S0 - k_P0 + td * k_D0;
    const bool ok = unsigned(id) < unsigned(k_L0) && ((sok >> i) & 1);
    if (i * 64 + lane < G::PLANE)
      lds_dma_f32(ok ? xc + (int64_t(id) * k_L1 * k_L2 * site + soff[i]) : kZeroWord, box + td * G::PLANE + i * 64);
  };
#pragma unroll
  for (int i = 0; i < G::PLANE_INSTR; i++) stage_copy(0, i);
  // Output positions: tiles blockIdx.z*NT .. of the plane (flattened (oh, ow)).
  int noff[NT];
  {
    const int p0 = 16 * int(blockIdx.z) * NT + li;
    const int nlive = k_plane_out - p0;  // tile ni holds a position if 16 ni < nlive
    OffStep os(p0, k_O2, 0, k_S1 * G::BWC, k_S2 / G::FF);
#pragma unroll
    for (int ni = 0; ni < NT; ni++) {
      noff[ni] = 16 * ni < nlive ? os.off : 0;
      os.next();
    }
  }
  int dpat[NP];
  fill_pat_deltas<G>(dpat, kg, std::make_integer_sequence<int, NP>{});
  // Byte offsets: position part per sub-tile, pattern part per distinct step shape.
  const int base_b = int(reinterpret_cast<uintptr_t>(box) - reinterpret_cast<uintptr_t>(smem));
  int nb[NT], dp[NP];
#pragma unroll
  for (int ni = 0; ni < NT; ni++) nb[ni] = base_b + 4 * noff[ni];
#pragma unroll
  for (int q = 0; q < NP; q++) dp[q] = 4 * dpat[q];

  v4f acc[NT];
#pragma unroll
  for (int ni = 0; ni < NT; ni++) acc[ni] = v4f{0.f, 0.f, 0.f, 0.f};
  // Weights (copied by every wave) and this wave's first plane have landed. A
  // plain barrier: the later planes are copied during the reduction and each
  // wave waits for its own copies of them.
  wait_vmem_le<0>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  {
    const char* bb = reinterpret_cast<const char*>(smem);
    const float* wl = wsh + li * G::WLD + c * G::KVOL + kg;  // A[m = li][k = 4s + kg] at wl[4s]
    // Operands of step s+1 are read while the matrix core works on step s. The
    // reduction indices past the channel's kernel volume (last step) take a zero
    // weight: what lies there in LDS belongs to the next channel.
    float av[2];
    float bv[2][NT];
    av[0] = (G::KVOL >= 4 || kg < G::KVOL) ? wl[0] : 0.0f;
#pragma unroll
    for (int ni = 0; ni < NT; ni++)
      bv[0][ni] = *reinterpret_cast<const float*>(bb + nb[ni] + dp[P.pid[0]] + 4 * G::koff(0));
    // Copies of planes 1 .. KDT-1 (in order), DPS per step, all issued before
    // the first step that reads plane 1.
    constexpr int TCOPY = (G::KDT - 1) * G::PLANE_INSTR;
    constexpr int DPS = G::FIRST_TD1 > 0 ? (TCOPY + G::FIRST_TD1 - 1) / G::FIRST_TD1 : TCOPY;
#pragma unroll
    for (int s = 0; s < G::NS; s++) {
      const int cu = s & 1, nx = cu ^ 1;
#pragma unroll
      for (int q = DPS * s; q < DPS * (s + 1) && q < TCOPY; q++) stage_copy(1 + q / G::PLANE_INSTR, q % G::PLANE_INSTR);
      if (s + 1 < G::NS) {
        // Step s+1 reads taps up to depth tap td_of(s+1): wait for its plane.
        if (G::td_of(s + 1) != G::td_of(s)) {
          if (G::td_of(s + 1) == 1) wait_vmem_le<(G::KDT > 2 ? (G::KDT - 2) * G::PLANE_INSTR : 0)>();
          else wait_vmem_le<0>();
        }
        av[nx] = wl[4 * (s + 1)];
        if (4 * (s + 1) + 3 >= G::KVOL) av[nx] = (4 * (s + 1) + kg < G::KVOL) ? av[nx] : 0.0f;
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
          bv[nx][ni] = *reinterpret_cast<const float*>(bb + nb[ni] + dp[P.pid[s + 1]] + 4 * G::koff(4 * (s + 1)));
      }
#pragma unroll
      for (int ni = 0; ni < NT; ni++)
        acc[ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[cu], bv[cu][ni], acc[ni], 0, 0, 0);
      // Interleave the next step's LDS reads with this step's matrix-core work.
#pragma unroll
      for (int i = 0; i < NT; i++) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
  }

  // Sum the NW partial tiles: every wave parks its tile, then wave w adds up the
  // (sub-tile, register) pairs p with p % NW == w and stores them.
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < NT; ni++)
#pragma unroll
    for (int r = 0; r < 4; r++) smem[((wave * NT + ni) * 4 + r) * 64 + lane] = acc[ni][r];
  __syncthreads();
  // All of this wave's partial reads are issued before the sums and stores.
  const int64_t out_plane = int64_t(k_O1) * k_O2;
  constexpr int NPR = (NT * 4 + NW - 1) / NW;  // (tile, register) pairs per wave
  float part[NPR][NW];
#pragma unroll
  for (int j = 0; j < NPR; j++) {
    const int pr = wave + NW * j;
#pragma unroll
    for (int w2 = 0; w2 < NW; w2++)
      part[j][w2] = pr < NT * 4 ? smem[((w2 * NT + (pr >> 2)) * 4 + (pr & 3)) * 64 + lane] : 0.0f;
  }
  // Channel ch of position p: NCDHW y[n][g*Coutg + ch][od][p], channels-last
  // y[n][od][p][g*Coutg + ch].
  float* yg = CL ? k_y + (int64_t(n) * k_O0 + od) * out_plane * k_Cout + int64_t(g) * k_Coutg
                 : k_y + (int64_t(n) * k_Cout + int64_t(g) * k_Coutg) * k_O0 * out_plane + int64_t(od) * out_plane;
  const int64_t ch_stride = CL ? 1 : int64_t(k_O0) * out_plane;
  const int64_t p_stride = CL ? k_Cout : 1;
#pragma unroll
  for (int j = 0; j < NPR; j++) {
    const int pr = wave + NW * j;
    const int ni = pr >> 2, r = pr & 3;
    float v = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < NW; w2++) v += part[j][w2];
    const int ch = 4 * kg + r;
    const int p = 16 * (int(blockIdx.z) * NT + ni) + li;
    const float b = r == 0 ? b4[0] : r == 1 ? b4[1] : r == 2 ? b4[2] : b4[3];
    if (pr < NT * 4 && ch < k_Coutg && p < k_plane_out) yg[ch * ch_stride + p * p_stride] = v + b;
  }
}

// ---------------------------------------------------------------------------
// conv_tap_split_pipe: the channel-split kernel with a short start and its
// cross-wave sums overlapped with products. The plane's tiles run in two
// batches (NT1, then NT2 tiles) over the same staged box.
// - Start: each wave copies its own channel's weights, one kernel depth tap at a
//   time, into its own LDS region, and its box one input plane at a time; it
//   starts on the first tap's weights and plane, and no barrier precedes the
//   products. The A operands are then held in VGPRs.
// - Tap rotation: box slot j holds depth tap (j + t0) % KD, with t0 chosen per
//   output depth so that three neighbouring depths (one XCD, one L2) start on
//   the same input plane: the burst of first copies reads a third of x.
// - Batch 1's partial tiles are parked in the (then free) weight region and a
//   counter in LDS is incremented; late in batch 2, wave w waits for the
//   counter, then sums batch-1 tile w over all waves and stores it. Batch 2's
//   tiles are parked in the box regions and summed after one barrier.
// ---------------------------------------------------------------------------
template <int NT1, int NT2, class G>
struct SplitPipeLds {
  // Weights of one depth tap: KPP floats from an aligned start at most 3 floats
  // below them, as WQT 16-byte slots per row (a multiple of 4: whole copies),
  // stored slot-major, [slot][row m], so one A read hits 64 distinct banks.
  static constexpr int WQT = ((G::KPP + 3 + 3) / 4 + 3) / 4 * 4;
  static constexpr int TAPW = WQT * 16 * 4;  // floats per depth tap
  static constexpr int WI_TAP = WQT / 4;     // copies per depth tap
  static constexpr int WREG = (G::KDT * TAPW > NT1 * 256) ? G::KDT * TAPW : NT1 * 256;
  static constexpr int XREG = (G::XSW > NT2 * 256) ? G::XSW : NT2 * 256;
  static constexpr int CNT = 4;  // floats reserved for the batch-1 counter
};

template <int NT1, int NT2, int NW, class G, bool CL = false>
__global__ __launch_bounds__(64 * NW) void conv_tap_split_pipe_kernel(ConvArgs a) {
  constexpr int NT = NT1 + NT2;
  using L = SplitPipeLds<NT1, NT2, G>;
  constexpr TapPatterns<G> P{};
  constexpr int NP = P.np;
  constexpr int NS = G::NS;
  constexpr int PI = G::PLANE_INSTR;
  constexpr int KDT = G::KDT;
  constexpr int STAGE = L::WI_TAP + PI;  // copies per depth tap (weights, then plane)
  constexpr int TCOPY = (KDT - 1) * STAGE;  // copies of slots 1 .. KD-1, issued during batch 1
  constexpr int DPS = G::FIRST_TD1 > 0 ? (TCOPY + G::FIRST_TD1 - 1) / G::FIRST_TD1 : TCOPY;
  static_assert(KDT * STAGE < 64, "vmcnt range");
  static_assert(NT1 <= NW && NT2 <= NW, "one parked tile per wave in each sum");
  static_assert(G::W4, "16-byte weight copies need C_in/groups * kvol to be a multiple of 4");
  __shared__ __align__(16) float smem[NW * (L::WREG + L::XREG) + L::CNT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4;
  const int li = lane & 15;
  // Every kernel argument used is read here, in one batch of scalar loads:
  // one memory round trip at the start instead of a chain of dependent ones.
  const float* xg = a.x;
  const float* wgl = a.w;
  const float* bg = a.bias;
  float* yglob = a.y;
  int Cin = a.Cin, Cout = a.Cout, Cg = a.Cg, Coutg = a.Coutg;
  int L0 = a.L0, L1 = a.L1, L2 = a.L2, S0 = a.S0, S1 = a.S1, S2 = a.S2, D0 = a.D0;
  int P0 = a.P0, P1 = a.P1, P2 = a.P2, O0 = a.O0, O1 = a.O1, O2 = a.O2, plane_out = a.plane_out;
  int spin_cap = a.spin_cap;
  int gx = gridDim.x, gy = gridDim.y;
  asm volatile("" : "+s"(xg), "+s"(wgl), "+s"(bg), "+s"(yglob), "+s"(Cin), "+s"(Cout), "+s"(Cg), "+s"(Coutg),
               "+s"(L0), "+s"(L1), "+s"(L2), "+s"(S0), "+s"(S1), "+s"(S2), "+s"(D0), "+s"(P0), "+s"(P1), "+s"(P2),
               "+s"(O0), "+s"(O1), "+s"(O2), "+s"(plane_out), "+s"(spin_cap), "+s"(gx), "+s"(gy));
  // XCD-aware item order, as in conv_tap_split.
  int item = blockIdx.x + gx * blockIdx.y;
  const int items = gx * gy;
  if ((items & 7) == 0) item = (item & 7) * (items >> 3) + (item >> 3);
  const int plane = item % gx;
  const int g = item / gx;
  const int n = plane / O0;
  const int od = plane - n * O0;
  const int c = wave;  // this wave's input channel within the group
  const int t0 = (KDT - 1) - od % KDT;  // depth tap of box slot 0
  float* wreg = smem + wave * L::WREG;
  float* box = smem + NW * L::WREG + wave * L::XREG;
  unsigned* counter = reinterpret_cast<unsigned*>(smem + NW * (L::WREG + L::XREG));

  // Bias loads go out before the copies, whose waits count the loads issued
  // after them.
  float b4[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int ch = 4 * kg + r;
    b4[r] = (bg && ch < Coutg) ? bg[g * Coutg + ch] : 0.0f;
  }
  // Copies, in the order they are waited for: for box slot j = 0 .. KD-1, the
  // weights of depth tap t = (j + t0) % KD, then its input plane.
  // Weights of tap t: row m, slot q <- floats ab_t + 4q .. of weight row
  // g*Coutg + m, ab_t the aligned float at or below the tap's first weight
  // (which sits at float o_t of the copy). Slots past the row, or rows past
  // C_out/g, read zero.
  const int cs = c * G::KVOL;
  const int64_t vol_in = int64_t(L0) * L1 * L2;
  const float* xc = CL ? xg + int64_t(n) * vol_in * Cin + (int64_t(g) * Cg + c)
                       : xg + (int64_t(n) * Cin + int64_t(g) * Cg + c) * vol_in;
  const int site = CL ? Cin : 1;
  int soff[PI];
  uint32_t sok = 0;
#pragma unroll
  for (int i = 0; i < PI; i++) {
    const int e = i * 64 + lane;
    const int zr = e / G::BWC, j = e - zr * G::BWC;
    const int ih = zr - P1, iw = G::FF * j - P2;
    const bool ok = e < G::PLANE && unsigned(ih) < unsigned(L1) && unsigned(iw) < unsigned(L2);
    soff[i] = ok ? (ih * L2 + iw) * site : 0;
    sok |= uint32_t(ok) << i;
  }
  // Per box slot: the weight block of its tap (wsrc, starting at float wab of
  // the rows) and its input plane (xsrc; null where the plane is padding).
  const float* wsrc[KDT];
  const float* xsrc[KDT];
  int wab[KDT];
  int tap[KDT];
#pragma unroll
  for (int j = 0; j < KDT; j++) {
    int t = j + t0;
    t = t >= KDT ? t - KDT : t;
    tap[j] = t;
    wab[j] = (cs + t * G::KPP) & ~3;
    wsrc[j] = wgl + int64_t(g) * Coutg * G::WROW + wab[j];
    const int id = od * S0 - P0 + t * D0;
    xsrc[j] = unsigned(id) < unsigned(L0) ? xc + int64_t(id) * L1 * L2 * site : nullptr;
    pin_sgpr(tap[j]);
    pin_sgpr(wab[j]);
    pin_sgpr(wsrc[j]);
    pin_sgpr(xsrc[j]);
  }
  const int wm = lane & 15, wq = lane >> 4;  // row and slot-in-copy of this lane's weight piece
  // Copy u (0 <= u < STAGE) of box slot j: the tap's weight copies, then its plane.
  auto copy = [&](int j, int u) {
    if (u < L::WI_TAP) {
      const int q = 4 * u + wq;
      const bool ok = wm < Coutg && wab[j] + 4 * q < G::WROW;
      lds_dma_f32x4(ok ? wsrc[j] + wm * G::WROW + 4 * q : kZeroWord, wreg + tap[j] * L::TAPW + 256 * u);
    } else {
      const int i = u - L::WI_TAP;
      const bool ok = xsrc[j] != nullptr && ((sok >> i) & 1);
      if (i * 64 + lane < G::PLANE) lds_dma_f32(ok ? xsrc[j] + soff[i] : kZeroWord, box + j * G::PLANE + i * 64);
    }
  };
  // Slot 0 now; slots 1 .. KD-1 during batch 1's first steps.
#pragma unroll
  for (int u = 0; u < STAGE; u++) copy(0, u);
  // The batch-1 counter starts at zero before any wave can increment it.
  if (wave == 0 && lane == 0) *counter = 0u;
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  int dpat[NP];
  fill_pat_deltas<G>(dpat, kg, std::make_integer_sequence<int, NP>{});
  const int base_b = int(reinterpret_cast<uintptr_t>(box) - reinterpret_cast<uintptr_t>(smem));
  int nb[NT], dp[NP];
  {
    const int p0 = 16 * int(blockIdx.z) * NT + li;
    const int nlive = plane_out - p0;  // tile ni holds a position if 16 ni < nlive
    OffStep os(p0, O2, base_b, 4 * S1 * G::BWC, 4 * (S2 / G::FF));
#pragma unroll
    for (int ni = 0; ni < NT; ni++) {
      nb[ni] = 16 * ni < nlive ? os.off : base_b;
      os.next();
    }
  }
#pragma unroll
  for (int q = 0; q < NP; q++) dp[q] = 4 * dpat[q];

  // A[m = li][k = 4s + kg] for box slot j = k / KPP (depth tap (j + t0) % KD),
  // in-tap index r = k % KPP; indices past the kernel volume take a zero weight.
  float av[NS];
  auto load_a = [&](auto sc) {
    constexpr int s = decltype(sc)::value;
    const int k = 4 * s + kg;
    const int j = k / G::KPP;
    const int r = k - j * G::KPP;
    int t = j + t0;
    t = t >= KDT ? t - KDT : t;
    const int f = ((cs + t * G::KPP) & 3) + r;
    const float v = wreg[t * L::TAPW + (f >> 2) * 64 + li * 4 + (f & 3)];
    av[s] = (4 * s + 3 < G::KVOL || k < G::KVOL) ? v : 0.0f;
  };
  // Slot 0's weights and plane have landed (this wave's own copies).
  wait_vmem_le<0>();
  static_for<NS>([&](auto sc) {
    if constexpr (G::td_of(decltype(sc)::value) == 0) load_a(sc);
  });

  const char* bb = reinterpret_cast<const char*>(smem);
  // Products of tiles T0 .. T0+BT-1 over the channel's NS k-steps; operands of
  // step s+1 are read while the matrix core works on step s. In batch 1 the
  // copies of the next box slot are waited for (and its A operands read) before
  // the first step that reads it. hook(s) runs after step s's products.
  auto products = [&](auto t0c, auto btc, v4f* acc, auto&& hook) {
    constexpr int T0 = decltype(t0c)::value, BT = decltype(btc)::value;
    float bv[2][BT];
#pragma unroll
    for (int ni = 0; ni < BT; ni++)
      bv[0][ni] = *reinterpret_cast<const float*>(bb + nb[T0 + ni] + dp[P.pid[0]] + 4 * G::koff(0));
    static_for<NS>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      constexpr int cu = s & 1, nx = cu ^ 1;
      if constexpr (T0 == 0) {
#pragma unroll
        for (int q = DPS * s; q < DPS * (s + 1) && q < TCOPY; q++) copy(1 + q / STAGE, q % STAGE);
      }
      if constexpr (s + 1 < NS) {
        if constexpr (T0 == 0 && G::td_of(s + 1) != G::td_of(s)) {
          // Copies issued so far that belong to slots after td_of(s + 1) may
          // still be in flight.
          constexpr int issued = DPS * (s + 1) < TCOPY ? DPS * (s + 1) : TCOPY;
          constexpr int later = issued - G::td_of(s + 1) * STAGE;
          static_assert(issued >= G::td_of(s + 1) * STAGE, "slot copies issued before their first step");
          wait_vmem_le<(later > 0 ? later : 0)>();
          static_for<NS>([&](auto s2) {
            if constexpr (G::td_of(decltype(s2)::value) == G::td_of(s + 1)) load_a(s2);
          });
        }
#pragma unroll
        for (int ni = 0; ni < BT; ni++)
          bv[nx][ni] = *reinterpret_cast<const float*>(bb + nb[T0 + ni] + dp[P.pid[s + 1]] + 4 * G::koff(4 * (s + 1)));
      }
#pragma unroll
      for (int ni = 0; ni < BT; ni++) acc[ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[cu][ni], acc[ni], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < BT; i++) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      hook(sc);
      // Step boundary for the scheduler: step s+1's operand reads stay here,
      // behind step s's products, instead of sinking next to their use.
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Output of tile T of this workgroup: channel 4 kg + r, position 16 T + li.
  const int64_t out_plane = int64_t(O1) * O2;
  float* yg = CL ? yglob + (int64_t(n) * O0 + od) * out_plane * Cout + int64_t(g) * Coutg
                 : yglob + (int64_t(n) * Cout + int64_t(g) * Coutg) * O0 * out_plane + int64_t(od) * out_plane;
  int64_t ch_stride = CL ? 1 : int64_t(O0) * out_plane;
  int64_t p_stride = CL ? Cout : 1;
  pin_sgpr(yg);
  pin_sgpr(ch_stride);
  pin_sgpr(p_stride);
  auto store_tile = [&](int T, const v4f& v) {
    const int p = 16 * (int(blockIdx.z) * NT + T) + li;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int ch = 4 * kg + r;
      if (ch < Coutg && p < plane_out) yg[ch * ch_stride + p * p_stride] = v[r] + b4[r];
    }
  };
  // Parked tile `slot` of every wave's region (region0 + w * stride), and their
  // sum in a fixed order.
  auto read_parked = [&](const float* region0, int stride, int slot, v4f* part) {
#pragma unroll
    for (int w2 = 0; w2 < NW; w2++)
      part[w2] = *reinterpret_cast<const v4f*>(region0 + w2 * stride + (slot * 64 + lane) * 4);
  };
  auto sum_parts = [&](const v4f* part) {
    v4f v = part[0];
#pragma unroll
    for (int w2 = 1; w2 < NW; w2++) v += part[w2];
    return v;
  };

  // Batch 1.
  {
    v4f acc[NT1];
#pragma unroll
    for (int ni = 0; ni < NT1; ni++) acc[ni] = v4f{0.f, 0.f, 0.f, 0.f};
    products(std::integral_constant<int, 0>{}, std::integral_constant<int, NT1>{}, acc, [](auto) {});
    // Every A operand was read from the weight region before the last steps'
    // products: park batch 1 there, then count this wave in.
#pragma unroll
    for (int ni = 0; ni < NT1; ni++) *reinterpret_cast<v4f*>(wreg + (ni * 64 + lane) * 4) = acc[ni];
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the parked tiles are in LDS
    asm volatile("" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  // Batch 2. Late in it, wave w < NT1 waits until every wave has parked batch 1
  // (each does so unconditionally after its own batch-1 products), then sums
  // batch-1 tile w and stores it. The wait is capped at spin_cap polls; a wave
  // that gives up stores NaN for its whole tile instead of a sum over tiles that
  // may not have been parked, so the event cannot pass unnoticed.
  constexpr int S_WAIT = NS > 8 ? NS - 7 : NS - 1;
  {
    v4f acc[NT2];
#pragma unroll
    for (int ni = 0; ni < NT2; ni++) acc[ni] = v4f{0.f, 0.f, 0.f, 0.f};
    v4f part[NW];
    const bool sums1 = wave < NT1;
    bool parked = false;
    products(std::integral_constant<int, NT1>{}, std::integral_constant<int, NT2>{}, acc, [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s == S_WAIT) {
        if (sums1) {
          for (int spin = 0; spin < spin_cap; spin++) {
            if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= unsigned(NW)) {
              parked = true;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          asm volatile("" ::: "memory");
          read_parked(smem, L::WREG, wave, part);
        }
      } else if constexpr (s == (S_WAIT + 3 < NS ? S_WAIT + 3 : NS - 1)) {
        if (sums1) {
          const float nan = __builtin_nanf("");
          store_tile(wave, parked ? sum_parts(part) : v4f{nan, nan, nan, nan});
        }
      }
    });
    // The box is no longer read by this wave: park batch 2 in it.
#pragma unroll
    for (int ni = 0; ni < NT2; ni++) *reinterpret_cast<v4f*>(box + (ni * 64 + lane) * 4) = acc[ni];
  }
  __syncthreads();
  if (wave < NT2) {
    v4f part[NW];
    read_parked(smem + NW * L::WREG, L::XREG, wave, part);
    store_tile(NT1 + wave, sum_parts(part));
  }
}

// ---------------------------------------------------------------------------
// conv_direct16: small convolutions, latency first. One single-wave workgroup
// per 16 output positions (flattened over n, od, oh, ow) and all output
// channels of a group (<= 16). The wave reads its A operands (weights) and B
// operands (input values at each position's taps) straight from global memory
// into registers: no LDS staging, no barrier, no cross-wave sum, so a launch
// costs one round of global loads, the products and the stores. Single-wave
// workgroups spread the waves over all compute units, so that no unit's load
// pipeline holds more than two of them. The reduction (C_in/groups x kernel
// taps, k-steps of 4) runs in two accumulator chains (even and odd k-steps).
// Build-time: C_in/groups, kernel, dilations; zero padding only.
// Channels-last (CL): x [N, D, H, W, C_in], y [N, D_out, H_out, W_out, C_out].
// ---------------------------------------------------------------------------
template <int CIN, int KD, int KH, int KW, int DD, int DH, int DW>
struct DirectGeo {
  static constexpr int CG = CIN;
  static constexpr int KVOL = KD * KH * KW;
  static constexpr int K = CIN * KVOL;
  static constexpr int NS = (K + 3) / 4;
  // (channel, depth, row, column) coefficients of reduction index k; indices
  // past K take tap 0 (their weights are zero).
  static constexpr int kc(int k) { return k < K ? k / KVOL : 0; }
  static constexpr int ktd(int k) { return k < K ? (k % KVOL) / (KH * KW) * DD : 0; }
  static constexpr int kth(int k) { return k < K ? (k % (KH * KW)) / KW * DH : 0; }
  static constexpr int ktw(int k) { return k < K ? (k % KW) * DW : 0; }
};

// Distinct per-step lane patterns of (channel, depth, row, column) deltas.
template <class G>
struct DirectPatterns {
  int np = 0;
  int pid[G::NS] = {};
  int pat[G::NS][4][4] = {};  // [pattern][kg][c, td, th, tw]
  constexpr DirectPatterns() {
    for (int s = 0; s < G::NS; s++) {
      int d[4][4] = {};
      for (int j = 0; j < 4; j++) {
        const int k = 4 * s + j, k0 = 4 * s;
        d[j][0] = G::kc(k) - G::kc(k0);
        d[j][1] = G::ktd(k) - G::ktd(k0);
        d[j][2] = G::kth(k) - G::kth(k0);
        d[j][3] = G::ktw(k) - G::ktw(k0);
      }
      int found = -1;
      for (int q = 0; q < np && found < 0; q++) {
        bool eq = true;
        for (int j = 0; j < 4; j++)
          for (int e = 0; e < 4; e++) eq = eq && pat[q][j][e] == d[j][e];
        if (eq) found = q;
      }
      if (found < 0) {
        for (int j = 0; j < 4; j++)
          for (int e = 0; e < 4; e++) pat[np][j][e] = d[j][e];
        found = np++;
      }
      pid[s] = found;
    }
  }
};

// Arguments of conv_direct16, precomputed on the host: element strides of the
// input, reciprocals of the output extents, so that the first instructions
// need no divide and every argument arrives in one round of scalar loads.
struct DirectArgs {
  const float* x;
  const float* w;
  const float* bias;
  float* y;
  int sc, sd, sh, sw, sn;  // input element strides: channel, depth, row, column, sample
  int ssd, ssh, ssw;       // input offset of one output step in depth, row, column
  int sg;                  // input offset of one group's first channel
  int O0, O1, O2, npos;    // output extents; npos = N * O0 * O1 * O2 (< 2^24)
  float r0, r1, r2;        // 1 / O0, 1 / O1, 1 / O2 (fp32)
  int Cout, Coutg;
};

template <class G, bool CL>
__global__ __launch_bounds__(64) void conv_direct16_kernel(DirectArgs a) {
  // Every argument in registers before any use: the scalar loads leave together
  // and meet one wait (otherwise they are spread over dependent rounds).
  asm volatile("" ::"s"(a.x), "s"(a.w), "s"(a.bias), "s"(a.y), "s"(a.sc), "s"(a.sd), "s"(a.sh), "s"(a.sw),
               "s"(a.sn), "s"(a.ssd), "s"(a.ssh), "s"(a.ssw), "s"(a.sg), "s"(a.O0), "s"(a.O1), "s"(a.O2),
               "s"(a.npos), "s"(a.r0), "s"(a.r1), "s"(a.r2), "s"(a.Cout), "s"(a.Coutg));
  __builtin_amdgcn_sched_barrier(0);
  constexpr DirectPatterns<G> P{};
  constexpr int NP = P.np;
  const int lane = threadIdx.x;
  const int kg = lane >> 4;
  const int li = lane & 15;
  const GlobalF* xg = (const GlobalF*)(a.x);
  const GlobalF* wg = (const GlobalF*)(a.w);
  const GlobalF* bg = (const GlobalF*)(a.bias);
  float* yg = a.y;
  const int Cout = a.Cout, Coutg = a.Coutg;
  const int O0 = a.O0, O1 = a.O1, O2 = a.O2;
  const int sc = a.sc, sd = a.sd, sh = a.sh, sw = a.sw;
  const int g = blockIdx.y;
  const int npos = a.npos;
  // This lane's position (clamped into range for the loads; stores skip it).
  const int p = int(blockIdx.x) * 16 + li;
  const bool valid = p < npos;
  const int pc = valid ? p : npos - 1;
  int ow, oh, od;
  int r = divmod_small(pc, O2, a.r2, ow);
  r = divmod_small(r, O1, a.r1, oh);
  const int n = divmod_small(r, O0, a.r0, od);
  const int base = n * a.sn + g * a.sg + od * a.ssd + oh * a.ssh + ow * a.ssw;
  // Lane part of each distinct step pattern.
  int dp[NP];
  static_for<NP>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    const int b0 = kg & 1, b1 = (kg >> 1) & 1;
    auto sel = [&](int e) {
      const int d0 = P.pat[q][0][e], d1 = P.pat[q][1][e], d2 = P.pat[q][2][e], d3 = P.pat[q][3][e];
      return d0 + b0 * (d1 - d0) + b1 * (d2 - d0) + (b0 & b1) * (d3 - d2 - d1 + d0);
    };
    dp[q] = base + sel(0) * sc + sel(1) * sd + sel(2) * sh + sel(3) * sw;
  });
  // Operands of every k-step, all loads issued before the first product.
  const bool arow = li < Coutg;
  const int wrow = (g * Coutg + (arow ? li : 0)) * G::K;
  float av[G::NS], bv[G::NS];
  static_for<G::NS>([&](auto sc_) {
    constexpr int s = decltype(sc_)::value;
    constexpr int k0 = 4 * s;
    const int tap0 = G::kc(k0) * sc + G::ktd(k0) * sd + G::kth(k0) * sh + G::ktw(k0) * sw;
    bv[s] = xg[dp[P.pid[s]] + tap0];
    const int k = k0 + kg;
    const bool ok = arow && k < G::K;
    const float wv = wg[wrow + (k < G::K ? k : 0)];
    av[s] = ok ? wv : 0.0f;
  });
  // Bias of this lane's four channels (register r: channel 4kg + r).
  float bias4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (bg) {
#pragma unroll
    for (int rr = 0; rr < 4; rr++) bias4[rr] = bg[g * Coutg + min(4 * kg + rr, Coutg - 1)];
  }
  // Keep every load ahead of the products: one round of memory latency.
  __builtin_amdgcn_sched_barrier(0);
  v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = v4f{0.f, 0.f, 0.f, 0.f};
  static_for<G::NS>([&](auto sc_) {
    constexpr int s = decltype(sc_)::value;
    if constexpr (s & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc1, 0, 0, 0);
    else acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc0, 0, 0, 0);
  });
  const v4f acc = acc0 + acc1;
  if (!valid) return;
  if constexpr (CL) {
    const int64_t opos = ((int64_t(n) * O0 + od) * O1 + oh) * O2 + ow;
    float* yp = yg + opos * Cout + g * Coutg;
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      const int ch = 4 * kg + rr;
      if (ch < Coutg) yp[ch] = acc[rr] + bias4[rr];
    }
  } else {
    const int64_t plane = int64_t(O0) * O1 * O2;
    const int64_t sp = (int64_t(od) * O1 + oh) * O2 + ow;
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      const int ch = 4 * kg + rr;
      if (ch < Coutg) yg[(int64_t(n) * Cout + g * Coutg + ch) * plane + sp] = acc[rr] + bias4[rr];
    }
  }
}

// ---------------------------------------------------------------------------
// conv_tap_kstream: one workgroup per (n, od) output plane and group, for few
// output channels per group (<= 16) and planes of at most 16 tiles of 16
// positions. Four compute waves, one per SIMD, split the plane's work (tiles x
// reduction) evenly and without a cross-wave reduction for all but T % 4 tiles:
// - compute wave w owns T/4 whole tiles and reduces them over the group's
//   entire reduction (C_in/groups x kernel taps, no per-channel padding);
// - each of the T % 4 remaining tiles is split by 16-deep blocks of the
//   reduction: wave w takes the blocks q with q % 4 == w (stream-K within the
//   workgroup), and the four partial tiles are summed in a fixed order at the end.
// Four copy waves issue every LDS DMA copy and do nothing else, so the compute
// waves' instruction streams hold only operand reads and products: with one
// compute wave per SIMD, address arithmetic or copy issue in its stream would
// stall the matrix core, and with copies in flight the compiler's wait-count
// tracking could only wait for an LDS read by draining all of them.
// Reduction order: block q holds reduction indices 16q .. 16q+15 as two pairs of
// k-steps; at k-step 2p + i, matrix row kg of the 4-deep step takes index
// 8p + 2kg + i. With that order the A operands of a k-step pair are, per lane,
// 2 consecutive weights of one output channel, and those of a block are 16-byte
// runs of w: one 16-byte LDS DMA copy per block stages them for all 64 lanes
// straight from w (layout [p][row][kg][2]), one 8-byte LDS read per k-step pair
// fetches them, and the 4 matrix rows of a k-step read taps at most 6 apart,
// so the B operand reads of a step mostly share LDS banks' addresses.
// The input box keeps every F-th input column (stride and dilation along W
// multiples of F) of every input row the plane reads, per (channel, depth tap)
// plane; planes are copied by 4-byte LDS DMA in the order the reduction
// consumes them, several blocks ahead. Each copy wave waits for its own copies
// and meets the compute waves at a barrier before the blocks that read them.
// ---------------------------------------------------------------------------
template <int CG, int KD, int KH, int KW, int DH, int DW, int F, int ROWS, int BW, int T, bool CLQ = false>
struct KsGeo {
  static constexpr int KVOL = KD * KH * KW;
  static constexpr int KPP = KH * KW;           // reduction indices per box plane
  static constexpr int K = CG * KVOL;           // group reduction length
  static_assert(K % 4 == 0, "16-byte weight copies");
  static constexpr int NQ = (K + 15) / 16;      // 16-deep reduction blocks
  static constexpr int NS = 4 * NQ;             // 4-deep k-steps
  static constexpr int FF = F, BWC = BW, ROWSC = ROWS, KDC = KD, KHC = KH, KWC = KW, DHC = DH, DWC = DW, CGC = CG;
  // CLQ (channels-last input, C_in/groups a multiple of 4): a box plane holds
  // one (channel quad, depth tap), 4 channels interleaved per site and copied
  // 16 bytes per lane; otherwise one (channel, depth tap), 4 bytes per lane.
  static_assert(!CLQ || CG % 4 == 0, "channel quads");
  static constexpr int CH = CLQ ? 4 : 1;        // channels per plane
  static constexpr int PLANE = ROWS * BW;       // box sites per plane
  static constexpr int PI = (PLANE + 63) / 64;  // copy instructions per plane
  static constexpr int PIW = (PI + 3) / 4;      // ... per wave (the rest pad to a multiple of 4)
  static constexpr int PSLOT = PI * 64 * CH;    // floats per plane slot (whole copies)
  static constexpr int NPL = CG / CH * KD;      // planes in the box
  static constexpr int FT = T / 4, R = T % 4;   // whole tiles per wave, split tiles
  static constexpr int NTW = FT + R;            // tiles a wave accumulates
  static constexpr int WQ = 4;                  // reduction blocks per weight stage (1 per copy wave)
  static constexpr int NWS = (NQ + WQ - 1) / WQ;
  // LDS (floats): box planes | weight operands [q][lane][4] | padding-copy target | split-tile partials
  static constexpr int WOFF = NPL * PSLOT;
  static constexpr int DUMMY = WOFF + NQ * 256;
  static constexpr int RED = DUMMY + 256;
  static constexpr int LDS = RED + 4 * (R > 0 ? R : 1) * 256;
  // Reduction index of matrix row kg at k-step s: k-steps 2p and 2p+1 take
  // indices 8p .. 8p+7, row kg the pair 8p + 2kg, 8p + 2kg + 1.
  static constexpr int kidx(int s, int kg) { return 8 * (s >> 1) + 2 * kg + (s & 1); }
  // LDS offset (floats) of reduction index k = (c, td, th, tw); indices past K
  // (zero weights) point at the box start.
  static constexpr int koff(int k) {
    if (k >= K) return 0;
    const int c = k / KVOL, r = k % KVOL, td = r / KPP, r2 = r % KPP, th = r2 / KW, tw = r2 % KW;
    return (c / CH * KD + td) * PSLOT + (th * DH * BW + tw * (DW / F)) * CH + c % CH;
  }
  // First block that reads box plane p = (channel / CH) * KD + td.
  static constexpr int plane_need(int p) { return ((p / KD) * CH * KVOL + (p % KD) * KPP) / 16; }
};

// Distinct per-step lane patterns koff(kidx(s, kg)) - koff(kidx(s, 0)).
template <class G>
struct KsPatterns {
  int np = 0;
  int pid[G::NS] = {};
  int pat[G::NS][4] = {};
  constexpr KsPatterns() {
    for (int s = 0; s < G::NS; s++) {
      int d[4] = {};
      for (int j = 0; j < 4; j++) d[j] = G::koff(G::kidx(s, j)) - G::koff(G::kidx(s, 0));
      int found = -1;
      for (int q = 0; q < np && found < 0; q++) {
        bool eq = true;
        for (int j = 0; j < 4; j++) eq = eq && pat[q][j] == d[j];
        if (eq) found = q;
      }
      if (found < 0) {
        for (int j = 0; j < 4; j++) pat[np][j] = d[j];
        found = np++;
      }
      pid[s] = found;
    }
  }
};

// Lane kg's share of distinct step pattern Q (from the two bits of kg).
template <class G, int Q>
__device__ __forceinline__ int ks_delta(int kg) {
  constexpr KsPatterns<G> P{};
  constexpr int d0 = P.pat[Q][0], d1 = P.pat[Q][1], d2 = P.pat[Q][2], d3 = P.pat[Q][3];
  const int b0 = kg & 1, b1 = (kg >> 1) & 1;
  return d0 + b0 * (d1 - d0) + b1 * (d2 - d0) + (b0 & b1) * (d3 - d2 - d1 + d0);
}
template <class G, int... Q>
__device__ __forceinline__ void fill_ks_deltas(int* dp, int kg, std::integer_sequence<int, Q...>) {
  ((dp[Q] = ks_delta<G, Q>(kg)), ...);
}

// Copy stages in the order they are needed: plane p = c * KD + td (first read by
// block p * KPP / 16) and weight stage r (blocks 16r .. 16r+15). Each stage is
// the same number of copy instructions in every wave, so a wave's own copy
// count (vmcnt) tells which stages it has landed.
template <class G>
struct KsSchedule {
  static constexpr int NST = G::NPL + G::NWS;
  static constexpr int EARLY = 2;  // a stage is waited for at least this many blocks before its first use
  static constexpr int LOOK = 14;  // and issued this many blocks before its first use
  // Waits (and barriers) at blocks 0, 2 and then every 4 blocks: between two
  // barriers after the start every wave takes the same number of split-tile
  // turns, and the first barrier waits only for what blocks 0 and 1 read.
  static constexpr bool wait_point(int q) { return q == 0 || q == 2 || q % 4 == 0; }
  static constexpr int next_wait_point(int q) {
    int r = q + 1;
    while (r < G::NQ && !wait_point(r)) r++;
    return r;
  }
  int type[NST] = {};  // 0: plane, 1: weights
  int idx[NST] = {};
  int need[NST] = {};
  int cnt[NST] = {};   // copy instructions per wave
  int wait_pre[G::NQ] = {};   // stages complete before block q's operands are read: prefix length
  int issue_pre[G::NQ] = {};  // stages issued by the end of block q's issue point
  int vm_allow[G::NQ] = {};   // vmcnt allowed at block q's wait (-1: no wait)
  int max_out = 0;
  constexpr KsSchedule() {
    int n = 0;
    for (int r = 0; r < G::NWS; r++) { type[n] = 1; idx[n] = r; need[n] = r * G::WQ; cnt[n] = G::WQ / 4; n++; }
    for (int p = 0; p < G::NPL; p++) { type[n] = 0; idx[n] = p; need[n] = G::plane_need(p); cnt[n] = G::PIW; n++; }
    // Stable insertion sort by first use (weights before planes on a tie).
    for (int i = 1; i < NST; i++)
      for (int j = i; j > 0 && need[j - 1] > need[j]; j--) {
        int t;
        t = type[j]; type[j] = type[j - 1]; type[j - 1] = t;
        t = idx[j]; idx[j] = idx[j - 1]; idx[j - 1] = t;
        t = need[j]; need[j] = need[j - 1]; need[j - 1] = t;
        t = cnt[j]; cnt[j] = cnt[j - 1]; cnt[j - 1] = t;
      }
    int waited = 0;
    for (int q = 0; q < G::NQ; q++) {
      int ip = 0, wp = 0;
      while (ip < NST && need[ip] <= q + LOOK) ip++;
      // at a wait point, every stage read before the next wait point (+ EARLY)
      if (wait_point(q))
        while (wp < NST && need[wp] <= next_wait_point(q) - 1 + EARLY) wp++;
      issue_pre[q] = ip;
      wait_pre[q] = wp;
      // The wait at block q comes before block q's issue: copies issued by
      // the end of block q-1 (or at the start, for q = 0) are in flight.
      const int issued = q == 0 ? issue_pre[0] : issue_pre[q - 1];
      if (wait_point(q) && wp > waited) {
        int later = 0;
        for (int s = wp; s < issued; s++) later += cnt[s];
        vm_allow[q] = later;
        waited = wp;
      } else {
        vm_allow[q] = -1;
      }
      int out = 0;
      for (int s = 0; s < ip; s++) out += cnt[s];
      if (out > max_out) max_out = out;
    }
  }
};

template <class G, bool CL>
__global__ __launch_bounds__(512) void conv_tap_kstream_kernel(ConvArgs a) {
  constexpr KsPatterns<G> P{};
  constexpr KsSchedule<G> SC{};
  constexpr int NP = P.np;
  constexpr int NTW = G::NTW;
  static_assert(G::NTW >= 1 && G::FT * 4 + G::R <= 16, "at most 16 tiles per plane");
  __shared__ __align__(16) float smem[G::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool copier = wid >= 4;
  const int wave = copier ? wid - 4 : wid;  // compute wave, or copy wave index
  const int kg = lane >> 4;
  const int li = lane & 15;
  // Every kernel argument used is read here, in one batch of scalar loads, and
  // pinned in scalar registers.
  const float* xg = a.x;
  const float* wgl = a.w;
  const float* bg = a.bias;
  float* yglob = a.y;
  int Cin = a.Cin, Cout = a.Cout, Cg = a.Cg, Coutg = a.Coutg;
  int L0 = a.L0, L1 = a.L1, L2 = a.L2, S0 = a.S0, S1 = a.S1, S2 = a.S2, D0 = a.D0;
  int P0 = a.P0, P1 = a.P1, P2 = a.P2, O0 = a.O0, O1 = a.O1, O2 = a.O2, plane_out = a.plane_out;
  int nitems = gridDim.x;
  int vec_store = a.vec_store;
  asm volatile("" : "+s"(xg), "+s"(wgl), "+s"(bg), "+s"(yglob), "+s"(Cin), "+s"(Cout), "+s"(Cg), "+s"(Coutg),
               "+s"(L0), "+s"(L1), "+s"(L2), "+s"(S0), "+s"(S1), "+s"(S2), "+s"(D0), "+s"(P0), "+s"(P1), "+s"(P2),
               "+s"(O0), "+s"(O1), "+s"(O2), "+s"(plane_out), "+s"(nitems), "+s"(vec_store));
  // Workgroups are dispatched round-robin over the 8 XCDs: give each XCD a
  // contiguous run of (plane, group) items, so the input planes that
  // neighbouring output depths share stay in that XCD's L2. Channels-last:
  // group fastest, so the groups of one plane, which split the channels of the
  // same input sites (and cache lines), share that L2 too; channels-first:
  // plane fastest, so an XCD's run covers twice the depths and re-reads fewer
  // planes at its ends.
  int item = blockIdx.x;
  if ((nitems & 7) == 0) item = (item & 7) * (nitems >> 3) + (item >> 3);
  const int ngroups = Cout / Coutg;
  const int nplanes = nitems / ngroups;
  const int plane = CL ? item / ngroups : item % nplanes;
  const int g = CL ? item - plane * ngroups : item / nplanes;
  const int n = plane / O0;
  const int od = plane - n * O0;
  float* box = smem;
  float* wts = smem + G::WOFF;

  if (copier) {
    // Copy sources. Plane element e = zr * BW + j <- input row zr - P1, column
    // F*j - P2 of the plane's channel and depth; copy wave w's copy i of a plane
    // moves elements (4i + w) * 64 + lane, the same in-plane offsets for every plane.
    // Channels-last input: sites C_in floats apart, a channel at its offset in the site.
    float* dummy = smem + G::DUMMY;
    const int64_t plane_in = int64_t(L1) * L2;
    const int64_t vol_in = int64_t(L0) * plane_in;
    const float* xg0 = CL ? xg + int64_t(n) * vol_in * Cin + int64_t(g) * Cg
                          : xg + (int64_t(n) * Cin + int64_t(g) * Cg) * vol_in;
    const int64_t c_step = CL ? 1 : vol_in;                      // next channel
    const int64_t d_step = CL ? plane_in * Cin : plane_in;       // next input depth
    const int site = CL ? Cin : 1;
    const int id0 = od * S0 - P0;
    int soff[G::PIW];
    uint32_t sok = 0;
#pragma unroll
    for (int i = 0; i < G::PIW; i++) {
      const int e = (4 * i + wave) * 64 + lane;
      const int zr = e / G::BWC, j = e - zr * G::BWC;
      const int ih = zr - P1, iw = G::FF * j - P2;
      const bool ok = e < G::PLANE && unsigned(ih) < unsigned(L1) && unsigned(iw) < unsigned(L2);
      soff[i] = ok ? (ih * L2 + iw) * site : 0;
      sok |= uint32_t(ok) << i;
    }
    const float* wg = wgl + int64_t(g) * Coutg * G::K;
    auto issue_stage = [&](auto stc) {
      constexpr int st = decltype(stc)::value;
      if constexpr (SC.type[st] == 0) {
        constexpr int p = SC.idx[st];
        constexpr int c = p / G::KDC * G::CH, td = p % G::KDC;  // first channel, depth tap
        const int id = id0 + td * D0;
        const bool dok = unsigned(id) < unsigned(L0);
        const float* pl = xg0 + c * c_step + int64_t(id) * d_step;
#pragma unroll
        for (int i = 0; i < G::PIW; i++) {
          const int ii = 4 * i + wave;  // copy instruction of the plane (wave-uniform)
          const bool real = ii < G::PI;
          const bool ok = real && dok && ((sok >> i) & 1);
          if constexpr (G::CH == 4)
            lds_dma_f32x4(ok ? pl + soff[i] : kZeroWord, real ? box + p * G::PSLOT + ii * 256 : dummy);
          else
            lds_dma_f32(ok ? pl + soff[i] : kZeroWord, real ? box + p * G::PSLOT + ii * 64 : dummy);
        }
      } else {
        constexpr int r = SC.idx[st];
        // Lane l of block q's copy: k-step pair p = 2q + l/32, row m = (l%32)/2,
        // weights 8p + 4(l%2) .. +3 of channel m -> floats 128p + 8m + 4(l%2).
        const int wl = lane & 31, wm = wl >> 1;
#pragma unroll
        for (int i = 0; i < G::WQ / 4; i++) {
          const int q = r * G::WQ + 4 * i + wave;  // reduction block (wave-uniform)
          const bool real = q < G::NQ;
          const int k = 16 * q + 8 * (lane >> 5) + 4 * (wl & 1);
          const bool ok = real && wm < Coutg && k < G::K;
          lds_dma_f32x4(ok ? wg + wm * G::K + k : kZeroWord, real ? wts + q * 256 : dummy);
        }
      }
    };
    // The stages first read within the look-ahead of block 0; then, at each of
    // the compute waves' barriers, this wave's copies of the stages that barrier
    // releases have landed, and the stages that enter the look-ahead are issued.
    static_for<SC.issue_pre[0]>([&](auto st) { issue_stage(st); });
    static_for<G::NQ>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      if constexpr (SC.vm_allow[q] >= 0) {
        static_assert(SC.vm_allow[q] < 64, "vmcnt range");
        wait_vmem_le<SC.vm_allow[q]>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      if constexpr (q > 0) {
        static_for<SC.issue_pre[q] - SC.issue_pre[q - 1]>([&](auto sc) {
          issue_stage(std::integral_constant<int, SC.issue_pre[q - 1] + decltype(sc)::value>{});
        });
      }
    });
    if constexpr (G::R > 0) __syncthreads();  // the split tiles' partial sums are parked
    return;
  }

  // Compute waves. Bias of the 4 channels this lane's accumulator registers
  // hold, read through a global-address-space pointer (a flat load would count
  // against the LDS counter too, and the compiler would then drain every LDS
  // read at each operand wait of the product loop), and waited for here.
  float b4[4];
  const GlobalF* bgg = (const GlobalF*)(bg);
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int ch = 4 * kg + r;
    b4[r] = (bg && ch < Coutg) ? bgg[g * Coutg + ch] : 0.0f;
  }
  // Tiles of this wave: whole tiles wave*FT .. wave*FT + FT-1, then the split
  // tiles 4FT .. T-1. Lane li's position in tile t is 16t + li.
  int nb[NTW];
  {
    OffStep os(16 * wave * G::FT + li, O2, 0, S1 * G::BWC * G::CH, S2 / G::FF * G::CH);
#pragma unroll
    for (int i = 0; i < G::FT; i++) {
      nb[i] = 16 * (wave * G::FT + i) + li < plane_out ? os.off : 0;
      os.next();
    }
    if constexpr (G::R > 0) {
      OffStep os2(16 * 4 * G::FT + li, O2, 0, S1 * G::BWC * G::CH, S2 / G::FF * G::CH);
#pragma unroll
      for (int i = 0; i < G::R; i++) {
        nb[G::FT + i] = 16 * (4 * G::FT + i) + li < plane_out ? os2.off : 0;
        os2.next();
      }
    }
  }
  int dpat[NP];
  fill_ks_deltas<G>(dpat, kg, std::make_integer_sequence<int, NP>{});
  int addr[NP][NTW];
#pragma unroll
  for (int q = 0; q < NP; q++)
#pragma unroll
    for (int t = 0; t < NTW; t++) addr[q][t] = 4 * (nb[t] + dpat[q]);

  v4f acc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; t++) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f acc2[G::R > 0 ? G::R : 1];  // the split tiles' odd k-steps (a second chain)
#pragma unroll
  for (int r = 0; r < G::R; r++) acc2[r] = v4f{0.f, 0.f, 0.f, 0.f};
  // With fewer than 3 whole tiles per wave, their odd k-steps accumulate in a
  // second chain too: consecutive products then do not wait for each other.
  constexpr bool WCH2 = G::FT > 0 && G::FT < 3;
  v4f accw[WCH2 ? G::FT : 1];
#pragma unroll
  for (int t = 0; t < (WCH2 ? G::FT : 1); t++) accw[t] = v4f{0.f, 0.f, 0.f, 0.f};
  wait_vmem_le<0>();  // no memory access of this path is left in flight in the product loop
  const char* bb = reinterpret_cast<const char*>(smem);
  // B operand of tile t at k-step S: one LDS read at (lane register + immediate).
  auto bread = [&](auto sc, int t) {
    constexpr int S = decltype(sc)::value;
    return *reinterpret_cast<const float*>(bb + addr[P.pid[S]][t] + 4 * G::koff(G::kidx(S, 0)));
  };
  // Operands are read two k-steps ahead of the products that use them, one or
  // two reads after each product in issue order (a burst of reads between two
  // products would hold back the second while they issue). A: a float2 per
  // k-step pair (two pairs buffered); B: per k-step and whole tile, three
  // k-steps buffered; the split tiles' B of a block, read only before this
  // wave's turns, two blocks buffered.
  float2 ap[2];
  float bs[3][G::FT > 0 ? G::FT : 1];
  float br[2][4][G::R > 0 ? G::R : 1];
  auto read_a = [&](auto pc) {
    constexpr int pp = decltype(pc)::value;
    ap[pp & 1] = *reinterpret_cast<const float2*>(wts + pp * 128 + li * 8 + kg * 2);
  };
  auto read_b = [&](auto sc, int t) {
    constexpr int S = decltype(sc)::value;
    bs[S % 3][t] = bread(std::integral_constant<int, S>{}, t);
  };
  auto read_r = [&](auto qc) {
    constexpr int q = decltype(qc)::value;
    static_for<4>([&](auto jc) {
      constexpr int S = 4 * q + decltype(jc)::value;
#pragma unroll
      for (int r = 0; r < G::R; r++) br[q & 1][decltype(jc)::value][r] = bread(std::integral_constant<int, S>{}, G::FT + r);
    });
  };

  static_for<G::NQ>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    // The stages this block and the next ones read have landed in every wave.
    if constexpr (SC.vm_allow[q] >= 0) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    if constexpr (q == 0) {
      read_a(std::integral_constant<int, 0>{});
#pragma unroll
      for (int t = 0; t < G::FT; t++) read_b(std::integral_constant<int, 0>{}, t);
#pragma unroll
      for (int t = 0; t < G::FT; t++) read_b(std::integral_constant<int, 1>{}, t);
      if constexpr (G::R > 0) {
        if (wave == 0) read_r(std::integral_constant<int, 0>{});
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    float aa[4];  // the block's A operands, kept for the split tiles' turn
    static_for<4>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int s = 4 * q + j;
      const float av = (s & 1) ? ap[(s >> 1) & 1].y : ap[(s >> 1) & 1].x;
      aa[j] = av;
      static_for<G::FT>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if constexpr (WCH2 && (s & 1)) accw[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bs[s % 3][t], accw[t], 0, 0, 0);
        else acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bs[s % 3][t], acc[t], 0, 0, 0);
        // Reads after this product: B of step s+2 for tile t; after the first
        // product of an odd step, A of pair s/2 + 1.
        constexpr bool rb = s + 2 < G::NS;
        constexpr bool ra = t == 0 && (s & 1) && (s >> 1) + 1 < G::NS / 2;
        if constexpr (rb) read_b(std::integral_constant<int, s + 2>{}, t);
        if constexpr (ra) read_a(std::integral_constant<int, (s >> 1) + 1>{});
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        constexpr int nr = (rb ? 1 : 0) + (ra ? 1 : 0);
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
      });
    });
    if constexpr (G::R > 0) {
      // The split tiles: this block's 4 k-steps if it is this wave's turn (two
      // chains, even and odd k-steps, added at the end); then the split tiles'
      // B operands of the next block if that is this wave's turn.
      if ((q & 3) == wave) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++)
#pragma unroll
          for (int r = 0; r < G::R; r++) {
            if (jj & 1) acc2[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(aa[jj], br[q & 1][jj][r], acc2[r], 0, 0, 0);
            else acc[G::FT + r] = __builtin_amdgcn_mfma_f32_16x16x4f32(aa[jj], br[q & 1][jj][r], acc[G::FT + r], 0, 0, 0);
          }
      }
      if constexpr (q + 1 < G::NQ) {
        if (((q + 1) & 3) == wave) read_r(std::integral_constant<int, q + 1>{});
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  });

  // Output: channel 4kg + r, position 16t + li of the (n, g*Coutg + ch, od)
  // plane; channels-last: of site (n, od, position), 4 consecutive channels.
  const int64_t out_plane = int64_t(O1) * O2;
  float* yg = CL ? yglob + (int64_t(n) * O0 + od) * out_plane * Cout + int64_t(g) * Coutg
                 : yglob + (int64_t(n) * Cout + int64_t(g) * Coutg) * O0 * out_plane + int64_t(od) * out_plane;
  const int64_t ch_stride = CL ? 1 : int64_t(O0) * out_plane;
  const int64_t p_stride = CL ? Cout : 1;
  if constexpr (WCH2) {
#pragma unroll
    for (int i = 0; i < G::FT; i++) acc[i] += accw[i];
  }
#pragma unroll
  for (int i = 0; i < G::FT; i++) {
    const int p = 16 * (wave * G::FT + i) + li;
    if constexpr (CL) {
      if (p < plane_out) {
        float* yp = yg + p * p_stride + 4 * kg;
        if (vec_store && 4 * kg + 4 <= Coutg) {
          *reinterpret_cast<v4f*>(yp) = v4f{acc[i][0] + b4[0], acc[i][1] + b4[1], acc[i][2] + b4[2], acc[i][3] + b4[3]};
        } else {
#pragma unroll
          for (int r = 0; r < 4; r++)
            if (4 * kg + r < Coutg) yp[r] = acc[i][r] + b4[r];
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int ch = 4 * kg + r;
        if (ch < Coutg && p < plane_out) yg[ch * ch_stride + p] = acc[i][r] + b4[r];
      }
    }
  }
  if constexpr (G::R > 0) {
    // Split tiles: park the partials, then wave w sums register w of every
    // split tile over the 4 compute waves (fixed order) and stores channel 4kg + w.
    float* red = smem + G::RED;
#pragma unroll
    for (int r = 0; r < G::R; r++)
      *reinterpret_cast<v4f*>(red + ((wave * G::R + r) * 64 + lane) * 4) = acc[G::FT + r] + acc2[r];
    __syncthreads();
    const int ch = 4 * kg + wave;
    const float bw_ = (bg && ch < Coutg) ? bgg[g * Coutg + ch] : 0.0f;
#pragma unroll
    for (int r = 0; r < G::R; r++) {
      float v = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < 4; w2++) v += red[((w2 * G::R + r) * 64 + lane) * 4 + wave];
      const int p = 16 * (4 * G::FT + r) + li;
      if (ch < Coutg && p < plane_out) {
        yg[ch * ch_stride + p * p_stride] = v + bw_;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fused_min_softmax_mfma4: Conv3d -> min over axis 0 -> softmax over channels
// for any geometry (the host permutes the axes for a minimum over H or W).
// One workgroup per (64-position tile of the (axis 1, axis 2) output plane,
// sample). The input box (every input plane the output depths read, the tile's
// rows) and the weights arrive by LDS DMA in one round of memory latency; the
// 4 waves share the output depths, each keeping running minima in registers.
// Groups are native: group g's outputs reduce over its own C_in/groups input
// channels only (no zero blocks), one group after the other. Matrix cores:
// 4x4x1 products with the weight operand broadcast from one 4-lane block, so a
// lane holds 4 channels of one position per product: 64 positions x 4
// channels per instruction.
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
  int kvol;
  int mode, dspan, rows, bw, boxc, row_tiles;
  int tile_pos;  // TILE_FLAT: consecutive output positions per tile (<= 64)
  int plane_out;
  // Element strides of x (per sample, per input channel, per spatial axis) and of
  // w (per kernel axis), in the kernel's axis order.
  int64_t xs_n, xs_c, xs0, xs1, xs2;
  int ws0, ws1, ws2;
  // Element strides of y per sample, per output channel and per output
  // position (y [N, C_out, positions] or channels-last [N, positions, C_out]).
  int64_t ys_n, ys_c, ys_p;
  int Cg, Coutg, groups;  // input / output channels per group, groups
  int cchunks;            // output-channel chunks per group (cpadg channels each, the last ragged)
  int kg;                 // reduction length of one group: Cg * kvol
  int kgp;                // kg rounded up to 4 (zero weights past kg)
  int kgs;                // floats per weight row in LDS (kgp, or kgp + 4 against bank conflicts)
  int cpadg;              // Coutg rounded up to 4: 4 * NG
  int nrows;              // input rows of the box: Cin * dspan * rows
  // LDS float offsets: koff (int per k), weights [group][channel][k], per-wave
  // minima of one group (0: in the box space), merged minima (groups > 1).
  int ko_off, wt_off, red_off, fin_off;
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
  extern __shared__ __align__(16) float smem[];
  float* Xs = smem;
  int* koff = reinterpret_cast<int*>(smem + a.ko_off);
  float* Wt = smem + a.wt_off;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x;
  const int n = blockIdx.y;

  int oh_first, oh_last, ow0 = 0, p0 = 0;
  if (a.mode == TILE_FLAT) {
    p0 = tile * a.tile_pos;
    const int p_last = min(p0 + a.tile_pos, a.plane_out) - 1;
    oh_first = p0 / a.O2;
    oh_last = p_last / a.O2;
  } else {
    oh_first = oh_last = tile / a.row_tiles;
    ow0 = (tile - oh_first * a.row_tiles) * 64;
  }
  const int iwb = ow0 * a.S2;
  const int ih0 = oh_first * a.S1 - a.P1;
  const int iw0 = iwb - a.P2;
  const int plane_stride = a.rows * a.bw;
  (void)oh_last;

  // Reduction offsets of one group's k (the group's first input channel at 0).
  for (int k = tid; k < a.kgp; k += 256) {
    int off = 0;
    if (k < a.kg) {
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

  // Box rows [channel][plane][row], one DMA per row and 64 columns; wave w
  // takes rows w, w+4, ... (row coordinates kept in scalar counters). No LDS
  // read while the copies are in flight.
  const float* x_n = a.x + int64_t(n) * a.xs_n;
  {
    int c = 0, zd = 0, zr = wave;
    while (zr >= a.rows) { zr -= a.rows; zd++; }
    for (int r = wave; r < a.nrows; r += 4) {
      while (zd >= a.dspan) { zd -= a.dspan; c++; }
      const int id = zd - a.P0;
      const int ih = ih0 + zr;
      const bool rv = (id >= 0) && (id < a.L0) && (ih >= 0) && (ih < a.L1);
      const float* src_row = x_n + c * a.xs_c + int64_t(rv ? id : 0) * a.xs0 + int64_t(rv ? ih : 0) * a.xs1;
      for (int col0 = 0; col0 < a.bw; col0 += 64) {
        const int col = col0 + lane;
        const int iw = iw0 + col;
        if (col < a.bw) {
          const bool ok = rv && iw >= 0 && iw < a.L2;
          lds_dma_f32(ok ? src_row + iw * a.xs2 : kZeroWord, Xs + r * a.bw + col0);
        }
      }
      zr += 4;
      while (zr >= a.rows) { zr -= a.rows; zd++; }
    }
  }
  // Weights [group][chunk][channel][k], rows of kgs floats; zero past kg and
  // past the group's Coutg channels.
  const int w_total = a.groups * a.cchunks * a.cpadg * a.kgs;
  const float inv_kgs = 1.0f / float(a.kgs), inv_cpadg = 1.0f / float(a.cpadg), inv_kvol = 1.0f / float(a.kvol);
  const float inv_k12 = 1.0f / float(a.K1 * a.K2), inv_k2 = 1.0f / float(a.K2);
  for (int i = wave; i * 64 < w_total; i += 4) {
    const int e = i * 64 + lane;
    if (e < w_total) {
      int k, c, cl, r, r2, th, tw;
      const int gc = divmod_small(e, a.kgs, inv_kgs, k);
      const int u = divmod_small(gc, a.cpadg, inv_cpadg, c);
      const int g = u / a.cchunks;
      c += (u - g * a.cchunks) * a.cpadg;  // channel within the group
      const bool ok = c < a.Coutg && k < a.kg;
      cl = divmod_small(ok ? k : 0, a.kvol, inv_kvol, r);
      const int td = divmod_small(r, a.K1 * a.K2, inv_k12, r2);
      th = divmod_small(r2, a.K2, inv_k2, tw);
      const float* src = a.w + (int64_t(g * a.Coutg + c) * a.Cg + cl) * a.kvol + td * a.ws0 + th * a.ws1 + tw * a.ws2;
      lds_dma_f32(ok ? src : kZeroWord, Wt + i * 64);
    }
  }
  wait_vmem_le<0>();
  __syncthreads();

  // This lane's output position.
  int oh, ow, valid;
  if (a.mode == TILE_FLAT) {
    const int p = p0 + lane;
    valid = lane < a.tile_pos && p < a.plane_out;
    oh = p / a.O2;
    ow = p - oh * a.O2;
  } else {
    oh = oh_first;
    ow = ow0 + lane;
    valid = ow < a.O2;
  }
  const int noff = valid ? (oh - oh_first) * a.S1 * a.bw + ow * a.S2 - iwb : 0;
  const int wlane = min(lane, a.cpadg - 1);
  const int nq = a.kgp >> 2;
  const int4* koff4 = reinterpret_cast<const int4*>(koff);
  const bool red_overlaps_box = a.red_off == 0;
  float* red = smem + a.red_off;
  float* fin = smem + a.fin_off;
  float* yp = a.y + int64_t(n) * a.ys_n + (int64_t(oh) * a.O2 + ow) * a.ys_p;

  const int units = a.groups * a.cchunks;
  for (int u = 0; u < units; u++) {
    const int g = u / a.cchunks;                    // conv group
    const int cbase = (u - g * a.cchunks) * a.cpadg;  // first channel of the chunk within the group
    const float4* wrow = reinterpret_cast<const float4*>(Wt + (u * a.cpadg + wlane) * a.kgs);
    const float* xg = Xs + g * a.Cg * a.boxc + noff;
    v4f mn[NG];
#pragma unroll
    for (int i = 0; i < NG; i++) mn[i] = v4f{INFINITY, INFINITY, INFINITY, INFINITY};
    for (int od = wave; od < a.O0; od += 4) {
      const float* xb = xg + od * a.S0 * plane_stride;
      v4f acc[NG];
#pragma unroll
      for (int i = 0; i < NG; i++) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
      // Software pipeline over k-quads, unrolled by two with operand sets A
      // (even quads) and B (odd quads): a set's LDS reads are issued while the
      // other set feeds the products, offsets one quad further ahead. Indices
      // past the last quad are clamped (in-bounds reads, never used).
      const int last = nq - 1;
      int4 koA = koff4[0];
      int4 koB = koff4[min(1, last)];
      float4 wA = wrow[0];
      float a0 = xb[koA.x], a1 = xb[koA.y], a2 = xb[koA.z], a3 = xb[koA.w];
      koA = koff4[min(2, last)];
      asm volatile("" ::: "memory");
      for (int q = 0; q < nq; q += 2) {
        const float4 wB = wrow[min(q + 1, last)];
        const float c0 = xb[koB.x], c1 = xb[koB.y], c2 = xb[koB.z], c3 = xb[koB.w];
        koB = koff4[min(q + 3, last)];
        mfma4_all<NG>(wA.x, a0, acc, std::make_integer_sequence<int, NG>{});
        mfma4_all<NG>(wA.y, a1, acc, std::make_integer_sequence<int, NG>{});
        mfma4_all<NG>(wA.z, a2, acc, std::make_integer_sequence<int, NG>{});
        mfma4_all<NG>(wA.w, a3, acc, std::make_integer_sequence<int, NG>{});
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * NG, 0);
        asm volatile("" ::: "memory");
        if (q + 1 < nq) {
          wA = wrow[min(q + 2, last)];
          a0 = xb[koA.x]; a1 = xb[koA.y]; a2 = xb[koA.z]; a3 = xb[koA.w];
          koA = koff4[min(q + 4, last)];
          mfma4_all<NG>(wB.x, c0, acc, std::make_integer_sequence<int, NG>{});
          mfma4_all<NG>(wB.y, c1, acc, std::make_integer_sequence<int, NG>{});
          mfma4_all<NG>(wB.z, c2, acc, std::make_integer_sequence<int, NG>{});
          mfma4_all<NG>(wB.w, c3, acc, std::make_integer_sequence<int, NG>{});
          __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 4 * NG, 0);
        }
        asm volatile("" ::: "memory");
      }
#pragma unroll
      for (int i = 0; i < NG; i++) {
        mn[i][0] = min_nan(mn[i][0], acc[i][0]);
        mn[i][1] = min_nan(mn[i][1], acc[i][1]);
        mn[i][2] = min_nan(mn[i][2], acc[i][2]);
        mn[i][3] = min_nan(mn[i][3], acc[i][3]);
      }
    }
    // Merge the four waves' minima of this group through LDS.
    if (red_overlaps_box) __syncthreads();  // the box is read for the last time above
#pragma unroll
    for (int i = 0; i < NG; i++)
#pragma unroll
      for (int r = 0; r < 4; r++) red[(wave * a.cpadg + 4 * i + r) * 64 + lane] = mn[i][r];
    __syncthreads();
    if (units == 1) {
      // One group: wave 0 merges and normalises in registers.
      if (wave == 0 && valid) {
        float m[4 * NG];
#pragma unroll
        for (int c = 0; c < 4 * NG; c++) {
          float v = red[c * 64 + lane];
          v = min_nan(v, red[(a.cpadg + c) * 64 + lane]);
          v = min_nan(v, red[(2 * a.cpadg + c) * 64 + lane]);
          v = min_nan(v, red[(3 * a.cpadg + c) * 64 + lane]);
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
#pragma unroll
        for (int c = 0; c < 4 * NG; c++)
          if (c < a.Cout) yp[int64_t(c) * a.ys_c] = m[c] * inv_den;
      }
      return;
    }
    // Several groups: the waves merge a quarter of the group's channels each
    // into fin[channel][position], then free red for the next group.
    for (int c = wave; c < a.cpadg && cbase + c < a.Coutg; c += 4) {
      float v = red[c * 64 + lane];
      v = min_nan(v, red[(a.cpadg + c) * 64 + lane]);
      v = min_nan(v, red[(2 * a.cpadg + c) * 64 + lane]);
      v = min_nan(v, red[(3 * a.cpadg + c) * 64 + lane]);
      const int co = g * a.Coutg + cbase + c;
      fin[co * 64 + lane] = v + (a.bias ? a.bias[co] : 0.0f);
    }
    __syncthreads();
  }
  // Softmax over all channels, in channel order (wave 0, one lane per position).
  if (wave == 0 && valid) {
    float mx = -INFINITY;
    for (int c = 0; c < a.Cout; c++) mx = fmaxf(mx, fin[c * 64 + lane]);
    float sum = 0.0f;
    for (int c = 0; c < a.Cout; c++) sum += expf(fin[c * 64 + lane] - mx);
    const float inv_den = 1.0f / sum;
    for (int c = 0; c < a.Cout; c++) yp[int64_t(c) * a.ys_c] = expf(fin[c * 64 + lane] - mx) * inv_den;
  }
}

// ---------------------------------------------------------------------------
// fused_stream: Conv3d -> min over depth -> softmax over channels for a fixed
// small geometry (stride 1, dilation 1, groups 1, kD = 3), streaming the input
// depth planes through LDS.
// - One wave owns a tile of output positions (h, w) of one sample and a
//   contiguous range of output depths (the depth range is split over DSPLIT
//   waves); the waves of a workgroup are independent (no barriers). A tile is
//   RT whole output rows (lanes past RT * W_out idle), so lane l reads staged
//   row l / W_out at column l % W_out and the 64 operand reads of one wave fall
//   on distinct LDS banks; or, with RT = 0, 64 consecutive positions of the
//   flattened plane.
// - Output depth od reads input planes od, od+1, od+2; planes sit in a ring of
//   four LDS slots and the plane three ahead is copied while od is reduced.
// - Matrix core: 4x4x1 MFMA with 16 blocks, the weight operand broadcast from
//   one block (cbsz 4, abid b): lane l accumulates channels 4g..4g+3 of position
//   l, so C_out is covered in steps of 4 channels with no padding, and every
//   weight (channel group, reduction index) pair sits in one of 16 lane quads of
//   a resident register.
// - The depth minimum, bias, and the softmax over all channels stay inside the
//   lane: nothing of the conv result leaves the registers. With DSPLIT > 1 the
//   partial minima of the depth ranges meet in LDS first.
// ---------------------------------------------------------------------------

template <int CIN, int KH, int KW_, int NG, int O2, int ROWS, int RT, int GRP, int E4>
struct StreamGeo {
  static constexpr int CIN_ = CIN, NG_ = NG, O2_ = O2, KW = KW_;
  // Conv groups: a channel block of group gq reduces over input channels
  // gq*CG .. gq*CG + CG - 1 only; NQG blocks per group.
  static constexpr int GRP_ = GRP, CG = CIN / GRP, NQG = NG / GRP;
  static_assert(CIN % GRP == 0 && NG % GRP == 0, "whole channel blocks per group");
  static constexpr int RT_ = RT;  // > 0: a wave tile is RT whole output rows; 0: 64 flattened positions
  static_assert(RT * O2 <= 64, "a row tile fits the wave");
  static constexpr int KD = 3;
  static constexpr int BW = O2 + KW_ - 1;       // input columns per staged row
  static constexpr int CH = ROWS * BW;           // floats per channel of a plane
  static constexpr int PLANE = CIN * CH;         // floats of one staged plane
  // Floats per copy: 4 (16-byte chunks along contiguous rows) or 1 (E4: one
  // element per lane, the column axis strided).
  static constexpr int UNIT = E4 ? 1 : 4;
  static_assert(BW % UNIT == 0, "rows are copied in whole chunks");
  static constexpr int CHUNKS = PLANE / UNIT;    // copies' elements per plane
  static constexpr int PI = (CHUNKS + 63) / 64;  // 64-lane copies per plane (the last one partial)
  static constexpr int SLOT = PLANE;
  static constexpr int NSLOT = 4;
  static constexpr int KHW = KH * KW_;
  static constexpr int KVOL = KD * KHW;
  static constexpr int KRED = CIN * KVOL;
  static constexpr int KREDG = CG * KVOL;        // reduction length of one output channel
  static constexpr int NT = CIN * KHW;           // staged values read per plane
  // With 16 or more output channels, channels 0..15 run on the 16x16x1 4-block
  // form (A broadcast from one block: one instruction per input value) and the
  // rest on the 4x4x1 16-block form; else every channel on the 4x4x1 form.
  static constexpr bool MIX = NG >= 4 && GRP == 1;
  static constexpr int NA16 = (KRED + 3) / 4;     // 16x16 weights: register j holds k = 4j .. 4j+3
  static constexpr int NG4 = MIX ? NG - 4 : NG;   // 4-channel groups on the 4x4x1 form
  static constexpr int CO4 = MIX ? 16 : 0;        // their first channel
  static constexpr int NPAIR = NG4 * KREDG;       // (channel block, reduction index) pairs
  static constexpr int NAREG = (NPAIR + 15) / 16;
  static constexpr int WAVES = 4;                // waves per workgroup
  // The rings; after the depth loop (depth range split over waves) the partial
  // minima, 4*NG registers per wave, and past them one 1024-float channel
  // transpose area per (sample, tile).
  static constexpr int RING_FLOATS = WAVES * NSLOT * SLOT;
  static constexpr int EPI_FLOATS = 4 * NG * 64 * WAVES + WAVES * 1024;
  static constexpr int LDS_FLOATS = RING_FLOATS > EPI_FLOATS ? RING_FLOATS : EPI_FLOATS;
  static_assert(NSLOT * SLOT >= 1024, "an undivided depth range transposes in its own ring");
  static_assert(PI < 64, "vmcnt range");
};

struct StreamArgs {
  const float* __restrict__ x;
  const float* __restrict__ w;
  const float* __restrict__ bias;
  float* __restrict__ y;
  int Cout;
  int L0, L1, L2;
  int P0, P1, P2;
  int O0, O1;
  int plane_out;
  int tiles_per_plane;
  int dsplit;      // waves per (sample, tile): the depth range is split over them
  int ods;         // output depths per wave (the last range may be shorter)
  int units;       // N * tiles_per_plane * dsplit
  // Element strides of x and of w along the kernel's axes 0, 1 and 2 (the
  // streamed, row and column axes): the host permutes D, H and W so that the
  // min axis is streamed.
  int plane_stride, row_stride, col_stride;
  int ws0, ws1, ws2;
  // Element strides of x per sample and per input channel, and of y per
  // sample, output channel and output position (NCDHW or channels-last).
  int64_t xs_n, ys_n;
  int xs_c, ys_c, ys_p;
};

// Index in w's [C_in, kD, kH, kW] block of reduction index k = (c, axis-0
// tap, axis-1 tap, axis-2 tap) in the kernel's axis order (k < KRED).
template <class G>
__device__ __forceinline__ int stream_widx(int k, const StreamArgs& a) {
  const int c = k / G::KVOL, r = k - c * G::KVOL;
  const int t0 = r / G::KHW, r2 = r - t0 * G::KHW;
  const int t1 = r2 / G::KW, t2 = r2 - t1 * G::KW;
  return c * G::KVOL + t0 * a.ws0 + t1 * a.ws1 + t2 * a.ws2;
}

template <class G>
__global__ __launch_bounds__(256, 4) void fused_stream_kernel(StreamArgs a) {
  constexpr int NG = G::NG_;
  __shared__ __align__(16) float smem[G::LDS_FLOATS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Waves of one (sample, tile) are consecutive units, so they share a workgroup
  // when dsplit divides the workgroup's wave count. Workgroups are dispatched
  // round-robin over the 8 XCDs: give each XCD a contiguous run of workgroups so
  // the input rows that neighbouring tiles share are fetched into one L2.
  int blk = blockIdx.x;
  if ((gridDim.x & 7) == 0) blk = (blk & 7) * (gridDim.x >> 3) + (blk >> 3);
  const int unit = blk * G::WAVES + wave;
  const bool live = unit < a.units;
  const int tu = unit / a.dsplit;
  const int part = unit - tu * a.dsplit;
  const int n = tu / a.tiles_per_plane;
  const int tile = tu - n * a.tiles_per_plane;
  // First output row of the tile and this lane's output position.
  const int oh_first = G::RT_ > 0 ? tile * G::RT_ : (tile * 64) / G::O2_;
  const int oh = G::RT_ > 0 ? oh_first + lane / G::O2_ : (tile * 64 + lane) / G::O2_;
  const int ow = G::RT_ > 0 ? lane - (lane / G::O2_) * G::O2_ : (tile * 64 + lane) - ((tile * 64 + lane) / G::O2_) * G::O2_;
  const int od0 = part * a.ods;
  const int od1 = live ? min(a.O0, od0 + a.ods) : od0;
  float* ring = smem + wave * (G::NSLOT * G::SLOT);

  // Weights of the 4x4x1 form: register r, lane 4b + i holds w[CO4 + 4q + i][k]
  // for pair 16r + b = q * KREDG + k (k within the block's group).
  float aw[G::NAREG];
#pragma unroll
  for (int r = 0; r < G::NAREG; r++) {
    const int pair = 16 * r + (lane >> 2);
    const int gq = pair / G::KREDG, k = pair - gq * G::KREDG;
    const int co = G::CO4 + 4 * gq + (lane & 3);
    aw[r] = (live && pair < G::NPAIR && co < a.Cout) ? a.w[co * G::KREDG + stream_widx<G>(k, a)] : 0.0f;
  }
  // Weights of the 16x16x1 form: register j, lane 16b + m holds w[m][4j + b].
  float a16[G::MIX ? G::NA16 : 1];
  if constexpr (G::MIX) {
#pragma unroll
    for (int j = 0; j < G::NA16; j++) {
      const int k = 4 * j + (lane >> 4), m = lane & 15;
      a16[j] = (live && k < G::KRED && m < a.Cout) ? a.w[m * G::KRED + stream_widx<G>(k, a)] : 0.0f;
    }
  }

  // Copy sources: copy i, lane l moves element e = 64i + l = (c, row, q) of the
  // slot (UNIT floats: 16 bytes, or 4 with E4) from input (c, ih0 + row,
  // columns UNIT*q ..) of the plane being staged (input rows are exactly BW
  // wide: no padding along the column axis).
  const int ih0 = oh_first - a.P1;
  const int chan_stride = a.xs_c;
  const float* xn = a.x + int64_t(n) * a.xs_n;
  int soff[G::PI];
  uint32_t sok = 0;
#pragma unroll
  for (int i = 0; i < G::PI; i++) {
    const int e = 64 * i + lane;
    const int c = e / (G::CH / G::UNIT), rem = e - c * (G::CH / G::UNIT);
    const int r = rem / (G::BW / G::UNIT), q = rem - r * (G::BW / G::UNIT);
    const int ih = ih0 + r;
    const bool ok = unsigned(ih) < unsigned(a.L1);
    soff[i] = ok ? int(c * chan_stride) + ih * a.row_stride + G::UNIT * q * a.col_stride : 0;
    sok |= uint32_t(ok) << i;
  }
  // Pinned in a scalar register: a kernel-argument load inside the depth loop
  // would come with a wait that drains the LDS reads in flight.
  int plane_elems = a.plane_stride;
  pin_sgpr(plane_elems);
  // Plane z (input depth z - P0) -> slot z % 4. Planes past od1 + 1 are copied
  // as zeros so every wave issues the same number of copies per step; lanes
  // past the plane's last chunk copy nothing.
  auto stage = [&](int z) {
    const int id = z - a.P0;
    const bool pok = live && (z < od1 + G::KD - 1) && unsigned(id) < unsigned(a.L0);
    const float* xp = xn + int64_t(pok ? id : 0) * plane_elems;
    float* dst = ring + (z & 3) * G::SLOT;
#pragma unroll
    for (int i = 0; i < G::PI; i++) {
      const bool ok = pok && ((sok >> i) & 1);
      if (64 * i + lane < G::CHUNKS) {
        if constexpr (G::UNIT == 4) lds_dma_f32x4(ok ? xp + soff[i] : kZeroWord, dst + 256 * i);
        else lds_dma_f32(ok ? xp + soff[i] : kZeroWord, dst + 64 * i);
      }
    }
  };

  // This lane's output position and its byte offset inside a slot.
  const int p = oh * G::O2_ + ow;
  const bool valid = live && (G::RT_ > 0 ? (lane < G::RT_ * G::O2_ && oh < a.O1) : p < a.plane_out);
  const int lbase = valid ? (oh - oh_first) * G::BW + ow : 0;
  const char* bbase = reinterpret_cast<const char*>(ring + lbase);

  v4f mn[NG];
#pragma unroll
  for (int q = 0; q < NG; q++) mn[q] = v4f{INFINITY, INFINITY, INFINITY, INFINITY};

  stage(od0);
  stage(od0 + 1);
  stage(od0 + 2);
  wait_vmem_le<3 * G::PI>();  // the weights (loaded before the copies)
  for (int od = od0; od < od1; od++) {
    // Plane od + 3 goes into the slot plane od - 1 used, once those reads have
    // returned; then planes od .. od + 2 are complete.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    stage(od + 3);
    wait_vmem_le<G::PI>();
    asm volatile("" ::: "memory");
    // Reduction in groups of one (depth tap, channel): the KH*KW staged values
    // of group g+1 are read while the matrix core works through group g.
    constexpr int NGRP = G::KD * G::CIN_;
    const char* bps[G::KD];
#pragma unroll
    for (int kd = 0; kd < G::KD; kd++) bps[kd] = bbase + ((od + kd) & 3) * (4 * G::SLOT);
    float bv[2][G::KHW];
    auto load_group = [&](auto GG, float* dst) {
      constexpr int g = decltype(GG)::value;
      constexpr int kd = g / G::CIN_, c = g % G::CIN_;
      static_for<G::KHW>([&](auto HH) {
        constexpr int hw = decltype(HH)::value;
        constexpr int kh = hw / G::KW, kw = hw % G::KW;
        dst[hw] = *reinterpret_cast<const float*>(bps[kd] + 4 * (c * G::CH + kh * G::BW + kw));
      });
    };
    load_group(std::integral_constant<int, 0>{}, bv[0]);
    v4f acc[G::NG4];
    v16f acc16;
    static_for<NGRP>([&](auto GG) {
      constexpr int g = decltype(GG)::value;
      constexpr int kd = g / G::CIN_, c = g % G::CIN_;
      constexpr int cur = g & 1;
      // Issue the next group's reads, then this group's products (the barriers
      // keep the scheduler from sinking the reads next to their uses).
      if constexpr (g + 1 < NGRP) load_group(std::integral_constant<int, g + 1>{}, bv[cur ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
      static_for<G::KHW>([&](auto HH) {
        constexpr int hw = decltype(HH)::value;
        constexpr int k = c * G::KVOL + kd * G::KHW + hw;
        if constexpr (G::MIX) {
          if constexpr (g == 0 && hw == 0)
            acc16 = __builtin_amdgcn_mfma_f32_16x16x1f32(a16[k / 4], bv[cur][hw], v16f{}, 2, k % 4, 0);
          else
            acc16 = __builtin_amdgcn_mfma_f32_16x16x1f32(a16[k / 4], bv[cur][hw], acc16, 2, k % 4, 0);
        }
        static_for<G::NG4>([&](auto QQ) {
          constexpr int q = decltype(QQ)::value;
          // Only the blocks of input channel c's group (all of them without groups).
          if constexpr (G::GRP_ == 1 || q / G::NQG == c / G::CG) {
            constexpr int pair = q * G::KREDG + (k - (c / G::CG) * G::CG * G::KVOL);
            constexpr int r = pair / 16, ab = pair % 16;
            if constexpr (kd == 0 && c % G::CG == 0 && hw == 0)
              acc[q] = __builtin_amdgcn_mfma_f32_4x4x1f32(aw[r], bv[cur][hw], v4f{0.f, 0.f, 0.f, 0.f}, 4, ab, 0);
            else
              acc[q] = __builtin_amdgcn_mfma_f32_4x4x1f32(aw[r], bv[cur][hw], acc[q], 4, ab, 0);
          }
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    // Running minimum, NaN-propagating like torch.min.
    // mn[q], q < 4 (16x16x1 form): registers 4q .. 4q+3 of its output, lane l
    // holding channel 4(l/16) + i of position 16q + l%16; mn[q] otherwise: the
    // 4x4x1 form, lane l holding channel 4q + i of position l.
#pragma unroll
    for (int q = 0; q < NG; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float v;
        if constexpr (G::MIX) v = q < 4 ? acc16[4 * q + i] : acc[q < 4 ? 0 : q - 4][i];
        else v = acc[q][i];
        mn[q][i] = min_nan(mn[q][i], v);
      }
  }

  float* yp = a.y + int64_t(n) * a.ys_n + int64_t(p) * a.ys_p;
  if (a.dsplit > 1) {
    // The parts of one (sample, tile) are consecutive waves of this workgroup:
    // part 0 takes the minimum over the others' partial minima. The ring is
    // reused once every wave's last (zero) copies have landed.
    wait_vmem_le<0>();
    __syncthreads();
    float* red = smem;
#pragma unroll
    for (int q = 0; q < NG; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) red[((wave * NG + q) * 4 + i) * 64 + lane] = mn[q][i];
    __syncthreads();
    if (part != 0) return;
    for (int o = 1; o < a.dsplit; o++)
#pragma unroll
      for (int q = 0; q < NG; q++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float v = red[(((wave + o) * NG + q) * 4 + i) * 64 + lane];
          mn[q][i] = min_nan(mn[q][i], v);
        }
  }

  // Channels 0..15 of the 16x16x1 form: through LDS to the lane of their
  // position. The region lies past the partial-minimum slots and is this
  // wave's own (every copy into the rings has landed).
  float m[4 * NG];
  if constexpr (G::MIX) {
    if (a.dsplit == 1) wait_vmem_le<0>();
    float* xch = a.dsplit > 1 ? smem + 4 * NG * 64 * G::WAVES + (wave / a.dsplit) * 1024 : ring;
#pragma unroll
    for (int q = 0; q < 4; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) xch[(4 * (lane >> 4) + i) * 64 + 16 * q + (lane & 15)] = mn[q][i];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's writes are done
#pragma unroll
    for (int c = 0; c < 16; c++) m[c] = xch[c * 64 + lane];
  } else {
#pragma unroll
    for (int q = 0; q < 4 && q < NG; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) m[4 * q + i] = mn[q][i];
  }
#pragma unroll
  for (int q = 4; q < NG; q++)
#pragma unroll
    for (int i = 0; i < 4; i++) m[4 * q + i] = mn[q][i];

  // Softmax over the channels of this lane's position. fp32 addition is
  // monotone, so adding the bias after the minimum equals adding it before.
  if (valid) {
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4 * NG; c++) {
      m[c] = c < a.Cout ? m[c] + (a.bias ? a.bias[c] : 0.0f) : -INFINITY;
      mx = fmaxf(mx, m[c]);
    }
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < 4 * NG; c++) {
      const float e = c < a.Cout ? expf(m[c] - mx) : 0.0f;
      m[c] = e;
      sum += e;
    }
    const float inv = 1.0f / sum;
#pragma unroll
    for (int c = 0; c < 4 * NG; c++)
      if (c < a.Cout) yp[int64_t(c) * a.ys_c] = m[c] * inv;
  }
}

// ---------------------------------------------------------------------------
// Calibration probes: the fp32 rates this chip reaches in practice, against
// which measured kernels are also reported (not part of the operation).
// - peak_mfma_kernel: each wave keeps 8 independent 16x16x4 fp32 MFMA
//   accumulation chains busy (each accumulator is reused 8 instructions later,
//   far past the instruction's latency).
// - peak_fma_kernel: each lane keeps 8 independent fp32 FMA chains (plain
//   v_fma_f32; the library is compiled without packed fp32).
// The results stay in registers; a store that no input can trigger keeps them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void peak_mfma_kernel(int64_t iters, float* __restrict__ sink) {
  const float av = 1.0f + 1e-7f * float(threadIdx.x), bv = 1.0f - 1e-7f * float(threadIdx.x);
  v4f acc[8];
#pragma unroll
  for (int j = 0; j < 8; j++) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int64_t i = 0; i < iters; i++) {
#pragma unroll
    for (int j = 0; j < 8; j++) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[j], 0, 0, 0);
  }
  float t = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; j++) t += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (t < 0.0f) sink[0] = t;  // every product is positive
}

__global__ __launch_bounds__(256) void peak_fma_kernel(int64_t iters, float* __restrict__ sink) {
  const float m = 0.999999f, c = 1e-6f * float(threadIdx.x & 7);
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; j++) v[j] = 1.0f + 0.125f * float(j);
  for (int64_t i = 0; i < iters; i++) {
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = __builtin_fmaf(v[j], m, c);
  }
  float t = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; j++) t += v[j];
  if (t < 0.0f) sink[0] = t;  // every chain stays positive
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

template <typename Fn>
static int set_lds_limit_once(Fn fn, std::once_flag& once, hipError_t& err) {
  std::call_once(once, [&] {
    err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                              int(kLdsLimit));
  });
  return err == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

template <int MT, int NT, int WM, int WN, int KS, bool CL = false>
static int launch_conv_cfg(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  static std::once_flag once;
  static hipError_t err = hipSuccess;
  auto fn = conv_mfma16_kernel<MT, NT, WM, WN, KS, CL>;
  if (set_lds_limit_once(fn, once, err) != CONV_OK) return CONV_ERR_HIP;
  dim3 grid(unsigned(p.grid[0]), unsigned(p.grid[1]), unsigned(p.grid[2]));
  hipLaunchKernelGGL(fn, grid, dim3(256), size_t(p.lds_bytes), stream, args);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

template <int MT, int NT, int WM, int WN, int NCH, class G>
static int launch_tap_geo(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  auto fn = conv_tap_kernel<MT, NT, WM, WN, NCH, G>;
  static_assert(4 * G::template lds_floats<NCH, WM, MT>() <= kLdsLimit, "tap specialisation exceeds LDS");
  if (4 * int64_t(G::template lds_floats<NCH, WM, MT>()) != p.lds_bytes) return CONV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(fn, dim3(unsigned(p.grid[0])), dim3(64 * WM * WN), 0, stream, args);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

template <int MT, int NT, int WM, int WN, int NCH, int KD, int KH, int KW, int DD, int DH, int DW, int CC, int KDSPAN,
          int ROWS, int BW>
static int launch_tap(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  return launch_tap_geo<MT, NT, WM, WN, NCH, TapGeo<KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW>>(args, p, stream);
}

static int launch_tap_cl_spec(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  switch (p.tap_spec) {
#define CONVHIP_TAP_CL_CASE(id, MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW, CCP)            \
  case id:                                                                                                       \
    return launch_tap_geo<MT, NT, WM, WN, NCH, TapGeoCL<KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW, CCP>>(args, p, \
                                                                                                           stream);
    CONVHIP_TAP_CL_SPECS(CONVHIP_TAP_CL_CASE)
#undef CONVHIP_TAP_CL_CASE
    default: return CONV_ERR_UNSUPPORTED;
  }
}

// Polls of the batch-1 counter before a wave of conv_tap_split_pipe gives up
// (and stores NaN for its tile): 2^22 (seconds; the waves of a workgroup are
// co-resident, so it is never reached), or CONVHIP_SPIN_CAP for tests that
// force the give-up path from the host.
static int split_spin_cap() {
  const char* s = std::getenv("CONVHIP_SPIN_CAP");
  if (!s || !*s) return 1 << 22;
  const long v = std::atol(s);
  return v < 0 ? 0 : (v > (1 << 22) ? (1 << 22) : int(v));
}

// Kernel family for the geometries the channel-split specialisations serve:
// unset = the planner's choice (the stream-K kernel where a specialisation
// fits, else the pipelined channel-split kernel); CONVHIP_SPLIT_PIPE=1 forces
// the pipelined channel-split kernel, =0 the one whose cross-wave sum follows
// all products (tests and A/B timings run each).
// CONVHIP_VALU=1: conv_fwd runs the vector-ALU direct kernel wherever it fits
// (for measuring it against the matrix-core kernels, and for its tests).
static bool force_valu() {
  const char* s = std::getenv("CONVHIP_VALU");
  return s && *s && std::atoi(s) != 0;
}

static int split_kernel_choice() {
  const char* s = std::getenv("CONVHIP_SPLIT_PIPE");
  if (!s || !*s) return 0;
  return std::atoi(s) ? 1 : 2;
}

template <int NT, int NW, int KD, int KH, int KW, int DD, int DH, int DW, int F, int ROWS, int BW, bool CL>
static int launch_split(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  using G = SplitGeo<KD, KH, KW, DD, DH, DW, F, ROWS, BW, NW>;
  const dim3 grid(unsigned(p.grid[0]), unsigned(p.grid[1]), unsigned(p.grid[2]));
  if constexpr (split_pipe_fits(NT, NW, G::WROW)) {
    if (p.split_pipe) {
      hipLaunchKernelGGL((conv_tap_split_pipe_kernel<(NT + 1) / 2, NT / 2, NW, G, CL>), grid, dim3(64 * NW), 0,
                         stream, args);
      return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
    }
  }
  hipLaunchKernelGGL((conv_tap_split_kernel<NT, NW, G, CL>), grid, dim3(64 * NW), 0, stream, args);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

template <bool CL>
static int launch_split_spec(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  switch (p.split_spec) {
#define CONVHIP_SPLIT_CASE(id, NT, NW, KD, KH, KW, DD, DH, DW, F, ROWS, BW, TS) \
  case id:                                                                  \
    return launch_split<NT, NW, KD, KH, KW, DD, DH, DW, F, ROWS, BW, CL>(args, p, stream);
    CONVHIP_SPLIT_SPECS(CONVHIP_SPLIT_CASE)
#undef CONVHIP_SPLIT_CASE
    default: return CONV_ERR_UNSUPPORTED;
  }
}

template <int CG, int KD, int KH, int KW, int DH, int DW, int F, int ROWS, int BW, int T, bool CL>
static int launch_kstream(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  using G = KsGeo<CG, KD, KH, KW, DH, DW, F, ROWS, BW, T, CL>;
  static_assert(4 * G::LDS <= kLdsLimit, "stream-K specialisation exceeds LDS");
  if (int64_t(4) * G::LDS != p.lds_bytes) return CONV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((conv_tap_kstream_kernel<G, CL>), dim3(unsigned(p.grid[0])), dim3(512), 0, stream, args);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

template <bool CL>
static int launch_ks_spec(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  switch (p.ks_spec) {
#define CONVHIP_KS_CASE(id, CG, KD, KH, KW, DH, DW, F, ROWS, BW, T) \
  case id:                                                        \
    return launch_kstream<CG, KD, KH, KW, DH, DW, F, ROWS, BW, T, CL>(args, p, stream);
    CONVHIP_KSTREAM_SPECS(CONVHIP_KS_CASE)
#undef CONVHIP_KS_CASE
    default: return CONV_ERR_UNSUPPORTED;
  }
}

template <int CIN, int KD, int KH, int KW, int DD, int DH, int DW, bool CL>
static int launch_direct(const ConvArgs& c, const ConvPlan& p, hipStream_t stream) {
  DirectArgs a;
  a.x = c.x; a.w = c.w; a.bias = c.bias; a.y = c.y;
  a.sw = CL ? c.Cin : 1;
  a.sh = c.L2 * a.sw;
  a.sd = c.L1 * a.sh;
  a.sc = CL ? 1 : c.L0 * a.sd;
  a.sn = c.L0 * c.L1 * c.L2 * c.Cin;
  a.ssd = c.S0 * a.sd; a.ssh = c.S1 * a.sh; a.ssw = c.S2 * a.sw;
  a.sg = CIN * a.sc;
  a.O0 = c.O0; a.O1 = c.O1; a.O2 = c.O2;
  a.npos = int(p.items);
  a.r0 = 1.0f / float(c.O0); a.r1 = 1.0f / float(c.O1); a.r2 = 1.0f / float(c.O2);
  a.Cout = c.Cout; a.Coutg = c.Coutg;
  hipLaunchKernelGGL((conv_direct16_kernel<DirectGeo<CIN, KD, KH, KW, DD, DH, DW>, CL>),
                     dim3(unsigned(p.grid[0]), unsigned(p.grid[1])), dim3(64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

template <bool CL>
static int launch_direct_spec(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  switch (p.direct_spec) {
#define CONVHIP_DIRECT_CASE(id, CIN, KD, KH, KW, DD, DH, DW) \
  case id:                                                 \
    return launch_direct<CIN, KD, KH, KW, DD, DH, DW, CL>(args, p, stream);
    CONVHIP_DIRECT_SPECS(CONVHIP_DIRECT_CASE)
#undef CONVHIP_DIRECT_CASE
    default: return CONV_ERR_UNSUPPORTED;
  }
}

static int launch_tap_spec(const ConvArgs& args, const ConvPlan& p, hipStream_t stream) {
  switch (p.tap_spec) {
#define CONVHIP_TAP_CASE(id, MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW) \
  case id:                                                                                        \
    return launch_tap<MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW>(args, p, stream);
    CONVHIP_TAP_SPECS(CONVHIP_TAP_CASE)
#undef CONVHIP_TAP_CASE
    default: return CONV_ERR_UNSUPPORTED;
  }
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

template <int CIN, int KH, int KW, int NG, int O2, int ROWS, int RT, int GRP, int E4>
static int launch_stream(const StreamArgs& args, const FusedPlan& p, hipStream_t stream) {
  using G = StreamGeo<CIN, KH, KW, NG, O2, ROWS, RT, GRP, E4>;
  if (int64_t(4) * G::LDS_FLOATS != p.lds_bytes || G::WAVES % p.dsplit != 0) return CONV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(fused_stream_kernel<G>, dim3(unsigned(p.grid[0])), dim3(64 * G::WAVES), 0, stream, args);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

static int launch_stream_spec(const StreamArgs& args, const FusedPlan& p, hipStream_t stream) {
  switch (p.spec) {
#define CONVHIP_FUSED_CASE(id, CIN, KH, KW, NG, O2, ROWS, RT, GRP, E4) \
  case id:                                                           \
    return launch_stream<CIN, KH, KW, NG, O2, ROWS, RT, GRP, E4>(args, p, stream);
    CONVHIP_FUSED_SPECS(CONVHIP_FUSED_CASE)
#undef CONVHIP_FUSED_CASE
    default: return CONV_ERR_UNSUPPORTED;
  }
}

// The generic implicit-GEMM kernel in the plan's tile configuration.
template <bool CL>
static int launch_generic(const ConvArgs& a, const ConvPlan& p, hipStream_t s) {
  switch (p.cfg) {
    case CFG_M64: return launch_conv_cfg<4, 4, 1, 4, 1, CL>(a, p, s);
    case CFG_M128: return launch_conv_cfg<4, 4, 2, 2, 1, CL>(a, p, s);
    case CFG_M32: return launch_conv_cfg<2, 4, 1, 4, 1, CL>(a, p, s);
    case CFG_M16: return launch_conv_cfg<1, 4, 1, 4, 1, CL>(a, p, s);
    case CFG_M16_N64_K4: return launch_conv_cfg<1, 4, 1, 1, 4, CL>(a, p, s);
    case CFG_M16_N128_K4: return launch_conv_cfg<1, 8, 1, 1, 4, CL>(a, p, s);
    case CFG_M16_N208_K4: return launch_conv_cfg<1, 13, 1, 1, 4, CL>(a, p, s);
    default: return launch_conv_cfg<1, 16, 1, 1, 4, CL>(a, p, s);
  }
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
  a.mode = p.mode; a.Cc = p.Cc; a.kc_pad = p.kc_pad; a.kdspan = p.kdspan;
  a.xs_floats = p.xs_floats; a.koff_ints = p.koff_ints; a.ws_floats = p.ws_floats;
  a.tiles_per_plane = int(p.tiles_per_plane); a.nchunks = p.nchunks; a.items = int(p.items);
  a.rows = p.rows; a.bw = p.bw; a.boxc = p.boxc; a.row_tiles = p.row_tiles; a.ctiles = p.ctiles;
  a.plane_out = int(g.plane_out());
  a.ccp = p.ccp;
  a.cl_vec = p.cl_vec ? 1 : 0;
  a.vec_store = 0;
  a.spin_cap = split_spin_cap();
  return a;
}

}  // namespace convhip

using namespace convhip;

// CONVHIP_CONV_CFG=<n> forces tile configuration n of conv_fwd (used by the tests
// to run every configuration on every case); unset or out of range = planner's choice.
static int forced_conv_cfg() {
  const char* s = std::getenv("CONVHIP_CONV_CFG");
  if (!s || !*s) return -1;
  const int v = std::atoi(s);
  return (v >= 0 && v < CFG_COUNT) ? v : -1;
}

// CONVHIP_TAP=0 keeps conv_fwd, conv_fwd_channels_last and conv3d_min_softmax off the build-time
// specialised kernels.
static int use_tap() {
  const char* s = std::getenv("CONVHIP_TAP");
  if (!s || !*s) return -1;
  return std::atoi(s) ? -1 : 0;
}

// Compute units of the current device (cached per device id).
static int device_num_cu() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// The fused kernels take the minimum over their axis 0. For a minimum over H or
// W the spatial axes are permuted (conv commutes with a permutation of the
// spatial axes applied to x, w, stride, dilation and padding alike); the two
// remaining axes keep their order, so the output [N, C_out, rest...] is
// contiguous in the permuted order too. perm[i] = original axis of kernel axis i.
static const int kFusedPerm[3][3] = {{0, 1, 2}, {1, 0, 2}, {2, 0, 1}};
static Geom fused_geom(const Geom& g0, int min_dim) {
  const int* perm = kFusedPerm[min_dim - 2];
  Geom g = g0;
  for (int i = 0; i < 3; i++) {
    g.L[i] = g0.L[perm[i]];
    g.K[i] = g0.K[perm[i]];
    g.S[i] = g0.S[perm[i]];
    g.Dl[i] = g0.Dl[perm[i]];
    g.P[i] = g0.P[perm[i]];
    g.O[i] = g0.O[perm[i]];
  }
  return g;
}

// The fused op on NCDHW tensors (g0.cl false) or channels-last ones (x [N, D,
// H, W, C_in], y [N, kept axes, C_out]); g0 holds the logical geometry.
static int fused_run(const Geom& g0, int min_dim, const float* x, const float* w, const float* bias, float* y,
                     convhip_stream_t stream) {
  if (min_dim < 2 || min_dim > 4) return CONV_ERR_PARAM;
  const int* perm = kFusedPerm[min_dim - 2];
  const Geom g = fused_geom(g0, min_dim);
  // Element strides of x per logical spatial axis (D, H, W), per input channel
  // and per sample; of w per kernel axis; of y per sample, output channel and
  // output position (y [N, C_out, kept axes], or channels-last).
  const int64_t vol = g0.L[0] * g0.L[1] * g0.L[2];
  const bool cl = g0.cl;
  const int64_t xst[3] = {g0.L[1] * g0.L[2] * (cl ? g0.Cin : 1), g0.L[2] * (cl ? g0.Cin : 1), cl ? g0.Cin : 1};
  const int64_t xs_c = cl ? 1 : vol, xs_n = g0.Cin * vol;
  const int64_t wst[3] = {g0.K[1] * g0.K[2], g0.K[2], 1};
  const int64_t plane = g.plane_out();
  const int64_t ys_n = g.Cout * plane, ys_c = cl ? 1 : plane, ys_p = cl ? g.Cout : 1;
  FusedPlan p;
  // The depth-streamed kernel streams over the min axis. With contiguous
  // columns (W, in NCDHW, for a minimum over D or H) it copies input rows in
  // 16-byte chunks (x 16-byte aligned); else single elements.
  const bool aligned = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  int rc = plan_fused(g, min_dim, &p, use_tap() != 0 && (aligned || min_dim == 4 || cl));
  if (rc != CONV_OK) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.spec >= 0) {
    StreamArgs sa;
    sa.x = x; sa.w = w; sa.bias = bias; sa.y = y;
    sa.Cout = int(g.Cout);
    sa.L0 = int(g.L[0]); sa.L1 = int(g.L[1]); sa.L2 = int(g.L[2]);
    sa.P0 = int(g.P[0]); sa.P1 = int(g.P[1]); sa.P2 = int(g.P[2]);
    sa.O0 = int(g.O[0]); sa.O1 = int(g.O[1]);
    sa.plane_out = int(g.plane_out());
    sa.tiles_per_plane = int(p.tiles_per_plane);
    sa.dsplit = p.dsplit;
    sa.ods = int((g.O[0] + p.dsplit - 1) / p.dsplit);
    sa.units = int(p.units);
    sa.plane_stride = int(xst[perm[0]]);
    sa.row_stride = int(xst[perm[1]]);
    sa.col_stride = int(xst[perm[2]]);
    sa.ws0 = int(wst[perm[0]]);
    sa.ws1 = int(wst[perm[1]]);
    sa.ws2 = int(wst[perm[2]]);
    sa.xs_n = xs_n;
    sa.xs_c = int(xs_c);
    sa.ys_n = ys_n;
    sa.ys_c = int(ys_c);
    sa.ys_p = int(ys_p);
    return launch_stream_spec(sa, p, s);
  }
  FusedArgs a;
  a.x = x; a.w = w; a.bias = bias; a.y = y;
  a.Cin = int(g.Cin); a.Cout = int(g.Cout);
  a.L0 = int(g.L[0]); a.L1 = int(g.L[1]); a.L2 = int(g.L[2]);
  a.K0 = int(g.K[0]); a.K1 = int(g.K[1]); a.K2 = int(g.K[2]);
  a.S0 = int(g.S[0]); a.S1 = int(g.S[1]); a.S2 = int(g.S[2]);
  a.D0 = int(g.Dl[0]); a.D1 = int(g.Dl[1]); a.D2 = int(g.Dl[2]);
  a.P0 = int(g.P[0]); a.P1 = int(g.P[1]); a.P2 = int(g.P[2]);
  a.O0 = int(g.O[0]); a.O1 = int(g.O[1]); a.O2 = int(g.O[2]);
  a.kvol = int(g.kvol());
  a.mode = p.mode; a.dspan = p.dspan; a.rows = p.rows; a.bw = p.bw; a.boxc = p.boxc; a.row_tiles = p.row_tiles;
  a.plane_out = int(g.plane_out());
  a.xs_c = xs_c;
  a.xs_n = xs_n;
  a.ys_n = ys_n;
  a.ys_c = ys_c;
  a.ys_p = ys_p;
  a.xs0 = xst[perm[0]];
  a.xs1 = xst[perm[1]];
  a.xs2 = xst[perm[2]];
  a.ws0 = int(wst[perm[0]]);
  a.ws1 = int(wst[perm[1]]);
  a.ws2 = int(wst[perm[2]]);
  a.Cg = int(g.Cg);
  a.Coutg = int(g.Coutg);
  a.groups = int(g.G);
  a.cchunks = p.cchunks;
  a.kg = p.kg; a.kgp = p.kgp; a.kgs = p.kgs; a.cpadg = p.cpad;
  a.tile_pos = p.tile_pos;
  a.nrows = p.nrows;
  a.ko_off = p.ko_off; a.wt_off = p.wt_off; a.red_off = p.red_off; a.fin_off = p.fin_off;
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
    case CONV_ERR_RANK: return "CONV_ERR_RANK: nd must be 1, 2 or 3";
    case CONV_ERR_SHAPE: return "CONV_ERR_SHAPE: bad dimension or weight shape";
    case CONV_ERR_GROUPS: return "CONV_ERR_GROUPS: groups < 1 or channels not divisible by groups";
    case CONV_ERR_PARAM: return "CONV_ERR_PARAM: stride/dilation < 1 or padding < 0";
    case CONV_ERR_EMPTY_OUTPUT: return "CONV_ERR_EMPTY_OUTPUT: an output length is <= 0";
    case CONV_ERR_UNSUPPORTED: return "CONV_ERR_UNSUPPORTED: valid arguments the library does not handle";
    case CONV_ERR_OVERFLOW: return "CONV_ERR_OVERFLOW: a size exceeds the index arithmetic";
    case CONV_ERR_HIP: return "CONV_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown conv_status";
  }
}

int conv_plan_describe(int nd, const int64_t* x_shape, const int64_t* w_shape, const int* stride,
                       const int* dilation, const int* padding, int groups, int fused, char* buf, int buflen) {
  if (!buf || buflen < 1) return CONV_ERR_NULL;
  buf[0] = 0;
  if (fused < 0 || fused > 7) return CONV_ERR_PARAM;
  Geom g;
  const bool cl = fused == 2 || fused >= 5;
  int rc = cl ? make_geom_channels_last(nd, x_shape, w_shape, stride, dilation, padding, groups, &g)
              : make_geom(nd, x_shape, w_shape, stride, dilation, padding, groups, &g);
  if (rc != CONV_OK) return rc;
  std::string s;
  if (fused == 1 || fused >= 3) {
    if (nd != 3) return CONV_ERR_RANK;
    const int min_dim = fused == 1 ? 2 : fused >= 5 ? fused - 3 : fused;
    FusedPlan p;
    rc = plan_fused(fused_geom(g, min_dim), min_dim, &p, use_tap() != 0);
    if (rc != CONV_OK) return rc;
    s = describe(fused_geom(g, min_dim), p);
  } else {
    ValuPlan vp;
    ConvPlan p;
    bool valu = force_valu() && plan_valu(g, &vp) == CONV_OK;
    if (!valu) {
      rc = plan_conv(g, &p, forced_conv_cfg(), 256, use_tap(), split_kernel_choice());
      valu = rc == CONV_ERR_UNSUPPORTED && plan_valu(g, &vp) == CONV_OK;
      if (!valu && rc != CONV_OK) return rc;
    }
    if (valu) {
      char t[256];
      std::snprintf(t, sizeof t, "conv_valu co=%d pp=%d threads=%d pairs=%d grid=%lldx%lld lds=%d", vp.co,
                    vp.pp, vp.threads, vp.pps, (long long)vp.grid[0], (long long)vp.grid[1], vp.lds_bytes);
      s = t;
    } else {
      s = describe(g, p);
    }
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
  ValuPlan vp;
  if (force_valu() && plan_valu(g, &vp) == CONV_OK) return launch_valu(g, vp, x, w, bias, y, stream);
  ConvPlan p;
  // The specialised kernels copy weights (and 1-D input rows) in 16-byte chunks:
  // they need 16-byte aligned pointers (any tensor allocation is; a sliced view
  // may not be).
  const bool aligned = ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(x)) & 15) == 0;
  rc = plan_conv(g, &p, forced_conv_cfg(), device_num_cu(), aligned ? use_tap() : 0, split_kernel_choice());
  // Geometries whose tiles the matrix-core kernels cannot stage in LDS (large
  // kernels over many channels) run on the vector-ALU kernel.
  if (rc == CONV_ERR_UNSUPPORTED && plan_valu(g, &vp) == CONV_OK) return launch_valu(g, vp, x, w, bias, y, stream);
  if (rc != CONV_OK) return rc;
  ConvArgs a = conv_args(g, p, x, w, bias, y);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.tap_spec >= 0) return launch_tap_spec(a, p, s);
  if (p.direct_spec >= 0) return launch_direct_spec<false>(a, p, s);
  if (p.ks_spec >= 0) return launch_ks_spec<false>(a, p, s);
  if (p.split_spec >= 0) return launch_split_spec<false>(a, p, s);
  return launch_generic<false>(a, p, s);
}

int conv_fwd_channels_last(int nd, const float* x, const int64_t* x_shape, const float* w, const int64_t* w_shape,
                           const float* bias, const int* stride, const int* dilation, const int* padding,
                           int groups, float* y, convhip_stream_t stream) {
  Geom g;
  int rc = make_geom_channels_last(nd, x_shape, w_shape, stride, dilation, padding, groups, &g);
  if (rc != CONV_OK) return rc;
  if (!x || !w || !y) return CONV_ERR_NULL;
  // 16-byte copies of channel quads need a 16-byte aligned x, 16-byte weight
  // copies an aligned w.
  g.x_aligned16 = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  g.w_aligned16 = (reinterpret_cast<uintptr_t>(w) & 15) == 0;
  ValuPlan vp;
  if (force_valu() && plan_valu(g, &vp) == CONV_OK) return launch_valu(g, vp, x, w, bias, y, stream);
  ConvPlan p;
  rc = plan_conv(g, &p, forced_conv_cfg(), device_num_cu(), use_tap(), split_kernel_choice());
  // Geometries no matrix-core kernel can stage run on the vector-ALU kernel.
  if (rc == CONV_ERR_UNSUPPORTED && plan_valu(g, &vp) == CONV_OK) return launch_valu(g, vp, x, w, bias, y, stream);
  if (rc != CONV_OK) return rc;
  ConvArgs a = conv_args(g, p, x, w, bias, y);
  a.vec_store = (g.Cout % 4 == 0 && g.Coutg % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0) ? 1 : 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.tap_spec >= 0) return launch_tap_cl_spec(a, p, s);
  if (p.direct_spec >= 0) return launch_direct_spec<true>(a, p, s);
  if (p.ks_spec >= 0) return launch_ks_spec<true>(a, p, s);
  if (p.split_spec >= 0) return launch_split_spec<true>(a, p, s);
  return launch_generic<true>(a, p, s);
}
int conv3d_min_softmax(const float* x, const int64_t* x_shape, const float* w, const int64_t* w_shape,
                       const float* bias, const int* stride, const int* dilation, const int* padding, int groups,
                       int min_dim, float* y, convhip_stream_t stream) {
  Geom g;
  int rc = make_geom(3, x_shape, w_shape, stride, dilation, padding, groups, &g);
  if (rc != CONV_OK) return rc;
  if (!x || !w || !y) return CONV_ERR_NULL;
  return fused_run(g, min_dim, x, w, bias, y, stream);
}

int conv3d_min_softmax_channels_last(const float* x, const int64_t* x_shape, const float* w, const int64_t* w_shape,
                                     const float* bias, const int* stride, const int* dilation, const int* padding,
                                     int groups, int min_dim, float* y, convhip_stream_t stream) {
  Geom g;
  int rc = make_geom_channels_last(3, x_shape, w_shape, stride, dilation, padding, groups, &g);
  if (rc != CONV_OK) return rc;
  if (!x || !w || !y) return CONV_ERR_NULL;
  return fused_run(g, min_dim, x, w, bias, y, stream);
}

int convhip_peak_probe(int kind, int64_t iters, float* sink, int64_t* flop, convhip_stream_t stream) {
  if (!sink || !flop) return CONV_ERR_NULL;
  // At most 2^22 rounds: about 2 s of matrix-core work per launch.
  if ((kind != 0 && kind != 1) || iters < 1 || iters > (int64_t(1) << 22)) return CONV_ERR_PARAM;
  // 4 workgroups of 4 waves per compute unit: 4 waves per SIMD.
  const int64_t blocks = 4 * int64_t(device_num_cu());
  const int64_t threads = blocks * 256;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (kind == 0) {
    *flop = (threads / 64) * iters * 8 * (2 * 16 * 16 * 4);
    hipLaunchKernelGGL(peak_mfma_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, iters, sink);
  } else {
    *flop = threads * iters * 8 * 2;
    hipLaunchKernelGGL(peak_fma_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, iters, sink);
  }
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_HIP;
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
