// Validation, output shapes and launch planning (host only).
#include "convhip_plan.h"

#include <algorithm>
#include <cstdio>
#include <limits>

#include "../../include/convhip.h"

namespace convhip {

int64_t out_len(int64_t L, int64_t k, int64_t s, int64_t d, int64_t p) {
  int64_t num = L + 2 * p - d * (k - 1) - 1;
  int64_t q = num / s;
  if (num % s != 0 && num < 0) q -= 1;  // floor, not truncation
  return q + 1;
}

int make_geom(int nd, const int64_t* xs, const int64_t* ws, const int* stride, const int* dilation,
              const int* padding, int groups, Geom* g) {
  if (nd < 1 || nd > 3) return CONV_ERR_RANK;
  if (!xs || !ws || !stride || !dilation || !padding || !g) return CONV_ERR_NULL;
  for (int i = 0; i < nd + 2; i++)
    if (xs[i] < 1 || ws[i] < 1) return CONV_ERR_SHAPE;
  if (groups < 1) return CONV_ERR_GROUPS;
  for (int a = 0; a < nd; a++)
    if (stride[a] < 1 || dilation[a] < 1 || padding[a] < 0) return CONV_ERR_PARAM;
  Geom r;
  r.nd = nd;
  r.N = xs[0];
  r.Cin = xs[1];
  r.Cout = ws[0];
  r.G = groups;
  if (r.Cin % groups != 0 || r.Cout % groups != 0) return CONV_ERR_GROUPS;
  r.Cg = r.Cin / groups;
  r.Coutg = r.Cout / groups;
  if (ws[1] != r.Cg) return CONV_ERR_SHAPE;
  for (int a = 0; a < nd; a++) {
    int ax = 3 - nd + a;
    r.L[ax] = xs[2 + a];
    r.K[ax] = ws[2 + a];
    r.S[ax] = stride[a];
    r.Dl[ax] = dilation[a];
    r.P[ax] = padding[a];
  }
  const int64_t kMax = std::numeric_limits<int32_t>::max();
  for (int a = 0; a < 3; a++) {
    if (r.L[a] > kMax || r.K[a] > kMax || r.S[a] > kMax || r.Dl[a] > kMax || r.P[a] > kMax)
      return CONV_ERR_OVERFLOW;
    r.O[a] = out_len(r.L[a], r.K[a], r.S[a], r.Dl[a], r.P[a]);
    if (r.O[a] < 1) return CONV_ERR_EMPTY_OUTPUT;
  }
  // Per-tensor element counts must fit int64 comfortably; per-axis and per-plane
  // indices are computed in 32 bits inside the kernels.
  const double xe = double(r.N) * r.Cin * r.L[0] * r.L[1] * r.L[2];
  const double ye = double(r.N) * r.Cout * r.O[0] * r.O[1] * r.O[2];
  if (xe > 4.0e18 || ye > 4.0e18) return CONV_ERR_OVERFLOW;
  if (r.N > kMax || r.Cin > kMax || r.Cout > kMax) return CONV_ERR_OVERFLOW;
  if (double(r.O[1]) * r.O[2] > double(kMax)) return CONV_ERR_OVERFLOW;
  if (double(r.Cg) * r.kvol() > double(kMax)) return CONV_ERR_OVERFLOW;
  *g = r;
  return CONV_OK;
}

int make_geom_channels_last(int nd, const int64_t* xs, const int64_t* ws, const int* stride, const int* dilation,
                            const int* padding, int groups, Geom* g) {
  if (nd < 1 || nd > 3) return CONV_ERR_RANK;
  if (!xs) return CONV_ERR_NULL;
  int64_t logical[5];
  logical[0] = xs[0];
  logical[1] = xs[nd + 1];
  for (int a = 0; a < nd; a++) logical[2 + a] = xs[1 + a];
  const int rc = make_geom(nd, logical, ws, stride, dilation, padding, groups, g);
  if (rc == CONV_OK) g->cl = true;
  return rc;
}

CfgShape cfg_shape(int cfg) {
  switch (cfg) {
    case CFG_M64: return {4, 4, 1, 4, 1};
    case CFG_M128: return {4, 4, 2, 2, 1};
    case CFG_M32: return {2, 4, 1, 4, 1};
    case CFG_M16: return {1, 4, 1, 4, 1};
    case CFG_M16_N64_K4: return {1, 4, 1, 1, 4};
    case CFG_M16_N128_K4: return {1, 8, 1, 1, 4};
    case CFG_M16_N208_K4: return {1, 13, 1, 1, 4};
    default: return {1, 16, 1, 1, 4};
  }
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Box geometry for a tiling mode with BN positions per tile.
static void box_dims(const Geom& g, int mode, int BN, int* rows, int* bw, int64_t* tiles, int* row_tiles) {
  if (mode == TILE_FLAT) {
    int64_t rows_out = std::min<int64_t>(g.O[1], (g.O[2] + BN - 2) / g.O[2] + 1);
    *rows = int((rows_out - 1) * g.S[1] + (g.K[1] - 1) * g.Dl[1] + 1);
    *bw = int((g.O[2] - 1) * g.S[2] + (g.K[2] - 1) * g.Dl[2] + 1);
    *tiles = ceil_div(g.plane_out(), BN);
    *row_tiles = 0;
  } else {
    *rows = int((g.K[1] - 1) * g.Dl[1] + 1);
    int64_t seg = std::min<int64_t>(BN, g.O[2]);
    *bw = int((seg - 1) * g.S[2] + (g.K[2] - 1) * g.Dl[2] + 1);
    *row_tiles = int(ceil_div(g.O[2], BN));
    *tiles = g.O[1] * (*row_tiles);
  }
}

const TapSpecDesc* tap_specs(int* count) {
#define CONVHIP_TAP_DESC(id, MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW) \
  {id, MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW},
  static const TapSpecDesc specs[] = {CONVHIP_TAP_SPECS(CONVHIP_TAP_DESC)};
#undef CONVHIP_TAP_DESC
  *count = int(sizeof(specs) / sizeof(specs[0]));
  return specs;
}

const TapClSpecDesc* tap_cl_specs(int* count) {
#define CONVHIP_TAP_CL_DESC(id, MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW, CCP) \
  {id, MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW, CCP},
  static const TapClSpecDesc specs[] = {CONVHIP_TAP_CL_SPECS(CONVHIP_TAP_CL_DESC)};
#undef CONVHIP_TAP_CL_DESC
  *count = int(sizeof(specs) / sizeof(specs[0]));
  return specs;
}

const SplitSpecDesc* split_specs(int* count) {
#define CONVHIP_SPLIT_DESC(id, NT, NW, KD, KH, KW, DD, DH, DW, F, ROWS, BW, TS) \
  {id, NT, NW, KD, KH, KW, DD, DH, DW, F, ROWS, BW, TS},
  static const SplitSpecDesc specs[] = {CONVHIP_SPLIT_SPECS(CONVHIP_SPLIT_DESC)};
#undef CONVHIP_SPLIT_DESC
  *count = int(sizeof(specs) / sizeof(specs[0]));
  return specs;
}

const DirectSpecDesc* direct_specs(int* count) {
#define CONVHIP_DIRECT_DESC(id, CIN, KD, KH, KW, DD, DH, DW) {id, CIN, KD, KH, KW, DD, DH, DW},
  static const DirectSpecDesc specs[] = {CONVHIP_DIRECT_SPECS(CONVHIP_DIRECT_DESC)};
#undef CONVHIP_DIRECT_DESC
  *count = int(sizeof(specs) / sizeof(specs[0]));
  return specs;
}

// Plan of a direct-kernel specialisation: the spec's channels, kernel and
// dilations, no padding, <= 16 output channels per group, a small problem, and
// every element offset (positions < 2^24, tensors < 2^31 elements) in 32 bits.
static bool plan_direct(const Geom& g, const DirectSpecDesc& d, ConvPlan* p) {
  if (g.Coutg > 16 || g.Cg != d.CIN) return false;
  if (g.K[0] != d.KD || g.K[1] != d.KH || g.K[2] != d.KW) return false;
  if (g.Dl[0] != d.DD || g.Dl[1] != d.DH || g.Dl[2] != d.DW) return false;
  if (g.P[0] != 0 || g.P[1] != 0 || g.P[2] != 0) return false;
  if (g.macs() > kDirectMaxMacs) return false;
  const int64_t npos = g.N * g.O[0] * g.O[1] * g.O[2];
  if (npos >= (int64_t(1) << 24)) return false;
  const int64_t xe = g.N * g.Cin * g.L[0] * g.L[1] * g.L[2];
  const int64_t ye = npos * g.Cout;
  if (xe >= (int64_t(1) << 31) || ye >= (int64_t(1) << 31) || g.G > 65535) return false;
  ConvPlan q;
  q.cfg = -1;
  q.direct_spec = d.id;
  q.threads = 64;
  q.BM = 16;
  q.BN = 16;
  q.Cc = d.CIN;
  q.kc_pad = int((int64_t(d.CIN) * d.KD * d.KH * d.KW + 3) / 4 * 4);
  q.items = npos;
  q.grid[0] = (npos + 15) / 16;
  q.grid[1] = g.G;
  q.grid[2] = 1;
  q.lds_bytes = 0;
  *p = q;
  return true;
}

const KsSpecDesc* ks_specs(int* count) {
#define CONVHIP_KS_DESC(id, CG, KD, KH, KW, DH, DW, F, ROWS, BW, T) {id, CG, KD, KH, KW, DH, DW, F, ROWS, BW, T},
  static const KsSpecDesc specs[] = {CONVHIP_KSTREAM_SPECS(CONVHIP_KS_DESC)};
#undef CONVHIP_KS_DESC
  *count = int(sizeof(specs) / sizeof(specs[0]));
  return specs;
}

// LDS floats of a stream-K specialisation (the kernel's layout: box planes of
// whole 64-float copies, the weight operands of every 16-deep reduction block,
// a 256-float target for padding copies, the split tiles' partial sums).
static int64_t ks_lds_floats(const KsSpecDesc& d) {
  const int64_t kred = int64_t(d.CG) * d.KD * d.KH * d.KW;
  const int64_t pslot = (int64_t(d.ROWS) * d.BW + 63) / 64 * 64;
  const int64_t nq = (kred + 15) / 16;
  const int64_t r = d.T % 4;
  return int64_t(d.CG) * d.KD * pslot + nq * 256 + 256 + 4 * (r > 0 ? r : 1) * 256;
}

// Plan of a stream-K specialisation if the geometry fits it: NCDHW tensors, the
// spec's channels, kernel and W/H dilations, W stride and dilation multiples of
// F, exactly T tiles per output plane, and a box within the staged extents.
static bool plan_kstream(const Geom& g, const KsSpecDesc& d, ConvPlan* p) {
  if (g.Coutg > 16 || g.Cg != d.CG) return false;
  if (g.K[0] != d.KD || g.K[1] != d.KH || g.K[2] != d.KW) return false;
  if (g.Dl[1] != d.DH || g.Dl[2] != d.DW) return false;
  if (g.S[2] % d.F != 0 || d.DW % d.F != 0) return false;
  // Channels-last: the box is copied as 16-byte channel quads.
  if (g.cl && (d.CG % 4 != 0 || g.Cin % 4 != 0 || !g.x_aligned16)) return false;
  if ((int64_t(d.CG) * d.KD * d.KH * d.KW) % 4 != 0) return false;
  if ((g.plane_out() + 15) / 16 != d.T) return false;
  const int64_t rows = (g.O[1] - 1) * g.S[1] + (g.K[1] - 1) * g.Dl[1] + 1;
  const int64_t bw = ((g.O[2] - 1) * g.S[2] + (g.K[2] - 1) * g.Dl[2]) / d.F + 1;
  if (rows > d.ROWS || bw > d.BW) return false;
  const int64_t items = g.N * g.O[0] * g.G;
  if (items > std::numeric_limits<int32_t>::max()) return false;
  // In-plane source offsets (times C_in for channels-last sites) in 32 bits.
  if (g.L[1] * g.L[2] * (g.cl ? g.Cin : 1) > std::numeric_limits<int32_t>::max() / 2) return false;
  const int64_t lds = 4 * ks_lds_floats(d);
  if (lds > kLdsLimit) return false;
  ConvPlan q;
  q.cfg = -1;
  q.ks_spec = d.id;
  q.threads = 256;
  q.BM = 16;
  q.BN = 16 * d.T;
  q.mode = TILE_FLAT;
  q.Cc = d.CG;
  q.kc_pad = int((int64_t(d.CG) * d.KD * d.KH * d.KW + 15) / 16 * 16);
  q.kdspan = d.KD;
  q.rows = int(rows);
  q.bw = int(bw);
  q.boxc = d.KD * d.ROWS * d.BW;
  q.tiles_per_plane = 1;
  q.ctiles = 1;
  q.nchunks = 1;
  q.items = items;
  q.lds_bytes = lds;
  q.grid[0] = items;
  q.grid[1] = 1;
  q.grid[2] = 1;
  *p = q;
  return true;
}

static bool plan_split(const Geom& g, const SplitSpecDesc& d, bool pipe, ConvPlan* p) {
  if (g.Coutg > 16 || g.Cg != d.NW) return false;
  if (g.K[0] != d.KD || g.K[1] != d.KH || g.K[2] != d.KW) return false;
  if (g.Dl[0] != d.DD || g.Dl[1] != d.DH || g.Dl[2] != d.DW) return false;
  if (g.S[2] % d.F != 0 || g.Dl[2] % d.F != 0) return false;
  // The plane's 16-position tiles fill TS groups of NT (the last group partly).
  if (g.plane_out() > 16 * d.NT * d.TS || g.plane_out() <= 16 * (d.NT * d.TS - d.NT)) return false;
  const int64_t kvol = int64_t(d.KD) * d.KH * d.KW;
  const int64_t rows = (g.O[1] - 1) * g.S[1] + (g.K[1] - 1) * g.Dl[1] + 1;
  const int64_t bw = ((g.O[2] - 1) * g.S[2] + (g.K[2] - 1) * g.Dl[2]) / d.F + 1;
  if (rows != d.ROWS || bw > d.BW) return false;  // rows may be staged wider (bank spread)
  if (g.N * g.O[0] > std::numeric_limits<int32_t>::max() || g.G > 65535) return false;
  // Channels-last: in-plane source offsets (row * W + column) * C_in in 32 bits;
  // 16-byte weight copies need an aligned w.
  if (g.cl && (g.L[1] * g.L[2] * g.Cin > std::numeric_limits<int32_t>::max() || !g.w_aligned16)) return false;
  ConvPlan q;
  q.cfg = -1;
  q.split_spec = d.id;
  q.threads = 64 * d.NW;
  q.BM = 16;
  q.BN = 16 * d.NT;
  q.mode = TILE_FLAT;
  q.Cc = 1;
  q.kc_pad = int((kvol + 3) / 4 * 4);
  q.kdspan = d.KD;
  q.rows = int(rows);
  q.bw = d.BW;
  q.boxc = int(d.KD * rows * d.BW);
  q.tiles_per_plane = 1;
  q.ctiles = 1;
  q.nchunks = 1;
  const int64_t xsw = (int64_t(q.boxc) + 3) / 4 * 4;
  const int64_t wrow = d.NW * kvol;
  const int64_t wld = (wrow % 4 == 0 && (wrow / 4) % 2 == 0) ? wrow + 4 : wrow;
  const int64_t wsh = (16 * wld + 4 + 3) / 4 * 4;
  q.lds_bytes = 4 * std::max<int64_t>(wsh + int64_t(d.NW) * xsw, int64_t(d.NW) * d.NT * 4 * 64);
  if (pipe && split_pipe_fits(d.NT, d.NW, int(wrow))) {
    // Per wave: the weights, one depth tap at a time (16 rows of a multiple of
    // 4 16-byte slots covering kH*kW + 3 floats), later batch 1's parked tiles;
    // the box, later batch 2's parked tiles; plus one counter.
    const int64_t wqt = ((int64_t(d.KH) * d.KW + 6) / 4 + 3) / 4 * 4;
    const int64_t wreg = std::max<int64_t>(int64_t(d.KD) * wqt * 64, int64_t((d.NT + 1) / 2) * 256);
    const int64_t xreg = std::max<int64_t>(xsw, int64_t(d.NT / 2) * 256);
    q.split_pipe = 1;
    q.lds_bytes = 4 * (int64_t(d.NW) * (wreg + xreg) + 4);
  }
  if (q.lds_bytes > kLdsLimit) return false;
  q.grid[0] = g.N * g.O[0];
  q.grid[1] = g.G;
  q.grid[2] = d.TS;
  *p = q;
  return true;
}

// Plan of a tap specialisation if the geometry is exactly the one it was built for.
static bool plan_tap(const Geom& g, const TapSpecDesc& d, int num_cu, ConvPlan* p) {
  const int BM = 16 * d.MT * d.WM, BN = 16 * d.NT * d.WN;
  if (g.G != 1 || g.Coutg > BM || g.Cg != int64_t(d.CC) * d.NCH) return false;
  if (g.K[0] != d.KD || g.K[1] != d.KH || g.K[2] != d.KW) return false;
  if (g.Dl[0] != d.DD || g.Dl[1] != d.DH || g.Dl[2] != d.DW) return false;
  const int mode = (g.O[2] * 2 <= BN) ? TILE_FLAT : TILE_ROW;
  int rows, bw, row_tiles;
  int64_t tiles;
  box_dims(g, mode, BN, &rows, &bw, &tiles, &row_tiles);
  const int kdspan = int((g.K[0] - 1) * g.Dl[0] + 1);
  // The box is staged at the spec's extents: a geometry whose tiles need fewer
  // rows or columns leaves the rest unread (copied from the input or zero).
  if (rows > d.ROWS || kdspan != d.KDSPAN || bw > d.BW) return false;
  // Specialisations with rows of a multiple of 4 floats copy the box in 16-byte
  // chunks starting at input column ow0*S - P: the input rows, that column and
  // the row length must be multiples of 4.
  if (d.BW % 4 == 0) {
    if (g.L[2] % 4 != 0 || g.P[2] % 4 != 0) return false;
    if (mode == TILE_ROW && (g.S[2] * BN) % 4 != 0) return false;
  }
  rows = d.ROWS;
  bw = d.BW;
  const int64_t items = tiles * g.N * g.O[0];
  if (items > std::numeric_limits<int32_t>::max()) return false;
  const int64_t kvol = int64_t(d.KD) * d.KH * d.KW;
  const int64_t ns = (d.CC * kvol + 3) / 4;
  const int64_t xs = (int64_t(d.CC) * kdspan * rows * bw + 255) / 256 * 256;
  const int64_t wf = (d.NCH * ns + 1) * d.WM * 64 * d.MT;
  const int64_t bytes = 4 * (2 * xs + wf);
  if (bytes > kLdsLimit) return false;
  ConvPlan q;
  q.cfg = -1;
  q.tap_spec = d.id;
  q.threads = 64 * d.WM * d.WN;
  q.BM = BM;
  q.BN = BN;
  q.mode = mode;
  q.Cc = d.CC;
  q.kc_pad = int(ns * 4);
  q.kdspan = kdspan;
  q.rows = rows;
  q.bw = bw;
  q.boxc = kdspan * rows * bw;
  q.xs_floats = int(xs);
  q.koff_ints = 0;
  q.ws_floats = int(wf);
  q.tiles_per_plane = tiles;
  q.row_tiles = row_tiles;
  q.ctiles = 1;
  q.nchunks = d.NCH;
  q.items = items;
  q.lds_bytes = bytes;
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(2, kLdsLimit / bytes));
  q.grid[0] = std::min<int64_t>(items, per_cu * num_cu);
  q.grid[1] = 1;
  q.grid[2] = 1;
  *p = q;
  return true;
}

// Channels-last box pitch (floats per site). The 16 position lanes of a
// matrix-core operand read sit stride_w * pitch floats apart; they fall in
// distinct banks (of 64) when gcd(stride_w * pitch, 64) <= 4. Scalar copies:
// Cc, else Cc + 1. Quad copies (vec): the multiple of 4 in [Cc, Cc + 12] with
// the smallest such gcd.
static int64_t bank_gcd(int64_t v) {
  int64_t g = 64;
  while (v % g != 0) g /= 2;
  return g;
}
static int cl_pitch(int64_t cc, int64_t stride_w, bool vec) {
  if (!vec) return int(bank_gcd(cc * stride_w) <= 4 ? cc : cc + 1);
  int64_t best = cc;
  for (int64_t p = cc; p <= cc + 12; p += 4)
    if (bank_gcd(p * stride_w) < bank_gcd(best * stride_w)) best = p;
  return int(best);
}

// Plan of a channels-last tap specialisation if the geometry is the one it was
// built for (copies in channel quads need a 16-byte aligned x with C_in a
// multiple of 4).
static bool plan_tap_cl(const Geom& g, const TapClSpecDesc& d, int num_cu, ConvPlan* p) {
  const int BM = 16 * d.MT * d.WM, BN = 16 * d.NT * d.WN;
  const bool quads = d.CC % 4 == 0 && d.CCP % 4 == 0;
  if (!g.cl || (quads && (!g.x_aligned16 || g.Cin % 4 != 0))) return false;
  if (g.G != 1 || g.Coutg > BM || g.Cg != int64_t(d.CC) * d.NCH) return false;
  if (g.K[0] != d.KD || g.K[1] != d.KH || g.K[2] != d.KW) return false;
  if (g.Dl[0] != d.DD || g.Dl[1] != d.DH || g.Dl[2] != d.DW) return false;
  const int mode = (g.O[2] * 2 <= BN) ? TILE_FLAT : TILE_ROW;
  int rows, bw, row_tiles;
  int64_t tiles;
  box_dims(g, mode, BN, &rows, &bw, &tiles, &row_tiles);
  const int kdspan = int((g.K[0] - 1) * g.Dl[0] + 1);
  // The box is staged at the spec's extents (fewer needed rows or sites are
  // left unread).
  if (rows > d.ROWS || kdspan != d.KDSPAN || bw > d.BW) return false;
  const int64_t items = tiles * g.N * g.O[0];
  if (items > std::numeric_limits<int32_t>::max()) return false;
  const int64_t kvol = int64_t(d.KD) * d.KH * d.KW;
  const int64_t ns = (d.CC * kvol + 3) / 4;
  const int64_t xs = (int64_t(d.CCP) * d.KDSPAN * d.ROWS * d.BW + 255) / 256 * 256;
  const int64_t wf = (d.NCH * ns + 1) * d.WM * 64 * d.MT;
  const int64_t bytes = 4 * (2 * xs + wf);
  if (bytes > kLdsLimit) return false;
  ConvPlan q;
  q.cfg = -1;
  q.tap_spec = d.id;
  q.threads = 64 * d.WM * d.WN;
  q.BM = BM;
  q.BN = BN;
  q.mode = mode;
  q.Cc = d.CC;
  q.kc_pad = int(ns * 4);
  q.kdspan = kdspan;
  q.rows = d.ROWS;
  q.bw = d.BW;
  q.boxc = kdspan * d.ROWS * d.BW;
  q.ccp = d.CCP;
  q.cl_vec = quads;
  q.xs_floats = int(xs);
  q.koff_ints = 0;
  q.ws_floats = int(wf);
  q.tiles_per_plane = tiles;
  q.row_tiles = row_tiles;
  q.ctiles = 1;
  q.nchunks = d.NCH;
  q.items = items;
  q.lds_bytes = bytes;
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(2, kLdsLimit / bytes));
  q.grid[0] = std::min<int64_t>(items, per_cu * num_cu);
  q.grid[1] = 1;
  q.grid[2] = 1;
  *p = q;
  return true;
}

int plan_conv(const Geom& g, ConvPlan* out, int force_cfg, int num_cu, int use_tap, int split_kernel) {
  const bool split_pipe = split_kernel != 2;
  if (g.cl) {
    if (use_tap != 0 && force_cfg < 0) {
      int n = 0;
      const TapClSpecDesc* specs = tap_cl_specs(&n);
      for (int i = 0; i < n; i++)
        if (plan_tap_cl(g, specs[i], num_cu, out)) return CONV_OK;
      if (split_kernel == 0) {
        const DirectSpecDesc* ds = direct_specs(&n);
        for (int i = 0; i < n; i++)
          if (plan_direct(g, ds[i], out)) return CONV_OK;
        const KsSpecDesc* ks = ks_specs(&n);
        for (int i = 0; i < n; i++)
          if (plan_kstream(g, ks[i], out)) return CONV_OK;
      }
      const SplitSpecDesc* ss = split_specs(&n);
      for (int i = 0; i < n; i++)
        if (plan_split(g, ss[i], split_pipe, out)) return CONV_OK;
    }
    use_tap = 0;
  }
  if (use_tap != 0 && force_cfg < 0) {
    int n = 0;
    const TapSpecDesc* specs = tap_specs(&n);
    for (int i = 0; i < n; i++)
      if (plan_tap(g, specs[i], num_cu, out)) return CONV_OK;
    if (split_kernel == 0) {
      const DirectSpecDesc* ds = direct_specs(&n);
      for (int i = 0; i < n; i++)
        if (plan_direct(g, ds[i], out)) return CONV_OK;
      const KsSpecDesc* ks = ks_specs(&n);
      for (int i = 0; i < n; i++)
        if (plan_kstream(g, ks[i], out)) return CONV_OK;
    }
    const SplitSpecDesc* ss = split_specs(&n);
    for (int i = 0; i < n; i++)
      if (plan_split(g, ss[i], split_pipe, out)) return CONV_OK;
  }
  ConvPlan p;
  if (force_cfg >= 0 && force_cfg < CFG_COUNT) {
    p.cfg = force_cfg;
  } else if (g.Coutg > 64) {
    p.cfg = CFG_M128;
  } else if (g.Coutg > 32) {
    p.cfg = CFG_M64;
  } else if (g.Coutg > 16) {
    p.cfg = CFG_M32;
  } else {
    // Few output channels: the reduction is split over the 4 waves of a block and
    // a tile covers a whole (n, od) plane when it fits, so no lanes idle on a
    // ragged plane tail. Large planes with many tiles take the unsplit tile.
    const int64_t plane = g.plane_out();
    if (plane <= 64) p.cfg = CFG_M16_N64_K4;
    else if (plane <= 128) p.cfg = CFG_M16_N128_K4;
    else if (plane <= 208) p.cfg = CFG_M16_N208_K4;
    else if (plane <= 256) p.cfg = CFG_M16_N256_K4;
    else {
      const int64_t tiles = g.N * g.O[0] * ceil_div(plane, 256) * g.G;
      p.cfg = tiles >= 2048 ? CFG_M16 : CFG_M16_N256_K4;
    }
  }
  const CfgShape cs = cfg_shape(p.cfg);
  p.BM = 16 * cs.MT * cs.WM;
  p.BN = 16 * cs.NT * cs.WN;
  // Flattened plane tiles when a tile covers at least two output rows; otherwise
  // row segments, so the box never spans a full long row.
  p.mode = (g.O[2] * 2 <= p.BN) ? TILE_FLAT : TILE_ROW;
  box_dims(g, p.mode, p.BN, &p.rows, &p.bw, &p.tiles_per_plane, &p.row_tiles);
  p.kdspan = int((g.K[0] - 1) * g.Dl[0] + 1);
  const int64_t boxc = int64_t(p.kdspan) * p.rows * p.bw;
  if (boxc > (int64_t(1) << 26)) return CONV_ERR_UNSUPPORTED;
  p.boxc = int(boxc);
  const int64_t red = cs.KS > 1 ? int64_t(cs.KS - 1) * cs.WM * cs.WN * cs.MT * cs.NT * 4 * 64 : 0;
  auto r4 = [](int64_t v) { return (v + 3) / 4 * 4; };
  // LDS: [koff table | 2 x (box | weight fragments)]. The box region is padded to
  // whole 256-float blocks (the DMA writes whole wave-wide rows of 64 slots); the
  // split-K partial sums reuse the two buffers after the reduction.
  auto r256 = [](int64_t v) { return (v + 255) / 256 * 256; };
  // Channels-last inputs whose group channels come in aligned quads are copied
  // 16 bytes per lane (chunks of a multiple of 4 channels).
  bool clvec = g.cl && g.x_aligned16 && g.Cg % 4 == 0 && g.Cin % 4 == 0;
  auto layout = [&](int64_t cc, int64_t* xs, int64_t* ko, int64_t* ws) {
    const int64_t kcp = r4(cc * g.kvol());
    *xs = r256((g.cl ? cl_pitch(cc, g.S[2], clvec) : cc) * p.boxc);
    *ko = r4(kcp + 8 * cs.KS);
    *ws = (kcp / 4 + cs.KS) * cs.WM * 64 * cs.MT;
    if (2 * (*xs + *ws) < red) *xs = r256(red / 2);
    return 4 * (*ko + 2 * (*xs + *ws));
  };
  // Channel chunk: among the chunk sizes whose staged box + weights fit the LDS
  // budget, take the one with the least padded reduction work (chunks x padded
  // taps per chunk), then the fewest chunks. Unsplit tiles keep room for two
  // workgroups per CU; split tiles are used where the grid is small.
  const int64_t budget = cs.KS > 1 ? kLdsLimit : 80 * 1024;  // double-buffered chunks
  auto choose = [&]() {
    const int64_t step = clvec ? 4 : 1;
    int best = 0;
    int64_t best_work = 0, best_chunks = 0;
    for (int64_t cc = step; cc <= std::min<int64_t>(g.Cg, 1024); cc += step) {
      int64_t xs, ko, ws;
      if (layout(cc, &xs, &ko, &ws) > budget) break;
      const int64_t chunks = ceil_div(g.Cg, cc);
      const int64_t work = chunks * r4(cc * g.kvol());
      if (best == 0 || work < best_work || (work == best_work && chunks < best_chunks)) {
        best = int(cc);
        best_work = work;
        best_chunks = chunks;
      }
    }
    return best;
  };
  int best = choose();
  if (best == 0 && clvec) {  // no quad chunk fits: scalar copies
    clvec = false;
    best = choose();
  }
  if (best == 0) {
    // Nothing fits the budget: one channel per chunk if it fits at all.
    int64_t xs, ko, ws;
    if (layout(1, &xs, &ko, &ws) > kLdsLimit) return CONV_ERR_UNSUPPORTED;
    best = 1;
  }
  p.Cc = best;
  p.ccp = g.cl ? cl_pitch(best, g.S[2], clvec) : 0;
  p.cl_vec = clvec;
  int64_t xs, ko, ws;
  p.lds_bytes = layout(p.Cc, &xs, &ko, &ws);
  p.xs_floats = int(xs);
  p.koff_ints = int(ko);
  p.ws_floats = int(ws);
  p.kc_pad = int(r4(int64_t(p.Cc) * g.kvol()));
  p.nchunks = int(ceil_div(g.Cg, p.Cc));
  p.ctiles = int(ceil_div(g.Coutg, p.BM));
  p.grid[0] = p.tiles_per_plane;
  p.grid[1] = g.N * g.O[0];
  p.grid[2] = g.G * p.ctiles;

  if (p.grid[0] > std::numeric_limits<int32_t>::max() || p.grid[1] > 65535 || p.grid[2] > 65535)
    return CONV_ERR_OVERFLOW;
  *out = p;
  return CONV_OK;
}

#define CONVHIP_FUSED_DESC(id, CIN, KH, KW, NG, O2, ROWS, RT, GRP, E4) {id, CIN, KH, KW, NG, O2, ROWS, RT, GRP, E4},
static const FusedSpecDesc kFusedSpecs[] = {CONVHIP_FUSED_SPECS(CONVHIP_FUSED_DESC)};
#undef CONVHIP_FUSED_DESC

const FusedSpecDesc* fused_specs(int* count) {
  *count = int(sizeof(kFusedSpecs) / sizeof(kFusedSpecs[0]));
  return kFusedSpecs;
}

// Plan of a depth-streamed specialisation if the geometry is the one it was built for.
static bool plan_fused_stream(const Geom& g, int min_dim, const FusedSpecDesc& d, FusedPlan* p) {
  // Columns along W, contiguous in NCDHW (16-byte row copies), for a minimum
  // over D or H; element copies for a minimum over W (columns along H) and for
  // channels-last input (columns C_in floats apart).
  if (d.E4 != ((min_dim == 4 || g.cl) ? 1 : 0)) return false;
  if (g.G != d.GRP || g.Cin != d.CIN || g.K[0] != 3 || g.K[1] != d.KH || g.K[2] != d.KW) return false;
  // A block of 4 output channels lies inside one group.
  if (d.GRP > 1 && g.Coutg % 4 != 0) return false;
  for (int i = 0; i < 3; i++)
    if (g.S[i] != 1 || g.Dl[i] != 1) return false;
  if ((g.Cout + 3) / 4 != d.NG || g.O[2] != d.O2) return false;
  // Input rows are copied whole (16-byte chunks unless E4): no padding along
  // the column axis.
  if (g.P[2] != 0 || g.L[2] != d.O2 + d.KW - 1 || (!d.E4 && g.L[2] % 4 != 0)) return false;
  const int64_t plane_out = g.plane_out();
  int64_t tiles;
  if (d.RT > 0) {
    // Tiles of RT whole output rows.
    if (d.RT * d.O2 > 64 || d.ROWS != d.RT + d.KH - 1) return false;
    tiles = (g.O[1] + d.RT - 1) / d.RT;
  } else {
    tiles = (plane_out + 63) / 64;
    for (int64_t t = 0; t < tiles; t++) {
      const int64_t p0 = 64 * t, p1 = std::min(p0 + 63, plane_out - 1);
      if (p1 / g.O[2] - p0 / g.O[2] + d.KH > d.ROWS) return false;
    }
  }
  if (g.Cin * g.L[0] * g.L[1] * g.L[2] > std::numeric_limits<int32_t>::max()) return false;
  // Two waves split the output depths of each tile: twice the waves in flight,
  // at the cost of staging two extra input planes per tile.
  const int dsplit = g.O[0] >= 2 ? 2 : 1;
  const int64_t units = g.N * tiles * dsplit;
  if (units > std::numeric_limits<int32_t>::max() - 4) return false;
  FusedPlan q;
  q.spec = d.id;
  q.dsplit = dsplit;
  q.units = units;
  q.ng = d.NG;
  q.cpad = 4 * d.NG;
  q.mode = TILE_FLAT;
  q.dspan = int(g.O[0] + 2);
  q.rows = d.ROWS;
  q.bw = d.O2 + d.KW - 1;
  q.kfull = int(g.Cin * g.kvol());
  q.tiles_per_plane = tiles;
  const int64_t slot = int64_t(d.CIN) * d.ROWS * q.bw;
  q.boxc = int(slot);
  // 4 waves x 4 ring slots, or the epilogue's partial minima and channel
  // transpose areas if larger.
  q.lds_bytes = 4 * std::max<int64_t>(4 * 4 * slot, 4 * int64_t(d.NG) * 64 * 4 + 4 * 1024);
  q.grid[0] = (units + 3) / 4;
  q.grid[1] = 1;
  q.grid[2] = 1;
  *p = q;
  return true;
}

int plan_fused(const Geom& g, int min_dim, FusedPlan* out, bool allow_spec) {
  if (g.nd != 3) return CONV_ERR_RANK;
  // g is in the kernels' axis order (the minimum over axis 0).
  if (min_dim < 2 || min_dim > 4) return CONV_ERR_UNSUPPORTED;
  if (allow_spec) {
    int ns = 0;
    const FusedSpecDesc* specs = fused_specs(&ns);
    for (int i = 0; i < ns; i++)
      if (plan_fused_stream(g, min_dim, specs[i], out)) return CONV_OK;
  }
  FusedPlan p;
  // At most 64 output channels (16 blocks of 4) per pass over a group's
  // reduction: more run as several channel chunks of the group, each reducing
  // over the group's whole input, their minima merged in LDS before the softmax.
  p.cchunks = int((g.Coutg + 63) / 64);
  p.cpad = int(((g.Coutg + p.cchunks - 1) / p.cchunks + 3) / 4 * 4);
  p.ng = p.cpad / 4;
  const int64_t units = g.G * p.cchunks;
  const int BN = 64;
  p.mode = (g.O[2] * 2 <= BN) ? TILE_FLAT : TILE_ROW;
  box_dims(g, p.mode, BN, &p.rows, &p.bw, &p.tiles_per_plane, &p.row_tiles);
  if (p.mode == TILE_FLAT && (BN / g.O[2]) * g.O[2] * 8 >= BN * 7) {
    // Tiles of whole output rows when they fill at least 7/8 of the lanes: the
    // box then holds exactly the rows those outputs read (64 consecutive
    // positions can straddle one more row), so more workgroups fit a unit.
    const int64_t r = BN / g.O[2];
    p.tile_pos = int(r * g.O[2]);
    p.rows = int((r - 1) * g.S[1] + (g.K[1] - 1) * g.Dl[1] + 1);
    p.tiles_per_plane = ceil_div(g.O[1], r);
  }
  p.dspan = int((g.O[0] - 1) * g.S[0] + (g.K[0] - 1) * g.Dl[0] + 1);
  const int64_t boxc = int64_t(p.dspan) * p.rows * p.bw;
  p.kfull = int(g.Cin * g.kvol());
  p.kg = int(g.Cg * g.kvol());
  p.kgp = (p.kg + 3) / 4 * 4;
  // Weight rows of an odd number of 16-byte quads: the lanes' 16-byte reads of
  // one k-quad fall in distinct banks.
  p.kgs = ((p.kgp / 4) % 2 == 1) ? p.kgp : p.kgp + 4;
  const int64_t nrows = g.Cin * int64_t(p.dspan) * p.rows;
  const int64_t box = g.Cin * boxc;
  const int64_t red = 4 * int64_t(p.cpad) * 64;  // per-wave minima of one group (chunk)
  // One pass: the minima reuse the box space once it is read for the last time.
  const int64_t region = units == 1 ? std::max(box, red) : box;
  int64_t off = (region + 3) / 4 * 4;
  const int64_t ko_off = off;
  off += p.kgp;
  off = (off + 3) / 4 * 4;
  const int64_t wt_off = off;
  off += units * int64_t(p.cpad) * p.kgs;
  int64_t red_off = 0, fin_off = 0;
  if (units > 1) {
    red_off = off;
    off += red;
    fin_off = off;
    off += g.Cout * 64;
  }
  p.lds_bytes = 4 * off;
  if (p.lds_bytes > kLdsLimit || boxc > (int64_t(1) << 28))
    return CONV_ERR_UNSUPPORTED;
  p.nrows = int(nrows);
  p.ko_off = int(ko_off);
  p.wt_off = int(wt_off);
  p.red_off = int(red_off);
  p.fin_off = int(fin_off);
  p.boxc = int(boxc);
  p.grid[0] = p.tiles_per_plane;
  p.grid[1] = g.N;
  p.grid[2] = 1;
  if (p.grid[0] > std::numeric_limits<int32_t>::max() || p.grid[1] > 65535) return CONV_ERR_OVERFLOW;
  *out = p;
  return CONV_OK;
}

std::string describe(const Geom& g, const ConvPlan& p) {
  char buf[512];
  CfgShape cs = cfg_shape(p.cfg);
  if (p.tap_spec >= 0 && g.cl) {
    int n = 0;
    const TapClSpecDesc& d = tap_cl_specs(&n)[p.tap_spec];
    cs = CfgShape{d.MT, d.NT, d.WM, d.WN, 1};
  } else if (p.tap_spec >= 0) {
    int n = 0;
    const TapSpecDesc& d = tap_specs(&n)[p.tap_spec];
    cs = CfgShape{d.MT, d.NT, d.WM, d.WN, 1};
  } else if (p.split_spec >= 0) {
    int n = 0;
    const SplitSpecDesc& d = split_specs(&n)[p.split_spec];
    cs = CfgShape{1, d.NT, 1, 1, d.NW};
  } else if (p.ks_spec >= 0) {
    int n = 0;
    const KsSpecDesc& d = ks_specs(&n)[p.ks_spec];
    cs = CfgShape{1, d.T, 1, 1, 4};
  } else if (p.direct_spec >= 0) {
    cs = CfgShape{1, 1, 1, 1, 1};
  }
  std::snprintf(buf, sizeof buf,
                "kernel=%s%s cfg=%d MT=%d NT=%d WM=%d WN=%d KS=%d BM=%d BN=%d mode=%s Cc=%d kc_pad=%d "
                "box=%dx%dx%d grid=%lldx%lldx%lld lds=%lld macs=%lld",
                p.tap_spec >= 0    ? "conv_tap"
                : p.direct_spec >= 0 ? "conv_direct16"
                : p.ks_spec >= 0   ? "conv_tap_kstream"
                : p.split_spec >= 0 ? (p.split_pipe ? "conv_tap_split pipe=1" : "conv_tap_split")
                                    : "conv_mfma16",
                g.cl ? (p.cl_vec ? " layout=channels_last copy=quad" : " layout=channels_last copy=scalar") : "",
                p.tap_spec >= 0      ? p.tap_spec
                : p.direct_spec >= 0 ? p.direct_spec
                : p.ks_spec >= 0     ? p.ks_spec
                : p.split_spec >= 0  ? p.split_spec
                                     : p.cfg,
                cs.MT, cs.NT,
                cs.WM, cs.WN, cs.KS, p.BM, p.BN, p.mode == TILE_FLAT ? "flat" : "row", p.Cc,
                p.kc_pad, p.kdspan, p.rows, p.bw, (long long)p.grid[0], (long long)p.grid[1],
                (long long)p.grid[2], (long long)p.lds_bytes, (long long)g.macs());
  return buf;
}

std::string describe(const Geom& g, const FusedPlan& p) {
  char buf[512];
  if (p.spec >= 0) {
    std::snprintf(buf, sizeof buf,
                  "kernel=fused_stream spec=%d ng=%d cpad=%d groups=%lld planes=%d rows=%d bw=%d tiles=%lld dsplit=%d "
                  "units=%lld grid=%lldx%lldx%lld lds=%lld macs=%lld",
                  p.spec, p.ng, p.cpad, (long long)g.G, p.dspan, p.rows, p.bw, (long long)p.tiles_per_plane, p.dsplit,
                  (long long)p.units,
                  (long long)p.grid[0], (long long)p.grid[1], (long long)p.grid[2], (long long)p.lds_bytes,
                  (long long)g.macs());
    return buf;
  }
  // Multiply-adds the matrix cores perform: every tile's 64 positions, every
  // output depth, each group's channels rounded up to 4, over the group's
  // reduction rounded up to 4 (no products across groups).
  const int64_t issued = int64_t(p.grid[0]) * p.grid[1] * 64 * g.O[0] * g.G * p.cchunks * p.cpad * p.kgp;
  std::snprintf(buf, sizeof buf,
                "kernel=fused_min_softmax_mfma4 ng=%d cpad=%d chunks=%d groups=%lld kred=%d mode=%s tile=%d "
                "box=%dx%dx%dx%d grid=%lldx%lldx%lld lds=%lld macs=%lld issued=%lld",
                p.ng, p.cpad, p.cchunks, (long long)g.G, p.kg, p.mode == TILE_FLAT ? "flat" : "row",
                p.mode == TILE_FLAT ? p.tile_pos : 64, int(g.Cin), p.dspan, p.rows,
                p.bw, (long long)p.grid[0], (long long)p.grid[1], (long long)p.grid[2], (long long)p.lds_bytes,
                (long long)g.macs(), (long long)issued);
  return buf;
}

}  // namespace convhip
