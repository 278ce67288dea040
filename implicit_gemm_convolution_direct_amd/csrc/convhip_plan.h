// Host-side geometry and launch planning shared by the library's kernels and
// entry points. Pure host code: no HIP calls, so it can be reasoned about and
// exercised without a GPU.
#pragma once

#include <cstdint>
#include <string>

namespace convhip {

// A convolution viewed on three spatial axes (D, H, W). A 1-D convolution is
// the case D = H = 1, kD = kH = 1 with its length on the W axis.
struct Geom {
  int nd = 3;
  bool cl = false;            // channels-last tensors: x [N, D, H, W, C_in], y [N, D_out, H_out, W_out, C_out]
  bool x_aligned16 = true;    // channels-last: x starts on a 16-byte boundary
  bool w_aligned16 = true;    // channels-last: w starts on a 16-byte boundary
  int64_t N = 0, Cin = 0, Cout = 0, G = 1, Cg = 0, Coutg = 0;
  int64_t L[3] = {1, 1, 1};   // input D, H, W
  int64_t K[3] = {1, 1, 1};   // kernel kD, kH, kW
  int64_t S[3] = {1, 1, 1};   // stride
  int64_t Dl[3] = {1, 1, 1};  // dilation
  int64_t P[3] = {0, 0, 0};   // zero padding (both sides)
  int64_t O[3] = {1, 1, 1};   // output D_out, H_out, W_out
  int64_t kvol() const { return K[0] * K[1] * K[2]; }
  int64_t kred() const { return Cg * kvol(); }           // reduction length per output
  int64_t plane_out() const { return O[1] * O[2]; }       // outputs per (n, co, od)
  int64_t macs() const { return N * Cout * O[0] * O[1] * O[2] * kred(); }
};

// Output length of one axis, floor division (may be <= 0).
int64_t out_len(int64_t L, int64_t k, int64_t s, int64_t d, int64_t p);

// Validate the user's arguments and fill g. Returns a conv_status value.
int make_geom(int nd, const int64_t* x_shape, const int64_t* w_shape, const int* stride,
              const int* dilation, const int* padding, int groups, Geom* g);
// The same for a channels-last input, x_shape = [N, spatial..., C_in]; sets g->cl.
int make_geom_channels_last(int nd, const int64_t* x_shape, const int64_t* w_shape, const int* stride,
                            const int* dilation, const int* padding, int groups, Geom* g);

// Tile configurations of the fp32 MFMA implicit-GEMM conv kernel. Each wave
// owns MT x NT tiles of 16 (output channels) x 16 (output positions); the block
// holds WM x WN such wave tiles, and KS waves split the reduction of each wave
// tile (their partial sums are added through LDS). WM * WN * KS = 4 waves.
struct CfgShape { int MT, NT, WM, WN, KS; };
enum ConvCfg : int {
  CFG_M64 = 0,       // 64 x 256, no split     (64 < C_out/g)
  CFG_M128 = 1,      // 128 x 128, no split    (C_out/g > 64)
  CFG_M32 = 2,       // 32 x 256, no split
  CFG_M16 = 3,       // 16 x 256, no split
  CFG_M16_N64_K4 = 4,    // 16 x 64, reduction split over 4 waves
  CFG_M16_N128_K4 = 5,   // 16 x 128, split 4
  CFG_M16_N208_K4 = 6,   // 16 x 208, split 4
  CFG_M16_N256_K4 = 7,   // 16 x 256, split 4
  CFG_COUNT = 8
};
CfgShape cfg_shape(int cfg);

// Tiling of output positions inside one (n, od) plane of H_out x W_out outputs.
enum TileMode : int {
  TILE_FLAT = 0,  // BN consecutive flattened (oh, ow) positions; box spans whole input rows
  TILE_ROW = 1,   // BN consecutive ow of one output row; box spans that segment only
};

struct ConvPlan {
  int cfg = CFG_M64;
  int BM = 0, BN = 0;
  int mode = TILE_FLAT;
  int Cc = 0;          // input channels staged per chunk
  int kc_pad = 0;      // Cc * kvol rounded up to a multiple of 4
  int kdspan = 0;      // input planes in the box: (kD-1)*dD + 1
  int rows = 0;        // input rows in the box (maximum over tiles)
  int bw = 0;          // input columns in the box
  int boxc = 0;        // floats per channel in the box: kdspan * rows * bw (channels-last: sites)
  int ccp = 0;         // channels-last: LDS floats per box site (Cc padded against bank conflicts)
  bool cl_vec = false; // channels-last: box copied in 16-byte channel quads
  int xs_floats = 0;   // LDS floats of the box region (box, or the split-K partial sums if larger)
  int koff_ints = 0;   // LDS ints of the tap-offset table (padded for prefetch)
  int ws_floats = 0;   // LDS floats of the weight fragments (padded for prefetch)
  int64_t tiles_per_plane = 0;
  int row_tiles = 0;   // TILE_ROW: tiles per output row
  int ctiles = 0;      // channel tiles per group
  int nchunks = 0;      // chunks of Cc input channels per tile
  int tap_spec = -1;    // >= 0: build-time specialised persistent kernel (grid[0] workgroups walk `items`)
  int split_spec = -1;  // >= 0: build-time specialised channel-split kernel
  int split_pipe = 0;   // channel-split kernel summing the first tile batch during the second's products
  int ks_spec = -1;     // >= 0: build-time specialised workgroup-stream-K kernel (one plane per workgroup)
  int direct_spec = -1; // >= 0: build-time specialised direct kernel (small convolutions, no LDS)
  int threads = 256;    // workgroup size
  int64_t items = 0;    // tap kernel: work items (tile, plane)
  int64_t grid[3] = {0, 0, 0};
  int64_t lds_bytes = 0;
};

// Plan for conv_fwd. Returns a conv_status (CONV_ERR_UNSUPPORTED if nothing fits).
// force_cfg >= 0 selects a tile configuration (tests cover every configuration).
// Build-time specialisations of the persistent tap-unrolled kernel: each fixes
// the tiling, the channel chunk, the kernel taps and dilations, and the staged
// box's extents: at most ROWS input rows per plane at a row pitch of BW floats
// (a geometry whose tiles need fewer rows or columns stages the box at the same
// pitch). X(id, MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW)
#define CONVHIP_TAP_SPECS(X)                                                      \
  /* Conv3d 3->64, kernel 3x5x7, inputs up to 64 wide whose 256-position tiles \
     span <= 10 input rows (64^3): 64 ch x 256 positions, 8 waves */            \
  X(0, 4, 2, 1, 8, 1, 3, 5, 7, 1, 1, 1, 3, 3, 10, 64)                            \
  /* Conv1d 64->128, k=3, stride 3, dilation 4: 128 ch x 256 positions; the   \
     774-float input segment is copied as 776 (16-byte chunks) */               \
  X(1, 4, 4, 2, 4, 8, 1, 1, 3, 1, 1, 4, 8, 1, 1, 776)                            \
  /* the Conv3d 3->64 kernel 3x5x7 on narrower inputs (tiles span <= 12 rows, \
     e.g. 48^3) */                                                               \
  X(2, 4, 2, 1, 8, 1, 3, 5, 7, 1, 1, 1, 3, 3, 12, 64)                            \
  /* Conv1d 64->96, k=3, dilation 2: 96 ch x 256 positions */                   \
  X(3, 3, 4, 2, 4, 8, 1, 1, 3, 1, 1, 2, 8, 1, 1, 776)

// Build-time specialisations of the channel-split kernel (one input channel per
// wave, <= 16 output channels per group).
// X(id, NT, NW, KD, KH, KW, DD, DH, DW, F, ROWS, BW, TS): the staged box keeps
// every F-th input column, ROWS input rows and BW kept columns per plane; each
// (n, od) output plane is split into TS workgroups of NT 16-position tiles.
#define CONVHIP_SPLIT_SPECS(X)                                                     \
  /* Conv3d 16->32, groups 2, kernel 3x5x7, stride (1,2,2), dilation (1,1,2) */  \
  X(0, 13, 8, 3, 5, 7, 1, 1, 2, 2, 35, 20, 1)                                     \
  /* Conv3d 3->8, kernel 3x3x3 on 16^3: 7 workgroups of 2 tiles per plane */   \
  X(1, 2, 3, 3, 3, 3, 1, 1, 1, 1, 16, 16, 7)

// The pipelined channel-split kernel runs a plane's NT tiles in two batches
// (ceil(NT/2), then floor(NT/2)), sums each batch's tiles one per wave, and
// copies each wave's weight slice in 16-byte pieces: it needs NT >= 8 (two
// batches worth overlapping), ceil(NT/2) <= NW and a group reduction length
// (C_in/groups * kvol) that is a multiple of 4.
constexpr bool split_pipe_fits(int NT, int NW, int wrow) {
  return NT >= 8 && (NT + 1) / 2 <= NW && wrow % 4 == 0;
}

// Build-time specialisations of the workgroup-stream-K kernel (conv_tap_kstream):
// one workgroup of 4 waves per (n, od) output plane and group, <= 16 output
// channels per group, the plane's T tiles of 16 positions split over the
// waves (T/4 whole tiles each, the T % 4 others split by reduction blocks).
// X(id, CG, KD, KH, KW, DH, DW, F, ROWS, BW, T): C_in/groups = CG, kernel
// KD x KH x KW, dilations DH, DW along H and W (any along D), and a staged box
// of at most ROWS input rows by BW kept columns (every F-th input column) per
// (channel, depth tap) plane; the rows and columns a geometry needs may be fewer.
#define CONVHIP_KSTREAM_SPECS(X)                                                   \
  /* Conv3d 16->32, groups 2, kernel 3x5x7, stride (1,2,2), dilation (1,1,2):  \
     32x32 inputs (16x13 outputs, 13 tiles) */                                   \
  X(0, 8, 3, 5, 7, 1, 2, 2, 35, 20, 13)                                          \
  /* the same on 24x24 inputs (12x9 outputs, 7 tiles): the box of exactly      \
     the rows and columns they read */                                           \
  X(1, 8, 3, 5, 7, 1, 2, 2, 27, 15, 7)

// Build-time specialisations of the direct kernel (conv_direct16) for small
// convolutions: one wave per 16 output positions and all <= 16 output channels
// of a group, operands read from global memory into registers. Zero padding 0.
// X(id, CIN, KD, KH, KW, DD, DH, DW): C_in/groups, kernel and dilations.
#define CONVHIP_DIRECT_SPECS(X)                     \
  /* Conv3d 3->8, kernel 3x3x3 (16^3 inputs) */   \
  X(0, 3, 3, 3, 3, 1, 1, 1)

struct DirectSpecDesc {
  int id, CIN, KD, KH, KW, DD, DH, DW;
};
const DirectSpecDesc* direct_specs(int* count);

// Largest convolution the direct kernel takes: its waves read every operand
// from global memory, which suits launches dominated by latency, not larger ones.
constexpr int64_t kDirectMaxMacs = 16ll << 20;

struct KsSpecDesc {
  int id, CG, KD, KH, KW, DH, DW, F, ROWS, BW, T;
};
const KsSpecDesc* ks_specs(int* count);

struct SplitSpecDesc {
  int id, NT, NW, KD, KH, KW, DD, DH, DW, F, ROWS, BW, TS;
};
const SplitSpecDesc* split_specs(int* count);

struct TapSpecDesc {
  int id, MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW;
};
const TapSpecDesc* tap_specs(int* count);

// The persistent tap kernel on channels-last input (x [N, spatial..., C_in]):
// the staged box holds CCP floats per input site (channels innermost; copied as
// 16-byte quads when CC and CCP are multiples of 4, else float by float).
// X(id, MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW, CCP)
// with BW input sites per box row.
#define CONVHIP_TAP_CL_SPECS(X)                                                       \
  /* Conv1d 64->128, k=3, stride 3, dilation 4: 128 ch x 256 positions, 8 input  \
     channels per chunk, 774 input sites per tile */                               \
  X(0, 4, 4, 2, 4, 8, 1, 1, 3, 1, 1, 4, 8, 1, 1, 774, 8)                            \
  /* Conv3d 3->64, kernel 3x5x7, 64^3 input: 64 ch x 256 positions, 8 waves */   \
  X(1, 4, 2, 1, 8, 1, 3, 5, 7, 1, 1, 1, 3, 3, 10, 64, 3)

struct TapClSpecDesc {
  int id, MT, NT, WM, WN, NCH, KD, KH, KW, DD, DH, DW, CC, KDSPAN, ROWS, BW, CCP;
};
const TapClSpecDesc* tap_cl_specs(int* count);

// num_cu: compute units of the device (sizes the persistent grid).
// use_tap: -1 planner's choice, 0 never use a tap specialisation. Channels-last
// geometries (g.cl) take the channels-last tap specialisations (tap_spec then
// indexes CONVHIP_TAP_CL_SPECS), the channel-split specialisations or the
// generic kernel.
// split_kernel: for geometries the channel-split family serves, 0 = the
// planner's choice (stream-K kernel, else the pipelined channel-split kernel),
// 1 = the pipelined channel-split kernel, 2 = the channel-split kernel that sums
// after all products.
int plan_conv(const Geom& g, ConvPlan* p, int force_cfg = -1, int num_cu = 256, int use_tap = -1,
              int split_kernel = 0);

// Direct convolution on the vector ALU (conv_valu_kernel, valu_kernels.hip):
// any geometry, channels-first or channels-last, whose weights of one (input channel, depth tap) pair,
// double-buffered (2 x kH x kW x CO floats), fit in 64 KiB of LDS. CO output
// channels and pp positions per lane, `threads` lanes per workgroup; grid[0]
// position blocks, grid[1] = groups x ncob channel blocks. conv_fwd takes it for geometries the
// matrix-core kernels cannot stage, and when CONVHIP_VALU=1 forces it.
struct ValuPlan {
  int co = 0, pp = 0, ncob = 0;
  int threads = 256;
  int pps = 1;  // (input channel, depth tap) pairs per staged LDS buffer
  int64_t grid[2] = {0, 0};
  int lds_bytes = 0;
};
int plan_valu(const Geom& g, ValuPlan* p);
// Enqueue the kernel on `stream` (a hipStream_t). Returns a conv_status.
int launch_valu(const Geom& g, const ValuPlan& p, const float* x, const float* w, const float* bias, float* y,
                void* stream);

// Build-time specialisations of the depth-streamed fused kernel (stride 1,
// dilation 1, kD = 3, streamed over the min axis): X(id, CIN, KH, KW, NG, O2,
// ROWS, RT, GRP, E4) with NG blocks of 4 output channels, O2 output columns,
// at most ROWS staged input rows per wave tile and GRP conv groups (each
// channel block reduces over its own group's CIN/GRP input channels only; with
// GRP > 1 a block may not straddle two groups: C_out/GRP a multiple of 4).
// E4 = 0: the column axis is W (contiguous), input rows copied in 16-byte
// chunks (minimum over D or H); E4 = 1: columns run along H with W streamed
// (minimum over W), every input element copied on its own (4 bytes). RT > 0:
// a wave tile is RT whole output rows (RT * O2 <= 64 positions, lanes past
// them idle; ROWS = RT + KH - 1); RT = 0: 64 consecutive positions.
#define CONVHIP_FUSED_SPECS(X)                                                    \
  /* Conv3d 3->24, kernel 3x3x3, 32x32 planes (30 output columns): tiles of 2 rows */ \
  X(0, 3, 3, 3, 6, 30, 4, 2, 1, 0)                                               \
  /* the same with 3 groups (1 input and 8 output channels per group) */       \
  X(1, 3, 3, 3, 6, 30, 4, 2, 3, 0)                                               \
  /* the same streamed over W (minimum over W): columns along H */               \
  X(2, 3, 3, 3, 6, 30, 4, 2, 1, 1)

struct FusedSpecDesc {
  int id, CIN, KH, KW, NG, O2, ROWS, RT, GRP, E4;
};
const FusedSpecDesc* fused_specs(int* count);

// Plan of the fused conv -> min over depth -> softmax over channels kernel.
struct FusedPlan {
  int spec = -1;       // >= 0: depth-streamed specialisation (one wave per 64 positions)
  int dsplit = 1;      // streamed: waves sharing the output depths of one 64-position tile
  int64_t units = 0;   // streamed: N * tiles_per_plane * dsplit waves
  int ng = 0;          // blocks of 4 output channels handled by one lane (per group)
  int cpad = 0;        // output channels per group rounded up to 4
  int mode = TILE_FLAT;
  int dspan = 0;       // input planes staged: (D_out-1)*sD + (kD-1)*dD + 1
  int rows = 0, bw = 0, boxc = 0;
  int kfull = 0;       // C_in * kvol
  // Generic kernel: reduction of one group (C_in/groups * kvol), rounded up to 4,
  // LDS weight row pitch; box rows; LDS float offsets of its regions.
  int kg = 0, kgp = 0, kgs = 0, nrows = 0;
  int cchunks = 1;     // generic kernel: output-channel chunks of at most 64 per group
  int tile_pos = 64;   // generic kernel, TILE_FLAT: output positions per tile
  int ko_off = 0, wt_off = 0, red_off = 0, fin_off = 0;
  int64_t tiles_per_plane = 0;
  int row_tiles = 0;
  int64_t grid[3] = {0, 0, 0};
  int64_t lds_bytes = 0;
};
// allow_spec: false skips the build-time specialisations (tests of the generic kernel).
int plan_fused(const Geom& g, int min_dim, FusedPlan* p, bool allow_spec = true);

std::string describe(const Geom& g, const ConvPlan& p);
std::string describe(const Geom& g, const FusedPlan& p);

constexpr int64_t kLdsLimit = 160 * 1024;  // bytes of LDS per workgroup on gfx950

}  // namespace convhip
