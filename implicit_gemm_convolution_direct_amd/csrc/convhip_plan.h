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

// Tile configurations of the fp32 MFMA implicit-GEMM conv kernel. Each wave
// owns MT x NT tiles of 16 (output channels) x 16 (output positions); the block
// is WM x WN waves.
enum ConvCfg : int {
  CFG_M16 = 0,   // MT=1 NT=4 WM=1 WN=4 : 16 channels x 256 positions
  CFG_M32 = 1,   // MT=2 NT=4 WM=1 WN=4 : 32 x 256
  CFG_M64 = 2,   // MT=4 NT=4 WM=1 WN=4 : 64 x 256
  CFG_M128 = 3,  // MT=4 NT=4 WM=2 WN=2 : 128 x 128
  CFG_COUNT = 4
};
struct CfgShape { int MT, NT, WM, WN; };
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
  int ldw = 0;         // LDS row stride (floats) of the staged weight chunk [k][m]
  int kdspan = 0;      // input planes in the box: (kD-1)*dD + 1
  int rows = 0;        // input rows in the box (maximum over tiles)
  int bw = 0;          // input columns in the box
  int boxc = 0;        // floats per channel in the box: kdspan * rows * bw
  int64_t tiles_per_plane = 0;
  int row_tiles = 0;   // TILE_ROW: tiles per output row
  int ctiles = 0;      // channel tiles per group
  int64_t grid[3] = {0, 0, 0};
  int64_t lds_bytes = 0;
};

// Plan for conv_fwd. Returns a conv_status (CONV_ERR_UNSUPPORTED if nothing fits).
int plan_conv(const Geom& g, ConvPlan* p);

// Plan of the fused conv -> min over depth -> softmax over channels kernel.
struct FusedPlan {
  int ng = 0;          // channel groups of 4 handled by one lane
  int cpad = 0;        // C_out rounded up to 4
  int mode = TILE_FLAT;
  int dspan = 0;       // input planes staged: (D_out-1)*sD + (kD-1)*dD + 1
  int rows = 0, bw = 0, boxc = 0;
  int kfull = 0;       // C_in * kvol
  int64_t tiles_per_plane = 0;
  int row_tiles = 0;
  int64_t grid[3] = {0, 0, 0};
  int64_t lds_bytes = 0;
};
int plan_fused(const Geom& g, int min_dim, FusedPlan* p);

std::string describe(const Geom& g, const ConvPlan& p);
std::string describe(const Geom& g, const FusedPlan& p);

constexpr int64_t kLdsLimit = 160 * 1024;  // bytes of LDS per workgroup on gfx950

}  // namespace convhip
