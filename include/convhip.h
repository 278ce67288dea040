/*
 * convhip.h -- C ABI of the MI355X (gfx950) fp32 convolution library.
 *
 * Operations (the problem statements of the POPCORNBENCH "Kimi-K2.6" pages
 * l1_p60 "Conv3d, asymmetric 3x5x7 kernel", l1_p76 "Conv1d, stride 3,
 * dilation 4" and l2_p24 "Conv3d + min + softmax", each page's opening turn):
 *
 *   conv_fwd            y = Conv{1,3}d(x, w, bias; stride, dilation, zero padding, groups)
 *   conv3d_min_softmax  y = softmax over channels of (min over depth of Conv3d(x, w, bias))
 *                       (and its channels-last form)
 *   min_over_axis, softmax_over_channels   that op's last two steps, unfused
 *
 * Conventions shared by every entry point
 *   - Tensors are fp32, contiguous, row-major (NCL / NCDHW). Pointers named x, w,
 *     bias, y are DEVICE pointers on the current HIP device; shape and parameter
 *     arrays are HOST pointers, read during the call only.
 *   - The caller owns every buffer. The library allocates no device memory.
 *   - Work is enqueued on `stream` (0 = the null stream); the call returns after
 *     enqueue. The caller synchronises before reading y.
 *   - Arguments are validated before anything is launched; a negative status is
 *     returned and nothing runs. A failed launch returns CONV_ERR_HIP.
 *   - y must not alias x, w or bias. Only zero padding exists.
 *   - Results are computed in fp32 with fp32 accumulation (products of fp32
 *     inputs summed by the matrix cores); no reduced-precision arithmetic.
 */
#ifndef CONVHIP_H
#define CONVHIP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t without including HIP headers: an opaque stream handle. */
typedef struct ihipStream_t *convhip_stream_t;

typedef enum {
  CONV_OK = 0,
  CONV_ERR_NULL = -1,         /* a required pointer is NULL */
  CONV_ERR_RANK = -2,         /* nd not 1, 2 or 3 */
  CONV_ERR_SHAPE = -3,        /* non-positive dimension, or w's C_in/groups mismatch */
  CONV_ERR_GROUPS = -4,       /* groups < 1, or C_in or C_out not divisible by groups */
  CONV_ERR_PARAM = -5,        /* stride < 1, dilation < 1 or padding < 0 */
  CONV_ERR_EMPTY_OUTPUT = -6, /* some output length <= 0 */
  CONV_ERR_UNSUPPORTED = -7,  /* valid, but not handled by the library (stated per entry point) */
  CONV_ERR_OVERFLOW = -8,     /* a size does not fit the index arithmetic */
  CONV_ERR_HIP = -9           /* the HIP runtime reported an error at launch */
} conv_status;

/*
 * Output length per spatial axis. The formula is the one page l1_p76 states in
 * its turns 1 and 2 when sizing the Conv1d output (174758 for L = 524280, k = 3,
 * stride 3, dilation 4); page l2_p24 turn 1 and page l1_p60's monologue apply it
 * per axis to their Conv3d outputs. Division is floor division here (the
 * pages' C code truncates toward zero, which gives one output, not zero, for a
 * numerator of -1):
 *   out[i] = floor((in[i] + 2*padding[i] - dilation[i]*(k[i]-1) - 1) / stride[i]) + 1
 * nd in {1, 2, 3}. Writes out_spatial[0..nd-1] (which may be <= 0) and returns
 * CONV_OK, or CONV_ERR_EMPTY_OUTPUT if any entry is <= 0 (the entries are still
 * written), or CONV_ERR_PARAM / CONV_ERR_NULL / CONV_ERR_RANK. Host only.
 */
int conv_out_shape(int nd, const int64_t *in_spatial, const int64_t *k_spatial,
                   const int *stride, const int *dilation, const int *padding,
                   int64_t *out_spatial);

/*
 * Forward convolution (pages l1_p60 and l1_p76, opening turns: nn.Conv3d /
 * nn.Conv1d forward).
 *   nd = 1: x [N, C_in, L],       w [C_out, C_in/groups, k],            y [N, C_out, L_out]
 *   nd = 2: x [N, C_in, H, W],    w [C_out, C_in/groups, kH, kW],       y [N, C_out, H_out, W_out]
 *   nd = 3: x [N, C_in, D, H, W], w [C_out, C_in/groups, kD, kH, kW],   y [N, C_out, D_out, H_out, W_out]
 *   (nd = 2 is the 3-D case with D = kD = 1: the pages' rank-generic loops
 *   cover it; it is the rank between their Conv1d and Conv3d.)
 *   y[n,co,o] = bias[co] + sum_{c', t} w[co,c',t] * x[n, g(co)*C_in/groups + c', o*stride + t*dilation - padding]
 *   with out-of-range input reading as 0 and g(co) = co / (C_out/groups).
 * x_shape / w_shape: nd+2 host entries. stride, dilation, padding: nd host
 * entries each. bias: device pointer to C_out floats, or NULL for none.
 * y: device buffer of N*C_out*prod(out) floats, preallocated by the caller.
 * fp32 products and fp32 accumulation in an unspecified order. A NaN input
 * makes NaN every output whose receptive field holds it; infinite inputs give
 * unspecified results (a padded zero-weight term may turn them into NaN).
 * Kernels: fp32 matrix cores wherever a tile's input box fits in LDS; other
 * geometries (large kernels over many channels) run on a vector-ALU direct
 * kernel. CONV_ERR_UNSUPPORTED only if neither fits: the vector kernel needs
 * 2 * kH * kW * CO * 4 bytes <= 64 KiB (CO = 8 if C_out/groups <= 8, else 16).
 */
int conv_fwd(int nd,
             const float *x, const int64_t *x_shape,
             const float *w, const int64_t *w_shape,
             const float *bias,
             const int *stride, const int *dilation, const int *padding, int groups,
             float *y, convhip_stream_t stream);

/*
 * Forward convolution on channels-last tensors (page l1_p60, opening turn: the
 * NDHWC layout is weighed there for coalesced input reads). The same operation
 * as conv_fwd; only the memory order of x and y differs:
 *   nd = 1: x [N, L, C_in],       y [N, L_out, C_out]
 *   nd = 2: x [N, H, W, C_in],    y [N, H_out, W_out, C_out]
 *   nd = 3: x [N, D, H, W, C_in], y [N, D_out, H_out, W_out, C_out]
 *   y[n,o,co] = bias[co] + sum_{c', t} w[co,c',t] * x[n, o*stride + t*dilation - padding, g(co)*C_in/groups + c']
 * x_shape: nd+2 host entries in the channels-last order above ([N, spatial..., C_in]).
 * w keeps the conv_fwd layout [C_out, C_in/groups, k...] (w_shape likewise);
 * bias [C_out] or NULL. y: device buffer of N*prod(out)*C_out floats. Status
 * codes, ownership, stream semantics and the kernel choice (matrix cores, or the
 * vector-ALU direct kernel where no matrix-core kernel fits) as conv_fwd. Any
 * pointer alignment is accepted (16-byte aligned y with C_out and C_out/groups
 * multiples of 4 takes vector stores).
 */
int conv_fwd_channels_last(int nd,
                           const float *x, const int64_t *x_shape,
                           const float *w, const int64_t *w_shape,
                           const float *bias,
                           const int *stride, const int *dilation, const int *padding, int groups,
                           float *y, convhip_stream_t stream);

/*
 * Fused Conv3d -> min over one spatial axis -> softmax over channels (page
 * l2_p24, opening turns: the module applies Conv3d, torch.min over dim 2, then
 * torch.softmax over dim 1; its `dim` argument names the min axis). The 5-D
 * conv result is never written to memory.
 *   x [N, C_in, D, H, W], w [C_out, C_in/groups, kD, kH, kW], bias [C_out] or NULL,
 *   min_dim 2, 3 or 4 (D, H or W); y holds the two other output axes in order:
 *   min_dim 2: y [N, C_out, H_out, W_out],
 *              y[n,:,h,w] = softmax_c( min_{od} conv3d(x,w,bias)[n,c,od,h,w] );
 *   min_dim 3: y [N, C_out, D_out, W_out];  min_dim 4: y [N, C_out, D_out, H_out].
 * Supported while one output tile's input box over the whole min axis, the
 * weights and the minima of all C_out channels at 64 positions fit in LDS
 * (160 KiB; more than 64 channels per group run as channel chunks of at most
 * 64); other valid arguments return CONV_ERR_UNSUPPORTED.
 * With groups > 1 each output channel reduces over its own group's C_in/groups
 * input channels only. A NaN input propagates as it does through the module's
 * torch.min (the minimum is NaN-propagating); infinite inputs: unspecified.
 */
int conv3d_min_softmax(const float *x, const int64_t *x_shape,
                       const float *w, const int64_t *w_shape, const float *bias,
                       const int *stride, const int *dilation, const int *padding, int groups,
                       int min_dim, float *y, convhip_stream_t stream);

/*
 * conv3d_min_softmax on channels-last tensors (the NDHWC layout that page
 * l1_p60's monologue weighs for coalesced input reads): the same operation,
 * with x stored [N, D, H, W, C_in] (x_shape in that order) and y stored with
 * the channels innermost, [N, kept axes..., C_out] (min_dim 2: [N, H_out,
 * W_out, C_out]; 3: [N, D_out, W_out, C_out]; 4: [N, D_out, H_out, C_out]).
 * min_dim keeps its meaning (2, 3, 4 = D, H, W). w keeps [C_out, C_in/groups,
 * kD, kH, kW]. Support, status codes and numerics as conv3d_min_softmax; any
 * pointer alignment is accepted.
 */
int conv3d_min_softmax_channels_last(const float *x, const int64_t *x_shape,
                                     const float *w, const int64_t *w_shape, const float *bias,
                                     const int *stride, const int *dilation, const int *padding, int groups,
                                     int min_dim, float *y, convhip_stream_t stream);

/*
 * The fused op's last two steps on their own, for running it unfused after
 * conv_fwd (page l2_p24, opening turns: torch.min over the chosen axis of the
 * Conv3d output, then torch.softmax over channels; the page also weighs writing
 * only these two steps as kernels over the library conv's output). The library
 * uses them to measure that chain beside conv3d_min_softmax. Both read their
 * input once and write their output once (HBM-bound).
 *
 * min_over_axis: y [N, C, D, H, W] (y_shape: 5 host entries), dim in {2, 3, 4};
 * out is y's shape with axis `dim` removed, out = the minimum along that axis.
 * Exact (a minimum rounds nothing). A NaN anywhere along the axis gives NaN, as
 * torch.min does. y and out are device pointers; out must not overlap y.
 * Returns CONV_OK, CONV_ERR_NULL, CONV_ERR_SHAPE (an entry < 1), CONV_ERR_PARAM
 * (dim outside 2..4), CONV_ERR_OVERFLOW (more than 2^40 elements) or CONV_ERR_HIP.
 */
int min_over_axis(const float *y, const int64_t *y_shape, int dim, float *out, convhip_stream_t stream);

/*
 * softmax_over_channels: z [N, C, S] (z_shape: 3 host entries; S is the product
 * of the trailing axes of an [N, C, ...] tensor), out the same shape:
 *   out[n,c,s] = exp(z[n,c,s] - M) / sum_c' exp(z[n,c',s] - M),  M = max_c z[n,c,s]
 * in fp32 (expf, one division per output). A NaN among a position's channels
 * makes that position's outputs NaN, as torch.softmax does; infinities:
 * unspecified. z and out are device pointers; out must not overlap z.
 * Returns CONV_OK, CONV_ERR_NULL, CONV_ERR_SHAPE, CONV_ERR_OVERFLOW or CONV_ERR_HIP.
 */
int softmax_over_channels(const float *z, const int64_t *z_shape, float *out, convhip_stream_t stream);

/*
 * Static text for a status code (never NULL). The codes name the failure
 * modes the pages run into (page l1_p76 turns 2-4: a launch the runtime
 * rejected, output lengths off by one, indices near INT_MAX; page
 * l2_p24 turn 3: a missing host binding) plus the argument checks of
 * PyTorch's Conv modules that the pages' problem statements inherit.
 */
const char *conv_status_string(int status);

/*
 * Describe the launch plan the library would use for these arguments (kernel
 * variant, tile, grid, LDS bytes): the host-side choices that page l1_p60's
 * monologue makes by hand (tile shape against shared-memory size and occupancy,
 * compile-time specialisation of the kernel size with a generic fallback) and
 * page l1_p76 turn 2 makes for the Conv1d (block of positions x channels, the
 * input slice per block). One line of text into buf (NUL-terminated,
 * truncated to buflen). fused = 0 for conv_fwd, 1 for conv3d_min_softmax with
 * min_dim 2, 3 or 4 for conv3d_min_softmax with that min_dim (then nd must be
 * 3, else CONV_ERR_RANK), 2 for conv_fwd_channels_last (x_shape in its
 * channels-last order), 5, 6 or 7 for conv3d_min_softmax_channels_last with
 * min_dim 2, 3 or 4; other values give CONV_ERR_PARAM. Host only; launches
 * nothing.
 * Returns a conv_status.
 */
int conv_plan_describe(int nd, const int64_t *x_shape, const int64_t *w_shape,
                       const int *stride, const int *dilation, const int *padding, int groups,
                       int fused, char *buf, int buflen);

/*
 * Seeded synthetic input generator on the device (not part of the operation:
 * it lets an input too large for the host be made in place). Writes
 * dst[i] for i in [0, count) from element index (start + i) of the SplitMix64
 * stream of `seed` (Steele, Lea & Flood, OOPSLA 2014): with
 * m = (splitmix64 output) >> 40,
 *   kind 0: m * 2^-24                        (uniform in [0,1))
 *   kind 1: fp32(fp32(2*m*2^-24 - 1) * bound) (uniform in [-bound, bound))
 *   kind 2: lo + ((m * span) >> 24)           (integers in [lo, lo+span))
 * dst is a device pointer. Returns CONV_OK, CONV_ERR_NULL, CONV_ERR_PARAM
 * (unknown kind, span < 1) or CONV_ERR_HIP.
 */
int convhip_synth_fill(float *dst, int64_t count, uint64_t seed, uint64_t start, int kind,
                       float bound, int lo, int span, convhip_stream_t stream);

/*
 * Calibration probe (not part of the operation): one launch that keeps every
 * SIMD of the device busy with independent fp32 arithmetic for `iters` rounds,
 * to measure the rate the chip reaches in practice. kind 0: 16x16x4 fp32
 * matrix-core instructions (8 independent accumulators per wave); kind 1:
 * plain fp32 FMA on the vector ALU (8 independent chains per lane). Enqueues on
 * `stream` and stores in *flop (host memory) the floating-point operations the
 * launch performs; the caller times it. sink is a device pointer to at least
 * one float, written by no input (it keeps the results live). Returns CONV_OK,
 * CONV_ERR_NULL, CONV_ERR_PARAM (kind not 0 or 1, iters outside [1, 2^22]: a
 * launch stays within about 2 s) or
 * CONV_ERR_HIP.
 */
int convhip_peak_probe(int kind, int64_t iters, float *sink, int64_t *flop, convhip_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVHIP_H */
