"""MI355X-native fp32 convolution: Python binding of the C-ABI library libconvhip.so.

Argument marshalling only. Every step of the computation runs in the library's
HIP kernels; there is no CPU or PyTorch fallback. If the library is not built,
importing works but every call raises.

Operations (POPCORNBENCH "Kimi-K2.6" pages l1_p60, l1_p76, l2_p24, opening turns):

* ``conv_fwd(x, w, bias, stride, dilation, padding, groups)`` -- Conv1d / Conv2d / Conv3d forward.
* ``conv_fwd_channels_last(x, w, ...)`` -- the same on channels-last tensors:
  x [N, spatial..., C_in] -> y [N, out..., C_out] (w keeps [C_out, C_in/groups, k...]).
* ``conv3d_min_softmax(x, w, bias, stride, dilation, padding, groups, min_dim=2)`` --
  softmax over channels of the minimum over depth of Conv3d, without writing the
  5-D conv result.
* ``conv3d_min_softmax_channels_last(x, w, ...)`` -- the same on channels-last
  tensors: x [N, D, H, W, C_in] -> y [N, kept axes..., C_out].
* ``min_over_axis(y, dim)``, ``softmax_over_channels(z)`` -- that op's last two
  steps as separate launches (its unfused form, measured beside it).
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libconvhip.so")

CONV_OK = 0
STATUS_NAMES = {
    0: "CONV_OK", -1: "CONV_ERR_NULL", -2: "CONV_ERR_RANK", -3: "CONV_ERR_SHAPE", -4: "CONV_ERR_GROUPS",
    -5: "CONV_ERR_PARAM", -6: "CONV_ERR_EMPTY_OUTPUT", -7: "CONV_ERR_UNSUPPORTED", -8: "CONV_ERR_OVERFLOW",
    -9: "CONV_ERR_HIP",
}
EXPORTED = ["conv_out_shape", "conv_fwd", "conv_fwd_channels_last", "conv3d_min_softmax",
            "conv3d_min_softmax_channels_last", "min_over_axis",
            "softmax_over_channels", "conv_status_string", "conv_plan_describe", "convhip_synth_fill",
            "convhip_peak_probe"]


class ConvError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               f"(run __graft_entry__.build() or python -m "
                               f"implicit_gemm_convolution_direct_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        i64p = ctypes.POINTER(ctypes.c_int64)
        ip = ctypes.POINTER(ctypes.c_int)
        vp = ctypes.c_void_p
        L.conv_out_shape.restype = ctypes.c_int
        L.conv_out_shape.argtypes = [ctypes.c_int, i64p, i64p, ip, ip, ip, i64p]
        L.conv_fwd.restype = ctypes.c_int
        L.conv_fwd.argtypes = [ctypes.c_int, vp, i64p, vp, i64p, vp, ip, ip, ip, ctypes.c_int, vp, vp]
        L.conv_fwd_channels_last.restype = ctypes.c_int
        L.conv_fwd_channels_last.argtypes = [ctypes.c_int, vp, i64p, vp, i64p, vp, ip, ip, ip, ctypes.c_int, vp, vp]
        L.conv3d_min_softmax.restype = ctypes.c_int
        L.conv3d_min_softmax.argtypes = [vp, i64p, vp, i64p, vp, ip, ip, ip, ctypes.c_int, ctypes.c_int, vp, vp]
        L.conv3d_min_softmax_channels_last.restype = ctypes.c_int
        L.conv3d_min_softmax_channels_last.argtypes = [vp, i64p, vp, i64p, vp, ip, ip, ip, ctypes.c_int, ctypes.c_int,
                                                       vp, vp]
        L.min_over_axis.restype = ctypes.c_int
        L.min_over_axis.argtypes = [vp, i64p, ctypes.c_int, vp, vp]
        L.softmax_over_channels.restype = ctypes.c_int
        L.softmax_over_channels.argtypes = [vp, i64p, vp, vp]
        L.conv_status_string.restype = ctypes.c_char_p
        L.conv_status_string.argtypes = [ctypes.c_int]
        L.conv_plan_describe.restype = ctypes.c_int
        L.conv_plan_describe.argtypes = [ctypes.c_int, i64p, i64p, ip, ip, ip, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_char_p, ctypes.c_int]
        L.convhip_synth_fill.restype = ctypes.c_int
        L.convhip_synth_fill.argtypes = [vp, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                         ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
        L.convhip_peak_probe.restype = ctypes.c_int
        L.convhip_peak_probe.argtypes = [ctypes.c_int, ctypes.c_int64, vp, ctypes.POINTER(ctypes.c_int64), vp]
        _lib = L
    return _lib


def status_string(status):
    try:
        return lib().conv_status_string(int(status)).decode()
    except RuntimeError:
        return STATUS_NAMES.get(int(status), f"status {status}")


def _i64(seq):
    return (ctypes.c_int64 * len(seq))(*[int(v) for v in seq])


def _i32(seq):
    return (ctypes.c_int * len(seq))(*[int(v) for v in seq])


def _vec(v, nd, name):
    if isinstance(v, int):
        return [v] * nd
    v = [int(t) for t in v]
    if len(v) != nd:
        raise ValueError(f"{name} needs {nd} entries, got {len(v)}")
    return v


def out_shape(in_spatial, k_spatial, stride, dilation, padding):
    """Output lengths via the library's conv_out_shape (host only)."""
    nd = len(in_spatial)
    out = (ctypes.c_int64 * nd)()
    rc = lib().conv_out_shape(nd, _i64(in_spatial), _i64(k_spatial), _i32(_vec(stride, nd, "stride")),
                              _i32(_vec(dilation, nd, "dilation")), _i32(_vec(padding, nd, "padding")), out)
    return rc, [int(v) for v in out]


def plan_describe(x_shape, w_shape, stride=1, dilation=1, padding=0, groups=1, fused=False, channels_last=False,
                  min_dim=2):
    """The library's launch plan; channels_last=True takes x_shape as [N, spatial..., C_in];
    fused=True describes conv3d_min_softmax (or its channels-last form) with that min_dim."""
    nd = len(x_shape) - 2
    buf = ctypes.create_string_buffer(1024)
    if fused:
        mode = int(min_dim) + 3 if channels_last else (1 if min_dim == 2 else int(min_dim))
    else:
        mode = 2 if channels_last else 0
    rc = lib().conv_plan_describe(nd, _i64(x_shape), _i64(w_shape), _i32(_vec(stride, nd, "stride")),
                                  _i32(_vec(dilation, nd, "dilation")), _i32(_vec(padding, nd, "padding")),
                                  int(groups), mode, buf, 1024)
    if rc != CONV_OK:
        raise ConvError(rc, "conv_plan_describe")
    return buf.value.decode()


def _check_meta(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32 (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_tensor(t, name):
    _check_meta(t, name)
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")


def _check_operands(x, w, bias, out):
    """Types, shapes and devices of a call's tensors, checked before anything is
    launched. The kernels read bias[co] for every output channel co, and the C ABI
    carries no bias length, so a bias of the wrong size is caught here; every
    tensor must sit on x's device, where the library launches."""
    _check_meta(x, "x")
    _check_meta(w, "w")
    if bias is not None:
        _check_meta(bias, "bias")
        if bias.dim() != 1 or bias.numel() != w.shape[0]:
            raise ValueError(f"bias must be 1-D with C_out = {w.shape[0]} entries (got shape {tuple(bias.shape)})")
    if out is not None:
        _check_meta(out, "out")
    for t, name in ((x, "x"), (w, "w"), (bias, "bias"), (out, "out")):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")
    for t, name in ((w, "w"), (bias, "bias"), (out, "out")):
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} is on {t.device} but x is on {x.device}: all operands must share one device")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device):
    """The caller's current stream on `device` (torch's), as the C ABI's stream handle."""
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(device.index if device.index is not None else torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# Marshalled shape/parameter arguments per call signature (the arrays are only
# read by the library during the call, so they can be reused).
_ARGS_CACHE = {}


def _conv_args(x_shape, w_shape, stride, dilation, padding, drop_axis=None):
    key = (x_shape, w_shape, stride if isinstance(stride, int) else tuple(stride),
           dilation if isinstance(dilation, int) else tuple(dilation),
           padding if isinstance(padding, int) else tuple(padding), drop_axis)
    hit = _ARGS_CACHE.get(key)
    if hit is not None:
        return hit
    nd = len(x_shape) - 2
    s, d, p = _vec(stride, nd, "stride"), _vec(dilation, nd, "dilation"), _vec(padding, nd, "padding")
    rc, o = out_shape(list(x_shape[2:]), list(w_shape[2:]), s, d, p)
    if rc != CONV_OK:
        raise ConvError(rc, "conv_out_shape")
    keep = o if drop_axis is None else [o[a] for a in range(nd) if a != drop_axis]
    val = (nd, _i64(x_shape), _i64(w_shape), _i32(s), _i32(d), _i32(p), (x_shape[0], w_shape[0], *keep))
    if len(_ARGS_CACHE) > 256:
        _ARGS_CACHE.clear()
    _ARGS_CACHE[key] = val
    return val


def conv_fwd(x, w, bias=None, stride=1, dilation=1, padding=0, groups=1, out=None):
    """y = Conv{1,2,3}d(x, w, bias) with zero padding; x [N,C,L], [N,C,H,W] or [N,C,D,H,W] fp32 on the GPU."""
    _check_operands(x, w, bias, out)
    nd = x.dim() - 2
    if nd not in (1, 2, 3) or w.dim() != x.dim():
        raise ValueError("x and w must both be 3-D (Conv1d), 4-D (Conv2d) or 5-D (Conv3d)")
    nd, xs, ws, s, d, p, shape = _conv_args(tuple(x.shape), tuple(w.shape), stride, dilation, padding)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    else:
        if tuple(out.shape) != shape:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    rc = lib().conv_fwd(nd, x.data_ptr(), xs, w.data_ptr(), ws, bias.data_ptr() if bias is not None else None,
                        s, d, p, int(groups), out.data_ptr(), _stream_handle(x.device))
    if rc != CONV_OK:
        raise ConvError(rc, "conv_fwd")
    return out


def conv_fwd_channels_last(x, w, bias=None, stride=1, dilation=1, padding=0, groups=1, out=None):
    """Channels-last convolution: x [N, L, C], [N, H, W, C] or [N, D, H, W, C] fp32 on the GPU
    (contiguous in that order), w [C_out, C_in/groups, k...]; returns y [N, out..., C_out]."""
    _check_operands(x, w, bias, out)
    nd = x.dim() - 2
    if nd not in (1, 2, 3) or w.dim() != x.dim():
        raise ValueError("x and w must both be 3-D, 4-D or 5-D")
    xs_cl = tuple(x.shape)
    logical = (xs_cl[0], xs_cl[-1], *xs_cl[1:-1])
    nd, _, ws, s, d, p, shape = _conv_args(logical, tuple(w.shape), stride, dilation, padding)
    shape = (shape[0], *shape[2:], shape[1])
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    else:
        if tuple(out.shape) != shape:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    rc = lib().conv_fwd_channels_last(nd, x.data_ptr(), _i64(xs_cl), w.data_ptr(), ws,
                                      bias.data_ptr() if bias is not None else None, s, d, p, int(groups),
                                      out.data_ptr(), _stream_handle(x.device))
    if rc != CONV_OK:
        raise ConvError(rc, "conv_fwd_channels_last")
    return out


def conv3d_min_softmax(x, w, bias=None, stride=1, dilation=1, padding=0, groups=1, min_dim=2, out=None):
    """softmax(min(Conv3d(x, w, bias), dim=min_dim), dim=1) without storing the conv result."""
    _check_operands(x, w, bias, out)
    if x.dim() != 5 or w.dim() != 5:
        raise ValueError("x and w must be 5-D")
    if min_dim not in (2, 3, 4):
        raise ValueError("min_dim must be 2, 3 or 4")
    _, xs, ws, s, d, p, shape = _conv_args(tuple(x.shape), tuple(w.shape), stride, dilation, padding,
                                           drop_axis=min_dim - 2)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    else:
        if tuple(out.shape) != shape:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    rc = lib().conv3d_min_softmax(x.data_ptr(), xs, w.data_ptr(), ws, bias.data_ptr() if bias is not None else None,
                                  s, d, p, int(groups), int(min_dim), out.data_ptr(), _stream_handle(x.device))
    if rc != CONV_OK:
        raise ConvError(rc, "conv3d_min_softmax")
    return out


def _check_out(out, shape, like):
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=like.device)
    _check_tensor(out, "out")
    if out.device != like.device:
        raise ValueError(f"out is on {out.device}, the input on {like.device}")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(shape)}")
    return out


def min_over_axis(y, dim, out=None):
    """torch.amin(y, dim) of a 5-D fp32 GPU tensor for dim 2, 3 or 4 (NaN-propagating)."""
    _check_tensor(y, "y")
    if y.dim() != 5:
        raise ValueError("y must be 5-D")
    if dim not in (2, 3, 4):
        raise ValueError("dim must be 2, 3 or 4")
    out = _check_out(out, tuple(v for a, v in enumerate(y.shape) if a != dim), y)
    rc = lib().min_over_axis(y.data_ptr(), _i64(y.shape), int(dim), out.data_ptr(), _stream_handle(y.device))
    if rc != CONV_OK:
        raise ConvError(rc, "min_over_axis")
    return out


def softmax_over_channels(z, out=None):
    """torch.softmax(z, dim=1) of an fp32 GPU tensor [N, C, ...]."""
    _check_tensor(z, "z")
    if z.dim() < 2:
        raise ValueError("z must be [N, C, ...]")
    out = _check_out(out, tuple(z.shape), z)
    S = 1
    for v in z.shape[2:]:
        S *= int(v)
    rc = lib().softmax_over_channels(z.data_ptr(), _i64((z.shape[0], z.shape[1], S)), out.data_ptr(),
                                     _stream_handle(z.device))
    if rc != CONV_OK:
        raise ConvError(rc, "softmax_over_channels")
    return out


def conv3d_min_softmax_channels_last(x, w, bias=None, stride=1, dilation=1, padding=0, groups=1, min_dim=2,
                                     out=None):
    """conv3d_min_softmax on channels-last tensors: x [N, D, H, W, C_in] -> y [N, kept axes..., C_out]
    (min_dim 2, 3, 4 = D, H, W); w keeps [C_out, C_in/groups, kD, kH, kW]."""
    _check_operands(x, w, bias, out)
    if x.dim() != 5 or w.dim() != 5:
        raise ValueError("x and w must be 5-D")
    if min_dim not in (2, 3, 4):
        raise ValueError("min_dim must be 2, 3 or 4")
    logical = (x.shape[0], x.shape[4], x.shape[1], x.shape[2], x.shape[3])
    _, _, ws, s, d, p, shape = _conv_args(tuple(logical), tuple(w.shape), stride, dilation, padding,
                                          drop_axis=min_dim - 2)
    shape = (shape[0], *shape[2:], shape[1])
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    elif tuple(out.shape) != shape:
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    rc = lib().conv3d_min_softmax_channels_last(x.data_ptr(), _i64(x.shape), w.data_ptr(), ws,
                                                bias.data_ptr() if bias is not None else None, s, d, p, int(groups),
                                                int(min_dim), out.data_ptr(), _stream_handle(x.device))
    if rc != CONV_OK:
        raise ConvError(rc, "conv3d_min_softmax_channels_last")
    return out


KIND_UNIFORM01, KIND_SYMMETRIC, KIND_INT = 0, 1, 2


def synth_fill(t, seed, kind=KIND_UNIFORM01, start=0, bound=1.0, lo=0, span=1):
    """Fill a contiguous fp32 GPU tensor in place with the library's SplitMix64 generator."""
    _check_tensor(t, "t")
    rc = lib().convhip_synth_fill(t.data_ptr(), t.numel(), int(seed) & (2 ** 64 - 1), int(start), int(kind),
                                  float(bound), int(lo), int(span), _stream_handle(t.device))
    if rc != CONV_OK:
        raise ConvError(rc, "convhip_synth_fill")
    return t


PROBE_MFMA_F32, PROBE_FMA_F32 = 0, 1


def peak_probe(kind, iters, sink):
    """Enqueue one calibration launch (kind PROBE_MFMA_F32 or PROBE_FMA_F32) on the
    current stream of sink's device; returns the floating-point operations it
    performs. sink: a GPU fp32 tensor of at least one element."""
    _check_tensor(sink, "sink")
    flop = ctypes.c_int64(0)
    rc = lib().convhip_peak_probe(int(kind), int(iters), sink.data_ptr(), ctypes.byref(flop),
                                  _stream_handle(sink.device))
    if rc != CONV_OK:
        raise ConvError(rc, "convhip_peak_probe")
    return flop.value
