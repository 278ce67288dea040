"""fp64 CPU oracle -- TEST INFRASTRUCTURE, not the product.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. The HIP library and its Python binding never do.

* ``conv``               -- oracle.c's nested-loop convolution, returns float64.
* ``conv_channels_last`` -- the same convolution on channels-last tensors
                           (x [N, spatial..., C_in] -> y [N, out..., C_out]): a
                           pure change of memory order around ``conv``.
* ``conv3d_min_softmax`` -- conv (composed) -> min over one axis -> softmax over channels.
* ``conv3d_min_softmax_channels_last`` -- the same on channels-last tensors (a pure
                           change of memory order around ``conv3d_min_softmax``).
* ``min_axis``           -- the minimum over one axis of a 5-D tensor (the fused op's
                           second step on its own).
* ``softmax_channels``   -- softmax over dim 1 (the fused op's last step on its own).
* ``out_len``            -- the output-length formula of one axis.
* ``brute``              -- a second, pure-Python statement of the same definition
                           for tiny inputs (pins oracle.c by brute force).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.build()
        lib = ctypes.CDLL(path)
        i64p = ctypes.POINTER(ctypes.c_int64)
        ip = ctypes.POINTER(ctypes.c_int)
        fp = ctypes.c_void_p
        lib.oracle_out_len.restype = ctypes.c_int64
        lib.oracle_out_len.argtypes = [ctypes.c_int64] * 5
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_conv.restype = ctypes.c_int
        lib.oracle_conv.argtypes = [ctypes.c_int, fp, i64p, fp, i64p, fp, ip, ip, ip, ctypes.c_int, fp]
        lib.oracle_conv3d_min_softmax.restype = ctypes.c_int
        lib.oracle_conv3d_min_softmax.argtypes = [fp, i64p, fp, i64p, fp, ip, ip, ip, ctypes.c_int,
                                                  ctypes.c_int, fp]
        lib.oracle_min_axis.restype = ctypes.c_int
        lib.oracle_min_axis.argtypes = [fp, i64p, ctypes.c_int, fp]
        lib.oracle_softmax_channels.restype = ctypes.c_int
        lib.oracle_softmax_channels.argtypes = [fp, i64p, fp]
        _LIB = lib
    return _LIB


def num_threads():
    return _lib().oracle_num_threads()


def out_len(L, k, s=1, d=1, p=0):
    return int(_lib().oracle_out_len(L, k, s, d, p))


def _i64(seq):
    return (ctypes.c_int64 * len(seq))(*[int(v) for v in seq])


def _i32(seq):
    return (ctypes.c_int * len(seq))(*[int(v) for v in seq])


def _vec(v, nd, name):
    if isinstance(v, int):
        return [v] * nd
    v = list(v)
    if len(v) != nd:
        raise ValueError(f"{name} must have {nd} entries")
    return v


def conv(x, w, bias=None, stride=1, dilation=1, padding=0, groups=1):
    """fp64 conv of fp32 numpy arrays; x [N,C,L] or [N,C,D,H,W]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    nd = x.ndim - 2
    stride, dilation, padding = (_vec(stride, nd, "stride"), _vec(dilation, nd, "dilation"),
                                 _vec(padding, nd, "padding"))
    out = [out_len(x.shape[2 + a], w.shape[2 + a], stride[a], dilation[a], padding[a]) for a in range(nd)]
    if min(out) < 1:
        raise ValueError(f"empty output {out}")
    y = np.empty((x.shape[0], w.shape[0], *out), dtype=np.float64)
    b = None
    if bias is not None:
        b = np.ascontiguousarray(bias, dtype=np.float32)
    rc = _lib().oracle_conv(nd, x.ctypes.data, _i64(x.shape), w.ctypes.data, _i64(w.shape),
                            b.ctypes.data if b is not None else None,
                            _i32(stride), _i32(dilation), _i32(padding), groups, y.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_conv rejected the arguments (code {rc})")
    return y


def conv_channels_last(x_cl, w, bias=None, stride=1, dilation=1, padding=0, groups=1):
    """fp64 conv of a channels-last input (page l1_p60, opening turn: the NDHWC
    layout). The operation is conv's; the channel axis moves to the end on the
    way in and on the way out."""
    x = np.moveaxis(np.asarray(x_cl, dtype=np.float32), -1, 1)
    return np.ascontiguousarray(np.moveaxis(conv(x, w, bias, stride, dilation, padding, groups), 1, -1))


def conv3d_min_softmax(x, w, bias=None, stride=1, dilation=1, padding=0, groups=1, min_dim=2):
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    stride, dilation, padding = _vec(stride, 3, "stride"), _vec(dilation, 3, "dilation"), _vec(padding, 3, "padding")
    o = [out_len(x.shape[2 + a], w.shape[2 + a], stride[a], dilation[a], padding[a]) for a in range(3)]
    if min(o) < 1:
        raise ValueError(f"empty output {o}")
    keep = [o[a] for a in range(3) if a != min_dim - 2]
    out = np.empty((x.shape[0], w.shape[0], *keep), dtype=np.float64)
    b = np.ascontiguousarray(bias, dtype=np.float32) if bias is not None else None
    rc = _lib().oracle_conv3d_min_softmax(x.ctypes.data, _i64(x.shape), w.ctypes.data, _i64(w.shape),
                                          b.ctypes.data if b is not None else None,
                                          _i32(stride), _i32(dilation), _i32(padding), groups, min_dim,
                                          out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_conv3d_min_softmax rejected the arguments (code {rc})")
    return out


def min_axis(y, dim):
    """Minimum of a 5-D float32 array over axis ``dim`` (2, 3 or 4); float32, exact."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    if y.ndim != 5:
        raise ValueError("min_axis takes a 5-D array")
    out = np.empty(tuple(v for a, v in enumerate(y.shape) if a != dim), dtype=np.float32)
    rc = _lib().oracle_min_axis(y.ctypes.data, _i64(y.shape), int(dim), out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_min_axis rejected the arguments (code {rc})")
    return out


def softmax_channels(z):
    """Softmax over axis 1 of a float32 array [N, C, ...], computed in float64."""
    z = np.ascontiguousarray(z, dtype=np.float32)
    if z.ndim < 2:
        raise ValueError("softmax_channels takes an array [N, C, ...]")
    S = int(np.prod(z.shape[2:])) if z.ndim > 2 else 1
    out = np.empty(z.shape, dtype=np.float64)
    rc = _lib().oracle_softmax_channels(z.ctypes.data, _i64((z.shape[0], z.shape[1], S)), out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_softmax_channels rejected the arguments (code {rc})")
    return out


def conv3d_min_softmax_channels_last(x_cl, w, bias=None, stride=1, dilation=1, padding=0, groups=1, min_dim=2):
    """conv3d_min_softmax for x stored [N, D, H, W, C_in]; returns float64 [N, kept axes..., C_out]:
    the channel axis moved in on the way in and out on the way out (min_dim keeps its
    meaning: 2, 3, 4 = D, H, W)."""
    x = np.moveaxis(np.asarray(x_cl, dtype=np.float32), -1, 1)
    y = conv3d_min_softmax(x, w, bias, stride, dilation, padding, groups, min_dim)
    return np.ascontiguousarray(np.moveaxis(y, 1, -1))
