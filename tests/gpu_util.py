"""Helpers for the GPU parity tests: move seeded numpy inputs to the GPU, call the
library through its binding, and apply the tolerance.

Tolerance (fp32 conv vs fp64 oracle): max |y_gpu - y_ref| <= 1e-4 * sqrt(K_red) *
max |y_ref| over the compared elements, with K_red = (C_in/groups) * prod(kernel)
the length of each output's dot product. Fused softmax outputs: 1e-5 absolute.
"""
import math
import sys

import numpy as np
import torch

import implicit_gemm_convolution_direct_amd as ch

FUSED_ATOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return torch.device("cuda:0")


def to_dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def gpu_conv(x, w, b, stride, dilation, padding, groups):
    y = ch.conv_fwd(to_dev(x), to_dev(w), to_dev(b), stride, dilation, padding, groups)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gpu_fused(x, w, b, stride=1, dilation=1, padding=0, groups=1, min_dim=2):
    y = ch.conv3d_min_softmax(to_dev(x), to_dev(w), to_dev(b), stride, dilation, padding, groups, min_dim)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def conv_tol(w_shape, y_ref):
    kred = int(np.prod(w_shape[1:]))
    return 1e-4 * math.sqrt(kred) * float(np.abs(y_ref).max())


def assert_conv_close(y, y_ref, w_shape, what=""):
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.isfinite(y).all(), what
    err = float(np.abs(y.astype(np.float64) - y_ref).max())
    tol = conv_tol(w_shape, y_ref)
    say(f"  {what}: max|err| = {err:.3e}  tol = {tol:.3e}")
    assert err <= tol, f"{what}: max err {err} > tol {tol}"
    return err
