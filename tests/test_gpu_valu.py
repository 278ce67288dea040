"""GPU parity of the vector-ALU direct kernel (conv_valu, forced with
CONVHIP_VALU=1) against the fp64 oracle.

Integer-valued inputs keep every partial sum an exact integer below 2^24, so
every case compares bit for bit whatever order the FMAs run in.
"""
import numpy as np
import pytest
import torch

import implicit_gemm_convolution_direct_amd as ch
import oracle
import synth
from gpu_util import dev, say, to_dev

pytestmark = pytest.mark.gpu


def _int_inputs(r, xs, ws, bias):
    x = r.integers(0, 4, size=xs).astype(np.float32)
    w = r.integers(-2, 3, size=ws).astype(np.float32)
    b = r.integers(-4, 5, size=ws[0]).astype(np.float32) if bias else None
    return x, w, b


def _conv(x, w, b, s, d, p, g):
    y = ch.conv_fwd(to_dev(x), to_dev(w), to_dev(b), s, d, p, g)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check(xs, ws, s, d, p, g, bias, seed, what):
    desc = ch.plan_describe(xs, ws, s, d, p, g)
    assert desc.startswith("conv_valu"), desc
    r = np.random.default_rng(seed)
    x, w, b = _int_inputs(r, xs, ws, bias)
    say(f"valu {what}: x={xs} w={ws} s={s} d={d} p={p} g={g}: {desc}")
    y = _conv(x, w, b, s, d, p, g)
    ref = oracle.conv(x, w, b, s, d, p, g)
    assert np.abs(ref).max() < 2 ** 24
    np.testing.assert_array_equal(y.astype(np.float64), ref)


@pytest.fixture(autouse=True)
def _force_valu(monkeypatch):
    monkeypatch.setenv("CONVHIP_VALU", "1")


VALU_CASES = [
    ((2, 3, 9, 8, 7), (8, 3, 3, 3, 3), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1, True),       # 8-channel blocks
    ((1, 4, 8, 9, 11), (6, 2, 3, 2, 3), (2, 1, 3), (1, 2, 1), (1, 0, 2), 2, False),     # groups, mixed s/d/p
    ((2, 16, 8, 10, 12), (32, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (1, 2, 3), 2, True),   # the general geometry
    ((1, 3, 5, 5, 40), (20, 3, 1, 1, 3), (1, 1, 3), (1, 1, 4), (0, 0, 0), 1, True),     # 16 + 4 channels
    ((3, 2, 4, 4, 4), (2, 1, 2, 2, 2), (1, 1, 1), (1, 1, 1), (2, 2, 2), 2, True),       # padding wider than kernel
    ((1, 2, 3, 3, 3), (70, 2, 3, 3, 3), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1, False),    # one output position
    ((1, 1, 1, 1, 600), (33, 1, 1, 1, 5), (1, 1, 1), (1, 1, 1), (2, 2, 2), 1, True),    # ragged last block
]


@pytest.mark.parametrize("case", range(len(VALU_CASES)))
def test_valu_kernel_integer_exact(case):
    xs, ws, s, d, p, g, bias = VALU_CASES[case]
    _check(xs, ws, s, d, p, g, bias, 900 + case, f"case {case}")


@pytest.mark.parametrize("nd", [1, 2])
def test_valu_kernel_lower_ranks(nd):
    if nd == 1:
        _check((2, 8, 1000), (12, 4, 3), (3,), (4,), (1,), 2, True, 950, "conv1d")
    else:
        _check((2, 5, 30, 41), (9, 5, 3, 4), (2, 1), (1, 2), (1, 2), 1, False, 951, "conv2d")


@pytest.mark.parametrize("name", ["tiny_conv3d", "general_conv3d", "asym_conv3d", "long_conv1d",
                                  "conv3d_min_softmax"])
def test_valu_kernel_on_workloads_integer_exact(name):
    """Whole workloads where they are small, two samples of the large ones."""
    cfg = synth.WORKLOADS[name]
    big = name in ("asym_conv3d", "long_conv1d", "conv3d_min_softmax")
    x, w, b = synth.make_inputs(name, n_samples=2 if big else None, integer=True)
    args = (list(cfg["stride"]), list(cfg["dilation"]), list(cfg["padding"]), cfg["groups"])
    desc = ch.plan_describe(x.shape, w.shape, *args)
    assert desc.startswith("conv_valu"), desc
    say(f"valu workload {name}: x={x.shape}: {desc}")
    y = _conv(x, w, b, *args)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, *args))


def test_large_kernels_fall_back_to_the_vector_kernel(monkeypatch):
    """An 11x11x11 kernel over 16 channels: no matrix-core kernel can stage its
    tiles, so conv_fwd takes the vector-ALU kernel without being forced."""
    monkeypatch.delenv("CONVHIP_VALU")
    _check((2, 16, 16, 16, 16), (8, 16, 11, 11, 11), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1, True, 960,
           "fallback 11^3")
    _check((1, 4, 24, 24, 24), (20, 2, 9, 9, 9), (2, 1, 1), (1, 2, 1), (3, 4, 4), 2, False, 961,
           "fallback 9^3 groups")


def _check_cl(xs_cl, ws, s, d, p, g, bias, seed, what):
    desc = ch.plan_describe(xs_cl, ws, s, d, p, g, channels_last=True)
    assert desc.startswith("conv_valu"), desc
    r = np.random.default_rng(seed)
    x, w, b = _int_inputs(r, xs_cl, ws, bias)
    say(f"valu channels-last {what}: x={xs_cl} w={ws}: {desc}")
    y = ch.conv_fwd_channels_last(to_dev(x), to_dev(w), to_dev(b), s, d, p, g)
    torch.cuda.synchronize()
    ref = oracle.conv_channels_last(x, w, b, s, d, p, g)
    np.testing.assert_array_equal(y.cpu().numpy().astype(np.float64), ref)


CL_CASES = [
    ((2, 9, 8, 7, 3), (8, 3, 3, 3, 3), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1, True),
    ((1, 8, 9, 11, 4), (6, 2, 3, 2, 3), (2, 1, 3), (1, 2, 1), (1, 0, 2), 2, False),
    ((2, 8, 10, 12, 16), (32, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (1, 2, 3), 2, True),
    ((8, 40, 40, 40, 3), (20, 3, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), 1, True),   # 256-lane groups
]


@pytest.mark.parametrize("case", range(len(CL_CASES)))
def test_valu_kernel_channels_last_integer_exact(case):
    xs, ws, s, d, p, g, bias = CL_CASES[case]
    _check_cl(xs, ws, s, d, p, g, bias, 970 + case, f"case {case}")


def test_large_kernels_fall_back_to_the_vector_kernel_channels_last(monkeypatch):
    monkeypatch.delenv("CONVHIP_VALU")
    _check_cl((2, 16, 16, 16, 16), (8, 16, 11, 11, 11), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1, True, 980,
              "fallback 11^3")
