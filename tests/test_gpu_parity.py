"""GPU parity: the HIP path (through the C-ABI binding) against the fp64 oracle.

* integer-valued inputs: every partial sum is an integer below 2**24, so the fp32
  GPU result must equal the oracle exactly, for every tile shape and tail;
* uniform inputs: within 1e-4 * sqrt(K_red) * max|y_ref| (conv) or 1e-5 (fused);
* the five workloads at full size in the bench's launch configuration (the two
  largest compared on a batch slice the oracle computes in seconds).
"""
import zlib

import numpy as np
import pytest
import torch

import implicit_gemm_convolution_direct_amd as ch
import oracle
import synth
from gpu_util import (FUSED_ATOL, assert_conv_close, dev, gpu_conv, gpu_fused, say, to_dev)

pytestmark = pytest.mark.gpu


def _int_inputs(r, xs, ws, bias):
    x = r.integers(0, 4, size=xs).astype(np.float32)
    w = r.integers(-2, 3, size=ws).astype(np.float32)
    b = r.integers(-4, 5, size=ws[0]).astype(np.float32) if bias else None
    return x, w, b


def _float_inputs(r, xs, ws, bias):
    x = r.random(xs, dtype=np.float32)
    fan = int(np.prod(ws[1:]))
    w = ((r.random(ws, dtype=np.float32) * 2 - 1) / np.sqrt(fan)).astype(np.float32)
    b = ((r.random(ws[0], dtype=np.float32) * 2 - 1) / np.sqrt(fan)).astype(np.float32) if bias else None
    return x, w, b


def _random_geometry(r, nd):
    g = int(r.choice([1, 1, 1, 2, 4]))
    cg = int(r.integers(1, 6))
    coutg = int(r.choice([1, 3, 8, 16, 20, 33, 64, 70, 128, 150]))
    if g > 1:
        coutg = min(coutg, 40)
    ks = [int(r.integers(1, 6)) for _ in range(nd)]
    s = [int(r.integers(1, 4)) for _ in range(nd)]
    d = [int(r.integers(1, 4)) for _ in range(nd)]
    p = [int(r.integers(0, 4)) for _ in range(nd)]
    Ls = []
    for a in range(nd):
        lo = max(1, d[a] * (ks[a] - 1) + 1 - 2 * p[a])
        span = {1: 700, 2: 60, 3: 20}[nd]
        Ls.append(int(r.integers(lo, lo + span)))
    N = int(r.integers(1, 3))
    return (N, g * cg, *Ls), (g * coutg, cg, *ks), s, d, p, g


RANDOM_CASES = [(nd, seed) for nd in (1, 2, 3) for seed in range(14)]


@pytest.mark.parametrize("nd,seed", RANDOM_CASES)
def test_random_shapes_integer_exact(nd, seed):
    r = np.random.default_rng(1000 * nd + seed)
    xs, ws, s, d, p, g = _random_geometry(r, nd)
    x, w, b = _int_inputs(r, xs, ws, bias=bool(seed % 2))
    say(f"case nd={nd} seed={seed} x={xs} w={ws} s={s} d={d} p={p} g={g}: "
        + ch.plan_describe(xs, ws, s, d, p, g))
    y = gpu_conv(x, w, b, s, d, p, g)
    ref = oracle.conv(x, w, b, s, d, p, g)
    assert np.abs(ref).max() < 2 ** 24
    np.testing.assert_array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("nd,seed", RANDOM_CASES[::2])
def test_random_shapes_float(nd, seed):
    r = np.random.default_rng(5000 + 1000 * nd + seed)
    xs, ws, s, d, p, g = _random_geometry(r, nd)
    x, w, b = _float_inputs(r, xs, ws, bias=bool(seed % 2))
    say(f"case nd={nd} seed={seed} x={xs} w={ws}")
    y = gpu_conv(x, w, b, s, d, p, g)
    assert_conv_close(y, oracle.conv(x, w, b, s, d, p, g), ws, f"random float nd={nd} seed={seed}")


EDGE_CASES = [
    # name, x shape, w shape, stride, dilation, padding, groups
    ("single_output", (1, 2, 3, 4, 5), (3, 2, 3, 4, 5), 1, 1, 0, 1),
    ("kernel_1x1x1", (2, 5, 4, 6, 7), (7, 5, 1, 1, 1), 1, 1, 0, 1),
    ("depthwise", (2, 6, 5, 9, 11), (6, 1, 3, 3, 3), 1, 1, 1, 6),
    ("padding_wider_than_kernel", (1, 2, 3, 3, 3), (4, 2, 2, 2, 2), 1, 1, 3, 1),
    ("stride_gt_kernel", (1, 3, 9, 17, 33), (5, 3, 2, 2, 2), (4, 3, 5), 1, 0, 1),
    ("one_output_channel", (2, 3, 6, 7, 8), (1, 3, 3, 3, 3), 1, 1, 0, 1),
    ("cout_129_two_channel_tiles", (1, 4, 300), (129, 4, 3), 3, 4, 0, 1),
    ("conv1d_long_row_tiles", (2, 3, 5000), (16, 3, 5), 1, 2, 2, 1),
    ("conv1d_k1", (1, 8, 1000), (24, 8, 1), 2, 1, 0, 1),
    ("wide_rows_3d", (1, 2, 3, 4, 600), (8, 2, 2, 2, 3), 1, 1, 1, 1),
    ("many_input_channels", (1, 200, 4, 4, 40), (16, 200, 1, 1, 3), 1, 1, 0, 1),
    # the long Conv1d's channel/kernel geometry where 16-byte row copies do not
    # apply (padding 2, length not a multiple of 4): generic kernel
    ("conv1d_unaligned_rows", (1, 64, 3001), (128, 64, 3), 3, 4, 2, 1),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_edge_cases_integer_exact(case):
    name, xs, ws, s, d, p, g = case
    r = np.random.default_rng(zlib.crc32(name.encode()))
    x, w, b = _int_inputs(r, xs, ws, bias=True)
    say(f"edge {name}: " + ch.plan_describe(xs, ws, s, d, p, g))
    y = gpu_conv(x, w, b, s, d, p, g)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, s, d, p, g))


def test_delta_kernel_on_gpu_is_exact_copy():
    r = np.random.default_rng(3)
    x = r.random((2, 4, 9, 10, 11), dtype=np.float32)
    w = np.zeros((4, 2, 3, 2, 3), dtype=np.float32)
    w[:, 1, 2, 1, 0] = 1.0
    y = gpu_conv(x, w, None, (2, 1, 3), (1, 2, 1), (1, 0, 2), 2)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, None, (2, 1, 3), (1, 2, 1), (1, 0, 2), 2))


def test_deterministic_and_stream_respected():
    r = np.random.default_rng(4)
    x, w, b = _float_inputs(r, (2, 3, 10, 12, 14), (20, 3, 3, 3, 3), True)
    xd, wd, bd = to_dev(x), to_dev(w), to_dev(b)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = ch.conv_fwd(xd, wd, bd)
        y2 = ch.conv_fwd(xd, wd, bd)
    s.synchronize()
    assert torch.equal(y1, y2)
    assert_conv_close(y1.cpu().numpy(), oracle.conv(x, w, b), w.shape, "side stream")


# ------------------------------------------------------------------ workloads
def _cfg_args(cfg):
    return cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"]


@pytest.mark.parametrize("name", ["tiny_conv3d", "general_conv3d"])
def test_workload_full_integer_exact(name):
    cfg = synth.WORKLOADS[name]
    x, w, b = synth.make_inputs(name, integer=True)
    say(f"workload {name} integer: " + ch.plan_describe(cfg["x"], cfg["w"], *_cfg_args(cfg)))
    y = gpu_conv(x, w, b, *_cfg_args(cfg))
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, *_cfg_args(cfg)))


@pytest.mark.parametrize("name", ["tiny_conv3d", "general_conv3d"])
def test_workload_full_float(name):
    cfg = synth.WORKLOADS[name]
    x, w, b = synth.make_inputs(name)
    say(f"workload {name}: " + ch.plan_describe(cfg["x"], cfg["w"], *_cfg_args(cfg)))
    y = gpu_conv(x, w, b, *_cfg_args(cfg))
    assert_conv_close(y, oracle.conv(x, w, b, *_cfg_args(cfg)), cfg["w"], name)


def test_general_conv3d_deterministic():
    """The channel-split kernels sum the per-wave partial tiles in a fixed order:
    repeated calls give identical bits."""
    name = "general_conv3d"
    cfg = synth.WORKLOADS[name]
    x, w, b = synth.make_inputs(name)
    xd, wd, bd = to_dev(x), to_dev(w), to_dev(b)
    y1 = ch.conv_fwd(xd, wd, bd, *_cfg_args(cfg))
    y2 = ch.conv_fwd(xd, wd, bd, *_cfg_args(cfg))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_workload_asym_conv3d_slices():
    name = "asym_conv3d"
    cfg = synth.WORKLOADS[name]
    x, w, b = synth.make_inputs(name)
    say(f"workload {name}: " + ch.plan_describe(cfg["x"], cfg["w"], *_cfg_args(cfg)))
    y = ch.conv_fwd(to_dev(x), to_dev(w), None, *_cfg_args(cfg))
    torch.cuda.synchronize()
    for n in (0, cfg["x"][0] - 1):
        ref = oracle.conv(x[n:n + 1], w, None, *_cfg_args(cfg))
        assert_conv_close(y[n:n + 1].cpu().numpy(), ref, cfg["w"], f"{name} n={n}")
    del y


def test_workload_long_conv1d_device_inputs_slices():
    """The 8.6 GB input is generated on the device; the host regenerates two samples,
    checks them bit for bit against the device copy, and compares the outputs."""
    name = "long_conv1d"
    cfg = synth.WORKLOADS[name]
    xs, ws = cfg["x"], cfg["w"]
    sx, sw, _ = cfg["seeds"]
    say(f"workload {name}: " + ch.plan_describe(xs, ws, *_cfg_args(cfg)))
    xd = torch.empty(xs, dtype=torch.float32, device=dev())
    ch.synth_fill(xd, sx, ch.KIND_UNIFORM01)
    _, w, _ = synth.make_inputs(name, n_samples=1)
    y = ch.conv_fwd(xd, to_dev(w), None, *_cfg_args(cfg))
    torch.cuda.synchronize()
    per = xs[1] * xs[2]
    for n in (0, xs[0] - 1):
        xh = synth.uniform01(sx, (1, *xs[1:]), start=n * per)
        np.testing.assert_array_equal(xd[n:n + 1].cpu().numpy(), xh)
        ref = oracle.conv(xh, w, None, *_cfg_args(cfg))
        assert_conv_close(y[n:n + 1].cpu().numpy(), ref, ws, f"{name} n={n}")
    del xd, y
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ fused
def test_fused_workload_full():
    name = "conv3d_min_softmax"
    cfg = synth.WORKLOADS[name]
    x, w, b = synth.make_inputs(name)
    say(f"workload {name}: " + ch.plan_describe(cfg["x"], cfg["w"], fused=True))
    y = gpu_fused(x, w, b)
    ref = oracle.conv3d_min_softmax(x, w, b)
    err = float(np.abs(y - ref).max())
    say(f"  fused max|err| = {err:.3e}")
    assert err <= FUSED_ATOL
    np.testing.assert_allclose(y.sum(axis=1), 1.0, atol=1e-5)


FUSED_CASES = [
    ("small", (2, 3, 6, 9, 10), (5, 3, 3, 3, 3), 1, 1, 0),
    ("strided_padded", (1, 2, 7, 8, 40), (10, 2, 2, 3, 2), (2, 1, 2), (1, 2, 1), (1, 1, 2)),
    ("row_tiles", (1, 3, 5, 4, 140), (3, 3, 1, 2, 3), 1, 1, 0),
    ("cout_1", (2, 3, 5, 6, 7), (1, 3, 3, 3, 3), 1, 1, 0),
    ("cout_64", (1, 2, 6, 10, 12), (64, 2, 3, 3, 3), 1, 1, 1),
    ("depth_out_1", (2, 3, 3, 12, 13), (24, 3, 3, 3, 3), 1, 1, 0),
    ("depth_out_2", (1, 3, 4, 12, 13), (24, 3, 3, 3, 3), 1, 1, 0),
    # the streamed kernel's channel/kernel geometry with padding along W: generic kernel
    ("stream_geometry_w_padded", (1, 3, 4, 9, 30), (22, 3, 3, 3, 3), 1, 1, (1, 2, 1)),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_cases(case):
    name, xs, ws, s, d, p = case
    r = np.random.default_rng(zlib.crc32(name.encode()))
    x, w, b = _float_inputs(r, xs, ws, True)
    say(f"fused {name}: " + ch.plan_describe(xs, ws, s, d, p, 1, fused=True))
    y = gpu_fused(x, w, b, s, d, p)
    ref = oracle.conv3d_min_softmax(x, w, b, s, d, p)
    err = float(np.abs(y - ref).max())
    say(f"  max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


STREAM_CASES = [
    # depth-streamed kernel geometry: C_in 3, kernel 3x3x3, stride 1, W_out 30
    ("full_planes", (2, 3, 6, 32, 32), (24, 3, 3, 3, 3), 0, True),
    ("short_plane", (1, 3, 5, 10, 32), (24, 3, 3, 3, 3), 0, True),
    ("padded_cout22", (1, 3, 4, 9, 32), (22, 3, 3, 3, 3), (1, 2, 0), False),
    ("cout21_depth1", (2, 3, 3, 7, 32), (21, 3, 3, 3, 3), (0, 1, 0), True),
    ("ragged_units", (3, 3, 8, 21, 32), (24, 3, 3, 3, 3), 0, True),
]


@pytest.mark.parametrize("case", STREAM_CASES, ids=[c[0] for c in STREAM_CASES])
def test_fused_stream_cases(case):
    name, xs, ws, p, bias = case
    desc = ch.plan_describe(xs, ws, 1, 1, p, 1, fused=True)
    assert "kernel=fused_stream" in desc, desc
    r = np.random.default_rng(900 + len(name))
    x, w, b = _float_inputs(r, xs, ws, bias)
    say(f"stream {name}: {desc}")
    y = gpu_fused(x, w, b, 1, 1, p)
    ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, p)
    err = float(np.abs(y - ref).max())
    say(f"  max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


MIN_AXIS_CASES = [
    # name, x, w, stride, dilation, padding, min_dim
    ("min_h_workload_like", (2, 3, 6, 12, 10), (24, 3, 3, 3, 3), 1, 1, 0, 3),
    ("min_w_workload_like", (2, 3, 6, 10, 12), (24, 3, 3, 3, 3), 1, 1, 0, 4),
    ("min_h_strided_padded", (1, 2, 7, 9, 11), (10, 2, 2, 3, 2), (2, 1, 2), (1, 2, 1), (1, 1, 2), 3),
    ("min_w_strided_padded", (1, 2, 7, 9, 13), (7, 2, 2, 3, 3), (1, 2, 2), (2, 1, 1), (1, 1, 2), 4),
    ("min_w_asym_kernel", (2, 3, 5, 6, 9), (5, 3, 1, 2, 4), 1, (1, 1, 2), (0, 1, 1), 4),
    ("min_h_single_row", (1, 3, 4, 3, 8), (6, 3, 2, 3, 3), 1, 1, 0, 3),
]


@pytest.mark.parametrize("case", MIN_AXIS_CASES, ids=[c[0] for c in MIN_AXIS_CASES])
def test_fused_min_over_h_or_w(case):
    """Minimum over H or W (min_dim 3, 4): the generic fused kernel with permuted
    axes, against the oracle's own minimum over that axis."""
    name, xs, ws, s, d, p, md = case
    r = np.random.default_rng(1300 + len(name))
    x, w, b = _float_inputs(r, xs, ws, True)
    y = gpu_fused(x, w, b, s, d, p, 1, md)
    ref = oracle.conv3d_min_softmax(x, w, b, s, d, p, 1, md)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    err = float(np.abs(y - ref).max())
    say(f"  {name}: max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


# Minimum over H on the depth-streamed kernel: it streams over H (the min
# axis) with rows along D, at the fused workload's channel, kernel and W extents.
STREAM_MIN_H_CASES = [
    ("two_samples", (2, 3, 6, 32, 32), True),
    ("ragged_d_tiles", (1, 3, 5, 20, 32), False),
    ("workload_slice", (2, 3, 24, 32, 32), True),
]


@pytest.mark.parametrize("case", STREAM_MIN_H_CASES, ids=[c[0] for c in STREAM_MIN_H_CASES])
def test_fused_stream_min_over_h(case):
    name, xs, bias = case
    ws = (24, 3, 3, 3, 3)
    desc = ch.plan_describe(xs, ws, 1, 1, 0, 1, fused=True, min_dim=3)
    assert "kernel=fused_stream" in desc, desc
    r = np.random.default_rng(zlib.crc32(name.encode()))
    x, w, b = _float_inputs(r, xs, ws, bias)
    say(f"stream min over H {name}: {desc}")
    y = gpu_fused(x, w, b, 1, 1, 0, 1, 3)
    ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, 0, 1, 3)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    err = float(np.abs(y - ref).max())
    say(f"  max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


# Minimum over W on the depth-streamed kernel: it streams over W with rows
# along D and columns along H, copying single input elements.
STREAM_MIN_W_CASES = [
    ("two_samples", (2, 3, 6, 32, 32), 0, True),
    ("short_w_ragged_d", (1, 3, 5, 32, 9), 0, False),
    ("padded_d_and_w", (1, 3, 7, 32, 12), (1, 0, 2), True),
    ("workload_slice", (2, 3, 24, 32, 32), 0, True),
]


@pytest.mark.parametrize("case", STREAM_MIN_W_CASES, ids=[c[0] for c in STREAM_MIN_W_CASES])
def test_fused_stream_min_over_w(case):
    name, xs, p, bias = case
    ws = (24, 3, 3, 3, 3)
    desc = ch.plan_describe(xs, ws, 1, 1, p, 1, fused=True, min_dim=4)
    assert "kernel=fused_stream spec=2" in desc, desc
    r = np.random.default_rng(zlib.crc32(name.encode()))
    x, w, b = _float_inputs(r, xs, ws, bias)
    say(f"stream min over W {name}: {desc}")
    y = gpu_fused(x, w, b, 1, 1, p, 1, 4)
    ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, p, 1, 4)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    err = float(np.abs(y - ref).max())
    say(f"  max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


def test_fused_stream_min_over_w_integer_minimum_exact():
    r = np.random.default_rng(1760)
    xs, ws = (2, 3, 5, 32, 11), (24, 3, 3, 3, 3)
    x, w, b = _int_inputs(r, xs, ws, True)
    assert "kernel=fused_stream spec=2" in ch.plan_describe(xs, ws, fused=True, min_dim=4)
    y = gpu_fused(x, w, b, 1, 1, 0, 1, 4)
    ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, 0, 1, 4)
    assert float(np.abs(y - ref).max()) <= FUSED_ATOL


GROUPED_FUSED_CASES = [
    ("groups2_min_d", (2, 4, 6, 8, 9), (6, 2, 3, 3, 3), 1, 1, 0, 2, 2),
    ("groups3_min_h_strided", (1, 6, 5, 9, 8), (9, 2, 2, 3, 2), (1, 2, 1), 1, (1, 1, 0), 3, 3),
    ("depthwise_min_w", (2, 4, 4, 6, 10), (4, 1, 2, 2, 3), 1, (1, 1, 2), 1, 4, 4),
]


@pytest.mark.parametrize("case", GROUPED_FUSED_CASES, ids=[c[0] for c in GROUPED_FUSED_CASES])
def test_fused_grouped(case):
    """Grouped convolutions in the fused op: each group reduces over its own
    input channels only."""
    name, xs, ws, s, d, p, g, md = case
    r = np.random.default_rng(1700 + len(name))
    x, w, b = _float_inputs(r, xs, ws, True)
    y = gpu_fused(x, w, b, s, d, p, g, md)
    ref = oracle.conv3d_min_softmax(x, w, b, s, d, p, g, md)
    err = float(np.abs(y - ref).max())
    say(f"  {name}: max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


@pytest.mark.parametrize("generic", [False, True])
def test_fused_grouped_workload_slice(generic, monkeypatch):
    """The fused workload's shape with groups 3 (w [24, 1, 3, 3, 3]) on a
    two-sample slice, against the oracle: on the depth-streamed kernel (each
    channel block reducing over its own group's input channel) and, with the
    specialisations off, on the generic fused kernel."""
    if generic:
        monkeypatch.setenv("CONVHIP_TAP", "0")
    cfg = synth.VARIANTS["conv3d_min_softmax_groups3"]
    x, w, b = synth.make_inputs("conv3d_min_softmax_groups3", n_samples=2, sample_start=5)
    desc = ch.plan_describe(x.shape, w.shape, 1, 1, 0, cfg["groups"], fused=True)
    if generic:
        assert "groups=3 kred=27" in desc, desc
    else:
        assert "kernel=fused_stream spec=1" in desc and "groups=3" in desc, desc
    say(f"fused groups3 slice: {desc}")
    y = gpu_fused(x, w, b, 1, 1, 0, cfg["groups"], 2)
    ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, 0, cfg["groups"], 2)
    err = float(np.abs(y - ref).max())
    say(f"  max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


# Conv groups on the depth-streamed kernel: 3 groups of 1 input and 8 output
# channels (each 4-channel block reduces over its own group's channel only).
STREAM_GROUP_CASES = [
    ("groups3_two_samples", (2, 3, 6, 32, 32), 0, True, 2),
    ("groups3_padded", (1, 3, 5, 9, 32), (1, 2, 0), False, 2),
    ("groups3_ragged_units", (3, 3, 8, 21, 32), 0, True, 2),
    ("groups3_min_over_h", (2, 3, 6, 20, 32), 0, True, 3),
]


@pytest.mark.parametrize("case", STREAM_GROUP_CASES, ids=[c[0] for c in STREAM_GROUP_CASES])
def test_fused_stream_groups(case):
    name, xs, p, bias, md = case
    ws = (24, 1, 3, 3, 3)
    desc = ch.plan_describe(xs, ws, 1, 1, p, 3, fused=True, min_dim=md)
    assert "kernel=fused_stream spec=1" in desc, desc
    r = np.random.default_rng(zlib.crc32(name.encode()))
    x, w, b = _float_inputs(r, xs, ws, bias)
    say(f"stream groups {name}: {desc}")
    y = gpu_fused(x, w, b, 1, 1, p, 3, md)
    ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, p, 3, md)
    err = float(np.abs(y - ref).max())
    say(f"  max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


def test_fused_stream_groups_integer_minimum_exact():
    """Integer inputs keep every conv sum exact, so the minimum is exact and the
    softmax error alone remains."""
    r = np.random.default_rng(1750)
    xs, ws = (2, 3, 5, 12, 32), (24, 1, 3, 3, 3)
    x, w, b = _int_inputs(r, xs, ws, True)
    y = gpu_fused(x, w, b, 1, 1, 0, 3, 2)
    ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, 0, 3, 2)
    assert float(np.abs(y - ref).max()) <= FUSED_ATOL


# More than 64 output channels per group: the generic fused kernel runs them as
# chunks of at most 64 channels and merges the chunks' minima before the softmax.
FUSED_CHUNK_CASES = [
    ("cout96_min_d", (2, 3, 6, 9, 10), (96, 3, 3, 3, 3), 1, 1, 0, 1, 2),
    ("cout150_min_h_padded", (1, 3, 5, 8, 12), (150, 3, 2, 3, 3), 1, 1, (1, 1, 1), 1, 3),
    ("groups2_cout160_min_w", (2, 4, 5, 7, 9), (160, 2, 2, 2, 3), (1, 1, 2), 1, 0, 2, 4),
    ("cout128_two_tiles", (2, 3, 8, 12, 12), (128, 3, 3, 3, 3), 1, 1, 0, 1, 2),
]


@pytest.mark.parametrize("case", FUSED_CHUNK_CASES, ids=[c[0] for c in FUSED_CHUNK_CASES])
def test_fused_channel_chunks(case):
    name, xs, ws, s, d, p, g, md = case
    desc = ch.plan_describe(xs, ws, s, d, p, g, fused=True, min_dim=md)
    assert "kernel=fused_min_softmax_mfma4" in desc and "chunks=1 " not in desc, desc
    r = np.random.default_rng(zlib.crc32(name.encode()))
    x, w, b = _float_inputs(r, xs, ws, True)
    say(f"fused channel chunks {name}: {desc}")
    y = gpu_fused(x, w, b, s, d, p, g, md)
    ref = oracle.conv3d_min_softmax(x, w, b, s, d, p, g, md)
    err = float(np.abs(y - ref).max())
    say(f"  max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


def test_fused_channel_chunks_integer_minimum_exact():
    r = np.random.default_rng(1780)
    xs, ws = (2, 3, 5, 7, 9), (100, 3, 2, 3, 2)
    x, w, b = _int_inputs(r, xs, ws, True)
    y = gpu_fused(x, w, b, 1, 1, 0, 1, 2)
    ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, 0, 1, 2)
    assert float(np.abs(y - ref).max()) <= FUSED_ATOL


CONV2D_CASES = [
    ("conv2d_workload_like", (2, 16, 32, 32), (32, 8, 5, 7), (2, 2), (1, 2), (2, 3), 2),
    ("conv2d_3x3", (1, 3, 40, 50), (8, 3, 3, 3), 1, 1, 1, 1),
    ("conv2d_1x1_strided", (2, 12, 17, 19), (20, 12, 1, 1), 2, 1, 0, 1),
]


@pytest.mark.parametrize("case", CONV2D_CASES, ids=[c[0] for c in CONV2D_CASES])
def test_conv2d_integer_exact(case):
    name, xs, ws, s, d, p, g = case
    r = np.random.default_rng(1900 + len(name))
    x, w, b = _int_inputs(r, xs, ws, bias=True)
    say(f"conv2d {name}: " + ch.plan_describe(xs, ws, s, d, p, g))
    y = gpu_conv(x, w, b, s, d, p, g)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, s, d, p, g))


def test_fused_min_axes_integer_exact_minimum():
    """Integer inputs make every conv value exact: the minimum over each axis is
    exact and only exp/division rounding remains."""
    r = np.random.default_rng(77)
    x, w, b = _int_inputs(r, (2, 3, 6, 7, 8), (8, 3, 3, 3, 3), bias=True)
    w = (w * 0.125).astype(np.float32)
    for md in (2, 3, 4):
        y = gpu_fused(x, w, b, 1, 1, 1, 1, md)
        ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, 1, 1, md)
        assert float(np.abs(y - ref).max()) <= 1e-6, md


def test_misaligned_pointers_take_generic_kernels():
    """Views that start 4 bytes past an allocation keep the specialised kernels
    (16-byte copies) out and still give the oracle's results."""
    cfg = synth.WORKLOADS["conv3d_min_softmax"]
    x, w, b = synth.make_inputs("conv3d_min_softmax", n_samples=2)
    xd = torch.empty(x.size + 1, dtype=torch.float32, device=dev())[1:].view(x.shape)
    xd.copy_(torch.from_numpy(x))
    assert xd.data_ptr() % 16 != 0
    y = ch.conv3d_min_softmax(xd, to_dev(w), to_dev(b), 1, 1, 0, 1, min_dim=2).cpu().numpy()
    assert float(np.abs(y - oracle.conv3d_min_softmax(x, w, b)).max()) <= FUSED_ATOL
    name = "general_conv3d"
    cfg = synth.WORKLOADS[name]
    x, w, b = synth.make_inputs(name, n_samples=1)
    wd = torch.empty(w.size + 1, dtype=torch.float32, device=dev())[1:].view(w.shape)
    wd.copy_(torch.from_numpy(w))
    assert wd.data_ptr() % 16 != 0
    y = ch.conv_fwd(to_dev(x), wd, to_dev(b), *_cfg_args(cfg)).cpu().numpy()
    assert_conv_close(y, oracle.conv(x, w, b, *_cfg_args(cfg)), w.shape, "misaligned w")


def test_fused_generic_kernel_on_workload_slice(monkeypatch):
    """With the specialisations off, the workload geometry runs on the generic
    fused kernel and agrees with the oracle too."""
    monkeypatch.setenv("CONVHIP_TAP", "0")
    cfg = synth.WORKLOADS["conv3d_min_softmax"]
    desc = ch.plan_describe(cfg["x"], cfg["w"], fused=True)
    assert "kernel=fused_min_softmax_mfma4" in desc, desc
    x, w, b = synth.make_inputs("conv3d_min_softmax", n_samples=3)
    y = gpu_fused(x, w, b)
    ref = oracle.conv3d_min_softmax(x, w, b)
    assert float(np.abs(y - ref).max()) <= FUSED_ATOL


def test_fused_integer_inputs_exact_minimum():
    """Integer inputs make every conv value exact, so the minimum is exact and only
    exp/division rounding remains."""
    x, w, b = synth.make_inputs("conv3d_min_softmax", integer=True, n_samples=4)
    w = (w * 0.125).astype(np.float32)  # keep exp in range; still exact (power-of-two scale)
    y = gpu_fused(x, w, b)
    ref = oracle.conv3d_min_softmax(x, w, b)
    assert float(np.abs(y - ref).max()) <= 1e-6


def test_synth_device_matches_host():
    t = torch.empty(1 << 20, dtype=torch.float32, device=dev())
    for kind, kw in [(0, {}), (1, dict(bound=synth.symmetric_bound(81))), (2, dict(lo=-2, span=5))]:
        ch.synth_fill(t, 0xABCDEF, kind, start=12345, **kw)
        host = synth.fill(kind, 0xABCDEF, t.numel(), start=12345, bound=kw.get("bound", 1.0),
                          lo=kw.get("lo", 0), span=kw.get("span", 1))
        np.testing.assert_array_equal(t.cpu().numpy(), host)


CFG_CASES = [
    ((2, 3, 9, 10, 11), (8, 3, 3, 3, 3), 1, 1, 0, 1),
    ((1, 4, 7, 9, 10), (6, 2, 2, 3, 2), (1, 2, 2), (1, 1, 2), (1, 2, 3), 2),
    ((1, 3, 40), (5, 3, 3), 3, 4, 0, 1),
    ((1, 4, 3, 12, 13), (16, 2, 2, 3, 3), 1, (1, 1, 2), 1, 2),
    ((2, 3, 4, 14, 14), (70, 3, 3, 3, 3), 1, 1, 0, 1),
    ((1, 5, 900), (33, 5, 3), 3, 4, 1, 1),
]


@pytest.mark.parametrize("cfg", range(8))
def test_every_tile_config_integer_exact(cfg, monkeypatch):
    """Each tile configuration of the conv kernel (forced through CONVHIP_CONV_CFG)
    gives the exact oracle result on shapes with ragged tiles and chunk tails."""
    monkeypatch.setenv("CONVHIP_CONV_CFG", str(cfg))
    r = np.random.default_rng(77 + cfg)
    for xs, ws, s, d, p, g in CFG_CASES:
        x, w, b = _int_inputs(r, xs, ws, bias=True)
        say(f"cfg {cfg}: x={xs} w={ws}: " + ch.plan_describe(xs, ws, s, d, p, g))
        y = gpu_conv(x, w, b, s, d, p, g)
        np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, s, d, p, g))


# Output widths around the 16-position tile step: one step wraps no row (width
# >= 16), exactly one (16 > width > 8) or several rows (width 1, 2, 3, 5, 8).
FLAT_WIDTHS = [1, 2, 3, 5, 8, 15, 16, 17, 31, 33]


@pytest.mark.parametrize("cfg", [None] + list(range(8)))
def test_flat_tile_positions_every_width(cfg, monkeypatch):
    """Tiles of 16 flattened (row, column) positions, stepped through planes of
    every width class, under the default plan and each forced tile configuration."""
    if cfg is not None:
        monkeypatch.setenv("CONVHIP_CONV_CFG", str(cfg))
    r = np.random.default_rng(900 + (cfg if cfg is not None else 9))
    for wo in FLAT_WIDTHS:
        for sw in (1, 2):
            xs, ws = (1, 3, 11, (wo - 1) * sw + 3), (8, 3, 3, 3)
            s, d, p, g = (1, sw), 1, 0, 1
            x, w, b = _int_inputs(r, xs, ws, bias=True)
            say(f"flat width {wo} stride {sw} cfg {cfg}: " + ch.plan_describe(xs, ws, s, d, p, g))
            y = gpu_conv(x, w, b, s, d, p, g)
            np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, s, d, p, g))


# Shapes that keep the geometry of a build-time specialisation (channel chunk,
# taps, dilations, staged box) with fewer samples / shorter extents, so the
# specialised persistent kernel runs on sizes the oracle checks in full.
TAP_CASES = [
    ((2, 3, 8, 64, 64), (64, 3, 3, 5, 7), 1, 1, 0, True),
    ((2, 3, 5, 64, 64), (40, 3, 3, 5, 7), 1, 1, 0, False),   # fewer output channels, one sample per item
    ((3, 3, 9, 64, 64), (64, 3, 3, 5, 7), 1, 1, 0, True),    # odd item count per workgroup
    ((2, 64, 3000), (128, 64, 3), 3, 4, 0, False),
    ((1, 64, 5000), (100, 64, 3), 3, 4, 4, True),            # padding, ragged last tile
    ((4, 64, 200000), (128, 64, 3), 3, 4, 0, False),         # several items per workgroup
]


@pytest.mark.parametrize("case", range(len(TAP_CASES)))
def test_tap_specialised_kernel_integer_exact(case):
    xs, ws, s, d, p, bias = TAP_CASES[case]
    desc = ch.plan_describe(xs, ws, s, d, p, 1)
    assert "kernel=conv_tap" in desc, desc
    r = np.random.default_rng(400 + case)
    x, w, b = _int_inputs(r, xs, ws, bias=bias)
    say(f"tap case {case}: x={xs} w={ws}: {desc}")
    y = gpu_conv(x, w, b, s, d, p, 1)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, s, d, p, 1))


SPLIT_CASES = [
    # general Conv3d geometry (groups 2, stride (1,2,2), dilation (1,1,2)) with fewer planes
    ((1, 16, 6, 32, 32), (32, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (1, 2, 3), 2),
    ((2, 16, 3, 32, 32), (20, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (0, 2, 3), 2),
    ((1, 8, 4, 32, 32), (16, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (1, 2, 3), 1),
    # depth stride 2 (the depth-tap rotation no longer lines up with the planes neighbours share)
    ((1, 16, 7, 32, 32), (32, 8, 3, 5, 7), (2, 2, 2), (1, 1, 2), (1, 2, 3), 2),
    # depth padding 2: whole padding planes in the box
    ((2, 16, 3, 32, 32), (32, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (2, 2, 3), 2),
    # tiny Conv3d geometry
    ((2, 3, 4, 16, 16), (8, 3, 3, 3, 3), 1, 1, 0, 1),
    ((1, 3, 5, 16, 16), (5, 3, 3, 3, 3), 1, 1, 0, 1),
]


@pytest.mark.parametrize("pipe", ["1", "0"])
@pytest.mark.parametrize("case", range(len(SPLIT_CASES)))
def test_split_specialised_kernel_integer_exact(case, pipe, monkeypatch):
    """Both channel-split kernels: the pipelined one (batch sums overlapped with
    products; the general geometry's 13 tiles) and the one summing at the end."""
    monkeypatch.setenv("CONVHIP_SPLIT_PIPE", pipe)
    xs, ws, s, d, p, g = SPLIT_CASES[case]
    desc = ch.plan_describe(xs, ws, s, d, p, g)
    assert "kernel=conv_tap_split" in desc, desc
    assert ("pipe=1" in desc) == (pipe == "1" and tuple(ws[2:]) == (3, 5, 7)), desc
    r = np.random.default_rng(500 + case)
    x, w, b = _int_inputs(r, xs, ws, bias=case % 2 == 0)
    say(f"split case {case}: x={xs} w={ws}: {desc}")
    y = gpu_conv(x, w, b, s, d, p, g)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, s, d, p, g))


# The general Conv3d's channel/kernel/dilation geometry on smaller batches and
# depths, with padding planes, depth stride 2 and fewer output channels: the
# workgroup-stream-K kernel (13 tiles per plane: 3 whole tiles per wave plus one
# tile split over the waves by reduction blocks).
KSTREAM_CASES = SPLIT_CASES[:5]


@pytest.mark.parametrize("case", range(len(KSTREAM_CASES)))
def test_kstream_specialised_kernel_integer_exact(case):
    xs, ws, s, d, p, g = KSTREAM_CASES[case]
    desc = ch.plan_describe(xs, ws, s, d, p, g)
    assert "kernel=conv_tap_kstream" in desc, desc
    r = np.random.default_rng(600 + case)
    x, w, b = _int_inputs(r, xs, ws, bias=case % 2 == 0)
    say(f"kstream case {case}: x={xs} w={ws}: {desc}")
    y = gpu_conv(x, w, b, s, d, p, g)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, s, d, p, g))


# The tiny Conv3d's channel/kernel geometry (3 input channels, 3x3x3, no
# padding) on ragged inputs: strides, 2 groups, a single output position, 16
# output channels and a last wave with one valid position. The direct kernel
# reads its operands from global memory, one wave per 16 positions.
DIRECT_CASES = [
    ((2, 3, 16, 16, 16), (8, 3, 3, 3, 3), 1, 1, 0, 1),
    ((1, 3, 9, 11, 13), (5, 3, 3, 3, 3), (2, 1, 3), 1, 0, 1),
    ((3, 6, 7, 8, 5), (10, 3, 3, 3, 3), (1, 2, 1), 1, 0, 2),
    ((1, 3, 3, 3, 3), (16, 3, 3, 3, 3), 1, 1, 0, 1),
    ((1, 3, 20, 20, 20), (16, 3, 3, 3, 3), 1, 1, 0, 1),
    ((17, 3, 3, 3, 3), (7, 3, 3, 3, 3), 1, 1, 0, 1),
]


@pytest.mark.parametrize("case", range(len(DIRECT_CASES)))
def test_direct_kernel_integer_exact(case):
    xs, ws, s, d, p, g = DIRECT_CASES[case]
    desc = ch.plan_describe(xs, ws, s, d, p, g)
    assert "kernel=conv_direct16" in desc, desc
    r = np.random.default_rng(800 + case)
    x, w, b = _int_inputs(r, xs, ws, bias=case % 2 == 0)
    say(f"direct case {case}: x={xs} w={ws}: {desc}")
    y = gpu_conv(x, w, b, s, d, p, g)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, s, d, p, g))


def test_tap_disabled_falls_back_to_streamed(monkeypatch):
    monkeypatch.setenv("CONVHIP_TAP", "0")
    xs, ws, s, d, p, _ = TAP_CASES[0]
    desc = ch.plan_describe(xs, ws, s, d, p, 1)
    assert "kernel=conv_mfma16 " in desc + " ", desc
    r = np.random.default_rng(5)
    x, w, b = _int_inputs(r, xs, ws, bias=True)
    y = gpu_conv(x, w, b, s, d, p, 1)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, s, d, p, 1))


def test_workloads_use_expected_kernels():
    cfg = synth.WORKLOADS["conv3d_min_softmax"]
    d = ch.plan_describe(cfg["x"], cfg["w"], fused=True)
    assert "kernel=fused_stream" in d, d
    for name, kernel in [("asym_conv3d", "conv_tap"), ("long_conv1d", "conv_tap"),
                         ("general_conv3d", "conv_tap_kstream"), ("tiny_conv3d", "conv_direct16")]:
        cfg = synth.WORKLOADS[name]
        d = ch.plan_describe(cfg["x"], cfg["w"], *_cfg_args(cfg)) + " "
        assert f"kernel={kernel}" in d, d


def test_peak_probes_run_and_count_their_work():
    """The calibration probes launch on the caller's stream and report the work
    of one launch: 4 workgroups of 4 waves per compute unit."""
    sink = torch.zeros(1, dtype=torch.float32, device=dev())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves = 4 * cus * 4
    assert ch.peak_probe(ch.PROBE_MFMA_F32, 3, sink) == waves * 3 * 8 * 2 * 16 * 16 * 4
    assert ch.peak_probe(ch.PROBE_FMA_F32, 3, sink) == waves * 64 * 3 * 8 * 2
    torch.cuda.synchronize()
    assert float(sink.cpu()[0]) == 0.0  # the guard store never fires


def test_split_pipe_wait_give_up_stores_nan(monkeypatch):
    """The pipelined channel-split kernel caps its wait for the other waves'
    batch-1 tiles. A wave that gives up stores NaN for its whole tile, never a
    sum over tiles that may not be parked yet. The cap is forced to zero from
    the host (every kernel still exits normally): each plane's batch-1 tiles
    (positions 0..111 of 208) are NaN, the rest exact; with the default cap the
    output is exact everywhere."""
    name = "general_conv3d"
    cfg = synth.WORKLOADS[name]
    monkeypatch.setenv("CONVHIP_SPLIT_PIPE", "1")
    desc = ch.plan_describe(cfg["x"], cfg["w"], *_cfg_args(cfg))
    assert "pipe=1" in desc, desc
    x, w, b = synth.make_inputs(name, integer=True, n_samples=1)
    ref = oracle.conv(x, w, b, *_cfg_args(cfg))
    monkeypatch.setenv("CONVHIP_SPIN_CAP", "0")
    y = gpu_conv(x, w, b, *_cfg_args(cfg)).reshape(ref.shape[0], ref.shape[1], ref.shape[2], -1)
    r = ref.reshape(y.shape)
    assert np.isnan(y[..., :112]).all()
    np.testing.assert_array_equal(y[..., 112:].astype(np.float64), r[..., 112:])
    monkeypatch.delenv("CONVHIP_SPIN_CAP")
    y = gpu_conv(x, w, b, *_cfg_args(cfg))
    np.testing.assert_array_equal(y.astype(np.float64), ref)


# Neighbours of the workloads that no specialisation was built for exactly:
# smaller inputs (the staged box at the specialisation's extents, fewer rows
# or columns read) and another dilation / channel count.
NEIGHBOUR_CASES = [
    # name, workload variant, batch samples checked (None: all), kernel
    ("asym_conv3d_48", 2, "kernel=conv_tap cfg=2"),
    ("general_conv3d_24", None, "kernel=conv_tap_kstream cfg=1"),
]


@pytest.mark.parametrize("case", NEIGHBOUR_CASES, ids=[c[0] for c in NEIGHBOUR_CASES])
def test_neighbour_shapes_integer_exact(case):
    name, nsamp, kernel = case
    cfg = synth.config(name)
    x, w, b = synth.make_inputs(name, integer=True, n_samples=nsamp)
    desc = ch.plan_describe(x.shape, cfg["w"], *_cfg_args(cfg))
    assert kernel in desc, desc
    say(f"neighbour {name} x={x.shape}: {desc}")
    y = gpu_conv(x, w, b, *_cfg_args(cfg))
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, *_cfg_args(cfg)))


@pytest.mark.parametrize("L,p,bias", [(20000, 0, False), (3000, 4, True)])
def test_neighbour_conv1d_96_channels_dilation_2_integer_exact(L, p, bias):
    """The long Conv1d with 96 output channels and dilation 2 (its own
    specialisation, 96 channels x 256 positions), on shorter rows."""
    xs, ws = (2, 64, L), (96, 64, 3)
    desc = ch.plan_describe(xs, ws, 3, 2, p, 1)
    assert "kernel=conv_tap cfg=3" in desc, desc
    r = np.random.default_rng(700 + L)
    x, w, b = _int_inputs(r, xs, ws, bias=bias)
    y = gpu_conv(x, w, b, 3, 2, p, 1)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, 3, 2, p, 1))


def test_tap_box_narrower_than_pitch_integer_exact():
    """The 12-row asymmetric-Conv3d specialisation on inputs of several widths
    (box columns fewer than its 64-float pitch, rows fewer than 12)."""
    r = np.random.default_rng(720)
    for W in (44, 48, 52, 56):
        xs, ws = (1, 3, 5, W, W), (64, 3, 3, 5, 7)
        desc = ch.plan_describe(xs, ws, 1, 1, 0, 1)
        assert "kernel=conv_tap" in desc, desc
        x, w, b = _int_inputs(r, xs, ws, bias=True)
        say(f"tap narrow W={W}: {desc}")
        y = gpu_conv(x, w, b, 1, 1, 0, 1)
        np.testing.assert_array_equal(y.astype(np.float64), oracle.conv(x, w, b, 1, 1, 0, 1))


# NaN inputs. A NaN reaches every output whose receptive field holds it, in the
# oracle and on the GPU alike: the kernels' padded reduction indices carry zero
# weights and read the position's own first tap, which lies in that field, and
# the fused op's minimum propagates NaN as torch.min does. (Infinities are not
# covered: a zero-weight padded index times an infinity is NaN where the
# definition gives an infinity.)
NAN_CASES = [
    ("direct", (2, 3, 16, 16, 16), (8, 3, 3, 3, 3), 1, 1, 0, 1, "conv_direct16"),
    ("kstream", (1, 16, 6, 32, 32), (32, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (1, 2, 3), 2, "conv_tap_kstream"),
    ("tap", (2, 3, 8, 64, 64), (64, 3, 3, 5, 7), 1, 1, 0, 1, "conv_tap"),
    ("tap_conv1d", (2, 64, 3000), (128, 64, 3), 3, 4, 0, 1, "conv_tap"),
    ("generic", (2, 5, 7, 9, 11), (6, 5, 2, 3, 2), (1, 2, 1), (2, 1, 1), (1, 0, 2), 1, "conv_mfma16"),
]


@pytest.mark.parametrize("case", NAN_CASES, ids=[c[0] for c in NAN_CASES])
def test_nan_inputs_propagate_like_the_definition(case):
    name, xs, ws, s, d, p, g, kernel = case
    desc = ch.plan_describe(xs, ws, s, d, p, g)
    assert f"kernel={kernel} " in desc + " ", desc
    r = np.random.default_rng(zlib.crc32(name.encode()))
    x, w, b = _int_inputs(r, xs, ws, bias=True)
    flat = x.reshape(-1)
    for i in r.choice(flat.size, size=3, replace=False):
        flat[i] = np.nan
    say(f"nan {name}: {desc}")
    y = gpu_conv(x, w, b, s, d, p, g).astype(np.float64)
    ref = oracle.conv(x, w, b, s, d, p, g)
    nan_ref = np.isnan(ref)
    assert nan_ref.any() and not nan_ref.all()
    np.testing.assert_array_equal(np.isnan(y), nan_ref)
    np.testing.assert_array_equal(y[~nan_ref], ref[~nan_ref])


@pytest.mark.parametrize("min_dim", [2, 3, 4])
def test_fused_nan_inputs_propagate_like_torch_min(min_dim):
    """min_dim 2 and 3 take the depth-streamed kernel, 4 the generic one."""
    xs, ws = (2, 3, 6, 32, 32), (24, 3, 3, 3, 3)
    r = np.random.default_rng(77 + min_dim)
    x, w, b = _float_inputs(r, xs, ws, True)
    x[0, 1, 2, 5, 7] = np.nan
    x[1, 0, 4, 20, 30] = np.nan
    desc = ch.plan_describe(xs, ws, 1, 1, 0, 1, fused=True, min_dim=min_dim)
    say(f"fused nan min_dim {min_dim}: {desc}")
    y = gpu_fused(x, w, b, 1, 1, 0, 1, min_dim)
    ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, 0, 1, min_dim)
    nan_ref = np.isnan(ref)
    assert nan_ref.any() and not nan_ref.all()
    np.testing.assert_array_equal(np.isnan(y), nan_ref)
    assert float(np.abs(y[~nan_ref] - ref[~nan_ref]).max()) <= FUSED_ATOL
