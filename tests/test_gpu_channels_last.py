"""GPU parity of the channels-last convolution (x [N, spatial..., C_in] ->
y [N, out..., C_out]) against the fp64 oracle on the same seeded inputs.

Integer-valued inputs keep every partial sum an exact fp32 integer, so those
cases compare bit for bit; uniform inputs use the conv tolerance
1e-4 * sqrt(K_red) * max|y_ref|.
"""
import zlib

import numpy as np
import pytest
import torch

import implicit_gemm_convolution_direct_amd as ch
import oracle
import synth
from gpu_util import assert_conv_close, dev, say, to_dev

pytestmark = pytest.mark.gpu


def _int_inputs(r, xs_cl, ws, bias):
    x = r.integers(0, 4, size=xs_cl).astype(np.float32)
    w = r.integers(-2, 3, size=ws).astype(np.float32)
    b = r.integers(-4, 5, size=ws[0]).astype(np.float32) if bias else None
    return x, w, b


def _float_inputs(r, xs_cl, ws, bias):
    x = r.random(xs_cl, dtype=np.float32)
    fan = int(np.prod(ws[1:]))
    w = ((r.random(ws, dtype=np.float32) * 2 - 1) / np.sqrt(fan)).astype(np.float32)
    b = ((r.random(ws[0], dtype=np.float32) * 2 - 1) / np.sqrt(fan)).astype(np.float32) if bias else None
    return x, w, b


def gpu_conv_cl(x, w, b, s, d, p, g, out=None):
    y = ch.conv_fwd_channels_last(to_dev(x), to_dev(w), to_dev(b), s, d, p, g, out=out)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _random_geometry(r, nd):
    g = int(r.choice([1, 1, 2, 4]))
    cg = int(r.choice([1, 2, 3, 5, 8, 16, 24]))
    coutg = int(r.choice([1, 3, 4, 8, 16, 20, 33, 64, 70, 128]))
    if g > 1:
        coutg = min(coutg, 40)
    ks = [int(r.integers(1, 6)) for _ in range(nd)]
    s = [int(r.integers(1, 4)) for _ in range(nd)]
    d = [int(r.integers(1, 4)) for _ in range(nd)]
    p = [int(r.integers(0, 4)) for _ in range(nd)]
    Ls = []
    for a in range(nd):
        lo = max(1, d[a] * (ks[a] - 1) + 1 - 2 * p[a])
        Ls.append(int(r.integers(lo, lo + {1: 500, 2: 40, 3: 14}[nd])))
    N = int(r.integers(1, 3))
    return (N, *Ls, g * cg), (g * coutg, cg, *ks), s, d, p, g


RANDOM_CASES = [(nd, seed) for nd in (1, 2, 3) for seed in range(8)]


def test_flat_tile_positions_every_width_channels_last():
    """Tiles of 16 flattened (row, column) positions over planes of every width
    class (a step wraps no row, one row, or several), channels-last."""
    r = np.random.default_rng(950)
    for wo in (1, 2, 3, 5, 8, 15, 16, 17, 31, 33):
        for sw in (1, 2):
            xs, ws = (1, 11, (wo - 1) * sw + 3, 4), (8, 4, 3, 3)
            s, d, p, g = (1, sw), 1, 0, 1
            x, w, b = _int_inputs(r, xs, ws, bias=True)
            say(f"cl flat width {wo} stride {sw}: " + ch.plan_describe(xs, ws, s, d, p, g, channels_last=True))
            y = gpu_conv_cl(x, w, b, s, d, p, g)
            np.testing.assert_array_equal(y.astype(np.float64), oracle.conv_channels_last(x, w, b, s, d, p, g))


@pytest.mark.parametrize("nd,seed", RANDOM_CASES)
def test_channels_last_random_integer_exact(nd, seed):
    r = np.random.default_rng(7000 + 100 * nd + seed)
    xs, ws, s, d, p, g = _random_geometry(r, nd)
    x, w, b = _int_inputs(r, xs, ws, bias=bool(seed % 2))
    say(f"cl case nd={nd} seed={seed} x={xs} w={ws} s={s} d={d} p={p} g={g}: "
        + ch.plan_describe(xs, ws, s, d, p, g, channels_last=True))
    y = gpu_conv_cl(x, w, b, s, d, p, g)
    ref = oracle.conv_channels_last(x, w, b, s, d, p, g)
    assert np.abs(ref).max() < 2 ** 24
    np.testing.assert_array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("nd,seed", RANDOM_CASES[::3])
def test_channels_last_random_float(nd, seed):
    r = np.random.default_rng(7500 + 100 * nd + seed)
    xs, ws, s, d, p, g = _random_geometry(r, nd)
    x, w, b = _float_inputs(r, xs, ws, bias=True)
    say(f"cl float nd={nd} seed={seed} x={xs} w={ws}")
    y = gpu_conv_cl(x, w, b, s, d, p, g)
    assert_conv_close(y, oracle.conv_channels_last(x, w, b, s, d, p, g), ws, f"cl float nd={nd} seed={seed}")


EDGE_CASES = [
    # name, x shape (channels last), w shape, stride, dilation, padding, groups
    ("cout_odd_scalar_stores", (2, 5, 6, 7, 3), (5, 3, 3, 3, 3), 1, 1, 1, 1),
    ("coutg_2_scalar_stores", (1, 6, 7, 8, 4), (4, 2, 2, 3, 3), 1, 1, 0, 2),
    ("depthwise", (2, 5, 9, 11, 6), (6, 1, 3, 3, 3), 1, 1, 1, 6),
    ("kernel_1x1x1", (2, 4, 6, 7, 5), (7, 5, 1, 1, 1), 1, 1, 0, 1),
    ("single_output", (1, 3, 4, 5, 2), (3, 2, 3, 4, 5), 1, 1, 0, 1),
    ("padding_wider_than_kernel", (1, 3, 3, 3, 2), (4, 2, 2, 2, 2), 1, 1, 3, 1),
    ("stride_gt_kernel", (1, 9, 17, 33, 3), (5, 3, 2, 2, 2), (4, 3, 5), 1, 0, 1),
    ("many_input_channels", (1, 4, 4, 40, 200), (16, 200, 1, 1, 3), 1, 1, 0, 1),
    ("cin64_conv1d_geometry", (2, 3001, 64), (128, 64, 3), 3, 4, 2, 1),
    ("cout_129_two_channel_tiles", (1, 300, 4), (129, 4, 3), 3, 4, 0, 1),
    ("conv1d_long_row_tiles", (2, 5000, 3), (16, 3, 5), 1, 2, 2, 1),
    ("conv2d", (2, 32, 32, 16), (32, 8, 5, 7), (2, 2), (1, 2), (2, 3), 2),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_channels_last_edge_cases_integer_exact(case):
    name, xs, ws, s, d, p, g = case
    r = np.random.default_rng(sum(map(ord, name)))
    x, w, b = _int_inputs(r, xs, ws, bias=True)
    say(f"cl edge {name}: " + ch.plan_describe(xs, ws, s, d, p, g, channels_last=True))
    y = gpu_conv_cl(x, w, b, s, d, p, g)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv_channels_last(x, w, b, s, d, p, g))


def test_channels_last_misaligned_output_and_input():
    """Views 4 bytes past an allocation: y takes the scalar stores, x the same
    copies; results unchanged."""
    r = np.random.default_rng(11)
    xs, ws = (2, 6, 7, 8, 4), (8, 4, 3, 3, 3)
    x, w, b = _int_inputs(r, xs, ws, bias=True)
    xd = torch.empty(x.size + 1, dtype=torch.float32, device=dev())[1:].view(xs)
    xd.copy_(torch.from_numpy(x))
    ys = (2, 4, 5, 6, 8)
    yd = torch.empty(int(np.prod(ys)) + 1, dtype=torch.float32, device=dev())[1:].view(ys)
    assert xd.data_ptr() % 16 != 0 and yd.data_ptr() % 16 != 0
    ch.conv_fwd_channels_last(xd, to_dev(w), to_dev(b), 1, 1, 0, 1, out=yd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(yd.cpu().numpy().astype(np.float64),
                                  oracle.conv_channels_last(x, w, b, 1, 1, 0, 1))


CFG_CASES = [
    ((2, 9, 10, 11, 3), (8, 3, 3, 3, 3), 1, 1, 0, 1),
    ((1, 7, 9, 10, 4), (6, 2, 2, 3, 2), (1, 2, 2), (1, 1, 2), (1, 2, 3), 2),
    ((1, 900, 5), (33, 5, 3), 3, 4, 1, 1),
    ((2, 4, 14, 14, 3), (70, 3, 3, 3, 3), 1, 1, 0, 1),
]


@pytest.mark.parametrize("cfg", range(8))
def test_channels_last_every_tile_config_integer_exact(cfg, monkeypatch):
    monkeypatch.setenv("CONVHIP_CONV_CFG", str(cfg))
    r = np.random.default_rng(88 + cfg)
    for xs, ws, s, d, p, g in CFG_CASES:
        x, w, b = _int_inputs(r, xs, ws, bias=True)
        say(f"cl cfg {cfg}: x={xs} w={ws}: " + ch.plan_describe(xs, ws, s, d, p, g, channels_last=True))
        y = gpu_conv_cl(x, w, b, s, d, p, g)
        np.testing.assert_array_equal(y.astype(np.float64), oracle.conv_channels_last(x, w, b, s, d, p, g))


def _cl_workload_inputs(name, integer=False, n_samples=None):
    """A workload's seeded inputs (NCDHW / NCL), moved to channels-last order."""
    x, w, b = synth.make_inputs(name, integer=integer, n_samples=n_samples)
    return np.ascontiguousarray(np.moveaxis(x, 1, -1)), w, b


@pytest.mark.parametrize("name", ["tiny_conv3d", "general_conv3d"])
def test_channels_last_workload_full(name):
    cfg = synth.WORKLOADS[name]
    args = (cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"])
    for integer in (True, False):
        x, w, b = _cl_workload_inputs(name, integer=integer)
        say(f"cl workload {name} integer={integer}: "
            + ch.plan_describe(x.shape, w.shape, *args, channels_last=True))
        y = gpu_conv_cl(x, w, b, *args)
        ref = oracle.conv_channels_last(x, w, b, *args)
        if integer:
            np.testing.assert_array_equal(y.astype(np.float64), ref)
        else:
            assert_conv_close(y, ref, w.shape, f"cl {name}")


def test_channels_last_matches_ncdhw_path_bit_for_bit_on_integers():
    """The two layouts give the same exact results (integer inputs)."""
    cfg = synth.WORKLOADS["general_conv3d"]
    args = (cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"])
    x, w, b = synth.make_inputs("general_conv3d", integer=True, n_samples=2)
    y_ncdhw = ch.conv_fwd(to_dev(x), to_dev(w), to_dev(b), *args)
    x_cl = to_dev(np.ascontiguousarray(np.moveaxis(x, 1, -1)))
    y_cl = ch.conv_fwd_channels_last(x_cl, to_dev(w), to_dev(b), *args)
    torch.cuda.synchronize()
    assert torch.equal(y_cl, y_ncdhw.movedim(1, -1))


def test_channels_last_asym_workload_slices():
    """Full-size asymmetric Conv3d in channels-last order, checked on two samples."""
    name = "asym_conv3d"
    cfg = synth.WORKLOADS[name]
    args = (cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"])
    x, w, _ = _cl_workload_inputs(name)
    say(f"cl workload {name}: " + ch.plan_describe(x.shape, w.shape, *args, channels_last=True))
    y = ch.conv_fwd_channels_last(to_dev(x), to_dev(w), None, *args)
    torch.cuda.synchronize()
    for n in (0, x.shape[0] - 1):
        ref = oracle.conv_channels_last(x[n:n + 1], w, None, *args)
        assert_conv_close(y[n:n + 1].cpu().numpy(), ref, w.shape, f"cl {name} sample {n}")


# Shapes with the geometries of the channels-last tap specialisations (Conv1d
# 64 -> <=128 channels, k = 3, dilation 4, 8 channels per chunk; Conv3d 3 -> <=64
# channels, kernel 3x5x7 on 64x64 planes) at sizes the oracle checks in full.
TAP_CL_CASES = [
    ((2, 3000, 64), (128, 64, 3), 3, 4, 0, False),
    ((1, 5000, 64), (100, 64, 3), 3, 4, 4, True),     # padding, fewer channels, ragged last tile
    ((2, 3001, 64), (128, 64, 3), 3, 4, 2, True),
    ((4, 200000, 64), (128, 64, 3), 3, 4, 0, False),  # several items per workgroup
    ((2, 2000, 64), (128, 64, 3), 2, 4, 1, True),     # stride 2: a narrower box inside the staged one
    # asymmetric Conv3d geometry (C_in = 3: float-by-float box copies)
    ((2, 8, 64, 64, 3), (64, 3, 3, 5, 7), 1, 1, 0, True),
    ((2, 5, 64, 64, 3), (40, 3, 3, 5, 7), 1, 1, 0, False),  # fewer output channels
    ((3, 9, 64, 64, 3), (64, 3, 3, 5, 7), 1, 1, 0, True),   # odd item count per workgroup
]


@pytest.mark.parametrize("case", range(len(TAP_CL_CASES)))
def test_channels_last_tap_kernel_integer_exact(case):
    xs, ws, s, d, p, bias = TAP_CL_CASES[case]
    desc = ch.plan_describe(xs, ws, s, d, p, 1, channels_last=True)
    assert "kernel=conv_tap " in desc and "layout=channels_last" in desc, desc
    r = np.random.default_rng(600 + case)
    x, w, b = _int_inputs(r, xs, ws, bias)
    say(f"cl tap case {case}: x={xs} w={ws}: {desc}")
    y = gpu_conv_cl(x, w, b, s, d, p, 1)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv_channels_last(x, w, b, s, d, p, 1))


def test_channels_last_tap_disabled_and_misaligned_take_generic(monkeypatch):
    """CONVHIP_TAP=0, or an x that is not 16-byte aligned, keep the channels-last
    call on the generic kernel; results unchanged."""
    xs, ws, s, d, p, _ = TAP_CL_CASES[0]
    r = np.random.default_rng(9)
    x, w, b = _int_inputs(r, xs, ws, True)
    ref = oracle.conv_channels_last(x, w, b, s, d, p, 1)
    xd = torch.empty(x.size + 1, dtype=torch.float32, device=dev())[1:].view(xs)
    xd.copy_(torch.from_numpy(x))
    assert xd.data_ptr() % 16 != 0
    y = ch.conv_fwd_channels_last(xd, to_dev(w), to_dev(b), s, d, p, 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy().astype(np.float64), ref)
    monkeypatch.setenv("CONVHIP_TAP", "0")
    desc = ch.plan_describe(xs, ws, s, d, p, 1, channels_last=True)
    assert "kernel=conv_mfma16 " in desc, desc
    np.testing.assert_array_equal(gpu_conv_cl(x, w, b, s, d, p, 1).astype(np.float64), ref)


def test_channels_last_long_conv1d_full_size_slices():
    """The long Conv1d in channels-last order at full size (x [64, 524280, 64],
    8.6 GB, generated on the device): two samples regenerated on the host are
    checked bit for bit against the device copy and their outputs against the
    oracle."""
    cfg = synth.WORKLOADS["long_conv1d"]
    N, C, L = cfg["x"]
    xs = (N, L, C)
    sx, _, _ = cfg["seeds"]
    args = (cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"])
    _, w, _ = synth.make_inputs("long_conv1d", n_samples=1)
    say("cl long conv1d: " + ch.plan_describe(xs, w.shape, *args, channels_last=True))
    xd = torch.empty(xs, dtype=torch.float32, device=dev())
    ch.synth_fill(xd, sx, ch.KIND_UNIFORM01)
    y = ch.conv_fwd_channels_last(xd, to_dev(w), None, *args)
    torch.cuda.synchronize()
    per = L * C
    for n in (0, N - 1):
        xh = synth.uniform01(sx, (1, L, C), start=n * per)
        np.testing.assert_array_equal(xd[n:n + 1].cpu().numpy(), xh)
        ref = oracle.conv_channels_last(xh, w, None, *args)
        assert_conv_close(y[n:n + 1].cpu().numpy(), ref, w.shape, f"cl long conv1d n={n}")
    del xd, y
    torch.cuda.empty_cache()


# Geometries of the channel-split specialisations (general and tiny Conv3d) in
# channels-last order, with fewer planes.
SPLIT_CL_CASES = [
    ((1, 6, 32, 32, 16), (32, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (1, 2, 3), 2),
    ((2, 3, 32, 32, 16), (20, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (0, 2, 3), 2),
    ((1, 4, 32, 32, 8), (16, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (1, 2, 3), 1),
    ((1, 7, 32, 32, 16), (32, 8, 3, 5, 7), (2, 2, 2), (1, 1, 2), (1, 2, 3), 2),
    ((2, 3, 32, 32, 16), (32, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (2, 2, 3), 2),
    ((2, 4, 16, 16, 3), (8, 3, 3, 3, 3), 1, 1, 0, 1),
    ((1, 5, 16, 16, 3), (5, 3, 3, 3, 3), 1, 1, 0, 1),
]


@pytest.mark.parametrize("pipe", ["1", "0"])
@pytest.mark.parametrize("case", range(len(SPLIT_CL_CASES)))
def test_channels_last_split_kernel_integer_exact(case, pipe, monkeypatch):
    monkeypatch.setenv("CONVHIP_SPLIT_PIPE", pipe)
    xs, ws, s, d, p, g = SPLIT_CL_CASES[case]
    desc = ch.plan_describe(xs, ws, s, d, p, g, channels_last=True)
    assert "kernel=conv_tap_split" in desc and "layout=channels_last" in desc, desc
    assert ("pipe=1" in desc) == (pipe == "1" and tuple(ws[2:]) == (3, 5, 7)), desc
    r = np.random.default_rng(700 + case)
    x, w, b = _int_inputs(r, xs, ws, bias=case % 2 == 0)
    say(f"cl split case {case}: x={xs} w={ws}: {desc}")
    y = gpu_conv_cl(x, w, b, s, d, p, g)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv_channels_last(x, w, b, s, d, p, g))


# The general Conv3d geometry's channels-last cases on the stream-K kernel (the
# planner's default for them).
KSTREAM_CL_CASES = SPLIT_CL_CASES[:5]


@pytest.mark.parametrize("case", range(len(KSTREAM_CL_CASES)))
def test_channels_last_kstream_kernel_integer_exact(case):
    xs, ws, s, d, p, g = KSTREAM_CL_CASES[case]
    desc = ch.plan_describe(xs, ws, s, d, p, g, channels_last=True)
    assert "kernel=conv_tap_kstream" in desc and "layout=channels_last" in desc, desc
    r = np.random.default_rng(1000 + case)
    x, w, b = _int_inputs(r, xs, ws, bias=case % 2 == 0)
    say(f"cl kstream case {case}: x={xs} w={ws}: {desc}")
    y = gpu_conv_cl(x, w, b, s, d, p, g)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv_channels_last(x, w, b, s, d, p, g))


# The direct kernel's cases in channels-last order.
DIRECT_CL_CASES = [
    ((2, 16, 16, 16, 3), (8, 3, 3, 3, 3), 1, 1, 0, 1),
    ((1, 9, 11, 13, 3), (5, 3, 3, 3, 3), (2, 1, 3), 1, 0, 1),
    ((3, 7, 8, 5, 6), (10, 3, 3, 3, 3), (1, 2, 1), 1, 0, 2),
    ((1, 3, 3, 3, 3), (16, 3, 3, 3, 3), 1, 1, 0, 1),
    ((17, 3, 3, 3, 3), (7, 3, 3, 3, 3), 1, 1, 0, 1),
]


@pytest.mark.parametrize("case", range(len(DIRECT_CL_CASES)))
def test_channels_last_direct_kernel_integer_exact(case):
    xs, ws, s, d, p, g = DIRECT_CL_CASES[case]
    desc = ch.plan_describe(xs, ws, s, d, p, g, channels_last=True)
    assert "kernel=conv_direct16" in desc and "layout=channels_last" in desc, desc
    r = np.random.default_rng(900 + case)
    x, w, b = _int_inputs(r, xs, ws, bias=case % 2 == 1)
    say(f"cl direct case {case}: x={xs} w={ws}: {desc}")
    y = gpu_conv_cl(x, w, b, s, d, p, g)
    np.testing.assert_array_equal(y.astype(np.float64), oracle.conv_channels_last(x, w, b, s, d, p, g))


def test_channels_last_split_geometry_misaligned_weights_take_generic():
    """A w view 4 bytes past its allocation keeps the channel-split kernel (16-byte
    weight copies) out; results unchanged."""
    xs, ws, s, d, p, g = SPLIT_CL_CASES[0]
    r = np.random.default_rng(12)
    x, w, b = _int_inputs(r, xs, ws, bias=True)
    wd = torch.empty(w.size + 1, dtype=torch.float32, device=dev())[1:].view(ws)
    wd.copy_(torch.from_numpy(w))
    assert wd.data_ptr() % 16 != 0
    y = ch.conv_fwd_channels_last(to_dev(x), wd, to_dev(b), s, d, p, g)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy().astype(np.float64), oracle.conv_channels_last(x, w, b, s, d, p, g))


# ------------------------------------------------- fused op, channels-last
FUSED_ATOL = 1e-5
FUSED_CL_CASES = [
    # name, x [N, D, H, W, C], w, stride, dilation, padding, groups, min_dim, streamed kernel expected
    ("workload_like_min_d", (2, 6, 32, 32, 3), (24, 3, 3, 3, 3), 1, 1, 0, 1, 2, True),
    ("workload_like_min_h", (2, 6, 20, 32, 3), (24, 3, 3, 3, 3), 1, 1, 0, 1, 3, True),
    ("workload_like_min_w", (1, 5, 32, 12, 3), (24, 3, 3, 3, 3), 1, 1, 0, 1, 4, True),
    ("groups3_min_d", (2, 5, 9, 32, 3), (24, 1, 3, 3, 3), 1, 1, (1, 2, 0), 3, 2, False),
    ("generic_strided_padded", (1, 7, 9, 11, 4), (10, 2, 2, 3, 2), (2, 1, 2), (1, 2, 1), (1, 1, 2), 2, 3, False),
    ("generic_min_w", (2, 5, 6, 9, 3), (5, 3, 1, 2, 4), 1, (1, 1, 2), (0, 1, 1), 1, 4, False),
]


@pytest.mark.parametrize("case", FUSED_CL_CASES, ids=[c[0] for c in FUSED_CL_CASES])
def test_fused_channels_last(case):
    """conv3d_min_softmax on x [N, D, H, W, C_in], y [N, kept axes, C_out], against the
    oracle on the same tensors with the channel axis moved."""
    name, xs, ws, s, d, p, g, md, streamed = case
    desc = ch.plan_describe(xs, ws, s, d, p, g, fused=True, channels_last=True, min_dim=md)
    assert ("kernel=fused_stream spec=" in desc) == streamed, desc
    r = np.random.default_rng(zlib.crc32(name.encode()))
    x, w, b = _float_inputs(r, xs, ws, True)
    say(f"fused channels-last {name}: {desc}")
    y = ch.conv3d_min_softmax_channels_last(to_dev(x), to_dev(w), to_dev(b), s, d, p, g, md)
    torch.cuda.synchronize()
    ref = oracle.conv3d_min_softmax_channels_last(x, w, b, s, d, p, g, md)
    assert tuple(y.shape) == ref.shape, (tuple(y.shape), ref.shape)
    err = float(np.abs(y.cpu().numpy() - ref).max())
    say(f"  max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


def test_fused_channels_last_matches_ncdhw_entry_point():
    """The fused workload's shape on two samples: the channels-last result is the
    NCDHW entry point's result with the channel axis moved, to fp32 rounding."""
    x, w, b = synth.make_inputs("conv3d_min_softmax", n_samples=2)
    xd, wd, bd = to_dev(x), to_dev(w), to_dev(b)
    x_cl = xd.permute(0, 2, 3, 4, 1).contiguous()
    for md in (2, 3, 4):
        y = ch.conv3d_min_softmax(xd, wd, bd, min_dim=md)
        y_cl = ch.conv3d_min_softmax_channels_last(x_cl, wd, bd, min_dim=md)
        torch.cuda.synchronize()
        err = float((y_cl - y.permute(0, 2, 3, 1)).abs().max())
        say(f"  min_dim {md}: channels-last vs NCDHW max|diff| = {err:.3e}")
        assert err <= FUSED_ATOL
