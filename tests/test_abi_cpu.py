"""The C-ABI library loads, exports every declared symbol, and validates
arguments on the host (no GPU needed: every case here returns before any
launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import implicit_gemm_convolution_direct_amd as ch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convhip.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\s*\*)\s*\**\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_names():
    decl = _declared_functions()
    assert set(decl) == set(ch.EXPORTED), decl


def test_library_exports_every_declared_symbol():
    lib = ch.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in ch.STATUS_NAMES.items():
        assert ch.status_string(code).startswith(name)


I64 = lambda *v: (ctypes.c_int64 * len(v))(*v)
I32 = lambda *v: (ctypes.c_int * len(v))(*v)
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _fwd(nd, xs, ws, s, d, p, g, x=FAKE, w=FAKE, y=FAKE):
    return ch.lib().conv_fwd(nd, x, I64(*xs), w, I64(*ws), None, I32(*s), I32(*d), I32(*p), g, y, None)


@pytest.mark.parametrize("args,expect", [
    ((4, (1, 1, 4, 4, 4, 4), (1, 1, 3, 3, 3, 3), (1,) * 4, (1,) * 4, (0,) * 4, 1), -2),  # rank
    ((0, (1, 1), (1, 1), (0,), (0,), (0,), 1), -2),                            # rank
    ((2, (1, 4, 2, 8), (4, 4, 3, 3), (1, 1), (1, 1), (0, 0), 1), -6),          # Conv2d, empty output
    ((3, (1, 4, 8, 8, 8), (4, 2, 3, 3, 3), (1,) * 3, (1,) * 3, (0,) * 3, 1), -3),  # C_in/groups mismatch
    ((3, (1, 4, 8, 8, 8), (4, 4, 3, 3, 3), (1,) * 3, (1,) * 3, (0,) * 3, 0), -4),  # groups < 1
    ((3, (1, 4, 8, 8, 8), (6, 1, 3, 3, 3), (1,) * 3, (1,) * 3, (0,) * 3, 4), -4),  # C_out % groups
    ((3, (1, 6, 8, 8, 8), (4, 2, 3, 3, 3), (1,) * 3, (1,) * 3, (0,) * 3, 4), -4),  # C_in % groups
    ((3, (1, 4, 8, 8, 8), (4, 4, 3, 3, 3), (0, 1, 1), (1,) * 3, (0,) * 3, 1), -5),  # stride
    ((3, (1, 4, 8, 8, 8), (4, 4, 3, 3, 3), (1,) * 3, (1, 0, 1), (0,) * 3, 1), -5),  # dilation
    ((3, (1, 4, 8, 8, 8), (4, 4, 3, 3, 3), (1,) * 3, (1,) * 3, (0, -1, 0), 1), -5),  # padding
    ((1, (1, 4, 8), (4, 4, 3), (3,), (4,), (0,), 1), -6),                      # empty output (8 = d(k-1))
    ((3, (1, 4, 8, 8, 2), (4, 4, 3, 3, 3), (1,) * 3, (1,) * 3, (0,) * 3, 1), -6),
    ((3, (0, 4, 8, 8, 8), (4, 4, 3, 3, 3), (1,) * 3, (1,) * 3, (0,) * 3, 1), -3),  # zero batch
])
def test_conv_fwd_validation_errors(args, expect):
    assert _fwd(*args) == expect


def test_conv_fwd_null_pointers():
    ok = (3, (1, 4, 8, 8, 8), (4, 4, 3, 3, 3), (1,) * 3, (1,) * 3, (0,) * 3, 1)
    assert _fwd(*ok, x=None) == -1
    assert _fwd(*ok, w=None) == -1
    assert _fwd(*ok, y=None) == -1
    lib = ch.lib()
    assert lib.conv_fwd(3, FAKE, None, FAKE, I64(4, 4, 3, 3, 3), None, I32(1, 1, 1), I32(1, 1, 1),
                        I32(0, 0, 0), 1, FAKE, None) == -1


def test_conv_fwd_channels_last_validation_errors():
    lib = ch.lib()
    one, zero = I32(1, 1, 1), I32(0, 0, 0)
    f = lambda nd=3, xs=(1, 8, 8, 8, 4), ws=(4, 4, 3, 3, 3), g=1, x=FAKE, y=FAKE, s=one: \
        lib.conv_fwd_channels_last(nd, x, I64(*xs) if xs else None, FAKE, I64(*ws), None, s, one, zero, g, y, None)
    assert f(nd=4) == -2
    assert f(xs=None) == -1
    assert f(x=None) == -1 and f(y=None) == -1
    assert f(xs=(1, 8, 8, 8, 2)) == -3                     # channel axis is the last entry
    assert f(xs=(1, 8, 8, 8, 6), ws=(4, 2, 3, 3, 3), g=4) == -4
    assert f(xs=(1, 8, 8, 2, 4)) == -6                     # W = 2 < kW
    assert f(s=I32(1, 0, 1)) == -5
    assert f(nd=1, xs=(1, 8, 4), ws=(4, 4, 9)) == -6
    buf = ctypes.create_string_buffer(256)
    assert lib.conv_plan_describe(3, I64(1, 8, 8, 8, 4), I64(4, 4, 3, 3, 3), one, one, zero, 1, 8, buf, 256) == -5
    assert lib.conv_plan_describe(3, I64(1, 8, 8, 8, 4), I64(4, 4, 3, 3, 3), one, one, zero, 1, -1, buf, 256) == -5


def test_fused_plan_per_min_axis(monkeypatch):
    """conv_plan_describe's fused modes: at the fused workload's geometry every
    min axis takes a depth-streamed specialisation that streams over it (min
    over D or H: columns along W, 16-byte row copies, spec 0; min over W:
    columns along H, element copies, spec 2); with the specialisations off,
    the generic fused kernel."""
    xs, ws = (128, 3, 24, 32, 32), (24, 3, 3, 3, 3)
    for md, spec in ((2, 0), (3, 0), (4, 2)):
        d = ch.plan_describe(xs, ws, fused=True, min_dim=md)
        assert f"kernel=fused_stream spec={spec} " in d, d
    d = ch.plan_describe((128, 3, 24, 30, 32), ws, fused=True, min_dim=4)  # H = 30: no spec fits
    assert "kernel=fused_min_softmax_mfma4" in d, d
    monkeypatch.setenv("CONVHIP_TAP", "0")
    d = ch.plan_describe(xs, ws, fused=True, min_dim=4)
    assert "kernel=fused_min_softmax_mfma4" in d, d
    one, zero = I32(1, 1, 1), I32(0, 0, 0)
    buf = ctypes.create_string_buffer(256)
    assert ch.lib().conv_plan_describe(1, I64(1, 8, 40), I64(4, 8, 3), one, one, zero, 1, 3, buf, 256) == -2


def test_channels_last_plans():
    for xs, ws, s, d, p, g, kernel in [
            ((4, 32, 32, 32, 16), (32, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (1, 2, 3), 2, "conv_tap_kstream"),
            ((2, 16, 16, 16, 3), (8, 3, 3, 3, 3), 1, 1, 0, 1, "conv_direct16"),
            ((2, 16, 16, 16, 4), (8, 4, 3, 3, 3), 1, 1, 0, 1, "conv_mfma16"),
            ((4, 4096, 64), (128, 64, 3), 3, 4, 0, 1, "conv_tap"),        # the long Conv1d geometry
            ((16, 64, 64, 64, 3), (64, 3, 3, 5, 7), 1, 1, 0, 1, "conv_tap"),  # the asymmetric Conv3d
            ((4, 4096, 64), (128, 64, 3), 2, 4, 0, 1, "conv_tap"),        # stride 2: a narrower box fits
            ((4, 4096, 64), (128, 64, 3), 3, 2, 0, 1, "conv_mfma16"),     # another dilation: generic
            ((4, 4096, 32), (128, 32, 3), 3, 4, 0, 1, "conv_mfma16")]:
        desc = ch.plan_describe(xs, ws, s, d, p, g, channels_last=True)
        fields = dict(t.split("=", 1) for t in desc.split() if "=" in t)
        assert fields["kernel"] == kernel and fields["layout"] == "channels_last", desc
        assert int(fields["lds"]) <= 160 * 1024, desc
        # generic kernel: channel quads (C_in/groups a multiple of 4) are copied 16 bytes at a time
        if kernel == "conv_mfma16":
            assert fields["copy"] == ("quad" if (xs[-1] // g) % 4 == 0 else "scalar"), desc


def test_direct_kernel_plans():
    """Small problems of the direct kernel's geometry take it in both layouts;
    padding, a larger problem, more than 16 output channels per group or a
    forced channel-split kernel do not."""
    k3 = (8, 3, 3, 3, 3)
    for xs, ws, s, p, g, cl, kernel in [
            ((2, 3, 16, 16, 16), k3, 1, 0, 1, False, "conv_direct16"),
            ((2, 16, 16, 16, 3), k3, 1, 0, 1, True, "conv_direct16"),
            ((1, 3, 9, 11, 13), (5, 3, 3, 3, 3), (2, 1, 3), 0, 1, False, "conv_direct16"),
            ((2, 3, 16, 16, 16), k3, 1, 1, 1, False, "conv_mfma16"),        # padding
            ((2, 3, 40, 40, 40), k3, 1, 0, 1, False, "conv_mfma16"),        # 71M MACs
            ((1, 3, 16, 16, 16), (17, 3, 3, 3, 3), 1, 0, 1, False, "conv_mfma16"),
            ((1, 6, 16, 16, 16), (8, 6, 3, 3, 3), 1, 0, 1, False, "conv_mfma16")]:
        desc = ch.plan_describe(xs, ws, s, 1, p, g, channels_last=cl)
        fields = dict(t.split("=", 1) for t in desc.split() if "=" in t)
        assert fields["kernel"] == kernel, desc
        if kernel == "conv_direct16":
            n_pos = xs[0] * np.prod([(l - 3) // st + 1 for l, st in
                                     zip(xs[2:] if not cl else xs[1:4], np.broadcast_to(s, 3))])
            assert fields["grid"] == f"{(n_pos + 15) // 16}x{g}x1" and fields["lds"] == "0", desc


def test_fused_generic_groups_are_native(monkeypatch):
    """Grouped fused calls reduce over C_in/groups input channels per output
    channel: the multiply-adds issued exceed the algorithmic count only by the
    padding of positions to 64, of each group's channels to 4 and of its
    reduction to 4, never by the number of groups (the generic fused kernel,
    specialisations off)."""
    monkeypatch.setenv("CONVHIP_TAP", "0")
    xs = (128, 3, 24, 32, 32)
    for ws, g, kred in [((24, 3, 3, 3, 3), 1, 81), ((24, 1, 3, 3, 3), 3, 27), ((12, 1, 3, 3, 3), 3, 27),
                        ((6, 2, 3, 3, 3), 3, 54)]:
        xg = (xs[0], ws[1] * g) + xs[2:]
        desc = ch.plan_describe(xg, ws, 1, 1, 0, g, fused=True, min_dim=4)
        f = dict(t.split("=", 1) for t in desc.split() if "=" in t)
        assert f["kernel"] == "fused_min_softmax_mfma4" and int(f["groups"]) == g and int(f["kred"]) == kred, desc
        coutg = ws[0] // g
        pad = (960 / 900) * (((kred + 3) // 4 * 4) / kred) * (((coutg + 3) // 4 * 4) / coutg)
        assert int(f["issued"]) == pytest.approx(int(f["macs"]) * pad, rel=1e-9), desc


def test_conv3d_min_softmax_validation_errors():
    lib = ch.lib()
    xs, ws = I64(2, 3, 6, 6, 6), I64(5, 3, 3, 3, 3)
    one, zero = I32(1, 1, 1), I32(0, 0, 0)
    f = lambda **kw: lib.conv3d_min_softmax(kw.get("x", FAKE), kw.get("xs", xs), FAKE, kw.get("ws", ws), None,
                                            kw.get("s", one), one, zero, kw.get("g", 1), kw.get("md", 2),
                                            kw.get("y", FAKE), None)
    assert f(y=None) == -1
    assert f(md=5) == -5
    assert f(md=3, ws=I64(2048, 3, 3, 3, 3)) == -7  # min over H: the weights of 2048 channels exceed LDS
    assert f(md=4, xs=I64(2, 3, 6, 6, 2)) == -6    # min over W of an empty output
    assert f(g=3) == -4                                                # C_out % groups
    assert f(ws=I64(2046, 1, 3, 3, 3), xs=I64(2, 3, 6, 6, 6), g=3) == -7  # grouped: weights exceed LDS
    assert f(ws=I64(2048, 3, 3, 3, 3)) == -7                             # weights exceed LDS
    assert f(xs=I64(2, 3, 2, 6, 6)) == -6
    assert f(s=I32(1, 0, 1)) == -5


def test_conv_out_shape_matches_pages():
    assert ch.out_shape([524280], [3], 3, 4, 0) == (0, [174758])
    assert ch.out_shape([24, 32, 32], [3, 3, 3], 1, 1, 0) == (0, [22, 30, 30])
    assert ch.out_shape([64, 64, 64], [3, 5, 7], 1, 1, 0) == (0, [62, 60, 58])
    assert ch.out_shape([32, 32, 32], [3, 5, 7], (1, 2, 2), (1, 1, 2), (1, 2, 3)) == (0, [32, 16, 13])
    assert ch.out_shape([8], [3], 3, 4, 0)[0] == -6


def test_plans_fit_lds_and_cover_workloads():
    import synth
    for name, cfg in synth.WORKLOADS.items():
        d = ch.plan_describe(cfg["x"], cfg["w"], cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"],
                             fused=cfg["fused"])
        fields = dict(t.split("=", 1) for t in d.split() if "=" in t)
        assert int(fields["lds"]) <= 160 * 1024, d
        gx, gy, gz = (int(v) for v in fields["grid"].split("x"))
        assert gx >= 1 and gy >= 1 and gz >= 1


def test_peak_probe_validates_before_launch():
    flop = ctypes.c_int64(0)
    L = ch.lib()
    assert L.convhip_peak_probe(2, 10, FAKE, ctypes.byref(flop), None) == -5   # unknown kind
    assert L.convhip_peak_probe(0, 0, FAKE, ctypes.byref(flop), None) == -5    # iters < 1
    assert L.convhip_peak_probe(0, (1 << 22) + 1, FAKE, ctypes.byref(flop), None) == -5  # too long a launch
    assert L.convhip_peak_probe(0, 10, None, ctypes.byref(flop), None) == -1   # no sink
    assert L.convhip_peak_probe(1, 10, FAKE, None, None) == -1                 # no flop output


def _cpu(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.float32)


@pytest.mark.parametrize("fn", ["conv_fwd", "conv_fwd_channels_last", "conv3d_min_softmax"])
@pytest.mark.parametrize("bias_shape", [(7,), (9,), (8, 1), ()])
def test_binding_rejects_bias_of_wrong_size_before_launch(fn, bias_shape):
    """The kernels read one bias value per output channel; the C ABI carries no
    bias length, so the binding rejects any bias that is not [C_out]."""
    x, w = _cpu(2, 3, 6, 6, 6), _cpu(8, 3, 3, 3, 3)
    with pytest.raises(ValueError, match="bias must be 1-D with C_out = 8"):
        getattr(ch, fn)(x, w, _cpu(*bias_shape))


@pytest.mark.parametrize("fn", ["conv_fwd", "conv_fwd_channels_last", "conv3d_min_softmax"])
def test_binding_rejects_host_tensors_before_launch(fn):
    x, w, b = _cpu(2, 3, 6, 6, 6), _cpu(8, 3, 3, 3, 3), _cpu(8)
    with pytest.raises(ValueError, match="must be on the GPU"):
        getattr(ch, fn)(x, w, b)


def test_binding_rejects_wrong_dtype_and_layout():
    import torch
    x, w = _cpu(2, 3, 6, 6, 6), _cpu(8, 3, 3, 3, 3)
    with pytest.raises(TypeError, match="bias must be float32"):
        ch.conv_fwd(x, w, torch.zeros(8, dtype=torch.float64))
    with pytest.raises(ValueError, match="w must be contiguous"):
        ch.conv_fwd(x, _cpu(8, 3, 3, 3, 6)[..., ::2])


def test_general_conv3d_kernel_choice(monkeypatch):
    """The general Conv3d geometry takes the workgroup-stream-K kernel; the
    channel-split kernels stay reachable for tests and A/B timings."""
    import synth
    cfg = synth.WORKLOADS["general_conv3d"]
    args = (cfg["x"], cfg["w"], cfg["stride"], cfg["dilation"], cfg["padding"], cfg["groups"])
    d = ch.plan_describe(*args)
    fields = dict(t.split("=", 1) for t in d.split() if "=" in t)
    assert fields["kernel"] == "conv_tap_kstream", d
    assert fields["grid"] == "256x1x1" and int(fields["lds"]) <= 160 * 1024, d
    monkeypatch.setenv("CONVHIP_SPLIT_PIPE", "1")
    assert "kernel=conv_tap_split pipe=1" in ch.plan_describe(*args)
    monkeypatch.setenv("CONVHIP_SPLIT_PIPE", "0")
    d = ch.plan_describe(*args)
    assert "kernel=conv_tap_split " in d and "pipe=1" not in d, d
    monkeypatch.delenv("CONVHIP_SPLIT_PIPE")
    # a plane of 12 tiles (16 x 12 outputs) is not the specialisation's 13
    d = ch.plan_describe((2, 16, 8, 32, 24), cfg["w"], *args[2:])
    assert "kernel=conv_tap_kstream" not in d, d


def test_unfused_steps_validation_errors():
    lib = ch.lib()
    ys = I64(2, 24, 22, 30, 30)
    assert lib.min_over_axis(FAKE, None, 2, FAKE, None) == -1
    assert lib.min_over_axis(None, ys, 2, FAKE, None) == -1
    assert lib.min_over_axis(FAKE, ys, 2, None, None) == -1
    assert lib.min_over_axis(FAKE, ys, 1, FAKE, None) == -5
    assert lib.min_over_axis(FAKE, ys, 5, FAKE, None) == -5
    assert lib.min_over_axis(FAKE, I64(2, 24, 0, 30, 30), 2, FAKE, None) == -3
    assert lib.min_over_axis(FAKE, I64(1 << 20, 1 << 10, 1 << 10, 4, 4), 2, FAKE, None) == -8
    zs = I64(2, 24, 900)
    assert lib.softmax_over_channels(FAKE, None, FAKE, None) == -1
    assert lib.softmax_over_channels(None, zs, FAKE, None) == -1
    assert lib.softmax_over_channels(FAKE, zs, None, None) == -1
    assert lib.softmax_over_channels(FAKE, I64(2, 0, 900), FAKE, None) == -3
    assert lib.softmax_over_channels(FAKE, I64(1 << 20, 1 << 12, 1 << 12), FAKE, None) == -8


def test_valu_switch_plans_the_vector_kernel(monkeypatch):
    """CONVHIP_VALU=1 routes conv_fwd and conv_fwd_channels_last to the
    vector-ALU direct kernel (8 or 16 output channels per lane); the fused op is
    unaffected."""
    monkeypatch.setenv("CONVHIP_VALU", "1")
    d = ch.plan_describe((2, 3, 16, 16, 16), (8, 3, 3, 3, 3))
    assert d.startswith("conv_valu co=8 pp=1 threads=64 pairs=9 grid=86x1"), d
    d = ch.plan_describe((4, 16, 32, 32, 32), (32, 8, 3, 5, 7), (1, 2, 2), (1, 1, 2), (1, 2, 3), 2)
    assert d.startswith("conv_valu co=16 pp=1 threads=64 pairs=1 grid=416x2"), d
    d = ch.plan_describe((16, 3, 64, 64, 64), (64, 3, 3, 5, 7))
    assert d.startswith("conv_valu co=16 pp=2 threads=256 pairs=7 grid=6743x4"), d
    with pytest.raises(ch.ConvError) as e:  # 2 x 92 x 92 x 8 x 4 B > 64 KiB of LDS, and no box fits either
        ch.plan_describe((1, 16, 4, 96, 96), (8, 16, 3, 92, 92))
    assert e.value.status == -7
    d = ch.plan_describe((2, 16, 16, 16, 3), (8, 3, 3, 3, 3), channels_last=True)
    assert d.startswith("conv_valu co=8 pp=1"), d
    assert "conv_valu" not in ch.plan_describe((128, 3, 24, 32, 32), (24, 3, 3, 3, 3), fused=True)


def test_large_kernels_plan_the_vector_fallback():
    """The matrix-core kernels cannot stage an 11^3 kernel over 16 channels; the
    vector-ALU kernel takes it (weights of one channel and depth tap in LDS)."""
    d = ch.plan_describe((2, 16, 16, 16, 16), (8, 16, 11, 11, 11))
    assert d.startswith("conv_valu co=8 pp=1"), d
    d = ch.plan_describe((1, 4, 24, 24, 24), (20, 2, 9, 9, 9), (2, 1, 1), (1, 2, 1), (3, 4, 4), 2)
    assert d.startswith("conv_valu co=16 pp=1"), d


def test_fused_stream_plans_native_groups():
    """The depth-streamed fused kernel takes the grouped workload (3 groups of 1
    input and 8 output channels) on its own specialisation; a group size that is
    not a whole number of 4-channel blocks stays on the generic fused kernel."""
    xs = (128, 3, 24, 32, 32)
    for md in (2, 3):
        d = ch.plan_describe(xs, (24, 1, 3, 3, 3), 1, 1, 0, 3, fused=True, min_dim=md)
        assert "kernel=fused_stream spec=1" in d and "groups=3" in d, d
    d = ch.plan_describe(xs, (24, 3, 3, 3, 3), fused=True)
    assert "kernel=fused_stream spec=0" in d and "groups=1" in d, d
    d = ch.plan_describe(xs, (18, 1, 3, 3, 3), 1, 1, 0, 3, fused=True)
    assert "kernel=fused_min_softmax_mfma4" in d, d


def test_large_kernels_plan_the_vector_fallback_channels_last():
    d = ch.plan_describe((2, 16, 16, 16, 16), (8, 16, 11, 11, 11), channels_last=True)
    assert d.startswith("conv_valu co=8 pp=1"), d


def test_fused_channels_last_plans():
    """The channels-last fused op (x [N, D, H, W, C]) takes the depth-streamed kernel's
    element-copy specialisation at the workload's geometry for every min axis, and the
    generic fused kernel elsewhere."""
    xs, ws = (128, 24, 32, 32, 3), (24, 3, 3, 3, 3)
    for md in (2, 3, 4):
        d = ch.plan_describe(xs, ws, fused=True, channels_last=True, min_dim=md)
        assert "kernel=fused_stream spec=2 " in d, d
    d = ch.plan_describe((128, 24, 32, 32, 3), (24, 1, 3, 3, 3), 1, 1, 0, 3, fused=True, channels_last=True)
    assert "kernel=fused_min_softmax_mfma4" in d, d
    lib = ch.lib()
    one, zero = I32(1, 1, 1), I32(0, 0, 0)
    f = lambda xs=(1, 6, 8, 8, 3), ws=(4, 3, 3, 3, 3), md=2, x=FAKE, y=FAKE: \
        lib.conv3d_min_softmax_channels_last(x, I64(*xs), FAKE, I64(*ws), None, one, one, zero, 1, md, y, None)
    assert f(x=None) == -1 and f(y=None) == -1
    assert f(md=5) == -5 and f(md=1) == -5
    assert f(xs=(1, 6, 8, 8, 4)) == -3          # C_in (last entry) does not match w
    assert f(xs=(1, 2, 8, 8, 3)) == -6          # empty output along D


def test_fused_generic_channel_chunks():
    """More than 64 output channels per group run as balanced chunks of at most 64
    (each reducing over the group's whole input); the multiply-adds issued are the
    algorithmic count times the padding of positions, chunks' channels and reduction."""
    for xs, ws, g, chunks, cpad in [((2, 3, 6, 9, 10), (96, 3, 3, 3, 3), 1, 2, 48),
                                    ((2, 3, 6, 9, 10), (150, 3, 3, 3, 3), 1, 3, 52),
                                    ((2, 4, 6, 9, 10), (160, 2, 3, 3, 3), 2, 2, 40),
                                    ((2, 3, 6, 9, 10), (64, 3, 3, 3, 3), 1, 1, 64)]:
        desc = ch.plan_describe(xs, ws, 1, 1, 0, g, fused=True)
        f = dict(t.split("=", 1) for t in desc.split() if "=" in t)
        assert f["kernel"] == "fused_min_softmax_mfma4" and int(f["chunks"]) == chunks, desc
        assert int(f["cpad"]) == cpad, desc
