"""Pins of the fp64 oracle to facts other than itself (CPU only).

Each test fixes something the pages or the mathematics determine: values the
pages print (tests/golden), brute force on tiny inputs (oracle/brute.py, an
independent pure-Python reading of the definition), a library routine the
definition reduces to (torch's float64 CPU convolution), closed forms and
invariants (delta kernel, linearity, bias additivity, group decomposition,
dilation / stride equivalences, 1-D = 3-D with unit axes, the exactly-once
input use of the stride-3 dilation-4 Conv1d, softmax rows summing to one,
the logistic form of a two-channel softmax, numpy's and torch's minima).
A dropped term, a flipped sign or index, a transposed operand or a wrong
padding offset in oracle.c fails at least the brute-force and delta tests.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- output length
def test_output_lengths_match_pages():
    rows = _golden_rows("output_lengths.txt")
    assert len(rows) >= 6
    for L, k, s, d, p, expect, _src in rows:
        assert oracle.out_len(int(L), int(k), int(s), int(d), int(p)) == int(expect)
        assert brute.out_len(int(L), int(k), int(s), int(d), int(p)) == int(expect)


def test_output_length_floor_semantics_and_empty_edge():
    # L = d(k-1) leaves no valid window: floor((d(k-1) - d(k-1) - 1)/s) + 1 = floor(-1/s) + 1 = 0.
    for k, d, s in [(3, 1, 1), (3, 4, 3), (5, 2, 2), (7, 2, 4)]:
        assert oracle.out_len(d * (k - 1), k, s, d, 0) == 0
        assert oracle.out_len(d * (k - 1) + 1, k, s, d, 0) == 1
    # C-style truncation would give 1 here; floor gives 0 (numerator -1, stride 3).
    assert oracle.out_len(8, 3, 3, 4, 0) == 0
    # Exhaustive check against the count of valid window starts.
    for L, k, s, d, p in itertools.product(range(1, 13), range(1, 5), range(1, 4), range(1, 4), range(0, 3)):
        count = sum(1 for o in range(0, 64) if o * s + (k - 1) * d <= L + 2 * p - 1)
        assert max(oracle.out_len(L, k, s, d, p), 0) == count


def test_problem_sizes_match_pages():
    vals = {r[0]: int(r[1]) for r in _golden_rows("problem_sizes.txt")}
    out = [oracle.out_len(n, 3) for n in (24, 32, 32)]
    assert 128 * 24 * out[0] * out[1] * out[2] == vals["conv3d_min_softmax.conv_out_elems"]
    assert 3 * 27 == vals["conv3d_min_softmax.mac_per_output"]
    assert 128 * 24 * out[1] * out[2] == vals["conv3d_min_softmax.min_out_elems"]
    assert 128 * out[1] * out[2] == vals["conv3d_min_softmax.softmax_rows"]
    assert 64 * 128 * oracle.out_len(524280, 3, 3, 4, 0) == vals["long_conv1d.out_elems"]
    assert 64 * 3 == vals["long_conv1d.mac_per_output"]
    assert 3 * 3 * 5 * 7 == vals["asym_conv3d.mac_per_output"]
    J = 64
    used = {3 * j + 4 * t for j in range(J) for t in range(3)}
    span = 3 * (J - 1) + 4 * 2 + 1
    assert span == vals["long_conv1d.slice_len_J64"]
    assert span - len(used) == vals["long_conv1d.unused_in_slice"]


# ---------------------------------------------------------------- brute force
def _random_case(r, nd):
    groups = int(r.choice([1, 1, 2, 3]))
    cg = int(r.integers(1, 3))
    cout_g = int(r.integers(1, 3))
    N = int(r.integers(1, 3))
    ks = [int(r.integers(1, 4)) for _ in range(nd)]
    s = [int(r.integers(1, 4)) for _ in range(nd)]
    d = [int(r.integers(1, 4)) for _ in range(nd)]
    p = [int(r.integers(0, 4)) for _ in range(nd)]
    Ls = []
    for a in range(nd):
        lo = max(1, d[a] * (ks[a] - 1) + 1 - 2 * p[a])
        Ls.append(int(r.integers(lo, lo + {1: 7, 2: 5, 3: 4}[nd])))
    x = r.standard_normal((N, groups * cg, *Ls)).astype(np.float32)
    w = r.standard_normal((groups * cout_g, cg, *ks)).astype(np.float32)
    b = r.standard_normal(groups * cout_g).astype(np.float32) if r.random() < 0.5 else None
    return x, w, b, s, d, p, groups


@pytest.mark.parametrize("nd", [1, 2, 3])
def test_oracle_matches_brute_force(nd):
    r = _rng(100 + nd)
    ncases = 150 if nd == 1 else 60
    for _ in range(ncases):
        x, w, b, s, d, p, g = _random_case(r, nd)
        yo = oracle.conv(x, w, b, s, d, p, g)
        yb = brute.conv(x, w, b, s, d, p, g)
        assert yo.shape == yb.shape
        np.testing.assert_allclose(yo, yb, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("nd", [1, 2, 3])
def test_channels_last_oracle_matches_brute_force(nd):
    """The channels-last oracle against a brute force that indexes x[n, pos..., c]
    directly (a swapped axis or a wrong channel offset fails here)."""
    r = _rng(300 + nd)
    for _ in range(40 if nd == 1 else 20):
        x, w, b, s, d, p, g = _random_case(r, nd)
        x_cl = np.ascontiguousarray(np.moveaxis(x, 1, -1))
        yo = oracle.conv_channels_last(x_cl, w, b, s, d, p, g)
        yb = brute.conv_channels_last(x_cl, w, b, s, d, p, g)
        assert yo.shape == yb.shape == (x.shape[0], *yo.shape[1:-1], w.shape[0])
        np.testing.assert_allclose(yo, yb, rtol=1e-12, atol=1e-12)


def test_channels_last_brute_force_against_torch_channels_last_3d():
    """torch's Conv3d on a channels_last_3d tensor (memory order N, D, H, W, C)."""
    r = _rng(310)
    for _ in range(6):
        x, w, b, s, d, p, g = _random_case(r, 3)
        xt = torch.from_numpy(x).double().contiguous(memory_format=torch.channels_last_3d)
        yt = F.conv3d(xt, torch.from_numpy(w).double(), None if b is None else torch.from_numpy(b).double(),
                      stride=s, padding=p, dilation=d, groups=g)
        yb = brute.conv_channels_last(np.moveaxis(x, 1, -1), w, b, s, d, p, g)
        np.testing.assert_allclose(yb, yt.permute(0, 2, 3, 4, 1).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("nd", [1, 2, 3])
def test_oracle_matches_torch_float64(nd):
    """The definition is what torch's float64 CPU convolution computes."""
    r = _rng(200 + nd)
    conv = {1: F.conv1d, 2: F.conv2d, 3: F.conv3d}[nd]
    for _ in range(25):
        x, w, b, s, d, p, g = _random_case(r, nd)
        yo = oracle.conv(x, w, b, s, d, p, g)
        yt = conv(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                  None if b is None else torch.from_numpy(b).double(),
                  stride=s, padding=p, dilation=d, groups=g).numpy()
        np.testing.assert_allclose(yo, yt, rtol=1e-12, atol=1e-12)


def test_oracle_matches_torch_on_workload_shapes_reduced():
    """The general-parameter Conv3d's parameters (groups 2, stride (1,2,2), padding (1,2,3),
    dilation (1,1,2)) on one sample of reduced spatial size."""
    r = _rng(7)
    x = r.random((1, 16, 9, 12, 14), dtype=np.float32)
    w = (r.random((32, 8, 3, 5, 7), dtype=np.float32) - 0.5)
    b = r.random(32, dtype=np.float32)
    yo = oracle.conv(x, w, b, (1, 2, 2), (1, 1, 2), (1, 2, 3), 2)
    yt = F.conv3d(torch.from_numpy(x).double(), torch.from_numpy(w).double(), torch.from_numpy(b).double(),
                  stride=(1, 2, 2), padding=(1, 2, 3), dilation=(1, 1, 2), groups=2).numpy()
    np.testing.assert_allclose(yo, yt, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_delta_kernel_is_shifted_strided_copy():
    """w = delta at tap t0 of input channel c0: y = x~[g*C_g + c0, o*s + t0*d - p], zero outside."""
    r = _rng(11)
    x = r.standard_normal((2, 4, 7, 8, 9)).astype(np.float32)
    ks, s, d, p, g = (2, 3, 3), (1, 2, 3), (2, 1, 2), (1, 2, 3), 2
    cg = 2
    for c0 in range(cg):
        for t0 in itertools.product(*[range(k) for k in ks]):
            w = np.zeros((4, cg, *ks), dtype=np.float32)
            w[:, c0][(slice(None),) + t0] = 1.0
            y = oracle.conv(x, w, None, s, d, p, g)
            for n, co in itertools.product(range(2), range(4)):
                gi = co // 2
                ci = gi * cg + c0
                for o in itertools.product(*[range(v) for v in y.shape[2:]]):
                    pos = [o[a] * s[a] + t0[a] * d[a] - p[a] for a in range(3)]
                    inside = all(0 <= pos[a] < x.shape[2 + a] for a in range(3))
                    expect = float(x[(n, ci) + tuple(pos)]) if inside else 0.0
                    assert y[(n, co) + o] == expect


def test_all_ones_counts_in_bounds_taps():
    """x = 1, w = 1: each output equals C_g times the number of taps that land inside."""
    x = np.ones((1, 6, 5, 6, 7), dtype=np.float32)
    w = np.ones((4, 3, 3, 2, 3), dtype=np.float32)
    s, d, p = (2, 1, 3), (1, 3, 2), (2, 1, 3)
    y = oracle.conv(x, w, None, s, d, p, 2)
    for o in itertools.product(*[range(v) for v in y.shape[2:]]):
        cnt = 1
        for a in range(3):
            cnt *= sum(1 for t in range(w.shape[2 + a]) if 0 <= o[a] * s[a] + t * d[a] - p[a] < x.shape[2 + a])
        assert np.all(y[(0, slice(None)) + o] == 3 * cnt)


def test_linearity_and_bias_additivity():
    """Inputs are small dyadic rationals (k/8), so every sum below is exact in fp32 and fp64."""
    r = _rng(12)
    q = lambda shape: (r.integers(-8, 9, size=shape) / 8.0).astype(np.float32)
    x1, x2 = q((2, 4, 6, 7, 8)), q((2, 4, 6, 7, 8))
    w1, w2 = q((6, 2, 3, 2, 3)), q((6, 2, 3, 2, 3))
    b = q((6,))
    args = ((1, 2, 1), (1, 1, 2), (1, 0, 2), 2)
    y11 = oracle.conv(x1, w1, None, *args)
    np.testing.assert_array_equal(oracle.conv(x1 + x2, w1, None, *args), y11 + oracle.conv(x2, w1, None, *args))
    np.testing.assert_array_equal(oracle.conv(x1, w1 + w2, None, *args), y11 + oracle.conv(x1, w2, None, *args))
    np.testing.assert_array_equal(oracle.conv(-3 * x1, w1, None, *args), -3 * y11)
    yb = oracle.conv(x1, w1, b, *args)
    np.testing.assert_array_equal(yb - y11, np.broadcast_to(b.astype(np.float64)[None, :, None, None, None], y11.shape))


def test_group_decomposition():
    r = _rng(13)
    g, cg, cog = 3, 2, 2
    x = r.standard_normal((2, g * cg, 5, 6, 7)).astype(np.float32)
    w = r.standard_normal((g * cog, cg, 2, 3, 2)).astype(np.float32)
    b = r.standard_normal(g * cog).astype(np.float32)
    y = oracle.conv(x, w, b, (1, 2, 1), (2, 1, 1), (1, 1, 0), g)
    parts = [oracle.conv(x[:, i * cg:(i + 1) * cg], w[i * cog:(i + 1) * cog], b[i * cog:(i + 1) * cog],
                         (1, 2, 1), (2, 1, 1), (1, 1, 0), 1) for i in range(g)]
    np.testing.assert_array_equal(y, np.concatenate(parts, axis=1))


def test_dilation_equals_zero_stuffed_kernel():
    r = _rng(14)
    x = r.standard_normal((1, 3, 9, 10, 11)).astype(np.float32)
    w = r.standard_normal((4, 3, 2, 3, 2)).astype(np.float32)
    d = (2, 3, 2)
    ws = np.zeros((4, 3, *[d[a] * (w.shape[2 + a] - 1) + 1 for a in range(3)]), dtype=np.float32)
    ws[:, :, ::d[0], ::d[1], ::d[2]] = w
    np.testing.assert_array_equal(oracle.conv(x, w, None, (1, 2, 1), d, (1, 2, 0), 1),
                                  oracle.conv(x, ws, None, (1, 2, 1), (1, 1, 1), (1, 2, 0), 1))


def test_stride_equals_subsampled_stride_one():
    r = _rng(15)
    x = r.standard_normal((2, 2, 9, 8, 10)).astype(np.float32)
    w = r.standard_normal((3, 2, 3, 2, 3)).astype(np.float32)
    s = (2, 3, 2)
    y1 = oracle.conv(x, w, None, 1, (1, 2, 1), (1, 0, 2), 1)
    ys = oracle.conv(x, w, None, s, (1, 2, 1), (1, 0, 2), 1)
    np.testing.assert_array_equal(ys, y1[:, :, ::s[0], ::s[1], ::s[2]])


def test_conv1d_equals_conv3d_with_unit_axes():
    r = _rng(16)
    x = r.standard_normal((2, 6, 40)).astype(np.float32)
    w = r.standard_normal((4, 3, 3)).astype(np.float32)
    b = r.standard_normal(4).astype(np.float32)
    y1 = oracle.conv(x, w, b, 3, 4, 2, 2)
    y3 = oracle.conv(x[:, :, None, None, :], w[:, :, None, None, :], b, (1, 1, 3), (1, 1, 4), (0, 0, 2), 2)
    np.testing.assert_array_equal(y1, y3[:, :, 0, 0, :])


def test_exactly_once_input_use_stride3_dilation4():
    """For k=3, s=3, d=4 each input index l with 8 <= l <= 3(L_out-1) feeds exactly one (j, t):
    a one-hot input gives exactly one nonzero output per channel, equal to the matching weight."""
    L = 61
    Lout = oracle.out_len(L, 3, 3, 4, 0)
    w = np.arange(1, 1 + 2 * 1 * 3, dtype=np.float32).reshape(2, 1, 3)
    for l in range(L):
        x = np.zeros((1, 1, L), dtype=np.float32)
        x[0, 0, l] = 1.0
        y = oracle.conv(x, w, None, 3, 4, 0, 1)
        nz = np.argwhere(y[0] != 0)
        hits = [(j, t) for j in range(Lout) for t in range(3) if 3 * j + 4 * t == l]
        assert len(nz) == 2 * len(hits)
        if 8 <= l <= 3 * (Lout - 1):
            assert len(hits) == 1
            j, t = hits[0]
            assert y[0, 0, j] == w[0, 0, t] and y[0, 1, j] == w[1, 0, t]


# ---------------------------------------------------------------- fused op
def _fused_case(r, N=2, C_in=3, C_out=5, D=6, H=5, W=6, k=(3, 2, 3)):
    x = r.standard_normal((N, C_in, D, H, W)).astype(np.float32)
    w = r.standard_normal((C_out, C_in, *k)).astype(np.float32) * 0.5
    b = r.standard_normal(C_out).astype(np.float32)
    return x, w, b


@pytest.mark.parametrize("min_dim", [2, 3, 4])
def test_fused_matches_brute_force(min_dim):
    r = _rng(20 + min_dim)
    x, w, b = _fused_case(r)
    s, d, p = (1, 2, 1), (1, 1, 2), (0, 1, 1)
    yo = oracle.conv3d_min_softmax(x, w, b, s, d, p, 1, min_dim)
    yb = brute.conv3d_min_softmax(x, w, b, s, d, p, 1, min_dim)
    np.testing.assert_allclose(yo, yb, rtol=1e-12, atol=1e-14)


def test_fused_matches_torch_composition():
    r = _rng(30)
    x, w, b = _fused_case(r, N=3, C_in=3, C_out=24, D=8, H=7, W=9, k=(3, 3, 3))
    yo = oracle.conv3d_min_softmax(x, w, b)
    t = F.conv3d(torch.from_numpy(x).double(), torch.from_numpy(w).double(), torch.from_numpy(b).double())
    t = torch.softmax(torch.min(t, dim=2)[0], dim=1).numpy()
    np.testing.assert_allclose(yo, t, rtol=1e-12, atol=1e-15)


def test_fused_rows_sum_to_one_and_shift_invariance():
    r = _rng(31)
    x, w, b = _fused_case(r, C_out=24)
    b = (np.round(b * 1024) / 1024).astype(np.float32)  # so that b + 4 is exact in fp32
    y = oracle.conv3d_min_softmax(x, w, b)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(y > 0)
    # a constant added to every channel's bias moves every min by the same amount (exact power of 2)
    y2 = oracle.conv3d_min_softmax(x, w, b + np.float32(4.0))
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-15)


def test_fused_equal_channels_give_uniform_softmax():
    r = _rng(32)
    x, w, _ = _fused_case(r, C_out=1)
    w = np.repeat(w, 6, axis=0)
    y = oracle.conv3d_min_softmax(x, w, np.zeros(6, dtype=np.float32))
    np.testing.assert_allclose(y, 1.0 / 6.0, rtol=1e-14)


def test_fused_min_is_over_depth_of_conv_with_bias():
    """Softmax is invertible up to a per-row constant: log(out) - log(out[:, :1]) recovers
    m - m[channel 0], where m is the depth-min of the biased conv."""
    r = _rng(33)
    x, w, b = _fused_case(r, C_out=4)
    y = oracle.conv3d_min_softmax(x, w, b)
    m = oracle.conv(x, w, b).min(axis=2)
    np.testing.assert_allclose(np.log(y) - np.log(y[:, :1]), m - m[:, :1], rtol=0, atol=1e-10)


def test_integer_inputs_give_exact_integer_outputs():
    """Integer-valued inputs (the exact-arithmetic distribution) yield integer outputs: the
    fp64 sums carry no rounding, so a GPU fp32 result can be compared bit for bit."""
    x, w, b = synth.make_inputs("tiny_conv3d", integer=True)
    y = oracle.conv(x, w, b)
    assert np.all(y == np.round(y))
    assert np.abs(y).max() < 2 ** 24


def test_fused_nan_propagates_like_torch_min():
    """A NaN in the input reaches every conv output whose window covers it; the
    minimum along the axis is then NaN (torch.min propagates NaN) and so is the
    whole softmax row. The oracle must agree with torch's composition on where
    the NaNs are and match it elsewhere."""
    r = _rng(34)
    x, w, b = _fused_case(r, N=2, C_in=2, C_out=5, D=6, H=7, W=8, k=(3, 3, 3))
    x[1, 0, 4, 2, 3] = np.nan
    for min_dim in (2, 3, 4):
        yo = oracle.conv3d_min_softmax(x, w, b, 1, 1, 0, 1, min_dim)
        t = F.conv3d(torch.from_numpy(x).double(), torch.from_numpy(w).double(), torch.from_numpy(b).double())
        t = torch.softmax(torch.min(t, dim=min_dim)[0], dim=1).numpy()
        assert np.isnan(t).any() and not np.isnan(t).all()
        np.testing.assert_array_equal(np.isnan(yo), np.isnan(t))
        ok = ~np.isnan(t)
        np.testing.assert_allclose(yo[ok], t[ok], rtol=1e-12, atol=1e-15)


# ------------------------------------------------ the unfused steps on their own
@pytest.mark.parametrize("dim", [2, 3, 4])
def test_min_axis_matches_numpy_and_brute_force(dim):
    """numpy's reduction (a library routine) on a ragged shape, and a pure-Python
    scan of the axis on a tiny one; both are exact, so equality is bitwise."""
    r = _rng(40 + dim)
    y = r.standard_normal((3, 5, 7, 6, 9)).astype(np.float32)
    np.testing.assert_array_equal(oracle.min_axis(y, dim), y.min(axis=dim))
    t = r.standard_normal((2, 2, 3, 2, 4)).astype(np.float32)
    got = oracle.min_axis(t, dim)
    for idx in itertools.product(*[range(v) for a, v in enumerate(t.shape) if a != dim]):
        vals = [float(t[idx[:dim] + (j,) + idx[dim:]]) for j in range(t.shape[dim])]
        assert got[idx] == min(vals)


def test_min_axis_nan_and_unit_axis():
    """A NaN anywhere along the axis gives NaN (numpy and torch.min both propagate
    it; np.fmin would drop it); an axis of length 1 is the identity."""
    r = _rng(44)
    y = r.standard_normal((2, 3, 4, 5, 6)).astype(np.float32)
    y[1, 2, 3, 0, 5] = np.nan
    y[0, 0, 0, 4, 1] = np.nan
    for dim in (2, 3, 4):
        got = oracle.min_axis(y, dim)
        ref = torch.min(torch.from_numpy(y), dim=dim)[0].numpy()
        np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
        assert np.isnan(got).sum() == 2
        np.testing.assert_array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    u = r.standard_normal((2, 3, 1, 4, 5)).astype(np.float32)
    np.testing.assert_array_equal(oracle.min_axis(u, 2), u[:, :, 0])


def test_softmax_channels_closed_forms():
    """Two channels give the logistic function of their difference; equal channels
    give 1/C; adding a constant to every channel changes nothing; rows sum to 1."""
    r = _rng(45)
    a = r.standard_normal((3, 1, 11)).astype(np.float32) * 4
    b = r.standard_normal((3, 1, 11)).astype(np.float32) * 4
    s = oracle.softmax_channels(np.concatenate([a, b], axis=1))
    np.testing.assert_allclose(s[:, 0], 1.0 / (1.0 + np.exp(b[:, 0].astype(np.float64) - a[:, 0])),
                               rtol=1e-14, atol=1e-300)
    e = np.repeat(a, 7, axis=1)
    np.testing.assert_allclose(oracle.softmax_channels(e), 1.0 / 7.0, rtol=1e-14)
    z = (np.round(r.standard_normal((2, 24, 5, 6)) * 1024) / 1024).astype(np.float32)  # z + 8 exact in fp32
    s = oracle.softmax_channels(z)
    assert s.shape == z.shape
    np.testing.assert_allclose(s.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.softmax_channels(z + np.float32(8.0)), s, rtol=1e-12, atol=1e-15)


def test_softmax_channels_matches_torch_float64_and_nan_rows():
    r = _rng(46)
    z = (r.standard_normal((3, 40, 7, 5)) * 6).astype(np.float32)
    z[2, 17, 3, 1] = np.nan
    got = oracle.softmax_channels(z)
    ref = torch.softmax(torch.from_numpy(z).double(), dim=1).numpy()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got).sum() == 40
    ok = ~np.isnan(ref)
    np.testing.assert_allclose(got[ok], ref[ok], rtol=1e-12, atol=1e-300)


def test_unfused_steps_compose_to_the_fused_oracle():
    """softmax_channels(min_axis(conv)) is the fused op; the only difference is the
    fp32 rounding of the conv output before the minimum (the unfused chain stores
    it in fp32), so the two agree to fp32 rounding of the logits."""
    r = _rng(47)
    x, w, b = _fused_case(r, N=2, C_in=3, C_out=24, D=7, H=6, W=8, k=(3, 3, 3))
    for min_dim in (2, 3, 4):
        y = oracle.conv(x, w, b).astype(np.float32)
        got = oracle.softmax_channels(oracle.min_axis(y, min_dim))
        ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, 0, 1, min_dim)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-6)


def test_fused_channels_last_oracle_matches_torch_on_moved_axes():
    """The channels-last fused oracle: x stored [N, D, H, W, C], y [N, kept, C];
    torch's float64 composition on the logical (permuted) tensor, for each min axis."""
    r = _rng(48)
    x_cl = r.standard_normal((2, 6, 5, 7, 3)).astype(np.float32)
    w = (r.standard_normal((8, 3, 3, 2, 3)) * 0.5).astype(np.float32)
    b = r.standard_normal(8).astype(np.float32)
    xt = torch.from_numpy(x_cl).double().permute(0, 4, 1, 2, 3)
    for md in (2, 3, 4):
        got = oracle.conv3d_min_softmax_channels_last(x_cl, w, b, 1, 1, (1, 0, 1), 1, md)
        t = F.conv3d(xt, torch.from_numpy(w).double(), torch.from_numpy(b).double(), padding=(1, 0, 1))
        t = torch.softmax(torch.min(t, dim=md)[0], dim=1).permute(0, 2, 3, 1).numpy()
        np.testing.assert_allclose(got, t, rtol=1e-12, atol=1e-15)
