"""GPU parity of the fused op's unfused steps (min_over_axis, softmax_over_channels)
against the oracle, and of the whole unfused chain against the fused kernel.

The minimum is exact, so it is compared bit for bit (NaN positions included).
Softmax in fp32: each output is exp(z - M) / sum with values in [0, 1]; expf is
within a few ulp and the C-term sum rounds at most C times, so the error is
below (C + 8) * 2^-24 absolute, the bound used here.
"""
import numpy as np
import pytest
import torch

import implicit_gemm_convolution_direct_amd as ch
import oracle
import synth
from gpu_util import FUSED_ATOL, dev, say, to_dev

pytestmark = pytest.mark.gpu


def _softmax_tol(C):
    return (C + 8) * 2.0 ** -24


MIN_CASES = [
    ((2, 5, 7, 6, 9), 2), ((2, 5, 7, 6, 9), 3), ((2, 5, 7, 6, 9), 4),      # odd inner sizes: scalar path
    ((3, 4, 6, 8, 12), 2), ((3, 4, 6, 8, 12), 3), ((3, 4, 6, 8, 12), 4),   # inner % 4 == 0: 16-byte path
    ((1, 1, 1, 1, 1), 2), ((2, 3, 1, 5, 8), 2), ((2, 3, 5, 1, 8), 3),      # unit axes
    ((1, 2, 3, 4, 2000), 4), ((5, 7, 300, 3, 4), 2),                        # long rows / long reduced axis
]


@pytest.mark.parametrize("shape,dim", MIN_CASES)
def test_min_over_axis_exact(shape, dim):
    say(f"min_over_axis {shape} dim {dim}")
    r = np.random.default_rng(1000 + dim + sum(shape))
    y = r.standard_normal(shape).astype(np.float32)
    got = ch.min_over_axis(to_dev(y), dim).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.min_axis(y, dim))


def test_min_over_axis_misaligned_input_takes_the_scalar_path():
    r = np.random.default_rng(1100)
    shape = (2, 3, 5, 4, 8)
    y = r.standard_normal(int(np.prod(shape)) + 1).astype(np.float32)
    t = to_dev(y)[1:].view(shape)
    assert t.data_ptr() % 16 != 0
    for dim in (2, 3, 4):
        got = ch.min_over_axis(t, dim).cpu().numpy()
        np.testing.assert_array_equal(got, oracle.min_axis(y[1:].reshape(shape), dim))


@pytest.mark.parametrize("dim", [2, 3, 4])
def test_min_over_axis_nan_propagates(dim):
    r = np.random.default_rng(1200 + dim)
    y = r.standard_normal((2, 4, 6, 5, 8)).astype(np.float32)
    y[0, 1, 0, 0, 0] = np.nan
    y[1, 3, 5, 4, 7] = np.nan
    y[1, 0, 2, 3, 4] = np.nan
    got = ch.min_over_axis(to_dev(y), dim).cpu().numpy()
    ref = oracle.min_axis(y, dim)
    assert np.isnan(ref).sum() == 3
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("dim", [2, 3, 4])
def test_min_over_axis_workload_shape(dim):
    """The conv output of the fused workload, [128, 24, 22, 30, 30]."""
    say(f"min_over_axis workload shape dim {dim}")
    y = np.random.default_rng(77).standard_normal((128, 24, 22, 30, 30), dtype=np.float32)
    got = ch.min_over_axis(to_dev(y), dim).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.min_axis(y, dim))


SOFTMAX_CASES = [(2, 24, 900), (3, 32, 17), (2, 33, 50), (1, 100, 7), (4, 1, 5), (2, 5, 1), (1, 64, 4097)]


@pytest.mark.parametrize("shape", SOFTMAX_CASES)
def test_softmax_over_channels(shape):
    say(f"softmax_over_channels {shape}")
    r = np.random.default_rng(1300 + sum(shape))
    z = (r.standard_normal(shape) * 5).astype(np.float32)
    got = ch.softmax_over_channels(to_dev(z)).cpu().numpy()
    ref = oracle.softmax_channels(z)
    err = float(np.abs(got - ref).max())
    say(f"  max|err| = {err:.3e}  tol = {_softmax_tol(shape[1]):.3e}")
    assert err <= _softmax_tol(shape[1])


@pytest.mark.parametrize("C", [24, 40])
def test_softmax_over_channels_nan_rows(C):
    r = np.random.default_rng(1400 + C)
    z = r.standard_normal((2, C, 6, 7)).astype(np.float32)
    z[1, C - 1, 5, 6] = np.nan
    z[0, 0, 0, 0] = np.nan
    got = ch.softmax_over_channels(to_dev(z)).cpu().numpy()
    ref = oracle.softmax_channels(z)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got).sum() == 2 * C
    ok = ~np.isnan(ref)
    assert float(np.abs(got[ok] - ref[ok]).max()) <= _softmax_tol(C)


def _chain(x, w, b, min_dim):
    y5 = ch.conv_fwd(x, w, b)
    return ch.softmax_over_channels(ch.min_over_axis(y5, min_dim))


@pytest.mark.parametrize("min_dim", [2, 3, 4])
def test_unfused_chain_matches_oracle_on_a_workload_slice(min_dim):
    """conv_fwd -> min_over_axis -> softmax_over_channels on 4 samples drawn like the
    fused workload's, against the fused oracle."""
    say(f"unfused chain slice min_dim {min_dim}")
    x, w, b = synth.make_inputs("conv3d_min_softmax", n_samples=4)
    got = _chain(to_dev(x), to_dev(w), to_dev(b), min_dim).cpu().numpy()
    ref = oracle.conv3d_min_softmax(x, w, b, 1, 1, 0, 1, min_dim)
    err = float(np.abs(got - ref).max())
    say(f"  max|err| = {err:.3e}")
    assert err <= FUSED_ATOL


def test_unfused_chain_matches_the_fused_kernel_on_the_workload():
    x, w, b = synth.make_inputs("conv3d_min_softmax")
    xd, wd, bd = to_dev(x), to_dev(w), to_dev(b)
    got = _chain(xd, wd, bd, 2)
    fused = ch.conv3d_min_softmax(xd, wd, bd)
    torch.cuda.synchronize()
    err = float((got - fused).abs().max())
    say(f"  unfused vs fused max|diff| = {err:.3e}")
    assert err <= FUSED_ATOL
