"""Host logic of bench.py (CPU only): the work it credits each workload with,
its entry names and roofline objects, the committed traffic summaries it reads,
and the one-GPU guard. The MAC counts are checked against the sizes the pages
print and against a count written out from the output shapes."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _macs(name):
    return bench.geometry(synth.config(name))[1]


def test_mac_counts_match_the_pages_sizes():
    # long Conv1d: 64 x 128 outputs channels x 174758 positions x 64 x 3 taps (page l1_p76, opening turn)
    assert _macs("long_conv1d") == 64 * 128 * 174758 * 64 * 3 == 274_870_566_912
    # fused op: [128, 24, 22, 30, 30] conv outputs x 81 (page l2_p24, opening turn)
    assert _macs("conv3d_min_softmax") == 128 * 24 * 22 * 30 * 30 * 81 == 4_926_873_600
    # asymmetric Conv3d: 220,938,240 outputs x 3 x 3 x 5 x 7 (page l1_p60, opening turn; recomputed size)
    assert _macs("asym_conv3d") == 220_938_240 * 315


def test_grouped_mac_counts_have_no_cross_group_products():
    dense = _macs("conv3d_min_softmax")
    assert _macs("conv3d_min_softmax_groups3") * 3 == dense
    out, macs, nbytes, conv_elems, y_elems = bench.geometry(synth.config("general_conv3d"))
    assert out == [32, 16, 13]
    assert macs == 4 * 32 * 32 * 16 * 13 * 8 * 105
    assert nbytes == 4 * (4 * 16 * 32 ** 3 + 32 * 8 * 105 + 32 + conv_elems)


def test_fused_output_bytes_drop_the_min_axis():
    for name, keep in (("conv3d_min_softmax", (30, 30)), ("conv3d_min_softmax_min_h", (22, 30)),
                       ("conv3d_min_softmax_min_w", (22, 30))):
        _, _, _, conv_elems, y_elems = bench.geometry(synth.config(name))
        assert y_elems == 128 * 24 * int(np.prod(keep))
        assert conv_elems == 128 * 24 * 22 * 30 * 30


def test_entry_names_round_trip():
    assert bench.ORDER[0] != "" and len(set(bench.ORDER)) == len(bench.ORDER)
    for name in bench.ORDER:
        base, cl, mode = bench.split_name(name)
        synth.config(base)  # every entry names a workload or a variant
        assert mode in (None, "generic", "valu")
        rebuilt = base + (bench.CL_SUFFIX if cl else "") + \
            {None: "", "generic": bench.GEN_SUFFIX, "valu": bench.VALU_SUFFIX}[mode]
        assert rebuilt == name


def test_roofline_objects():
    r = bench.roofline(78.65, "general_conv3d")
    assert r["bound"] == "mfma" and r["peak"] == 157.3 and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(0.5, abs=1e-4)
    assert bench.roofline(10.0, "asym_conv3d_valu")["bound"] == "alu"
    assert bench.roofline(0.9, "tiny_conv3d", latency_bound=True)["limited_by"] == "launch latency"


def test_traffic_is_read_only_for_the_current_sources(tmp_path, monkeypatch):
    """The committed summaries carry the kernel-source hash they were taken on:
    a matching one is read, a stale one gives null."""
    v = bench.read_traffic("long_conv1d")
    if v is not None:
        assert 1.4e10 < v < 1.5e10  # about 14.3 GB of algorithmic traffic per launch, measured 1.01x
    fake = tmp_path / "profiles"
    fake.mkdir()
    (fake / "traffic_x.txt").write_text("kernel_src_sha256_16 = 0000000000000000\nhbm_bytes_per_launch = 5\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("x") is None
    (fake / "traffic_y.txt").write_text(f"kernel_src_sha256_16 = {bench.kernel_source_hash()}\n"
                                        "hbm_bytes_per_launch = 5\n")
    assert bench.read_traffic("y") == 5.0


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
