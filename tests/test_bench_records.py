"""The committed counter summaries that bench.py attaches to its roofline objects (CPU only).

bench.py reports HBM traffic and MFMA busy fractions only when the counters were taken on the
current attention kernel source; these tests check that rule and the internal consistency of
the stored MFMA figures (busy fraction x clock against the counted MFMA work and duration).
"""
import json
import os

import pytest

import bench

KERNELS = ["attn_fwd_kernel<128>, sparse 720p layer", "attn_fwd_kernel<128>, dense 720p",
           "cluster_attn_kernel<128>, 720p clustering layer", "block_attn_kernel<128>, 720p block-sparse layer",
           "block_mass_kernel<128>, 720p search"]


def _mfma():
    with open(bench.MFMA_FILE) as fh:
        return json.load(fh)


def test_mfma_record_is_self_consistent():
    t = _mfma()
    for name in KERNELS:
        k = t["kernels"][name]
        assert 0.0 < k["mfma_busy"] < 1.0, name
        assert 1.0 < k["clock_ghz"] < 2.6, name
        # FLOP/s counted by the hardware against the MFMA pipes' rate at the measured clock
        counted_rate = k["counted_tflop"] * 1e12 / (k["us"] * 1e-6)
        pipe_rate = bench.PEAK_BF16_TFLOPS * 1e12 * k["clock_ghz"] / 2.4
        assert abs(counted_rate / pipe_rate - k["mfma_busy"]) < 0.05 * k["mfma_busy"], name
        # the counted work covers the computed tiles, plus at most a few percent of pipeline ends
        assert 1.0 <= k["counted_tflop"] / k["computed_tile_tflop"] < 1.05, name


def test_mfma_loader_follows_the_kernel_source(monkeypatch):
    t = _mfma()
    if t["kernel_sha"] != bench.kernel_sha():
        assert bench.measured_mfma(KERNELS[0]) == {}
        return
    got = bench.measured_mfma(KERNELS[0])
    assert got["mfma_busy"] == round(t["kernels"][KERNELS[0]]["mfma_busy"], 3)
    assert bench.measured_mfma("no such kernel") == {}
    monkeypatch.setattr(bench, "kernel_sha", lambda: "0" * 16)
    assert bench.measured_mfma(KERNELS[0]) == {}


@pytest.mark.parametrize("path", [bench.TRAFFIC_FILE, bench.CLUSTER_TRAFFIC_FILE, bench.BLOCK_TRAFFIC_FILE])
def test_traffic_loader_follows_the_kernel_source(monkeypatch, path):
    assert os.path.exists(path)
    with open(path) as fh:
        t = json.load(fh)
    if t["kernel_sha"] == bench.kernel_sha():
        assert bench.measured_traffic(path) == t["bytes_per_launch"] > 0
    monkeypatch.setattr(bench, "kernel_sha", lambda: "0" * 16)
    assert bench.measured_traffic(path) is None
