"""The rocprofv3 harness (rocprof_report.py) and the counter figures bench.py attaches (CPU only).

tests/data/rocprof holds the CSV output of one `rocprof_report.py collect` run on an MI355X,
trimmed by `rocprof_report.py fixture` to the library's kernels and the calibration copy.  The
committed JSON summaries under profiles/ were reduced from that run, so reducing the fixture
must give them back figure for figure.
"""
import json
import os

import pytest

import bench
import rocprof_report as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIXTURE = os.path.join(ROOT, "tests", "data", "rocprof")
PROFILES = os.path.join(ROOT, "profiles")
JSONS = ["attn_fwd_hunyuan720p_traffic.json", "hbm_kernels_hunyuan720p_traffic.json",
         "cluster_attn_hunyuan720p_svg2_traffic.json", "block_attn_hunyuan720p_blocks_traffic.json",
         "mfma_busy_hunyuan720p.json"]


@pytest.fixture(scope="module")
def reduced(tmp_path_factory):
    out = tmp_path_factory.mktemp("reduced")
    names = R.reduce_all(FIXTURE, str(out))
    return str(out), names


def _load(d, n):
    with open(os.path.join(d, n)) as fh:
        return json.load(fh)


def _strip_sha(t):
    return {k: v for k, v in t.items() if not k.endswith("_sha")}


@pytest.mark.parametrize("name", JSONS)
def test_fixture_reproduces_committed_summaries(reduced, name):
    out, names = reduced
    assert name in names
    got, want = _load(out, name), _load(PROFILES, name)
    # the source hashes are those of the tree that reduces; the figures must be identical
    assert _strip_sha(got) == _strip_sha(want)


def test_every_summary_names_its_commands(reduced):
    out, names = reduced
    for n in names:
        if n.endswith(".md"):
            text = open(os.path.join(out, n)).read()
            assert "rocprofv3 " in text and "$R/bench.py" in text, n
            assert open(os.path.join(PROFILES, n)).read().split("\n")[0] == text.split("\n")[0], n


def test_calibration_and_units():
    cal = R.copy_scale(FIXTURE)
    # a 1 GiB copy writes 1 GiB: WRITE_SIZE counts KiB one to one; FETCH_SIZE counts half
    assert abs(cal["write"]["scale"] - 1.0) < 1e-3 and abs(cal["fetch"]["scale"] - 2.0) < 1e-2
    t = R.traffic(FIXTURE, "qknorm_rope_kernel", "layer", cal)
    # norm/RoPE moves exactly its algorithmic bytes: Q and K read and written once
    assert abs(t["bytes_per_launch"] / R.HBM_KERNELS["qknorm_rope"][2] - 1.0) < 0.01


def test_attention_dispatch_split():
    trace = R.find_csv(FIXTURE, "trace_layer", "kernel_trace")
    d = R.dispatches(trace, "attn_fwd_kernel")
    sparse, dense = R.sparse_ids([x[0] for x in d], "attn_fwd_kernel"), [x[0] for x in d][-R.DENSE_TAIL:]
    us = {x[0]: x[2] for x in d}
    # the dense comparison launches are an order of magnitude longer than every sparse one
    assert min(us[i] for i in dense) > 8 * max(us[i] for i in sparse)
    st = R.reduce_trace(trace, timed_steps=4)
    assert st["attn_fwd_kernel<128> sparse, the 4 timed steps"]["dispatches"] == 4


def test_mfma_record_is_self_consistent():
    t = _load(PROFILES, "mfma_busy_hunyuan720p.json")
    for name, k in t["kernels"].items():
        assert 0.0 < k["mfma_busy"] < 1.0, name
        assert 1.0 < k["clock_ghz"] < 2.6, name
        # FLOP/s counted by the hardware against the matrix pipes' rate at the measured clock
        rate = k["counted_tflop_per_launch"] * 1e12 / (k["mean_us"] * 1e-6)
        pipe = bench.PEAK_BF16_TFLOPS * 1e12 * k["clock_ghz"] / 2.4
        if name not in ("kmeans_assign",):   # short launches: ramp-up dominates
            assert abs(rate / pipe - k["mfma_busy"]) < 0.05 * k["mfma_busy"], name


def test_short_names():
    assert R.short_name("void svg::(anonymous namespace)::attn_fwd_kernel<128>(svg::AttnArgs, int)") == \
        "attn_fwd_kernel<128>"
    assert R.short_name("svg::(anonymous namespace)::block_mask_kernel(svg::BlockMaskArgs)") == "block_mask_kernel"
    assert R.short_name("void svg::(anonymous namespace)::profile_partial_kernel<128, 1>(svg::ProfileArgs)") == \
        "profile_partial_kernel<128, 1>"


def test_bench_loaders_follow_the_kernel_source(monkeypatch):
    t = _load(PROFILES, "attn_fwd_hunyuan720p_traffic.json")
    if t["kernel_sha"] == bench.kernel_sha():
        assert bench.measured_traffic() == t["bytes_per_launch"] > 0
        assert bench.measured_mfma("attn_fwd sparse")["mfma_busy"] > 0
    h = _load(PROFILES, "hbm_kernels_hunyuan720p_traffic.json")
    if h["kernel_sha"] == bench.kernel_sha("hbm"):
        assert set(bench.measured_hbm_traffic()) == {"qknorm_rope", "profile_partial", "permute_rows"}
    monkeypatch.setattr(bench, "kernel_sha", lambda group="attn_fwd": "0" * 16)
    assert bench.measured_traffic() is None and bench.measured_hbm_traffic() == {}
    assert bench.measured_mfma("attn_fwd sparse") == {}
