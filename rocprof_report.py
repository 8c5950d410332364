#!/usr/bin/env python3
"""rocprofv3 harness of the benchmark: runs the profiler passes behind the committed summaries and
reduces their CSV output to the summaries under profiles/ (JSON that bench.py reads, Markdown to
read).

    python rocprof_report.py collect --raw gpurun_out/prof    # on a GPU machine: every pass
    python rocprof_report.py reduce  --raw gpurun_out/prof --out profiles
    python rocprof_report.py fixture --raw gpurun_out/prof --out tests/data/rocprof

`collect` runs each pass as its own `timeout -k 10 <s> rocprofv3 ... -- <python> -u bench.py ...`
child (from /tmp, TMPDIR=/tmp), stops at the first failure and prints every command before it
runs; this process never touches the GPU itself.  `reduce` needs only the CSV files.  `fixture`
keeps the rows of the library's own kernels and of the calibration copy (the CPU test of this
harness reduces them).

The summaries, for three workloads of bench.py at the HunyuanVideo-720p grid (the benchmarked
layer; the semantic clustering leg; the block-sparse leg):
  * per-kernel launch durations (kernel trace): mean, median, min, max;
  * HBM bytes per launch of each leg's attention kernel and, for the layer, of the norm/RoPE
    kernel, the profiling pass and the layout-transformation kernel: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for a plain 1 GiB device copy
    (which moves 1 GiB each way), against the algorithmic bytes and the 8 TB/s HBM peak;
  * MFMA utilisation: SQ_VALU_MFMA_BUSY_CYCLES over the cycles of all SIMDs (GRBM_GUI_ACTIVE,
    summed over the XCDs, counts every cycle once per XCD), the clock over the kernel's own
    duration, and the matrix work that SQ_INSTS_VALU_MFMA_MOPS_BF16 counts.

Every JSON summary carries a hash of the kernel sources it was taken on; bench.py attaches a
figure to its output only while the source still has that hash.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import shlex
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "spatial_temporal_sparse_amd", "csrc")

PEAK_HBM_GBS = 8000.0
N_XCC = 8            # XCDs of an MI355X
N_SIMD = 1024        # 256 CUs x 4 SIMDs
MFMA_FLOP_PER_MOP = 512
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE"]

# The 720p grid: B=1, H=24, S=118800, D=128 bf16; the layer's planted inputs choose 12 temporal heads.
S720, H720, D720 = 118800, 24, 128
HEAD_BYTES = S720 * D720 * 2                 # one head of one tensor
QKVO_BYTES = 4 * H720 * HEAD_BYTES           # an attention kernel: Q, K, V read once, O written once
HBM_KERNELS = {  # key: (kernel name pattern, pass suffix, algorithmic bytes per launch)
    "qknorm_rope": ("qknorm_rope_kernel", "layer", 4 * H720 * HEAD_BYTES),        # Q, K read and written
    "profile_partial": ("profile_partial_kernel", "layer", 2 * H720 * HEAD_BYTES),  # K, V read once
    "permute_rows": ("permute_rows_kernel", "explicit", 2 * 12 * HEAD_BYTES),     # one tensor, 12 heads, r + w
}

# Source files whose code each summary depends on (comments and whitespace do not count).
SOURCES = {
    "attn_fwd": ("attn_fwd.hip", "svg_internal.h"),
    "hbm": ("qknorm_rope.hip", "profile_heads.hip", "permute.hip", "svg_internal.h"),
    "search": ("block_search.hip", "svg_internal.h"),
}

# bench.py launches its dense comparison (the same attention kernel run dense) twice, after every
# sparse launch of the layer workload: the last two attn_fwd_kernel dispatches are the dense ones.
DENSE_TAIL = 2

WORKLOADS = {
    # name: bench options, title, attention kernel, its key in the MFMA record, traffic JSON,
    #       extra MFMA kernels {pattern: key}
    "layer": {"bench": [], "title": "the benchmarked 720p layer (QK-RMSNorm + 3D RoPE, profiling, block-sparse "
                                    "attention, fused layout)",
              "attn": "attn_fwd_kernel", "traffic_json": "attn_fwd_hunyuan720p_traffic.json",
              "trace_md": "kernel_trace_hunyuan720p_layer.md", "traffic_md": "traffic_hunyuan720p.md",
              "extra_mfma": {}},
    "svg2": {"bench": ["--workload", "hunyuan720p_svg2"],
             "title": "the semantic clustering leg at 720p (k-means, centroid top-p, cluster attention)",
             "attn": "cluster_attn_kernel", "traffic_json": "cluster_attn_hunyuan720p_svg2_traffic.json",
             "trace_md": "kernel_trace_hunyuan720p_svg2.md", "traffic_md": "traffic_hunyuan720p_svg2.md",
             "extra_mfma": {"kmeans_assign_kernel": "kmeans_assign"}},
    "blocks": {"bench": ["--workload", "hunyuan720p_blocks"],
               "title": "the block-sparse leg at 720p (dense step with LSE, LSE-cached block search, block attention)",
               "attn": "block_attn_kernel", "traffic_json": "block_attn_hunyuan720p_blocks_traffic.json",
               "trace_md": "kernel_trace_hunyuan720p_blocks.md", "traffic_md": "traffic_hunyuan720p_blocks.md",
               "extra_mfma": {"block_mass_kernel": "block_mass"}},
}

NO_EXTRAS = ["--no-cpu-baseline", "--no-isolated"]
SHORT = ["--steps", "2", "--warmup", "0", "--layers", "1", "--no-compare"]


def _passes():
    p = {}
    for wl, w in WORKLOADS.items():
        trace_steps = ["--steps", "4", "--warmup", "1", "--no-compare"] if wl == "layer" else ["--steps", "2",
                                                                                                "--warmup", "1"]
        p[f"trace_{wl}"] = (["--kernel-trace", "--stats"], w["bench"] + trace_steps + NO_EXTRAS, 300)
        p[f"fetch_{wl}"] = (["--kernel-trace", "--pmc", "FETCH_SIZE"], w["bench"] + SHORT + NO_EXTRAS, 240)
        p[f"write_{wl}"] = (["--kernel-trace", "--pmc", "WRITE_SIZE"], w["bench"] + SHORT + NO_EXTRAS, 240)
        pat = "|".join([w["attn"], *w["extra_mfma"]])
        p[f"mfma_{wl}"] = (["--kernel-trace", "--pmc", *MFMA_COUNTERS, "--kernel-include-regex", pat],
                           w["bench"] + SHORT + NO_EXTRAS, 240)
    explicit = ["--steps", "2", "--warmup", "0", "--layers", "1", "--no-compare", "--layout", "explicit"] + NO_EXTRAS
    p["trace_explicit"] = (["--kernel-trace", "--stats"],
                           ["--steps", "4", "--warmup", "1", "--no-compare", "--layout", "explicit"] + NO_EXTRAS, 300)
    p["fetch_explicit"] = (["--kernel-trace", "--pmc", "FETCH_SIZE", "--kernel-include-regex", "permute_rows"],
                           explicit, 240)
    p["write_explicit"] = (["--kernel-trace", "--pmc", "WRITE_SIZE", "--kernel-include-regex", "permute_rows"],
                           explicit, 240)
    p["copy_fetch"] = (["--kernel-trace", "--pmc", "FETCH_SIZE"], ["--copy-calibration"], 120)
    p["copy_write"] = (["--kernel-trace", "--pmc", "WRITE_SIZE"], ["--copy-calibration"], 120)
    return p


PASSES = _passes()


# ----------------------------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------------------------
def source_sha(group):
    h = hashlib.sha256()
    for f in SOURCES[group]:
        with open(os.path.join(CSRC, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def pass_command(name, raw, python=sys.executable, bench=None):
    prof, args, _ = PASSES[name]
    out = os.path.join(raw, name)
    bench = bench or os.path.join(ROOT, "bench.py")
    return ["rocprofv3", *prof, "--output-format", "csv", "-d", out, "-o", "run", "--", python, "-u", bench, *args]


def display_command(name):
    """The command of a pass as typed from /tmp with the repository at $R."""
    return " ".join(shlex.quote(a) if "$" not in a else a
                    for a in pass_command(name, "$R/gpurun_out/prof", "python3", "$R/bench.py"))


def find_csv(raw, name, kind):
    hits = sorted(glob.glob(os.path.join(raw, name, "**", f"*{kind}.csv"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{kind}.csv under {os.path.join(raw, name)}")
    return hits[0]


def read_rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def short_name(name):
    """'void svg::(anonymous namespace)::attn_fwd_kernel<128>(svg::AttnArgs, int)' -> 'attn_fwd_kernel<128>'."""
    n = re.sub(r"^void\s+", "", name)
    n = re.sub(r"^svg::(\(anonymous namespace\)::)?", "", n)
    depth, out = 0, []
    for ch in n:                      # drop the parameter list, keep template arguments
        if ch == "(" and depth == 0 and out:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out)


def dispatches(trace_csv, pattern):
    """[(dispatch id, kernel name, duration in us)] of kernels whose name matches `pattern`, in
    dispatch order."""
    out = []
    for r in read_rows(trace_csv):
        name = r["Kernel_Name"]
        if re.search(pattern, name):
            out.append((int(r["Dispatch_Id"]), name, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    out.sort()
    return out


def counters(counter_csv, pattern, counter):
    """{dispatch id: value} of one counter for kernels whose name matches `pattern` (values of one
    dispatch summed, should the CSV split them over rows), in dispatch order."""
    vals = {}
    for r in read_rows(counter_csv):
        if r["Counter_Name"] == counter and re.search(pattern, r["Kernel_Name"]):
            d = int(r["Dispatch_Id"])
            vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
    return dict(sorted(vals.items()))


def stats_us(durations):
    return {"dispatches": len(durations), "mean_us": statistics.fmean(durations),
            "median_us": statistics.median(durations), "min_us": min(durations), "max_us": max(durations)}


def sparse_ids(ids, attn):
    """The sparse dispatches among an attention kernel's dispatch ids (see DENSE_TAIL)."""
    return ids[:-DENSE_TAIL] if attn == "attn_fwd_kernel" else ids


# ----------------------------------------------------------------------------------------------
# reductions
# ----------------------------------------------------------------------------------------------
def reduce_trace(trace_csv, timed_steps=None):
    """Per-kernel statistics of the library's kernels; the layer's attention kernel split into
    sparse (all, and the last `timed_steps`: the timed steps) and dense dispatches."""
    by = {}
    for _, name, us in dispatches(trace_csv, r"svg::|__amd_rocclr_copy"):
        by.setdefault(short_name(name), []).append(us)
    out = {}
    for name, us in by.items():
        if name.startswith("attn_fwd_kernel") and len(us) > DENSE_TAIL:
            sparse = us[:-DENSE_TAIL]
            out[f"{name} sparse, all dispatches"] = stats_us(sparse)
            if timed_steps:
                out[f"{name} sparse, the {timed_steps} timed steps"] = stats_us(sparse[-timed_steps:])
            out[f"{name} dense"] = stats_us(us[-DENSE_TAIL:])
        else:
            out[name] = stats_us(us)
    return dict(sorted(out.items(), key=lambda kv: -kv[1]["mean_us"] * kv[1]["dispatches"]))


def copy_scale(raw):
    """KiB that FETCH_SIZE / WRITE_SIZE report per GiB a plain device copy reads / writes, and
    the factors that turn the counters into bytes."""
    res = {}
    for what, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        vals = list(counters(find_csv(raw, f"copy_{what}", "counter_collection"), r"[Cc]opy", counter).values())
        if not vals:
            raise ValueError(f"copy_{what}: no copy dispatch in the counter CSV")
        per_gib = statistics.median(vals)          # each dispatch copies 1 GiB
        res[what] = {"kib_per_gib": per_gib, "scale": (1 << 20) / per_gib}
    return res


def traffic(raw, pattern, suffix, cal, select=None):
    """Scaled HBM bytes per launch of the kernels matching `pattern` in the fetch_/write_<suffix>
    passes (optionally only the dispatch ids `select` keeps), and their mean duration there."""
    fp, wp = f"fetch_{suffix}", f"write_{suffix}"
    f = counters(find_csv(raw, fp, "counter_collection"), pattern, "FETCH_SIZE")
    w = counters(find_csv(raw, wp, "counter_collection"), pattern, "WRITE_SIZE")
    fi, wi = list(f), list(w)
    if select is not None:
        fi, wi = select(fi), select(wi)
    fk, wk = [f[i] for i in fi], [w[i] for i in wi]
    if not fk or not wk:
        raise ValueError(f"no {pattern} dispatch with FETCH_SIZE and WRITE_SIZE in {fp} / {wp}")
    dur = {d: us for d, _, us in dispatches(find_csv(raw, fp, "kernel_trace"), pattern)}
    fb = statistics.fmean(fk) * 1024 * cal["fetch"]["scale"]
    wb = statistics.fmean(wk) * 1024 * cal["write"]["scale"]
    return {"fetch_kib_raw": fk, "write_kib_raw": wk, "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
            "bytes_per_launch": fb + wb, "mean_us_counter_run": statistics.fmean(dur[i] for i in fi if i in dur)}


def mfma(raw, wl, pattern, select=None):
    """MFMA busy fraction, clock and counted work of the dispatches matching `pattern` in the
    mfma_<wl> pass (optionally only the ids `select` keeps)."""
    path = find_csv(raw, f"mfma_{wl}", "counter_collection")
    busy, mops, grbm = (counters(path, pattern, c) for c in MFMA_COUNTERS)
    dur = {d: us for d, _, us in dispatches(find_csv(raw, f"mfma_{wl}", "kernel_trace"), pattern)}
    ids = sorted(set(busy) & set(mops) & set(grbm) & set(dur))
    if select is not None:
        ids = select(ids)
    if not ids:
        raise ValueError(f"mfma_{wl}: no {pattern} dispatch with all counters")
    cyc = sum(grbm[i] for i in ids) / N_XCC
    us = sum(dur[i] for i in ids)
    return {"dispatches": len(ids), "mean_us": us / len(ids),
            "mfma_busy": sum(busy[i] for i in ids) / (cyc * N_SIMD),
            "clock_ghz": cyc / (us * 1e3),
            "counted_tflop_per_launch": sum(mops[i] for i in ids) * MFMA_FLOP_PER_MOP / len(ids) / 1e12}


def _write(out_dir, name, text):
    with open(os.path.join(out_dir, name), "w") as fh:
        fh.write(text if isinstance(text, str) else json.dumps(text, indent=1) + "\n")
    return name


def _cmd_block(names):
    return ["Commands (from /tmp, TMPDIR=/tmp, repository root R):", ""] + ["    " + display_command(n) for n in names]


def reduce_all(raw, out_dir, workloads=None):
    """Every summary whose passes are present under `raw`; returns the file names written."""
    os.makedirs(out_dir, exist_ok=True)
    workloads = [w for w in (workloads or WORKLOADS) if os.path.isdir(os.path.join(raw, f"trace_{w}"))]
    cal = copy_scale(raw)
    sha = {g: source_sha(g) for g in SOURCES}
    written = []
    mfma_rec = {"kernel_sha": sha["attn_fwd"], "search_sha": sha["search"], "counters": MFMA_COUNTERS,
                "n_xcc": N_XCC, "n_simd": N_SIMD, "kernels": {}}
    cal_line = (f"Calibration: a plain 1 GiB device copy reads FETCH_SIZE = {cal['fetch']['kib_per_gib']:.0f} KiB "
                f"and WRITE_SIZE = {cal['write']['kib_per_gib']:.0f} KiB, so the counters are scaled by "
                f"{cal['fetch']['scale']:.3f} (fetch) and {cal['write']['scale']:.3f} (write) to bytes.  "
                "FETCH_SIZE counts every L2 miss, whether the 256 MB Infinity Cache or HBM serves it.")

    for wl in workloads:
        w = WORKLOADS[wl]
        # kernel trace(s)
        traces = [(f"trace_{wl}", w["trace_md"], w["title"])]
        if wl == "layer":
            traces.append(("trace_explicit", "kernel_trace_hunyuan720p_explicit.md",
                           "the 720p layer with the explicit layout (separate permute / unpermute passes)"))
        for pname, fname, title in traces:
            if not os.path.isdir(os.path.join(raw, pname)):
                continue
            st = reduce_trace(find_csv(raw, pname, "kernel_trace"), timed_steps=4 if wl == "layer" else None)
            md = [f"# Kernel trace: {title}", ""] + _cmd_block([pname]) + [
                "", "Grid: B=1, H=24, F=33 x 45 x 80 (S=118800), D=128, bf16.  Reduced by `python rocprof_report.py "
                    "reduce`; the library's kernels only.", "",
                "| kernel | dispatches | mean us | median us | min us | max us |", "|---|---|---|---|---|---|"]
            md += [f"| {k} | {v['dispatches']} | {v['mean_us']:.1f} | {v['median_us']:.1f} | {v['min_us']:.1f} | "
                   f"{v['max_us']:.1f} |" for k, v in st.items()]
            written.append(_write(out_dir, fname, "\n".join(md) + "\n"))

        # traffic of the attention kernel (and, for the layer, of the HBM-bound kernels)
        att = traffic(raw, w["attn"], wl, cal, select=lambda ids, a=w["attn"]: sparse_ids(ids, a))
        att.update({"kernel": f"{w['attn']}<128>, {w['title']}", "kernel_sha": sha["attn_fwd"], "copy": cal,
                    "algorithmic_bytes": QKVO_BYTES})
        written.append(_write(out_dir, w["traffic_json"], att))
        rows = [(f"{w['attn']}<128>" + (" (sparse dispatches)" if wl == "layer" else ""), att)]
        passes = [f"fetch_{wl}", f"write_{wl}"]
        if wl == "layer":
            hbm = {}
            for key, (pat, suffix, algo) in HBM_KERNELS.items():
                t = traffic(raw, pat, suffix, cal)
                t["algorithmic_bytes"] = algo
                hbm[key] = t
                rows.append((key, t))
            passes += ["fetch_explicit", "write_explicit"]
            written.append(_write(out_dir, "hbm_kernels_hunyuan720p_traffic.json",
                                  {"kernel_sha": sha["hbm"], "copy": cal, "kernels": hbm}))
        md = [f"# HBM traffic per launch: {w['title']}", ""] + _cmd_block(passes + ["copy_fetch", "copy_write"]) + [
            "", cal_line, "",
            "| kernel | dispatches | fetched GB | written GB | total GB | algorithmic GB | total / algorithmic | "
            "mean us (counter run) | counted GB/s | algorithmic GB/s | algorithmic / 8 TB/s |",
            "|---|---|---|---|---|---|---|---|---|---|---|"]
        for k, v in rows:
            us = v["mean_us_counter_run"]
            algo = v["algorithmic_bytes"]
            md.append(f"| {k} | {len(v['fetch_kib_raw'])} | {v['fetch_bytes_per_launch'] / 1e9:.3f} | "
                      f"{v['write_bytes_per_launch'] / 1e9:.3f} | {v['bytes_per_launch'] / 1e9:.3f} | {algo / 1e9:.3f} | "
                      f"{v['bytes_per_launch'] / algo:.2f} | {us:.1f} | {v['bytes_per_launch'] / (us * 1e3):.0f} | "
                      f"{algo / (us * 1e3):.0f} | {algo / (us * 1e3) / PEAK_HBM_GBS:.3f} |")
        md += ["", "Counter runs serialise dispatches, so the durations above are each kernel's own.  Algorithmic "
                   "bytes: an attention kernel reads Q, K and V once and writes O once; qknorm_rope reads and writes "
                   "Q and K; profile_partial reads K and V; one permute_rows launch moves one tensor of the 12 "
                   "temporal heads.",
               f"Kernel source hashes: attention {sha['attn_fwd']}, HBM-bound kernels {sha['hbm']}."]
        written.append(_write(out_dir, w["traffic_md"], "\n".join(md) + "\n"))

        # MFMA utilisation
        if os.path.isdir(os.path.join(raw, f"mfma_{wl}")):
            if wl == "layer":
                mfma_rec["kernels"]["attn_fwd sparse"] = mfma(raw, wl, w["attn"], lambda ids: ids[:-DENSE_TAIL])
                mfma_rec["kernels"]["attn_fwd dense"] = mfma(raw, wl, w["attn"], lambda ids: ids[-DENSE_TAIL:])
            else:
                mfma_rec["kernels"][w["attn"].replace("_kernel", "")] = mfma(raw, wl, w["attn"])
            for pat, key in w["extra_mfma"].items():
                mfma_rec["kernels"][key] = mfma(raw, wl, pat)

    if mfma_rec["kernels"]:
        written.append(_write(out_dir, "mfma_busy_hunyuan720p.json", mfma_rec))
        md = ["# MFMA utilisation at the 720p grid (hardware counters)", ""] + _cmd_block(
            [f"mfma_{w}" for w in workloads if os.path.isdir(os.path.join(raw, f"mfma_{w}"))]) + [
            "", f"cycles = GRBM_GUI_ACTIVE / {N_XCC} (each XCD counts every cycle); MFMA busy = "
                f"SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {N_SIMD} SIMDs); clock = cycles / duration; counted work = "
                f"SQ_INSTS_VALU_MFMA_MOPS_BF16 x {MFMA_FLOP_PER_MOP} FLOP.  The fraction of the 2.5 PFLOP/s bf16 peak "
                "(quoted at 2.4 GHz) that a kernel reaches is about its MFMA busy fraction times clock / 2.4 GHz.", "",
            "| kernel | dispatches | mean us | MFMA busy | clock GHz | counted TFLOP per launch |",
            "|---|---|---|---|---|---|"]
        md += [f"| {k} | {v['dispatches']} | {v['mean_us']:.1f} | {v['mfma_busy']:.3f} | {v['clock_ghz']:.2f} | "
               f"{v['counted_tflop_per_launch']:.3f} |" for k, v in mfma_rec["kernels"].items()]
        md.append(f"\nKernel source hashes: attention {sha['attn_fwd']}, block search {sha['search']}.")
        written.append(_write(out_dir, "mfma_busy_hunyuan720p.md", "\n".join(md) + "\n"))
    return written


FIXTURE_COLUMNS = ("Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Counter_Name", "Counter_Value")


def make_fixture(raw, out):
    """Copies of the raw CSVs holding only the rows of the library's kernels and the copy kernel,
    and only the columns the reductions read."""
    keep = re.compile(r"svg::|__amd_rocclr_copy")
    n = 0
    for path in sorted(glob.glob(os.path.join(raw, "*", "**", "*.csv"), recursive=True)):
        if not re.search(r"(kernel_trace|counter_collection)\.csv$", path):
            continue
        rel = os.path.relpath(path, raw)
        with open(path, newline="") as fh:
            rows = list(csv.reader(fh))
        head, body = rows[0], rows[1:]
        col = head.index("Kernel_Name")
        cols = [i for i, h in enumerate(head) if h in FIXTURE_COLUMNS]
        body = [[r[i] for i in cols] for r in body if keep.search(r[col])]
        head = [head[i] for i in cols]
        dst = os.path.join(out, rel)
        os.makedirs(os.path.dirname(dst), exist_ok=True)
        with open(dst, "w", newline="") as fh:
            wtr = csv.writer(fh, quoting=csv.QUOTE_MINIMAL, lineterminator="\n")
            wtr.writerow(head)
            wtr.writerows(body)
        n += 1
    return n


def collect(raw, names):
    raw = os.path.abspath(raw)
    os.makedirs(raw, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for name in names:
        cmd = ["timeout", "-k", "10", str(PASSES[name][2]), *pass_command(name, raw)]
        print(f"[rocprof_report] pass {name}: {' '.join(cmd)}", flush=True)
        with open(os.path.join(raw, f"{name}.log"), "w") as log:
            rc = subprocess.call(cmd, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT)
        print(f"[rocprof_report] pass {name}: exit {rc}", flush=True)
        if rc != 0:
            return rc
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("collect", help="run the rocprofv3 passes (GPU box)")
    c.add_argument("--raw", required=True, help="directory for the raw rocprofv3 output")
    c.add_argument("--passes", nargs="*", default=list(PASSES), choices=list(PASSES))
    r = sub.add_parser("reduce", help="reduce the raw CSV output to the summaries")
    r.add_argument("--raw", required=True)
    r.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    r.add_argument("--workloads", nargs="*", choices=list(WORKLOADS))
    f = sub.add_parser("fixture", help="trim the raw CSV output to the library's kernels")
    f.add_argument("--raw", required=True)
    f.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "collect":
        sys.exit(collect(a.raw, a.passes))
    if a.cmd == "fixture":
        print(f"{make_fixture(a.raw, a.out)} CSV files written under {a.out}")
        return
    for name in reduce_all(a.raw, a.out, a.workloads):
        print(os.path.join(a.out, name))


if __name__ == "__main__":
    main()
