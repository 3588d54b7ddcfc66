"""rocprofv3 runs of bench.py and their summaries (kernel times and HBM traffic).

    python -m shared_prefix_kv_amd.profiling run --config NAME [--out-dir DIR] [--bench-arg=ARG]...
    python -m shared_prefix_kv_amd.profiling summarize \\
        --stats DIR --fetch DIR --write DIR --config NAME --out FILE [--cmd "..."]...

``run`` (on the MI355X) runs the five rocprofv3 passes below one after the
other as child processes, each under its own time limit, and then writes the
summary to profiles/<kernel>.<config>.txt and a copy of it into the output
folder; this process itself never touches the GPU.

DIR are rocprofv3 output folders (``-f csv``): ``--stats`` from
``--kernel-trace --stats``, ``--fetch`` / ``--write`` from ``--pmc FETCH_SIZE``
and ``--pmc WRITE_SIZE`` runs of ``bench.py --profile-only --copy-calibration``.

FETCH_SIZE and WRITE_SIZE are per-dispatch byte counters (KiB) whose scale
on this chip is taken from the calibration copy that bench.py launches in the
same process: an elementwise kernel that reads and writes a known number of
bytes.  The factor (known bytes / counter bytes) is applied to every other
kernel's counters.

The summary ends with one ``json:`` line that bench.py reads back to fill in
the roofline's measured traffic, but only while the sources that built the
library are unchanged (``source_sha256``).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

ATTENTION = "fca_attention_kernel"  # both passes in one launch
GQA_GROUPED = "fca_attention_grouped_kernel"  # plans with one launch per pass: grouped pass
GQA_SUFFIX = "fca_attention_suffix_kernel"  # plans with one launch per pass: per-request pass
MLA_GROUPED = "fca_mla_grouped_kernel"  # latent cache: grouped-pass launch
MLA_SUFFIX = "fca_mla_suffix_kernel"  # latent cache: per-request-pass launch
MERGE = "fca_merge_kernel"
CALIBRATION = "mul"  # torch.mul elementwise kernel of the calibration copy
ATTENTION_KERNELS = (ATTENTION, GQA_GROUPED, GQA_SUFFIX, MLA_GROUPED, MLA_SUFFIX)


def source_sha256() -> str:
    """Hash of the HIP sources and the public header the library is built from."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*"))) + [os.path.join(ROOT, "include", "fca.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _one(dirpath: str, suffix: str) -> str:
    found = sorted(glob.glob(os.path.join(dirpath, "**", f"*{suffix}"), recursive=True))
    if not found:
        raise FileNotFoundError(f"no *{suffix} under {dirpath}")
    return found[0]


def _short(name: str) -> str:
    """Kernel name without namespaces, template arguments or parameters."""
    base = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
    return base.split("::")[-1][:42]


def kernel_stats(dirpath: str) -> list[dict]:
    rows = []
    with open(_one(dirpath, "kernel_stats.csv")) as fh:
        for r in csv.DictReader(fh):
            rows.append(
                dict(
                    name=r["Name"],
                    calls=int(r["Calls"]),
                    avg_us=float(r["AverageNs"]) / 1e3,
                    min_us=float(r["MinNs"]) / 1e3,
                    max_us=float(r["MaxNs"]) / 1e3,
                    share=float(r["Percentage"]),
                )
            )
    return rows


def kernel_durations(dirpath: str, key: str) -> list[float]:
    """Per-dispatch durations (us) of kernels whose name contains `key`, in
    dispatch order."""
    rows = []
    with open(_one(dirpath, "kernel_trace.csv")) as fh:
        for r in csv.DictReader(fh):
            if key in r["Kernel_Name"]:
                rows.append((int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    return [d for _, d in sorted(rows)]


def counters(dirpath: str, counter: str) -> dict[str, list[float]]:
    """Counter values (bytes) per dispatch in dispatch order, grouped by kernel
    name."""
    by = {}
    with open(_one(dirpath, "counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            by.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"]) * 1024.0))
    return {k: [v for _, v in sorted(vals)] for k, vals in by.items()}


def _pick(by: dict[str, list[float]], key: str) -> list[float]:
    vals = []
    for name, v in by.items():
        if key == CALIBRATION:
            if "vectorized_elementwise_kernel" in name and "MulFunctor" in name:
                vals += v
        elif key in name:
            vals += v
    return vals


UTIL_COUNTERS = ("MfmaUtil", "LdsUtil", "LDSBankConflict", "SQ_INSTS_VALU_MFMA_MOPS_BF16")
MOPS_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F16",)


def utilisation(dirpath: str, kernels, durations, mops_dir: str | None = None) -> dict:
    """Median per dispatch of the matrix-core and LDS counters of a
    ``--pmc MfmaUtil LdsUtil LDSBankConflict SQ_INSTS_VALU_MFMA_MOPS_BF16``
    run, per kernel, plus the bf16 matrix rate from the operation count
    (512 per unit) over the kernel's median duration; with ``mops_dir`` (a
    ``--pmc SQ_INSTS_VALU_MFMA_MOPS_F16`` run) the fp16 rate as well."""
    res = {}
    sources = [(dirpath, UTIL_COUNTERS)]
    if mops_dir and glob.glob(os.path.join(mops_dir, "**", "*counter_collection.csv"), recursive=True):
        sources.append((mops_dir, MOPS_COUNTERS))
    for key in kernels:
        row = {}
        for d_, counters in sources:
            for c in counters:
                vals = _pick({k: v for k, v in _raw_counters(d_, c).items()}, key)
                if vals:
                    row[c] = statistics.median(vals)
        if row:
            d = durations.get(key)
            for c, name in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", "bf16_TFLOPs"), ("SQ_INSTS_VALU_MFMA_MOPS_F16", "f16_TFLOPs")):
                if d and c in row:
                    row[name] = row[c] * 512 / (statistics.median(d) * 1e-6) / 1e12
            res[key] = row
    return res


def _raw_counters(dirpath: str, counter: str) -> dict[str, list[float]]:
    """Counter values per dispatch (as written, no scaling), by kernel name."""
    by = {}
    with open(_one(dirpath, "counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                by.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return {k: [v for _, v in sorted(vals)] for k, vals in by.items()}


def summarize(stats_dir, fetch_dir, write_dir, config, copy_bytes, algorithmic_bytes, cmds, out, util_dir=None,
              mops_dir=None):
    stats = kernel_stats(stats_dir)
    att_kernels = [k for k in ATTENTION_KERNELS if kernel_durations(stats_dir, k)]
    if not att_kernels:
        raise RuntimeError("no attention kernel in the kernel trace")
    durations = {k: kernel_durations(stats_dir, k) for k in att_kernels + [MERGE]}
    # the launch the roofline is taken on: the longest attention launch
    kernel = max(att_kernels, key=lambda k: statistics.median(durations[k]))
    fetch = counters(fetch_dir, "FETCH_SIZE")
    write = counters(write_dir, "WRITE_SIZE")
    cal_f = _pick(fetch, CALIBRATION)
    cal_w = _pick(write, CALIBRATION)
    if not cal_f or not cal_w:
        raise RuntimeError("calibration copy not found in the counter runs")
    f_factor = copy_bytes / statistics.median(cal_f)
    w_factor = copy_bytes / statistics.median(cal_w)
    res = {}
    for key in att_kernels + [MERGE]:
        fv, wv = _pick(fetch, key), _pick(write, key)
        if fv and wv:
            res[key] = dict(
                dispatches=len(fv),
                fetch_counter_bytes=statistics.median(fv),
                write_counter_bytes=statistics.median(wv),
                fetch_bytes=statistics.median(fv) * f_factor,
                write_bytes=statistics.median(wv) * w_factor,
            )
    att = res.get(kernel)
    lines = [
        f"# {kernel} on the {config} workload: kernel times and HBM traffic (rocprofv3)",
        "",
        "Commands (from the repository root, on the MI355X):",
    ]
    lines += [f"  {c}" for c in cmds]
    lines += [
        "",
        f"source_sha256: {source_sha256()}",
        "",
        "Kernel trace statistics (--kernel-trace --stats), fca kernels:",
        f"  {'kernel':42s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s}",
    ]
    for r in stats:
        if "fca" in r["name"]:
            lines.append(f"  {_short(r['name']):42s} {r['calls']:6d} {r['avg_us']:9.2f} {r['min_us']:9.2f} {r['max_us']:9.2f}")
    for k, d in durations.items():
        if d:
            lines.append(f"  {k}: median of {len(d)} dispatches {statistics.median(d):.2f} us, mean {statistics.fmean(d):.2f} us")
    lines += [
        "",
        f"Counter calibration: the copy reads and writes {copy_bytes} bytes per dispatch;",
        f"  FETCH_SIZE reads {statistics.median(cal_f):.0f} bytes -> factor {f_factor:.4f}",
        f"  WRITE_SIZE reads {statistics.median(cal_w):.0f} bytes -> factor {w_factor:.4f}",
        "",
        "HBM traffic per dispatch (median over dispatches, calibrated):",
    ]
    for key, v in res.items():
        lines.append(
            f"  {key:24s} fetch {v['fetch_bytes'] / 1e6:9.2f} MB  write {v['write_bytes'] / 1e6:8.2f} MB"
            f"  (counters {v['fetch_counter_bytes'] / 1e6:.2f} / {v['write_counter_bytes'] / 1e6:.2f} MB,"
            f" {v['dispatches']} dispatches)"
        )
    if att and algorithmic_bytes:
        lines.append(
            f"  algorithmic bytes per {kernel} launch {algorithmic_bytes / 1e6:.2f} MB;"
            f" measured / algorithmic = {(att['fetch_bytes'] + att['write_bytes']) / algorithmic_bytes:.3f}"
        )
    util = {}
    if util_dir:
        util = utilisation(util_dir, att_kernels + [MERGE], durations, mops_dir)
        lines += [
            "",
            "Matrix cores and LDS per dispatch (median; rocprofv3 derived counters MfmaUtil, LdsUtil,",
            "LDSBankConflict in percent of GPU-active time, and the bf16 / fp16 MFMA operation counts):",
        ]
        for key, v in util.items():
            lines.append(
                f"  {key:24s} MFMA busy {v.get('MfmaUtil', float('nan')):6.1f} %  LDS active {v.get('LdsUtil', float('nan')):6.1f} %"
                f"  LDS bank conflicts {v.get('LDSBankConflict', float('nan')):5.1f} %"
                + (f"  bf16 MFMA {v['bf16_TFLOPs']:7.1f} TFLOP/s" if "bf16_TFLOPs" in v else "")
                + (f"  fp16 MFMA {v['f16_TFLOPs']:7.1f} TFLOP/s" if "f16_TFLOPs" in v else "")
            )
    payload = dict(
        config=config,
        source_sha256=source_sha256(),
        kernel=kernel,
        avg_launch_us=statistics.median(durations[kernel]),
        launch_us={k: statistics.median(d) for k, d in durations.items() if d},
        fetch_factor=f_factor,
        write_factor=w_factor,
        traffic=res,
        util=util,
    )
    lines += ["", "json: " + json.dumps(payload)]
    text = "\n".join(lines) + "\n"
    with open(out, "w") as fh:
        fh.write(text)
    return text


def load_traffic(config: str):
    """Calibrated traffic per attention dispatch from the committed summary,
    or None if there is none or the sources changed since it was taken."""
    paths = [os.path.join(ROOT, "profiles", f"{k}.{config}.txt") for k in ATTENTION_KERNELS]
    paths = [p for p in paths if os.path.exists(p)]
    if not paths:
        return None
    path = paths[0]
    with open(path) as fh:
        for line in fh:
            if line.startswith("json: "):
                d = json.loads(line[6:])
                if d.get("source_sha256") != source_sha256():
                    return None
                return d
    return None


PASSES = [
    ("stats", ["--kernel-trace", "--stats"]),
    ("fetch", ["--pmc", "FETCH_SIZE"]),
    ("write", ["--pmc", "WRITE_SIZE"]),
    ("util", ["--pmc", "MfmaUtil", "LdsUtil", "LDSBankConflict", "SQ_INSTS_VALU_MFMA_MOPS_BF16"]),
    ("mops", ["--pmc", "SQ_INSTS_VALU_MFMA_MOPS_F16"]),
]
OPTIONAL_PASSES = ("mops",)


def run(config: str, out_dir: str, extra: list[str], timeout_s: int = 300) -> str:
    """The rocprofv3 passes of ``bench.py --profile-only`` for one
    workload, then the summary; returns its path."""
    import subprocess
    import sys

    out_dir = os.path.abspath(out_dir)
    variant = "non_cascade" if "--no-cascade" in extra else "separate_passes" if "--separate-passes" in extra else ""
    config_dir = config + ("_" + variant if variant else "")
    bench = [sys.executable, os.path.join(ROOT, "bench.py"), "--config", config, "--profile-only", "--copy-calibration",
             "--no-cpu-baseline", *extra]
    env = dict(os.environ, TMPDIR="/tmp")
    cmds = ["cd /tmp && export TMPDIR=/tmp"]
    for name, opts in PASSES:
        d = os.path.join(out_dir, config_dir, name)
        cmd = ["timeout", "-k", "10", str(timeout_s), "rocprofv3", *opts, "-f", "csv", "-d", d, "-o", "run", "--", *bench]
        shown = " ".join(cmd).replace(out_dir, "<out>").replace(ROOT, "<repo>").replace(sys.executable, "python3")
        cmds.append(shown)
        print("[profile]", shown, flush=True)
        res = subprocess.run(cmd, cwd="/tmp", env=env)
        # rocprofv3 may end with a signal after the program finished and its
        # files are complete; a missing result file is what counts as failure
        found = glob.glob(os.path.join(d, "**", "*kernel_stats.csv" if name == "stats" else "*counter_collection.csv"),
                          recursive=True)
        if not found and name not in OPTIONAL_PASSES:
            raise RuntimeError(f"rocprofv3 pass {name} left no results (exit {res.returncode})")
    # algorithmic bytes of the dominant launch, as bench.py reports them
    algo = 0
    tmp = os.path.join(out_dir, config_dir, "algorithmic.json")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", config, "--profile-only",
                          "--no-cpu-baseline", *extra], capture_output=True, text=True, env=env, timeout=timeout_s)
    if res.returncode == 0 and res.stdout.strip():
        line = json.loads(res.stdout.strip().splitlines()[-1])
        algo = int(line["roofline"].get("bytes_per_launch", 0))
        with open(tmp, "w") as fh:
            fh.write(json.dumps(line["roofline"]))
    kernel = _dominant_kernel(os.path.join(out_dir, config_dir, "stats"))
    label = config + ("." + variant if variant else "")
    out = os.path.join(ROOT, "profiles", f"{kernel}.{label}.txt")
    summ = [
        f"python3 -m shared_prefix_kv_amd.profiling summarize --stats {out_dir}/{config_dir}/stats --fetch "
        f"{out_dir}/{config_dir}/fetch --write {out_dir}/{config_dir}/write --util {out_dir}/{config_dir}/util --mops {out_dir}/{config_dir}/mops --config {label} "
        f"--copy-bytes {COPY_BYTES} --algorithmic-bytes {algo} --out profiles/{kernel}.{label}.txt".replace(out_dir, "<out>").replace(ROOT, "<repo>")
    ]
    cmds = [f"python3 -m shared_prefix_kv_amd.profiling run --config {config} --out-dir <out>"
            + "".join(f" --bench-arg={a}" for a in extra),
            "which runs:"] + ["  " + c for c in cmds + summ]
    text = summarize(os.path.join(out_dir, config_dir, "stats"), os.path.join(out_dir, config_dir, "fetch"),
                     os.path.join(out_dir, config_dir, "write"), label, COPY_BYTES, algo, cmds, out,
                     os.path.join(out_dir, config_dir, "util"), os.path.join(out_dir, config_dir, "mops"))
    # a copy beside the raw rocprofv3 results
    with open(os.path.join(out_dir, os.path.basename(out)), "w") as fh:
        fh.write(text)
    return out


COPY_BYTES = 1 << 30  # the calibration copy bench.py launches (--copy-calibration)


def _dominant_kernel(stats_dir: str) -> str:
    ks = [k for k in ATTENTION_KERNELS if kernel_durations(stats_dir, k)]
    return max(ks, key=lambda k: statistics.median(kernel_durations(stats_dir, k)))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--config", required=True)
    r.add_argument("--out-dir", default=os.path.join(ROOT, "_build", "prof"))
    r.add_argument("--bench-arg", action="append", default=[], help="extra bench.py argument (repeatable)")
    s = sub.add_parser("summarize")
    s.add_argument("--stats", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--config", required=True)
    s.add_argument("--copy-bytes", type=int, required=True)
    s.add_argument("--algorithmic-bytes", type=int, default=0)
    s.add_argument("--cmd", action="append", default=[])
    s.add_argument("--util", default=None, help="rocprofv3 folder of the matrix-core / LDS counter run")
    s.add_argument("--mops", default=None, help="rocprofv3 folder of the fp16 MFMA operation-count run")
    s.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "run":
        print(open(run(a.config, a.out_dir, a.bench_arg)).read(), end="")
        return
    print(summarize(a.stats, a.fetch, a.write, a.config, a.copy_bytes, a.algorithmic_bytes, a.cmd, a.out, a.util, a.mops), end="")


if __name__ == "__main__":
    main()
