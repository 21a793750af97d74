"""Summaries of rocprofv3 output for the kernels of libdspark.

    python -m draft_verify_sampling_bias_amd.profsum stats KERNEL_STATS_CSV --command CMD > out.txt
    python -m draft_verify_sampling_bias_amd.profsum traffic --kernel NAME \
        --fetch CSV --write CSV --calib-fetch CSV --calib-write CSV --calib-bytes N \
        --alg-bytes N --commands TEXT > out.txt

`stats` condenses a `--kernel-trace --stats` kernel table (calls, total and
average duration per kernel).  `calls` lists one kernel's durations from a
`--kernel-trace` table in call order, grouped per size of a sweep.  `mfma` reports a kernel's bf16 MFMA work and
utilisation from SQ counters and its traced average duration.  `sq` averages
any SQ counters of one kernel per dispatch over several `--pmc` runs and
derives the shares of wave cycles.  `traffic` turns two `--pmc FETCH_SIZE` /
`--pmc WRITE_SIZE` runs (KiB per dispatch) into HBM bytes per launch of one
kernel, each counter scaled by what it reads for a device copy of known size
(the calibration runs), and records a SHA-256 over the fused bias kernel's
source files so that a reader can tell when the figures are stale.  `read_traffic` parses
such a file back.
"""
import argparse
import csv
import hashlib
import os
import sys
from collections import defaultdict


# files the fused bias kernel is compiled from (its figures go stale when any changes)
TILE_SOURCES = ("bias_tile.hip", "dspark_device.h", "launchers.h", "plan.h")
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def tile_source_hash():
    return source_hash([os.path.join(CSRC, n) for n in TILE_SOURCES])


def _short(name, width=100):
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= width else name[: width - 3] + "..."


def stats_text(csv_path, command):
    rows = list(csv.DictReader(open(csv_path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# rocprofv3 kernel statistics", f"# command: {command}",
           f"# {'calls':>6} {'total_us':>10} {'avg_us':>9} {'min_us':>8} {'max_us':>8} {'pct':>6}  kernel"]
    for r in rows:
        out.append(f"  {int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e3:10.1f} "
                   f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:8.2f} "
                   f"{float(r['MaxNs']) / 1e3:8.2f} {float(r['Percentage']):6.2f}  {_short(r['Name'])}")
    return "\n".join(out) + "\n"


def calls_text(trace_csv, kernel, group, labels, command):
    """Durations of the dispatches of one kernel (name substring) in call
    order, grouped: one line per group of `group` calls with its label."""
    rows = [r for r in csv.DictReader(open(trace_csv)) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    names = [_short(r["Kernel_Name"], 60) for r in rows]
    if len(dur) != group * len(labels):
        raise SystemExit(f"{len(dur)} dispatches of {kernel!r}, expected {group} x {len(labels)}")
    out = [f"# kernel durations by call group (rocprofv3 --kernel-trace), {group} calls per size",
           f"# command: {command}",
           f"# {'median_us':>10} {'min_us':>8}  size / kernel"]
    for i, lab in enumerate(labels):
        d = sorted(dur[i * group:(i + 1) * group])
        out.append(f"  {d[len(d) // 2]:10.2f} {d[0]:8.2f}  {lab}  [{names[i * group]}]")
    return "\n".join(out) + "\n"


def _per_dispatch(csv_path, counter):
    """{kernel name: [value per dispatch]} for one counter (KiB)."""
    acc = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        acc[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in acc.items()}


def _pick(table, pattern):
    keys = [k for k in table if pattern in k]
    if len(keys) != 1:
        raise SystemExit(f"kernel pattern {pattern!r} matches {keys}")
    return table[keys[0]]


def _calib_factor(csv_path, counter, true_bytes):
    """true bytes / counter bytes for the largest dispatch of the copy run."""
    vals = [v for lst in _per_dispatch(csv_path, counter).values() for v in lst]
    top = max(vals)
    return true_bytes / (top * 1024.0), top


def traffic_text(kernel, fetch_csv, write_csv, cfetch_csv, cwrite_csv, calib_bytes, alg_bytes, commands):
    f = _pick(_per_dispatch(fetch_csv, "FETCH_SIZE"), kernel)
    w = _pick(_per_dispatch(write_csv, "WRITE_SIZE"), kernel)
    ff, ftop = _calib_factor(cfetch_csv, "FETCH_SIZE", calib_bytes)
    wf, wtop = _calib_factor(cwrite_csv, "WRITE_SIZE", calib_bytes)
    f_kib = sum(f) / len(f)
    w_kib = sum(w) / len(w)
    total = f_kib * 1024 * ff + w_kib * 1024 * wf
    lines = [
        "# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch)",
        *[f"# command: {c}" for c in commands],
        f"kernel: {kernel}",
        f"kernel_sources: {' '.join(TILE_SOURCES)}",
        f"kernel_source_sha256_16: {tile_source_hash()}",
        f"dispatches_fetch: {len(f)}",
        f"dispatches_write: {len(w)}",
        f"fetch_kib_per_dispatch: {f_kib:.1f}",
        f"write_kib_per_dispatch: {w_kib:.1f}",
        f"calib_copy_bytes: {calib_bytes}",
        f"calib_fetch_kib: {ftop:.1f}",
        f"calib_write_kib: {wtop:.1f}",
        f"fetch_scale: {ff:.4f}",
        f"write_scale: {wf:.4f}",
        f"bytes_per_launch: {int(round(total))}",
        f"algorithmic_bytes_per_launch: {alg_bytes}",
        f"traffic_over_algorithmic: {total / alg_bytes:.4f}",
    ]
    return "\n".join(lines) + "\n"


def mfma_text(kernel, counters_csv, stats_csv, flops_per_launch, peak_tflops, commands):
    """MFMA work and utilisation of one kernel: bf16 MFMA MOPs per dispatch
    (one MOP = 512 FLOPs), MFMA busy cycles, and the achieved rate over the
    kernel's average duration from a kernel-trace run."""
    table = {}
    for cn in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES"):
        vals = _pick(_per_dispatch(counters_csv, cn), kernel)
        table[cn] = sum(vals) / len(vals)
    rows = [r for r in csv.DictReader(open(stats_csv)) if kernel in r["Name"]]
    if len(rows) != 1:
        raise SystemExit(f"kernel pattern {kernel!r} matches {len(rows)} rows of {stats_csv}")
    avg_ns = float(rows[0]["AverageNs"])
    flops = table["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
    tflops = flops / (avg_ns * 1e-9) / 1e12
    lines = [
        "# MFMA work of one kernel from rocprofv3 --pmc (per dispatch) and its average duration",
        *[f"# command: {c}" for c in commands],
        f"kernel: {kernel}",
        f"kernel_source_sha256_16: {tile_source_hash()}",
        *[f"{k.lower()}_per_dispatch: {v:.1f}" for k, v in table.items()],
        f"mfma_flops_per_dispatch: {flops:.0f}",
        f"algorithmic_flops_per_launch: {flops_per_launch}",
        f"avg_duration_us: {avg_ns / 1e3:.2f}",
        f"achieved_tflops: {tflops:.1f}",
        f"peak_tflops_bf16_dense: {peak_tflops}",
        f"mfma_utilisation: {tflops / peak_tflops:.4f}",
    ]
    return "\n".join(lines) + "\n"


def sq_text(kernel, csvs, commands):
    """Per-dispatch averages (summed over the chip) of every counter found for
    one kernel in the given counter CSVs, with the shares of wave cycles."""
    table = {}
    n_disp = {}
    for path in csvs:
        names = {r["Counter_Name"] for r in csv.DictReader(open(path))}
        for cn in sorted(names):
            vals = _pick(_per_dispatch(path, cn), kernel)
            table[cn] = sum(vals) / len(vals)
            n_disp[cn] = len(vals)
    lines = ["# SQ counters per dispatch of one kernel (summed over the chip, averaged over its dispatches)",
             *[f"# command: {c}" for c in commands],
             f"kernel: {kernel}",
             f"kernel_source_sha256_16: {tile_source_hash()}",
             f"dispatches: {min(n_disp.values())}"]
    lines += [f"{k}: {v:.0f}" for k, v in sorted(table.items())]
    wc = table.get("SQ_WAVE_CYCLES")
    waves = table.get("SQ_WAVES")
    if wc:
        lines.append("# derived (SQ_WAVE_CYCLES and the active / wait counters count in the same units)")
        for k in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_VMEM",
                  "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_LDS"):
            if k in table:
                lines.append(f"share_of_wave_cycles_{k[3:].lower()}: {table[k] / wc:.3f}")
    if waves:
        for k in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD"):
            if k in table:
                lines.append(f"per_wavefront_{k[3:].lower()}: {table[k] / waves:.0f}")
    if "SQ_LDS_BANK_CONFLICT" in table and "SQ_INSTS_LDS" in table:
        lines.append(f"lds_bank_conflict_cycles_per_lds_instruction: "
                     f"{table['SQ_LDS_BANK_CONFLICT'] / table['SQ_INSTS_LDS']:.3f}")
    return "\n".join(lines) + "\n"


def read_traffic(path):
    """key: value pairs of a traffic summary (comments skipped)."""
    out = {}
    with open(path) as fh:
        for ln in fh:
            ln = ln.strip()
            if not ln or ln.startswith("#") or ":" not in ln:
                continue
            k, v = ln.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    for k in ("fetch", "write", "calib-fetch", "calib-write"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--alg-bytes", type=int, required=True)
    t.add_argument("--commands", action="append", default=[])
    c = sub.add_parser("calls")
    c.add_argument("trace_csv")
    c.add_argument("--kernel", required=True)
    c.add_argument("--group", type=int, required=True)
    c.add_argument("--labels", required=True, help="comma-separated, one per group")
    c.add_argument("--command", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--kernel", required=True)
    m.add_argument("--counters", required=True)
    m.add_argument("--stats", required=True)
    m.add_argument("--flops", type=int, required=True)
    m.add_argument("--peak-tflops", type=float, default=2500.0)
    m.add_argument("--commands", action="append", default=[])
    q = sub.add_parser("sq")
    q.add_argument("--kernel", required=True)
    q.add_argument("--counters", action="append", required=True)
    q.add_argument("--commands", action="append", default=[])
    a = ap.parse_args(argv)
    if a.mode == "sq":
        sys.stdout.write(sq_text(a.kernel, a.counters, a.commands))
        return
    if a.mode == "calls":
        sys.stdout.write(calls_text(a.trace_csv, a.kernel, a.group, a.labels.split(","), a.command))
        return
    if a.mode == "mfma":
        sys.stdout.write(mfma_text(a.kernel, a.counters, a.stats, a.flops, a.peak_tflops, a.commands))
        return
    if a.mode == "stats":
        sys.stdout.write(stats_text(a.csv, a.command))
    else:
        sys.stdout.write(traffic_text(a.kernel, a.fetch, a.write, a.calib_fetch, a.calib_write, a.calib_bytes,
                                      a.alg_bytes, a.commands))


if __name__ == "__main__":
    main()
