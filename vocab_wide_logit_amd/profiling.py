"""Summaries of rocprofv3 runs of ``bench.py`` (kernel durations and HBM
traffic counters), written as short text files, and the reader ``bench.py``
uses to attach the measured traffic of the row kernel to its roofline figure.

    python -m vocab_wide_logit_amd.profiling stats  <kernel_stats.csv> <kernel_trace.csv> <out.txt> <command...>
    python -m vocab_wide_logit_amd.profiling pmc    <fetch counter csv> <write counter csv> <out.txt> [--grid=N] <command...>
    python -m vocab_wide_logit_amd.profiling sq     <SQ counter csv> <out.txt> [--grid=N] <command...>
    python -m vocab_wide_logit_amd.profiling kernel <trace csv> <fetch csv> <write csv> <SQ csv> <out.txt>
                                                    <kernel regex> <grid> <algorithmic bytes> <workload> <command...>
    python -m vocab_wide_logit_amd.profiling counters <counter csv> <out.txt> <kernel regex> <workload> <command...>

The traffic summary scales the row kernel's FETCH_SIZE and WRITE_SIZE (KiB per
dispatch) by what the same counters read for a plain elementwise copy of a
known size in the same process, so the figure is in bytes per launch.
"""
from __future__ import annotations

import csv
import hashlib
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# sources whose change invalidates a recorded traffic figure, per mode
KERNEL_SOURCES = {
    "asym": ("asym_kernels.hpp", "asym_ab.hip", "vwl_device.hpp", "vwl_internal.hpp"),
    "rapid": ("rapid.hip", "vwl_device.hpp", "vwl_internal.hpp"),
}
# the bench's dominant kernel of each mode: bf16 AsymSpec with delta = a - b
# under the CDA gate (any vectors per thread), and the RAPID row kernel
ROW_KERNEL_RE = {"asym": r"asym_rows_kernel<1, \d+, 0, 0>", "rapid": r"rapid_rows_kernel"}
COPY_KERNEL_RE = r"neg_kernel"        # torch.neg(src, out=dst): reads and writes COPY_BYTES
COPY_BYTES = 1 << 30


def source_hash(mode: str = "asym") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[mode]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(names)


def short_name(name: str) -> str:
    name = name.strip().replace("(anonymous namespace)::", "")
    m = re.match(r"^(?:void\s+)?([^(]*)", name)
    base = m.group(1) if m else name
    return base.strip()[:110]


def _shape_table(trace_csv: str):
    """Per (kernel, grid) launch shape: calls, mean, median, min and max
    duration in microseconds, from the kernel trace.  Workloads that launch
    the same kernel at different grids are told apart this way."""
    groups = {}
    for r in _rows(trace_csv):
        key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])),
               int(r["Workgroup_Size_X"]))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault(key, []).append(dur)
    out = []
    for (name, wgs, wgsize), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        ds = sorted(d)
        out.append("%-70s %7d %5d %7d %11.2f %11.2f %11.2f %11.2f" % (
            name[:70], wgs, wgsize, len(d), sum(d) / len(d), ds[len(ds) // 2], ds[0], ds[-1]))
    return out


def summarize_stats(stats_csv: str, out_path: str, command: str, trace_csv: str | None = None) -> None:
    rows = _rows(stats_csv)
    lines = ["# rocprofv3 kernel statistics", "",
             "command: " + command, "source hash (asym kernels): " + source_hash("asym"),
             "source hash (rapid kernels): " + source_hash("rapid"), "",
             "%-100s %7s %11s %11s %11s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "total_ms")]
    for r in rows:
        name = short_name(_col(r, "Name", "KernelName", "Kernel_Name"))
        calls = int(_col(r, "Calls"))
        avg = float(_col(r, "AverageNs")) / 1e3
        mn = float(_col(r, "MinNs")) / 1e3
        mx = float(_col(r, "MaxNs")) / 1e3
        tot = float(_col(r, "TotalDurationNs")) / 1e6
        lines.append("%-100s %7d %11.2f %11.2f %11.2f %12.3f" % (name, calls, avg, mn, mx, tot))
    if trace_csv:
        lines += ["", "per launch shape (kernel trace):", "",
                  "%-70s %7s %5s %7s %11s %11s %11s %11s" % ("kernel", "wgs", "wgsz", "calls", "avg_us",
                                                            "median_us", "min_us", "max_us")]
        lines += _shape_table(trace_csv)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(path: str, counter: str, kernel_re: str, grid_wgs: int | None = None):
    """Mean over dispatches of the kernels matching kernel_re (and, when
    given, launched with grid_wgs workgroups) of the counter (summed over its
    instances within a dispatch), and the dispatch count."""
    per = {}
    for r in _rows(path):
        if _col(r, "Counter_Name") != counter:
            continue
        if not re.search(kernel_re, short_name(_col(r, "Kernel_Name"))):
            continue
        if grid_wgs is not None and int(_col(r, "Grid_Size")) // max(1, int(_col(r, "Workgroup_Size"))) != grid_wgs:
            continue
        d = _col(r, "Dispatch_Id")
        per[d] = per.get(d, 0.0) + float(_col(r, "Counter_Value"))
    if not per:
        raise ValueError("no %s dispatches of /%s/ in %s" % (counter, kernel_re, path))
    return sum(per.values()) / len(per), len(per)


def summarize_pmc(fetch_csv: str, write_csv: str, out_path: str, command: str, mode: str = "asym",
                  grid_wgs: int | None = None) -> dict:
    kre = ROW_KERNEL_RE[mode]
    f_rows, n_f = _per_dispatch(fetch_csv, "FETCH_SIZE", kre, grid_wgs)
    w_rows, n_w = _per_dispatch(write_csv, "WRITE_SIZE", kre, grid_wgs)
    f_copy, _ = _per_dispatch(fetch_csv, "FETCH_SIZE", COPY_KERNEL_RE)
    w_copy, _ = _per_dispatch(write_csv, "WRITE_SIZE", COPY_KERNEL_RE)
    kib = 1024.0
    fetch_factor = f_copy * kib / COPY_BYTES     # counter bytes per true byte read
    write_factor = w_copy * kib / COPY_BYTES
    fetch_b = f_rows * kib / fetch_factor
    write_b = w_rows * kib / write_factor
    res = {"mode": mode, "kernel_regex": kre, "grid_workgroups": grid_wgs, "source_hash": source_hash(mode),
           "fetch_kib_per_dispatch": f_rows, "write_kib_per_dispatch": w_rows,
           "dispatches_fetch": n_f, "dispatches_write": n_w,
           "copy_bytes": COPY_BYTES, "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
           "fetch_factor": fetch_factor, "write_factor": write_factor,
           "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
           "traffic_bytes_per_launch": fetch_b + write_b}
    lines = ["# HBM traffic of the row kernel from rocprofv3 counters", "",
             "command: " + command, ""]
    lines += ["%s: %s" % (k, v) for k, v in res.items()]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return res


SQ_COUNTERS = ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU",
               "SQ_INSTS_SALU", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "GRBM_GUI_ACTIVE")
N_SIMD = 256 * 4      # compute units x SIMDs
N_XCD = 8             # GRBM_GUI_ACTIVE is summed over the accelerator complex dies


def summarize_sq(sq_csv: str, out_path: str, command: str, mode: str = "asym", grid_wgs: int | None = None) -> dict:
    """Instruction-issue counters of the row kernel, per dispatch, and the
    VALU busy fraction: SQ_ACTIVE_INST_VALU counts quad-cycles (one per
    wave64 VALU instruction on a 16-lane SIMD, more for transcendentals),
    summed over all SIMDs; GRBM_GUI_ACTIVE counts busy cycles per die."""
    kre = ROW_KERNEL_RE[mode]
    res = {"mode": mode, "kernel_regex": kre, "grid_workgroups": grid_wgs, "source_hash": source_hash(mode)}
    n = 0
    for c in SQ_COUNTERS:
        v, n = _per_dispatch(sq_csv, c, kre, grid_wgs)
        res[c] = v
    res["dispatches"] = n
    cycles = res["GRBM_GUI_ACTIVE"] / N_XCD
    valu_cycles = res["SQ_ACTIVE_INST_VALU"] * 4.0 / N_SIMD
    res["kernel_cycles"] = cycles
    res["valu_cycles_per_simd"] = valu_cycles
    res["valu_busy"] = valu_cycles / cycles
    res["valu_cycles_per_inst"] = 4.0 * res["SQ_ACTIVE_INST_VALU"] / res["SQ_INSTS_VALU"]
    lines = ["# VALU issue of the row kernel from rocprofv3 SQ counters", "",
             "command: " + command, ""]
    lines += ["%s: %s" % (k, v) for k, v in res.items()]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return res


def _trace_durations(trace_csv: str, kernel_re: str, grid_wgs: int):
    d = []
    for r in _rows(trace_csv):
        if not re.search(kernel_re, short_name(r["Kernel_Name"])):
            continue
        if int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])) != grid_wgs:
            continue
        d.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return d


def summarize_kernel(trace_csv: str, fetch_csv: str, write_csv: str, sq_csv: str, out_path: str, command: str,
                     kernel_re: str, grid_wgs: int, algorithmic_bytes: float, what: str) -> dict:
    """One kernel at one launch shape (a workload): its duration from the
    kernel trace, its HBM traffic (FETCH_SIZE and WRITE_SIZE per dispatch,
    scaled by what the same counters read for the calibration copy of
    COPY_BYTES in the same runs) against its algorithmic bytes, and its
    instruction-issue counters (VALU busy as in summarize_sq)."""
    d = sorted(_trace_durations(trace_csv, kernel_re, grid_wgs))
    f_k, n_f = _per_dispatch(fetch_csv, "FETCH_SIZE", kernel_re, grid_wgs)
    w_k, n_w = _per_dispatch(write_csv, "WRITE_SIZE", kernel_re, grid_wgs)
    f_copy, _ = _per_dispatch(fetch_csv, "FETCH_SIZE", COPY_KERNEL_RE)
    w_copy, _ = _per_dispatch(write_csv, "WRITE_SIZE", COPY_KERNEL_RE)
    kib = 1024.0
    fetch_b = f_k * kib / (f_copy * kib / COPY_BYTES)
    write_b = w_k * kib / (w_copy * kib / COPY_BYTES)
    res = {"kernel_regex": kernel_re, "grid_workgroups": grid_wgs, "workload": what,
           "trace_launches": len(d), "avg_us": sum(d) / len(d), "median_us": d[len(d) // 2],
           "algorithmic_bytes_per_launch": algorithmic_bytes,
           "algorithmic_gbs_at_avg": algorithmic_bytes / (sum(d) / len(d) * 1e-6) / 1e9,
           "fetch_kib_per_dispatch": f_k, "write_kib_per_dispatch": w_k, "dispatches_fetch": n_f,
           "dispatches_write": n_w, "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
           "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
           "traffic_bytes_per_launch": fetch_b + write_b,
           "traffic_over_algorithmic": (fetch_b + write_b) / algorithmic_bytes}
    for c in SQ_COUNTERS:
        res[c], n = _per_dispatch(sq_csv, c, kernel_re, grid_wgs)
    cycles = res["GRBM_GUI_ACTIVE"] / N_XCD
    res["valu_busy"] = res["SQ_ACTIVE_INST_VALU"] * 4.0 / N_SIMD / cycles
    res["valu_cycles_per_inst"] = 4.0 * res["SQ_ACTIVE_INST_VALU"] / res["SQ_INSTS_VALU"]
    lines = ["# %s: duration, HBM traffic and instruction issue from rocprofv3" % what, "",
             "command: " + command, ""]
    lines += ["%s: %s" % (k, v) for k, v in res.items()]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return res


def read_summary(path: str, mode: str = "asym"):
    """Key/value pairs of a counter summary, or None when the file is missing
    or the kernel sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ": " in line and not line.startswith("#"):
                k, v = line.rstrip("\n").split(": ", 1)
                kv[k] = v
    if kv.get("source_hash") != source_hash(mode) or kv.get("mode") != mode:
        return None
    return kv


def read_traffic(path: str, mode: str = "asym"):
    """Traffic bytes per launch recorded in a summary, or None when the file
    is missing or the kernel sources changed since it was taken."""
    kv = read_summary(path, mode)
    return None if kv is None else float(kv["traffic_bytes_per_launch"])


def summarize_counters(csv_path: str, out_path: str, command: str, kernel_re: str, workload: str) -> dict:
    """Every counter of one --pmc run, per dispatch of the kernels matching
    kernel_re (summed over its instances within a dispatch, averaged over
    the dispatches), with the derived rates the counters allow: the L2 hit
    fraction (TCC_HIT_sum, TCC_MISS_sum), the texture addressers' busy
    fraction (TA_BUSY_avr over GRBM_GUI_ACTIVE / 8 dies) and the matrix
    cores' busy fraction (SQ_VALU_MFMA_BUSY_CYCLES per SIMD over the same)."""
    names = sorted({_col(r, "Counter_Name") for r in _rows(csv_path)})
    out = {"kernel_regex": kernel_re, "workload": workload}
    for n in names:
        try:
            out[n], out["dispatches"] = _per_dispatch(csv_path, n, kernel_re)
        except ValueError:
            pass
    if "TCC_HIT_sum" in out and "TCC_MISS_sum" in out:
        out["l2_hit_fraction"] = out["TCC_HIT_sum"] / max(1.0, out["TCC_HIT_sum"] + out["TCC_MISS_sum"])
        out["l2_line_requests"] = out["TCC_HIT_sum"] + out["TCC_MISS_sum"]
    if "GRBM_GUI_ACTIVE" in out:
        die_cycles = out["GRBM_GUI_ACTIVE"] / 8.0
        out["die_cycles"] = die_cycles
        if "TA_BUSY_avr" in out:
            out["ta_busy"] = out["TA_BUSY_avr"] / die_cycles
        if "SQ_VALU_MFMA_BUSY_CYCLES" in out:
            out["mfma_busy"] = out["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024.0 / die_cycles
    lines = ["# %s: counters per dispatch from rocprofv3" % workload, "", "command: " + command, ""]
    lines += ["%s: %s" % (k, v) for k, v in out.items()]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out


def _grid_arg(argv):
    """An optional leading --grid=N (workgroups of the launches to keep)."""
    if argv and argv[0].startswith("--grid="):
        return int(argv[0].split("=", 1)[1]), argv[1:]
    return None, argv


def main(argv):
    if len(argv) >= 4 and argv[0] == "stats":
        summarize_stats(argv[1], argv[3], " ".join(argv[4:]), trace_csv=argv[2])
    elif len(argv) >= 4 and argv[0] == "pmc":
        grid, rest = _grid_arg(argv[4:])
        print(summarize_pmc(argv[1], argv[2], argv[3], " ".join(rest), grid_wgs=grid))
    elif len(argv) >= 3 and argv[0] == "sq":
        grid, rest = _grid_arg(argv[3:])
        print(summarize_sq(argv[1], argv[2], " ".join(rest), grid_wgs=grid))
    elif len(argv) >= 5 and argv[0] == "counters":
        print(summarize_counters(argv[1], argv[2], " ".join(argv[5:]), argv[3], argv[4]))
    elif len(argv) >= 10 and argv[0] == "kernel":
        print(summarize_kernel(argv[1], argv[2], argv[3], argv[4], argv[5], " ".join(argv[10:]), argv[6],
                               int(argv[7]), float(argv[8]), argv[9]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
