"""Turn rocprofv3 output into the short text summaries kept under profiles/.

    python -m mamba_ssd_prefill_amd.profile_summary trace    <rocprof dir> <out.md> "<command>"
    python -m mamba_ssd_prefill_amd.profile_summary counters <rocprof dir> <out.md> "<command>"
    python -m mamba_ssd_prefill_amd.profile_summary metrics  <out.md> "<cmd1 ;; cmd2 ...>" <dir1> <dir2> ...
    python -m mamba_ssd_prefill_amd.profile_summary traffic <FETCH_SIZE dir> <WRITE_SIZE dir> \\
           <workload> <chunk> <out.json> "<fetch command>" "<write command>"

`trace` tabulates run_kernel_stats.csv of a --kernel-trace --stats run.  `traffic` reads
two --pmc runs of ``bench.py --counters`` (which first copies 1 GiB device to device) and
scales each counter so that the copy kernel reads and writes exactly 1 GiB; it writes the
HBM bytes per launch of the fused kernel, with the hash of the kernel sources it was taken
on (bench.py ignores a summary whose hash no longer matches).
"""
import csv
import glob
import json
import os
import subprocess
import sys

from .build import source_hash

GIB_KIB = 1024.0 * 1024.0  # 1 GiB in KiB (the counters' unit)


def _rows(d, name):
    paths = glob.glob(os.path.join(d, "**", name), recursive=True)
    if not paths:
        raise FileNotFoundError("no %s under %s" % (name, d))
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


def _demangle_ssd(name):
    """ssd:: kernel names from their Itanium mangling (the template forms used here only)."""
    if not name.startswith("_ZN3ssd"):
        return None
    i = len("_ZN3ssd")
    j = i
    while j < len(name) and name[j].isdigit():
        j += 1
    if j == i:
        return None
    n = int(name[i:j])
    out = "ssd::" + name[j:j + n]
    k = j + n
    if k < len(name) and name[k] == "I":
        k += 1
        args = []
        while k < len(name) and name[k] != "E":
            if name.startswith("DF16b", k):
                args.append("bf16")
                k += 5
            elif name.startswith("DF16_", k):
                args.append("f16")
                k += 5
            elif name[k] == "f":
                args.append("float")
                k += 1
            elif name.startswith("Lb0E", k) or name.startswith("Lb1E", k):
                args.append("packed" if name[k + 2] == "1" else "plain")
                k += 4
            elif name.startswith("Li", k):
                e = name.index("E", k)
                args.append(name[k + 2:e])
                k = e + 1
            else:
                return None
        out += "<" + ", ".join(args) + ">"
    return out


# rocprofv3 prints some names already demangled, and its demangler reads the __bf16 template
# argument followed by float (mangled "DF16bf") as "bool _Accum"
_GARBLED = {"ssd::k_decode<bool _Accum, ": "ssd::k_decode<bf16, float, "}


def short(name):
    """Demangled kernel name without its argument list."""
    for bad, good in _GARBLED.items():
        name = name.replace(bad, good)
    d = _demangle_ssd(name)
    if d:
        return d
    try:
        name = subprocess.run(["c++filt", name], capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        pass
    depth = 0
    for i, ch in enumerate(name):  # cut at the parameter list (the first '(' outside <...>)
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return name[:i]
    return name


def trace(d, out, command):
    rows = _rows(d, "*kernel_stats.csv")
    lines = ["# Kernel trace: %s" % os.path.basename(out).rsplit(".", 1)[0], "",
             "Command (from the repository root, on one MI355X):", "", "    " + command, "",
             "| kernel | calls | avg us | min us | max us | total % |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.1f |" % (
            short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_kernel(d, counter):
    acc = {}
    for r in _rows(d, "*counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def traffic(fetch_dir, write_dir, workload, chunk, out, fetch_cmd, write_cmd):
    f = _per_kernel(fetch_dir, "FETCH_SIZE")
    w = _per_kernel(write_dir, "WRITE_SIZE")
    copy = [k for k in f if "copyBuffer" in k]
    cf = GIB_KIB / max(max(f[k]) for k in copy)
    cw = GIB_KIB / max(max(w[k]) for k in copy if k in w)
    kernels = {}
    for k in f:
        if not k.startswith("_ZN3ssd") and "ssd::" not in k:
            continue
        fr = sum(f[k]) / len(f[k]) * cf * 1024
        wr = sum(w.get(k, [0.0])) / max(1, len(w.get(k, []))) * cw * 1024
        kernels[short(k)] = {"read_bytes": fr, "write_bytes": wr, "dispatches": len(f[k])}
    fused = [k for k in kernels if "k_fused" in k]
    res = {"workload": workload, "chunk_size": int(chunk), "kernel_source_hash": source_hash(),
           "calibration": {"fetch_scale": cf, "write_scale": cw,
                           "how": "1 GiB device-to-device copy measured in the same run"},
           "commands": [fetch_cmd, write_cmd], "kernels": kernels}
    if fused:
        k = kernels[fused[0]]
        res["kernel"] = fused[0]
        res["bytes_per_launch"] = k["read_bytes"] + k["write_bytes"]
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")


def counters(d, out, command):
    """Per-kernel averages of every counter of one --pmc run, with per-wave instruction counts
    (when SQ_WAVES was collected) or the share of wave cycles (when SQ_WAVE_CYCLES was)."""
    acc = {}
    for r in _rows(d, "*counter_collection.csv"):
        k = short(r["Kernel_Name"])
        if not k.startswith("ssd::"):
            continue
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for v in acc.values() for c in v})
    per_wave = [c for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS") if c in names and "SQ_WAVES" in names]
    shares = [c for c in names if "SQ_WAVE_CYCLES" in names and c.startswith(("SQ_WAIT", "SQ_ACTIVE"))]
    extra = ["%s per wave" % c[len("SQ_INSTS_"):] for c in per_wave] + ["%s share" % c[len("SQ_"):] for c in shares]
    if per_wave:
        note = "Average per dispatch; the `per wave` columns divide by SQ_WAVES."
    else:
        note = "Average per dispatch; the `share` columns divide by SQ_WAVE_CYCLES (the fraction of its life a wave spends so)."
    lines = ["# SQ counters: %s" % os.path.basename(out).rsplit(".", 1)[0], "",
             "Command (from the repository root, on one MI355X):", "", "    " + command, "", note, "",
             "| kernel | " + " | ".join(names + extra) + " |",
             "|---|" + "---:|" * (len(names) + len(extra))]
    for k, v in sorted(acc.items()):
        avg = {c: sum(x) / len(x) for c, x in v.items()}
        wv = avg.get("SQ_WAVES", 0.0) or 1.0
        wc = avg.get("SQ_WAVE_CYCLES", 0.0) or 1.0
        cells = ["%.4g" % avg.get(c, float("nan")) for c in names]
        cells += ["%.0f" % (avg.get(c, 0.0) / wv) for c in per_wave]
        cells += ["%.3f" % (avg.get(c, 0.0) / wc) for c in shares]
        lines.append("| %s | %s |" % (k, " | ".join(cells)))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def metrics(out, command, dirs):
    """Per-kernel averages of the counters of several --pmc runs (one directory each, same
    program), with the derived figures the counters define on gfx950:
      MFMA busy %   = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs) * 100
      occupancy %   = 4 * SQ_WAVE_CYCLES / (GRBM_GUI_ACTIVE * CUs * 32) * 100 (resident waves
                      per CU against the 32 a CU holds; SQ_WAVE_CYCLES counts in units of 4)
      L2 hit %      = TCC_HIT / (TCC_HIT + TCC_MISS) * 100
      LDS conflict  = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (conflict cycles per LDS cycle)
    GRBM_GUI_ACTIVE as collected here is the sum of the 8 XCDs' counters (each close to the
    kernel's duration in cycles), so it is divided by 8 first (rocprofv3's own derived metrics
    take the largest XCD's value instead)."""
    acc = {}
    for d in dirs:
        for r in _rows(d, "*counter_collection.csv"):
            k = short(r["Kernel_Name"])
            if not k.startswith("ssd::"):
                continue
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    cus, simds = 256, 1024
    names = sorted({c for v in acc.values() for c in v})
    lines = ["# Counters: %s" % os.path.basename(out).rsplit(".", 1)[0], "",
             "Commands (from the repository root, on one MI355X), one --pmc pass each:", ""]
    lines += ["    " + c for c in command.split(" ;; ")]
    lines += ["", "Average per dispatch.", "",
              "| kernel | " + " | ".join(names) + " | MFMA busy % | occupancy % | L2 hit % | LDS conflict / LDS cycle |",
              "|---|" + "---:|" * (len(names) + 4)]
    for k, v in sorted(acc.items()):
        a = {c: sum(x) / len(x) for c, x in v.items()}
        g = a.get("GRBM_GUI_ACTIVE")
        g = g / 8.0 if g else g
        mf = 100 * a["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * simds) if g and "SQ_VALU_MFMA_BUSY_CYCLES" in a else None
        oc = 100 * 4 * a["SQ_WAVE_CYCLES"] / (g * cus * 32) if g and "SQ_WAVE_CYCLES" in a else None
        hm = a.get("TCC_HIT_sum", 0.0) + a.get("TCC_MISS_sum", 0.0)
        l2 = 100 * a["TCC_HIT_sum"] / hm if hm else None
        lc = (a["SQ_LDS_BANK_CONFLICT"] / a["SQ_LDS_IDX_ACTIVE"]) if a.get("SQ_LDS_IDX_ACTIVE") else None
        f = lambda x, fmt: "-" if x is None else fmt % x  # noqa: E731
        cells = ["%.4g" % a[c] if c in a else "-" for c in names]
        cells += [f(mf, "%.1f"), f(oc, "%.1f"), f(l2, "%.1f"), f(lc, "%.3f")]
        lines.append("| %s | %s |" % (k, " | ".join(cells)))
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main(argv):
    if len(argv) >= 4 and argv[0] == "trace":
        trace(argv[1], argv[2], argv[3])
    elif len(argv) >= 4 and argv[0] == "counters":
        counters(argv[1], argv[2], argv[3])
    elif len(argv) >= 4 and argv[0] == "metrics":
        metrics(argv[1], argv[2], argv[3:])
    elif len(argv) >= 8 and argv[0] == "traffic":
        traffic(*argv[1:8])
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
