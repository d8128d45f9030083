"""Turn rocprofv3 output into the short summaries kept under profiles/.

  python -m gated_delta_rule_prep_amd.prof_summary stats <kernel_stats.csv> [title]
      markdown table of the --stats kernel summary.
  python -m gated_delta_rule_prep_amd.prof_summary traffic <workload> <fetch_dir> <write_dir> <copy_bytes>
      per-kernel HBM bytes per dispatch from a FETCH_SIZE pass and a WRITE_SIZE
      pass (counter_collection.csv under each directory).  Both counters are in
      KiB per dispatch; each is scaled by what it reads for the plain copy of
      copy_bytes bytes that bench.py --copy-mib runs after the workload (the
      copy reads and writes exactly copy_bytes), so that the figures are bytes.
      Prints one JSON object: {"workload", "scale", "kernels": {name: {fetch,
      write}}, "source_hash"}.
  python -m gated_delta_rule_prep_amd.prof_summary counters <kernel> <units> <dir>...
      mean per dispatch of every counter the passes under the directories
      collected for <kernel> (short name, e.g. recur_kernel), and that mean
      divided by <units> (the work units of one dispatch, e.g. workgroup
      chunk steps); prints one JSON object {counter: [per dispatch, per unit]}.

The source hash covers the code of the kernels' HIP sources and headers
(comments and layout left out), so a reader (bench.py) can tell whether the
counters still describe the current kernels.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["csrc/kda_device.h", "csrc/kda_internal.h", "csrc/kda_lds_pipe.h", "csrc/kda_step16.h",
                  "csrc/kda_sched.hip", "csrc/kda_prep.hip", "csrc/kda_recur.hip", "csrc/kda_prep32.hip",
                  "csrc/kda_recur32.hip", "csrc/kda_prep64.hip", "csrc/kda_recur64.hip", "csrc/kda_fused.hip",
                  "csrc/kda_decode.hip", "csrc/kda_segment.hip", "../include/kda.h"]


_TOKEN = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def code_only(text: str) -> str:
    """The source with its comments removed and each run of white space
    made one space (string and character literals kept as they are)."""
    text = _TOKEN.sub(lambda m: " " if m.group(0).startswith("/") else m.group(0), text)
    return " ".join(text.split())


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), encoding="utf-8") as f:
            h.update(rel.encode() + b"\0" + code_only(f.read()).encode())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    m = re.search(r"(sched_kernel|prep32_kernel|prep64_kernel|prep_kernel|recur32_kernel|recur64_kernel|recur_kernel|fused_kernel|decode_kernel|"
                  r"seg_cu_kernel|identity_kernel|zero_kernel|prefix_kernel|copyBuffer|elementwise_kernel)",
                  name)
    return m.group(1) if m else name[:40]


def stats_name(name: str) -> str:
    """short_name with the template arguments, which tell tile shapes apart
    (recur_kernel<WC, LD, PV>)."""
    t = re.search(r"_kernel(<[^>]*>)", name)
    return short_name(name) + (t.group(1).replace(" ", "") if t else "")


def counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def per_dispatch(rows, counter):
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def copy_value(vals, expect_kib):
    """The copy dispatches are the copyBuffer ones whose counter is within a
    factor 4 of the copy size (input uploads are far smaller)."""
    c = [v for v in vals.get("copyBuffer", []) if expect_kib / 4 <= v <= expect_kib * 4]
    if not c:
        raise SystemExit("no copy dispatch of the expected size")
    return statistics.median(c)


def traffic(workload, fetch_dir, write_dir, copy_bytes):
    f = per_dispatch(counter_rows(fetch_dir), "FETCH_SIZE")
    w = per_dispatch(counter_rows(write_dir), "WRITE_SIZE")
    kib = copy_bytes / 1024.0
    fs = copy_bytes / copy_value(f, kib)   # bytes per counter unit
    ws = copy_bytes / copy_value(w, kib)
    kernels = {}
    for k in ("sched_kernel", "prep_kernel", "recur_kernel", "prep32_kernel", "recur32_kernel", "prep64_kernel",
              "recur64_kernel", "fused_kernel", "decode_kernel"):
        if k in f and k in w:
            kernels[k] = {"fetch_bytes": int(statistics.median(f[k]) * fs),
                          "write_bytes": int(statistics.median(w[k]) * ws), "dispatches": len(f[k])}
    return {"workload": workload, "scale": {"fetch_bytes_per_unit": fs, "write_bytes_per_unit": ws},
            "kernels": kernels, "source_hash": source_hash()}


def counters(kernel, units, dirs):
    vals = {}
    for d in dirs:
        for r in counter_rows(d):
            if short_name(r["Kernel_Name"]) == kernel:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {c: [statistics.mean(v), statistics.mean(v) / units] for c, v in sorted(vals.items())}


def stats(path, title=""):
    with open(path) as fh:
        rows = list(csv.DictReader(fh))
    lines = ["| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.1f %% |" % (
            stats_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return ("### " + title + "\n\n" if title else "") + "\n".join(lines)


def main(argv):
    if len(argv) >= 2 and argv[1] == "stats":
        print(stats(argv[2], argv[3] if len(argv) > 3 else ""))
    elif len(argv) == 6 and argv[1] == "traffic":
        print(json.dumps(traffic(argv[2], argv[3], argv[4], int(argv[5]))))
    elif len(argv) >= 5 and argv[1] == "counters":
        print(json.dumps(counters(argv[2], float(argv[3]), argv[4:])))
    elif len(argv) == 2 and argv[1] == "hash":
        print(source_hash())
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
