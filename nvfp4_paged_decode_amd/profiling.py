"""Summaries of rocprofv3 output for the kernels of this library.

Three commands, each printing a short text summary (to stdout or --out):

  python -m nvfp4_paged_decode_amd.profiling stats DIR [--command TEXT]
      per-kernel dispatch count and average/min/max duration from a
      `rocprofv3 --kernel-trace --stats --output-format csv -d DIR` run.

  python -m nvfp4_paged_decode_amd.profiling counters --fetch DIR --write DIR
          --workload NAME [--yardstick-bytes N] [--command TEXT]
      HBM traffic per dispatch from two `rocprofv3 --pmc` runs (FETCH_SIZE,
      then WRITE_SIZE; both counters report KiB per dispatch).  Each counter
      is scaled by what it reads for the benchmark's plain streams, which
      nothing else launches: FETCH_SIZE by the read stream (N bytes read per
      dispatch), WRITE_SIZE by the write stream (N bytes written), averaged
      over their dispatches, so the result is in true bytes.  The
      summary ends with one `traffic` line per benchmark leg, which bench.py
      reads back together with the digest of that leg's kernel sources the
      counters were taken on (a figure for other sources is not reported).

  python -m nvfp4_paged_decode_amd.profiling pmc DIR [DIR ...] [--command TEXT]
      per-kernel wave occupancy and issue picture from `rocprofv3 --pmc`
      runs of the PMC_PASSES counter sets: shares of wave-cycles waiting,
      issuing, on VALU and on LDS, MFMA-busy share of all SIMDs, and LDS
      cycles lost to bank conflicts.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")


#: Kernel sources each benchmark leg's kernels are compiled from (the
#: launchers that set their grids included).
LEG_SOURCES = {
    "sort": ("order.hip", "common.hpp"),
    "quantize": ("codec.hip", "common.hpp"),
    "dequantize": ("codec.hip", "common.hpp"),
    "append": ("codec.hip", "common.hpp"),
    "gather": ("codec.hip", "common.hpp"),
    "decode": ("decode.hip", "decode_gqa.hip", "decode_gqa_mfma.hip", "decode_mla.hip",
               "decode_plan.hpp", "common.hpp"),
}


def source_digest(leg: str | None = None) -> str:
    """sha256 over the kernel sources of `leg` (all of them for None): file
    names and contents, sorted."""
    names = LEG_SOURCES[leg] if leg else [n for n in os.listdir(CSRC)
                                          if n.endswith((".hip", ".hpp", ".h"))]
    h = hashlib.sha256()
    for name in sorted(names):
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    n = re.sub(r"(kvfp4::)?\(anonymous namespace\)::", "", name)
    n = n.replace("void ", "")
    if "copyBuffer" in n:
        return "copyBuffer"
    if "reduce_kernel" in n:
        return "torch_reduce"
    if "FillFunctor" in n:
        return "torch_fill"
    return n.split("(")[0].strip()


def leg_of(kernel: str) -> str | None:
    """Benchmark leg a kernel belongs to."""
    if kernel.startswith(("quantize_kernel", "quantize_rounds_kernel")):
        return "quantize"
    if kernel.startswith("sort_pages_kernel"):
        return "sort"
    if kernel.startswith("dequantize_kernel"):
        return "dequantize"
    if kernel.startswith("append_kernel"):
        return "append"
    if kernel.startswith("gather_kernel"):
        return "gather"
    if kernel.startswith(("decode_", "merge_")):
        return "decode"
    return None


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def stats(d: str) -> list[str]:
    rows = list(csv.DictReader(open(_find(d, "kernel_stats.csv"))))
    out = [f"{'kernel':<52} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'share%':>7}"]
    for r in rows:
        out.append(f"{short_name(r['Name'])[:52]:<52} {int(r['Calls']):>6} "
                   f"{float(r['AverageNs']) / 1e3:>10.2f} {float(r['MinNs']) / 1e3:>10.2f} "
                   f"{float(r['MaxNs']) / 1e3:>10.2f} {float(r['Percentage']):>7.2f}")
    return out


def _counter(d: str, counter: str) -> dict[str, list[float]]:
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] == counter:
            per[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return per


#: The benchmark's plain streams (libkvfp4_yardstick.so): each dispatch of
#: READ_STREAM reads, and each of WRITE_STREAM writes, the yardstick size.
READ_STREAM, WRITE_STREAM = "read_kernel<8>", "write_kernel<4>"


def counters(fetch_dir: str, write_dir: str, yardstick_bytes: int, workload: str) -> list[str]:
    fetch = _counter(fetch_dir, "FETCH_SIZE")
    write = _counter(write_dir, "WRITE_SIZE")
    if READ_STREAM not in fetch or WRITE_STREAM not in write:
        raise SystemExit("no read / write stream dispatches to calibrate against")
    f_kib = sum(fetch[READ_STREAM]) / len(fetch[READ_STREAM])
    w_kib = sum(write[WRITE_STREAM]) / len(write[WRITE_STREAM])
    f_cal = yardstick_bytes / (1024.0 * f_kib)
    w_cal = yardstick_bytes / (1024.0 * w_kib)
    out = [f"calibration: {READ_STREAM} reads {yardstick_bytes} B per dispatch, FETCH_SIZE "
           f"{f_kib:.0f} KiB ({len(fetch[READ_STREAM])} dispatches); {WRITE_STREAM} writes "
           f"{yardstick_bytes} B per dispatch, WRITE_SIZE {w_kib:.0f} KiB "
           f"({len(write[WRITE_STREAM])} dispatches)",
           f"scale: fetch x{f_cal:.4f}, write x{w_cal:.4f} (bytes per counter KiB / 1024)",
           "",
           f"{'kernel':<44} {'disp':>5} {'FETCH_KiB':>12} {'WRITE_KiB':>12} {'read_B':>14} {'written_B':>14}"]
    legs = collections.defaultdict(lambda: [0.0, 0.0])
    for k in sorted(set(fetch) | set(write)):
        fv, wv = fetch.get(k, [0.0]), write.get(k, [0.0])
        fa, wa = sum(fv) / len(fv), sum(wv) / len(wv)
        rb, wb = fa * 1024 * f_cal, wa * 1024 * w_cal
        out.append(f"{k[:44]:<44} {len(fv):>5} {fa:>12.0f} {wa:>12.0f} {rb:>14.0f} {wb:>14.0f}")
        leg = leg_of(k)
        if leg:
            legs[leg][0] += rb
            legs[leg][1] += wb
    out.append("")
    for leg, (rb, wb) in sorted(legs.items()):
        out.append(f"traffic workload={workload} leg={leg} read_bytes={rb:.0f} "
                   f"written_bytes={wb:.0f} total_bytes={rb + wb:.0f} "
                   f"sources={source_digest(leg)}")
    return out


#: Counter passes for the occupancy / issue picture of each kernel.  One
#: rocprofv3 --pmc run per pass (the SQ block collects at most 8 counters in
#: a run, GRBM 2).
PMC_PASSES = (
    ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
     "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"),
    ("SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS", "SQ_INSTS_LDS",
     "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_ACTIVE_INST_VMEM", "SQ_INST_CYCLES_VMEM_RD",
     "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE"),
)

#: SIMDs of an MI355X (256 CUs x 4), the denominator of MFMA busy cycles,
#: and its XCDs: rocprofv3 sums GRBM_GUI_ACTIVE over the 8 XCDs, so the
#: kernel's own cycle count is that sum over 8
SIMDS = 1024
XCDS = 8


def _all_counters(d: str) -> dict[str, dict[str, list[float]]]:
    """kernel -> counter -> per-dispatch values, from one --pmc run."""
    per: dict = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        per[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return per


def pmc(dirs: list[str], kernels_prefix=("decode_", "merge_", "quantize_", "dequantize_")):
    """Per-kernel averages of the PMC_PASSES counters (one directory per
    pass) and the fractions derived from them:

    wait%   SQ_WAIT_ANY / SQ_WAVE_CYCLES  (wave-cycles spent waiting on anything)
    issue%  SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES  (wave-cycles issuing)
    valu%   SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES
    lds%    SQ_ACTIVE_INST_LDS / SQ_WAVE_CYCLES
    mfma%   SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024
            SIMDs): MFMA pipes busy, as a share of every SIMD over the
            kernel's cycles
    bank%   SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS  (LDS cycles lost to
            bank conflicts per LDS-active cycle)
    """
    merged: dict = collections.defaultdict(dict)
    for d in dirs:
        for k, cs in _all_counters(d).items():
            for c, vals in cs.items():
                merged[k].setdefault(c, vals)
    out = [f"{'kernel':<40} {'disp':>4} {'wait%':>6} {'issue%':>6} {'valu%':>6} {'lds%':>6} "
           f"{'mfma%':>6} {'bank%':>6} {'waves':>8} {'gui_cyc':>9}"]

    def avg(cs, c):
        v = cs.get(c)
        return sum(v) / len(v) if v else None

    def pct(a, b):
        return f"{100.0 * a / b:6.1f}" if a is not None and b else f"{'-':>6}"

    raw = []
    for k in sorted(merged):
        if not k.startswith(kernels_prefix):
            continue
        cs = merged[k]
        wc = avg(cs, "SQ_WAVE_CYCLES")
        gui = avg(cs, "GRBM_GUI_ACTIVE")
        n = max(len(v) for v in cs.values())
        mfma_den = gui / XCDS * SIMDS if gui else None
        out.append(f"{k[:40]:<40} {n:>4} {pct(avg(cs, 'SQ_WAIT_ANY'), wc)} "
                   f"{pct(avg(cs, 'SQ_ACTIVE_INST_ANY'), wc)} "
                   f"{pct(avg(cs, 'SQ_ACTIVE_INST_VALU'), wc)} "
                   f"{pct(avg(cs, 'SQ_ACTIVE_INST_LDS'), wc)} "
                   f"{pct(avg(cs, 'SQ_VALU_MFMA_BUSY_CYCLES'), mfma_den)} "
                   f"{pct(avg(cs, 'SQ_LDS_BANK_CONFLICT'), avg(cs, 'SQ_ACTIVE_INST_LDS'))} "
                   f"{(avg(cs, 'SQ_WAVES') or 0):>8.0f} {(gui or 0):>9.0f}")
        raw.append(f"raw {k}: " + " ".join(f"{c}={avg(cs, c):.0f}" for c in sorted(cs)))
    return out + [""] + raw


def read_traffic(path: str, workload: str, leg: str) -> int | None:
    """Total HBM bytes per call of `leg`, if `path` holds a figure taken on
    the current kernel sources for this workload; else None."""
    if not os.path.exists(path):
        return None
    digest = source_digest(leg)
    for line in open(path):
        if not line.startswith("traffic "):
            continue
        kv = dict(p.split("=", 1) for p in line.split()[1:])
        if kv.get("workload") == workload and kv.get("leg") == leg and kv.get("sources") == digest:
            return int(kv["total_bytes"])
    return None


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--yardstick-bytes", type=int, default=1 << 30)
    c.add_argument("--workload", required=True)
    m = sub.add_parser("pmc")
    m.add_argument("dirs", nargs="+", help="one rocprofv3 --pmc output directory per pass")
    for q in (s, c, m):
        q.add_argument("--command", default="", help="the command(s) that produced DIR")
        q.add_argument("--out")
    a = p.parse_args(argv)
    if a.cmd == "stats":
        lines = stats(a.dir)
    elif a.cmd == "pmc":
        lines = pmc(a.dirs)
    else:
        lines = counters(a.fetch, a.write, a.yardstick_bytes, a.workload)
    head = [f"# {l}" for l in a.command.splitlines() if l.strip()]
    text = "\n".join(head + [""] + lines if head else lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
