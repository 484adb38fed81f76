"""Summaries of rocprofv3 output for the MSA kernels (text for profiles/, and the HBM
traffic table bench.py reports).

    python -m block_sparse_long_05_amd.profiling stats <kernel_stats.csv> [--cmd "..."]
    python -m block_sparse_long_05_amd.profiling traffic --fetch <dir> --write <dir>
            --copy-mib N --out <traffic.json> [--cmd "..."]
    python -m block_sparse_long_05_amd.profiling traffic-text <traffic.json> [--workloads "..."]

`traffic` reads the counter CSVs of two rocprofv3 --pmc runs (FETCH_SIZE, then
WRITE_SIZE, KiB per dispatch) taken with bench.py --copy-calibration-mib N, scales each
counter by what it reads for that plain N MiB device copy (read and written bytes are
known exactly), and stores bytes per launch for each MSA kernel together with a hash
of the kernel's source file.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# kernel-name fragment -> source files that define it (beyond the shared headers)
KERNEL_SOURCES = {
    "index_scores_prefill": ("index_scores.hip",),
    "index_scores_decode": ("index_scores.hip",),
    "index_topk": ("index_scores.hip",),
    "block_topk": ("block_topk.hip", "msa_select.h"),
    "kv_": ("attn_tile.hip",),
    "qtile_attn": ("attn_tile.hip",),
    "dense_attn": ("attn_tile.hip",),
    "gather_attn": ("attn_gather.hip",),
    "decode_combine": ("attn_gather.hip",),
    "kl_": ("index_kl.hip",),
    "decode_attn": ("decode_attn.hip", "msa_select.h"),
}
# device headers every kernel source includes: a change there can change any kernel
SHARED_HEADERS = ("msa_device.h", "msa_tile.h", "msa_launch.h")


def source_hash(kernel_name: str):
    """Hash of the kernel's source file and the shared device headers; None for a kernel
    this table does not know (its stored traffic is then never taken as current)."""
    for frag, src in KERNEL_SOURCES.items():
        if frag in kernel_name:
            h = hashlib.sha256()
            for f in src + SHARED_HEADERS:
                path = os.path.join(CSRC, f)
                if os.path.exists(path):
                    h.update(open(path, "rb").read())
            return h.hexdigest()[:16]
    return None


def short_name(name: str) -> str:
    base = name.split("(")[0].replace("void ", "").strip()
    if base.startswith("Cijk_"):  # a hipBLASLt GEMM kernel: its tile and MFMA shape suffice
        parts = [x for x in base.split("_") if x.startswith(("MT", "MI"))]
        return "hipBLASLt GEMM " + " ".join(parts[:2])
    return base


def stats_text(stats_csv: str, cmd: str = "") -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = ["rocprofv3 --kernel-trace --stats: MSA kernels (durations in microseconds)"]
    if cmd:
        out.append(f"command: {cmd}")
    out.append(f"{'calls':>6} {'avg_us':>11} {'min_us':>11} {'max_us':>11}  kernel")
    for r in rows:
        if "msa::" not in r["Name"]:
            continue
        out.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:11.1f} "
                   f"{float(r['MinNs']) / 1e3:11.1f} {float(r['MaxNs']) / 1e3:11.1f}  "
                   f"{short_name(r['Name'])}")
    return "\n".join(out) + "\n"


_per_dispatch = collections.defaultdict(lambda: collections.defaultdict(list))


def counter_means(directory: str) -> dict:
    """{kernel name: {counter: mean value per dispatch}} from a --pmc run's CSVs."""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = r.get("Kernel_Name") or ""
            ctr = r.get("Counter_Name")
            if ctr is None:
                continue
            agg[name][ctr].append(float(r["Counter_Value"]))
            _per_dispatch[ctr][name].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in agg.items()}


def _copy_value(means: dict, counter: str) -> float:
    # the runtime's device-to-device copy kernel; the calibration copy is its largest
    # dispatch in the run
    vals = [max(v) for name, v in _per_dispatch.get(counter, {}).items() if "copyBuffer" in name]
    if not vals:
        raise SystemExit(f"no copy kernel found for {counter}")
    return max(vals)  # the calibration copy is by far the largest dispatch


def bench_launches(log: str) -> dict:
    """{'prefill': ..., 'decode': ...}: the workload and launch configuration of each leg,
    from the JSON line bench.py printed in the profiled run."""
    line = [x for x in open(log).read().splitlines() if x.startswith("{")][-1]
    d = json.loads(line)
    return {k: d[k]["launch"] for k in ("prefill", "decode") if d.get(k)}


def traffic(fetch_dir: str, write_dir: str, copy_mib: float, cmd: str = "",
            bench_log: str = "") -> dict:
    fm, wm = counter_means(fetch_dir), counter_means(write_dir)
    copy_bytes = copy_mib * (1 << 20)
    f_copy = _copy_value(fm, "FETCH_SIZE") * 1024.0
    w_copy = _copy_value(wm, "WRITE_SIZE") * 1024.0
    fs, ws = copy_bytes / f_copy, copy_bytes / w_copy
    kernels = {}
    for name in sorted(set(fm) | set(wm)):
        if "msa::" not in name:
            continue
        rd = fm.get(name, {}).get("FETCH_SIZE")
        wr = wm.get(name, {}).get("WRITE_SIZE")
        kernels[short_name(name)] = dict(
            read_bytes=None if rd is None else rd * 1024.0 * fs,
            write_bytes=None if wr is None else wr * 1024.0 * ws,
            source_hash=source_hash(name))
    return dict(copy_mib=copy_mib, fetch_scale=fs, write_scale=ws, command=cmd,
                launches=bench_launches(bench_log) if bench_log else {}, kernels=kernels)


def traffic_text(t: dict, workloads: str = "") -> str:
    out = ["HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (two runs),",
           f"scaled by the same counters for a plain {t['copy_mib']:.0f} MiB device copy: "
           f"fetch x{t['fetch_scale']:.3f}, write x{t['write_scale']:.3f}"]
    if t.get("command"):
        out.append(f"command: {t['command']}")
    if workloads:
        out.append(f"workloads: {workloads}")
    out += ["", f"{'read_GB':>10} {'write_GB':>10}  kernel"]
    rows = sorted(t["kernels"].items(), key=lambda kv: -((kv[1]["read_bytes"] or 0) +
                                                       (kv[1]["write_bytes"] or 0)))
    for name, v in rows:
        out.append(f"{(v['read_bytes'] or 0) / 1e9:10.3f} {(v['write_bytes'] or 0) / 1e9:10.3f}  {name}")
    return "\n".join(out) + "\n"


def _agent(directory: str) -> dict:
    for f in glob.glob(os.path.join(directory, "**", "*agent_info.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Name", "").startswith("gfx"):
                return r
    return {}


def mfma_text(directory: str, cmd: str = "", min_ms: float = 0.1) -> str:
    """MFMA use per kernel from a --pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES
    SQ_INSTS_VALU_MFMA_MOPS_BF16 run: the shader clock the kernel ran at (GRBM_GUI_ACTIVE per
    XCD over the dispatch time), the fraction of SIMD cycles the matrix cores were busy
    (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x SIMDs): the profiler's MfmaUtil),
    and the bf16 MFMA FLOP/s the MOPS counter implies (512 FLOP per unit) against the spec
    peak and against the peak at the measured clock (CUs x 4096 bf16 FLOP per cycle)."""
    agent = _agent(directory)
    nxcc = int(agent.get("Num_Xcc", 8))
    simds = int(agent.get("Simd_Count", 1024))
    cus = int(agent.get("Cu_Count", 256))
    fmax = float(agent.get("Max_Engine_Clk_Fcompute", 2400)) * 1e6
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = short_name(r.get("Kernel_Name") or "")
            acc[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                acc[name]["_ns"].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    out = ["MFMA use per kernel from rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES "
           "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 (one run)",
           f"device: {agent.get('Name', '?')}, {cus} CUs, {simds} SIMDs, {nxcc} XCDs, "
           f"max shader clock {fmax / 1e9:.2f} GHz; bf16 peak {cus * 4096 * fmax / 1e12:.0f} "
           f"TFLOP/s at that clock"]
    if cmd:
        out.append(f"command: {cmd}")
    out += ["clock = GRBM_GUI_ACTIVE / XCDs / dispatch time; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES "
            "/ (GRBM_GUI_ACTIVE / XCDs x SIMDs); TF/s = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 / "
            "dispatch time; frac_at_clock = TF/s over CUs x 4096 x clock",
            "",
            f"{'calls':>5} {'avg_ms':>9} {'clock_GHz':>9} {'mfma_busy':>9} {'TF/s':>7} "
            f"{'frac_spec':>9} {'frac_at_clock':>13} {'bf16_FLOP':>10}  kernel"]
    rows = []
    for name, c in acc.items():
        if not c.get("_ns") or "GRBM_GUI_ACTIVE" not in c:
            continue
        ns = sum(c["_ns"]) / len(c["_ns"])
        if ns < min_ms * 1e6:
            continue
        g = sum(c["GRBM_GUI_ACTIVE"]) / len(c["GRBM_GUI_ACTIVE"]) / nxcc
        clk = g / (ns * 1e-9)
        busy = (sum(c.get("SQ_VALU_MFMA_BUSY_CYCLES", [0])) /
                max(1, len(c.get("SQ_VALU_MFMA_BUSY_CYCLES", [0])))) / (g * simds)
        mops = sum(c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0])) / max(
            1, len(c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0])))
        tf = 512.0 * mops / (ns * 1e-9) / 1e12
        rows.append((ns, len(c["_ns"]), clk, busy, tf, 512.0 * mops, name))
    for ns, n, clk, busy, tf, fl, name in sorted(rows, reverse=True):
        out.append(f"{n:5d} {ns / 1e6:9.3f} {clk / 1e9:9.2f} {busy:9.3f} {tf:7.0f} "
                   f"{tf * 1e12 / (cus * 4096 * fmax):9.3f} "
                   f"{(tf * 1e12 / (cus * 4096 * clk)) if clk > 0 else 0:13.3f} {fl:10.3e}  {name}")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--cmd", default="")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--copy-mib", type=float, required=True)
    b.add_argument("--out", required=True)
    b.add_argument("--cmd", default="")
    b.add_argument("--bench-log", default="",
                   help="output of the profiled bench.py run (its workloads and launches)")
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--cmd", default="")
    m.add_argument("--min-ms", type=float, default=0.1)
    c = sub.add_parser("traffic-text")
    c.add_argument("json")
    c.add_argument("--workloads", default="")
    args = ap.parse_args()
    if args.what == "stats":
        print(stats_text(args.csv, args.cmd), end="")
    elif args.what == "mfma":
        print(mfma_text(args.dir, args.cmd, args.min_ms), end="")
    elif args.what == "traffic-text":
        print(traffic_text(json.load(open(args.json)), args.workloads), end="")
    else:
        t = traffic(args.fetch, args.write, args.copy_mib, args.cmd, args.bench_log)
        with open(args.out, "w") as f:
            json.dump(t, f, indent=1)
        for k, v in t["kernels"].items():
            print(f"{k}: read {v['read_bytes']}, write {v['write_bytes']}")
        print(f"scale: fetch x{t['fetch_scale']:.3f}, write x{t['write_scale']:.3f}")


if __name__ == "__main__":
    main()
