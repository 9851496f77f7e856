"""Summaries of rocprofv3 CSV output for the kernels of this library.

    python -m gguf_block_quantized_qmv_amd.rocprof_summary trace DIR [--kernel NAME] [--per-step N] [--window A:B]
    python -m gguf_block_quantized_qmv_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR --kernel NAME \
        --read-bytes B [--read-pick median|max] [--copy-bytes C] [--algo-bytes A]
    python -m gguf_block_quantized_qmv_amd.rocprof_summary mfma DIR --kernel NAME [--flops F] [--simds S]
    python -m gguf_block_quantized_qmv_amd.rocprof_summary counters DIR [DIR ...] --kernel NAME [--ratio A/B ...]

DIR is a rocprofv3 output directory (`-d DIR -f csv`): `trace` reads its
*_kernel_trace.csv (run with --kernel-trace), `traffic` and `mfma` its
*_counter_collection.csv (run with --pmc). Each prints a Markdown table.

trace    per (kernel, grid, workgroup) group: dispatches and the mean, median,
         min and max duration; with --per-step N the kernel time of N
         dispatches at the median and the mean (one step of N launches);
         --window A:B keeps only the matching dispatches A..B-1 in dispatch
         order (e.g. one timed region of a run).
traffic  HBM bytes per dispatch from a FETCH_SIZE pass and a WRITE_SIZE pass,
         each scaled to bytes by a dispatch of known size in the same pass:
         FETCH_SIZE by the streaming-read kernel over --read-bytes bytes (its
         median dispatch, or with --read-pick max its largest), and
         WRITE_SIZE by the runtime's device copy of --copy-bytes bytes.
mfma     MFMA utilisation per dispatch: SQ_VALU_MFMA_BUSY_CYCLES (summed over
         SIMDs) / (active cycles * SIMDs), the active cycles being
         GRBM_GUI_ACTIVE over the --xcds instances it is summed across (the
         implied clock, active cycles / duration, is printed as a check), and
         the bf16 MFMA work from SQ_INSTS_VALU_MFMA_MOPS_BF16 (units of 512
         flops), checked against --flops when given.
counters per (kernel, grid, workgroup) group over one or more --pmc passes:
         the median of every counter collected, and each --ratio A/B as the
         ratio of the two medians (A and B counter names from any pass).
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import statistics
import sys


def short_name(name: str) -> str:
    """Kernel name without its namespace prefix, return type and argument list."""
    import re
    name = re.sub(r"^void ", "", name)
    name = name.replace("qmv::(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in name:          # drop the top-level argument list, keep template arguments
        if ch == "(" and depth == 0 and out and not out[-1].endswith("operator"):
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out)


def _csv(directory: str, suffix: str):
    paths = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not paths:
        raise SystemExit(f"no *{suffix} under {directory}")
    rows = []
    for p in paths:
        with open(p, newline="") as f:
            rows.extend(csv.DictReader(f))
    for r in rows:
        r["Kernel_Name"] = short_name(r["Kernel_Name"])
    return rows


def _grid(r) -> int:
    if "Grid_Size" in r:
        return int(r["Grid_Size"])
    return int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])


def _wg(r) -> int:
    if "Workgroup_Size" in r:
        return int(r["Workgroup_Size"])
    return int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])


def trace(args) -> None:
    rows = [r for r in _csv(args.dir, "kernel_trace.csv") if not args.kernel or args.kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    if args.window:
        a, b = (int(v) if v else None for v in args.window.split(":"))
        rows = rows[a:b]
    groups = collections.OrderedDict()
    for r in rows:
        key = (r["Kernel_Name"], _grid(r) // max(1, _wg(r)), _wg(r))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("| kernel | workgroups | threads | dispatches | mean ns | median ns | min ns | max ns |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|")
    alld = []
    for (name, nwg, wg), d in groups.items():
        alld += d
        print(f"| {name} | {nwg} | {wg} | {len(d)} | {statistics.fmean(d):.0f} | {statistics.median(d):.0f} | "
              f"{min(d)} | {max(d)} |")
    if alld:
        print(f"\nAll {len(alld)} dispatches: mean {statistics.fmean(alld):.0f} ns, median "
              f"{statistics.median(alld):.0f} ns.")
    if args.per_step and alld:
        n = args.per_step
        share = {k: len(v) / len(alld) for k, v in groups.items()}
        med = sum(share[k] * n * statistics.median(v) for k, v in groups.items())
        mean = sum(share[k] * n * statistics.fmean(v) for k, v in groups.items())
        print(f"Kernel time of one step of {n} dispatches (each group in its share of the dispatches): "
              f"{med / 1e6:.4f} ms at the group medians, {mean / 1e6:.4f} ms at the group means.")


def _counter(rows, name):
    return [r for r in rows if r["Counter_Name"] == name]


def _by_group(rows, kernel):
    g = collections.OrderedDict()
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        if kernel in r["Kernel_Name"]:
            key = (r["Kernel_Name"], _grid(r) // max(1, _wg(r)), _wg(r))
            g.setdefault(key, []).append(float(r["Counter_Value"]))
    return g


def traffic(args) -> None:
    fetch = _counter(_csv(args.fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    write = _counter(_csv(args.write_dir, "counter_collection.csv"), "WRITE_SIZE")
    rd = [float(r["Counter_Value"]) for r in fetch if "stream_read_kernel" in r["Kernel_Name"]]
    cp = [float(r["Counter_Value"]) for r in write if "copyBuffer" in r["Kernel_Name"]]
    if not rd:
        raise SystemExit("no stream_read_kernel dispatch in the FETCH_SIZE pass to scale it by")
    ref = max(rd) if args.read_pick == "max" else statistics.median(rd)
    f_scale = args.read_bytes / (ref * 1024)
    print(f"FETCH_SIZE scale: the streaming read of {args.read_bytes} B reads {ref:.1f} KiB "
          f"({args.read_pick} of {len(rd)}), x {f_scale:.4f} to bytes.")
    if cp:
        w_scale = args.copy_bytes / (max(cp) * 1024)
        print(f"WRITE_SIZE scale: the {args.copy_bytes} B device copy writes {max(cp):.1f} KiB, x {w_scale:.4f} to bytes.")
    else:
        w_scale = 1.0
        print("WRITE_SIZE scale: no device copy in the pass, taken as x 1.0 (KiB of 1024 B).")
    gf, gw = _by_group(fetch, args.kernel), _by_group(write, args.kernel)
    print()
    print("| kernel | workgroups x threads | dispatches | FETCH_SIZE KiB (median) | WRITE_SIZE KiB (median) | "
          "HBM bytes | x algorithmic |")
    print("|---|---|---:|---:|---:|---:|---:|")
    for key, fv in gf.items():
        wv = gw.get(key, [])
        f = statistics.median(fv)
        w = statistics.median(wv) if wv else float("nan")
        hbm = f * 1024 * f_scale + (w * 1024 * w_scale if wv else 0.0)
        ratio = f"{hbm / args.algo_bytes:.4f}" if args.algo_bytes else "-"
        print(f"| {key[0]} | {key[1]} x {key[2]} | {len(fv)} | {f:.1f} | {w:.1f} | {hbm:.0f} | {ratio} |")


def mfma(args) -> None:
    rows = _csv(args.dir, "counter_collection.csv")
    per = collections.OrderedDict()
    for r in rows:
        if args.kernel in r["Kernel_Name"]:
            d = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "wg": _wg(r),
                                                        "nwg": _grid(r) // max(1, _wg(r)),
                                                        "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of {args.kernel}")
    groups = collections.OrderedDict()
    for d in per.values():
        groups.setdefault((d["name"], d["nwg"], d["wg"]), []).append(d)
    print("| kernel | workgroups x threads | dispatches | duration ns (median) | MFMA busy (SIMD-cycles) | "
          "GRBM_GUI_ACTIVE | implied clock GHz | MFMA util | bf16 MFMA flops | vs expected |")
    print("|---|---|---:|---:|---:|---:|---:|---:|---:|---:|")
    for key, ds in groups.items():
        ns = statistics.median(d["ns"] for d in ds)
        busy = statistics.median(d.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) for d in ds)
        gui = statistics.median(d.get("GRBM_GUI_ACTIVE", float("nan")) for d in ds)
        mops = statistics.median(d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", float("nan")) for d in ds)
        active = gui / args.xcds
        util = busy / (active * args.simds) if gui else float("nan")
        flops = mops * 512
        vs = f"{flops / args.flops:.4f}" if args.flops else "-"
        print(f"| {key[0]} | {key[1]} x {key[2]} | {len(ds)} | {ns:.0f} | {busy:.4g} | {gui:.4g} | "
              f"{active / ns:.3f} | {util:.4f} | {flops:.4g} | {vs} |")
    extra = sorted({c for d in per.values() for c in d} - {"name", "wg", "nwg", "ns", "SQ_VALU_MFMA_BUSY_CYCLES",
                                                             "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16"})
    if extra:
        print()
        print("| kernel | workgroups x threads | " + " | ".join(extra) + " |")
        print("|---|---|" + "---:|" * len(extra))
        for key, ds in groups.items():
            vals = [statistics.median(d.get(c, float("nan")) for d in ds) for c in extra]
            print(f"| {key[0]} | {key[1]} x {key[2]} | " + " | ".join(f"{v:.4g}" for v in vals) + " |")


def counters(args) -> None:
    groups = collections.OrderedDict()
    for d in args.dirs:
        for r in _csv(d, "counter_collection.csv"):
            if args.kernel in r["Kernel_Name"]:
                key = (short_name(r["Kernel_Name"]), _grid(r) // max(1, _wg(r)), _wg(r))
                groups.setdefault(key, collections.defaultdict(list))[r["Counter_Name"]].append(
                    float(r["Counter_Value"]))
    if not groups:
        raise SystemExit(f"no dispatch of {args.kernel}")
    names = sorted({c for g in groups.values() for c in g})
    print("| kernel | workgroups x threads | " + " | ".join(names) + " |")
    print("|---|---|" + "---:|" * len(names))
    for key, g in groups.items():
        vals = [f"{statistics.median(g[c]):.4g}" if g.get(c) else "-" for c in names]
        print(f"| {key[0]} | {key[1]} x {key[2]} | " + " | ".join(vals) + " |")
    if args.ratio:
        print()
        print("| kernel | workgroups x threads | " + " | ".join(args.ratio) + " |")
        print("|---|---|" + "---:|" * len(args.ratio))
        for key, g in groups.items():
            out = []
            for rt in args.ratio:
                a, b = rt.split("/")
                out.append(f"{statistics.median(g[a]) / statistics.median(g[b]):.4g}" if g.get(a) and g.get(b) else "-")
            print(f"| {key[0]} | {key[1]} x {key[2]} | " + " | ".join(out) + " |")


def main(argv=None) -> None:
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = p.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--kernel", default="")
    t.add_argument("--per-step", type=int, default=0)
    t.add_argument("--window", default="", help="A:B -- only the matching dispatches A..B-1, in dispatch order")
    t.set_defaults(fn=trace)
    f = sub.add_parser("traffic")
    f.add_argument("fetch_dir")
    f.add_argument("write_dir")
    f.add_argument("--kernel", required=True)
    f.add_argument("--read-bytes", type=float, required=True)
    f.add_argument("--read-pick", choices=("median", "max"), default="median",
                   help="which streaming-read dispatch is the one of --read-bytes: the median (all reads of one "
                        "size) or the largest (one long read among shorter ones)")
    f.add_argument("--copy-bytes", type=float, default=float(1 << 32))
    f.add_argument("--algo-bytes", type=float, default=0.0)
    f.set_defaults(fn=traffic)
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--kernel", required=True)
    m.add_argument("--flops", type=float, default=0.0)
    m.add_argument("--simds", type=int, default=1024, help="SIMDs on the device (MI355X: 256 CUs x 4)")
    m.add_argument("--xcds", type=int, default=8, help="instances GRBM_GUI_ACTIVE is summed over (MI355X: 8 XCDs)")
    m.set_defaults(fn=mfma)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--ratio", action="append", default=[], help="A/B: ratio of the medians of counters A and B")
    c.set_defaults(fn=counters)
    args = p.parse_args(argv)
    args.fn(args)


if __name__ == "__main__":
    main(sys.argv[1:])
