"""Summaries of rocprofv3 output for the decode kernels.

    python -m quantized_kv_cache_token_amd.profsum stats <dir> [--match REGEX]
    python -m quantized_kv_cache_token_amd.profsum dispatches <dir> [--match REGEX]
    python -m quantized_kv_cache_token_amd.profsum traffic --fetch <dir> --write <dir>
        --kernel REGEX [--kernel REGEX ...] --workload NAME --alg-bytes N [--fused] [--merged]
        --out FILE [--command TEXT]

`stats` prints per-kernel call counts and durations from a
`rocprofv3 --kernel-trace --stats --output-format csv` run.

`dispatches` groups the same run's kernel trace by kernel and grid size, which
separates, say, the one-row appends of decode steps from prefill appends.

`traffic` turns two counter runs (`--pmc FETCH_SIZE`, then `--pmc
WRITE_SIZE`, both of `bench.py --copy-probe`) into HBM bytes per launch of
each named kernel (the split kernel and the merge), and their sum: the bytes
of one decode step's attention.  Both counters read in KiB per dispatch.  Each is scaled by what
the same counter reads for the streaming probe, which reads exactly 1 GiB and
writes exactly 1 GiB, so that the figure is in true bytes.  The
result goes to a JSON file keyed by the hash of the decode kernel sources:
bench.py reports it only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_BYTES = 1 << 30          # the streaming probe reads and writes 1 GiB
PROBE_REGEX = r"neg_kernel"    # its kernel: an elementwise negation over fp32
# the sources of the split kernel and the merge the traffic record describes
DECODE_SOURCES = ("decode_mfma.hip", "decode.hip", "merge128.h", "quant_device.h", "wave_util.h",
                  "lkv_internal.h")


def kernel_source_hash() -> str:
    """Hash of the matrix-core split kernel's sources (ties a counter summary
    to them)."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        path = os.path.join(HERE, "csrc", name)
        if os.path.exists(path):
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = re.sub(r"\(.*$", "", name) if not name.startswith("void ") else re.sub(r"\(.*$", "", name[5:])
    return name if len(name) < 90 else name[:87] + "..."


def _one(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if len(hits) != 1:
        raise SystemExit(f"expected one *{suffix} under {d}, found {len(hits)}")
    return hits[0]


def stats(d: str, match: str | None) -> str:
    rows = list(csv.DictReader(open(_one(d, "kernel_stats.csv"))))
    out = ["| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        if match and not re.search(match, r["Name"]):
            continue
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out)


def dispatches(d: str, match: str | None) -> str:
    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(_one(d, "kernel_trace.csv"))):
        if match and not re.search(match, r["Kernel_Name"]):
            continue
        grid = (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        groups[(r["Kernel_Name"], grid, wg)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| kernel | grid (threads) | workgroup | dispatches | avg us | median us | min us | max us |",
           "|---|---|---:|---:|---:|---:|---:|---:|"]
    for (name, grid, wg), t in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        t = sorted(t)
        out.append(f"| `{_short(name)}` | {grid[0]}x{grid[1]}x{grid[2]} | {wg} | {len(t)} | {sum(t) / len(t):.2f} | "
                   f"{t[len(t) // 2]:.2f} | {t[0]:.2f} | {t[-1]:.2f} |")
    return "\n".join(out)


def _per_dispatch(d: str, counter: str) -> dict[str, list[float]]:
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(_one(d, "counter_collection.csv"))):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def _mean_of(vals: dict[str, list[float]], regex: str) -> tuple[str, float, int]:
    names = [n for n in vals if re.search(regex, n)]
    if len(names) != 1:
        raise SystemExit(f"{regex!r} matches {len(names)} kernels: {[_short(n) for n in names]}")
    v = vals[names[0]]
    return names[0], sum(v) / len(v), len(v)


def traffic(fetch_dir: str, write_dir: str, kernels: list[str], workload: str, alg_bytes: int, fused: bool,
            merged: bool,
            command: str) -> dict:
    f = _per_dispatch(fetch_dir, "FETCH_SIZE")
    w = _per_dispatch(write_dir, "WRITE_SIZE")
    _, pf, _ = _mean_of(f, PROBE_REGEX)
    _, pw, _ = _mean_of(w, PROBE_REGEX)
    sf = PROBE_BYTES / (pf * 1024.0)
    sw = PROBE_BYTES / (pw * 1024.0)
    per, total = [], 0.0
    for kernel in kernels:
        kname, kf, nf = _mean_of(f, kernel)
        _, kw, nw = _mean_of(w, kernel)
        fetch_b = kf * 1024.0 * sf
        write_b = kw * 1024.0 * sw
        total += fetch_b + write_b
        per.append({"kernel": _short(kname), "dispatches": [nf, nw], "fetch_kib_raw": round(kf, 2),
                    "write_kib_raw": round(kw, 2), "hbm_fetch_bytes_per_launch": int(fetch_b),
                    "hbm_write_bytes_per_launch": int(write_b)})
    return {
        "workload": workload, "fused": fused, "merged": merged, "source_hash": kernel_source_hash(), "kernels": per,
        "probe_fetch_kib_raw": round(pf, 2), "probe_write_kib_raw": round(pw, 2),
        "scale_fetch": round(sf, 5), "scale_write": round(sw, 5),
        "hbm_bytes_per_step": int(total), "alg_bytes_per_step": alg_bytes,
        "traffic_over_alg": round(total / alg_bytes, 4),
        "command": command,
    }


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--match")
    g = sub.add_parser("dispatches")
    g.add_argument("dir")
    g.add_argument("--match")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, action="append")
    t.add_argument("--fused", action="store_true")
    t.add_argument("--merged", action="store_true", help="the split kernel also merges (one kernel per step)")
    t.add_argument("--workload", required=True)
    t.add_argument("--alg-bytes", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", default="")
    a = p.parse_args(argv)
    if a.cmd == "stats":
        print(stats(a.dir, a.match))
    elif a.cmd == "dispatches":
        print(dispatches(a.dir, a.match))
    else:
        rec = traffic(a.fetch, a.write, a.kernel, a.workload, a.alg_bytes, a.fused, a.merged, a.command)
        with open(a.out, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        json.dump(rec, sys.stdout, indent=1)
        print()


if __name__ == "__main__":
    main()
