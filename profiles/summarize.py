"""Summarise a rocprofv3 kernel trace (csv) into a short text table.

    python profiles/summarize.py <prefix>_kernel_trace.csv "<command that made it>" > out.md

Groups dispatches by kernel name and grid size (one row per launch shape)
and reports calls, average / min / max duration in microseconds.
"""
import collections
import csv
import sys


def main(path, command):
    rows = list(csv.DictReader(open(path)))
    agg = collections.defaultdict(list)
    for r in rows:
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
               int(r["Workgroup_Size_X"]))
        agg[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    print(f"command: `{command}`\n")
    print("| kernel | threads | wg | calls | avg us | min us | max us |")
    print("|---|---|---|---|---|---|---|")
    for (name, grid, wg), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        print(f"| {short} | {grid} | {wg} | {len(v)} | {sum(v) / len(v):.3f} | {min(v):.3f} "
              f"| {max(v):.3f} |")


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
