"""Summarise rocprofv3 CSV output (kernel stats, or counter passes) as Markdown.

usage: python -m exact_attention_69_amd.profsum stats <run_kernel_stats.csv> "<command>"
       python -m exact_attention_69_amd.profsum pmc <dir with p*/run_counter_collection.csv> "<command>"
"""
import collections
import csv
import glob
import re
import sys

KERNEL_RE = re.compile(r"(fwd_bf16_kernel|bwd_kv_bf16_kernel|bwd_q_bf16_kernel|bwd_rowdot_kernel|fwd_f32_kernel|"
                       r"bwd_kv_f32_kernel|bwd_q_f32_kernel|elementwise_kernel|copy\w*)(?:I[A-Za-z]*Li(\d+))?")


def short(name):
    m = KERNEL_RE.search(name)
    if not m:
        return name[:60]
    return m.group(1) + (f"<{m.group(2)}>" if m.group(2) else "")


def stats(path, cmd):
    rows = list(csv.DictReader(open(path)))
    out = [f"Command: `{cmd}`", "", "| kernel | calls | avg duration (ms) | total (ms) | % |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out)


def pmc(directory, cmd):
    res = collections.defaultdict(lambda: collections.defaultdict(dict))
    for path in sorted(glob.glob(directory + "/p*/run_counter_collection.csv")):
        for row in csv.DictReader(open(path)):
            k = short(row["Kernel_Name"])
            d = res[k][row["Counter_Name"]]
            d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    out = [f"Command: `{cmd}`", "", "Per-dispatch averages (summed over all counter instances):", ""]
    for k, cs in res.items():
        out.append(f"### {k}")
        out.append("| counter | avg per dispatch | dispatches |")
        out.append("|---|---|---|")
        for c, per in sorted(cs.items()):
            out.append(f"| {c} | {sum(per.values()) / len(per):.6g} | {len(per)} |")
        out.append("")
    return "\n".join(out)


if __name__ == "__main__":
    mode, path, cmd = sys.argv[1], sys.argv[2], sys.argv[3]
    print(stats(path, cmd) if mode == "stats" else pmc(path, cmd))
