"""Summarise rocprofv3 CSV output (kernel stats, or counter passes) as Markdown.

usage: python -m exact_attention_69_amd.profsum stats <run_kernel_stats.csv> "<command>"
       python -m exact_attention_69_amd.profsum pmc <dir with p*/run_counter_collection.csv> "<command>"
       python -m exact_attention_69_amd.profsum traffic <dir> <workload> <copy MiB> "<commands>"
       python -m exact_attention_69_amd.profsum sparseio <dir> <workload,...> <copy MiB> <LDS KiB> "<commands>"

`traffic` reads <dir>/kt/run_kernel_stats.csv (a --kernel-trace --stats run)
and <dir>/p*/run_counter_collection.csv (counter passes over the same
program, which also ran one plain device copy of <copy MiB> MiB), scales
FETCH_SIZE / WRITE_SIZE by what they read for that copy, and writes the
per-kernel table plus a JSON block that bench.py reads for the roofline's
`traffic` while the kernel sources still hash to the recorded value.
"""
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def kernel_sources(kernel=None):
    """Source files a kernel is built from: the file that defines it, the
    units that include that file, and every shared header (all sources when
    `kernel` is None or not found)."""
    files = sorted(glob.glob(os.path.join(CSRC, "*")))
    if kernel is None:
        return files
    base = re.match(r"[A-Za-z_0-9]+", kernel).group(0)
    pat = re.compile(r"__global__[^;{]*?\b" + re.escape(base) + r"\s*\(")
    home = [f for f in files if pat.search(open(f, encoding="utf-8", errors="replace").read())]
    if not home:
        return files
    # units that compile the home file under other settings (#include "home")
    inc = {f for f in files for h in home
           if f'#include "{os.path.basename(h)}"' in open(f, encoding="utf-8", errors="replace").read()}
    return sorted(set(home) | inc | {f for f in files if f.endswith(".hpp")})


def kernel_source_sha256(kernel=None):
    """SHA-256 over the names and contents of kernel_sources(kernel), sorted
    by name."""
    h = hashlib.sha256()
    for f in kernel_sources(kernel):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()

KERNEL_RE = re.compile(r"(fwd_bf16_kernel|fwd_pair_kernel|bwd_kv_bf16_kernel|bwd_kv_pair_kernel|bwd_q_bf16_kernel|"
                       r"bwd_q_pair_kernel|"
                       r"bwd_rowdot_kernel|fwd_f32_kernel|"
                       r"bwd_kv_f32_kernel|bwd_q_f32_kernel|pattern_bitmap_kernel|pattern_list_kernel|"
                       r"pattern_layout_full_kernel|pattern_gather_kernel|fwd_full_merge_kernel|full_sum_kernel|fwd_fp8_kernel|"
                       r"quant_\w+?kernel|"
                       r"elementwise_kernel|copy\w*)(I\w*?E(?:EvP|Ev$|EEv))?")
# mask mode (second template argument of the bf16 and paired kernels); the unmasked one is unnamed
MODE_NAMES = {"1": "window", "2": "pattern", "3": "full"}


def short(name):
    m = KERNEL_RE.search(name)
    if not m:
        return name[:60]
    args = re.findall(r"Li(\d+)E", m.group(2) or "")
    if not args:  # a demangled name: kernel<a, b>(...)
        t = re.match(r"<([\d, ]+)>", name[m.end(1):])
        args = [a.strip() for a in t.group(1).split(",")] if t else []
    if not args:
        return m.group(1)
    label = args[0]
    if len(args) > 1 and m.group(1).endswith(("bf16_kernel", "pair_kernel")) and args[1] in MODE_NAMES:
        label += "," + MODE_NAMES[args[1]]
    elif len(args) > 1 and m.group(1) == "full_sum_kernel":
        label += "," + args[1]
    return f"{m.group(1)}<{label}>"


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


def _counters(directory):
    res = collections.defaultdict(lambda: collections.defaultdict(dict))
    for path in sorted(glob.glob(directory + "/p*/run_counter_collection.csv")):
        for row in csv.DictReader(open(path)):
            d = res[short(row["Kernel_Name"])][row["Counter_Name"]]
            d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    return {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in res.items()}


def overlap(cnt):
    """Table of how a kernel's SIMD cycles split between the matrix cores and
    the vector ALU, from the counters (kernels that have them all), or []."""
    need = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES",
            "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")
    rows = []
    for k, cs in cnt.items():
        if not all(c in cs for c in need) or not cs["GRBM_GUI_ACTIVE"] or not cs["SQ_VALU_MFMA_BUSY_CYCLES"]:
            continue
        simd = 1024 * cs["GRBM_GUI_ACTIVE"] / 8  # SIMD cycles of the launch
        mfma = 100 * cs["SQ_VALU_MFMA_BUSY_CYCLES"] / simd
        valu = 100 * 4 * cs["SQ_ACTIVE_INST_VALU"] / simd
        co = 100 * cs["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd
        wait = 100 * cs["SQ_WAIT_ANY"] / cs["SQ_WAVE_CYCLES"] if cs["SQ_WAVE_CYCLES"] else 0.0
        fifo = cs.get("SQ_LDS_DATA_FIFO_FULL")
        rows.append(f"| {k} | {mfma:.1f} | {valu:.1f} | {co:.1f} | {mfma + valu - co:.1f} | {wait:.1f} | "
                    + (f"{fifo:.3g} |" if fifo is not None else "- |"))
    if not rows:
        return []
    return ["Matrix cores and vector ALU (per SIMD cycle of the launch):", "",
            "| kernel | MFMA busy % | VALU issue % | both at once % | either % | waves waiting % | "
            "LDS data FIFO full |", "|---|---|---|---|---|---|---|"] + rows + [
            "", "VALU issue % = 4 x SQ_ACTIVE_INST_VALU (a wave64 vector instruction occupies the 16-lane SIMD "
            "for 4 cycles) / SIMD cycles; both at once % = SQ_VALU_MFMA_COEXEC_CYCLES / SIMD cycles; either % "
            "= MFMA + VALU - both; waves waiting % = SQ_WAIT_ANY / SQ_WAVE_CYCLES."]


def algorithmic_bytes(wl, kernel):
    """(read, write) bytes a kernel must move at least, per launch."""
    eb = 2 if wl.dtype == "bf16" else 4
    t = wl.B * wl.H * wl.n * wl.d * eb
    tkv = wl.B * wl.Hkv * wl.n * wl.d * eb
    r = wl.B * wl.H * wl.n * 4
    if kernel.startswith("fwd"):
        return t + 2 * tkv, t + r                      # Q, K, V -> O, LSE
    if kernel.startswith("bwd_rowdot"):
        return 2 * t + r, 2 * r                        # O, dO, LSE -> D, LSE*log2e
    if kernel.startswith("bwd_kv"):
        return 2 * t + 2 * tkv + 2 * r, 2 * tkv        # Q, dO, K, V, LSE*log2e, D -> dK, dV
    if kernel.startswith("bwd_q"):
        return 2 * t + 2 * tkv + 2 * r, t              # Q, dO, K, V, LSE*log2e, D -> dQ
    return None


def traffic(directory, workload_name, copy_mib, cmds):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import workload
    wl = workload(workload_name)
    kt = {short(r["Name"]): r for r in csv.DictReader(open(os.path.join(directory, "kt", "run_kernel_stats.csv")))}
    cnt = _counters(directory)
    copy = [k for k in cnt if "copy" in k.lower()]
    if not copy:
        raise SystemExit("no copy kernel in the counter passes (run them with --copy-calibration)")
    c = cnt[copy[0]]
    copy_kib = copy_mib * 1024.0
    fs, ws = copy_kib / c["FETCH_SIZE"], copy_kib / c["WRITE_SIZE"]
    out = [f"# HBM traffic and counters: one bench step of {wl.name}, MI355X", "",
           "Commands (one counter set per run; each counter run also performs one plain device copy of "
           f"{copy_mib} MiB, whose counters calibrate the HBM figures):", "", "```"] + cmds + ["```", "",
           f"Calibration ({copy[0]} moving {copy_mib} MiB = {copy_kib:.0f} KiB): FETCH_SIZE read "
           f"{c['FETCH_SIZE']:.0f} KiB -> fetch scale {fs:.4f}; WRITE_SIZE read {c['WRITE_SIZE']:.0f} KiB -> "
           f"write scale {ws:.4f}.", "",
           "| kernel | avg ms (trace) | HBM read MiB (scaled) | HBM write MiB (scaled) | algorithmic read / write "
           "MiB | HBM GB/s | MFMA busy % | clock GHz | LDS bank conflicts | MFMA TFLOP executed |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    js = {"workload": wl.name, "fetch_scale": round(fs, 6), "write_scale": round(ws, 6), "kernels": {}}
    for k, cs in cnt.items():
        if k in copy or "FETCH_SIZE" not in cs or k not in kt:
            continue
        ms = float(kt[k]["AverageNs"]) / 1e6
        rd, wr = cs["FETCH_SIZE"] * fs * 1024, cs["WRITE_SIZE"] * ws * 1024
        alg = algorithmic_bytes(wl, k)
        gui = cs.get("GRBM_GUI_ACTIVE", 0.0) / 8  # per-XCD cycles
        busy = 100.0 * cs.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * gui) if gui else 0.0
        clock = gui / (ms * 1e6) if ms else 0.0
        mops = cs.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / 1e12
        algs = f"{alg[0] / 2**20:.0f} / {alg[1] / 2**20:.0f}" if alg else "-"
        out.append(f"| {k} | {ms:.3f} | {rd / 2**20:.0f} | {wr / 2**20:.0f} | {algs} | {(rd + wr) / (ms * 1e6):.0f} | "
                   f"{busy:.1f} | {clock:.2f} | {cs.get('SQ_LDS_BANK_CONFLICT', 0.0):.0f} | {mops:.3f} |")
        js["kernels"][k] = {"avg_ms_trace": round(ms, 4), "fetch_kib": round(cs["FETCH_SIZE"], 1),
                            "write_kib": round(cs["WRITE_SIZE"], 1), "hbm_bytes_per_launch": int(rd + wr),
                            "sources": [os.path.basename(f) for f in kernel_sources(k)],
                            "source_sha256": kernel_source_sha256(k)}
    out += ["", "MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE/8 XCDs); clock = "
            "(GRBM_GUI_ACTIVE/8) / trace duration; executed MFMA TFLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512.", ""]
    ov = overlap(cnt)
    if ov:
        out += ov + [""]
    out += [
            "Machine-readable (read by bench.py; a kernel's entry is valid only while the file that defines it and "
            "the shared headers, listed in `sources`, still hash to its `source_sha256`):",
            "", "```json", json.dumps(js, indent=1), "```"]
    return "\n".join(out)


# Kernels of the pattern forward call and backward call (the plan kernels run
# in both and are reported apart).
_FWD_CALL = ("fwd_bf16_kernel", "fwd_full_merge_kernel")
_PLAN = ("pattern_bitmap_kernel", "pattern_list_kernel", "pattern_layout_full_kernel")


def _sums(path):
    """{short kernel name: {counter: total over dispatches}}, {kernel: dispatches}."""
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for row in csv.DictReader(open(path)):
        k = short(row["Kernel_Name"])
        tot[k][row["Counter_Name"]] += float(row["Counter_Value"])
        disp[k].add(row["Dispatch_Id"])
    return tot, {k: len(v) for k, v in disp.items()}


def sparse_io(directory, names, copy_mib, lds_kib, cmds):
    """Per-step HBM bytes and L1->L2 read bytes of the pattern calls for each
    workload (counter passes under <directory>/<workload>/p1..p3), set beside
    the block-sparse I/O bound's terms: Z_input (nonzeros of the inputs),
    Z_QK (visible pairs), M (fast memory, elements)."""
    import math
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import draw_pattern, pattern_pair_count, workload
    M = lds_kib * 1024 // 2  # bf16 elements
    head = ["| workload | n | random blocks | Z_QK / n^2 | call | Z_input | Z_QK | split point Z_in^2/Z_QK "
            "(per head) | sum of Z_in^2/M | sum of Z_in sqrt(Z_QK/M) | HBM read+write (MiB) | HBM / compulsory | "
            "L1->L2 reads (MiB) | L1->L2 / (2 B x sum of Z_in sqrt(Z_QK/M)) | L1->L2 bytes per visible pair |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    rows = []
    creq = 0.0
    for name in names:
        wl = workload(name)
        window, glob_, layout = draw_pattern(wl)
        zqk = pattern_pair_count(wl.n, window, glob_, layout) * wl.B * wl.H
        f, nf = _sums(os.path.join(directory, name, "p1", "run_counter_collection.csv"))
        w, _ = _sums(os.path.join(directory, name, "p2", "run_counter_collection.csv"))
        r, _ = _sums(os.path.join(directory, name, "p3", "run_counter_collection.csv"))
        copy = [k for k in f if "copy" in k.lower()]
        cf = copy_mib * 1024.0 / f[copy[0]]["FETCH_SIZE"]
        cw = copy_mib * 1024.0 / w[copy[0]]["WRITE_SIZE"]
        creq = copy_mib * 2.0**20 / r[copy[0]]["TCP_TCC_READ_REQ_sum"]  # bytes per L1->L2 read request
        steps = nf.get(next(k for k in nf if k.startswith("fwd_bf16_kernel") and k.endswith("pattern>")), 1)
        nd = wl.B * wl.H * wl.n * wl.d
        for call, zin, comp in (("fwd", 3 * nd, (3 * nd + nd) * 2 + wl.B * wl.H * wl.n * 4),
                                ("bwd", 5 * nd, (5 * nd + 3 * nd) * 2 + 4 * wl.B * wl.H * wl.n * 4)):
            ks = [k for k in f if k not in copy and not k.startswith(_PLAN) and
                  (k.startswith(_FWD_CALL) if call == "fwd" else k.startswith(("bwd_", "full_sum")))]
            hbm = sum(f[k]["FETCH_SIZE"] * cf + w[k]["WRITE_SIZE"] * cw for k in ks) * 1024 / steps
            l2 = sum(r[k]["TCP_TCC_READ_REQ_sum"] for k in ks) * creq / steps
            # the bound is per attention problem (one head); summed over the heads
            bh = wl.B * wl.H
            zin_h, zqk_h = zin / bh, zqk / bh
            small = bh * zin_h * math.sqrt(zqk_h / M)
            large = bh * zin_h**2 / M
            rows.append(f"| {name} | {wl.n} | {wl.bigbird[2]} | {zqk_h / wl.n**2:.4f} | {call} | "
                        f"{zin:.3g} | {zqk:.3g} | {zin_h**2 / zqk_h:.3g} | {large:.3g} | {small:.3g} | "
                        f"{hbm / 2**20:.0f} | {hbm / comp:.2f} | "
                        f"{l2 / 2**20:.0f} | {l2 / (2 * small):.2f} | {l2 / zqk:.2f} |")
    return "\n".join(["Commands:", "", "```"] + cmds + ["```", "",
                      f"M = {lds_kib} KiB of LDS per CU = {M} bf16 elements.  Compulsory HBM bytes: the call's "
                      "inputs read once and outputs written once (fwd: Q, K, V -> O, LSE; bwd: Q, K, V, O, dO, "
                      "LSE -> dQ, dK, dV, with D and LSE*log2(e) written and read).  HBM bytes are FETCH_SIZE and "
                      "WRITE_SIZE scaled by a plain copy of known size; L1->L2 bytes are TCP_TCC_READ_REQ_sum "
                      f"times the bytes per request of the same copy ({creq:.0f} B).  Per bench step, summed over "
                      "the call's kernels (plan kernels excluded).  Z_input and Z_QK are totals over the B*H "
                      "heads; the bound's terms are taken per head and summed.", ""] + head + rows)


if __name__ == "__main__":
    nargs = {"stats": 2, "pmc": 2, "traffic": 4, "sparseio": 5}
    mode = sys.argv[1] if len(sys.argv) > 1 else ""
    if mode not in nargs or len(sys.argv) < 2 + nargs[mode]:
        print(__doc__.strip())
        sys.exit(2)
    if mode == "traffic":
        print(traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5].split("\n")))
    elif mode == "sparseio":  # <dir> <workload,workload,...> <copy MiB> <LDS KiB> <commands>
        print(sparse_io(sys.argv[2], sys.argv[3].split(","), int(sys.argv[4]), int(sys.argv[5]),
                        sys.argv[6].split("\n")))
    else:
        path, cmd = sys.argv[2], sys.argv[3]
        print(stats(path, cmd) if mode == "stats" else pmc(path, cmd))
