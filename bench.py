"""Benchmark: exact attention forward + backward on one MI355X.

A step is one forward (attn_fwd) plus one backward (the three stage calls
attn_bwd_rowdot, attn_bwd_dkdv, attn_bwd_dq -- exactly the kernels attn_bwd
launches) over the whole batch of the n = 8192, d = 128 workload (B = 2,
H = 32, bf16, Q scaled by 3), inputs resident in device memory.  Throughput counts the algorithmic FLOPs
4*B*H*n^2*d (forward) + 10*B*H*n^2*d (backward), scaled by the fraction of
(query, key) pairs a window lets through.

The follow-on variants (grouped-query attention: K/V heads shared by groups
of query heads, through the *_gqa entry points) are timed the same way after
the main workload, with fewer steps, and reported under "variants".

Prints ONE JSON line.  Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--cpu-seconds S] [--no-variants]
                  [--variant-steps K] [--copy-calibration MIB]

--copy-calibration MIB also runs one plain device-to-device copy of MIB MiB
after the timed steps; under rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE give
the counters' scale for a transfer of known size.
"""

import argparse
import statistics
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s and % bf16 MFMA peak at n=8192, d=128 (1 GPU)"
DEFAULT_WORKLOAD = "bf16_b2h32_n8192_d128_q3"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3, "fp8": 5033.2}
PEAK_HBM_GBS = 8000.0


_PAIRS = {}


def flops(wl, pairs=False):
    """Algorithmic (fwd, bwd) FLOPs: 4 and 10 x visible pairs x d, over all
    heads (FP8 workloads: forward only); with pairs=True, the visible
    (query, key) pairs of one head."""
    from workloads import draw_pattern, pair_count, pattern_pair_count
    if wl.name not in _PAIRS:
        if wl.has_pattern:
            window, glob, layout = draw_pattern(wl)
            _PAIRS[wl.name] = pattern_pair_count(wl.n, window, glob, layout)
        else:
            _PAIRS[wl.name] = pair_count(wl.n, wl.window)
    if pairs:
        return _PAIRS[wl.name]
    p = _PAIRS[wl.name] * wl.B * wl.H
    return 4.0 * p * wl.d, 0.0 if wl.fp8 else 10.0 * p * wl.d


def hbm_bytes(wl):
    """Algorithmic HBM bytes per call: fwd reads Q,K,V and writes O, LSE;
    bwd reads Q,K,V,O,dO,LSE, writes dQ,dK,dV and writes+reads D.  K, V, dK
    and dV have the workload's key/value head count."""
    eb = 2 if wl.dtype == "bf16" else 4
    t = wl.B * wl.H * wl.n * wl.d * eb
    tkv = wl.B * wl.Hkv * wl.n * wl.d * eb
    r = wl.B * wl.H * wl.n * 4
    if wl.fp8:  # E4M3 Q, K, V in; bf16 O and fp32 LSE out; forward only
        t8 = wl.B * wl.H * wl.n * wl.d
        return 3 * t8 + 2 * t8 + r, 0
    return 2 * t + 2 * tkv + r, 4 * t + 4 * tkv + 3 * r


def measured_traffic(wl, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 summary
    (FETCH_SIZE / WRITE_SIZE scaled by a plain copy of known size), or None
    when the summary is for another workload or the kernel's sources (its own
    file and the shared headers) changed since the counters were taken."""
    import re
    from exact_attention_69_amd.profsum import kernel_source_sha256
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_counters_{wl.name}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    info = json.loads(m.group(1))
    k = info.get("kernels", {}).get(kernel)
    if info.get("workload") != wl.name or k is None or k.get("source_sha256") != kernel_source_sha256(kernel):
        return None
    return int(k["hbm_bytes_per_launch"])


def cpu_baseline(wl, seconds):
    """Time the fp64 oracle (as it stands) on whole heads of the workload
    until about `seconds` of CPU work; report TFLOP/s on the same FLOP count."""
    import numpy as np
    import oracle
    from workloads import draw_head
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    fwd_f, bwd_f = flops(wl)
    per_head = (fwd_f + bwd_f) / (wl.B * wl.H)
    done, t_total, heads = 0.0, 0.0, []
    h = 0
    while t_total < seconds and h < wl.B * wl.H:
        b, hh = divmod(h, wl.H)
        q, k, v, do = (draw_head(wl, x, b, hh) for x in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        oracle.attention_forward(q, k, v, wl.scale, wl.window)
        oracle.attention_backward(q, k, v, do, wl.scale, wl.window)
        t_total += time.perf_counter() - t0
        done += per_head
        heads.append((b, hh))
        h += 1
    return {"value": done / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd on {len(heads)} of {wl.B * wl.H} heads (b,h)={heads[0]}.."
                      f"{heads[-1]}, {t_total:.1f} s, BLAS threads={threads}, host cpus={os.cpu_count()}"}


def kernel_names(wl):
    """Short names (as the profile summaries write them) of the four kernels
    of a step: forward, rowdot, dK/dV, dQ.  In bf16 the forward and the dQ
    pass at d = 256 and the dK/dV pass at d = 256, and at d = 128 without a
    window, run on the paired-wave kernels."""
    t, d = wl.dtype, wl.d
    if t != "bf16":
        return [f"fwd_{t}_kernel<{d}>", f"bwd_rowdot_kernel<{d}>", f"bwd_kv_{t}_kernel<{d}>", f"bwd_q_{t}_kernel<{d}>"]
    m = ",window" if wl.window >= 0 else ""
    fwd = "fwd_pair_kernel" if d == 256 else "fwd_bf16_kernel"
    kv = "bwd_kv_pair_kernel" if d == 256 or (d == 128 and wl.window < 0) else "bwd_kv_bf16_kernel"
    dq = "bwd_q_pair_kernel" if d == 256 else "bwd_q_bf16_kernel"
    return [f"{fwd}<{d}{m}>", f"bwd_rowdot_kernel<{d}>", f"{kv}<{d}{m}>", f"{dq}<{d}{m}>"]


def time_steps(wl, steps, warmup, graph=False, one_call=False):
    """Run `warmup` untimed and `steps` timed steps of the workload with its
    inputs resident on the GPU; returns (names and average ms of the calls of
    a step, ms per step, wall seconds of the timed region).  Dense workloads
    time the four kernels of a step (forward, rowdot, dK/dV, dQ) one call
    each, or with one_call=True the forward and the whole backward as one
    attn_bwd call (which, with a window, runs its dK/dV and dQ kernels side
    by side on two streams); sparse-pattern workloads time attn_fwd_pattern
    and attn_bwd_pattern (each including its plan kernels).  With graph=True the step's calls are
    captured once in a HIP graph and the graph is replayed instead (the same
    kernels, without the host's per-call overhead); only the whole steps are
    timed then."""
    import numpy as np
    import torch
    import exact_attention_69_amd as ea
    from workloads import draw_inputs, draw_pattern

    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    x = draw_inputs(wl)
    t = {k: torch.from_numpy(v).to(dev, tdt) for k, v in x.items()}
    del x
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.n), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    code = ea.EXATTN_BF16 if wl.dtype == "bf16" else ea.EXATTN_F32
    # events are recorded on this stream; the calls launch on the current
    # stream (the same one, except inside a graph capture, where it is the
    # capture stream)
    stream = torch.cuda.current_stream(dev)
    if wl.fp8:
        from workloads import draw_signs
        sg = torch.from_numpy(draw_signs(wl)).to(dev) if wl.rotate else None
        # inputs quantised once (E4M3 codes resident in HBM); the timed call
        # is the FP8 forward
        q8, qs = ea.attn_quant_fp8(q, sg, ea.EXATTN_FP8_ROWS, stream=None)
        k8, ks = ea.attn_quant_fp8(k, sg, ea.EXATTN_FP8_ROWS, stream=None)
        v8, vs = ea.attn_quant_fp8(v, None, ea.EXATTN_FP8_V_TRANSPOSED, stream=None)
        names = [f"fwd_fp8_kernel<{wl.d}>"]
        calls = (lambda: ea.attn_fwd_fp8(q8, k8, v8, qs, ks, vs, q.shape, wl.scale, rotated=wl.rotate, out=o,
                                         lse=lse, stream=None),)
    elif wl.has_pattern:
        window, glob, layout = draw_pattern(wl)
        pat = ea.AttnPattern(window, torch.from_numpy(glob).to(dev) if len(glob) else None,
                             torch.from_numpy(layout).to(dev) if layout is not None else None)
        ws = torch.empty(ea.attn_pattern_workspace_bytes(code, wl.B, wl.H, wl.n, wl.d), dtype=torch.uint8,
                         device=dev)
        names = ["attn_fwd_pattern", "attn_bwd_pattern"]
        calls = (lambda: ea.attn_fwd_pattern(q, k, v, pat, wl.scale, out=o, lse=lse, workspace=ws, stream=None),
                 lambda: ea.attn_bwd_pattern(q, k, v, o, do, lse, pat, wl.scale, workspace=ws, dq=dq, dk=dk, dv=dv,
                                             stream=None))
    else:
        ws = torch.empty(max(ea.attn_bwd_workspace_bytes(code, wl.B, wl.H, wl.n, wl.d), 256), dtype=torch.uint8,
                         device=dev)
        gqa = wl.Hkv != wl.H
        attn_fwd = ea.attn_fwd_gqa if gqa else ea.attn_fwd
        attn_bwd_dkdv = ea.attn_bwd_dkdv_gqa if gqa else ea.attn_bwd_dkdv
        attn_bwd_dq = ea.attn_bwd_dq_gqa if gqa else ea.attn_bwd_dq
        names = kernel_names(wl)
        # The backward runs as its three stage calls (the same three kernels
        # that attn_bwd launches), so that every kernel has its own events.
        calls = (lambda: attn_fwd(q, k, v, wl.scale, wl.window, out=o, lse=lse, stream=None),
                 lambda: ea.attn_bwd_rowdot(o, do, lse, workspace=ws, stream=None),
                 lambda: attn_bwd_dkdv(q, k, v, do, lse, ws, wl.scale, wl.window, dk=dk, dv=dv, stream=None),
                 lambda: attn_bwd_dq(q, k, v, do, lse, ws, wl.scale, wl.window, dq=dq, stream=None))
        if one_call:
            attn_bwd = ea.attn_bwd_gqa if gqa else ea.attn_bwd
            names = ["attn_fwd", "attn_bwd"]
            calls = (calls[0],
                     lambda: attn_bwd(q, k, v, o, do, lse, wl.scale, wl.window, workspace=ws, dq=dq, dk=dk, dv=dv,
                                      stream=None))
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        replay_stream = torch.cuda.current_stream(dev)
        for e0, e1 in ev:
            e0.record(replay_stream)
            g.replay()
            e1.record(replay_stream)
        torch.cuda.synchronize()
        time_steps.last_step_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
        return names, [], statistics.median(time_steps.last_step_ms), 0.0

    # Whole steps, bracketed by device syncs, timed with events on the stream
    # the kernels are launched on; one event between consecutive calls.
    nk = len(calls)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for s in range(steps):
        ev[s][0].record(stream)
        for i, c in enumerate(calls):
            c()
            ev[s][i + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    kms = [sum(e[i].elapsed_time(e[i + 1]) for e in ev) / steps for i in range(nk)]
    time_steps.last_step_ms = [e[0].elapsed_time(e[nk]) for e in ev]  # per step, for medians
    return names, kms, start.elapsed_time(end) / steps, wall


def time_fp8_end_to_end(wl, steps, warmup=2):
    """Mean ms of the whole FP8 path from bf16 inputs in HBM: the three
    quantiser calls (Q and K with the rotation when the workload has one,
    V in the forward's transposed layout) and the FP8 forward, HIP events on
    the stream the calls are launched on."""
    import torch
    import exact_attention_69_amd as ea
    from workloads import draw_inputs, draw_signs
    dev = torch.device("cuda:0")
    x = draw_inputs(wl)
    q, k, v = (torch.from_numpy(x[n]).to(dev, torch.bfloat16) for n in ("q", "k", "v"))
    del x
    sg = torch.from_numpy(draw_signs(wl)).to(dev) if wl.rotate else None
    stream = torch.cuda.current_stream(dev)

    def step():
        q8, qs = ea.attn_quant_fp8(q, sg, ea.EXATTN_FP8_ROWS)
        k8, ks = ea.attn_quant_fp8(k, sg, ea.EXATTN_FP8_ROWS)
        v8, vs = ea.attn_quant_fp8(v, None, ea.EXATTN_FP8_V_TRANSPOSED)
        return ea.attn_fwd_fp8(q8, k8, v8, qs, ks, vs, q.shape, wl.scale, rotated=wl.rotate)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration timings of the other workloads")
    ap.add_argument("--variant-steps", type=int, default=10)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the attention path runs on a single device); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    from workloads import VARIANTS, workload

    wl = workload(args.workload)
    fwd_f, bwd_f = flops(wl)
    names, kms, ms, wall = time_steps(wl, args.steps, args.warmup)
    main_step_ms = list(time_steps.last_step_ms)
    nk = len(kms)
    fwd_ms = kms[0]
    bwd_ms = sum(kms[1:])
    peak = PEAK_TFLOPS["fp8" if wl.fp8 else wl.dtype]
    value = (fwd_f + bwd_f) / (ms * 1e-3) / 1e12

    # FLOPs per launch of each kernel (pairs = visible (i, j)).  Counted: the
    # kernel's share of the metric's 4 (forward) + 10 (backward) x pairs x d.
    # Executed: the matrix work the kernel does, which for the dQ pass adds the
    # second recomputation of S and dP that the metric does not count.
    #   forward       counted 4, executed 4  (S = Q K^T and O = P V)
    #   dK/dV pass    counted 8, executed 8  (S, dP = dO V^T, dV = P^T dO, dK = dS^T Q)
    #   dQ pass       counted 2, executed 6  (S and dP again, then dQ = dS K)
    #   rowdot        memory bound (reads O, dO and LSE, writes D and LSE*log2e)
    #   (sparse patterns: one forward call and one backward call, each with
    #   its plan kernels; counted = executed is not claimed there)
    if wl.has_pattern:
        kernel_counted = kernel_executed = [fwd_f, bwd_f]
    else:
        kernel_counted = [fwd_f, None, 0.8 * bwd_f, 0.2 * bwd_f]
        kernel_executed = [fwd_f, None, 0.8 * bwd_f, 0.6 * bwd_f]
    dom = max(range(nk), key=lambda i: kms[i])
    ach = kernel_counted[dom] / (kms[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": measured_traffic(wl, names[dom]), "kernel": names[dom],
                "counted_flops_per_launch": kernel_counted[dom], "executed_flops_per_launch": kernel_executed[dom],
                "avg_launch_ms": round(kms[dom], 4),
                "step_frac_counted": round(value / peak, 4)}
    fwd_tflops = fwd_f / (fwd_ms * 1e-3) / 1e12

    variants = {}
    if not args.no_variants:
        for vw in VARIANTS:
            vn, vk, vms, _ = time_steps(vw, args.variant_steps, 3)
            vf, vb = flops(vw)
            entry = {"value": round((vf + vb) / (vms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                     "ms_per_step": round(vms, 4), "steps": args.variant_steps, "B": vw.B, "H": vw.H, "Hkv": vw.Hkv,
                     "n": vw.n, "d": vw.d, "window": vw.window, "kernel_ms": {vn[i]: round(vk[i], 4) for i in range(len(vn))}}
            if vw.fp8:
                e2e_ms = time_fp8_end_to_end(vw, args.variant_steps)
                entry.update(rotated=vw.rotate, peak_tflops=PEAK_TFLOPS["fp8"],
                             pct_fp8_peak=round(100.0 * (vf / (vms * 1e-3) / 1e12) / PEAK_TFLOPS["fp8"], 2),
                             note="value and ms_per_step: the FP8 forward on E4M3 inputs quantised beforehand "
                                  "(O bf16); quant_fwd_*: the three quantiser calls from bf16 inputs plus the forward",
                             quant_fwd_ms=round(e2e_ms, 4),
                             quant_fwd_tflops=round(vf / (e2e_ms * 1e-3) / 1e12, 2))
            elif vw.has_pattern:
                entry.update(n_global=vw.n_global, bigbird=list(vw.bigbird), visible_pairs_per_head=flops(vw, pairs=True),
                             fwd_tflops=round(vf / (vk[0] * 1e-3) / 1e12, 2),
                             bwd_tflops=round(vb / (vk[1] * 1e-3) / 1e12, 2))
            else:
                entry["kernel_tflops_counted"] = {vn[i]: round(f / (vk[i] * 1e-3) / 1e12, 2)
                                                  for i, f in enumerate([vf, None, 0.8 * vb, 0.2 * vb]) if f}
                entry["kernel_tflops_executed"] = {vn[i]: round(f / (vk[i] * 1e-3) / 1e12, 2)
                                                   for i, f in enumerate([vf, None, 0.8 * vb, 0.6 * vb]) if f}
            entry["hbm_gbs_algorithmic"] = round(sum(hbm_bytes(vw)) / (vms * 1e-3) / 1e9, 1)
            variants[vw.name] = entry

    # Every workload shape: forward, backward and whole-step times (events;
    # per-kernel means, step median over >= 20 steps, 5 at n >= 32768, after
    # 5 warm-up steps) and TFLOP/s on the counted FLOPs.
    configs = {}
    if not args.no_configs:
        from workloads import WORKLOADS
        for cw in WORKLOADS:
            if cw.name == wl.name:
                cn, ck, cms, per = names, kms, ms, main_step_ms
            else:
                cn, ck, cms, _ = time_steps(cw, 5 if cw.n >= 32768 else 20, 5)
                per = list(time_steps.last_step_ms)
            cf, cb = flops(cw)
            med = statistics.median(per)
            cpeak = PEAK_TFLOPS[cw.dtype]
            configs[cw.name] = {
                "dtype": cw.dtype, "B": cw.B, "H": cw.H, "n": cw.n, "d": cw.d, "window": cw.window,
                "steps": len(per), "fwd_ms": round(ck[0], 4), "bwd_ms": round(sum(ck[1:]), 4),
                "step_ms_median": round(med, 4), "fwd_tflops": round(cf / (ck[0] * 1e-3) / 1e12, 2),
                "bwd_tflops": round(cb / (sum(ck[1:]) * 1e-3) / 1e12, 2),
                "tflops": round((cf + cb) / (med * 1e-3) / 1e12, 2), "peak_tflops": cpeak,
                "pct_peak": round(100.0 * (cf + cb) / (med * 1e-3) / 1e12 / cpeak, 2),
                "kernel_ms": {cn[i]: round(ck[i], 4) for i in range(len(cn))}}
            # the same step replayed from a HIP graph (no per-call host overhead)
            _, _, gms, _ = time_steps(cw, 5 if cw.n >= 32768 else 20, 2, graph=True)
            configs[cw.name]["step_ms_graph_median"] = round(gms, 4)
            configs[cw.name]["tflops_graph"] = round((cf + cb) / (gms * 1e-3) / 1e12, 2)
            if cw.window >= 0 and not cw.has_pattern and not cw.fp8:
                # With a window a single attn_bwd call runs its two gradient
                # passes on two streams: the step as a caller runs it
                # (attn_fwd, then one attn_bwd call), timed in turns with the
                # stage calls above so that both see the same clock.
                one, staged = [], []
                for _ in range(2):
                    time_steps(cw, 10, 2, one_call=True)
                    one += time_steps.last_step_ms
                    time_steps(cw, 10, 2)
                    staged += time_steps.last_step_ms
                oms, sms = statistics.median(one), statistics.median(staged)
                configs[cw.name]["step_ms_one_call_median"] = round(oms, 4)
                configs[cw.name]["step_ms_stage_calls_alternating_median"] = round(sms, 4)
                # < 1: the one-call step is faster (same clock, unlike the
                # step_ms_median taken earlier in the run)
                configs[cw.name]["one_call_over_stage_calls"] = round(oms / sms, 4)

    if args.copy_calibration:
        import torch
        dev = torch.device("cuda:0")
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8" if wl.fp8 else wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "n": wl.n, "d": wl.d, "window": wl.window,
                   "q_mult": wl.q_mult, "scale": wl.scale},
        "pct_fp8_peak" if wl.fp8 else "pct_bf16_peak": round(100.0 * value / peak, 2),
        "detail": {"fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
                   "kernel_ms": {names[i]: round(kms[i], 4) for i in range(nk)},
                   "kernel_tflops_counted": {names[i]: round(kernel_counted[i] / (kms[i] * 1e-3) / 1e12, 2)
                                             for i in range(nk) if kernel_counted[i]},
                   "kernel_tflops_executed": {names[i]: round(kernel_executed[i] / (kms[i] * 1e-3) / 1e12, 2)
                                              for i in range(nk) if kernel_executed[i]},
                   "fwd_tflops": round(fwd_tflops, 2), "bwd_tflops": round(bwd_f / (bwd_ms * 1e-3) / 1e12, 2) if bwd_ms else None,
                   "flops_per_step": fwd_f + bwd_f, "wall_s_timed": round(wall, 3),
                   "fwd_hbm_gbs_algorithmic": round(hbm_bytes(wl)[0] / (fwd_ms * 1e-3) / 1e9, 1),
                   "bwd_hbm_gbs_algorithmic": round(hbm_bytes(wl)[1] / (bwd_ms * 1e-3) / 1e9, 1) if bwd_ms else None},
        "roofline": roofline,
    }
    if variants:
        out["variants"] = variants
    if configs:
        out["configs"] = configs
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
