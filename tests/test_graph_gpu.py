"""Capture of the entry points in a HIP graph (torch.cuda.CUDAGraph).

The calls are stream ordered, launch kernels only (no allocation, no memset,
no host synchronisation), so a captured step replays like the eager one.
Each graph is replayed several times; before every replay new inputs are
copied into its static tensors, and after it an eager call on the same
inputs (eager work between the replays) must give the same outputs bit for
bit (the kernels are deterministic).
"""

import numpy as np
import pytest

from helpers import draw_inputs, make_case, to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(step):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    return g, outs


def _replays(wl, static, step, eager, label):
    import torch
    g, outs = _capture(step)
    for r in range(REPLAYS):
        fresh = to_device(draw_inputs(make_case(wl.B, wl.H, wl.n, wl.d, "bf16", seed=1000 + r)), "bf16")
        for k, t in static.items():
            t.copy_(fresh[k])
        g.replay()
        ref = eager({k: t.clone() for k, t in static.items()})
        torch.cuda.synchronize()
        for name, a, b in zip(ref.keys(), outs, ref.values()):
            assert torch.equal(a, b), f"{label}: replay {r}: {name} differs from the eager call"
        print(f"[graph] {label}: replay {r} equal", flush=True)


def test_dense_step_in_a_graph():
    import exact_attention_69_amd as ea
    wl = make_case(1, 2, 600, 128, "bf16", seed=1)
    static = to_device(draw_inputs(wl), "bf16")

    def run(t):
        o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], wl.scale, 40)
        dq, dk, dv = ea.attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, wl.scale, 40)
        return o, lse, dq, dk, dv

    _replays(wl, static, lambda: run(static),
             lambda t: dict(zip(("o", "lse", "dq", "dk", "dv"), run(t))), "dense window 40")


def test_pattern_step_in_a_graph():
    import torch
    import exact_attention_69_amd as ea
    n, d = 1500, 128
    wl = make_case(1, 2, n, d, "bf16", seed=2)
    static = to_device(draw_inputs(wl), "bf16")
    nb = -(-n // 64)
    lay = np.eye(nb, dtype=np.uint8)
    lay[0, :] = lay[:, 0] = 1
    pat = ea.AttnPattern(16, torch.tensor([3, 700, 1499], dtype=torch.int32, device="cuda"),
                         torch.from_numpy(lay).to("cuda"))
    ws = torch.empty(ea.attn_pattern_workspace_bytes(ea.EXATTN_BF16, 1, 2, n, d), dtype=torch.uint8, device="cuda")

    def run(t, w):
        o, lse = ea.attn_fwd_pattern(t["q"], t["k"], t["v"], pat, wl.scale, workspace=w)
        dq, dk, dv = ea.attn_bwd_pattern(t["q"], t["k"], t["v"], o, t["do"], lse, pat, wl.scale, workspace=w)
        return o, lse, dq, dk, dv

    ws_eager = torch.empty_like(ws)
    _replays(wl, static, lambda: run(static, ws),
             lambda t: dict(zip(("o", "lse", "dq", "dk", "dv"), run(t, ws_eager))), "pattern")


def test_fp8_step_in_a_graph():
    import torch
    import exact_attention_69_amd as ea
    from workloads import draw_signs
    wl = make_case(1, 2, 700, 128, "bf16", seed=3)
    static = to_device(draw_inputs(wl), "bf16")
    sg = torch.from_numpy(draw_signs(wl)).to("cuda")

    def run(t):
        q8, qs = ea.attn_quant_fp8(t["q"], sg, ea.EXATTN_FP8_ROWS)
        k8, ks = ea.attn_quant_fp8(t["k"], sg, ea.EXATTN_FP8_ROWS)
        v8, vs = ea.attn_quant_fp8(t["v"], None, ea.EXATTN_FP8_V_TRANSPOSED)
        return ea.attn_fwd_fp8(q8, k8, v8, qs, ks, vs, t["q"].shape, wl.scale, rotated=True)

    _replays(wl, static, lambda: run(static), lambda t: dict(zip(("o", "lse"), run(t))), "fp8")


def test_dense_d256_forward_on_a_large_grid_in_a_graph():
    """The paired-wave d=256 forward (a grid of 512 workgroups)."""
    import exact_attention_69_amd as ea
    wl = make_case(2, 16, 2048, 256, "bf16", seed=4)
    static = to_device(draw_inputs(wl, ("q", "k", "v")), "bf16")

    def run(t):
        return ea.attn_fwd(t["q"], t["k"], t["v"], wl.scale)

    _replays(wl, static, lambda: run(static), lambda t: dict(zip(("o", "lse"), run(t))), "dense d=256")
