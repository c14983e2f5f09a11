"""attn_bwd_noalloc (the backward whose row arrays live in the library's
fixed per-GPU scratch buffer) against attn_bwd, through the C ABI: two calls
in a row, the second on a smaller problem, each bit-equal to attn_bwd on the
same inputs (same kernels, same arithmetic), and the first also within the
oracle's tolerances."""

import numpy as np
import pytest

from helpers import check_outputs, draw_inputs, make_case, oracle_case, to_device

pytestmark = pytest.mark.gpu


def _noalloc_vs_attn_bwd(wl, check_oracle):
    import torch
    import exact_attention_69_amd as ea
    print(f"[noalloc] {wl.name} window={wl.window}", flush=True)
    inputs = draw_inputs(wl)
    t = to_device(inputs, wl.dtype)
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], wl.scale, wl.window)
    ref = ea.attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, wl.scale, wl.window)
    out = [torch.full_like(t["q"], float("nan")) for _ in range(3)]
    got = ea.attn_bwd_noalloc(t["q"], t["k"], t["v"], o, t["do"], lse, wl.scale, wl.window,
                              dq=out[0], dk=out[1], dv=out[2])
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), f"{wl.name} {name}: differs from attn_bwd"
    if check_oracle:
        r = oracle_case(wl, inputs)
        g = {k: v.float().cpu().numpy() for k, v in zip(("dq", "dk", "dv"), got)}
        errs = check_outputs(wl.dtype, g, {k: r[k] for k in ("dq", "dk", "dv")}, wl.name)
        print(f"[noalloc] {wl.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)


def test_noalloc_backward_two_calls_second_smaller():
    _noalloc_vs_attn_bwd(make_case(2, 3, 777, 128, "bf16", seed=91), check_oracle=True)
    _noalloc_vs_attn_bwd(make_case(1, 2, 300, 64, "bf16", window=40, seed=92), check_oracle=False)


def test_noalloc_backward_fp32_and_d256():
    _noalloc_vs_attn_bwd(make_case(1, 1, 256, 64, "f32", seed=93), check_oracle=True)
    _noalloc_vs_attn_bwd(make_case(1, 2, 200, 256, "bf16", seed=94), check_oracle=False)


def test_noalloc_backward_at_the_scratch_limit():
    # B*H*n = 2^21 rows: the two row arrays fill the 16 MiB buffer exactly
    import exact_attention_69_amd as ea
    rows = ea.EXATTN_NOALLOC_SCRATCH_BYTES // 8
    wl = make_case(1, 64, rows // 64, 64, "bf16", seed=95)
    _noalloc_vs_attn_bwd(wl, check_oracle=False)
