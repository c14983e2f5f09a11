"""Problems past 2^31 elements per tensor (the size limit is 2^31 rows,
B*H*n; element offsets are 64-bit in every kernel).  131 080 heads of
n = 128, d = 128 put every tensor at 2^31 + 2^17 elements (4 GiB of bf16);
the first and the last heads (the last one lies wholly past element 2^31)
are compared with the fp64 oracle, with and without a window.  Inputs are
drawn on the device from a seeded generator (the oracle gets exactly those
bf16 values)."""

import numpy as np
import pytest

from helpers import check_outputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("window", [-1, 40])
def test_bf16_tensors_past_2_31_elements(window):
    import torch

    import exact_attention_69_amd as ea
    import oracle

    B, H, n, d = 1, (1 << 17) + 8, 128, 128
    assert B * H * n * d > (1 << 31)
    print(f"[large] B={B} H={H} n={n} d={d} window={window}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(6931 + window)
    q, k, v, do = (torch.randn(B, H, n, d, device="cuda", dtype=torch.bfloat16, generator=g) for _ in range(4))
    scale = 1.0 / np.sqrt(d)
    o, lse = ea.attn_fwd(q, k, v, scale, window)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, do, lse, scale, window)
    torch.cuda.synchronize()
    for h in (0, H - 1):
        x = {name: t[0, h].float().cpu().numpy()[None] for name, t in (("q", q), ("k", k), ("v", v), ("do", do))}
        O, L = oracle.attention_forward(x["q"], x["k"], x["v"], scale, window)
        dQ, dK, dV = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], scale, window)
        got = {"o": o[0, h].float().cpu().numpy()[None], "lse": lse[0, h].cpu().numpy()[None],
               "dq": dq[0, h].float().cpu().numpy()[None], "dk": dk[0, h].float().cpu().numpy()[None],
               "dv": dv[0, h].float().cpu().numpy()[None]}
        errs = check_outputs("bf16", got, {"o": O, "lse": L, "dq": dQ, "dk": dK, "dv": dV}, f"head {h}")
        print(f"[large] head {h}: " + " ".join(f"{kk}={vv:.2e}" for kk, vv in errs.items()), flush=True)
