"""GPU parity of the grouped-query entry points (K/V heads shared by groups of
consecutive query heads) against the fp64 oracle, through the C ABI.

Cases cover multi-query (one K/V head), groups of 2-4, every head dim, both
element types, windows, ragged tails and a single row; a full-size
grouped-query problem checks whole key/value groups against the oracle and
every head against the exact-gradient identities.
"""

import sys
import time

import numpy as np
import pytest

from helpers import (check_outputs, draw_inputs, invariant_errors, make_case, oracle_case, run_gpu,
                     select_heads, to_device)
from workloads import VARIANTS

pytestmark = pytest.mark.gpu


def _run(B, H, Hkv, n, d, dtype, window=-1, seed=11):
    wl = make_case(B, H, n, d, dtype, window, seed=seed, kv_heads=Hkv)
    print(f"[gqa] {wl.name}", flush=True)
    inputs = draw_inputs(wl)
    got = run_gpu(wl, inputs)
    assert got["dk"].shape == (B, Hkv, n, d) and got["dv"].shape == (B, Hkv, n, d)
    ref = oracle_case(wl, inputs)
    errs = check_outputs(dtype, got, ref, wl.name)
    print(f"[gqa] {wl.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)


GQA_CASES = [
    # B, H, Hkv, n, d, dtype, window
    (1, 4, 1, 300, 128, "bf16", -1),   # multi-query
    (2, 8, 2, 257, 64, "bf16", -1),
    (1, 6, 3, 200, 256, "bf16", -1),
    (1, 4, 2, 333, 128, "bf16", 3),
    (1, 4, 2, 700, 128, "bf16", 70),
    (1, 4, 1, 600, 256, "bf16", 100),
    (1, 2, 1, 1, 64, "bf16", -1),      # a single row
    (1, 4, 2, 77, 64, "f32", -1),
    (1, 3, 1, 129, 256, "f32", -1),
    (1, 4, 1, 200, 128, "f32", 5),
]


@pytest.mark.parametrize("B,H,Hkv,n,d,dtype,window", GQA_CASES)
def test_gqa_parity(B, H, Hkv, n, d, dtype, window):
    _run(B, H, Hkv, n, d, dtype, window)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gqa_with_one_head_per_group_is_the_multi_head_call(dtype):
    import torch
    import exact_attention_69_amd as ea
    wl = make_case(2, 3, 250, 128 if dtype == "bf16" else 64, dtype, 30)
    t = to_device(draw_inputs(wl), dtype)
    a = ea.attn_fwd(t["q"], t["k"], t["v"], window=30)
    b = ea.attn_fwd_gqa(t["q"], t["k"], t["v"], window=30)
    ga = ea.attn_bwd(t["q"], t["k"], t["v"], a[0], t["do"], a[1], window=30)
    gb = ea.attn_bwd_gqa(t["q"], t["k"], t["v"], b[0], t["do"], b[1], window=30)
    torch.cuda.synchronize()
    for x, y in zip(a + ga, b + gb):
        assert torch.equal(x, y)


def test_gqa_forward_and_dq_equal_multi_head_on_repeated_kv():
    # The forward and the query-side pass read the shared K/V head in place of
    # a private copy: with K/V repeated per query head the multi-head call
    # must give the same bits.  dK/dV of the shared head equal the group sum
    # of the multi-head dK/dV up to fp32 summation order and bf16 rounding.
    import torch
    import exact_attention_69_amd as ea
    wl = make_case(1, 8, 400, 128, "bf16", kv_heads=2)
    t = to_device(draw_inputs(wl), "bf16")
    kr = t["k"].repeat_interleave(4, dim=1).contiguous()
    vr = t["v"].repeat_interleave(4, dim=1).contiguous()
    o1, l1 = ea.attn_fwd_gqa(t["q"], t["k"], t["v"])
    o2, l2 = ea.attn_fwd(t["q"], kr, vr)
    dq1, dk1, dv1 = ea.attn_bwd_gqa(t["q"], t["k"], t["v"], o1, t["do"], l1)
    dq2, dk2, dv2 = ea.attn_bwd(t["q"], kr, vr, o2, t["do"], l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(dq1, dq2)
    for g1, g2 in ((dk1, dk2), (dv1, dv2)):
        s2 = g2.float().reshape(1, 2, 4, 400, 128).sum(dim=2)
        err = (g1.float() - s2).norm() / s2.norm()
        assert err < 1e-2, float(err)


@pytest.mark.parametrize("dtype,window", [("bf16", -1), ("bf16", 40), ("f32", 7)])
def test_gqa_staged_backward_matches_one_call(dtype, window):
    import torch
    import exact_attention_69_amd as ea
    wl = make_case(2, 6, 333, 128 if dtype == "bf16" else 64, dtype, window, kv_heads=2)
    t = to_device(draw_inputs(wl), dtype)
    o, lse = ea.attn_fwd_gqa(t["q"], t["k"], t["v"], window=window)
    ref = ea.attn_bwd_gqa(t["q"], t["k"], t["v"], o, t["do"], lse, window=window)
    ws = ea.attn_bwd_rowdot(o, t["do"], lse)
    dk, dv = ea.attn_bwd_dkdv_gqa(t["q"], t["k"], t["v"], t["do"], lse, ws, window=window)
    dq = ea.attn_bwd_dq_gqa(t["q"], t["k"], t["v"], t["do"], lse, ws, window=window)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a, b)


# flat key/value heads (b*Hkv + g) checked against the oracle with all the
# query heads of their groups
GQA_ORACLE_GROUPS = {"bf16_b2h32kv8_n8192_d128_gqa": [0, 15]}


GQA_VARIANTS = [w for w in VARIANTS if w.Hkv != w.H]


@pytest.mark.parametrize("wl", GQA_VARIANTS, ids=[w.name for w in GQA_VARIANTS])
def test_gqa_full_size(wl):
    t0 = time.time()
    print(f"[gqa-full] {wl.name}: drawing inputs", flush=True)
    inputs = draw_inputs(wl)
    print(f"[gqa-full] {wl.name}: GPU fwd+bwd ({time.time() - t0:.1f}s)", flush=True)
    got = run_gpu(wl, inputs)
    groups = GQA_ORACLE_GROUPS[wl.name]
    print(f"[gqa-full] {wl.name}: oracle on key/value heads {groups} ({time.time() - t0:.1f}s)", flush=True)
    ref = oracle_case(wl, inputs, groups)
    errs = check_outputs(wl.dtype, select_heads(got, wl, groups), ref, wl.name)
    print(f"[gqa-full] {wl.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    inv = invariant_errors(inputs, got, wl)
    print(f"[gqa-full] {wl.name}: invariants " + " ".join(f"{k}={v:.2e}" for k, v in inv.items())
          + f" ({time.time() - t0:.1f}s)", flush=True)
    sys.stdout.flush()
    for k, v in inv.items():
        assert v <= 2e-2, f"{wl.name}: invariant {k} = {v:.3e}"
