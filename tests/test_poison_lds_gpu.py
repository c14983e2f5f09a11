"""Reads of LDS before any write, caught with a poisoned debug build.

libexattn_poison.so is the same library built with EXATTN_POISON_LDS: every
kernel fills its LDS arrays with 0xFF bytes (NaN in bf16, fp32 and E4M3, -1 as
an int) before it starts work.  A kernel that reads a tile buffer, a row
statistic or a partial sum that none of its copies or stores wrote first then
sees NaN instead of whatever the previous kernel left there.  Each case runs
the same entry points on the ordinary build and on the debug build, from the
same device inputs; the outputs must agree bit for bit and be finite.  The
cases cover every kernel family: the bf16 forward and both backward passes at
d = 64, 128, 256 (ragged n, windows, shared key/value heads, the allocation-free
backward), the fp32 path, the pattern plan and pattern kernels (window, global
tokens, block layout), and the FP8 quantiser and forward.
"""

import os

import numpy as np
import pytest

from helpers import make_case, to_device
from workloads import draw_inputs, draw_signs

pytestmark = pytest.mark.gpu

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "exact_attention_69_amd")
POISON_LIB = os.path.join(PKG, "libexattn_poison.so")


@pytest.fixture(scope="module")
def poison_lib():
    from exact_attention_69_amd import _binding
    if not os.path.exists(POISON_LIB):
        raise RuntimeError(f"{POISON_LIB} is missing: build it with `python -m exact_attention_69_amd.build`")
    _binding.load_library()  # the ordinary build first: it stays the default
    return _binding.load_library(POISON_LIB)


def run_both(poison_lib, monkeypatch, run):
    """run() on the ordinary build, then on the poisoned one; each returns a
    dict of device tensors, copied to the host here."""
    import torch
    from exact_attention_69_amd import _binding

    def host(d):
        torch.cuda.synchronize()
        return {k: v.cpu() for k, v in d.items()}

    normal = host(run())
    with monkeypatch.context() as m:
        m.setattr(_binding, "_lib", poison_lib)
        poisoned = host(run())
    return normal, poisoned


def assert_same(normal, poisoned, label):
    import torch
    for k in normal:
        a, b = normal[k], poisoned[k]
        if a.is_floating_point():
            assert bool(torch.isfinite(a.float()).all()), f"{label}: {k} of the ordinary build is not finite"
        assert torch.equal(a, b), f"{label}: {k} differs under poisoned LDS (a read before a write)"


DENSE = [
    # B, H, Hkv, n, d, dtype, window
    (1, 2, 0, 300, 64, "bf16", -1),
    (1, 2, 0, 1000, 64, "bf16", 37),
    (1, 2, 0, 333, 128, "bf16", -1),
    (1, 2, 0, 1000, 128, "bf16", 100),
    (1, 1, 0, 1, 128, "bf16", -1),
    (1, 2, 0, 300, 256, "bf16", -1),
    (1, 2, 0, 700, 256, "bf16", 64),
    (1, 4, 2, 500, 128, "bf16", -1),
    (1, 4, 1, 400, 64, "bf16", 50),
    (1, 2, 0, 200, 64, "f32", -1),
    (1, 2, 0, 150, 128, "f32", 20),
]


@pytest.mark.parametrize("B,H,Hkv,n,d,dtype,window", DENSE)
def test_dense_paths_read_no_unwritten_lds(poison_lib, monkeypatch, B, H, Hkv, n, d, dtype, window):
    import exact_attention_69_amd as ea
    wl = make_case(B, H, n, d, dtype, window, q_mult=3.0, seed=900 + n + d, kv_heads=Hkv)
    print(f"[poison] {wl.name}", flush=True)
    t = to_device(draw_inputs(wl), dtype)
    gqa = wl.Hkv != wl.H
    fwd, bwd = (ea.attn_fwd_gqa, ea.attn_bwd_gqa) if gqa else (ea.attn_fwd, ea.attn_bwd)

    def run():
        o, lse = fwd(t["q"], t["k"], t["v"], wl.scale, wl.window)
        dq, dk, dv = bwd(t["q"], t["k"], t["v"], o, t["do"], lse, wl.scale, wl.window)
        out = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
        if not gqa and dtype == "bf16":
            dq2, dk2, dv2 = ea.attn_bwd_noalloc(t["q"], t["k"], t["v"], o, t["do"], lse, wl.scale, wl.window)
            out.update(dq_noalloc=dq2, dk_noalloc=dk2, dv_noalloc=dv2)
        return out

    assert_same(*run_both(poison_lib, monkeypatch, run), wl.name)


def test_pattern_paths_read_no_unwritten_lds(poison_lib, monkeypatch):
    import torch
    import exact_attention_69_amd as ea
    for n, d, window, glob, density in ((700, 64, 20, (7, 300, 699), 0.1), (1100, 128, -1, (), 0.05),
                                        (600, 128, 33, (0, 5), None)):
        wl = make_case(1, 2, n, d, "bf16", seed=950 + n)
        print(f"[poison] pattern {wl.name} window={window} globals={glob} layout={density}", flush=True)
        t = to_device(draw_inputs(wl), "bf16")
        g = torch.tensor(glob, dtype=torch.int32, device="cuda") if glob else None
        lay = None
        if density is not None:
            nb = (n + 63) // 64
            rng = np.random.default_rng(n)
            m = (rng.random((nb, nb)) < density) | np.eye(nb, dtype=bool)
            lay = torch.from_numpy(m.astype(np.uint8)).to("cuda")
        pat = ea.AttnPattern(window, g, lay)

        def run():
            o, lse = ea.attn_fwd_pattern(t["q"], t["k"], t["v"], pat, wl.scale)
            dq, dk, dv = ea.attn_bwd_pattern(t["q"], t["k"], t["v"], o, t["do"], lse, pat, wl.scale)
            return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)

        assert_same(*run_both(poison_lib, monkeypatch, run), f"pattern {wl.name}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rotate", [False, True])
def test_fp8_paths_read_no_unwritten_lds(poison_lib, monkeypatch, d, rotate):
    import torch
    import exact_attention_69_amd as ea
    wl = make_case(1, 2, 300, d, "bf16", seed=970 + d)
    print(f"[poison] fp8 {wl.name} rotate={rotate}", flush=True)
    x = draw_inputs(wl, ("q", "k", "v"))
    t = to_device(x, "bf16")
    sg = torch.from_numpy(draw_signs(wl)).to("cuda") if rotate else None

    def run():
        q8, qs = ea.attn_quant_fp8(t["q"], sg, ea.EXATTN_FP8_ROWS)
        k8, ks = ea.attn_quant_fp8(t["k"], sg, ea.EXATTN_FP8_ROWS)
        v8, vs = ea.attn_quant_fp8(t["v"], None, ea.EXATTN_FP8_V_TRANSPOSED)
        o, lse = ea.attn_fwd_fp8(q8, k8, v8, qs, ks, vs, t["q"].shape, wl.scale, rotated=rotate)
        return dict(q8=q8, qs=qs, k8=k8, ks=ks, v8=v8, vs=vs, o=o, lse=lse)

    assert_same(*run_both(poison_lib, monkeypatch, run), f"fp8 {wl.name} rotate={rotate}")
