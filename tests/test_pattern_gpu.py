"""GPU parity of the sparse-pattern entry points (window + global tokens +
64-token block layout) against the fp64 oracle, through the C ABI.

Small cases cover every head dim, ragged lengths and tiles that the pattern
covers fully (by the layout, by global rows or keys, by the band), partly,
or not at all; a layout with an empty block row exercises the empty-row
convention.  The two full-size variants (Longformer, BigBird) are checked on
whole heads against the oracle and on every head against the exact-gradient
identities.
"""

import sys
import time

import numpy as np
import pytest

import oracle
from helpers import check_outputs, draw_inputs, invariant_errors, make_case, to_device
from workloads import VARIANTS, draw_pattern

pytestmark = pytest.mark.gpu


def run_pattern(wl, inputs, window, glob, layout, backward=True):
    import torch
    import exact_attention_69_amd as ea
    t = to_device(inputs, wl.dtype)
    g = torch.from_numpy(np.asarray(glob, dtype=np.int32)).to("cuda") if len(glob) else None
    lay = torch.from_numpy(np.ascontiguousarray(layout, dtype=np.uint8)).to("cuda") if layout is not None else None
    pat = ea.AttnPattern(window, g, lay)
    o, lse = ea.attn_fwd_pattern(t["q"], t["k"], t["v"], pat, wl.scale)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = ea.attn_bwd_pattern(t["q"], t["k"], t["v"], o, t["do"], lse, pat, wl.scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in out.items()}


def oracle_pattern(wl, inputs, window, glob, layout, heads=None):
    pat = oracle.Pattern(wl.n, window, tuple(int(x) for x in glob), 64 if layout is not None else 0,
                         None if layout is None else layout.astype(bool))
    q, k, v, do = (inputs[x] for x in ("q", "k", "v", "do"))
    if heads is not None:
        sel = lambda a: a.reshape(-1, wl.n, wl.d)[heads]
        q, k, v, do = sel(q), sel(k), sel(v), sel(do)
    O, lse = oracle.attention_forward_pattern(q, k, v, wl.scale, pat)
    dq, dk, dv = oracle.attention_backward_pattern(q, k, v, do, wl.scale, pat)
    return {"o": O, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def random_layout(n, density, seed, diag=True):
    nb = -(-n // 64)
    g = np.random.default_rng(seed)
    lay = g.random((nb, nb)) < density
    if diag:
        lay |= np.eye(nb, dtype=bool)
    return lay.astype(np.uint8)


CASES = [
    # name, n, d, window, globals, layout(density or None)
    ("longformer_d64", 300, 64, 16, (0, 5, 130, 299), None),
    ("longformer_d128", 777, 128, 40, (0, 1, 2, 400), None),
    ("longformer_d256", 520, 256, 20, (3, 511), None),
    ("bigbird_d64", 700, 64, -1, (), 0.2),
    ("bigbird_d128", 1000, 128, -1, (), 0.15),
    ("bigbird_d256", 450, 256, -1, (), 0.3),
    ("union_d128", 900, 128, 7, (0, 450), 0.1),
    ("window_only_d128", 640, 128, 33, (), None),
    ("all_global_d64", 200, 64, 2, tuple(range(0, 200, 1)), None),
]


@pytest.mark.parametrize("name,n,d,window,glob,density", CASES, ids=[c[0] for c in CASES])
def test_pattern_parity(name, n, d, window, glob, density):
    wl = make_case(1, 2, n, d, "bf16", seed=7 * n + d)
    print(f"[pattern] {name}", flush=True)
    layout = None if density is None else random_layout(n, density, seed=n)
    inputs = draw_inputs(wl)
    got = run_pattern(wl, inputs, window, glob, layout)
    ref = oracle_pattern(wl, inputs, window, glob, layout)
    errs = check_outputs("bf16", got, ref, name)
    print(f"[pattern] {name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)


def bigbird_layout(n, n_glob_blocks, density, seed):
    """Random blocks plus the diagonal, with the first block rows and columns
    set in every block (their positions are full rows and full keys)."""
    lay = random_layout(n, density, seed).astype(bool)
    lay[:n_glob_blocks, :] = True
    lay[:, :n_glob_blocks] = True
    return lay.astype(np.uint8)


# Full positions (rows that see every key, keys every row sees) go through
# their own pass: one workgroup per chunk of the other side, chunks merged.
# n >= 2048 gives several chunks on every pass; many full positions give
# several workgroups of them and a single chunk.
FULL_CASES = [
    # name, n, d, window, globals, layout builder or None
    ("chunks_globals_d128", 4096, 128, 64, (0, 1, 2000, 4095), None),
    ("chunks_layout_d128", 4096, 128, -1, (), lambda n: bigbird_layout(n, 2, 0.03, n)),
    ("chunks_union_d64", 2500, 64, 20, (7, 1234, 2499), lambda n: bigbird_layout(n, 1, 0.05, n)),
    ("chunks_union_d256", 2112, 256, 30, (100, 2111), lambda n: bigbird_layout(n, 1, 0.05, n)),
    ("many_full_rows_d128", 3000, 128, 10, tuple(range(0, 3000, 7)), None),
    ("ragged_tail_global_d128", 2049, 128, 5, (2048,), None),
]


@pytest.mark.parametrize("name,n,d,window,glob,builder", FULL_CASES, ids=[c[0] for c in FULL_CASES])
def test_pattern_full_positions(name, n, d, window, glob, builder):
    wl = make_case(1, 2, n, d, "bf16", seed=11 * n + d)
    print(f"[pattern-full-pos] {name}", flush=True)
    layout = None if builder is None else builder(n)
    inputs = draw_inputs(wl)
    got = run_pattern(wl, inputs, window, glob, layout)
    ref = oracle_pattern(wl, inputs, window, glob, layout)
    errs = check_outputs("bf16", got, ref, name)
    print(f"[pattern-full-pos] {name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)


def test_pattern_full_positions_repeat_bitwise():
    # the chunk merge and sums run in a fixed order: two calls agree bit for bit
    n, d = 4096, 128
    wl = make_case(1, 2, n, d, "bf16", seed=3)
    layout = bigbird_layout(n, 2, 0.03, 5)
    inputs = draw_inputs(wl)
    a = run_pattern(wl, inputs, 16, (0, 3000), layout)
    b = run_pattern(wl, inputs, 16, (0, 3000), layout)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_pattern_duplicate_and_out_of_range_globals():
    # global_idx may repeat positions and hold positions outside [0, n): the
    # pattern is that of the distinct positions inside
    n, d = 700, 128
    wl = make_case(1, 2, n, d, "bf16", seed=21)
    raw = (5, 5, -3, 17, n, n + 100, 17, 640)
    inputs = draw_inputs(wl)
    got = run_pattern(wl, inputs, 9, raw, None)
    ref = oracle_pattern(wl, inputs, 9, (5, 17, 640), None)
    check_outputs("bf16", got, ref, "dup_globals")


@pytest.mark.parametrize("n", [1, 2, 33])
def test_pattern_tiny(n):
    wl = make_case(1, 2, n, 64, "bf16", seed=40 + n)
    inputs = draw_inputs(wl)
    for window, glob in ((0, ()), (-1, (0,)), (1, (n - 1,))):
        got = run_pattern(wl, inputs, window, glob, None)
        ref = oracle_pattern(wl, inputs, window, glob, None)
        check_outputs("bf16", got, ref, f"tiny n={n} w={window} g={glob}")


def test_pattern_all_rows_empty():
    # an empty layout, no window, no globals: every row sees nothing
    n, d = 300, 128
    wl = make_case(1, 2, n, d, "bf16", seed=8)
    layout = np.zeros((-(-n // 64),) * 2, dtype=np.uint8)
    got = run_pattern(wl, draw_inputs(wl), -1, (), layout)
    assert np.all(got["o"] == 0.0) and np.all(np.isneginf(got["lse"]))
    for k in ("dq", "dk", "dv"):
        assert np.all(got[k] == 0.0), k


def test_pattern_full_layout_is_dense_attention():
    # every block set: every row and key is a full position; the pattern
    # passes have nothing to do and the full-position passes compute it all
    import torch
    import exact_attention_69_amd as ea
    n, d = 1000, 128
    wl = make_case(1, 2, n, d, "bf16", seed=9)
    inputs = draw_inputs(wl)
    layout = np.ones((-(-n // 64),) * 2, dtype=np.uint8)
    got = run_pattern(wl, inputs, -1, (), layout)
    ref = oracle_pattern(wl, inputs, -1, (), layout)
    check_outputs("bf16", got, ref, "full_layout")
    t = to_device(inputs, "bf16")
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], wl.scale, -1)
    torch.cuda.synchronize()
    np.testing.assert_allclose(got["lse"], lse.cpu().numpy(), atol=1e-4, rtol=1e-5)


def test_pattern_window_covering_everything_is_dense_attention():
    import torch
    import exact_attention_69_amd as ea
    n, d = 800, 64
    wl = make_case(1, 2, n, d, "bf16", seed=10)
    inputs = draw_inputs(wl)
    got = run_pattern(wl, inputs, n, (3,), None)
    t = to_device(inputs, "bf16")
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], wl.scale, -1)
    torch.cuda.synchronize()
    np.testing.assert_allclose(got["o"], o.float().cpu().numpy(), atol=2e-2, rtol=0)
    np.testing.assert_allclose(got["lse"], lse.cpu().numpy(), atol=1e-4, rtol=1e-5)


def test_pattern_empty_rows_follow_the_convention():
    # no window, no globals, a layout whose second block row is empty: rows
    # 64..127 get O = 0, LSE = -inf, dQ = 0; the rest match the oracle.
    n, d = 256, 128
    wl = make_case(1, 1, n, d, "bf16", seed=77)
    layout = np.array([[1, 1, 0, 0], [0, 0, 0, 0], [0, 1, 1, 0], [1, 0, 0, 1]], dtype=np.uint8)
    inputs = draw_inputs(wl)
    got = run_pattern(wl, inputs, -1, (), layout)
    assert np.all(got["o"][0, 0, 64:128] == 0.0)
    assert np.all(np.isneginf(got["lse"][0, 0, 64:128]))
    assert np.all(got["dq"][0, 0, 64:128] == 0.0)
    ref = oracle_pattern(wl, inputs, -1, (), layout)
    keep = np.r_[0:64, 128:256]
    sub = lambda d_: {k: (v[..., keep] if k == "lse" else v[..., keep, :]) for k, v in d_.items() if k in ("o", "lse", "dq")}
    check_outputs("bf16", sub(got), sub(ref), "empty_rows")
    check_outputs("bf16", {k: got[k] for k in ("dk", "dv")}, {k: ref[k] for k in ("dk", "dv")}, "empty_rows")


def test_pattern_window_matches_window_entry_point():
    # a window-only pattern and the plain windowed call compute the same
    # attention (up to the order of the summation over tiles)
    import torch
    import exact_attention_69_amd as ea
    wl = make_case(1, 2, 700, 128, "bf16", seed=5)
    inputs = draw_inputs(wl)
    got = run_pattern(wl, inputs, 50, (), None)
    t = to_device(inputs, "bf16")
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], wl.scale, 50)
    torch.cuda.synchronize()
    np.testing.assert_allclose(got["o"], o.float().cpu().numpy(), atol=2e-2, rtol=0)
    np.testing.assert_allclose(got["lse"], lse.cpu().numpy(), atol=1e-4, rtol=1e-5)


PATTERN_VARIANTS = [w for w in VARIANTS if w.has_pattern]


@pytest.mark.parametrize("wl", PATTERN_VARIANTS, ids=[w.name for w in PATTERN_VARIANTS])
def test_pattern_full_size(wl):
    t0 = time.time()
    print(f"[pattern-full] {wl.name}: drawing inputs", flush=True)
    window, glob, layout = draw_pattern(wl)
    inputs = draw_inputs(wl)
    print(f"[pattern-full] {wl.name}: GPU fwd+bwd ({time.time() - t0:.1f}s)", flush=True)
    got = run_pattern(wl, inputs, window, glob, layout)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert np.all(np.isfinite(got[key])), f"{wl.name}: non-finite {key}"
    heads = [0, wl.B * wl.H - 1]
    print(f"[pattern-full] {wl.name}: oracle on heads {heads} ({time.time() - t0:.1f}s)", flush=True)
    ref = oracle_pattern(wl, inputs, window, glob, layout, heads)
    sel = {k: (v.reshape(-1, wl.n)[heads] if k == "lse" else v.reshape(-1, wl.n, wl.d)[heads]) for k, v in got.items()}
    errs = check_outputs(wl.dtype, sel, ref, wl.name)
    print(f"[pattern-full] {wl.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    inv = invariant_errors(inputs, got, wl)
    print(f"[pattern-full] {wl.name}: invariants " + " ".join(f"{k}={v:.2e}" for k, v in inv.items())
          + f" ({time.time() - t0:.1f}s)", flush=True)
    sys.stdout.flush()
    for k, v in inv.items():
        assert v <= 2e-2, f"{wl.name}: invariant {k} = {v:.3e}"
