"""GPU parity of the HIP path against the fp64 oracle on oracle-sized shapes.

Shapes span several tiles and leave ragged tails (n not a multiple of any
tile size); windows cover the diagonal-only case, windows narrower than a
tile and windows wider than several tiles.  Every call goes through the
C-ABI library.
"""

import sys

import numpy as np
import pytest

from helpers import check_outputs, draw_inputs, make_case, oracle_case, run_gpu

pytestmark = pytest.mark.gpu


def _run(B, H, n, d, dtype, window=-1, q_mult=1.0, seed=7):
    wl = make_case(B, H, n, d, dtype, window, q_mult, seed)
    print(f"[parity] {wl.name} q_mult={q_mult}", flush=True)
    sys.stdout.flush()
    inputs = draw_inputs(wl)
    got = run_gpu(wl, inputs)
    ref = oracle_case(wl, inputs)
    errs = check_outputs(dtype, got, ref, wl.name)
    print(f"[parity] {wl.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    return errs


F32_CASES = [
    (1, 1, 256, 64, -1),     # the single-head fp32 workload
    (1, 2, 77, 64, -1),
    (2, 1, 300, 128, -1),
    (1, 1, 129, 256, -1),
    (1, 2, 100, 64, 0),
    (1, 1, 200, 128, 5),
    (1, 1, 90, 256, 40),
]


@pytest.mark.parametrize("B,H,n,d,window", F32_CASES)
def test_f32_parity(B, H, n, d, window):
    _run(B, H, n, d, "f32", window)


BF16_CASES = [
    (1, 2, 300, 64, -1, 1.0),
    (2, 1, 257, 128, -1, 1.0),
    (1, 1, 200, 256, -1, 1.0),
    (1, 1, 1, 64, -1, 1.0),       # a single row
    (1, 1, 33, 128, -1, 1.0),     # shorter than one tile
    (1, 1, 384, 128, -1, 3.0),    # peaky rows (Q scaled by 3)
    (1, 1, 320, 64, 0, 1.0),      # window 0: O = V
    (1, 1, 333, 128, 3, 1.0),     # window narrower than a tile
    (1, 1, 700, 128, 70, 1.0),    # window spanning a few tiles
    (1, 1, 600, 256, 100, 1.0),
    (1, 1, 513, 64, 200, 1.0),
    # the paired-wave kernels at d=256: a single row, one partial tile, a
    # ragged multi-head grid with peaky rows, windows narrower than a tile
    (1, 1, 1, 256, -1, 1.0),
    (1, 1, 33, 256, -1, 1.0),
    (2, 3, 257, 256, -1, 3.0),
    (1, 2, 300, 256, 0, 1.0),
    (1, 1, 333, 256, 3, 1.0),
]


@pytest.mark.parametrize("B,H,n,d,window,q_mult", BF16_CASES)
def test_bf16_parity(B, H, n, d, window, q_mult):
    _run(B, H, n, d, "bf16", window, q_mult)


@pytest.mark.parametrize("d", [64, 256])
def test_window_zero_identities_bf16(d):
    # window = 0: each row sees only its own key, so O = V exactly (bf16 in,
    # bf16 out), LSE = scale q.k, and dQ = dK = 0, dV = dO.
    wl = make_case(1, 1, 130, d, "bf16", 0)
    inputs = draw_inputs(wl)
    got = run_gpu(wl, inputs)
    np.testing.assert_array_equal(got["o"], inputs["v"])
    np.testing.assert_allclose(got["lse"], wl.scale * np.sum(inputs["q"][0, 0].astype(np.float64) *
                                                             inputs["k"][0, 0], axis=-1)[None, None], rtol=1e-5,
                               atol=1e-5)
    assert np.max(np.abs(got["dq"])) < 1e-4 and np.max(np.abs(got["dk"])) < 1e-4
    np.testing.assert_array_equal(got["dv"], inputs["do"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", [0, 5, 20, 100, -1])
def test_visible_key_sets_are_exact(d, window, dtype):
    # Q = 0 makes every visible score equal, so LSE_i = ln(#keys row i sees)
    # and O_i is the mean of those keys' values.  With V[j] = e_(j mod d) the
    # output of row i counts its visible keys per residue class: a single key
    # leaked through (or wrongly dropped by) the tail or window mask changes
    # LSE by at least ln(1 + 1/(2*window+1)) and O by a whole 1/count.
    import torch
    import exact_attention_69_amd as ea
    import oracle
    n = 2 * d + 45
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.zeros(1, 1, n, d, device="cuda", dtype=tdt)
    k = torch.randn(1, 1, n, d, device="cuda").to(tdt)
    vv = np.zeros((n, d), dtype=np.float32)
    vv[np.arange(n), np.arange(n) % d] = 1.0
    v = torch.from_numpy(vv)[None, None].to("cuda", tdt)
    o, lse = ea.attn_fwd(q, k, v, window=window)
    torch.cuda.synchronize()
    cnt = oracle.keys_per_row(n, window)
    np.testing.assert_allclose(lse[0, 0].cpu().numpy(), np.log(cnt), rtol=0, atol=2e-5)
    O, _ = oracle.attention_forward(np.zeros((n, d)), k[0, 0].float().cpu().numpy(), vv, 1.0, window)
    np.testing.assert_allclose(o[0, 0].float().cpu().numpy(), O, rtol=0, atol=4e-3 if dtype == "bf16" else 1e-6)


def test_forward_is_deterministic():
    import torch
    import exact_attention_69_amd as ea
    from helpers import to_device
    wl = make_case(2, 2, 500, 128, "bf16")
    t = to_device(draw_inputs(wl, ("q", "k", "v")), "bf16")
    o1, l1 = ea.attn_fwd(t["q"], t["k"], t["v"])
    for _ in range(3):
        o2, l2 = ea.attn_fwd(t["q"], t["k"], t["v"])
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", [-1, 300])
def test_repeated_forward_is_bit_exact_over_many_workgroups(d, window):
    """Regression test for a copy that overwrote the first K tile while other
    waves could still be reading it: the grid here has 128-256 workgroups,
    so waves drift apart, and every repeat must match the first bit for
    bit."""
    import torch
    import exact_attention_69_amd as ea
    from helpers import to_device
    wl = make_case(2, 8, 2048, d, "bf16", window=window, q_mult=3.0, seed=41 + d)
    print(f"[parity] repeated forward {wl.name}", flush=True)
    t = to_device(draw_inputs(wl, ("q", "k", "v")), "bf16")
    o1, l1 = ea.attn_fwd(t["q"], t["k"], t["v"], window=window)
    for _ in range(30):
        o2, l2 = ea.attn_fwd(t["q"], t["k"], t["v"], window=window, out=torch.empty_like(o1))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", [-1, 300])
def test_repeated_backward_is_bit_exact_over_many_workgroups(d, window):
    """The three backward stages on grids of 128-256 workgroups, repeated:
    every repeat matches the first bit for bit (no atomics, and every tile
    buffer is refilled only after a barrier that follows its last read)."""
    import torch
    import exact_attention_69_amd as ea
    from helpers import to_device
    wl = make_case(2, 8, 2048, d, "bf16", window=window, q_mult=3.0, seed=53 + d)
    print(f"[parity] repeated backward {wl.name}", flush=True)
    t = to_device(draw_inputs(wl), "bf16")
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], window=window)
    g1 = ea.attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, window=window)
    for _ in range(10):
        g2 = ea.attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, window=window)
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)


@pytest.mark.parametrize("n", [2048, 1990])
def test_dense_d256_paired_kernels_on_a_large_grid(n):
    """d=256 runs every pass on the paired-wave kernels.  On a grid of 512
    workgroups (n=1990 leaves a ragged last tile) the all-keys kernels agree
    with the window kernels given a window of n (every key visible) to bf16
    rounding, repeat bit for bit, and two heads match the oracle."""
    import torch
    import exact_attention_69_amd as ea
    from helpers import BF16_GRAD_FRO_REL, BF16_LSE_MAX_REL, BF16_O_MAX_REL, fro_rel, to_device
    B, H, d = 2, 16, 256
    wl = make_case(B, H, n, d, "bf16", q_mult=3.0, seed=47)
    print(f"[parity] paired d=256 forward and backward {wl.name}", flush=True)
    x = draw_inputs(wl)
    t = to_device(x, "bf16")
    o2, l2 = ea.attn_fwd(t["q"], t["k"], t["v"], wl.scale)
    g2 = ea.attn_bwd(t["q"], t["k"], t["v"], o2, t["do"], l2, wl.scale)
    for _ in range(5):  # repeats are bit-exact
        o3, l3 = ea.attn_fwd(t["q"], t["k"], t["v"], wl.scale)
        g3 = ea.attn_bwd(t["q"], t["k"], t["v"], o2, t["do"], l2, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(o2, o3) and torch.equal(l2, l3)
        assert all(torch.equal(a, b) for a, b in zip(g2, g3))
    o1, l1 = ea.attn_fwd(t["q"], t["k"], t["v"], wl.scale, window=n)
    g1 = ea.attn_bwd(t["q"], t["k"], t["v"], o2, t["do"], l2, wl.scale, window=n)
    torch.cuda.synchronize()
    assert float((o2.float() - o1.float()).abs().max()) <= 1e-2 * float(o1.float().abs().max())
    assert float((l2 - l1).abs().max()) <= 1e-5 * float(l1.abs().max())
    for a, b in zip(g2, g1):
        assert fro_rel(a.float().cpu().numpy(), b.float().cpu().numpy()) <= 1e-2
    import oracle
    for h in (0, B * H - 1):
        sel = lambda a: a.reshape(B * H, n, d)[h][None, None]
        q, k, v, do = (sel(x[key]) for key in ("q", "k", "v", "do"))
        O, L = oracle.attention_forward(q, k, v, wl.scale)
        dQ, dK, dV = oracle.attention_backward(q, k, v, do, wl.scale)
        og = o2.reshape(B * H, n, d)[h].float().cpu().numpy()
        lg = l2.reshape(B * H, n)[h].cpu().numpy()
        assert np.max(np.abs(og - O[0, 0])) <= BF16_O_MAX_REL * np.max(np.abs(O))
        assert np.max(np.abs(lg - L[0, 0])) <= BF16_LSE_MAX_REL * np.max(np.abs(L))
        for got, ref in zip(g2, (dQ, dK, dV)):
            gh = got.reshape(B * H, n, d)[h].float().cpu().numpy()
            assert fro_rel(gh, ref[0, 0]) <= BF16_GRAD_FRO_REL


def test_backward_is_deterministic():
    import torch
    import exact_attention_69_amd as ea
    from helpers import to_device
    wl = make_case(1, 2, 300, 64, "bf16", window=50)
    t = to_device(draw_inputs(wl), "bf16")
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], window=50)
    g1 = ea.attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, window=50)
    g2 = ea.attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, window=50)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_outputs_written_on_other_stream():
    import torch
    import exact_attention_69_amd as ea
    from helpers import to_device
    wl = make_case(1, 1, 256, 64, "bf16")
    inputs = draw_inputs(wl)
    t = to_device(inputs, "bf16")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = ea.attn_fwd(t["q"], t["k"], t["v"])
    s.synchronize()
    ref = oracle_case(wl, inputs)
    check_outputs("bf16", {"o": o.float().cpu().numpy(), "lse": lse.cpu().numpy()}, ref, "stream")


@pytest.mark.parametrize("dtype,window", [("bf16", -1), ("bf16", 40), ("f32", -1)])
def test_staged_backward_matches_attn_bwd(dtype, window):
    # rowdot, then dK/dV and dQ as separate calls (dQ on a second stream)
    # produce exactly the bits of the one-call backward.
    import torch
    import exact_attention_69_amd as ea
    from helpers import to_device
    wl = make_case(2, 2, 333, 128 if dtype == "bf16" else 64, dtype, window)
    t = to_device(draw_inputs(wl), dtype)
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], window=window)
    ref = ea.attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, window=window)
    ws = ea.attn_bwd_rowdot(o, t["do"], lse)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    dk, dv = ea.attn_bwd_dkdv(t["q"], t["k"], t["v"], t["do"], lse, ws, window=window)
    with torch.cuda.stream(side):
        dq = ea.attn_bwd_dq(t["q"], t["k"], t["v"], t["do"], lse, ws, window=window, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,Hkv", [(64, 2), (128, 4), (256, 1)])
def test_windowed_backward_on_two_streams_stays_ordered_on_its_stream(d, Hkv):
    """With a window, attn_bwd puts its dK/dV stage on a second stream forked
    from the call's stream after the rowdot stage and joined back before it
    returns.  Two calls in a row on a stream that is not the current one write
    into the same gradient tensors; copies taken on that stream right after
    each call, with no host synchronisation, must equal the one-stream staged
    backward (rowdot, dK/dV, dQ in order) bit for bit."""
    import torch
    import exact_attention_69_amd as ea
    B, H, n, w = 2, 4, 1500, 100
    print(f"[parity] two-stream backward d={d} Hkv={Hkv} n={n} window={w}", flush=True)
    cur = torch.cuda.current_stream()
    s = torch.cuda.Stream()
    dq = torch.empty(B, H, n, d, dtype=torch.bfloat16, device="cuda")
    dk = torch.empty(B, Hkv, n, d, dtype=torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    got, want, keep = [], [], []
    for seed in (5, 6):
        g = torch.Generator().manual_seed(seed)
        q, do = (torch.randn(B, H, n, d, generator=g).bfloat16().cuda() for _ in range(2))
        k, v = (torch.randn(B, Hkv, n, d, generator=g).bfloat16().cuda() for _ in range(2))
        s.wait_stream(cur)
        o, lse = ea.attn_fwd_gqa(q, k, v, window=w, stream=s)
        ea.attn_bwd_gqa(q, k, v, o, do, lse, window=w, dq=dq, dk=dk, dv=dv, stream=s)
        with torch.cuda.stream(s):
            got.append(tuple(x.clone() for x in (dq, dk, dv)))
        ws = ea.attn_bwd_rowdot(o, do, lse, stream=s)
        rk, rv = ea.attn_bwd_dkdv_gqa(q, k, v, do, lse, ws, window=w, stream=s)
        rq = ea.attn_bwd_dq_gqa(q, k, v, do, lse, ws, window=w, stream=s)
        want.append((rq, rk, rv))
        keep.append((q, k, v, do, o, lse, ws))
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    assert not torch.equal(got[0][0], got[1][0])


def test_binding_checks_caller_outputs():
    """Outputs handed to the binding must have the exact shape, dtype and
    layout of the ones it would allocate; a wrong one is refused before any
    launch, and a right one receives the same bits as an allocated one."""
    import torch
    import exact_attention_69_amd as ea
    g = torch.Generator().manual_seed(3)
    q, k, v, do = (torch.randn(1, 2, 100, 64, generator=g).bfloat16().cuda() for _ in range(4))
    o, lse = ea.attn_fwd(q, k, v)
    bad = [dict(out=torch.empty(1, 2, 99, 64, dtype=torch.bfloat16, device="cuda")),
           dict(out=torch.empty(1, 2, 100, 64, dtype=torch.float32, device="cuda")),
           dict(lse=torch.empty(1, 2, 100, dtype=torch.bfloat16, device="cuda")),
           dict(out=torch.empty(1, 2, 64, 100, dtype=torch.bfloat16, device="cuda").transpose(2, 3))]
    for kw in bad:
        with pytest.raises(ValueError):
            ea.attn_fwd(q, k, v, **kw)
    with pytest.raises(ValueError):
        ea.attn_bwd(q, k, v, o, do, lse, dk=torch.empty(1, 2, 100, 32, dtype=torch.bfloat16, device="cuda"))
    # a workspace in host memory, or a strided one, is refused as well
    with pytest.raises(ValueError):
        ea.attn_bwd(q, k, v, o, do, lse, workspace=torch.empty(1 << 16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        ea.attn_bwd_rowdot(o, do, lse, workspace=torch.empty(2, 1 << 16, dtype=torch.uint8, device="cuda")[:, ::2])
    o2 = torch.empty_like(q)
    lse2 = torch.empty_like(lse)
    ea.attn_fwd(q, k, v, out=o2, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_windowed_backward_from_two_threads():
    """Two host threads, each with its own stream and inputs, call the
    windowed attn_bwd (whose dK/dV stage goes to the device's shared second
    stream) six times each at the same time.  Every call's gradients must
    equal that thread's one-stream staged backward bit for bit."""
    import threading
    import torch
    import exact_attention_69_amd as ea
    B, H, n, d, w = 1, 4, 700, 128, 64
    print(f"[parity] two-thread windowed backward n={n} d={d} window={w}", flush=True)
    cur = torch.cuda.current_stream()
    jobs = []
    for seed in (11, 12):
        g = torch.Generator().manual_seed(seed)
        q, k, v, do = (torch.randn(B, H, n, d, generator=g).bfloat16().cuda() for _ in range(4))
        o, lse = ea.attn_fwd(q, k, v, window=w)
        ws = ea.attn_bwd_rowdot(o, do, lse)
        rk, rv = ea.attn_bwd_dkdv(q, k, v, do, lse, ws, window=w)
        rq = ea.attn_bwd_dq(q, k, v, do, lse, ws, window=w)
        jobs.append(dict(args=(q, k, v, o, do, lse), ref=(rq, rk, rv), stream=torch.cuda.Stream(), got=[]))
    torch.cuda.synchronize()
    errors = []

    def work(job):
        try:
            s = job["stream"]
            s.wait_stream(cur)
            with torch.cuda.stream(s):
                for _ in range(6):
                    out = ea.attn_bwd(*job["args"], window=w, stream=s)
                    job["got"].append(tuple(x.clone() for x in out))
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for job in jobs:
        assert len(job["got"]) == 6
        for got in job["got"]:
            for x, y in zip(got, job["ref"]):
                assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rowdot_workspace_holds_negated_d_and_base2_lse(dtype):
    """attn_bwd_rowdot's workspace: -D = -rowsum(dO * O) in the first region
    and LSE * log2(e) in the second (each region starts on a 256-byte
    boundary), from the O and dO the call was handed."""
    import torch

    import exact_attention_69_amd as ea
    from helpers import to_device

    B, H, n, d = 1, 2, 300, 128
    wl = make_case(B, H, n, d, dtype, seed=31)
    print(f"[parity] rowdot workspace {wl.name}", flush=True)
    t = to_device(draw_inputs(wl), dtype)
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], wl.scale)
    ws = ea.attn_bwd_rowdot(o, t["do"], lse)
    torch.cuda.synchronize()
    rows = B * H * n
    region = -(-rows * 4 // 256) * 256 // 4
    w = ws.view(torch.float32).cpu().numpy().astype(np.float64)
    o64 = o.float().cpu().numpy().astype(np.float64).reshape(rows, d)
    do64 = t["do"].float().cpu().numpy().astype(np.float64).reshape(rows, d)
    neg_d = -np.sum(o64 * do64, axis=1)
    scale = np.max(np.abs(o64)) * np.max(np.abs(do64)) * d
    assert np.max(np.abs(w[:rows] - neg_d)) <= 1e-6 * scale
    lse2 = lse.cpu().numpy().astype(np.float64).reshape(rows) * np.log2(np.e)
    assert np.max(np.abs(w[region:region + rows] - lse2)) <= 1e-6 * np.max(np.abs(lse2))


def test_explicit_stream_allocations_belong_to_that_stream():
    """attn_bwd(stream=s) called while another stream is current: the
    workspace it allocates and frees must not be handed to work on the current
    stream while s still runs.  A spin kernel holds s back, the call queues
    behind it, and same-size tensors are then allocated and filled with NaN
    on the current stream; the gradients must still equal an eager call's bit
    for bit."""
    import torch
    import exact_attention_69_amd as ea
    from helpers import to_device
    wl = make_case(1, 2, 300, 128, "bf16", seed=77)
    print(f"[parity] explicit stream {wl.name}", flush=True)
    t = to_device(draw_inputs(wl), "bf16")
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"])
    ref = ea.attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse)
    torch.cuda.synchronize()
    ws_bytes = max(ea.attn_bwd_workspace_bytes(ea.EXATTN_BF16, *wl_shape(wl)), 256)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        torch.cuda._sleep(50_000_000)  # a bounded spin (clock cycles) ahead of the call on s
    got = ea.attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, stream=s)
    junk = [torch.empty(ws_bytes, dtype=torch.uint8, device="cuda").fill_(0xFF) for _ in range(4)]
    junk += [torch.empty_like(t["q"]).fill_(float("nan")) for _ in range(3)]
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    del junk


def wl_shape(wl):
    return wl.B, wl.H, wl.n, wl.d
