"""A seeded sweep of small problems: HIP path against the fp64 oracle.

The hand-picked shapes of the other parity tests are chosen for the tile
boundaries they cross.  This sweep adds 40 shapes drawn from a fixed
generator: every head dim, both element types, one to four query heads with
every valid key/value head count, lengths from 1 to 1100 rows (mostly not
multiples of any tile), and windows from 0 to past the sequence length as
well as none.  Each case runs the forward and the backward through the C ABI
and compares O, LSE, dQ, dK and dV element by element with the oracle, to
the same tolerances as the rest of the parity tests.
"""

import numpy as np
import pytest

from helpers import check_outputs, draw_inputs, make_case, oracle_case, run_gpu

pytestmark = pytest.mark.gpu


def _cases(count=40, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        d = int(rng.choice([64, 128, 256]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        H = int(rng.integers(1, 5))
        Hkv = int(rng.choice([h for h in range(1, H + 1) if H % h == 0]))
        B = int(rng.integers(1, 3))
        n = int(rng.choice([1, 2, 31, 33]) if rng.random() < 0.15 else rng.integers(3, 1101))
        r = rng.random()
        window = -1 if r < 0.4 else 0 if r < 0.5 else int(rng.integers(1, n + 40))
        # keep the oracle's work per case small
        while B * H * n * n * d > 6e8 and n > 64:
            n //= 2
        out.append((i, B, H, Hkv, n, d, dtype, window))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"s{c[0]}_b{c[1]}h{c[2]}kv{c[3]}n{c[4]}d{c[5]}{c[6]}w{c[7]}")
def test_sweep_matches_oracle(case):
    i, B, H, Hkv, n, d, dtype, window = case
    wl = make_case(B, H, n, d, dtype, window, seed=5000 + i, kv_heads=Hkv if Hkv != H else 0)
    print(f"[sweep] {wl.name}", flush=True)
    inputs = draw_inputs(wl)
    got = run_gpu(wl, inputs)
    ref = oracle_case(wl, inputs)
    errs = check_outputs(dtype, got, ref, wl.name)
    print(f"[sweep] {wl.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
