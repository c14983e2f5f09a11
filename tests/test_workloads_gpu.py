"""GPU parity at the five full workload sizes, launched exactly as bench.py does.

For each workload the whole problem runs on the GPU; the fp64 oracle checks
selected heads completely (every output element of those heads), and
whole-tensor identities of the exact gradients check every head.
"""

import sys
import time

import numpy as np
import pytest

from helpers import check_outputs, invariant_errors, oracle_case, run_gpu, select_heads
from workloads import WORKLOADS, draw_inputs

pytestmark = pytest.mark.gpu

# flat (b*H + h) head indices compared against the oracle, per workload
ORACLE_HEADS = {
    "single_head_f32_n256_d64": [0],
    "bf16_b4h16_n2048_d64": [0, 37],
    "bf16_b2h32_n8192_d128_q3": [0, 63],
    "bf16_b1h16_n32768_d128": [0],
    "bf16_b2h8_n16384_d256_w512": [0, 15],
}
INVARIANT_TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.mark.parametrize("wl", WORKLOADS, ids=[w.name for w in WORKLOADS])
def test_workload_parity(wl):
    t0 = time.time()
    print(f"[workload] {wl.name}: drawing inputs", flush=True)
    inputs = draw_inputs(wl)
    print(f"[workload] {wl.name}: GPU fwd+bwd ({time.time() - t0:.1f}s)", flush=True)
    got = run_gpu(wl, inputs)
    heads = ORACLE_HEADS[wl.name]
    print(f"[workload] {wl.name}: oracle on heads {heads} ({time.time() - t0:.1f}s)", flush=True)
    ref = oracle_case(wl, inputs, heads)
    errs = check_outputs(wl.dtype, select_heads(got, wl, heads), ref, wl.name)
    print(f"[workload] {wl.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert np.all(np.isfinite(got[key])), f"{wl.name}: non-finite {key}"
    inv = invariant_errors(inputs, got, wl)
    print(f"[workload] {wl.name}: invariants " + " ".join(f"{k}={v:.2e}" for k, v in inv.items())
          + f" ({time.time() - t0:.1f}s)", flush=True)
    sys.stdout.flush()
    tol = INVARIANT_TOL[wl.dtype]
    for k, v in inv.items():
        assert v <= tol, f"{wl.name}: invariant {k} = {v:.3e} > {tol}"
