"""CPU checks of the test helpers themselves: on exact (oracle) gradients the
identities that the full-size GPU tests measure are zero up to rounding, and
the head selection lines GPU outputs up with the oracle's sampled heads."""

import numpy as np

import oracle
from helpers import invariant_errors, make_case, oracle_case, select_heads
from workloads import draw_inputs


def _oracle_outputs(wl, inputs):
    ref = oracle_case(wl, inputs)
    return {k: np.asarray(v, dtype=np.float32) for k, v in ref.items()}


def test_invariants_vanish_on_exact_gradients():
    for kv in (0, 1, 2):
        wl = make_case(2, 4, 40, 8, "f32", seed=3, kv_heads=kv)
        inputs = draw_inputs(wl)
        inv = invariant_errors(inputs, _oracle_outputs(wl, inputs), wl)
        assert max(inv.values()) < 1e-5, (kv, inv)


def test_invariants_see_a_planted_error():
    wl = make_case(1, 4, 30, 8, "f32", seed=4, kv_heads=2)
    inputs = draw_inputs(wl)
    out = _oracle_outputs(wl, inputs)
    out["dv"][0, 1, 5] += 0.5
    assert invariant_errors(inputs, out, wl)["sum_dv"] > 1e-3


def test_select_heads_matches_oracle_on_sampled_groups():
    wl = make_case(2, 6, 20, 8, "f32", seed=5, kv_heads=2)
    inputs = draw_inputs(wl)
    full = _oracle_outputs(wl, inputs)
    part = oracle_case(wl, inputs, [1, 3])
    sel = select_heads(full, wl, [1, 3])
    for k in part:
        assert sel[k].shape == part[k].shape, k
        np.testing.assert_allclose(sel[k], part[k], rtol=1e-5, atol=1e-6)
    # and the group structure: key/value head 3 is batch 1, group 1, whose
    # query heads are 3, 4, 5 of that batch
    O, _ = oracle.attention_forward(inputs["q"][1, 3:6], np.repeat(inputs["k"][1, 1:2], 3, 0),
                                    np.repeat(inputs["v"][1, 1:2], 3, 0), wl.scale)
    np.testing.assert_allclose(part["o"][1], O, rtol=1e-12)
