"""Pins of the fp64 oracle to facts other than itself (CPU only).

Each test checks the oracle against something the pages or the mathematics
fix: closed forms, invariants, finite differences, the corrected two-block
softmax merge, and an independent library routine (PyTorch's float64 CPU
scaled_dot_product_attention and its autograd).  The tests are chosen so that
a dropped term, a wrong sign, a wrong scale, a transposed operand or a wrong
window bound in the oracle fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import pair_count, round_to_bf16, draw_head, workload

RNG = np.random.default_rng(1234)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
WINDOWS = [-1, 0, 1, 2, 5]


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def window_mask(n, window):
    i = np.arange(n)
    if window < 0:
        return np.ones((n, n), dtype=bool)
    return np.abs(i[:, None] - i[None, :]) <= window


# --------------------------------------------------------------------------
# Forward: closed forms and invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("window", WINDOWS)
def test_probability_rows_sum_to_one_and_respect_window(window):
    n, d = 13, 4
    q, k = rand(2, n, d), rand(2, n, d)
    P = oracle.attention_probs(q, k, 0.7, window)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert np.all(P[:, ~window_mask(n, window)] == 0.0)
    assert np.all(P[:, window_mask(n, window)] > 0.0)


@pytest.mark.parametrize("window", WINDOWS)
def test_zero_query_gives_window_mean_of_values(window):
    # Q = 0: every score is 0, so each row averages its visible values and
    # LSE = ln(#keys).
    n, d = 11, 3
    q = np.zeros((n, d))
    k, v = rand(n, d), rand(n, d)
    O, lse = oracle.attention_forward(q, k, v, 0.5, window)
    for i in range(n):
        lo, hi = oracle.key_range(i, n, window)
        np.testing.assert_allclose(O[i], v[lo:hi].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert lse[i] == pytest.approx(math.log(hi - lo), abs=1e-14)


def test_constant_values_give_constant_output():
    n, d = 17, 5
    q, k = rand(n, d, scale=3), rand(n, d)
    v = np.ones((n, d))
    for window in WINDOWS:
        O, _ = oracle.attention_forward(q, k, v, 0.9, window)
        np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-14)


def test_window_zero_is_identity():
    n, d, s = 9, 4, 0.37
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    O, lse = oracle.attention_forward(q, k, v, s, 0)
    np.testing.assert_allclose(O, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, s * np.sum(q * k, axis=1), rtol=1e-14, atol=1e-14)


def test_key_value_permutation_invariance():
    n, d = 15, 6
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    perm = RNG.permutation(n)
    O1, lse1 = oracle.attention_forward(q, k, v, 0.4)
    O2, lse2 = oracle.attention_forward(q, k[perm], v[perm], 0.4)
    np.testing.assert_allclose(O1, O2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("window", WINDOWS)
def test_key_shift_changes_only_lse(window):
    # Adding u to every key adds scale*q_i.u to every score of row i: the
    # softmax is unchanged and LSE shifts by that amount.
    n, d, s = 12, 4, 0.6
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    u = rand(d)
    O1, lse1 = oracle.attention_forward(q, k, v, s, window)
    O2, lse2 = oracle.attention_forward(q, k + u, v, s, window)
    np.testing.assert_allclose(O1, O2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2 - lse1, s * q @ u, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", WINDOWS)
def test_lse_bounds(window):
    n, d, s = 14, 5, 1.3
    q, k, v = rand(n, d, scale=2), rand(n, d), rand(n, d)
    _, lse = oracle.attention_forward(q, k, v, s, window)
    S = s * q @ k.T
    S[~window_mask(n, window)] = -np.inf
    smax = S.max(axis=1)
    cnt = oracle.keys_per_row(n, window)
    assert np.all(lse >= smax - 1e-13)
    assert np.all(lse <= smax + np.log(cnt) + 1e-13)


def test_scale_enters_scores_linearly():
    # scale*Q K^T: doubling the scale equals doubling Q.
    n, d = 10, 4
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    O1, l1 = oracle.attention_forward(q, k, v, 0.8)
    O2, l2 = oracle.attention_forward(2 * q, k, v, 0.4)
    np.testing.assert_allclose(O1, O2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-14)


def test_one_dominant_key_selects_its_value():
    # A score far above the others makes the row's output that key's value
    # (the sharp-retrieval limit of softmax attention).
    n, d = 8, 3
    k = rand(n, d)
    q = 200.0 * k[[5]] / np.linalg.norm(k[5]) ** 2 * np.ones((1, 1))
    q = np.repeat(q, n, axis=0)
    kk = k.copy()
    kk[np.arange(n) != 5] *= 0.0
    v = rand(n, d)
    O, lse = oracle.attention_forward(q, kk, v, 1.0)
    np.testing.assert_allclose(O, np.repeat(v[[5]], n, axis=0), rtol=1e-12, atol=1e-12)
    assert lse[0] == pytest.approx(200.0, rel=1e-12)


# --------------------------------------------------------------------------
# Forward: blocking inside the oracle and the single-row helpers
# --------------------------------------------------------------------------

@pytest.mark.parametrize("window", [-1, 3, 20])
def test_row_blocking_and_band_do_not_change_result(window):
    n, d = 70, 8
    q, k, v, do = rand(2, n, d), rand(2, n, d), rand(2, n, d), rand(2, n, d)
    ref = oracle.attention_forward(q, k, v, 0.3, window, row_block=n, band=False)
    refb = oracle.attention_backward(q, k, v, do, 0.3, window, row_block=n, band=False)
    for rb in (1, 7, 32):
        for band in (False, True):
            got = oracle.attention_forward(q, k, v, 0.3, window, row_block=rb, band=band)
            gotb = oracle.attention_backward(q, k, v, do, 0.3, window, row_block=rb, band=band)
            for a, b in zip(got + gotb, ref + refb):
                np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("window", [-1, 4])
def test_single_row_helpers_match_full_oracle(window):
    n, d = 40, 6
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    O, lse = oracle.attention_forward(q, k, v, 0.45, window)
    dq, _, _ = oracle.attention_backward(q, k, v, do, 0.45, window)
    rows = [0, 3, 17, 39]
    Or, lr = oracle.forward_rows(q, k, v, 0.45, window, rows)
    dqr = oracle.backward_dq_rows(q, k, v, do, 0.45, window, rows)
    np.testing.assert_allclose(Or, O[rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lr, lse[rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dqr, dq[rows], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# Independent library routine: PyTorch float64 on the CPU
# --------------------------------------------------------------------------

@pytest.mark.parametrize("window", [-1, 0, 3])
@pytest.mark.parametrize("n,d", [(1, 4), (9, 8), (33, 16)])
def test_matches_torch_sdpa_and_autograd(n, d, window):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    s = 1.0 / math.sqrt(d)
    q, k, v, do = rand(2, n, d), rand(2, n, d), rand(2, n, d), rand(2, n, d)
    O, lse = oracle.attention_forward(q, k, v, s, window)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, s, window)

    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    mask = torch.tensor(window_mask(n, window))
    tO = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=s)
    tO.backward(torch.tensor(do, dtype=torch.float64))
    np.testing.assert_allclose(O, tO.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)

    from scipy.special import logsumexp
    S = s * np.einsum("bid,bjd->bij", q, k)
    S[:, ~window_mask(n, window)] = -np.inf
    np.testing.assert_allclose(lse, logsumexp(S, axis=-1), rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Grouped-query attention (K/V heads shared by groups of query heads)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (6, 1), (8, 2)])
@pytest.mark.parametrize("window", [-1, 2])
def test_gqa_matches_torch_sdpa_enable_gqa(H, Hkv, window):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    n, d = 11, 6
    s = 1.0 / math.sqrt(d)
    q, do = rand(2, H, n, d), rand(2, H, n, d)
    k, v = rand(2, Hkv, n, d), rand(2, Hkv, n, d)
    O, lse = oracle.attention_forward_gqa(q, k, v, s, window)
    dq, dk, dv = oracle.attention_backward_gqa(q, k, v, do, s, window)
    assert dk.shape == k.shape and dv.shape == v.shape and dq.shape == q.shape
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    mask = torch.tensor(window_mask(n, window))
    tO = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=s, enable_gqa=True)
    tO.backward(torch.tensor(do, dtype=torch.float64))
    np.testing.assert_allclose(O, tO.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_gqa_with_one_group_is_multi_head():
    q, k, v, do = rand(1, 3, 9, 4), rand(1, 3, 9, 4), rand(1, 3, 9, 4), rand(1, 3, 9, 4)
    a = oracle.attention_forward_gqa(q, k, v, 0.5) + oracle.attention_backward_gqa(q, k, v, do, 0.5)
    b = oracle.attention_forward(q, k, v, 0.5) + oracle.attention_backward(q, k, v, do, 0.5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_gqa_identical_query_heads_scale_kv_gradients():
    # If every query head of a group carries the same Q and dO, the group's
    # dK and dV are G times those of a single head.
    n, d, G = 10, 4, 3
    q1, do1 = rand(1, 1, n, d), rand(1, 1, n, d)
    k, v = rand(1, 1, n, d), rand(1, 1, n, d)
    q, do = np.repeat(q1, G, axis=1), np.repeat(do1, G, axis=1)
    _, dk, dv = oracle.attention_backward_gqa(q, k, v, do, 0.6)
    _, dk1, dv1 = oracle.attention_backward(q1, k, v, do1, 0.6)
    np.testing.assert_allclose(dk, G * dk1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dv, G * dv1, rtol=1e-13, atol=1e-14)


def test_gqa_rejects_ragged_groups():
    with pytest.raises(ValueError):
        oracle.attention_forward_gqa(rand(1, 5, 4, 2), rand(1, 2, 4, 2), rand(1, 2, 4, 2), 1.0)


# --------------------------------------------------------------------------
# Backward: finite differences, closed forms, invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("window", [-1, 0, 1, 2])
@pytest.mark.parametrize("n,d", [(3, 2), (7, 5), (16, 8)])
def test_backward_matches_central_differences(n, d, window):
    s = 0.8
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    grads = oracle.attention_backward(q, k, v, do, s, window)

    def loss(q_, k_, v_):
        return float(np.sum(oracle.attention_forward(q_, k_, v_, s, window)[0] * do))

    h = 1e-6
    for which, g in enumerate(grads):
        args = [q, k, v]
        fd = np.zeros_like(args[which])
        for idx in np.ndindex(*fd.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        scale_ = max(1.0, np.abs(g).max())
        np.testing.assert_allclose(g, fd, rtol=0, atol=2e-8 * scale_)


@pytest.mark.parametrize("window", [-1, 1, 4])
def test_zero_query_backward_closed_form(window):
    n, d = 10, 3
    q = np.zeros((n, d))
    k, v, do = rand(n, d), rand(n, d), rand(n, d)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.7, window)
    np.testing.assert_allclose(dk, 0.0, rtol=0, atol=1e-14)
    cnt = oracle.keys_per_row(n, window)
    expect = np.zeros((n, d))
    for i in range(n):
        lo, hi = oracle.key_range(i, n, window)
        expect[lo:hi] += do[i] / cnt[i]
    np.testing.assert_allclose(dv, expect, rtol=1e-13, atol=1e-14)


def test_zero_key_gives_zero_dq():
    n, d = 9, 4
    q, v, do = rand(n, d), rand(n, d), rand(n, d)
    dq, _, _ = oracle.attention_backward(q, np.zeros((n, d)), v, do, 0.7)
    np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-14)


def test_window_zero_backward_closed_form():
    n, d = 9, 4
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.7, 0)
    np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)


@pytest.mark.parametrize("window", [-1, 2, 6])
def test_backward_invariants(window):
    n, d, s = 25, 6, 0.55
    q, k, v, do = rand(n, d, scale=2), rand(n, d), rand(n, d), rand(n, d)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, s, window)
    # softmax is invariant to a common shift of a row's scores: sum_j dK_j = 0
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-12)
    # probability rows sum to one: sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)
    # scores are invariant under Q -> tQ, K -> K/t
    assert np.sum(dq * q) == pytest.approx(np.sum(dk * k), rel=1e-11, abs=1e-11)


# --------------------------------------------------------------------------
# Two-block softmax merge (unite.ai page, second formula of its maths section)
# --------------------------------------------------------------------------

def _softmax(x):
    from scipy.special import softmax
    return softmax(np.asarray(x, dtype=np.float64))


def _literal_page_merge(x, y):
    # The combination formula exactly as printed: a softmax of the two block
    # softmaxes rescaled to the common maximum, with no block sums.
    m_x, m_y = np.max(x), np.max(y)
    m = max(m_x, m_y)
    return _softmax(np.concatenate([_softmax(x) * np.exp(m_x - m), _softmax(y) * np.exp(m_y - m)]))


def test_merge_counterexample():
    x, y = np.array([0.0]), np.array([0.0, 0.0])
    got = oracle.merge_softmax_blocks(x, y)
    np.testing.assert_allclose(got, [1 / 3, 1 / 3, 1 / 3], rtol=0, atol=1e-16)
    literal = _literal_page_merge(x, y)
    assert np.max(np.abs(literal - 1 / 3)) > 0.1  # the printed form is not the softmax


@pytest.mark.parametrize("trial", range(5))
def test_merge_equals_softmax_of_union(trial):
    x = rand(int(RNG.integers(1, 20)), scale=5)
    y = rand(int(RNG.integers(1, 20)), scale=5) + RNG.normal() * 10
    got = oracle.merge_softmax_blocks(x, y)
    np.testing.assert_allclose(got, _softmax(np.concatenate([x, y])), rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("window", [-1, 3])
def test_merge_of_partial_outputs_equals_full_attention(window):
    n, d, s = 20, 5, 0.9
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    O, lse = oracle.attention_forward(q, k, v, s, window)
    split = 8
    S = s * q @ k.T
    S[~window_mask(n, window)] = -np.inf

    def part(cols):
        Sc = S[:, cols]
        m = Sc.max(axis=1, keepdims=True)
        e = np.exp(Sc - m)
        return (e @ v[cols]) / e.sum(1, keepdims=True), (m + np.log(e.sum(1, keepdims=True)))[:, 0]

    # rows whose window lies wholly in one part get lse = -inf there; use the
    # no-window case and rows with keys on both sides for the merge check
    rows = [i for i in range(n) if oracle.key_range(i, n, window)[0] < split <= oracle.key_range(i, n, window)[1] - 1]
    Ox, lx = part(np.arange(0, split))
    Oy, ly = part(np.arange(split, n))
    Om, lm = oracle.merge_partial_outputs(Ox[rows], lx[rows], Oy[rows], ly[rows])
    np.testing.assert_allclose(Om, O[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lm, lse[rows], rtol=1e-13, atol=1e-13)


def test_online_softmax_over_key_blocks_is_exact():
    # Tiling exactness (llmis.ru chapter 3.1, section 5): an independent
    # online softmax over key blocks, keeping a running max, running sum and
    # unnormalised output, reproduces the oracle for any block size.
    n, d, s = 50, 7, 0.5
    q, k, v = rand(n, d, scale=3), rand(n, d), rand(n, d)
    O, lse = oracle.attention_forward(q, k, v, s)
    for bc in (1, 7, 16, 50):
        m = np.full(n, -np.inf)
        l = np.zeros(n)
        acc = np.zeros((n, d))
        for c0 in range(0, n, bc):
            Sb = s * q @ k[c0:c0 + bc].T
            m_new = np.maximum(m, Sb.max(axis=1))
            alpha = np.exp(m - m_new)
            Pb = np.exp(Sb - m_new[:, None])
            l = alpha * l + Pb.sum(axis=1)
            acc = alpha[:, None] * acc + Pb @ v[c0:c0 + bc]
            m = m_new
        np.testing.assert_allclose(acc / l[:, None], O, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(m + np.log(l), lse, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Workload helpers: page facts and bf16 rounding
# --------------------------------------------------------------------------

def test_page_cost_facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)["facts"]
    f0, f1, f2, f3 = facts
    assert pair_count(f0["n"], -1) == f0["entries"]
    assert pair_count(f1["n_to"], -1) // pair_count(f1["n_from"], -1) == f1["ratio"]
    assert pair_count(f2["n_to"], -1) // pair_count(f2["n_from"], -1) == f2["ratio"]
    # a symmetric window of half-width h has total width 2h+1 ~ w
    h = f3["window_width"] // 2
    assert round(pair_count(f3["n"], -1) / pair_count(f3["n"], h)) == f3["ratio_rounded"]


@pytest.mark.parametrize("n,w", [(1, 0), (5, 0), (5, 1), (9, 3), (16, 15), (16, 40), (300, 17)])
def test_pair_count_matches_mask(n, w):
    assert pair_count(n, w) == int(window_mask(n, w).sum())
    assert pair_count(n, w) == int(oracle.keys_per_row(n, w).sum())


def test_bf16_rounding():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38], dtype=np.float32)
    got = round_to_bf16(x)
    # ties go to even: 1+2^-8 is halfway between 1 and 1+2^-7 -> 1
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, got[5]], dtype=np.float32))
    assert (got.view(np.uint32) & 0xFFFF == 0).all()
    torch = pytest.importorskip("torch")
    y = RNG.standard_normal(10000).astype(np.float32)
    ref = torch.tensor(y).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_to_bf16(y), ref)


def test_draw_head_is_deterministic_and_peaky_scale():
    wl = workload("bf16_b2h32_n8192_d128_q3")
    a = draw_head(wl, "q", 1, 5, n=64)
    b = draw_head(wl, "q", 1, 5, n=64)
    np.testing.assert_array_equal(a, b)
    assert 2.0 < a.std() < 4.0
    c = draw_head(wl, "k", 1, 5, n=64)
    assert 0.7 < c.std() < 1.3
