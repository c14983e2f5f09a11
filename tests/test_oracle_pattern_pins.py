"""Pins of the sparse-pattern oracle (window + global tokens + block layout)
to facts other than itself (CPU only): PyTorch's float64 masked
scaled_dot_product_attention and autograd, closed forms for Q = 0, the
Longformer property that a global row attends to everything, independent
blocks under a block-diagonal layout, the plain-window oracle, finite
differences, and the empty-row convention."""

import math

import numpy as np
import pytest

import oracle
from oracle import Pattern

RNG = np.random.default_rng(4321)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def random_pattern(n, window, n_global, block, density, seed):
    g = np.random.default_rng(seed)
    glob = tuple(sorted(g.choice(n, size=n_global, replace=False))) if n_global else ()
    layout = None
    if block:
        nb = -(-n // block)
        layout = g.random((nb, nb)) < density
    return Pattern(n, window, glob, block, layout)


PATTERNS = [
    (40, 3, 0, 0, 0.0),     # window only
    (40, 2, 3, 0, 0.0),     # Longformer: window + global tokens
    (40, -1, 0, 8, 0.3),    # block layout only (may leave rows empty: excluded below)
    (45, 1, 2, 8, 0.25),    # all three, ragged last block
    (33, 0, 1, 16, 0.2),
]


@pytest.mark.parametrize("n,window,n_global,block,density", PATTERNS)
def test_matches_torch_masked_sdpa_and_autograd(n, window, n_global, block, density):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    pat = random_pattern(n, window, n_global, block, density, seed=n + 7 * n_global)
    vis = pat.visible(np.arange(n))
    keep = vis.any(axis=1)  # torch returns NaN for rows with no visible key
    d, s = 6, 1.0 / math.sqrt(6)
    q, k, v, do = rand(2, n, d), rand(2, n, d), rand(2, n, d), rand(2, n, d)
    do[:, ~keep] = 0.0
    O, lse = oracle.attention_forward_pattern(q, k, v, s, pat)
    dq, dk, dv = oracle.attention_backward_pattern(q, k, v, do, s, pat)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    tO = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(vis), scale=s)
    tO = torch.where(torch.tensor(keep)[:, None], tO, torch.zeros_like(tO))
    tO.backward(torch.tensor(do))
    np.testing.assert_allclose(O[:, keep], tO.detach().numpy()[:, keep], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)
    # LSE independently: log of the masked sum of exponentials
    S = s * np.einsum("hid,hjd->hij", q, k)
    ref = np.log(np.where(vis, np.exp(S), 0.0).sum(-1)[:, keep])
    np.testing.assert_allclose(lse[:, keep], ref, rtol=1e-12, atol=1e-12)


def test_window_only_pattern_equals_window_oracle():
    n, d = 50, 5
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    for w in (0, 2, 7):
        a = oracle.attention_forward_pattern(q, k, v, 0.4, Pattern(n, w)) + \
            oracle.attention_backward_pattern(q, k, v, do, 0.4, Pattern(n, w))
        b = oracle.attention_forward(q, k, v, 0.4, w) + oracle.attention_backward(q, k, v, do, 0.4, w)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


def test_zero_query_counts_visible_keys():
    # Q = 0: LSE_i = ln(#visible keys of row i), O_i = their mean value.
    n, d = 36, 4
    pat = random_pattern(n, 2, 3, 6, 0.3, seed=11)
    k, v = rand(n, d), rand(n, d)
    O, lse = oracle.attention_forward_pattern(np.zeros((n, d)), k, v, 0.7, pat)
    vis = pat.visible(np.arange(n))
    for i in range(n):
        cnt = vis[i].sum()
        assert lse[i] == pytest.approx(math.log(cnt), abs=1e-13)
        np.testing.assert_allclose(O[i], v[vis[i]].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_global_rows_attend_everything_and_everyone_attends_globals():
    n, d, w = 30, 4, 1
    glob = (0, 17)
    pat = Pattern(n, w, glob)
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    O, lse = oracle.attention_forward_pattern(q, k, v, 0.5, pat)
    Of, lf = oracle.attention_forward(q, k, v, 0.5, -1)
    for g in glob:  # a global row is plain full attention
        np.testing.assert_allclose(O[g], Of[g], rtol=1e-12, atol=1e-13)
        assert lse[g] == pytest.approx(lf[g], rel=1e-13)
    # a non-global row sees its window plus the global keys, nothing else
    i = 9
    keys = sorted(set(range(i - w, i + w + 1)) | set(glob))
    S = 0.5 * q[i] @ k[keys].T
    p = np.exp(S - S.max())
    np.testing.assert_allclose(O[i], (p / p.sum()) @ v[keys], rtol=1e-12, atol=1e-13)


def test_block_diagonal_layout_is_independent_blocks():
    n, b, d = 48, 16, 5
    layout = np.eye(n // b, dtype=bool)
    pat = Pattern(n, -1, (), b, layout)
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    O, lse = oracle.attention_forward_pattern(q, k, v, 0.3, pat)
    dq, dk, dv = oracle.attention_backward_pattern(q, k, v, do, 0.3, pat)
    for r in range(0, n, b):
        sl = slice(r, r + b)
        Ob, lb = oracle.attention_forward(q[sl], k[sl], v[sl], 0.3)
        gq, gk, gv = oracle.attention_backward(q[sl], k[sl], v[sl], do[sl], 0.3)
        np.testing.assert_allclose(O[sl], Ob, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[sl], lb, rtol=1e-13, atol=1e-13)
        for x, y in ((dq[sl], gq), (dk[sl], gk), (dv[sl], gv)):
            np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-12)


def test_full_layout_is_dense_attention():
    n, b, d = 40, 8, 4
    pat = Pattern(n, -1, (), b, np.ones((5, 5), dtype=bool))
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    for x, y in zip(oracle.attention_forward_pattern(q, k, v, 0.6, pat), oracle.attention_forward(q, k, v, 0.6)):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


def test_gradients_match_finite_differences():
    n, d, s = 14, 3, 0.8
    pat = random_pattern(n, 1, 2, 4, 0.3, seed=5)
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    dq, dk, dv = oracle.attention_backward_pattern(q, k, v, do, s, pat)
    L = lambda a, b_, c: np.sum(oracle.attention_forward_pattern(a, b_, c, s, pat)[0] * do)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0), (5, 2), (13, 1)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (L(*args_p) - L(*args_m)) / (2 * eps)
            assert g[idx] == pytest.approx(fd, rel=1e-6, abs=1e-8), (name, idx)


def test_empty_rows_follow_the_convention():
    # no window, no globals, a layout with an empty block row: those rows get
    # O = 0, LSE = -inf, zero dQ, and add nothing to dK, dV.
    n, b, d = 24, 8, 3
    layout = np.array([[1, 1, 0], [0, 0, 0], [0, 1, 1]], dtype=bool)
    pat = Pattern(n, -1, (), b, layout)
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    O, lse = oracle.attention_forward_pattern(q, k, v, 0.5, pat)
    dq, dk, dv = oracle.attention_backward_pattern(q, k, v, do, 0.5, pat)
    assert np.all(O[8:16] == 0.0) and np.all(np.isneginf(lse[8:16])) and np.all(dq[8:16] == 0.0)
    do2 = do.copy()
    do2[8:16] = rand(8, d)  # changing dO of empty rows changes nothing
    _, dk2, dv2 = oracle.attention_backward_pattern(q, k, v, do2, 0.5, pat)
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)
    assert np.all(np.isfinite(lse[:8])) and np.all(np.isfinite(lse[16:]))


def test_row_blocking_does_not_change_result():
    n, d = 70, 4
    pat = random_pattern(n, 3, 4, 16, 0.3, seed=9)
    q, k, v, do = rand(2, n, d), rand(2, n, d), rand(2, n, d), rand(2, n, d)
    ref = oracle.attention_forward_pattern(q, k, v, 0.3, pat, row_block=n) + \
        oracle.attention_backward_pattern(q, k, v, do, 0.3, pat, row_block=n)
    got = oracle.attention_forward_pattern(q, k, v, 0.3, pat, row_block=9) + \
        oracle.attention_backward_pattern(q, k, v, do, 0.3, pat, row_block=9)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
