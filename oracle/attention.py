"""fp64 CPU oracle for exact scaled dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library.

What is computed, and where the pages define it
------------------------------------------------
* Forward.  ``O = softmax(scale * Q K^T) V`` for Q, K, V of shape (n, d) per
  (batch, head), as the llmis.ru chapter 3.1 "The cost of attention" states in
  its section 2 (why self-attention is quadratic), with ``scale = 1/sqrt(d)``
  there; the unite.ai page "Flash Attention: Revolucionando a Eficiencia dos
  Modelos Transformer", section "Atencao Padrao: Um Resumo Rapido", builds the
  same (n, n) score matrix, applies a row softmax and multiplies by V.
  The softmax is evaluated in the max-subtracted form the unite.ai page gives
  as its first formula in "A Matematica por tras da Flash Attention":
  ``softmax(x) = exp(x - m) / sum(exp(x - m))`` with ``m = max(x)``.
* Log-sum-exp.  ``LSE_i = m_i + ln(l_i)`` (natural log), the single per-row
  statistic that an online-softmax forward keeps (running max m and running
  sum l, the llmis.ru chapter's section 5 on FlashAttention).
* Sliding window.  The Longformer local pattern of the llmis.ru chapter's
  section 3: each query attends a fixed number of neighbours on both sides.
  Reading used here: row i attends keys j with ``|i - j| <= window``
  (symmetric, inclusive, truncated at the sequence ends); ``window < 0`` means
  no mask.  Masked scores are -inf, so their probabilities are exactly 0.
* Backward.  The pages do not write the gradient formulas; they say only that
  the backward recomputes the attention blocks instead of storing them (the
  unite.ai page, "Entenda a Flash Attention", item 2; the llmis.ru chapter's
  section 5).  The gradients below are the chain rule applied to the forward
  definition, for the scalar loss ``L = sum(O * dO)``:
  ``dV = P^T dO``, ``dP = dO V^T``, ``D_i = sum_k dO_ik O_ik``,
  ``dS = P * (dP - D)``, ``dQ = scale dS K``, ``dK = scale dS^T Q``.
* Two-block merge.  The second formula of "A Matematica por tras da Flash
  Attention" (softmax of the union of two blocks from the blocks' own
  softmaxes and maxima) is printed without the block sums; the reading used
  here restores them: with ``m = max(m_x, m_y)``,
  ``l = e^(m_x - m) l_x + e^(m_y - m) l_y`` and
  ``softmax(x u y) = [e^(m_x - m) l_x softmax(x), e^(m_y - m) l_y softmax(y)] / l``.

Rows are processed in blocks of at most ``row_block`` rows so that the score
block fits in memory; every block still spans all the keys its rows can see,
so this is the plain two-pass softmax of the definition, not an online one.
With a window, the columns that the whole row block cannot see are skipped:
their probabilities are exactly zero, so the result is unchanged (a test shows
it equals the fully masked dense form).
"""

import numpy as np

__all__ = [
    "attention_forward_gqa",
    "attention_backward_gqa",
    "key_range",
    "keys_per_row",
    "attention_probs",
    "attention_forward",
    "attention_backward",
    "forward_rows",
    "backward_dq_rows",
    "softmax_block_stats",
    "merge_softmax_blocks",
    "merge_partial_outputs",
]


def key_range(i, n, window):
    """Half-open range [lo, hi) of the keys query row ``i`` attends to.

    Longformer local window (llmis.ru chapter 3.1, section 3), read as
    ``|i - j| <= window``; ``window < 0`` attends to all ``n`` keys.
    """
    if window < 0:
        return 0, n
    return max(0, i - window), min(n, i + window + 1)


def keys_per_row(n, window):
    """Number of keys each of the ``n`` query rows attends to (int64 array)."""
    i = np.arange(n, dtype=np.int64)
    if window < 0:
        return np.full(n, n, dtype=np.int64)
    lo = np.maximum(0, i - window)
    hi = np.minimum(n, i + window + 1)
    return hi - lo


def _as_f64(*arrays):
    return tuple(np.asarray(a, dtype=np.float64) for a in arrays)


def _block_columns(r0, r1, n, window, band):
    """Key columns a row block [r0, r1) must look at."""
    if window < 0 or not band:
        return 0, n
    return max(0, r0 - window), min(n, r1 - 1 + window + 1)


def _scores(Qb, K, scale, rows, c0, c1, window):
    """Masked scaled scores for query rows ``rows`` against keys [c0, c1)."""
    S = scale * (Qb @ K[c0:c1].T)
    if window >= 0:
        cols = np.arange(c0, c1)
        outside = np.abs(rows[:, None] - cols[None, :]) > window
        S[outside] = -np.inf
    return S


def _softmax_rows(S):
    """Max-subtracted row softmax; returns P, row max m and row sum l."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return E / l, m, l


def attention_probs(q, k, scale, window=-1):
    """Full probability matrix P = softmax(scale Q K^T) for small inputs.

    ``q``, ``k``: arrays of shape (..., n, d).  Returns (..., n, n) fp64.
    """
    q, k = _as_f64(q, k)
    n = q.shape[-2]
    out = np.empty(q.shape[:-1] + (n,), dtype=np.float64)
    rows = np.arange(n)
    for idx in np.ndindex(*q.shape[:-2]):
        S = _scores(q[idx], k[idx], scale, rows, 0, n, window)
        out[idx] = _softmax_rows(S)[0]
    return out


def attention_forward(q, k, v, scale, window=-1, row_block=1024, band=True):
    """Exact attention forward in fp64.

    ``q``, ``k``, ``v``: (..., n, d) arrays of any float dtype (upcast to fp64).
    Returns ``(O, LSE)`` with O of shape (..., n, d) and LSE (natural log) of
    shape (..., n), both fp64.
    """
    q, k, v = _as_f64(q, k, v)
    n = q.shape[-2]
    O = np.empty(q.shape, dtype=np.float64)
    LSE = np.empty(q.shape[:-1], dtype=np.float64)
    for idx in np.ndindex(*q.shape[:-2]):
        Q, K, V = q[idx], k[idx], v[idx]
        for r0 in range(0, n, row_block):
            r1 = min(n, r0 + row_block)
            c0, c1 = _block_columns(r0, r1, n, window, band)
            S = _scores(Q[r0:r1], K, scale, np.arange(r0, r1), c0, c1, window)
            P, m, l = _softmax_rows(S)
            O[idx][r0:r1] = P @ V[c0:c1]
            LSE[idx][r0:r1] = (m + np.log(l))[:, 0]
    return O, LSE


def attention_backward(q, k, v, do, scale, window=-1, row_block=1024, band=True):
    """Gradients (dQ, dK, dV) of ``L = sum(O * dO)`` in fp64.

    P is recomputed from Q and K (nothing from a forward pass is reused), and
    ``D = rowsum(dO * O)`` uses the oracle's own fp64 O.
    """
    q, k, v, do = _as_f64(q, k, v, do)
    n = q.shape[-2]
    dQ = np.zeros(q.shape, dtype=np.float64)
    dK = np.zeros(k.shape, dtype=np.float64)
    dV = np.zeros(v.shape, dtype=np.float64)
    for idx in np.ndindex(*q.shape[:-2]):
        Q, K, V, dO = q[idx], k[idx], v[idx], do[idx]
        for r0 in range(0, n, row_block):
            r1 = min(n, r0 + row_block)
            c0, c1 = _block_columns(r0, r1, n, window, band)
            S = _scores(Q[r0:r1], K, scale, np.arange(r0, r1), c0, c1, window)
            P = _softmax_rows(S)[0]
            Ob = P @ V[c0:c1]
            dOb = dO[r0:r1]
            dP = dOb @ V[c0:c1].T
            D = np.sum(dOb * Ob, axis=1, keepdims=True)
            dS = P * (dP - D)
            dQ[idx][r0:r1] = scale * (dS @ K[c0:c1])
            dK[idx][c0:c1] += scale * (dS.T @ Q[r0:r1])
            dV[idx][c0:c1] += P.T @ dOb
    return dQ, dK, dV


def forward_rows(Q, K, V, scale, window, rows):
    """O and LSE for selected query rows of ONE head (2-D Q, K, V).

    Used to check single outputs of a large problem one by one.
    """
    Q, K, V = _as_f64(Q, K, V)
    rows = np.asarray(rows, dtype=np.int64)
    n = K.shape[0]
    S = _scores(Q[rows], K, scale, rows, 0, n, window)
    P, m, l = _softmax_rows(S)
    return P @ V, (m + np.log(l))[:, 0]


def backward_dq_rows(Q, K, V, dO, scale, window, rows):
    """dQ for selected query rows of ONE head (2-D inputs).

    A row of dQ needs only that row's probabilities, its own O and dO.
    """
    Q, K, V, dO = _as_f64(Q, K, V, dO)
    rows = np.asarray(rows, dtype=np.int64)
    n = K.shape[0]
    S = _scores(Q[rows], K, scale, rows, 0, n, window)
    P = _softmax_rows(S)[0]
    Ob = P @ V
    dP = dO[rows] @ V.T
    D = np.sum(dO[rows] * Ob, axis=1, keepdims=True)
    dS = P * (dP - D)
    return scale * (dS @ K)


def softmax_block_stats(x):
    """Block statistics of a score vector: (max m, sum of exp(x - m))."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    return m, np.exp(x - m).sum()


def merge_softmax_blocks(x, y):
    """Softmax of the concatenation of x and y, built from the two blocks.

    Each block contributes only its own softmax and statistics (m, l); the
    blocks are rescaled to the common maximum and renormalised by the merged
    sum (the corrected reading of the unite.ai page's combination formula).
    """
    x, y = _as_f64(x, y)
    m_x, l_x = softmax_block_stats(x)
    m_y, l_y = softmax_block_stats(y)
    sx = np.exp(x - m_x) / l_x
    sy = np.exp(y - m_y) / l_y
    m = max(m_x, m_y)
    ax = np.exp(m_x - m) * l_x
    ay = np.exp(m_y - m) * l_y
    l = ax + ay
    return np.concatenate([ax * sx, ay * sy]) / l


def merge_partial_outputs(O_x, lse_x, O_y, lse_y):
    """Merge attention results computed over two disjoint key sets.

    ``O_x`` (rows, d) and ``lse_x`` (rows,) are the normalised output and
    log-sum-exp over the first key set, likewise for y.  Returns the output
    and log-sum-exp over the union, the same merge written with LSE.
    """
    O_x, lse_x, O_y, lse_y = _as_f64(O_x, lse_x, O_y, lse_y)
    m = np.maximum(lse_x, lse_y)
    lse = m + np.log(np.exp(lse_x - m) + np.exp(lse_y - m))
    wx = np.exp(lse_x - lse)[..., None]
    wy = np.exp(lse_y - lse)[..., None]
    return wx * O_x + wy * O_y, lse


def _group_size(q, k):
    H, Hkv = q.shape[-3], k.shape[-3]
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"query heads ({H}) must be a multiple of key/value heads ({Hkv})")
    return H // Hkv


def attention_forward_gqa(q, k, v, scale, window=-1, **kw):
    """Grouped-query attention forward (the FlashAttention-2 variants of the
    unite.ai page, section "FlashAttention-2", item 3).

    ``q``: (B, H, n, d); ``k``, ``v``: (B, Hkv, n, d) with H a multiple of
    Hkv.  Query head h attends with key/value head h // (H / Hkv): the query
    heads of one group are consecutive (Hkv = 1 is multi-query attention,
    Hkv = H the plain multi-head case).  Defined as ordinary attention with
    each key/value head repeated for its group.
    """
    G = _group_size(q, k)
    return attention_forward(q, np.repeat(np.asarray(k), G, axis=-3), np.repeat(np.asarray(v), G, axis=-3),
                             scale, window, **kw)


def attention_backward_gqa(q, k, v, do, scale, window=-1, **kw):
    """Gradients of grouped-query attention: dQ per query head; dK and dV of a
    key/value head are the sums over the query heads of its group (each
    repeated copy of K and V receives its own gradient)."""
    G = _group_size(q, k)
    dq, dk, dv = attention_backward(q, np.repeat(np.asarray(k), G, axis=-3), np.repeat(np.asarray(v), G, axis=-3),
                                    do, scale, window, **kw)
    shp = k.shape[:-3] + (k.shape[-3], G) + k.shape[-2:]
    return dq, dk.reshape(shp).sum(axis=-3), dv.reshape(shp).sum(axis=-3)
