"""fp64 CPU oracle for attention restricted to a sparse pattern.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library.

The pattern is the union of the three sparse components the llmis.ru chapter
3.1 "The cost of attention" describes in its section 3 (Longformer and
BigBird):

* a sliding window: row i sees key j when |i - j| <= window (symmetric and
  inclusive, the reading used for the plain window as well; window < 0
  adds nothing);
* global tokens: a global position attends to every key and every query
  attends to it, with no window restriction (Longformer's task tokens);
* a block layout: with block size b, row i sees key j when
  layout[i // b, j // b] is set (BigBird's local, global and random blocks
  are all entries of this layout).

Attention over the pattern is the softmax of the definition taken over the
visible keys only (masked scores are -inf, so their probabilities are exactly
zero).  Reading for a row that sees no key at all (possible only when the
pattern has no window): its output is 0, its log-sum-exp is -inf (the limit
of an empty sum) and it contributes nothing to any gradient.

Rows are processed in blocks of at most ``row_block`` rows; each block still
spans all n keys, so this is the plain two-pass softmax of the definition.
"""

from dataclasses import dataclass

import numpy as np

__all__ = ["Pattern", "attention_forward_pattern", "attention_backward_pattern"]


@dataclass
class Pattern:
    """Sparse attention pattern over a sequence of length ``n``."""

    n: int
    window: int = -1
    global_idx: tuple = ()
    layout_block: int = 0
    layout: np.ndarray = None  # (ceil(n / b), ceil(n / b)) bool

    def __post_init__(self):
        self.is_global = np.zeros(self.n, dtype=bool)
        if len(self.global_idx):
            self.is_global[np.asarray(self.global_idx, dtype=np.int64)] = True
        if self.layout_block:
            nb = -(-self.n // self.layout_block)
            self.layout = np.asarray(self.layout, dtype=bool)
            if self.layout.shape != (nb, nb):
                raise ValueError(f"layout must be {nb} x {nb} blocks")

    def visible(self, rows):
        """Boolean (len(rows), n): which keys each of ``rows`` sees."""
        rows = np.asarray(rows, dtype=np.int64)
        cols = np.arange(self.n)
        vis = np.zeros((len(rows), self.n), dtype=bool)
        if self.window >= 0:
            vis |= np.abs(rows[:, None] - cols[None, :]) <= self.window
        vis |= self.is_global[rows][:, None]
        vis |= self.is_global[None, :]
        if self.layout_block:
            b = self.layout_block
            vis |= self.layout[rows // b][:, cols // b]
        return vis


def _as_f64(*arrays):
    return tuple(np.asarray(a, dtype=np.float64) for a in arrays)


def _probs(Qb, K, scale, vis):
    """Masked softmax rows; returns (P, lse) with empty rows P = 0, lse = -inf."""
    S = np.where(vis, scale * (Qb @ K.T), -np.inf)
    m = S.max(axis=1, keepdims=True)
    empty = ~vis.any(axis=1, keepdims=True)
    m = np.where(empty, 0.0, m)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = np.where(empty, 0.0, E / np.where(empty, 1.0, l))
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))[:, 0]
    return P, lse


def attention_forward_pattern(q, k, v, scale, pattern, row_block=1024):
    """O = softmax over the visible keys of scale * Q K^T, times V; and LSE.

    ``q``, ``k``, ``v``: (..., n, d), any float dtype (upcast to fp64).
    """
    q, k, v = _as_f64(q, k, v)
    n = q.shape[-2]
    O = np.empty(q.shape, dtype=np.float64)
    LSE = np.empty(q.shape[:-1], dtype=np.float64)
    for idx in np.ndindex(*q.shape[:-2]):
        for r0 in range(0, n, row_block):
            r1 = min(n, r0 + row_block)
            P, lse = _probs(q[idx][r0:r1], k[idx], scale, pattern.visible(np.arange(r0, r1)))
            O[idx][r0:r1] = P @ v[idx]
            LSE[idx][r0:r1] = lse
    return O, LSE


def attention_backward_pattern(q, k, v, do, scale, pattern, row_block=1024):
    """Gradients (dQ, dK, dV) of sum(O * dO), by the same chain rule as the
    dense oracle: dV = P^T dO, dP = dO V^T, D = rowsum(dO * O),
    dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q (masked P = 0)."""
    q, k, v, do = _as_f64(q, k, v, do)
    n = q.shape[-2]
    dQ = np.zeros(q.shape, dtype=np.float64)
    dK = np.zeros(k.shape, dtype=np.float64)
    dV = np.zeros(v.shape, dtype=np.float64)
    for idx in np.ndindex(*q.shape[:-2]):
        Q, K, V, dO = q[idx], k[idx], v[idx], do[idx]
        for r0 in range(0, n, row_block):
            r1 = min(n, r0 + row_block)
            P, _ = _probs(Q[r0:r1], K, scale, pattern.visible(np.arange(r0, r1)))
            Ob = P @ V
            dOb = dO[r0:r1]
            D = np.sum(dOb * Ob, axis=1, keepdims=True)
            dS = P * (dOb @ V.T - D)
            dQ[idx][r0:r1] = scale * (dS @ K)
            dK[idx] += scale * (dS.T @ Q[r0:r1])
            dV[idx] += P.T @ dOb
    return dQ, dK, dV
