"""CPU oracle for the FP8 attention forward (FlashAttention-3's FP8 support
and its "incoherent processing", the unite.ai page "Flash Attention:
Revolucionando a Eficiencia dos Modelos Transformer", section
"FlashAttention-3", items 2 and 3; llmis.ru chapter 3.1, section 6).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library.

Readings (the pages name the techniques without formulas):

* Format: OCP FP8 E4M3 (4 exponent bits, bias 7, 3 mantissa bits, largest
  finite value 448, subnormal step 2**-9), round to nearest even, values
  beyond +-448 saturate.
* Incoherent processing: Q and K are multiplied by the same random
  orthogonal-up-to-scale matrix M = diag(signs) H before quantisation, H the
  Sylvester Hadamard matrix of order d (entries +-1, H H^T = d I).  Then
  (Q M)(K M)^T = d Q K^T, so the scores are unchanged once divided by d; the
  rotation spreads outlier columns over all d columns, which shrinks the
  per-head absolute maximum that sets the quantisation step.  V is not
  rotated.
* Scaling: one scale per (batch, head) and tensor: s = amax / 448 of the
  (rotated) head, s = 1 for an all-zero head; the code of x is
  e4m3(clamp(x * (448 / amax), -448, 448)).  The quantisation decisions are
  taken in fp32, as on the GPU: the rotation is a fast Walsh-Hadamard
  transform in fp32 with stages h = 1, 2, 4, ... (only additions and
  subtractions, so every step is exactly rounded the same way on both
  sides), 448 / amax and the product are fp32 operations.
* Attention: S = scale / d_rot * (s_q s_k) * Q8 K8^T with d_rot = d when
  rotated, else 1; softmax over the keys; O = s_v * P V8.  The oracle
  evaluates it in fp64 on the dequantised codes.  The GPU additionally
  rounds P to E4M3 before the P V product (values <= 2**8 by its lazy
  rescaling); that rounding is what the FP8 tolerance covers.
"""

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_round", "fwht_f32", "quantize_head", "attention_forward_fp8"]

E4M3_MAX = 448.0


def e4m3_round(x):
    """Round float32 values to the nearest E4M3 value (ties to even),
    saturating at +-448.  Returns float32 values (exactly representable)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # step: 2**(e - 3) in the normal range (a >= 2**-6), 2**-9 below
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)
    r = np.round(a / step) * step  # numpy rounds half to even
    return (np.sign(x) * np.minimum(r, E4M3_MAX)).astype(np.float32)


def fwht_f32(x):
    """Unnormalised fast Walsh-Hadamard transform along the last axis, in
    float32, stages h = 1, 2, 4, ...: x M for the Sylvester matrix H."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def quantize_head(x, signs=None):
    """Quantise one (n, d) head: returns (codes as float32 E4M3 values, scale)
    with x ~= codes * scale (after the rotation when `signs` is given)."""
    x = np.asarray(x, dtype=np.float32)
    if signs is not None:
        x = fwht_f32(x * np.asarray(signs, dtype=np.float32))
    amax = np.float32(np.max(np.abs(x)))
    if amax == 0:
        return np.zeros_like(x), np.float32(1.0)
    inv = np.float32(E4M3_MAX) / amax
    codes = e4m3_round(np.clip(x * inv, -E4M3_MAX, E4M3_MAX))
    return codes, np.float32(amax / np.float32(E4M3_MAX))


def attention_forward_fp8(q, k, v, scale, signs=None):
    """FP8 attention forward of [B, H, n, d] inputs: per-head quantisation of
    Q, K (rotated when `signs` is given) and V, then the exact softmax
    attention of the dequantised values in fp64.  Returns (O, LSE)."""
    from .attention import attention_forward
    q, k, v = (np.asarray(t, dtype=np.float32) for t in (q, k, v))
    d = q.shape[-1]
    d_rot = d if signs is not None else 1
    O = np.empty(q.shape, dtype=np.float64)
    LSE = np.empty(q.shape[:-1], dtype=np.float64)
    for idx in np.ndindex(*q.shape[:-2]):
        q8, sq = quantize_head(q[idx], signs)
        k8, sk = quantize_head(k[idx], signs)
        v8, sv = quantize_head(v[idx])
        eff = float(scale) / d_rot * float(sq) * float(sk)
        o, lse = attention_forward(q8, k8, v8.astype(np.float64) * float(sv), eff)
        O[idx], LSE[idx] = o, lse
    return O, LSE
