"""Pins of the FP8 oracle (CPU only): the E4M3 rounding against the format's
own value table (decoded from its bit layout), the fast Walsh-Hadamard
transform against SciPy's Hadamard matrix, the scores' invariance under the
rotation, the quantiser's scale and error bound, and the attention on
exactly representable inputs against the dense oracle."""

import math

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(8)


def e4m3_table():
    """All finite E4M3 values from the bit layout: sign, 4-bit exponent
    (bias 7), 3-bit mantissa; exponent 0 is subnormal; 0x7f/0xff are NaN."""
    vals = []
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            continue
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals.append(-v if s else v)
    return np.unique(np.array(vals))


def test_table_is_the_e4m3_format():
    t = e4m3_table()
    assert t.max() == 448.0 and t.min() == -448.0
    assert len(t) == 253  # 254 finite codes, +0 and -0 coincide
    assert np.min(t[t > 0]) == 2.0 ** -9


def test_representable_values_round_to_themselves():
    t = e4m3_table().astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_round(t), t)


def test_midpoints_round_to_even_and_others_to_nearest():
    t = e4m3_table()
    pos = t[t >= 0]
    codes = {v: i for i, v in enumerate(pos)}
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = (lo + hi) / 2
        got = float(oracle.e4m3_round(np.float32(mid)))
        # the even neighbour has an even mantissa (an even index in the
        # sorted non-negative list, since codes count up by one)
        even = lo if codes[lo] % 2 == 0 else hi
        assert got == even, (lo, hi, got)
        for f in (0.25, 0.75):
            x = np.float32(lo + f * (hi - lo))
            want = lo if f < 0.5 else hi
            assert float(oracle.e4m3_round(x)) == want
            assert float(oracle.e4m3_round(-x)) == -want


def test_saturation_and_sign():
    assert float(oracle.e4m3_round(np.float32(1e6))) == 448.0
    assert float(oracle.e4m3_round(np.float32(-500))) == -448.0
    x = RNG.standard_normal(1000).astype(np.float32) * 50
    np.testing.assert_array_equal(oracle.e4m3_round(-x), -oracle.e4m3_round(x))


def test_fwht_equals_hadamard_matrix():
    scipy_linalg = pytest.importorskip("scipy.linalg")
    for d in (2, 8, 64, 128, 256):
        H = scipy_linalg.hadamard(d)
        x = RNG.integers(-50, 50, size=(7, d)).astype(np.float32)  # exact in fp32
        np.testing.assert_array_equal(oracle.fwht_f32(x), (x.astype(np.float64) @ H).astype(np.float32))


def test_rotation_scales_scores_by_d():
    d = 64
    signs = RNG.choice([-1.0, 1.0], size=d)
    q, k = RNG.standard_normal((5, d)), RNG.standard_normal((6, d))
    qr = oracle.fwht_f32(q * signs).astype(np.float64)
    kr = oracle.fwht_f32(k * signs).astype(np.float64)
    np.testing.assert_allclose(qr @ kr.T, d * (q @ k.T), rtol=1e-5, atol=1e-4)


def test_quantize_head_scale_and_error_bound():
    x = RNG.standard_normal((40, 64)).astype(np.float32) * 3
    codes, s = oracle.quantize_head(x)
    assert float(np.max(np.abs(codes))) == 448.0
    assert s == pytest.approx(float(np.max(np.abs(x))) / 448.0, rel=1e-7)
    deq = codes.astype(np.float64) * float(s)
    # relative error <= 2**-4 in the normal range, absolute <= half a
    # subnormal step below it
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 0.5 * 2.0 ** -9 * float(s))
    assert np.all(err <= bound * (1 + 1e-6))
    zero_codes, one = oracle.quantize_head(np.zeros((3, 8), np.float32))
    assert np.all(zero_codes == 0) and one == 1.0


def test_attention_on_representable_inputs_equals_dense_oracle():
    # Inputs whose per-head quantisation is exact (small integers whose
    # absolute maximum is 448 / 2**k): the FP8 forward then equals the
    # dense attention of the same values.
    n, d = 24, 16
    q = RNG.integers(-7, 8, size=(1, 2, n, d)).astype(np.float32) / 4
    k = RNG.integers(-7, 8, size=(1, 2, n, d)).astype(np.float32) / 4
    v = RNG.integers(-7, 8, size=(1, 2, n, d)).astype(np.float32) / 8
    for t in (q, k, v):
        t[..., 0, 0] = 7 / (4 if t is not v else 8)  # amax = 7/4 (or 7/8) in every head
    O, lse = oracle.attention_forward_fp8(q, k, v, 0.3)
    Od, ld = oracle.attention_forward(q, k, v, 0.3)
    np.testing.assert_allclose(O, Od, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ld, rtol=1e-12, atol=1e-12)


def test_fp8_attention_error_is_bounded():
    # E4M3 keeps 3 mantissa bits: each input carries <= 2**-4 relative error,
    # so O stays within ~2**-4 of max|O| and the scores within a few 1e-2.
    n, d = 64, 64
    q, k, v = (RNG.standard_normal((1, 2, n, d)).astype(np.float32) for _ in range(3))
    s = 1 / math.sqrt(d)
    O8, l8 = oracle.attention_forward_fp8(q, k, v, s)
    Od, ld = oracle.attention_forward(q, k, v, s)
    assert np.max(np.abs(O8 - Od)) / np.max(np.abs(Od)) < 0.15
    assert np.max(np.abs(l8 - ld)) < 0.1


def score_error(q, k, signs):
    d = q.shape[-1]
    q8, sq = oracle.quantize_head(q, signs)
    k8, sk = oracle.quantize_head(k, signs)
    d_rot = d if signs is not None else 1
    S8 = (q8.astype(np.float64) @ k8.astype(np.float64).T) * float(sq) * float(sk) / d_rot
    S = q.astype(np.float64) @ k.astype(np.float64).T
    return np.sqrt(np.mean((S8 - S) ** 2))


def test_rotation_reduces_quantisation_error_with_outlier_columns():
    # A few outlier columns set the per-head scale, so plain quantisation
    # leaves the other columns with few levels; the rotation spreads the
    # outliers over all columns and the score error drops.
    n, d = 128, 128
    q = RNG.standard_normal((n, d)).astype(np.float32)
    k = RNG.standard_normal((n, d)).astype(np.float32)
    q[:, :3] *= 60.0
    k[:, :3] *= 60.0
    signs = RNG.choice([-1.0, 1.0], size=d)
    plain, rotated = score_error(q, k, None), score_error(q, k, signs)
    assert rotated < 0.5 * plain, (plain, rotated)
    # without outliers the rotation changes what is computed by rounding only
    qn, kn = RNG.standard_normal((n, d)).astype(np.float32), RNG.standard_normal((n, d)).astype(np.float32)
    assert score_error(qn, kn, signs) < 2 * score_error(qn, kn, None) + 1e-3


def test_rotation_leaves_exact_attention_unchanged():
    n, d = 32, 64
    signs = RNG.choice([-1.0, 1.0], size=d)
    q, k, v = (RNG.standard_normal((n, d)).astype(np.float32) for _ in range(3))
    s = 1 / math.sqrt(d)
    qr, kr = oracle.fwht_f32(q * signs), oracle.fwht_f32(k * signs)
    Or, lr = oracle.attention_forward(qr, kr, v, s / d)
    Od, ld = oracle.attention_forward(q, k, v, s)
    np.testing.assert_allclose(Or, Od, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(lr, ld, rtol=1e-5, atol=1e-5)


def test_rotated_attention_on_representable_inputs_equals_dense_oracle():
    # The rotated branch, pinned exactly: choose the rotated values first.
    # With M = diag(signs) H (M M^T = d I), Q = Y M^T / d gives Q M = Y, so
    # the fast Walsh-Hadamard transform of Q * signs returns Y exactly (every
    # partial sum is a small multiple of 1/64).  Y holds multiples of 1/4 with
    # absolute maximum 7/4, so each rotated head quantises exactly (codes =
    # 256 Y, scale 1/256).  The FP8 forward must then reproduce the dense
    # attention of the unrotated Q, K: the scores (Q M)(K M)^T are d Q K^T, and
    # only the division by d (not by sqrt(d), not by 1) undoes that.
    scipy_linalg = pytest.importorskip("scipy.linalg")
    n, d = 20, 16
    signs = RNG.choice([-1.0, 1.0], size=d)
    M = np.diag(signs) @ scipy_linalg.hadamard(d).astype(np.float64)
    ys = []
    for _ in range(2):
        y = RNG.integers(-7, 8, size=(1, 2, n, d)).astype(np.float64) / 4
        y[..., 0, 0] = 7 / 4  # amax 7/4 in every head
        ys.append(y)
    q, k = ((y @ M.T / d).astype(np.float32) for y in ys)
    for x, y in zip((q, k), ys):  # the construction is exact in fp32
        np.testing.assert_array_equal(oracle.fwht_f32(x * signs.astype(np.float32)), y.astype(np.float32))
    v = RNG.integers(-7, 8, size=(1, 2, n, d)).astype(np.float32) / 8
    v[..., 0, 0] = 7 / 8
    for s in (1 / math.sqrt(d), 0.7):
        O, lse = oracle.attention_forward_fp8(q, k, v, s, signs)
        Od, ld = oracle.attention_forward(q, k, v, s)
        np.testing.assert_allclose(O, Od, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, ld, rtol=1e-12, atol=1e-12)


def test_rotated_fp8_attention_error_is_bounded():
    # Random inputs through the rotated branch stay within the quantisation
    # error of the dense attention of the unrotated inputs.  A score scale off
    # by sqrt(d) (or not divided by d at all) moves the log-sum-exp by far
    # more than this bound.
    n, d = 64, 64
    signs = RNG.choice([-1.0, 1.0], size=d)
    q, k, v = (RNG.standard_normal((1, 2, n, d)).astype(np.float32) for _ in range(3))
    s = 1 / math.sqrt(d)
    O8, l8 = oracle.attention_forward_fp8(q, k, v, s, signs)
    Od, ld = oracle.attention_forward(q, k, v, s)
    assert np.max(np.abs(O8 - Od)) / np.max(np.abs(Od)) < 0.15
    assert np.max(np.abs(l8 - ld)) < 0.1
