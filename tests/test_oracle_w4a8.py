"""Pins of the W4A8 middle-tier oracle (oracle/w4a8.py) against exact rational
arithmetic, hand-worked rounding ties, pure-Python integer loops, a lossless
special case where W4A8 must equal W4A16, and the error ordering the tier
exists for."""

from fractions import Fraction

import numpy as np

import oracle
import synth


def _f32(fr):
    """Fraction -> nearest float32, ties to even (re-derived, not numpy's divide)."""
    c = np.float32(float(fr))
    cands = {c, np.nextafter(c, np.float32(-np.inf)), np.nextafter(c, np.float32(np.inf))}
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - fr),
                                     int(np.array(v, np.float32).view(np.uint32)) & 1))


def _codes8(vals, s):
    if s == 0:
        return [0] * len(vals)
    S = Fraction(float(s))
    return [max(-128, min(127, round(Fraction(float(_f32(Fraction(float(v)) / S))))))
            for v in vals]


def test_quant_act8_hand_ties():
    """Row 0: max 127, so s = 1 exactly and the codes are rne(x): 2.5 -> 2,
    3.5 -> 4, -0.5 -> 0, 126.5 -> 126, -126.5 -> -126, -127 -> -127.
    Row 1: max 254, s = 2: 5 -> 2 (2.5), 7 -> 4 (3.5), 253 -> 126 (126.5)."""
    r0 = [127.0, 2.5, 3.5, -0.5, 126.5, -126.5, -127.0, 1.25]
    r1 = [254.0, 5.0, 7.0, 253.0, -3.0, 0.0, 1.0, -254.0]
    x = np.zeros((2, 128), np.float32)
    x[0, :8], x[1, :8] = r0, r1
    X = synth.to_bf16_bits(x)
    assert np.array_equal(synth.from_bf16_bits(X), x)
    q, s = oracle.quant_act8(X)
    assert s.tolist() == [1.0, 2.0]
    assert q[0, :8].tolist() == [127, 2, 4, 0, 126, -126, -127, 1]
    assert q[1, :8].tolist() == [127, 2, 4, 126, -2, 0, 0, -127]
    assert not q[:, 8:].any()


def test_quant_act8_matches_exact_rational():
    rng = synth.make_rng(120)
    X = synth.activations(rng, 4, 384, n_outliers=2)
    q, s = oracle.quant_act8(X)
    xf = synth.from_bf16_bits(X)
    for m in range(4):
        a = max(abs(Fraction(float(v))) for v in xf[m])
        sm = _f32(a / 127)
        assert sm == s[m]
        assert q[m].tolist() == _codes8(xf[m], sm)


def test_quant_act8_range_zero_row_and_error_bound():
    rng = synth.make_rng(121)
    X = synth.activations(rng, 12, 2048, n_outliers=3)
    X[5] = 0
    q, s = oracle.quant_act8(X)
    assert s[5] == 0 and not q[5].any()
    nz = [m for m in range(12) if m != 5]
    assert np.all(np.abs(q[nz].astype(np.int32)).max(axis=1) == 127)
    assert q.min() >= -127
    x = synth.from_bf16_bits(X).astype(np.float64)
    err = np.abs(x - s.astype(np.float64)[:, None] * q)
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 1e-6))


def test_w4a8_partials_brute_force():
    rng = synth.make_rng(122)
    W = synth.weights(rng, 5, 256)
    X = synth.activations(rng, 3, 256, n_outliers=1)
    Wq, Ws = oracle.pack_w4(W)
    q, s = oracle.quant_act8(X)
    P = oracle.w4a8_partials(q, Wq)
    qa = q.astype(int).tolist()
    qw = oracle.unpack_nibbles(Wq).astype(int).tolist()
    for m in range(3):
        for n in range(5):
            for g in range(2):
                assert P[m, n, g] == sum(qa[m][k] * qw[n][k] for k in range(128 * g, 128 * g + 128))
    Y = oracle.gemm_w4a8(q, s, Wq, Ws)
    ws = Ws.view(np.float16).astype(np.float64)
    want = np.einsum("mng,ng->mn", P.astype(np.float64), ws) * s.astype(np.float64)[:, None]
    assert np.allclose(Y, want, rtol=1e-13, atol=0)


def test_lossless_activations_make_w4a8_equal_w4a16():
    """Rows c * 2^e with integer c in [-127, 127] and some |c| = 127: the
    8-bit codes are exactly c, and W4A8 equals W4A16."""
    rng = synth.make_rng(123)
    M, N, K = 4, 32, 512
    c = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
    c[:, 40] = 127
    c[1, 40] = -127
    e = np.array([0, -5, 3, -12], dtype=np.float32)
    xs = c * (np.float32(2.0) ** e)[:, None]
    X = synth.to_bf16_bits(xs)
    assert np.array_equal(synth.from_bf16_bits(X), xs)
    W = synth.weights(rng, N, K)
    Wq, Ws = oracle.pack_w4(W)
    q, s = oracle.quant_act8(X)
    assert np.array_equal(q, c.astype(np.int8))
    assert np.array_equal(s, np.float32(2.0) ** e)
    Y8 = oracle.gemm_w4a8(q, s, Wq, Ws)
    Y16 = oracle.gemm_w4a16(X, Wq, Ws)
    assert np.allclose(Y8, Y16, rtol=1e-12, atol=1e-12 * np.abs(Y16).max())


def test_w4a8_sits_between_the_two_modes():
    """On activations with x20 outlier channels the 8-bit codes keep the
    inliers: the layer's error against the exact product is a small fraction
    of W4A4's and close to W4A16's (whose error is the weights' alone)."""
    rng = synth.make_rng(124)
    M, N, K = 8, 256, 3584
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K, n_outliers=synth.outlier_count(K))
    y = synth.from_bf16_bits(X).astype(np.float64) @ W.astype(np.float64).T
    Wq, Ws = oracle.pack_w4(W)
    e4 = np.linalg.norm(oracle.gemm_w4a4(*oracle.quant_act(X), Wq, Ws) - y)
    e8 = np.linalg.norm(oracle.gemm_w4a8(*oracle.quant_act8(X), Wq, Ws) - y)
    e16 = np.linalg.norm(oracle.gemm_w4a16(X, Wq, Ws) - y)
    assert e8 < 0.3 * e4, (e8, e4)
    assert e8 < 1.2 * e16, (e8, e16)
