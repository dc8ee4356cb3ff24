"""Pins of the oracle's weight packer, activation quantizer and GEMMs.

Each test checks the oracle against something other than itself: hand-worked
fixtures (tests/golden, with their derivations), exact rational arithmetic
(``fractions.Fraction``) that re-derives IEEE rounding from its definition,
pure-Python integer loops, and a special case where the two modes must agree.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


# ----------------------------------------------------------------------------
# exact-rational references (independent of numpy's float arithmetic)
# ----------------------------------------------------------------------------
def _round_to(fr, dtype):
    """Fraction -> nearest value of ``dtype`` (float32 / float16), ties to even."""
    c = dtype(float(fr))
    cands = {dtype(c), np.nextafter(c, dtype(-np.inf)), np.nextafter(c, dtype(np.inf))}
    ubits = np.uint32 if dtype is np.float32 else np.uint16

    def key(v):
        return (abs(Fraction(float(v)) - fr), int(np.array(v, dtype=dtype).view(ubits)) & 1)
    return min(cands, key=key)


def _rne_int(fr):
    """round half to even of an exact rational (Python's round on Fraction)."""
    return round(fr)


def _codes_exact(vals_f32, scale_f32):
    out = []
    s = Fraction(float(scale_f32))
    for v in vals_f32:
        if s == 0:
            out.append(0)
            continue
        qf = _round_to(Fraction(float(v)) / s, np.float32)      # IEEE fp32 divide
        out.append(max(-8, min(7, _rne_int(Fraction(float(qf))))))
    return out


# ----------------------------------------------------------------------------
# nibble format
# ----------------------------------------------------------------------------
def test_nibble_table_exhaustive():
    allb = np.arange(256, dtype=np.uint8).reshape(256, 1)
    codes = oracle.unpack_nibbles(allb)
    assert codes.shape == (256, 2)
    for b in range(256):
        lo, hi = b & 0xF, b >> 4
        assert codes[b, 0] == (lo - 16 if lo >= 8 else lo)
        assert codes[b, 1] == (hi - 16 if hi >= 8 else hi)
    assert np.array_equal(oracle.pack_nibbles(codes), allb)
    # all 16 codes appear in both positions
    assert sorted(set(codes[:, 0].tolist())) == list(range(-8, 8))
    assert sorted(set(codes[:, 1].tolist())) == list(range(-8, 8))


def test_nibble_hand_examples(golden):
    g = golden("w4_nibbles.json")
    for c in g["cases"]:
        got = oracle.pack_nibbles(np.array([c["codes"]], dtype=np.int8))
        assert int(got[0, 0]) == c["byte"], c
        assert oracle.unpack_nibbles(got)[0].tolist() == c["codes"]


def test_nibble_order_multi_byte():
    q = np.array([[1, 2, 3, 4, -5, -6]], dtype=np.int8)
    b = oracle.pack_nibbles(q)
    assert b.tolist() == [[0x21, 0x43, 0xAB]]


# ----------------------------------------------------------------------------
# weight packer
# ----------------------------------------------------------------------------
def test_pack_w4_hand(golden):
    g = golden("pack_w4_hand.json")
    K = 128 * len(g["groups"])
    W = np.zeros((1, K), dtype=np.float32)
    for j, grp in enumerate(g["groups"]):
        for k, v in grp["values"].items():
            W[0, 128 * j + int(k)] = np.float32(v)
    Wq, Ws = oracle.pack_w4(W)
    q = oracle.unpack_nibbles(Wq)[0]
    for j, grp in enumerate(g["groups"]):
        assert int(Ws[0, j]) == grp["scale_bits"], (j, int(Ws[0, j]))
        want = np.zeros(128, dtype=np.int8)
        for k, c in grp["codes"].items():
            want[int(k)] = c
        assert np.array_equal(q[128 * j:128 * (j + 1)], want), j


def test_pack_w4_matches_exact_rational():
    rng = synth.make_rng(90)
    W = synth.weights(rng, 3, 256)
    W[1, :128] *= np.float32(1e-3)
    W[2, 5] = np.float32(0.3)          # a large element in one group
    Wq, Ws = oracle.pack_w4(W)
    q = oracle.unpack_nibbles(Wq)
    for n in range(W.shape[0]):
        for j in range(2):
            grp = W[n, 128 * j:128 * (j + 1)]
            a = max(abs(Fraction(float(v))) for v in grp)
            s32 = _round_to(a / 7, np.float32)
            s16 = _round_to(Fraction(float(s32)), np.float16)
            assert int(np.array(s16, np.float16).view(np.uint16)) == int(Ws[n, j])
            assert q[n, 128 * j:128 * (j + 1)].tolist() == _codes_exact(grp, np.float32(s16))


def test_pack_w4_idempotent_and_bounded():
    rng = synth.make_rng(91)
    W = synth.weights(rng, 64, 1024)
    Wq, Ws = oracle.pack_w4(W)
    D = oracle.dequant_w4(Wq, Ws)                      # exact q*s
    D32 = D.astype(np.float32)
    assert np.array_equal(D32.astype(np.float64), D)   # q*s is exact in fp32
    Wq2, Ws2 = oracle.pack_w4(D32)
    assert np.array_equal(Wq, Wq2) and np.array_equal(Ws, Ws2)
    s = Ws.view(np.float16).astype(np.float64)
    s_full = np.repeat(s, 128, axis=1)
    err = np.abs(W.astype(np.float64) - D)
    assert np.all(err <= s_full * (0.5 + 1e-6))
    q = oracle.unpack_nibbles(Wq).reshape(64, 8, 128)
    # the largest element of every group maps to +-7; -8 is not produced
    assert np.all(np.abs(q).max(axis=2) == 7)
    assert q.min() >= -7


def test_pack_w4_underflowed_scale_clamps():
    # absmax/7 below half the smallest fp16 subnormal: the scale rounds to 0
    W = np.zeros((1, 128), dtype=np.float32)
    W[0, 0] = np.float32(2.0 ** -27)
    Wq, Ws = oracle.pack_w4(W)
    assert int(Ws[0, 0]) == 0 and not Wq.any()
    # absmax/7 = 1.4 * 2^-24 rounds to the smallest subnormal 2^-24; the
    # ratio 9.8 rounds to 10 and is clamped to 7 (and -9.8 to -8)
    W[0, 0] = np.float32(9.8 * 2.0 ** -24)
    W[0, 1] = np.float32(-9.8 * 2.0 ** -24)
    Wq, Ws = oracle.pack_w4(W)
    assert int(Ws[0, 0]) == 1
    q = oracle.unpack_nibbles(Wq)[0]
    assert q[0] == 7 and q[1] == -8


def test_pack_w4_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.pack_w4(np.zeros((2, 100), np.float32))
    W = np.zeros((1, 128), np.float32)
    W[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.pack_w4(W)
    W[0, 3] = np.float32(1e6)      # 1e6/7 overflows fp16
    with pytest.raises(ValueError):
        oracle.pack_w4(W)


# ----------------------------------------------------------------------------
# activation quantizer
# ----------------------------------------------------------------------------
def test_quant_act_hand(golden):
    g = golden("quant_act_hand.json")
    rows = g["rows"]
    X = np.zeros((len(rows), 128), dtype=np.uint16)
    for m, row in enumerate(rows):
        for k, v in row.get("values", {}).items():
            X[m, int(k)] = synth.to_bf16_bits(np.array([v], np.float32))[0]
        for k, b in row.get("bf16_bits", {}).items():
            X[m, int(k)] = b
    Xq, Xs = oracle.quant_act(X)
    q = oracle.unpack_nibbles(Xq)
    for m, row in enumerate(rows):
        assert int(Xs[m:m + 1].view(np.uint32)[0]) == row["scale_bits"], m
        want = np.zeros(128, np.int8)
        for k, c in row["codes"].items():
            want[int(k)] = c
        assert np.array_equal(q[m], want), m


def test_quant_act_matches_exact_rational():
    rng = synth.make_rng(92)
    X = synth.activations(rng, 4, 256, n_outliers=2)
    Xq, Xs = oracle.quant_act(X)
    q = oracle.unpack_nibbles(Xq)
    xf = synth.from_bf16_bits(X)
    for m in range(4):
        a = max(abs(Fraction(float(v))) for v in xf[m])
        s = _round_to(a / 7, np.float32)
        assert np.float32(s) == Xs[m]
        assert q[m].tolist() == _codes_exact(xf[m], np.float32(s))


def test_quant_act_divides_not_reciprocal():
    """Rows where x / s and x * (1/s) round to different codes: the oracle
    must give the correctly rounded quotient's code."""
    rng = np.random.default_rng(7)
    n = 400000
    a = synth.from_bf16_bits(synth.to_bf16_bits(
        np.abs(rng.standard_normal(n).astype(np.float32)) * 4 + np.float32(0.1)))
    x = synth.from_bf16_bits(synth.to_bf16_bits(rng.uniform(-1, 1, n).astype(np.float32) * a))
    s = a / np.float32(7)
    div = np.rint(x / s)
    rec = np.rint(x * (np.float32(1) / s))
    idx = np.nonzero(div != rec)[0][:24]
    assert idx.size >= 8
    X = np.zeros((idx.size, 128), np.uint16)
    X[:, 0] = synth.to_bf16_bits(a[idx])
    X[:, 1] = synth.to_bf16_bits(x[idx])
    Xq, Xs = oracle.quant_act(X)
    q = oracle.unpack_nibbles(Xq)
    for r, i in enumerate(idx):
        want = _codes_exact([x[i]], Xs[r])[0]
        assert q[r, 1] == want
        assert q[r, 1] != rec[i]


def test_quant_act_code_range_and_zero_row():
    rng = synth.make_rng(93)
    X = synth.activations(rng, 16, 3584, n_outliers=4)
    X[3] = 0
    Xq, Xs = oracle.quant_act(X)
    q = oracle.unpack_nibbles(Xq)
    assert Xs[3] == 0 and not q[3].any()
    nz = [m for m in range(16) if m != 3]
    assert np.all(np.abs(q[nz]).max(axis=1) == 7)
    assert q.min() >= -7


# ----------------------------------------------------------------------------
# W4A4 and W4A16
# ----------------------------------------------------------------------------
def _tiny_case(seed, M, N, K, outliers=1):
    rng = synth.make_rng(seed)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K, n_outliers=outliers)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    return X, Xq, Xs, Wq, Ws


def test_w4a4_partials_brute_force():
    X, Xq, Xs, Wq, Ws = _tiny_case(94, 3, 5, 256)
    P = oracle.w4a4_partials(Xq, Wq)
    qa = oracle.unpack_nibbles(Xq).tolist()
    qw = oracle.unpack_nibbles(Wq).tolist()
    for m in range(3):
        for n in range(5):
            for g in range(2):
                want = 0
                for k in range(128 * g, 128 * g + 128):
                    want += qa[m][k] * qw[n][k]
                assert P[m, n, g] == want


def test_w4a4_exact_rational():
    X, Xq, Xs, Wq, Ws = _tiny_case(95, 2, 4, 256)
    Y = oracle.gemm_w4a4(Xq, Xs, Wq, Ws)
    qa = oracle.unpack_nibbles(Xq).tolist()
    qw = oracle.unpack_nibbles(Wq).tolist()
    ws = Ws.view(np.float16)
    for m in range(2):
        for n in range(4):
            tot = Fraction(0)
            for g in range(2):
                p = sum(qa[m][k] * qw[n][k] for k in range(128 * g, 128 * g + 128))
                tot += Fraction(float(ws[n, g])) * p
            tot *= Fraction(float(Xs[m]))
            assert abs(Fraction(float(Y[m, n])) - tot) <= abs(tot) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


def test_w4a16_exact_rational():
    X, Xq, Xs, Wq, Ws = _tiny_case(96, 2, 4, 256)
    Y = oracle.gemm_w4a16(X, Wq, Ws)
    xf = synth.from_bf16_bits(X)
    qw = oracle.unpack_nibbles(Wq).tolist()
    ws = Ws.view(np.float16)
    for m in range(2):
        for n in range(4):
            tot = Fraction(0)
            for g in range(2):
                acc = sum(Fraction(float(xf[m, k])) * qw[n][k] for k in range(128 * g, 128 * g + 128))
                tot += Fraction(float(ws[n, g])) * acc
            assert abs(Fraction(float(Y[m, n])) - tot) <= abs(tot) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


def test_w4a16_equals_dense_dequant():
    X, Xq, Xs, Wq, Ws = _tiny_case(97, 8, 96, 1024, outliers=4)
    Y = oracle.gemm_w4a16(X, Wq, Ws)
    D = oracle.dequant_w4(Wq, Ws)
    ref = synth.from_bf16_bits(X).astype(np.float64) @ D.T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_lossless_activations_make_modes_agree():
    """If each row is c * 2^e with integer c in [-7, 7] and some |c| = 7,
    activation quantization is lossless and W4A4 equals W4A16."""
    rng = synth.make_rng(98)
    M, N, K = 4, 32, 512
    c = rng.integers(-7, 8, size=(M, K)).astype(np.float32)
    c[:, 17] = 7
    c[2, 17] = -7
    e = np.array([0, -3, 4, -10], dtype=np.float32)
    xs = c * (np.float32(2.0) ** e)[:, None]
    X = synth.to_bf16_bits(xs)
    assert np.array_equal(synth.from_bf16_bits(X), xs)
    W = synth.weights(rng, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    assert np.array_equal(oracle.unpack_nibbles(Xq), c.astype(np.int8))
    assert np.array_equal(Xs, (np.float32(2.0) ** e))
    Y4 = oracle.gemm_w4a4(Xq, Xs, Wq, Ws)
    Y16 = oracle.gemm_w4a16(X, Wq, Ws)
    assert np.allclose(Y4, Y16, rtol=1e-12, atol=1e-12 * np.abs(Y16).max())


def test_w4a4_is_lossy_with_outliers():
    """The drafter is the lossy mode: with x20 outlier channels the two modes
    differ by far more than rounding (a guard against testing W4A4 against
    W4A16 by mistake)."""
    X, Xq, Xs, Wq, Ws = _tiny_case(99, 8, 64, 1024, outliers=4)
    Y4 = oracle.gemm_w4a4(Xq, Xs, Wq, Ws)
    Y16 = oracle.gemm_w4a16(X, Wq, Ws)
    assert np.abs(Y4 - Y16).max() > 0.05 * np.abs(Y16).max()


# ----------------------------------------------------------------------------
# storage order of the shared buffer
# ----------------------------------------------------------------------------
def test_tile_is_a_permutation_with_zero_padding():
    rng = np.random.default_rng(3)
    for N, K in ((1, 128), (16, 256), (37, 384), (64, 1024)):
        Wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        T = oracle.tile_w4(Wq)
        Np = -(-N // 16) * 16
        assert T.shape == (Np, K // 2)
        assert np.array_equal(oracle.untile_w4(T, N), Wq)
        # multiset of bytes = the row-major bytes plus zero padding
        pad = np.zeros((Np - N) * (K // 2), np.uint8)
        assert np.array_equal(np.sort(T.ravel()), np.sort(np.concatenate([Wq.ravel(), pad])))


def test_tile_hand_positions():
    """Tile (b, g) starts at byte (b*G + g)*1024; slot l holds row 16b + l%16,
    row bytes 64g + 16(l//16) .. +16 (hand-derived from the definition)."""
    N, K = 32, 256                      # G = 2 groups, 2 row blocks
    Wq = np.zeros((N, K // 2), np.uint8)
    Wq[17, 64 + 16 * 2 + 5] = 0xAB     # row 17 = block 1, r 1; group 1, chunk 2, byte 5
    Wq[3, 0] = 0x11                     # row 3 = block 0, r 3; group 0, chunk 0, byte 0
    flat = oracle.tile_w4(Wq).ravel()
    G = 2
    pos1 = ((1 * G + 1) * 64 + (16 * 2 + 1)) * 16 + 5
    pos2 = ((0 * G + 0) * 64 + (16 * 0 + 3)) * 16 + 0
    assert flat[pos1] == 0xAB and flat[pos2] == 0x11
    assert np.count_nonzero(flat) == 2


def test_tile_scales_permutation_and_positions():
    rng = np.random.default_rng(4)
    for N, G in ((1, 1), (16, 3), (37, 5)):
        Ws = rng.integers(1, 60000, size=(N, G), dtype=np.uint16)
        T = oracle.tile_scales(Ws)
        Np = -(-N // 16) * 16
        assert T.shape == (Np, G)
        assert np.array_equal(oracle.untile_scales(T, N), Ws)
        assert np.count_nonzero(T) == N * G
    Ws = np.zeros((32, 2), np.uint16)
    Ws[19, 1] = 7                      # block 1, r 3, group 1
    flat = oracle.tile_scales(Ws).ravel()
    assert flat[(1 * 2 + 1) * 16 + 3] == 7
