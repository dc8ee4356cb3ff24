"""Pins of the rotation oracle (oracle/rotate.py) against mathematics that
does not come from the oracle itself: scipy's Hadamard matrix, the
involution H H = 128 I, the invariance of the layer's product, the spreading
of a single spike, and the purpose of the rotation (smaller W4A4 error when
activations carry outlier channels)."""

import numpy as np
import scipy.linalg

import oracle
import synth


H = scipy.linalg.hadamard(128).astype(np.float64)   # Sylvester order


def test_fast_transform_equals_the_hadamard_matrix_on_small_integers():
    rng = np.random.default_rng(1)
    x = rng.integers(-8, 9, size=(5, 3 * 128)).astype(np.float32)
    got = oracle.fwht128_f32(x).astype(np.float64)
    want = np.concatenate([x[:, g * 128:(g + 1) * 128].astype(np.float64) @ H.T
                           for g in range(3)], axis=1)
    assert np.array_equal(got, want)          # every partial sum is exact in fp32


def test_fast_transform_within_fp32_rounding_in_general():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((7, 256)) * np.exp(rng.uniform(-4, 4, (7, 256)))).astype(np.float32)
    got = oracle.fwht128_f32(x).astype(np.float64)
    for g in range(2):
        blk = x[:, g * 128:(g + 1) * 128].astype(np.float64)
        want = blk @ H.T
        # seven stages, each one rounding of a partial sum bounded by sum|x|
        bound = 7 * 2.0 ** -24 * np.abs(blk).sum(axis=1, keepdims=True)
        assert np.all(np.abs(got[:, g * 128:(g + 1) * 128] - want) <= bound)


def test_applying_it_twice_gives_128_x():
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, size=(4, 128)).astype(np.float32)
    assert np.array_equal(oracle.fwht128_f32(oracle.fwht128_f32(x)), 128 * x)


def test_rotation_keeps_the_layer_product():
    rng = synth.make_rng(60)
    W = synth.weights(rng, 24, 384)
    X = synth.activations(rng, 5, 384, n_outliers=2)
    x = oracle.bf16_bits_to_f32(X).astype(np.float64)
    y = x @ W.astype(np.float64).T
    yr = oracle.rotate_x(X).astype(np.float64) @ oracle.rotate_w(W).astype(np.float64).T
    assert np.max(np.abs(yr - y)) <= 1e-5 * np.max(np.abs(y))


def test_a_spike_spreads_evenly_over_its_group():
    X = np.zeros((1, 256), np.float32)
    X[0, 128 + 37] = 3000.0
    xr = oracle.rotate_x(oracle.f32_to_bf16_bits(X))
    b = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(X))[0, 128 + 37]
    assert np.all(xr[0, :128] == 0)
    assert np.all(np.abs(xr[0, 128:]) == b / 16)
    # signs follow row 37 of H
    assert np.array_equal(np.sign(xr[0, 128:]), H[:, 37])


def test_verifier_input_is_the_bf16_rounding_of_the_rotation():
    rng = synth.make_rng(61)
    X = synth.activations(rng, 3, 256, n_outliers=1)
    assert np.array_equal(oracle.rotate_x_bf16(X), oracle.f32_to_bf16_bits(oracle.rotate_x(X)))


def test_rotation_cuts_the_w4a4_error_on_outlier_channels():
    """The purpose of the transform: per-token INT4 codes lose most inlier
    channels when a few channels are x20; rotated, the outliers are spread
    over their groups and the W4A4 layer is much closer to the exact product."""
    rng = synth.make_rng(62)
    M, N, K = 8, 256, 1024
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K, n_outliers=4)
    y = oracle.bf16_bits_to_f32(X).astype(np.float64) @ W.astype(np.float64).T
    Wq, Ws = oracle.pack_w4(W)
    y4 = oracle.gemm_w4a4(*oracle.quant_act(X), Wq, Ws)
    Wrq, Wrs = oracle.pack_w4(oracle.rotate_w(W))
    y4r = oracle.gemm_w4a4(*oracle.quant_act_rot(X), Wrq, Wrs)
    e = np.linalg.norm(y4 - y) / np.linalg.norm(y)
    er = np.linalg.norm(y4r - y) / np.linalg.norm(y)
    assert er < 0.5 * e, (e, er)
