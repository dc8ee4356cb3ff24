"""GPU parity of the per-group Walsh-Hadamard rotation and the rotated
quantizer against the CPU oracle (oracle/rotate.py), through the C ABI.

Bars: fp32 and bf16 outputs of the rotation bit-exact (the transform's
operations and their order are fixed); codes and scales of the rotated
quantizer bit-exact; layers on rotated operands within 2e-3 * max|y|.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import quantization_self_speculation_amd as q
from gpu_util import assert_close, dev, dev_bf16, dev_f16, host, host_bits16, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(1, 128), (17, 384), (300, 1024), (5, 18944)])
def test_rotate_w_bitexact(N, K):
    say(f"rotate_w N={N} K={K}")
    rng = synth.make_rng(70)
    W = synth.weights(rng, N, K)
    W[0, :7] = [0.0, -0.0, 1e-40, -1e35, 1e35, 1.5, -2.5]   # zeros, a subnormal, large values
    want = oracle.rotate_w(W)
    got = host(q.rotate_w(dev(W)))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    Wd = dev(W)
    q.rotate_w(Wd, Wr=Wd)                       # in place
    assert np.array_equal(host(Wd).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("M,K", [(1, 128), (8, 3584), (33, 18944)])
def test_rotate_x_bitexact(M, K):
    say(f"rotate_x M={M} K={K}")
    rng = synth.make_rng(71)
    X = synth.activations(rng, M, K, n_outliers=synth.outlier_count(K))
    want = oracle.rotate_x_bf16(X)
    Xd = dev_bf16(X)
    assert np.array_equal(host_bits16(q.rotate_x(Xd)), want)
    q.rotate_x(Xd, Xr=Xd)                       # in place
    assert np.array_equal(host_bits16(Xd), want)


# every row-length band of the rotated quantizer's launch
@pytest.mark.parametrize("K", [128, 3584, 4096, 4224, 16384, 16512, 32768, 32896, 65664])
def test_quant_act_rot_bitexact(K):
    M = 3
    say(f"quant_act_rot K={K}")
    rng = synth.make_rng(72)
    X = synth.activations(rng, M, K, n_outliers=synth.outlier_count(K))
    X[2] = 0                                      # scale 0: codes 0
    Xq_ref, Xs_ref = oracle.quant_act_rot(X)
    Xq, Xs = q.quant_act_rot(dev_bf16(X))
    assert np.array_equal(host(Xs).view(np.uint32), Xs_ref.view(np.uint32))
    assert np.array_equal(host(Xq), Xq_ref)


@pytest.mark.parametrize("M,N,K", [(8, 1024, 1024), (8, 4608, 3584), (40, 300, 1152)])
def test_rotated_layers(M, N, K):
    """Both modes on the rotated shared buffer: the drafter on the rotated
    codes, the verifier on the rotated bf16 input, each against the oracle;
    and the drafter's error against the exact product drops with the
    rotation (x20 outlier channels)."""
    say(f"rotated layers M={M} N={N} K={K}")
    rng = synth.make_rng(73)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K, n_outliers=max(4, synth.outlier_count(K)))
    Wr = oracle.rotate_w(W)
    Wq_r, Ws_r = oracle.pack_w4(Wr)
    Wq_d, Ws_d = q.pack_w4(q.rotate_w(dev(W)))
    assert np.array_equal(host(Wq_d), oracle.tile_w4(Wq_r))
    assert np.array_equal(host_bits16(Ws_d), oracle.tile_scales(Ws_r))
    Xd = dev_bf16(X)
    Xq_d, Xs_d = q.quant_act_rot(Xd)
    Y4 = host(q.gemm_w4a4(Xq_d, Xs_d, Wq_d, Ws_d, N=N))
    want4 = oracle.gemm_w4a4(*oracle.quant_act_rot(X), Wq_r, Ws_r)
    assert_close(Y4, want4, what="rotated w4a4")
    Y16 = host(q.gemm_w4a16(q.rotate_x(Xd), Wq_d, Ws_d, N=N))
    assert_close(Y16, oracle.gemm_w4a16(oracle.rotate_x_bf16(X), Wq_r, Ws_r), what="rotated w4a16")
    # the purpose: the drafter's layer is closer to the exact product
    y = oracle.bf16_bits_to_f32(X).astype(np.float64) @ W.astype(np.float64).T
    Wq_p, Ws_p = q.pack_w4(dev(W))
    Y4p = host(q.gemm_w4a4(*q.quant_act(Xd), Wq_p, Ws_p, N=N))
    e_plain = np.linalg.norm(Y4p - y) / np.linalg.norm(y)
    e_rot = np.linalg.norm(Y4 - y) / np.linalg.norm(y)
    say(f"  w4a4 error vs exact: plain {e_plain:.3f}, rotated {e_rot:.3f}")
    assert e_rot < 0.6 * e_plain
