"""GPU parity of the W4A8 middle tier (qspec_quant_act8, qspec_gemm_w4a8;
SKINNY and STREAM families) against the oracle (oracle/w4a8.py), through the C ABI: the 8-bit codes and
scales bit-exact in every row-length band of the quantizer's launch, Y
within 2e-3 * max|y| on ragged shapes with and without a k-split, rows
bitwise independent of M, and the lossless case where W4A8 meets W4A16."""

import numpy as np
import pytest

import oracle
import synth
import quantization_self_speculation_amd as q
from quantization_self_speculation_amd.binding import QSpecError
from gpu_util import assert_close, dev, dev_bf16, dev_f16, host, say

pytestmark = pytest.mark.gpu


def dev_w(Wq):
    return dev(oracle.tile_w4(Wq))


def dev_s(Ws):
    return dev_f16(oracle.tile_scales(Ws))


def _case(seed, M, N, K):
    rng = synth.make_rng(seed)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K, n_outliers=synth.outlier_count(K))
    return W, X


# one shape per launch band of the quantizer (16-byte chunks per row:
# <= 512, <= 2048, <= 4096, <= 8192, beyond), and the largest K accepted
@pytest.mark.parametrize("M,K", [(3, 128), (8, 3584), (5, 8192), (4, 18944), (2, 65536),
                                 (2, 131072), (1, 1 << 20)])
def test_quant_act8_bitexact(M, K):
    say(f"quant_act8 M={M} K={K}")
    X = synth.activations(synth.make_rng(130), M, K, n_outliers=4)
    if M >= 3:
        X[1] = 0                                   # a zero row: s = 0, codes 0
        t = np.zeros(K, np.float32)                # rounding ties at s = 1
        t[:8] = [127.0, 2.5, 3.5, -0.5, 126.5, -126.5, -127.0, 1.25]
        X[2] = synth.to_bf16_bits(t)
    q_ref, s_ref = oracle.quant_act8(X)
    Xq, Xs = q.quant_act8(dev_bf16(X))
    assert np.array_equal(host(Xs).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(Xq), q_ref)


SHAPES = [
    (1, 64, 128),
    (5, 1000, 2048),     # k-split, ragged N
    (8, 4608, 3584),     # Qwen2.5-7B QKV at the draft batch
    (16, 3584, 18944),   # Qwen2.5-7B down, k-split
    (40, 1030, 2048),    # three activation blocks, k-split, ragged N
    (80, 9000, 1024),    # more than one 64-row activation chunk
    (300, 512, 1024),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("variant", [q.GEMM_AUTO, q.GEMM_SKINNY, q.GEMM_STREAM])
def test_gemm_w4a8_parity(M, N, K, variant):
    if variant == q.GEMM_STREAM and M > 16:
        pytest.skip("the STREAM family takes M <= 16")
    say(f"gemm_w4a8 M={M} N={N} K={K} variant={variant}")
    W, X = _case(132, M, N, K)
    Wq, Ws = oracle.pack_w4(W)
    qa, s = oracle.quant_act8(X)
    args = (dev(qa), dev(s), dev_w(Wq), dev_s(Ws))
    Y = host(q.gemm_w4a8(*args, variant=variant, N=N))
    assert_close(Y, oracle.gemm_w4a8(qa, s, Wq, Ws), what="w4a8")
    # the same family with its int32 group partials stored: P exact, Y bitwise
    # the same as without them
    Yp, P = q.gemm_w4a8(*args, variant=variant, partials=True, N=N)
    assert np.array_equal(host(P), oracle.w4a8_partials(qa, Wq))
    assert np.array_equal(host(Yp).view(np.uint32), Y.view(np.uint32))


def test_gemm_w4a8_row_invariance():
    """Within a family rows are bitwise independent of M: SKINNY at M = 80 and
    its subsets, STREAM at M = 16 and its subsets."""
    N, K = 3584, 18944
    W, X = _case(133, 80, N, K)
    Wq, Ws = oracle.pack_w4(W)
    qa, s = oracle.quant_act8(X)
    args = (dev_w(Wq), dev_s(Ws))
    SK, ST = q.GEMM_SKINNY, q.GEMM_STREAM
    Y80 = host(q.gemm_w4a8(dev(qa), dev(s), *args, variant=SK, N=N))
    for lo, hi in ((0, 16), (16, 24), (41, 42), (79, 80)):
        Y = host(q.gemm_w4a8(dev(qa[lo:hi].copy()), dev(s[lo:hi].copy()), *args, variant=SK, N=N))
        assert np.array_equal(Y80[lo:hi].view(np.uint32), Y.view(np.uint32)), (lo, hi)
    Y16 = host(q.gemm_w4a8(dev(qa[:16].copy()), dev(s[:16].copy()), *args, variant=ST, N=N))
    for lo, hi in ((0, 5), (9, 10), (15, 16)):
        Y = host(q.gemm_w4a8(dev(qa[lo:hi].copy()), dev(s[lo:hi].copy()), *args, variant=ST, N=N))
        assert np.array_equal(Y16[lo:hi].view(np.uint32), Y.view(np.uint32)), (lo, hi)
    assert_close(Y16, oracle.gemm_w4a8(qa[:16], s[:16], Wq, Ws), what="w4a8 stream")


def test_gemm_w4a8_lossless_meets_w4a16():
    """Activations c * 2^e with integer |c| <= 127 and max |c| = 127: the
    codes are exact, so the GPU's W4A8 and W4A16 layers agree to rounding."""
    rng = synth.make_rng(134)
    M, N, K = 8, 1024, 2048
    c = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
    c[:, 9] = 127
    xs = c * (np.float32(2.0) ** rng.integers(-8, 8, size=M).astype(np.float32))[:, None]
    X = synth.to_bf16_bits(xs)
    W = synth.weights(rng, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = q.quant_act8(dev_bf16(X))
    assert np.array_equal(host(Xq), c.astype(np.int8))
    Y8 = host(q.gemm_w4a8(Xq, Xs, dev_w(Wq), dev_s(Ws), N=N))
    Y16 = host(q.gemm_w4a16(dev_bf16(X), dev_w(Wq), dev_s(Ws), N=N))
    assert_close(Y8, Y16, what="w4a8 vs w4a16 (lossless activations)")
    assert_close(Y8, oracle.gemm_w4a16(X, Wq, Ws), what="w4a8 vs the W4A16 oracle")


def test_gemm_w4a8_rejects_other_families():
    W, X = _case(135, 8, 64, 256)
    Wq, Ws = oracle.pack_w4(W)
    qa, s = oracle.quant_act8(X)
    for v in (q.GEMM_GEMV, q.GEMM_TILED):
        with pytest.raises(QSpecError):
            q.gemm_w4a8(dev(qa), dev(s), dev_w(Wq), dev_s(Ws), variant=v, N=64)
