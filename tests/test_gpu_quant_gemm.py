"""GPU parity of the packer, the activation quantizer and both GEMMs against
the CPU oracle, through the C ABI (python binding -> libqspec.so).

Bars: bit-exact for packed bytes, scales and int32 group partials; for fp
outputs max|err| <= 2e-3 * max|y| against the oracle's fp64 result.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import quantization_self_speculation_amd as q
from gpu_util import (assert_close, dev, dev_bf16, dev_f16, host, host_bits16, say)

pytestmark = pytest.mark.gpu

W4A16_VARIANTS = [q.GEMM_AUTO, q.GEMM_GEMV, q.GEMM_SKINNY, q.GEMM_TILED, q.GEMM_STREAM]
W4A4_VARIANTS = [q.GEMM_AUTO, q.GEMM_SKINNY, q.GEMM_TILED, q.GEMM_STREAM]
STREAM_MAX_M = 16   # the STREAM family takes M <= 16

# (M, N, K): the small single-layer case, ragged tails in M and N, odd group
# counts, several m-chunks and split-K shapes
SHAPES = [
    (8, 1024, 1024),
    (1, 100, 384),
    (5, 72, 256),
    (17, 200, 512),
    (40, 48, 1152),
    (70, 130, 640),
    (3, 4608, 3584),
    (300, 600, 1152),
    (16, 3584, 18944),
    (11, 200, 2688),
    (9, 40, 128),
    (1, 1, 128),
    (128, 96, 256),
    (129, 96, 256),
    (72, 8200, 256),    # W4A16 SKINNY without a k-split: one 80-row activation block
    (9, 8208, 256),     # STREAM on a wide grid (513 row blocks: the integer modes' 3-deep ring)
]


def _cases(variants):
    return [(M, N, K, v) for (M, N, K) in SHAPES for v in variants
            if v != q.GEMM_STREAM or M <= STREAM_MAX_M]


def dev_w(Wq):
    """oracle row-major packed bytes -> device buffer in the tiled storage order"""
    return dev(oracle.tile_w4(Wq))


def dev_s(Ws):
    """oracle row-major fp16 scale bits -> device buffer in the tiled order"""
    return dev_f16(oracle.tile_scales(Ws))


def _case(seed, M, N, K, outliers=None):
    rng = synth.make_rng(seed)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K, n_outliers=outliers if outliers is not None
                          else synth.outlier_count(K))
    return W, X


# ------------------------------------------------------------------ packer
@pytest.mark.parametrize("N,K", [(1024, 1024), (17, 384), (100, 256), (5, 18944), (1, 128)])
def test_pack_w4_bitexact(N, K):
    say(f"pack_w4 N={N} K={K}")
    W, _ = _case(10, 1, N, K)
    W[0, :128] *= np.float32(1e-6)       # a tiny-scale group
    W[min(1, N - 1), 128:256] = 0        # an all-zero group
    Wq_ref, Ws_ref = oracle.pack_w4(W)
    Wq, Ws = q.pack_w4(dev(W))
    assert np.array_equal(host(Wq), oracle.tile_w4(Wq_ref))
    assert np.array_equal(host_bits16(Ws), oracle.tile_scales(Ws_ref))


def test_pack_w4_hand_and_subnormal(golden):
    g = golden("pack_w4_hand.json")
    W = np.zeros((3, 384), dtype=np.float32)
    for j, grp in enumerate(g["groups"]):
        for k, v in grp["values"].items():
            W[0, 128 * j + int(k)] = np.float32(v)
    W[1, 0] = np.float32(9.8 * 2.0 ** -24)     # fp16-subnormal scale, clamped codes
    W[1, 1] = np.float32(-9.8 * 2.0 ** -24)
    W[2, 0] = np.float32(2.0 ** -27)           # scale underflows to 0
    Wq_ref, Ws_ref = oracle.pack_w4(W)
    Wq, Ws = q.pack_w4(dev(W))
    assert np.array_equal(host(Wq), oracle.tile_w4(Wq_ref))
    assert np.array_equal(host_bits16(Ws), oracle.tile_scales(Ws_ref))
    assert Ws_ref[0].tolist() == [grp["scale_bits"] for grp in g["groups"]]


# ------------------------------------------------------------------ quantizer
@pytest.mark.parametrize("M,K,outl", [(8, 1024, 4), (1, 18944, 19), (33, 3584, 4), (3, 128, 0)])
def test_quant_act_bitexact(M, K, outl):
    say(f"quant_act M={M} K={K}")
    _, X = _case(11, M, 8, K, outliers=outl)
    if M > 2:
        X[2] = 0
    Xq_ref, Xs_ref = oracle.quant_act(X)
    Xq, Xs = q.quant_act(dev_bf16(X))
    assert np.array_equal(host(Xq), Xq_ref)
    assert np.array_equal(host(Xs).view(np.uint32), Xs_ref.view(np.uint32))


# every row-length band of the quantizer's launch (16-byte chunks per row:
# <= 512, <= 2048, <= 4096, <= 8192, and the two-pass kernel beyond), at
# both sides of each boundary, up to the largest K the library accepts
@pytest.mark.parametrize("K", [4096, 4224, 16384, 16512, 32768, 32896, 65536, 65664, 1 << 20])
def test_quant_act_row_length_bands(K):
    M = 3
    say(f"quant_act band K={K}")
    rng = synth.make_rng(24)
    X = synth.activations(rng, M, K, n_outliers=synth.outlier_count(K))
    X[1, K - 1] = synth.to_bf16_bits(np.array([-512.0], np.float32))[0]  # absmax at the last element
    Xq_ref, Xs_ref = oracle.quant_act(X)
    Xq, Xs = q.quant_act(dev_bf16(X))
    assert np.array_equal(host(Xq), Xq_ref)
    assert np.array_equal(host(Xs).view(np.uint32), Xs_ref.view(np.uint32))


def test_quant_act_hand_ties_subnormal_and_division(golden):
    g = golden("quant_act_hand.json")
    rows = g["rows"]
    X = np.zeros((len(rows), 128), dtype=np.uint16)
    for m, row in enumerate(rows):
        for k, v in row.get("values", {}).items():
            X[m, int(k)] = synth.to_bf16_bits(np.array([v], np.float32))[0]
        for k, bb in row.get("bf16_bits", {}).items():
            X[m, int(k)] = bb
    # rows where x / s and x * (1 / s) round to different codes
    rng = np.random.default_rng(7)
    n = 400000
    a = synth.from_bf16_bits(synth.to_bf16_bits(
        np.abs(rng.standard_normal(n).astype(np.float32)) * 4 + np.float32(0.1)))
    x = synth.from_bf16_bits(synth.to_bf16_bits(rng.uniform(-1, 1, n).astype(np.float32) * a))
    s = a / np.float32(7)
    idx = np.nonzero(np.rint(x / s) != np.rint(x * (np.float32(1) / s)))[0][:32]
    D = np.zeros((idx.size, 128), np.uint16)
    D[:, 0] = synth.to_bf16_bits(a[idx])
    D[:, 1] = synth.to_bf16_bits(x[idx])
    X = np.concatenate([X, D])
    Xq_ref, Xs_ref = oracle.quant_act(X)
    Xq, Xs = q.quant_act(dev_bf16(X))
    assert np.array_equal(host(Xs).view(np.uint32), Xs_ref.view(np.uint32))
    assert np.array_equal(host(Xq), Xq_ref)


# ------------------------------------------------------------------ W4A4
@pytest.mark.parametrize("M,N,K,variant", _cases(W4A4_VARIANTS))
def test_w4a4_parity(M, N, K, variant):
    say(f"w4a4 M={M} N={N} K={K} variant={variant}")
    W, X = _case(12, M, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    Xq_d, Xs_d, Wq_d, Ws_d = dev(Xq), dev(Xs), dev_w(Wq), dev_s(Ws)
    # P comes from the family that computes Y (the same kernel code with its
    # integer group sums stored), so it checks that family's MFMA chain
    Y, P = q.gemm_w4a4(Xq_d, Xs_d, Wq_d, Ws_d, variant=variant, partials=True, N=N)
    assert np.array_equal(host(P), oracle.w4a4_partials(Xq, Wq))
    want = oracle.gemm_w4a4(Xq, Xs, Wq, Ws)
    assert_close(host(Y), want, what="w4a4")
    # without the partials output: bitwise the same Y
    Y2 = q.gemm_w4a4(Xq_d, Xs_d, Wq_d, Ws_d, variant=variant, N=N)
    assert np.array_equal(host(Y2).view(np.uint32), host(Y).view(np.uint32))


@pytest.mark.parametrize("K", [3584, 18944])
def test_w4a4_massive_outlier_rows(K):
    """Every row holds one channel about 1000x the others, so per-token
    quantization zeroes every other code and |y| is small: the fp32 scale
    epilogue's rounding must stay within the bar in every family."""
    M, N = 70, 200
    say(f"w4a4 massive-outlier rows K={K}")
    rng = synth.make_rng(22)
    W = synth.weights(rng, N, K)
    Xf = synth.from_bf16_bits(synth.activations(rng, M, K, n_outliers=0)).copy()
    Xf[np.arange(M), rng.integers(0, K, size=M)] = np.float32(3000.0)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(synth.to_bf16_bits(Xf))
    want = oracle.gemm_w4a4(Xq, Xs, Wq, Ws)
    Xq_d, Xs_d, Wq_d, Ws_d = dev(Xq), dev(Xs), dev_w(Wq), dev_s(Ws)
    for v in W4A4_VARIANTS:
        if v == q.GEMM_STREAM:
            Y = q.gemm_w4a4(dev(Xq[:16].copy()), dev(Xs[:16].copy()), Wq_d, Ws_d, variant=v, N=N)
            e = assert_close(host(Y), want[:16], what=f"w4a4 massive outliers variant={v}")
        else:
            Y = q.gemm_w4a4(Xq_d, Xs_d, Wq_d, Ws_d, variant=v, N=N)
            e = assert_close(host(Y), want, what=f"w4a4 massive outliers variant={v}")
        say(f"  variant={v} max|err| / max|y| = {e:.2e}")


def test_w4a4_gpu_quantized_chain():
    """quant_act on the GPU feeding the GEMM equals the oracle chain."""
    N = 1024
    W, X = _case(13, 8, N, 1024, outliers=4)
    Wq, Ws = oracle.pack_w4(W)
    X_d, Wq_d, Ws_d = dev_bf16(X), dev_w(Wq), dev_s(Ws)   # kept alive across the launches
    Xq_d, Xs_d = q.quant_act(X_d)
    Y = q.gemm_w4a4(Xq_d, Xs_d, Wq_d, Ws_d, N=N)
    Xq, Xs = oracle.quant_act(X)
    assert_close(host(Y), oracle.gemm_w4a4(Xq, Xs, Wq, Ws), what="w4a4 chain")


# ------------------------------------------------------------------ W4A16
@pytest.mark.parametrize("M,N,K,variant", _cases(W4A16_VARIANTS))
def test_w4a16_parity(M, N, K, variant):
    say(f"w4a16 M={M} N={N} K={K} variant={variant}")
    W, X = _case(14, M, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Y = q.gemm_w4a16(dev_bf16(X), dev_w(Wq), dev_s(Ws), variant=variant, N=N)
    assert_close(host(Y), oracle.gemm_w4a16(X, Wq, Ws), what="w4a16")


def test_w4a16_zero_and_lossless_rows():
    """All-zero rows give exact zeros; rows of small integers times a power of
    two make W4A4 and W4A16 agree (both against the oracle)."""
    M, N, K = 4, 96, 512
    rng = synth.make_rng(15)
    W = synth.weights(rng, N, K)
    c = rng.integers(-7, 8, size=(M, K)).astype(np.float32)
    c[:, 3] = 7
    c[1] = 0
    X = synth.to_bf16_bits(c * np.float32(0.25))
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    for v in W4A16_VARIANTS:
        Y16 = host(q.gemm_w4a16(dev_bf16(X), dev_w(Wq), dev_s(Ws), variant=v, N=N))
        assert np.all(Y16[1] == 0)
        assert_close(Y16, oracle.gemm_w4a16(X, Wq, Ws))
    Y4 = host(q.gemm_w4a4(dev(Xq), dev(Xs), dev_w(Wq), dev_s(Ws), N=N))
    assert np.all(Y4[1] == 0)
    assert_close(Y4, oracle.gemm_w4a16(X, Wq, Ws))


@pytest.mark.parametrize("M,N,K", [(5, 16448, 256), (7, 24576, 384), (2, 37888, 256),
                                   (33, 16448, 256), (40, 37888, 256)])
def test_skinny_workgroup_sizes(M, N, K):
    """Decode and verify shapes whose skinny workgroups are sized to spread
    evenly over the CUs (5, 8 and 10 wavefronts, ragged last tile; one and
    three 16-row activation blocks): both modes against the oracle."""
    say(f"skinny workgroup sizes M={M} N={N} K={K}")
    W, X = _case(23, M, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    Wq_d, Ws_d = dev_w(Wq), dev_s(Ws)
    V = q.GEMM_SKINNY
    assert_close(host(q.gemm_w4a16(dev_bf16(X), Wq_d, Ws_d, variant=V, N=N)),
                 oracle.gemm_w4a16(X, Wq, Ws), what="w4a16")
    assert_close(host(q.gemm_w4a4(dev(Xq), dev(Xs), Wq_d, Ws_d, variant=V, N=N)),
                 oracle.gemm_w4a4(Xq, Xs, Wq, Ws), what="w4a4")


# ------------------------------------------------------------------ invariance
def test_stream_row_invariance_both_modes():
    """STREAM family: rows bitwise identical at M = 16, 8, 5, 4 and 1 (a k-split
    of up to 16 wavefronts reduced in LDS in fixed order; W4A16 loads the
    activations of at most 4 / 8 rows with one / two loads per group and
    moves them to their MFMA lanes by DPP shifts)."""
    N, K = 1000, 18944
    W, X = _case(19, 16, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    Wq_d, Ws_d = dev_w(Wq), dev_s(Ws)
    V = q.GEMM_STREAM
    Y16 = host(q.gemm_w4a16(dev_bf16(X), Wq_d, Ws_d, variant=V, N=N))
    Z16 = host(q.gemm_w4a4(dev(Xq), dev(Xs), Wq_d, Ws_d, variant=V, N=N))
    for lo, hi in ((0, 5), (9, 10), (15, 16), (0, 4), (12, 16), (3, 11), (8, 16), (5, 8)):
        Y = host(q.gemm_w4a16(dev_bf16(X[lo:hi].copy()), Wq_d, Ws_d, variant=V, N=N))
        Z = host(q.gemm_w4a4(dev(Xq[lo:hi].copy()), dev(Xs[lo:hi].copy()), Wq_d, Ws_d,
                             variant=V, N=N))
        assert np.array_equal(Y16[lo:hi].view(np.uint32), Y.view(np.uint32)), (lo, hi)
        assert np.array_equal(Z16[lo:hi].view(np.uint32), Z.view(np.uint32)), (lo, hi)
    assert_close(Y16, oracle.gemm_w4a16(X, Wq, Ws))
    assert_close(Z16, oracle.gemm_w4a4(Xq, Xs, Wq, Ws))


@pytest.mark.parametrize("N,K", [(200, 18944), (1001, 2688)])
def test_w4a16_stream_few_rows(N, K):
    """W4A16 STREAM with at most 8 rows: one (M <= 4) or two (M <= 8)
    activation loads per lane and group, each MFMA fragment moved into its
    lane by a DPP row shift.  Every M from 1 to 8 against the oracle, and
    bitwise the rows of the 16-row call (four loads per lane); ragged N, on
    the three-group ring (K = 18944: 9 groups per wavefront) and the
    two-group one (K = 2688: 2 groups per wavefront)."""
    W, X = _case(41, 16, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Wq_d, Ws_d = dev_w(Wq), dev_s(Ws)
    V = q.GEMM_STREAM
    Y16 = host(q.gemm_w4a16(dev_bf16(X), Wq_d, Ws_d, variant=V, N=N))
    for M in range(1, 9):
        say(f"stream few rows N={N} K={K} M={M}")
        lo = (3 * M) % (17 - M)  # a window that is not always at row 0
        Y = host(q.gemm_w4a16(dev_bf16(X[lo:lo + M].copy()), Wq_d, Ws_d, variant=V, N=N))
        assert np.array_equal(Y.view(np.uint32), Y16[lo:lo + M].view(np.uint32)), (M, lo)
        assert_close(Y, oracle.gemm_w4a16(X[lo:lo + M], Wq, Ws), what=f"w4a16 stream M={M}")


@pytest.mark.parametrize("variant,N", [(q.GEMM_GEMV, 2048), (q.GEMM_SKINNY, 2048),
                                       (q.GEMM_SKINNY, 11264), (q.GEMM_TILED, 2048)])
def test_w4a16_row_invariance(variant, N):
    """Within one kernel family row r of Y is bitwise identical at any M
    (SKINNY at N = 11264 runs 80 rows as one 80-row block, 16 as one)."""
    K = 2048
    W, X = _case(16, 80, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Wq_d, Ws_d, X_d = dev_w(Wq), dev_s(Ws), dev_bf16(X)
    Y80 = host(q.gemm_w4a16(X_d, Wq_d, Ws_d, variant=variant, N=N))
    Y16 = host(q.gemm_w4a16(X_d[:16].contiguous(), Wq_d, Ws_d, variant=variant, N=N))
    assert np.array_equal(Y80[:16].view(np.uint32), Y16.view(np.uint32))
    for r in (0, 37, 79):
        Y1 = host(q.gemm_w4a16(X_d[r:r + 1].contiguous(), Wq_d, Ws_d, variant=variant, N=N))
        assert np.array_equal(Y80[r:r + 1].view(np.uint32), Y1.view(np.uint32)), r


@pytest.mark.parametrize("N,K", [(1024, 2048), (3584, 18944), (4608, 3584), (8192, 1024)])
def test_w4a4_row_invariance(N, K):
    """SKINNY family, W4A4: rows bitwise identical at M = 80 (four activation
    blocks per workgroup), 16, 8, 5 and 1 (one block, the workgroup size
    balanced over the CUs).  The k-split is a function of N and K only: 8, 3
    and 2 slices for the first three shapes, none for N = 8192."""
    W, X = _case(17, 80, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    args = (dev_w(Wq), dev_s(Ws))
    Y80 = host(q.gemm_w4a4(dev(Xq), dev(Xs), *args, variant=q.GEMM_SKINNY, N=N))
    for lo, hi in ((0, 16), (16, 24), (40, 45), (41, 42), (79, 80)):
        Y = host(q.gemm_w4a4(dev(Xq[lo:hi].copy()), dev(Xs[lo:hi].copy()), *args,
                             variant=q.GEMM_SKINNY, N=N))
        assert np.array_equal(Y80[lo:hi].view(np.uint32), Y.view(np.uint32)), (lo, hi)
    assert_close(Y80, oracle.gemm_w4a4(Xq, Xs, Wq, Ws), what="w4a4 M=80")


# ------------------------------------------------------------------ bf16 output
# every W4A4 family, vector and ragged N, with and without a k-split
BF16_CASES = [
    (8, 1001, 2048, q.GEMM_STREAM),     # ragged N
    (8, 4608, 3584, q.GEMM_AUTO),
    (5, 1028, 1024, q.GEMM_SKINNY),     # k-split over several workgroups
    (40, 9000, 1024, q.GEMM_SKINNY),    # three activation blocks, no k-split
    (40, 1030, 2048, q.GEMM_SKINNY),    # k-split, ragged N
    (300, 1030, 1024, q.GEMM_TILED),    # ragged N
    (300, 4096, 1024, q.GEMM_AUTO),
]


@pytest.mark.parametrize("M,N,K,variant", BF16_CASES)
def test_w4a4_bf16_output(M, N, K, variant):
    """qspec_gemm_w4a4_bf16: each output is the round-to-nearest-even bf16 of
    the fp32 value qspec_gemm_w4a4 stores (same variant), bit for bit, and so
    within the fp32 tolerance plus half a bf16 unit (2^-9 relative) of the
    oracle."""
    say(f"w4a4 bf16 output M={M} N={N} K={K} variant={variant}")
    W, X = _case(31, M, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    args = (dev(Xq), dev(Xs), dev_w(Wq), dev_s(Ws))
    y32 = host(q.gemm_w4a4(*args, variant=variant, N=N))
    bits = host_bits16(q.gemm_w4a4_bf16(*args, variant=variant, N=N))
    assert np.array_equal(bits, oracle.f32_to_bf16_bits(y32.astype(np.float32)))
    want = oracle.gemm_w4a4(Xq, Xs, Wq, Ws)
    err = np.abs(oracle.bf16_bits_to_f32(bits).astype(np.float64) - want)
    assert np.all(err <= 2e-3 * np.abs(want).max() + 2.0 ** -9 * np.abs(want) + 1e-30)


SK, TI = q.GEMM_SKINNY, q.GEMM_TILED


@pytest.mark.parametrize("M,N,K,fam16,fam4", [
    (300, 1000, 8192, SK, SK),    # long K, small tiled grid: SKINNY beyond the limit
    (200, 1000, 8192, SK, SK),
    (300, 1000, 1024, TI, TI),    # short K: TILED beyond the limit
    (96, 37888, 1024, TI, TI),    # wide N: TILED below the limit (>= 256 tiles)
    (64, 37888, 1024, TI, SK),    # W4A4 takes TILED only from 96 rows
    (40, 37888, 1024, SK, SK),    # the verify batch stays SKINNY
])
def test_auto_family_choice(M, N, K, fam16, fam4):
    """AUTO names one family per (M, N, K): its result is bitwise that
    family's, and within tolerance of the oracle, in both modes."""
    say(f"auto family M={M} N={N} K={K}")
    W, X = _case(33, M, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    a4 = (dev(Xq), dev(Xs), dev_w(Wq), dev_s(Ws))
    y4 = host(q.gemm_w4a4(*a4, N=N))
    assert np.array_equal(y4.view(np.uint32), host(q.gemm_w4a4(*a4, variant=fam4, N=N)).view(np.uint32))
    assert_close(y4, oracle.gemm_w4a4(Xq, Xs, Wq, Ws), what="w4a4 auto")
    a16 = (dev_bf16(X), dev_w(Wq), dev_s(Ws))
    y16 = host(q.gemm_w4a16(*a16, N=N))
    assert np.array_equal(y16.view(np.uint32), host(q.gemm_w4a16(*a16, variant=fam16, N=N)).view(np.uint32))
    assert_close(y16, oracle.gemm_w4a16(X, Wq, Ws), what="w4a16 auto")


def test_determinism():
    N = 4608
    W, X = _case(18, 40, N, 3584)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    a16 = (dev_bf16(X), dev_w(Wq), dev_s(Ws))
    a4 = (dev(Xq), dev(Xs), dev_w(Wq), dev_s(Ws))
    y1 = host(q.gemm_w4a16(*a16, N=N))
    y2 = host(q.gemm_w4a16(*a16, N=N))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    z1 = host(q.gemm_w4a4(*a4, N=N))
    z2 = host(q.gemm_w4a4(*a4, N=N))
    assert np.array_equal(z1.view(np.uint32), z2.view(np.uint32))


# ------------------------------------------------------------------ full-size shapes
QWEN7B = {"qkv": (4608, 3584), "o": (3584, 3584), "gate_up": (37888, 3584), "down": (3584, 18944)}
LLAMA8B_HEAD = (128256, 4096)


def _sampled_cols(N, rng, count=512):
    return np.sort(rng.choice(N, size=min(N, count), replace=False))


@pytest.mark.parametrize("proj", list(QWEN7B))
def test_qwen7b_decode_shapes(proj):
    """Decode/verify batch sizes of the Qwen2.5-7B projections: W4A4 at
    M = 1, 8, 32 and W4A16 at M = 5, 40 on the same packed buffer (checked on
    sampled output columns, which the oracle computes from those weight rows)."""
    N, K = QWEN7B[proj]
    rng = synth.make_rng(1)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, 40, K, n_outliers=synth.outlier_count(K))
    cols = _sampled_cols(N, rng)
    Wq, Ws = oracle.pack_w4(W[cols])          # oracle packs the sampled rows only
    Wq_d, Ws_d = q.pack_w4(dev(W))            # the device packs everything
    assert np.array_equal(oracle.untile_w4(host(Wq_d), N)[cols], Wq)
    assert np.array_equal(oracle.untile_scales(host_bits16(Ws_d), N)[cols], Ws)
    for M in (1, 8, 32):
        say(f"{proj} w4a4 M={M}")
        Xq_d, Xs_d = q.quant_act(dev_bf16(X[:M].copy()))
        Y = host(q.gemm_w4a4(Xq_d, Xs_d, Wq_d, Ws_d, N=N))
        Xq, Xs = oracle.quant_act(X[:M])
        assert np.array_equal(host(Xq_d), Xq)
        assert_close(Y[:, cols], oracle.gemm_w4a4(Xq, Xs, Wq, Ws), what=f"w4a4 M={M}")
    for M in (5, 40):
        say(f"{proj} w4a16 M={M}")
        Y = host(q.gemm_w4a16(dev_bf16(X[:M].copy()), Wq_d, Ws_d, N=N))
        assert_close(Y[:, cols], oracle.gemm_w4a16(X[:M], Wq, Ws), what=f"w4a16 M={M}")


def _dev_index(Y, rows, cols):
    """Y[rows][:, cols] gathered on the device, then copied to the host."""
    r = torch.from_numpy(np.asarray(rows, np.int64)).to(Y.device)
    c = torch.from_numpy(np.asarray(cols, np.int64)).to(Y.device)
    return host(Y.index_select(0, r).index_select(1, c))


@pytest.mark.parametrize("proj", list(QWEN7B))
def test_qwen7b_prefill_shapes(proj):
    """M = 2048 prefill on the same packed buffer, all four projections (the
    TILED family in both modes; gate|up walks about 9.5 tiles per persistent
    W4A4 workgroup): sampled rows and columns against the oracle, and for the
    W4A4 layer the exact int32 group partials of the sampled rows over every
    column, with Y bitwise the same as without the partials output."""
    N, K = QWEN7B[proj]
    rng = synth.make_rng(2)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, 2048, K)
    rows = np.sort(rng.choice(2048, size=24, replace=False))
    cols = _sampled_cols(N, rng, 256)
    Wq_all, Ws_all = q.pack_w4(dev(W))
    Wq, Ws = oracle.pack_w4(W[cols])
    say(f"{proj} prefill w4a16")
    Y = q.gemm_w4a16(dev_bf16(X), Wq_all, Ws_all, N=N)
    assert_close(_dev_index(Y, rows, cols), oracle.gemm_w4a16(X[rows], Wq, Ws))
    del Y
    say(f"{proj} prefill w4a4")
    Xq_d, Xs_d = q.quant_act(dev_bf16(X))
    Y4 = q.gemm_w4a4(Xq_d, Xs_d, Wq_all, Ws_all, N=N)
    Xq, Xs = oracle.quant_act(X[rows])
    assert_close(_dev_index(Y4, rows, cols), oracle.gemm_w4a4(Xq, Xs, Wq, Ws))
    say(f"{proj} prefill w4a4 partials")
    Y4p, P = q.gemm_w4a4(Xq_d, Xs_d, Wq_all, Ws_all, partials=True, N=N)
    assert torch.equal(Y4p.view(torch.int32), Y4.view(torch.int32))
    del Y4, Y4p
    r = torch.from_numpy(rows.astype(np.int64)).to(P.device)
    Pr = host(P.index_select(0, r))
    del P
    Wq_host = oracle.untile_w4(host(Wq_all), N)
    assert np.array_equal(Pr, oracle.w4a4_partials(Xq, Wq_host))


@pytest.mark.parametrize("K", [128, 384])
def test_tiled_several_tiles_per_workgroup(K):
    """The W4A4 prefill grid is persistent (512 workgroups walking the
    tiles): M = 2100, N = 4000 makes 528 tile slots, so the first workgroups
    carry a second tile, with ragged M and N tails and one or three groups
    per tile (the group pipeline runs across the tile boundary)."""
    M, N = 2100, 4000
    say(f"tiled several tiles per workgroup K={K}")
    rng = synth.make_rng(23)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K, n_outliers=1)
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    Wq_d, Ws_d = dev_w(Wq), dev_s(Ws)
    Y = q.gemm_w4a4(dev(Xq), dev(Xs), Wq_d, Ws_d, variant=q.GEMM_TILED, N=N)
    assert_close(host(Y), oracle.gemm_w4a4(Xq, Xs, Wq, Ws), what="w4a4 tiled, several tiles")
    Y16 = q.gemm_w4a16(dev_bf16(X), Wq_d, Ws_d, variant=q.GEMM_TILED, N=N)
    assert_close(host(Y16), oracle.gemm_w4a16(X, Wq, Ws), what="w4a16 tiled")


def test_largest_k():
    """K = 2^20 (8192 groups, the largest the library accepts) in every
    family of both modes: the k-split plans and the 32-bit buffer offsets at
    their limit."""
    M, N, K = 3, 40, 1 << 20
    rng = synth.make_rng(25)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K, n_outliers=synth.outlier_count(K))
    Wq, Ws = oracle.pack_w4(W)
    Xq, Xs = oracle.quant_act(X)
    Wq_d, Ws_d = dev_w(Wq), dev_s(Ws)
    want4 = oracle.gemm_w4a4(Xq, Xs, Wq, Ws)
    want16 = oracle.gemm_w4a16(X, Wq, Ws)
    for v in W4A4_VARIANTS:
        say(f"largest K w4a4 variant={v}")
        Y = q.gemm_w4a4(dev(Xq), dev(Xs), Wq_d, Ws_d, variant=v, N=N)
        assert_close(host(Y), want4, what=f"w4a4 K=2^20 variant={v}")
    for v in W4A16_VARIANTS:
        say(f"largest K w4a16 variant={v}")
        Y = q.gemm_w4a16(dev_bf16(X), Wq_d, Ws_d, variant=v, N=N)
        assert_close(host(Y), want16, what=f"w4a16 K=2^20 variant={v}")


LLAMA8B = {"qkv": (6144, 4096), "o": (4096, 4096), "gate_up": (28672, 4096),
           "down": (4096, 14336), "lm_head": (128256, 4096)}


@pytest.mark.parametrize("proj", list(LLAMA8B))
def test_llama8b_verify_batch_shapes(proj):
    """Llama-3-8B-shaped layers at the verify batch of 32 sequences
    (M = 32 (gamma + 1) = 160 and 288, gamma 4 / 8) in W4A16, AUTO: sampled
    output columns against the oracle, computed from those weight rows."""
    N, K = LLAMA8B[proj]
    rng = synth.make_rng(4)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, 288, K, n_outliers=synth.outlier_count(K))
    cols = _sampled_cols(N, rng, 384)
    Wq, Ws = oracle.pack_w4(W[cols])
    Wq_d, Ws_d = q.pack_w4(dev(W))
    del W
    for M in (160, 288):
        say(f"llama8b {proj} w4a16 M={M}")
        Y = host(q.gemm_w4a16(dev_bf16(X[:M].copy()), Wq_d, Ws_d, N=N))
        assert_close(Y[:, cols], oracle.gemm_w4a16(X[:M], Wq, Ws), what=f"{proj} M={M}")


def test_llama8b_lm_head_gemv():
    N, K = LLAMA8B_HEAD
    rng = synth.make_rng(3)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, 1, K)
    cols = _sampled_cols(N, rng, 2048)
    Wq, Ws = oracle.pack_w4(W[cols])
    Wq_d, Ws_d = q.pack_w4(dev(W))
    del W
    for v in W4A16_VARIANTS:
        say(f"lm_head variant={v}")
        Y = host(q.gemm_w4a16(dev_bf16(X), Wq_d, Ws_d, variant=v, N=N))
        assert_close(Y[:, cols], oracle.gemm_w4a16(X, Wq, Ws))


# ------------------------------------------------------------------ graphs
def test_graph_replays_match_eager():
    """The library's launches captured in a HIP graph (split-K shapes whose
    in-kernel reduction relies on workspace counters the kernels reset) give
    the eager result on every replay, with eager work in between."""
    M4, M16, N, K = 8, 40, 3584, 18944          # a split-K shape in both modes
    W, X = _case(19, M16, N, K)
    Wq, Ws = oracle.pack_w4(W)
    Wq_d, Ws_d, X_d = dev_w(Wq), dev_s(Ws), dev_bf16(X)
    X4 = X_d[:M4].contiguous()
    Xq, Xs = q.quant_act(X4)
    Y4 = torch.empty((M4, N), dtype=torch.float32, device="cuda")
    Y16 = torch.empty((M16, N), dtype=torch.float32, device="cuda")
    ws4 = torch.zeros(q.workspace_bytes(1, M4, N, K), dtype=torch.uint8, device="cuda")
    ws16 = torch.zeros(q.workspace_bytes(2, M16, N, K), dtype=torch.uint8, device="cuda")
    # the W4A8 tier and the bf16 output on the same split-K shape, each with
    # a workspace of its own
    X8q, X8s = q.quant_act8(X4)
    Y8 = torch.empty((M4, N), dtype=torch.float32, device="cuda")
    Yb = torch.empty((M4, N), dtype=torch.bfloat16, device="cuda")
    ws8 = torch.zeros(q.workspace_bytes(4, M4, N, K), dtype=torch.uint8, device="cuda")
    wsb = torch.zeros(q.workspace_bytes(1, M4, N, K), dtype=torch.uint8, device="cuda")

    def body():
        q.quant_act(X4, Xq, Xs)
        q.gemm_w4a4(Xq, Xs, Wq_d, Ws_d, Y=Y4, ws=ws4, N=N)
        q.gemm_w4a16(X_d, Wq_d, Ws_d, Y=Y16, ws=ws16, N=N)
        q.quant_act8(X4, X8q, X8s)
        q.gemm_w4a8(X8q, X8s, Wq_d, Ws_d, Y=Y8, ws=ws8, N=N)
        q.gemm_w4a4_bf16(Xq, Xs, Wq_d, Ws_d, variant=q.GEMM_SKINNY, Y=Yb, ws=wsb, N=N)

    body()
    torch.cuda.synchronize()
    e4, e16 = host(Y4).copy(), host(Y16).copy()
    e8, eb = host(Y8).copy(), host_bits16(Yb).copy()
    assert_close(e16, oracle.gemm_w4a16(X, Wq, Ws))
    assert_close(e8, oracle.gemm_w4a8(*oracle.quant_act8(X[:M4]), Wq, Ws), what="w4a8")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        body()
    for rep in range(3):
        for t in (Y4, Y16, Y8, Yb):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y4).view(np.uint32), e4.view(np.uint32)), rep
        assert np.array_equal(host(Y16).view(np.uint32), e16.view(np.uint32)), rep
        assert np.array_equal(host(Y8).view(np.uint32), e8.view(np.uint32)), rep
        assert np.array_equal(host_bits16(Yb), eb), rep
        body()                                   # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(host(Y16).view(np.uint32), e16.view(np.uint32)), rep
        assert np.array_equal(host(Y8).view(np.uint32), e8.view(np.uint32)), rep


def test_workspace_reused_across_shapes():
    """One zero-filled workspace serves a run of k-split calls of different
    shapes and modes (different counter counts and slice counts) and of the
    GEMV family: each call leaves its arrival counters at zero, and every
    family's partials go to the other half of the workspace, so each call
    finds its counters clear whatever partials the earlier calls left."""
    shapes = [(8, 3584, 18944), (40, 4608, 3584), (5, 1028, 1024), (16, 2048, 5632)]
    nb = max(q.workspace_bytes(op, M, N, K) for (M, N, K) in shapes for op in (1, 2))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    cases = []
    for i, (M, N, K) in enumerate(shapes):
        W, X = _case(20 + i, M, N, K)
        Wq, Ws = oracle.pack_w4(W)
        Xq, Xs = oracle.quant_act(X)
        cases.append((M, N, K, X, Xq, Xs, Wq, Ws, dev_w(Wq), dev_s(Ws)))
    for rep in range(2):
        for (M, N, K, X, Xq, Xs, Wq, Ws, Wq_d, Ws_d) in cases:
            want16, want4 = oracle.gemm_w4a16(X, Wq, Ws), oracle.gemm_w4a4(Xq, Xs, Wq, Ws)
            # k-split calls of both modes and the GEMV family's partials,
            # interleaved on one workspace
            say(f"workspace reuse rep={rep} M={M} N={N} K={K}")
            Y = q.gemm_w4a16(dev_bf16(X), Wq_d, Ws_d, variant=q.GEMM_SKINNY, ws=ws, N=N)
            assert_close(host(Y), want16, what="w4a16 reused ws")
            Y = q.gemm_w4a16(dev_bf16(X), Wq_d, Ws_d, variant=q.GEMM_GEMV, ws=ws, N=N)
            assert_close(host(Y), want16, what="w4a16 GEMV reused ws")
            Y = q.gemm_w4a4(dev(Xq), dev(Xs), Wq_d, Ws_d, variant=q.GEMM_SKINNY, ws=ws, N=N)
            assert_close(host(Y), want4, what="w4a4 reused ws")
