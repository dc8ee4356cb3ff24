"""Oracle: the per-group Walsh-Hadamard rotation in front of the quantizers.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix and what is read into them
---------------------------------------------
[QSpec, Builds on] lists "QuaRot: Outlier-Free 4-Bit Inference in Rotated
LLMs" and "SmoothQuant" among the works QSpec builds on; the pages print
nothing of either beyond the title.  The reading taken here is the plainest
one that keeps the shared INT4 format of ``oracle.quant`` unchanged:

* an orthogonal rotation by a Walsh-Hadamard matrix applied block-diagonally,
  one 128 x 128 block per quantization group, so a rotated group is still a
  group and the per-group scales of the shared buffer keep their meaning;
* H is the Sylvester Hadamard matrix of order 128 (entries +-1,
  H[i][j] = (-1)^popcount(i & j)), so H H^T = 128 I;
* activations are rotated as x' = H x / 16 and weights as w' = H w / 8 (per
  group), so x' . w' = x^T H^T H w / 128 = x . w: the layer's product is
  unchanged in exact arithmetic, and both scales are powers of two (exact);
* the rotation is computed as the fast transform: stages s = 0 .. 6; at stage
  s every pair of positions (i, i + 2^s) with bit s of i clear becomes
  (a + b, a - b), each add and subtract one fp32 operation (round to nearest
  even); then the power-of-two scale.  This fixes every bit of x', so the
  codes the quantizer derives from it are unique;
* drafter input: the codes of x' (its fp32 values, not rounded to bf16) by the
  activation quantizer of ``oracle.quant``; verifier input: bf16(x') (round
  to nearest even); weights: ``pack_w4(w')``.

Parity pins (tests/test_oracle_rotate.py): the fast transform equals the
product by scipy's Hadamard matrix exactly on small-integer inputs and to
fp32 rounding in general; applying it twice gives 128 x exactly on small
integers; x' . w' = x . w in fp64 to the fp32 rounding of the transform; a
single spike spreads into 128 values of equal magnitude; on activations with
x20 outlier channels the W4A4 layer's error against the exact product drops
with the rotation.
"""

import numpy as np

from .quant import GROUP, bf16_bits_to_f32, f32_to_bf16_bits, quant_act_values

X_SHIFT = 4   # activations: x' = H x / 2^4
W_SHIFT = 3   # weights:     w' = H w / 2^3   (4 + 3 = log2(128))


def fwht128_f32(x):
    """Unnormalised fast Walsh-Hadamard transform of every 128-block of the
    last axis, in fp32, stage by stage (s = 0 .. 6; pair (i, i + 2^s) with
    bit s of i clear -> (a + b, a - b))."""
    x = np.array(x, dtype=np.float32, copy=True)
    K = x.shape[-1]
    if K % GROUP:
        raise ValueError("the last axis must be a multiple of 128")
    lead = x.shape[:-1]
    v = x.reshape(-1, K // GROUP, GROUP)
    for s in range(7):
        h = 1 << s
        w = v.reshape(v.shape[0], v.shape[1], GROUP // (2 * h), 2, h)
        a = w[:, :, :, 0, :].copy()
        b = w[:, :, :, 1, :].copy()
        w[:, :, :, 0, :] = a + b      # float32 + float32: one rounding
        w[:, :, :, 1, :] = a - b
        v = w.reshape(v.shape)
    return v.reshape(lead + (K,))


def _pow2(x, shift):
    return (x * np.float32(2.0 ** -shift)).astype(np.float32)   # exact


def rotate_x(X_bits):
    """bf16 activations [M, K] (bits) -> x' = H x / 16 per group, fp32."""
    return _pow2(fwht128_f32(bf16_bits_to_f32(X_bits)), X_SHIFT)


def rotate_x_bf16(X_bits):
    """The verifier's rotated input: bf16(x') (round to nearest even)."""
    return f32_to_bf16_bits(rotate_x(X_bits))


def rotate_w(W):
    """fp32 weights [N, K] -> w' = H w / 8 per group, fp32."""
    return _pow2(fwht128_f32(np.asarray(W, dtype=np.float32)), W_SHIFT)


def quant_act_rot(X_bits):
    """The drafter's rotated input: codes and scales of x' = H x / 16."""
    return quant_act_values(rotate_x(X_bits))
