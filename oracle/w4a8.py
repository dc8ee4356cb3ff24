"""Oracle: a W4A8 middle tier on the shared INT4 buffer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix and what is read into them
---------------------------------------------
[SpecQuant, Abstract (arXiv)] derives several precisions from one base model,
an 8-bit variant between INT4 and FP16 among them; [QSpec, Builds on] lists
QServe, whose scheme pairs 4-bit weights with 8-bit activations.  The pages
print no formula for either.  The reading taken here keeps QSpec's shared
buffer (no extra weight copy): the packed INT4 weights and fp16 group scales
of ``oracle.quant.pack_w4`` are read unchanged, and only the activations move
to 8 bits, quantized the way ``oracle.quant.quant_act`` quantizes them at
4 bits with the symmetric 8-bit range:

* per token row m: a = max_k |x[m,k]| (exact), s = a / 127 (fp32 IEEE
  divide), kept as fp32 in Xs[m];
* code q = clamp(rne(x / s), -128, 127) (fp32 IEEE divide, round half to
  even); a == 0 gives s = 0 and all codes 0; -128 is never reached, since
  |x / s| <= 127 (1 + 2^-23) rounds to 127;
* codes stored one signed byte each, row-major [M][K];
* P[m,n,g] = sum_{k in g} q[m,k] qw[n,k] exactly (|P| <= 128 * 127 * 8),
  Y[m,n] = Xs[m] * sum_g float(Ws[n,g]) * P[m,n,g], groups in ascending
  order, in fp64.

Parity pins (tests/test_oracle_w4a8.py): hand-built rows with every rounding
tie and the clamp, brute-force integer partials on tiny shapes, the lossless
closed form (activations c * 2^e with |c| <= 127 integer and max |c| = 127:
the codes are exact and W4A8 equals W4A16 up to fp64 rounding), the
quantization error bound |x - s q| <= s / 2, and the error ordering on
Qwen2.5-7B-shaped activations with x20 outlier channels (W4A8 error against
the exact product far below W4A4's).
"""

import numpy as np

from .quant import GROUP, bf16_bits_to_f32, unpack_nibbles

QMAX8 = 127
QLO8, QHI8 = -128, 127


def quant_act8(X_bits):
    """bf16 activations [M, K] (bits) -> (codes int8 [M, K], scales fp32 [M])."""
    x = bf16_bits_to_f32(X_bits)
    if x.ndim != 2:
        raise ValueError("X must be 2-D [M, K]")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite activation")
    a = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = (a / np.float32(QMAX8)).astype(np.float32)            # IEEE fp32 divide
    safe = np.where(s == 0, np.float32(1), s)
    ratio = (x / safe[:, None]).astype(np.float32)            # IEEE fp32 divide
    q = np.clip(np.rint(ratio), QLO8, QHI8)
    q = np.where((s == 0)[:, None], 0, q).astype(np.int8)
    return q, s


def w4a8_partials(Xq8, Wq, group=GROUP):
    """P[m, n, g] = sum_{k in group g} q[m,k] * qw[n,k], exact, int32 (one
    fp64 matmul of integer-valued matrices per group: every partial sum is an
    integer below 2^21, exact in fp64)."""
    qa = np.asarray(Xq8, dtype=np.int8).astype(np.float64)
    qw = unpack_nibbles(Wq).astype(np.float64)
    M, K = qa.shape
    if qw.shape[1] != K:
        raise ValueError("K mismatch")
    G = K // group
    P = np.empty((M, qw.shape[0], G), dtype=np.int32)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        P[:, :, g] = (qa[:, sl] @ qw[:, sl].T).astype(np.int32)
    return P


def gemm_w4a8(Xq8, Xs, Wq, Ws, group=GROUP):
    """Y = Xs[m] * sum_g Ws[n,g] * P[m,n,g] (fp64), groups ascending."""
    qa = np.asarray(Xq8, dtype=np.int8).astype(np.float64)
    qw = unpack_nibbles(Wq).astype(np.float64)
    M, K = qa.shape
    N = qw.shape[0]
    if Ws.shape != (N, K // group):
        raise ValueError("weight buffer shape mismatch")
    ws = np.asarray(Ws, dtype=np.uint16).view(np.float16).astype(np.float64)
    Y = np.zeros((M, N), dtype=np.float64)
    for g in range(K // group):
        sl = slice(g * group, (g + 1) * group)
        Y += (qa[:, sl] @ qw[:, sl].T) * ws[None, :, g]
    return Y * np.asarray(Xs, dtype=np.float64)[:, None]
