"""Oracle: shared INT4 weight format, activation quantizer and both GEMMs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix and what is read into them
---------------------------------------------
[QSpec, Abstract (arXiv)] and [QSpec-blog, paragraphs 2 and 4]: one set of
4-bit weights serves two modes -- W4A4 (weights *and* activations at four
bits, the fast lossy drafter) and W4A16 (weights at four bits, activations at
16 bits, the accurate verifier).  The pages print no quantizer formula, no
group size, no scale precision and no bit layout.  Readings taken here:

* weights: symmetric INT4, one fp16 scale per row and per group of 128
  consecutive K; scale = fp16(absmax / 7) with an IEEE fp32 divide then a
  round-to-nearest-even to fp16; code = clamp(rne(w / scale), -8, 7) with an
  IEEE fp32 divide by the *rounded* scale; an all-zero (or underflowed-scale)
  group has code 0 everywhere.
* activations: one fp32 scale per token row over all K, scale = absmax / 7
  (IEEE fp32 divide, no fp16 rounding); code = clamp(rne(x / scale), -8, 7)
  with an IEEE fp32 divide (not a multiply by the reciprocal).
* packing: two's-complement nibbles, element 2i in the low nibble of byte i
  of its row, element 2i+1 in the high nibble.
* storage order of the packed weights (a layout choice, no arithmetic): rows
  are padded with zero codes to a multiple of 16 and the row-major bytes are
  re-ordered in 1 KiB tiles, one per (16-row block b, group g); inside a tile,
  16-byte slot l holds the 32 codes k in [128 g + 32 (l // 16), +32) of row
  16 b + (l % 16).  The fp16 scales are padded the same way and stored as
  32-byte tiles, one per (16-row block b, group g), row order inside.
  ``tile_w4`` / ``untile_w4`` and ``tile_scales`` / ``untile_scales``
  convert.
* W4A4: per-group integer partials P[m,n,g] = sum_k qa*qw (exact), then
  Y = a_scale[m] * sum_g w_scale[n,g] * P[m,n,g].
* W4A16: Y = sum_g w_scale[n,g] * sum_k x[m,k]*q[n,k] with x the bf16 value.

Precision: every decision that turns a float into an integer (absmax, the
divide, the rounding, the clamp) is taken in fp32 exactly as stated above --
the same precision the kernels use, and IEEE-defined, so the result is unique.
Sums of products are taken in fp64.

Parity pins (tests/test_oracle_quant.py): exhaustive nibble table, hand
examples, pack idempotence and error bound, round-half-even ties, divide vs
reciprocal cases checked with exact rational arithmetic, brute-force integer
dot products, exact-rational W4A16 on tiny shapes, and the lossless special
case where W4A4 and W4A16 coincide.
"""

import numpy as np

GROUP = 128
QMAX = 7          # symmetric int4: largest code magnitude used for the scale
QLO, QHI = -8, 7  # two's-complement int4 range (the clamp)


# --------------------------------------------------------------------------
# bf16 helpers (bf16 values travel as their 16 raw bits in uint16 arrays)
# --------------------------------------------------------------------------
def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> the exact float32 values they encode."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x):
    """float32 -> bf16 bits, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


# --------------------------------------------------------------------------
# nibble packing
# --------------------------------------------------------------------------
def pack_nibbles(q):
    """int codes [R, K] in [-8, 7] -> bytes [R, K/2]; even k low, odd k high."""
    q = np.asarray(q)
    if q.shape[-1] % 2:
        raise ValueError("K must be even")
    if q.size and (q.min() < QLO or q.max() > QHI):
        raise ValueError("codes outside [-8, 7]")
    lo = (q[..., 0::2].astype(np.int64) & 0xF)
    hi = (q[..., 1::2].astype(np.int64) & 0xF)
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(b):
    """bytes [R, K/2] -> int8 codes [R, K] (two's-complement nibbles)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int16)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# --------------------------------------------------------------------------
# storage order of the shared weight buffer (pure re-layout)
# --------------------------------------------------------------------------
TILE_ROWS = 16


def tile_w4(Wq):
    """row-major packed bytes [N, K/2] -> tiled bytes [ceil(N/16)*16, K/2].

    Tile (b, g) = bytes [(b*G + g) * 1024, +1024) of the flat buffer; slot l
    (16 bytes) = row 16b + l%16, row bytes [64 g + 16 (l//16), +16).
    """
    Wq = np.asarray(Wq, dtype=np.uint8)
    N, KB = Wq.shape
    if KB % 64:
        raise ValueError("K must be a multiple of 128")
    G = KB // 64
    Np = -(-N // TILE_ROWS) * TILE_ROWS
    R = np.zeros((Np, KB), dtype=np.uint8)
    R[:N] = Wq
    # [b, r, g, c, j] with row = 16b + r, byte = 64g + 16c + j
    T = R.reshape(Np // 16, 16, G, 4, 16)
    # tile order [b, g, c, r, j]: slot l = 16c + r
    T = T.transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(T).reshape(Np, KB)


def tile_scales(Ws):
    """row-major fp16 scale bits [N, G] -> tiled [ceil(N/16)*16, G]:
    element (b*G + g)*16 + r of the flat buffer = scale of row 16b + r, group g."""
    Ws = np.asarray(Ws, dtype=np.uint16)
    N, G = Ws.shape
    Np = -(-N // TILE_ROWS) * TILE_ROWS
    R = np.zeros((Np, G), dtype=np.uint16)
    R[:N] = Ws
    T = R.reshape(Np // 16, 16, G).transpose(0, 2, 1)
    return np.ascontiguousarray(T).reshape(Np, G)


def untile_scales(Wt, N):
    Wt = np.asarray(Wt, dtype=np.uint16)
    Np, G = Wt.shape
    T = Wt.reshape(Np // 16, G, 16).transpose(0, 2, 1)
    return np.ascontiguousarray(T).reshape(Np, G)[:N]


def untile_w4(Wt, N):
    """inverse of tile_w4 -> row-major [N, K/2] (padding rows dropped)."""
    Wt = np.asarray(Wt, dtype=np.uint8)
    Np, KB = Wt.shape
    G = KB // 64
    T = Wt.reshape(Np // 16, G, 4, 16, 16).transpose(0, 3, 1, 2, 4)
    return np.ascontiguousarray(T).reshape(Np, KB)[:N]


# --------------------------------------------------------------------------
# weights: the one packed buffer both modes read
# --------------------------------------------------------------------------
def pack_w4(W, group=GROUP):
    """Quantize fp32 weights [N, K] to the shared INT4 buffer.

    [QSpec, Abstract (arXiv)]: the drafter and the verifier reuse the same
    weights; [QSpec-blog, paragraph 4]: both configurations share the same
    underlying quantized weights.  Per (row n, group j):
        a  = max_k |W[n,k]|
        s  = fp16( fp32(a) / 7 )                       (stored scale)
        q  = clamp( rne( W[n,k] / fp32(s) ), -8, 7 )   (0 if s == 0)
    Returns (Wq uint8 [N, K/2], Ws uint16 [N, K/group] = fp16 bits).
    Raises ValueError for non-finite W or a scale that overflows fp16.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.ndim != 2:
        raise ValueError("W must be 2-D [N, K]")
    N, K = W.shape
    if group != GROUP or K % group:
        raise ValueError("group must be 128 and divide K")
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    G = K // group
    Wg = W.reshape(N, G, group)
    a = np.abs(Wg).max(axis=2)                                # exact, fp32
    with np.errstate(over="ignore"):
        s16 = (a / np.float32(QMAX)).astype(np.float16)      # IEEE fp32 /, RNE to fp16
    if not np.all(np.isfinite(s16)):
        raise ValueError("group scale overflows fp16")
    s32 = s16.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1), s32)
    ratio = Wg / safe[:, :, None]                             # IEEE fp32 divide
    q = np.clip(np.rint(ratio), QLO, QHI)                      # rne, then clamp
    q = np.where((s32 == 0)[:, :, None], 0, q).astype(np.int8).reshape(N, K)
    return pack_nibbles(q), s16.view(np.uint16).copy()


def dequant_w4(Wq, Ws, group=GROUP):
    """codes * scale as exact fp64 values [N, K] (for checks only)."""
    q = unpack_nibbles(Wq).astype(np.float64)
    s = np.asarray(Ws, dtype=np.uint16).view(np.float16).astype(np.float64)
    N, K = q.shape
    return (q.reshape(N, K // group, group) * s[:, :, None]).reshape(N, K)


# --------------------------------------------------------------------------
# activations: per-token quantizer of the W4A4 (draft) mode
# --------------------------------------------------------------------------
def quant_act(X_bits):
    """Quantize bf16 activations [M, K] (uint16 bits) to packed INT4.

    [QSpec-blog, paragraph 2]: the W4A4 scheme quantizes both weights and
    activations; [QSpec, Abstract (arXiv)]: "low-precision joint quantization"
    drafts.  Per token row m (reading: one scale over all K):
        a  = max_k |x[m,k]|,  s = fp32(a) / 7   (IEEE fp32, kept in fp32)
        q  = clamp( rne( x[m,k] / s ), -8, 7 )  (IEEE fp32 divide; 0 if a == 0)
    Returns (Xq uint8 [M, K/2], Xs float32 [M]).
    """
    return quant_act_values(bf16_bits_to_f32(X_bits))


def quant_act_values(x):
    """The quantizer of ``quant_act`` on fp32 values [M, K] (the bf16 inputs
    widened, or the fp32 output of the rotation in ``oracle.rotate``)."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("X must be 2-D [M, K]")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite activation")
    a = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = (a / np.float32(QMAX)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1), s)
    ratio = x / safe[:, None]                                 # IEEE fp32 divide
    q = np.clip(np.rint(ratio), QLO, QHI)
    q = np.where((s == 0)[:, None], 0, q).astype(np.int8)
    return pack_nibbles(q), s


# --------------------------------------------------------------------------
# W4A4: integer per-group partials, fp epilogue
# --------------------------------------------------------------------------
def _check_gemm_shapes(M, K, Wq, Ws, group):
    N = Wq.shape[0]
    if Wq.shape != (N, K // 2) or Ws.shape != (N, K // group):
        raise ValueError("weight buffer shape mismatch")
    return N


def w4a4_partials(Xq, Wq, group=GROUP):
    """P[m, n, g] = sum_{k in group g} qa[m,k] * qw[n,k], exact, int32.

    The products are integers with |P| <= 128*64, so an fp64 matmul of the
    integer-valued code matrices is exact; one matmul per group.
    """
    qa = unpack_nibbles(Xq).astype(np.float64)
    qw = unpack_nibbles(Wq).astype(np.float64)
    M, K = qa.shape
    N = qw.shape[0]
    G = K // group
    P = np.empty((M, N, G), dtype=np.int32)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        P[:, :, g] = (qa[:, sl] @ qw[:, sl].T).astype(np.int64)
    return P


def gemm_w4a4(Xq, Xs, Wq, Ws, group=GROUP):
    """Draft-mode linear layer: Y = Xs[m] * sum_g Ws[n,g] * P[m,n,g] (fp64).

    [QSpec, Abstract (arXiv)] low-precision joint quantization for drafting.
    Groups are accumulated in ascending g; nothing depends on M.
    """
    Xq = np.asarray(Xq, dtype=np.uint8)
    M, K = Xq.shape[0], 2 * Xq.shape[1]
    N = _check_gemm_shapes(M, K, Wq, Ws, group)
    qa = unpack_nibbles(Xq).astype(np.float64)
    qw = unpack_nibbles(Wq).astype(np.float64)
    ws = np.asarray(Ws, dtype=np.uint16).view(np.float16).astype(np.float64)
    Y = np.zeros((M, N), dtype=np.float64)
    for g in range(K // group):
        sl = slice(g * group, (g + 1) * group)
        Pg = qa[:, sl] @ qw[:, sl].T                     # exact integers
        Y += Pg * ws[None, :, g]
    return Y * np.asarray(Xs, dtype=np.float64)[:, None]


# --------------------------------------------------------------------------
# W4A16: weight-only dequantized GEMM
# --------------------------------------------------------------------------
def gemm_w4a16(X_bits, Wq, Ws, group=GROUP):
    """Verify-mode linear layer: Y = sum_g Ws[n,g] * sum_k x[m,k] q[n,k] (fp64).

    [QSpec, Abstract (arXiv)] high-precision weight-only quantization for
    verification; [QSpec-blog, paragraph 2] W4A16 keeps activations at higher
    precision.  x is the exact bf16 value; q the integer code.
    """
    x = bf16_bits_to_f32(X_bits).astype(np.float64)
    M, K = x.shape
    N = _check_gemm_shapes(M, K, Wq, Ws, group)
    q = unpack_nibbles(Wq).astype(np.float64)
    ws = np.asarray(Ws, dtype=np.uint16).view(np.float16).astype(np.float64)
    Y = np.zeros((M, N), dtype=np.float64)
    for g in range(K // group):
        sl = slice(g * group, (g + 1) * group)
        Y += (x[:, sl] @ q[:, sl].T) * ws[None, :, g]
    return Y
