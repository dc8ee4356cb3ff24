"""Oracle: a decoder that runs every linear layer on the shared INT4 buffer
in either mode, and the greedy self-speculative loop over it.

TEST INFRASTRUCTURE ONLY (see the package header): plain numpy, fp64
arithmetic with rounding to fp32 / bf16 only at the points listed below.

What the pages fix, and what is a reading:

* [QSpec, Abstract (arXiv)]: drafting runs the model with low-precision joint
  (weight and activation) quantization, verification with weight-only
  quantization; both stages reuse the same weights and the same KV cache.
  Here: draft forwards call ``quant_act`` + ``gemm_w4a4``, verify forwards
  call ``gemm_w4a16``, on one ``pack_w4`` buffer per matrix, and both write
  one KV cache; the verify pass overwrites the KV rows of every position it
  processes.
* [SpecQuant-review, method paragraph "Verification ..."]: the draft
  proposes a block, the parent checks the block in parallel, accepts a full
  match and rewrites the first mismatch.  Greedy form: ``verify_greedy``.
* [QSpec-blog, paragraph 2]: W4A4 drafts, W4A16 verifies; verification keeps
  the output that of the high-precision scheme.  Consequence used as a pin:
  greedy self-speculation emits exactly the pure W4A16 greedy tokens.
* [SpecQuant, Abstract (arXiv)] and ["Speculative Decoding Meets
  Quantization: Compatibility Evaluation and Hierarchical Framework Design",
  Abstract (arXiv)]: variants of one base model at several precisions, a
  middle precision among the drafters.  Here a third mode, ``w4a8``: the
  same INT4 weights with 8-bit per-token activation codes (``w4a8.py``), as
  the drafter of the same loop; the same pin holds for it.

The pages name no architecture.  Reading (plain Llama-style decoder):
pre-norm RMSNorm (weight 1, epsilon from the config); RoPE, rotate-half
convention, base from the config; grouped-query causal attention with scale
1/sqrt(head_dim); SwiGLU MLP down(silu(gate) * up) with gate|up as one matrix
(gate rows first); no biases; untied INT4 lm_head; bf16 embedding.

Rounding points (the GPU path rounds at the same places): the residual
stream is fp32; every GEMM input is bf16 (normalised activations, attention
output, silu * up); every GEMM output is fp32; the KV cache is bf16 (keys
after RoPE); queries after RoPE are fp32; logits are fp32.  Everything
between two rounding points is fp64 here.  Rows are processed independently
(one query per row over its own sequence's cache), so a row's result does not
depend on which other rows share its pass.

Parity status: pinned by tests/test_oracle_model.py -- RoPE identities
(position 0, norm preservation, relative-position dot products), attention
closed forms (one key, constant query), RMSNorm scale invariance, direct
fp64 -> bf16 rounding against hand-built ties, and the self-speculation
invariant (tokens and committed KV rows equal pure W4A16 greedy decoding).
"""

import numpy as np

from .quant import bf16_bits_to_f32, gemm_w4a4, gemm_w4a16, pack_w4, quant_act
from .verify import verify_greedy
from .w4a8 import gemm_w4a8, quant_act8

DRAFT, VERIFY, DRAFT8 = "w4a4", "w4a16", "w4a8"


# --------------------------------------------------------------------------
# rounding helpers
# --------------------------------------------------------------------------
def to_bf16_bits(x):
    """fp64 values -> bf16 bits, one round-to-nearest-even step from the
    exact value (no intermediate fp32 rounding).  bf16 keeps 8 significant
    bits; values below 2**-126 fall on the subnormal grid 2**-133."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value")
    e = np.frexp(x)[1]
    e = np.maximum(e, -125)
    y = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)      # rint: ties to even
    if np.any(np.abs(y) > 3.3895313892515355e38):
        raise ValueError("bf16 overflow")
    return (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_values(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------
# model pieces
# --------------------------------------------------------------------------
def rmsnorm(x, eps):
    """x / sqrt(mean(x^2) + eps) per row, weight 1 (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope_inv_freq(head_dim, base):
    """base ** (-2 i / head_dim), i = 0 .. head_dim/2 - 1."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def rope(x, pos, base):
    """Rotate-half RoPE on the last axis of x [..., head_dim] at integer
    positions pos (broadcast over the leading axes): the pair (x_i, x_{i+h})
    with h = head_dim/2 turns by the angle pos * inv_freq_i."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(2 * h, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def attend(q, keys, values):
    """One query head q [hd] over keys/values [T, hd]: softmax(K q / sqrt(hd))
    weighted sum of values (fp64, max-subtracted)."""
    s = keys @ q / np.sqrt(q.shape[-1])
    p = np.exp(s - s.max())
    return (p / p.sum()) @ values


class Model:
    """Packed weights of one decoder (from synth.model_weights)."""

    def __init__(self, cfg, w):
        self.cfg = cfg
        self.emb = bf16_bits_to_f32(w["emb"])               # fp32 values of the bf16 table
        self.layers = [{k: pack_w4(L[k]) for k in ("qkv", "o", "gu", "down")}
                       for L in w["layers"]]
        self.lm = pack_w4(w["lm"])


class KVCache:
    """bf16-valued keys (after RoPE) and values, [layer][B, n_kv, cap, hd]."""

    def __init__(self, cfg, B, cap):
        shape = (cfg.n_layers, B, cfg.n_kv, cap, cfg.head_dim)
        self.k = np.zeros(shape, dtype=np.float64)
        self.v = np.zeros(shape, dtype=np.float64)
        self.cap = cap


def linear(mode, x_bits, packed):
    """bf16 input bits [M, K] -> fp32 output [M, N] in draft (W4A4 or W4A8)
    or verify mode."""
    Wq, Ws = packed
    if mode == VERIFY:
        y = gemm_w4a16(x_bits, Wq, Ws)
    elif mode == DRAFT:
        Xq, Xs = quant_act(x_bits)
        y = gemm_w4a4(Xq, Xs, Wq, Ws)
    elif mode == DRAFT8:
        Xq8, Xs8 = quant_act8(x_bits)
        y = gemm_w4a8(Xq8, Xs8, Wq, Ws)
    else:
        raise ValueError(mode)
    return y.astype(np.float32)


def forward(model, kv, seq, pos, tok, mode):
    """Run rows (sequence seq[m], position pos[m], token tok[m]) through the
    decoder in `mode`; writes the rows' keys/values into `kv` (all rows of a
    layer before any row attends) and returns fp32 logits [M, V]."""
    cfg = model.cfg
    seq = np.asarray(seq, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    tok = np.asarray(tok, dtype=np.int64)
    M = seq.shape[0]
    if np.any(pos >= kv.cap) or np.any(pos < 0):
        raise ValueError("position outside the KV cache")
    H, Hkv, hd = cfg.n_heads, cfg.n_kv, cfg.head_dim
    grp = H // Hkv
    x = model.emb[tok].astype(np.float32)                    # fp32 residual stream
    for li, L in enumerate(model.layers):
        h = to_bf16_bits(rmsnorm(x, cfg.eps))
        qkv = linear(mode, h, L["qkv"]).astype(np.float64)
        q = qkv[:, :cfg.q_dim].reshape(M, H, hd)
        k = qkv[:, cfg.q_dim:cfg.q_dim + cfg.kv_dim].reshape(M, Hkv, hd)
        v = qkv[:, cfg.q_dim + cfg.kv_dim:].reshape(M, Hkv, hd)
        q = rope(q, pos[:, None], cfg.rope_base).astype(np.float32).astype(np.float64)
        k = bf16_values(to_bf16_bits(rope(k, pos[:, None], cfg.rope_base)))
        v = bf16_values(to_bf16_bits(v))
        for m in range(M):
            kv.k[li, seq[m], :, pos[m]] = k[m]
            kv.v[li, seq[m], :, pos[m]] = v[m]
        att = np.empty((M, H, hd), dtype=np.float64)
        for m in range(M):
            T = pos[m] + 1
            for hh in range(H):
                g = hh // grp
                att[m, hh] = attend(q[m, hh], kv.k[li, seq[m], g, :T], kv.v[li, seq[m], g, :T])
        o = linear(mode, to_bf16_bits(att.reshape(M, H * hd)), L["o"])
        x = (x + o).astype(np.float32)
        h2 = to_bf16_bits(rmsnorm(x, cfg.eps))
        gu = linear(mode, h2, L["gu"]).astype(np.float64)
        a = to_bf16_bits(silu(gu[:, :cfg.ffn]) * gu[:, cfg.ffn:])
        d = linear(mode, a, L["down"])
        x = (x + d).astype(np.float32)
    hf = to_bf16_bits(rmsnorm(x, cfg.eps))
    return linear(mode, hf, model.lm)


def argmax_first(logits):
    """index of the largest value per row; the lowest index among equals."""
    return np.argmax(logits, axis=-1).astype(np.int32)


# --------------------------------------------------------------------------
# decoding loops
# --------------------------------------------------------------------------
def prefill(model, kv, prompts):
    """W4A16 over every prompt position; the last position's argmax is each
    sequence's first generated token."""
    B, P = prompts.shape
    seq = np.repeat(np.arange(B), P)
    pos = np.tile(np.arange(P), B)
    logits = forward(model, kv, seq, pos, prompts.reshape(-1), VERIFY)
    return argmax_first(logits.reshape(B, P, -1)[:, -1])


def kv_capacity(P, n_gen, gamma):
    return P + n_gen + gamma + 1


def top2_margin(logits):
    """(largest - second largest) / max|value| per row (0 for an exact tie)."""
    part = np.sort(logits.astype(np.float64), axis=-1)
    scale = np.maximum(np.abs(part[..., 0]), np.abs(part[..., -1]))
    return (part[..., -1] - part[..., -2]) / scale


def greedy_decode(model, prompts, n_gen, gamma=4, with_margins=False):
    """Pure W4A16 greedy decoding: one token per sequence per forward.
    Returns (tokens [B, n_gen], kv), plus the relative top-2 logit margin
    behind every token [B, n_gen] when with_margins is set."""
    B, P = prompts.shape
    kv = KVCache(model.cfg, B, kv_capacity(P, n_gen, gamma))
    if with_margins:
        Bq, Pq = prompts.shape
        seq = np.repeat(np.arange(Bq), Pq)
        pos = np.tile(np.arange(Pq), Bq)
        lg = forward(model, kv, seq, pos, prompts.reshape(-1), VERIFY).reshape(Bq, Pq, -1)[:, -1]
        last = argmax_first(lg)
        margins = [top2_margin(lg)]
    else:
        last = prefill(model, kv, prompts)
    out = [last]
    L = np.full(B, P + 1)
    for _ in range(n_gen - 1):
        logits = forward(model, kv, np.arange(B), L - 1, last, VERIFY)
        last = argmax_first(logits)
        out.append(last)
        if with_margins:
            margins.append(top2_margin(logits))
        L += 1
    toks = np.stack(out, axis=1)
    if with_margins:
        return toks, kv, np.stack(margins, axis=1)
    return toks, kv


def selfspec_greedy(model, prompts, n_gen, gamma, trace=None, draft_mode=DRAFT):
    """Greedy self-speculation: per round, gamma draft forwards in
    `draft_mode` (W4A4, or the W4A8 tier; one row per active sequence, each
    at its own position), one W4A16 verify forward
    over [last, d_0 .. d_{gamma-1}] that overwrites those KV rows, then the
    greedy acceptance rule; each sequence advances by n_accept + 1.  A
    sequence stops once it has n_gen tokens.  Returns (tokens [B, n_gen],
    kv, stats) with stats = dict(accepted, drafted, rounds).  With a list
    `trace`, every round appends dict(act = the active sequences, drafts
    [nA, gamma], n_accept [nA], draft_margin [nA, gamma] = the relative top-2
    margin of the draft logits behind each drafted token, verify_margin
    [nA, gamma + 1] = the same for the verify logits at each position)."""
    B, P = prompts.shape
    kv = KVCache(model.cfg, B, kv_capacity(P, n_gen, gamma))
    last = prefill(model, kv, prompts)
    gen = [[int(t)] for t in last]
    L = np.full(B, P + 1)
    accepted = drafted = rounds = 0
    while True:
        act = np.array([b for b in range(B) if len(gen[b]) < n_gen], dtype=np.int64)
        if act.size == 0:
            break
        rounds += 1
        nA = act.size
        vtok = np.zeros((nA, gamma + 1), dtype=np.int32)
        vtok[:, 0] = last[act]
        dmargin = np.zeros((nA, gamma))
        for j in range(gamma):
            logits = forward(model, kv, act, L[act] - 1 + j, vtok[:, j], draft_mode)
            vtok[:, j + 1] = argmax_first(logits)
            dmargin[:, j] = top2_margin(logits)
        seq = np.repeat(act, gamma + 1)
        pos = (L[act][:, None] - 1 + np.arange(gamma + 1)[None, :]).reshape(-1)
        logits = forward(model, kv, seq, pos, vtok.reshape(-1), VERIFY)
        n, out = verify_greedy(logits.reshape(nA, gamma + 1, -1), vtok[:, 1:].copy())
        if trace is not None:
            trace.append(dict(act=act.copy(), drafts=vtok[:, 1:].copy(), n_accept=n.copy(),
                              draft_margin=dmargin,
                              verify_margin=top2_margin(logits).reshape(nA, gamma + 1)))
        for i, b in enumerate(act):
            k = int(n[i])
            gen[b].extend(int(t) for t in out[i, :k + 1])
            L[b] += k + 1
            last[b] = out[i, k]
            accepted += k
            drafted += gamma
    toks = np.array([g[:n_gen] for g in gen], dtype=np.int32)
    return toks, kv, dict(accepted=accepted, drafted=drafted, rounds=rounds)
