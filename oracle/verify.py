"""Oracle: the draft/verify acceptance step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[QSpec-blog, paragraph 3]: a draft proposes several tokens, the target checks
them in one parallel pass, and the output distribution equals the target's.
[SpecQuant-review, method paragraph]: the draft emits a block, the parent
checks it in parallel, a full match is accepted, and the parent rewrites the
first mismatch.  [QSpec, Builds on] lists "Fast Inference from Transformers
via Speculative Decoding" and "Accelerating Large Language Model Decoding with
Speculative Sampling"; the sampling rule below is the standard rule of those
papers (the pages name it but print no formula).

Layouts: target logits [B, gamma+1, V] fp32, draft logits [B, gamma, V] fp32,
draft tokens [B, gamma] int32, u_accept [B, gamma] and u_sample [B] uniforms
in [0, 1) supplied by the caller.  Outputs: n_accept [B] int32 and
out_tok [B, gamma+1] int32 padded with -1.

Greedy (temperature 0):
    t_i = argmax_v L_t[b,i,v] (lowest index on ties), i = 0..gamma
    n   = first i with d_i != t_i, else gamma
    out = d_0..d_{n-1}, t_n.
Sampling (temperature 1):
    p_i = softmax(L_t[b,i]), q_i = softmax(L_d[b,i])            (fp64)
    for i < gamma: accept d_i iff u_accept[b,i] <= p_i(d_i) / q_i(d_i)
                   (if q_i(d_i) == 0: accept iff p_i(d_i) > 0)
    at the first reject n = i: r = max(0, p_n - q_n), or p_n if sum r == 0
    if all accepted:   n = gamma, r = p_gamma
    emitted = smallest j with C_j > u_sample[b] * R  (C = cumsum r, R = C_{V-1});
              if none, the last j with r_j > 0.
Near ties: the kernels compute the same quantities from fp32 logits with
their own summation order -- fp32 exponentials of the exactly carried
difference (about 2 ulp), fp64 sums -- so a decision can differ from exact
arithmetic only where the oracle's value sits close to the threshold:
within 1e-6 (relative) of p/q for an accept test, or within 5e-7 * R of a
cumulative boundary for the inverse-CDF draw (R = total residual mass; at a
vocabulary of 1e5 the boundaries are only ~1e-5 * R apart, so the window is
tied to the kernels' error, not to the spacing).  ``verify_sample`` reports
such sequences in ``flagged``; decisions must match on every other sequence.

Parity pins (tests/test_oracle_verify.py): planted-draft greedy cases for
every n in 0..gamma, a chi-square test of the speculative-sampling theorem
(first emitted token ~ p_0) and of P(accept) = sum_v min(p_v, q_v), the
residual distribution of the first emitted token after a forced reject, and
hand-worked tiny cases.
"""

import numpy as np

NEAR_TIE_ACCEPT_REL = 1e-6   # of p/q
NEAR_TIE_CDF_REL = 5e-7      # of the total residual mass R


def softmax64(logits):
    """softmax over the last axis in fp64 with max subtraction."""
    l = np.asarray(logits, dtype=np.float64)
    m = l.max(axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=-1, keepdims=True)


def _check(target_logits, draft_tok):
    t = np.asarray(target_logits, dtype=np.float32)
    d = np.asarray(draft_tok, dtype=np.int64)
    if t.ndim != 3 or d.ndim != 2 or t.shape[0] != d.shape[0] or t.shape[1] != d.shape[1] + 1:
        raise ValueError("shape mismatch")
    V = t.shape[2]
    if d.size and (d.min() < 0 or d.max() >= V):
        raise ValueError("draft token out of range")
    return t, d


def verify_greedy(target_logits, draft_tok):
    """Greedy acceptance -> (n_accept [B] int32, out_tok [B, gamma+1] int32)."""
    t, d = _check(target_logits, draft_tok)
    B, G1, V = t.shape
    gamma = G1 - 1
    n_acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, G1), -1, dtype=np.int32)
    for b in range(B):
        top = np.argmax(t[b], axis=-1)          # first index of the max
        n = gamma
        for i in range(gamma):
            if d[b, i] != top[i]:
                n = i
                break
        out[b, :n] = d[b, :n]
        out[b, n] = top[n]
        n_acc[b] = n
    return n_acc, out


def _inverse_cdf(r, u):
    """smallest j with cumsum(r)_j > u * sum(r); fallback last j with r_j > 0."""
    C = np.cumsum(r)
    R = C[-1]
    thr = u * R
    hits = np.nonzero(C > thr)[0]
    if hits.size:
        j = int(hits[0])
    else:
        j = int(np.nonzero(r > 0)[0][-1])
    lo = C[j - 1] if j > 0 else 0.0
    w = NEAR_TIE_CDF_REL * R
    near = (abs(thr - C[j]) <= w) or (j > 0 and abs(thr - lo) <= w)
    return j, bool(near)


def verify_sample(target_logits, draft_logits, draft_tok, u_accept, u_sample):
    """Speculative sampling at temperature 1.

    Returns (n_accept [B] int32, out_tok [B, gamma+1] int32, flagged [B] bool).
    """
    t, d = _check(target_logits, draft_tok)
    q_log = np.asarray(draft_logits, dtype=np.float32)
    ua = np.asarray(u_accept, dtype=np.float64)
    us = np.asarray(u_sample, dtype=np.float64)
    B, G1, V = t.shape
    gamma = G1 - 1
    if q_log.shape != (B, gamma, V) or ua.shape != (B, gamma) or us.shape != (B,):
        raise ValueError("shape mismatch")
    n_acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, G1), -1, dtype=np.int32)
    flagged = np.zeros(B, dtype=bool)
    for b in range(B):
        n = gamma
        r = None
        for i in range(gamma):
            p = softmax64(t[b, i])
            q = softmax64(q_log[b, i])
            x = int(d[b, i])
            if q[x] > 0:
                ratio = p[x] / q[x]
                if abs(ua[b, i] - ratio) <= NEAR_TIE_ACCEPT_REL * ratio:
                    flagged[b] = True
                accept = ua[b, i] <= ratio
            else:
                accept = p[x] > 0
            if not accept:
                n = i
                r = np.maximum(0.0, p - q)
                if r.sum() == 0:
                    r = p
                break
        if r is None:
            r = softmax64(t[b, gamma])
        j, near = _inverse_cdf(r, us[b])
        flagged[b] |= near
        out[b, :n] = d[b, :n]
        out[b, n] = j
        n_acc[b] = n
    return n_acc, out, flagged
