"""Pins of the oracle's acceptance step.

Hand-worked fixtures (tests/golden/verify_hand.json), planted greedy drafts
for every acceptance length, and statistical tests of the speculative
sampling theorem: the first emitted token is distributed as the target's
p_0, the acceptance probability of a draft drawn from q is sum_v min(p, q),
and after a rejection the emitted token follows norm(max(0, p - q)).
"""

import numpy as np
import pytest
from scipy import stats

import oracle
import oracle.verify as ov
import synth


def test_greedy_hand(golden):
    g = golden("verify_hand.json")
    for c in g["greedy"]:
        n, out = oracle.verify_greedy(np.array(c["target"], np.float32), np.array(c["draft"], np.int32))
        assert n.tolist() == c["n_accept"], c["derivation"]
        assert out.tolist() == c["out"], c["derivation"]


def test_sample_hand(golden):
    g = golden("verify_hand.json")
    for c in g["sample"]:
        n, out, fl = oracle.verify_sample(
            np.array(c["target"], np.float32), np.array(c["draft_logits"], np.float32),
            np.array(c["draft"], np.int32), np.array(c["u_accept"], np.float32),
            np.array(c["u_sample"], np.float32))
        if "flagged" in c:
            assert fl.tolist() == c["flagged"], c["derivation"]
            continue
        assert not fl.any(), c["derivation"]
        assert n.tolist() == c["n_accept"], c["derivation"]
        assert out.tolist() == c["out"], c["derivation"]


def test_inverse_cdf_hand(golden):
    g = golden("verify_hand.json")
    for c in g["inverse_cdf"]:
        j, _ = ov._inverse_cdf(np.array(c["r"], np.float64), c["u"])
        assert j == c["j"], c["derivation"]


@pytest.mark.parametrize("gamma", [1, 4, 8])
def test_greedy_planted_every_length(gamma):
    rng = synth.make_rng(80 + gamma)
    B, V = 3 * (gamma + 1), 1000
    tgt, _ = synth.verify_logits(rng, B, gamma, V)
    n_star = np.arange(B) % (gamma + 1)
    d = synth.plant_greedy(rng, tgt, n_star)
    n, out = oracle.verify_greedy(tgt, d)
    assert np.array_equal(n, n_star)
    for b in range(B):
        k = n_star[b]
        assert out[b, :k].tolist() == d[b, :k].tolist()
        assert out[b, k] == int(np.argmax(tgt[b, k]))
        assert out[b, k] != (d[b, k] if k < gamma else -2)
        assert np.all(out[b, k + 1:] == -1)


def test_greedy_tie_goes_to_lowest_index():
    t = np.zeros((1, 2, 6), np.float32)
    t[0, 0, [2, 4]] = 5.0
    t[0, 1, [1, 3, 5]] = 2.0
    n, out = oracle.verify_greedy(t, np.array([[2]], np.int32))
    assert n[0] == 1 and out[0].tolist() == [2, 1]
    n, out = oracle.verify_greedy(t, np.array([[4]], np.int32))
    assert n[0] == 0 and out[0].tolist() == [2, -1]


def _fixed_pq(V=8, seed=3):
    rng = np.random.default_rng(seed)
    lt = (rng.standard_normal(V) * 1.5).astype(np.float32)
    ld = (0.6 * lt + rng.standard_normal(V).astype(np.float32)).astype(np.float32)
    p = np.exp(lt.astype(np.float64) - lt.max()); p /= p.sum()
    q = np.exp(ld.astype(np.float64) - ld.max()); q /= q.sum()
    return lt, ld, p, q


def test_speculative_sampling_theorem_chi2():
    """First emitted token ~ p_0 whatever the draft distribution."""
    V, T = 8, 60000
    lt, ld, p, q = _fixed_pq(V)
    rng = synth.make_rng(81)
    tgt = np.broadcast_to(lt, (T, 2, V)).astype(np.float32)
    drf = np.broadcast_to(ld, (T, 1, V)).astype(np.float32)
    d = rng.choice(V, size=(T, 1), p=q).astype(np.int32)
    ua = synth.uniforms(rng, (T, 1))
    us = synth.uniforms(rng, (T,))
    n, out, _ = oracle.verify_sample(tgt, drf, d, ua, us)
    first = out[:, 0]
    counts = np.bincount(first, minlength=V)
    chi = stats.chisquare(counts, p * T)
    assert chi.pvalue > 1e-4, (counts, p * T)
    # acceptance probability of a draft drawn from q is sum_v min(p_v, q_v)
    acc = (n == 1).mean()
    pa = np.minimum(p, q).sum()
    assert abs(acc - pa) < 5 * np.sqrt(pa * (1 - pa) / T)


def test_residual_distribution_after_reject_chi2():
    """Conditioned on a rejection the token follows norm(max(0, p - q))."""
    V, T = 8, 40000
    lt, ld, p, q = _fixed_pq(V, seed=5)
    rng = synth.make_rng(82)
    tgt = np.broadcast_to(lt, (T, 2, V)).astype(np.float32)
    drf = np.broadcast_to(ld, (T, 1, V)).astype(np.float32)
    # pick drafts where p < q so rejection is possible, force u close to 1
    cand = np.nonzero(p < q)[0]
    d = rng.choice(cand, size=(T, 1)).astype(np.int32)
    ua = np.full((T, 1), np.float32(0.999999), np.float32)
    us = synth.uniforms(rng, (T,))
    n, out, _ = oracle.verify_sample(tgt, drf, d, ua, us)
    assert np.all(n == 0)
    r = np.maximum(0.0, p - q)
    r /= r.sum()
    counts = np.bincount(out[:, 0], minlength=V)
    assert np.all(counts[r == 0] == 0)
    keep = r > 0
    chi = stats.chisquare(counts[keep], r[keep] * T)
    assert chi.pvalue > 1e-4


def test_bonus_token_when_all_accepted():
    V = 16
    rng = synth.make_rng(83)
    tgt, drf = synth.verify_logits(rng, 4, 3, V)
    d = synth.gumbel_drafts(rng, drf)
    ua = np.zeros((4, 3), np.float32)        # u = 0 <= any ratio: accept all
    us = np.array([0.0, 0.25, 0.5, 0.999], np.float32)
    n, out, _ = oracle.verify_sample(tgt, drf, d, ua, us)
    assert np.all(n == 3)
    for b in range(4):
        p = oracle.softmax64(tgt[b, 3])
        C = np.cumsum(p)
        assert out[b, 3] == int(np.searchsorted(C, us[b] * C[-1], side="right"))
        assert out[b, :3].tolist() == d[b].tolist()


def test_sample_shapes_rejected():
    t = np.zeros((1, 3, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.verify_sample(t, np.zeros((1, 1, 4), np.float32), np.zeros((1, 2), np.int32),
                             np.zeros((1, 2), np.float32), np.zeros(1, np.float32))
    with pytest.raises(ValueError):
        oracle.verify_greedy(t, np.array([[0, 4]], np.int32))
