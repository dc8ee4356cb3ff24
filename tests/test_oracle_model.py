"""Pins of the oracle decoder and its greedy self-speculative loop."""

import numpy as np
import pytest

import oracle.model as om
import synth
from oracle import f32_to_bf16_bits


# ------------------------------------------------------------ rounding
def test_direct_bf16_rounding_hand_cases():
    one = 1.0
    cases = [
        (one + 2.0 ** -8, one),                        # tie -> even (mantissa 0)
        (one + 3 * 2.0 ** -8, one + 2.0 ** -6),        # tie -> even (round up)
        (one + 2.0 ** -8 + 2.0 ** -40, one + 2.0 ** -7),  # just above the tie: up
        (-(one + 2.0 ** -8 + 2.0 ** -40), -(one + 2.0 ** -7)),
        (2.0 ** -130 * 1.5, 2.0 ** -130 * 1.5),        # subnormal grid point
        (2.0 ** -134, 0.0),                             # half of the smallest step: tie -> 0
    ]
    for x, want in cases:
        got = om.bf16_values(om.to_bf16_bits(np.array([x])))[0]
        assert got == want, (x, got, want)
    # the fp32 route would double-round the third case down to 1.0
    via32 = om.bf16_values(f32_to_bf16_bits(np.array([one + 2.0 ** -8 + 2.0 ** -40], np.float32)))
    assert via32[0] == one


def test_direct_bf16_rounding_matches_fp32_route_on_fp32_values():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    assert np.array_equal(om.to_bf16_bits(x.astype(np.float64)), f32_to_bf16_bits(x))


# ------------------------------------------------------------ RoPE
def test_rope_identities():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 128))
    k = rng.standard_normal((3, 128))
    # position 0 is the identity
    assert np.array_equal(om.rope(q, np.zeros(3), 1e4), q)
    # a rotation of each (i, i + 64) pair keeps the pair's norm
    r = om.rope(q, np.array([1, 17, 389]), 1e4)
    n0 = q[:, :64] ** 2 + q[:, 64:] ** 2
    n1 = r[:, :64] ** 2 + r[:, 64:] ** 2
    assert np.allclose(n0, n1, rtol=1e-13, atol=0)
    # the score depends on the position difference only
    d1 = np.sum(om.rope(q, np.array([5] * 3), 1e4) * om.rope(k, np.array([2] * 3), 1e4), axis=1)
    d2 = np.sum(om.rope(q, np.array([13] * 3), 1e4) * om.rope(k, np.array([10] * 3), 1e4), axis=1)
    assert np.allclose(d1, d2, rtol=1e-12, atol=1e-12)
    # pair 0 turns by exactly `pos` radians (inv_freq_0 = 1), the last pair by
    # pos * base**(-126/128)
    e = np.zeros(128)
    e[0] = 1.0
    r = om.rope(e, np.array(3.0), 1e4)
    assert np.isclose(r[0], np.cos(3.0), rtol=1e-15) and np.isclose(r[64], np.sin(3.0), rtol=1e-15)
    e = np.zeros(128)
    e[63] = 1.0
    r = om.rope(e, np.array(3.0), 1e4)
    a = 3.0 * 1e4 ** (-126 / 128)
    assert np.isclose(r[63], np.cos(a), rtol=1e-15) and np.isclose(r[127], np.sin(a), rtol=1e-15)


# ------------------------------------------------------------ attention / norm / silu
def test_attention_closed_forms():
    rng = np.random.default_rng(2)
    keys = rng.standard_normal((7, 128))
    vals = rng.standard_normal((7, 128))
    q = rng.standard_normal(128)
    # one key: the output is that key's value
    assert np.array_equal(om.attend(q, keys[:1], vals[:1]), vals[0])
    # a zero query weights every value equally
    assert np.allclose(om.attend(np.zeros(128), keys, vals), vals.mean(axis=0), rtol=1e-14, atol=1e-15)
    # a dominant key takes (almost) all the weight
    k2 = keys.copy()
    k2[4] = q * 50.0
    assert np.allclose(om.attend(q, k2, vals), vals[4], atol=1e-12)


def test_rmsnorm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 256))
    y = om.rmsnorm(x, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    assert np.allclose(om.rmsnorm(x * 1024.0, 0.0), y, rtol=1e-14)
    # epsilon matters only for tiny rows
    assert np.allclose(om.rmsnorm(x, 1e-6), y, rtol=1e-5)


def test_silu_points():
    assert om.silu(np.array([0.0]))[0] == 0.0
    assert np.isclose(om.silu(np.array([1.0]))[0], 0.7310585786300049, rtol=1e-15)
    assert np.isclose(om.silu(np.array([-1.0]))[0], -0.2689414213699951, rtol=1e-15)
    assert np.isclose(om.silu(np.array([40.0]))[0], 40.0, rtol=1e-15)


# ------------------------------------------------------------ the loop
def _tiny(seed, B=3, P=12):
    rng = synth.make_rng(40, seed)
    cfg = synth.TINY_MODEL
    model = om.Model(cfg, synth.model_weights(rng, cfg))
    return model, synth.prompts(rng, B, P, cfg.vocab)


@pytest.mark.parametrize("seed,gamma,draft", [(0, 4, om.DRAFT), (1, 1, om.DRAFT), (2, 3, om.DRAFT),
                                              (0, 4, om.DRAFT8), (3, 2, om.DRAFT8)])
def test_selfspec_equals_pure_greedy(seed, gamma, draft):
    """Greedy self-speculation emits exactly the pure W4A16 greedy tokens,
    and the KV rows of every committed position equal pure decoding's, with
    the W4A4 drafter and with the W4A8 tier as the drafter."""
    model, prompts = _tiny(seed)
    n_gen = 20
    want, kv_ref = om.greedy_decode(model, prompts, n_gen, gamma)
    got, kv, st = om.selfspec_greedy(model, prompts, n_gen, gamma, draft_mode=draft)
    assert np.array_equal(got, want)
    assert 0 <= st["accepted"] <= st["drafted"] and st["rounds"] >= (n_gen - 1 + gamma) // (gamma + 1)
    # committed positions: prompt + generated tokens that were fed back
    B, P = prompts.shape
    T = P + n_gen - 1
    assert np.array_equal(kv.k[:, :, :, :T], kv_ref.k[:, :, :, :T])
    assert np.array_equal(kv.v[:, :, :, :T], kv_ref.v[:, :, :, :T])


def test_draft_mode_differs_and_rows_are_independent():
    """The W4A4 draft forward is a different function (lossy activations);
    a row's logits do not depend on the other rows of its pass."""
    model, prompts = _tiny(5, B=2, P=6)
    cfg = model.cfg
    kv = om.KVCache(cfg, 2, 16)
    om.prefill(model, kv, prompts)
    kv2 = om.KVCache(cfg, 2, 16)
    kv2.k[:], kv2.v[:] = kv.k, kv.v
    both = om.forward(model, kv, [0, 1], [6, 6], [3, 9], om.VERIFY)
    one = om.forward(model, kv2, [1], [6], [9], om.VERIFY)
    assert np.array_equal(both[1], one[0])
    kv3 = om.KVCache(cfg, 2, 16)
    kv3.k[:], kv3.v[:] = kv.k, kv.v
    dr = om.forward(model, kv3, [0, 1], [6, 6], [3, 9], om.DRAFT)
    assert not np.array_equal(dr, both)
    # the W4A8 tier lies between: closer to the verify logits than W4A4
    kv4 = om.KVCache(cfg, 2, 16)
    kv4.k[:], kv4.v[:] = kv.k, kv.v
    d8 = om.forward(model, kv4, [0, 1], [6, 6], [3, 9], om.DRAFT8)
    assert not np.array_equal(d8, both)
    assert np.abs(d8 - both).max() < np.abs(dr - both).max()


def test_w4a4_drafts_part_under_one_ulp_perturbation():
    """What the drafter comparison's parting rule rests on: perturbing every
    GEMM output of the oracle's own self-speculation by at most one fp32 ulp
    (the size of a different summation order) leaves the emitted tokens
    alone -- greedy verification keeps them the pure ones -- but can move a
    4-bit activation code somewhere, and the W4A4 drafts then part from the
    unperturbed run at a drafted token whose top-2 draft-logit margin is
    several percent (well above the 2e-3 layer tolerance), so a comparison of
    drafts across implementations cannot demand a tighter margin."""
    cfg = synth.TINY_MODEL
    rng = synth.make_rng(41, 2)
    w = synth.model_weights(rng, cfg)
    prompts = synth.prompts(rng, 4, 16, cfg.vocab)
    model = om.Model(cfg, w)
    ref_tr, pert_tr = [], []
    ref, _, _ = om.selfspec_greedy(model, prompts, 32, 3, trace=ref_tr)
    linear = om.linear
    prng = np.random.default_rng(123)

    def perturbed(mode, xb, packed):
        y = linear(mode, xb, packed)
        ulp = prng.choice([-1.0, 0.0, 1.0], size=y.shape) * 2.0 ** -23
        return (y * (1.0 + ulp)).astype(np.float32)

    om.linear = perturbed
    try:
        pert, _, _ = om.selfspec_greedy(model, prompts, 32, 3, trace=pert_tr)
    finally:
        om.linear = linear
    assert np.array_equal(ref, pert)
    margin = None
    for a, b in zip(ref_tr, pert_tr):
        assert np.array_equal(a["act"], b["act"])
        if not np.array_equal(a["drafts"], b["drafts"]):
            i, j = [int(x[0]) for x in np.nonzero(a["drafts"] != b["drafts"])]
            margin = a["draft_margin"][i, j]
            break
    assert margin is not None, "the drafts did not part"
    assert 1e-2 < margin <= 0.1, margin
