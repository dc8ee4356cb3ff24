"""GPU parity of the decoder kernels and of the end-to-end greedy
self-speculative loop against the oracle decoder."""

import numpy as np
import pytest
import torch

import oracle
import oracle.model as om
import synth
import quantization_self_speculation_amd as q
from quantization_self_speculation_amd import binding as qb
from quantization_self_speculation_amd.e2e import Decoder
from gpu_util import dev, dev_bf16, host, host_bits16, say

pytestmark = pytest.mark.gpu

BF16_ULP = 2.0 ** -7   # relative spacing of bf16 values


def _bf16_close(got_bits, want_bits, frac_exact=0.99):
    """bf16 outputs: at most one unit in the last place apart, and almost all
    identical (both sides round a value computed in a different order)."""
    g = om.bf16_values(got_bits)
    w = om.bf16_values(want_bits)
    tol = np.abs(w) * BF16_ULP * 1.0001 + 1e-38
    assert np.all(np.abs(g - w) <= tol), np.abs(g - w).max()
    assert np.mean(got_bits == want_bits) >= frac_exact, np.mean(got_bits == want_bits)


# ------------------------------------------------------------------ kernels
def test_embed_and_add_rmsnorm():
    rng = synth.make_rng(50)
    V, d, M = 300, 256, 9
    emb = synth.to_bf16_bits(rng.standard_normal((V, d), dtype=np.float32))
    tok = rng.integers(0, V, M).astype(np.int32)
    x = torch.empty((M, d), dtype=torch.float32, device="cuda:0")
    qb.embed(dev_bf16(emb), dev(tok), x)
    want = om.bf16_values(emb)[tok]
    assert np.array_equal(host(x), want.astype(np.float32))
    add = rng.standard_normal((M, d)).astype(np.float32)
    y = torch.empty((M, d), dtype=torch.bfloat16, device="cuda:0")
    qb.add_rmsnorm(x, dev(add), y, 1e-6)
    xs = (want.astype(np.float32) + add).astype(np.float32)
    assert np.array_equal(host(x), xs)                      # the fp32 residual, exactly
    _bf16_close(host_bits16(y), om.to_bf16_bits(om.rmsnorm(xs, 1e-6)), frac_exact=0.999)
    # strided rows (every third row), no add
    y2 = torch.empty((3, d), dtype=torch.bfloat16, device="cuda:0")
    qb.add_rmsnorm(x[2::3], None, y2, 1e-6)
    _bf16_close(host_bits16(y2), om.to_bf16_bits(om.rmsnorm(xs[2::3], 1e-6)), frac_exact=0.999)


def test_rope_kv_and_attention():
    rng = synth.make_rng(51)
    H, Hkv, hd, B, cap = 4, 2, 128, 3, 40
    M = 7
    seq = np.array([0, 1, 2, 0, 1, 2, 2], np.int32)
    pos = np.array([0, 5, 39, 17, 6, 12, 38], np.int32)
    qkv = rng.standard_normal((M, (H + 2 * Hkv) * hd)).astype(np.float32)
    kc = torch.zeros((B, Hkv, cap, hd), dtype=torch.bfloat16, device="cuda:0")
    vc = torch.zeros_like(kc)
    # pre-fill the cache with known bf16 values (the positions not written here)
    k0 = synth.to_bf16_bits(rng.standard_normal((B, Hkv, cap, hd), dtype=np.float32))
    v0 = synth.to_bf16_bits(rng.standard_normal((B, Hkv, cap, hd), dtype=np.float32))
    kc.copy_(dev_bf16(k0))
    vc.copy_(dev_bf16(v0))
    qo = torch.empty((M, H * hd), dtype=torch.float32, device="cuda:0")
    qb.rope_kv(dev(qkv), dev(seq), dev(pos), qo, kc, vc, H, Hkv, 10000.0)
    qq = qkv[:, :H * hd].reshape(M, H, hd).astype(np.float64)
    kk = qkv[:, H * hd:(H + Hkv) * hd].reshape(M, Hkv, hd).astype(np.float64)
    vv = qkv[:, (H + Hkv) * hd:].reshape(M, Hkv, hd)
    q_want = om.rope(qq, pos[:, None], 10000.0).astype(np.float32)
    np.testing.assert_allclose(host(qo).reshape(M, H, hd), q_want, rtol=2e-6, atol=1e-6)
    k_want = k0.copy()
    v_want = v0.copy()
    for m in range(M):
        k_want[seq[m], :, pos[m]] = om.to_bf16_bits(om.rope(kk[m], np.full(Hkv, pos[m]), 10000.0))
        v_want[seq[m], :, pos[m]] = synth.to_bf16_bits(vv[m])
    assert np.array_equal(host_bits16(vc), v_want)
    _bf16_close(host_bits16(kc), k_want, frac_exact=0.999)
    # attention over the cache as it now stands
    out = torch.empty((M, H * hd), dtype=torch.bfloat16, device="cuda:0")
    qb.attention(qo, kc, vc, dev(seq), dev(pos), out, H, Hkv)
    K = om.bf16_values(host_bits16(kc))
    Vv = om.bf16_values(host_bits16(vc))
    Q = host(qo).reshape(M, H, hd).astype(np.float64)
    want = np.empty((M, H, hd))
    for m in range(M):
        for h in range(H):
            g = h // (H // Hkv)
            T = pos[m] + 1
            want[m, h] = om.attend(Q[m, h], K[seq[m], g, :T], Vv[seq[m], g, :T])
    got = om.bf16_values(host_bits16(out)).reshape(M, H, hd)
    err = np.abs(got - want)
    assert np.all(err <= np.abs(want) * 2 * BF16_ULP + 1e-5), err.max()


def test_silu_mul_and_argmax():
    rng = synth.make_rng(52)
    M, F = 5, 700
    gu = (rng.standard_normal((M, 2 * F)) * 3).astype(np.float32)
    a = torch.empty((M, F), dtype=torch.bfloat16, device="cuda:0")
    qb.silu_mul(dev(gu), a)
    want = om.to_bf16_bits(om.silu(gu[:, :F].astype(np.float64)) * gu[:, F:])
    _bf16_close(host_bits16(a), want, frac_exact=0.998)
    V = 1000
    x = rng.standard_normal((6, V)).astype(np.float32)
    x[1, 10] = x[1, 900] = x[1].max() + 1.0          # tie: the lower index wins
    x[2, :] = 0.0                                     # all equal: index 0
    x[3, V - 1] = 50.0
    x[4, :] = -np.inf                                 # all -inf: index 0
    x[5, :] = -np.inf
    x[5, 777] = -1e30                                 # one finite value among -inf
    out = torch.full((12,), -7, dtype=torch.int32, device="cuda:0")
    qb.argmax(dev(x), out, out_stride=2)
    got = host(out)
    assert np.array_equal(got[0::2], om.argmax_first(x))
    assert np.all(got[1::2] == -7)
    assert got[2] == 10 and got[4] == 0 and got[6] == V - 1 and got[8] == 0 and got[10] == 777


@pytest.mark.parametrize("M,d", [(9, 256), (37, 2048), (3, 4096)])
def test_quantizer_fused_into_rmsnorm(M, d):
    """add_rmsnorm_quant: the bf16 output and the residual are bitwise those
    of add_rmsnorm, and the 4-bit codes and scales bitwise those of quant_act
    on the bf16 rows -- and of the oracle's quantizer on them (with and
    without the residual add, row-strided x)."""
    say(f"fused quantizer M={M} d={d}")
    rng = synth.make_rng(56)
    big = torch.from_numpy(rng.standard_normal((M, d + 128)).astype(np.float32)).to("cuda:0")
    add = torch.from_numpy(rng.standard_normal((M, d)).astype(np.float32)).to("cuda:0")
    for a_ in (None, add):
        x1 = big.clone()[:, :d]
        x2 = big.clone()[:, :d]
        y1 = torch.empty((M, d), dtype=torch.bfloat16, device="cuda:0")
        y2 = torch.empty_like(y1)
        yq = torch.empty((M, d // 2), dtype=torch.uint8, device="cuda:0")
        ys = torch.empty((M,), dtype=torch.float32, device="cuda:0")
        qb.add_rmsnorm(x1, a_, y1, 1e-6)
        qb.add_rmsnorm_quant(x2, a_, y2, yq, ys, 1e-6)
        q1, s1 = q.quant_act(y1)
        assert np.array_equal(host_bits16(y1), host_bits16(y2))
        assert np.array_equal(host(x1).view(np.uint32), host(x2).view(np.uint32))
        assert np.array_equal(host(yq), host(q1))
        assert np.array_equal(host(ys).view(np.uint32), host(s1).view(np.uint32))
        qo, so = oracle.quant_act(host_bits16(y2))
        assert np.array_equal(host(yq), qo) and np.array_equal(host(ys), so)


def test_spec_prepare_and_commit():
    B, g = 3, 2
    length = np.array([10, 4, 7], np.int32)
    vtok = np.array([[5, 6, 7], [8, 9, 1], [2, 3, 4]], np.int32)
    seq = torch.zeros(9, dtype=torch.int32, device="cuda:0")
    pos, tok = torch.zeros_like(seq), torch.zeros_like(seq)
    drafts = torch.zeros(B * g, dtype=torch.int32, device="cuda:0")
    L, Vt = dev(length), dev(vtok.reshape(-1))
    qb.spec_prepare(0, B, g, 1, L, Vt, None, seq, pos, tok)
    assert np.array_equal(host(seq)[:3], [0, 1, 2])
    assert np.array_equal(host(pos)[:3], length)                 # len - 1 + 1
    assert np.array_equal(host(tok)[:3], vtok[:, 1])
    qb.spec_prepare(1, B, g, 0, L, Vt, drafts, seq, pos, tok)
    assert np.array_equal(host(seq), np.repeat([0, 1, 2], 3))
    assert np.array_equal(host(pos), (length[:, None] - 1 + np.arange(3)).reshape(-1))
    assert np.array_equal(host(tok), vtok.reshape(-1))
    assert np.array_equal(host(drafts).reshape(B, g), vtok[:, 1:])
    # commit: sequence 1 is already finished (n_gen == max_gen)
    n_acc = dev(np.array([2, 1, 0], np.int32))
    out_tok = dev(np.array([[11, 12, 13], [21, 22, -1], [31, -1, -1]], np.int32).reshape(-1))
    gen = torch.zeros((B, 8), dtype=torch.int32, device="cuda:0")
    n_gen = dev(np.array([1, 5, 3], np.int32))
    stats = torch.tensor([4, 4, 9], dtype=torch.int64, device="cuda:0")
    qb.spec_commit(B, g, n_acc, out_tok, L, Vt, g + 1, gen, n_gen, 5, stats)
    G = host(gen)
    assert np.array_equal(G[0, 1:4], [11, 12, 13]) and np.all(G[1] == 0)
    assert G[2, 3] == 31
    assert np.array_equal(host(n_gen), [4, 5, 4])
    assert np.array_equal(host(L), [13, 4, 8])
    assert np.array_equal(host(Vt).reshape(B, 3)[:, 0], [13, 8, 31])
    assert np.array_equal(host(stats), [4 + 2, 4 + 2, 2])


# ------------------------------------------------------------------ end to end
def _tiny_case(seed, B, P):
    rng = synth.make_rng(41, seed)
    cfg = synth.TINY_MODEL
    w = synth.model_weights(rng, cfg)
    return cfg, w, synth.prompts(rng, B, P, cfg.vocab)


def _first_divergence(a, b):
    d = np.nonzero(a != b)[0]
    return int(d[0]) if d.size else None


@pytest.mark.parametrize("seed,gamma", [(0, 4), (1, 2)])
def test_e2e_tiny_selfspec_equals_pure_and_oracle(seed, gamma):
    B, P, n_gen = 4, 16, 32
    cfg, w, prompts = _tiny_case(seed, B, P)
    say(f"tiny e2e seed={seed} gamma={gamma}")
    dec = Decoder(cfg, w, B, P, n_gen, gamma)
    pure = dec.run(prompts, speculative=False)
    spec = dec.run(prompts, speculative=True)
    assert np.array_equal(spec["tokens"], pure["tokens"])
    assert 0 <= spec["accepted"] <= gamma * spec["active_rows"]
    # eager (no graph) gives the same tokens
    spec2 = dec.run(prompts, speculative=True, use_graph=False)
    assert np.array_equal(spec2["tokens"], spec["tokens"])
    assert spec2["accepted"] == spec["accepted"]
    # against the oracle: identical up to the first divergence, which may only
    # happen where the oracle's top-2 logits are closer than twice the logit
    # error the fp tolerance allows (2 * 2e-3 of the row's largest |logit|)
    model = om.Model(cfg, w)
    want, _, margins = om.greedy_decode(model, prompts, n_gen, gamma, with_margins=True)
    for bi in range(B):
        k = _first_divergence(pure["tokens"][bi], want[bi])
        if k is not None:
            say(f"  seq {bi}: diverges at {k}, oracle relative margin {margins[bi, k]:.3e}")
            assert margins[bi, k] <= 4e-3, (bi, k, margins[bi, k])
    matched = sum((_first_divergence(pure["tokens"][i], want[i]) or n_gen) for i in range(B))
    assert matched >= B * n_gen // 2


def test_e2e_forwards_against_oracle():
    """After a shared prefill, every linear layer of a W4A16 and of a W4A4
    forward matches the oracle layer applied to the GPU's own bf16 input,
    within the fp tolerance (op-by-op parity).  The whole W4A16 forward's
    logits are also compared with the oracle forward: there the two sides
    differ at the bf16 rounding points, where a value computed in a different
    order can round one bf16 unit (2**-8 relative) the other way, so that
    comparison allows 1e-2 of max|logit|.  The W4A4 forward is checked op by op
    only:
    each linear layer's output against the oracle layer applied to the GPU's
    own bf16 input (the quantizer rounds, so a one-ulp difference upstream may
    move a code, and whole-forward W4A4 values are not comparable)."""
    B, P = 2, 8
    cfg, w, prompts = _tiny_case(7, B, P)
    dec = Decoder(cfg, w, B, P, 4, 2)
    dec.reset()
    dec.prefill(prompts)
    model = om.Model(cfg, w)
    kv = om.KVCache(cfg, B, dec.cap)
    first = om.prefill(model, kv, prompts)
    assert np.array_equal(host(dec.first), first)
    toks = np.array([3, 77], np.int32)
    packed = {(li, k): model.layers[li][k] for li in range(cfg.n_layers)
              for k in ("qkv", "o", "gu", "down")}
    packed.update({(cfg.n_layers, "lm"): model.lm})
    for mode in (om.VERIFY, om.DRAFT):
        dec.seq[:B].copy_(torch.arange(B, dtype=torch.int32))
        dec.pos[:B].fill_(P)
        dec.tok[:B].copy_(torch.from_numpy(toks))
        trace = []
        got = host(dec.forward(mode, B, q.GEMM_SKINNY, trace=trace)).astype(np.float64)
        assert len(trace) == 4 * cfg.n_layers + 1
        for li, name, X, Y in trace:
            xb = X.cpu().view(torch.int16).numpy().view(np.uint16)
            ref = om.linear(mode, xb, packed[(li, name)])
            yg = Y.cpu().numpy().astype(np.float64)
            e = np.abs(yg - ref).max() / np.abs(ref).max()
            assert e <= 2e-3, (mode, li, name, e)
        if mode == om.VERIFY:
            kv2 = om.KVCache(cfg, B, dec.cap)
            kv2.k[:], kv2.v[:] = kv.k, kv.v
            want = om.forward(model, kv2, [0, 1], [P, P], toks, mode)
            err = np.abs(got - want).max() / np.abs(want).max()
            say(f"  w4a16 forward logits rel err {err:.2e}")
            assert err <= 1e-2


def test_e2e_model_selfspec_equals_pure():
    """The 8-layer d=2048 decoder at batch 16, 128-token prompts: greedy
    self-speculation (W4A4 draft, gamma 4) emits the pure W4A16 tokens."""
    cfg = synth.E2E_MODEL
    rng = synth.make_rng(4, 0)
    w = synth.model_weights(rng, cfg)
    prompts = synth.prompts(rng, 16, 128, cfg.vocab)
    say("e2e model: packing")
    dec = Decoder(cfg, w, 16, 128, 64, 4)
    del w
    pure = dec.run(prompts, speculative=False)
    spec = dec.run(prompts, speculative=True)
    say(f"  rounds {spec['rounds']} accepted {spec['accepted']} of {4 * spec['active_rows']}")
    assert np.array_equal(spec["tokens"], pure["tokens"])
