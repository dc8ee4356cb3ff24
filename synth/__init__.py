"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only *makes inputs*: random draws, the float32 -> bf16 storage
conversion of generated activations, and the construction of logits and
draft tokens with a known structure.  It holds none of the quantization,
GEMM or acceptance arithmetic; neither the oracle nor the GPU path imports
the other through it.

Recipe (fixed draw order per case: weights, activations, outlier channels,
logits, uniforms):

* generator: ``numpy.random.default_rng(1000 * case + trial)``;
* weights: fp32 N(0, 0.02) (0.02 is the standard deviation);
* activations: fp32 N(0, 1); a set of outlier channels (columns) chosen
  without replacement is multiplied by 20; then stored as bf16 (round to
  nearest even);
* verify logits: target = 3 z1, draft = 3 (rho z1 + sqrt(1 - rho^2) z2),
  z1, z2 standard normal, fp32;
* draft tokens: Gumbel-max draws from softmax(draft logits), or planted
  tokens with a forced target argmax for greedy cases;
* uniforms: fp32 in [0, 1).

Decoder model for the end-to-end self-speculative loop (sizes only, plus the
seeded draws): ``ModelConfig`` lists the shapes and the two model constants
(RMSNorm epsilon, RoPE base); ``model_weights`` draws, in this order, the
embedding (N(0, 0.02), stored as bf16), then per layer the fused QKV, O,
fused gate|up (gate rows first) and down matrices, then the lm_head, all fp32
N(0, 0.02); ``prompts`` draws uniform token ids.
"""

from dataclasses import dataclass

import numpy as np

__all__ = [
    "make_rng", "outlier_count", "to_bf16_bits", "from_bf16_bits", "weights",
    "activations", "verify_logits", "plant_greedy", "gumbel_drafts",
    "uniforms", "ModelConfig", "TINY_MODEL", "E2E_MODEL", "model_weights", "prompts",
]


def make_rng(case, trial=0):
    return np.random.default_rng(1000 * int(case) + int(trial))


def outlier_count(K, frac=0.001):
    """0.1 % of the channels, at least one."""
    return max(1, int(round(frac * K)))


def to_bf16_bits(x):
    """float32 -> bf16 storage bits, round to nearest even (finite input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def from_bf16_bits(b):
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weights(rng, N, K, std=0.02):
    return (rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


def activations(rng, M, K, n_outliers=0, factor=20.0, std=1.0):
    """bf16 bits [M, K]: N(0, std) with ``n_outliers`` channels scaled by ``factor``."""
    x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(std)
    if n_outliers:
        cols = rng.choice(K, size=n_outliers, replace=False)
        x[:, cols] *= np.float32(factor)
    return to_bf16_bits(x)


def verify_logits(rng, B, gamma, V, rho=0.9, sigma=3.0):
    """(target [B, gamma+1, V], draft [B, gamma, V]) fp32, correlated rho."""
    z1 = rng.standard_normal((B, gamma + 1, V), dtype=np.float32)
    z2 = rng.standard_normal((B, gamma, V), dtype=np.float32)
    tgt = (np.float32(sigma) * z1).astype(np.float32)
    c = np.float32(np.sqrt(1.0 - rho * rho))
    drf = (np.float32(sigma) * (np.float32(rho) * z1[:, :gamma] + c * z2)).astype(np.float32)
    return tgt, drf


def plant_greedy(rng, target, n_star):
    """Plant a known target argmax in every row and drafts that match it for
    the first ``n_star[b]`` positions then differ (n_star[b] == gamma: all
    match).  Modifies ``target`` in place; returns int32 drafts [B, gamma]."""
    B, G1, V = target.shape
    gamma = G1 - 1
    top = rng.integers(0, V, size=(B, G1))
    for b in range(B):
        for i in range(G1):
            row = target[b, i]
            row[top[b, i]] = row.max() + np.float32(1.0)
    d = top[:, :gamma].copy()
    for b in range(B):
        n = int(n_star[b])
        if n < gamma:
            d[b, n] = (top[b, n] + 1 + rng.integers(0, V - 1)) % V
    return d.astype(np.int32)


def gumbel_drafts(rng, draft_logits):
    """One draw per row from softmax(draft_logits) by the Gumbel-max trick."""
    u = rng.random(draft_logits.shape)
    g = -np.log(-np.log(np.clip(u, 1e-300, 1.0 - 1e-16)))
    return np.argmax(draft_logits.astype(np.float64) + g, axis=-1).astype(np.int32)


def uniforms(rng, shape):
    return rng.random(shape, dtype=np.float32)


@dataclass(frozen=True)
class ModelConfig:
    vocab: int
    d: int
    n_layers: int
    n_heads: int
    n_kv: int
    head_dim: int
    ffn: int
    eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv * self.head_dim

    @property
    def qkv_rows(self):
        return self.q_dim + 2 * self.kv_dim


# the end-to-end workload: 8 layers, d 2048, 16 query / 4 key-value heads of
# 128, SwiGLU hidden 5632, vocabulary 32000
E2E_MODEL = ModelConfig(vocab=32000, d=2048, n_layers=8, n_heads=16, n_kv=4, head_dim=128,
                        ffn=5632)
# the same layer shapes (16 query / 4 key-value heads, d 2048, SwiGLU 5632,
# vocabulary 32000) with two layers, small enough for the CPU oracle
E2E_MODEL_2L = ModelConfig(vocab=32000, d=2048, n_layers=2, n_heads=16, n_kv=4, head_dim=128,
                           ffn=5632)
# a two-layer model of the same structure for CPU-sized tests
TINY_MODEL = ModelConfig(vocab=512, d=256, n_layers=2, n_heads=2, n_kv=1, head_dim=128, ffn=768)


def model_weights(rng, cfg, std=0.02):
    """dict(emb = bf16 bits [V, d], layers = [dict(qkv, o, gu, down) fp32],
    lm = fp32 [V, d]); every matrix is [out features, in features]."""
    emb = to_bf16_bits(weights(rng, cfg.vocab, cfg.d, std))
    layers = []
    for _ in range(cfg.n_layers):
        layers.append(dict(qkv=weights(rng, cfg.qkv_rows, cfg.d, std),
                           o=weights(rng, cfg.d, cfg.q_dim, std),
                           gu=weights(rng, 2 * cfg.ffn, cfg.d, std),
                           down=weights(rng, cfg.d, cfg.ffn, std)))
    lm = weights(rng, cfg.vocab, cfg.d, std)
    return dict(emb=emb, layers=layers, lm=lm)


def prompts(rng, B, P, vocab):
    return rng.integers(0, vocab, size=(B, P)).astype(np.int32)
