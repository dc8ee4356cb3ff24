"""qspec_verify_noalloc (the verify step on the library's fixed per-device
scratch, for callers that cannot allocate) against qspec_verify with a
workspace: bitwise the same n_accept and out_tok in both modes, on two calls
in a row, the second with a smaller input (the scratch keeps the first call's
contents); sizes past the fixed scratch are rejected on the host."""

import ctypes

import numpy as np
import pytest
import torch

import synth
import quantization_self_speculation_amd as q
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def _inputs(seed, B, gamma, V):
    rng = synth.make_rng(300, seed)
    tgt, drf = synth.verify_logits(rng, B, gamma, V)
    d = synth.gumbel_drafts(rng, drf)
    ua = synth.uniforms(rng, (B, gamma))
    us = synth.uniforms(rng, (B,))
    return [dev(a) for a in (tgt, d, drf, ua, us)]


def _both(mode, tgt, d, drf, ua, us):
    if mode == q.VERIFY_GREEDY:
        a = q.verify(mode, tgt, d)
        n = torch.full_like(a[0], -9)
        o = torch.full_like(a[1], -9)
        b = q.verify_noalloc(mode, tgt, d, n_accept=n, out_tok=o)
    else:
        a = q.verify(mode, tgt, d, drf, ua, us)
        n = torch.full_like(a[0], -9)
        o = torch.full_like(a[1], -9)
        b = q.verify_noalloc(mode, tgt, d, drf, ua, us, n_accept=n, out_tok=o)
    return [host(t) for t in a], [host(t) for t in b]


@pytest.mark.parametrize("mode", [q.VERIFY_GREEDY, q.VERIFY_SAMPLE])
def test_noalloc_matches_workspace_call_twice(mode):
    for seed, (B, gamma, V) in enumerate([(32, 8, 128256), (5, 3, 50257)]):
        say(f"verify_noalloc mode={mode} B={B} gamma={gamma} V={V}")
        (n1, o1), (n2, o2) = _both(mode, *_inputs(seed, B, gamma, V))
        assert np.array_equal(n1, n2), (B, gamma, V)
        assert np.array_equal(o1, o2), (B, gamma, V)


def test_noalloc_rejects_sizes_past_the_scratch():
    # B = 3000, gamma = 8, V = 2^23 needs far more scratch than the fixed
    # array holds: rejected on the host before anything is launched (the
    # pointers are never dereferenced); the workspace call still takes them
    L = q.lib()
    A = ctypes.c_void_p(0x10000)
    need = q.workspace_bytes(3, 3000, 8, 1 << 23)
    assert need > (8 << 20)
    assert L.qspec_verify_noalloc(0, 3000, 8, 1 << 23, A, None, A, None, None, A, A, None) == -5
    assert b"scratch" in L.qspec_last_error()
    assert q.workspace_bytes(3, 256, 8, 152064) <= (8 << 20)
