"""Guard canaries around every output of the C ABI.

Each call is made through ctypes with output buffers of exactly the size
include/qspec.h states (Wq [Np][K/2], Ws [Np][K/128] with Np = ceil(N/16)*16;
Y [M][N]; P [M][N][K/128]; Xq, Xs; n_accept, out_tok; the workspace of
qspec_workspace_bytes, zero-filled for a GEMM), each followed by 4 KiB of
poisoned slack.  After the
call the slack must hold the poison, the inputs must be unchanged, and the
outputs must match the oracle -- over ragged M and N in every GEMM family of
every mode, the quantizers, the rotations and both verify modes.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import quantization_self_speculation_amd as q
from gpu_util import assert_close, dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu

SLACK = 4096
POISON = 0xA5
P_ = ctypes.c_void_p


class Guarded:
    """`nbytes` of device memory followed by SLACK poisoned bytes."""

    def __init__(self, nbytes, fill=POISON):
        self.n = int(nbytes)
        self.t = torch.full((self.n + SLACK,), fill, dtype=torch.uint8, device="cuda:0")
        self.t[self.n:].fill_(POISON)

    @property
    def ptr(self):
        return P_(self.t.data_ptr())

    def view(self, dtype, shape):
        return self.t[:self.n].view(dtype).view(*shape)

    def intact(self):
        torch.cuda.synchronize()
        return bool((self.t[self.n:] == POISON).all().item())


def _ok(status, what):
    L = q.lib()
    assert status == 0, f"{what}: {L.qspec_last_error().decode()}"


def _stream():
    return P_(torch.cuda.current_stream().cuda_stream)


def _ws(op, a, b, c):
    # a GEMM workspace holds zeros when first used (the header's contract);
    # a verify workspace may hold anything
    return Guarded(max(q.workspace_bytes(op, a, b, c), 0), fill=0x3C if op == 3 else 0)


def _pack(W):
    """qspec_pack_w4 into exactly-sized guarded buffers; checks the canaries
    and the bytes against the oracle."""
    L = q.lib()
    N, K = W.shape
    Np, G = -(-N // 16) * 16, K // 128
    Wd = dev(W)
    Wq = Guarded(Np * K // 2)
    Ws = Guarded(Np * G * 2)
    _ok(L.qspec_pack_w4(P_(Wd.data_ptr()), N, K, 128, Wq.ptr, Ws.ptr, _stream()), "pack_w4")
    assert Wq.intact() and Ws.intact(), f"pack_w4 N={N} K={K} wrote past its buffers"
    Wq_r, Ws_r = oracle.pack_w4(W)
    assert np.array_equal(host(Wq.view(torch.uint8, (Np, K // 2))), oracle.tile_w4(Wq_r))
    got_s = host(Ws.view(torch.int16, (Np, G))).view(np.uint16)
    assert np.array_equal(got_s, oracle.tile_scales(Ws_r))
    assert torch.equal(Wd, dev(W))
    return Wq, Ws, Wq_r, Ws_r


@pytest.mark.parametrize("N,K", [(100, 384), (1001, 256), (16, 128), (1, 640)])
def test_pack_w4_exact_buffers(N, K):
    say(f"canary pack_w4 N={N} K={K}")
    _pack(synth.weights(synth.make_rng(200), N, K))


@pytest.mark.parametrize("M,K", [(5, 384), (1, 128), (3, 4224)])
def test_quantizers_exact_buffers(M, K):
    say(f"canary quantizers M={M} K={K}")
    L = q.lib()
    X = synth.activations(synth.make_rng(201), M, K, n_outliers=1)
    Xd = dev_bf16(X)
    x_in = Xd.clone()
    # 4-bit codes
    Xq, Xs = Guarded(M * K // 2), Guarded(M * 4)
    _ok(L.qspec_quant_act(P_(Xd.data_ptr()), M, K, Xq.ptr, Xs.ptr, _stream()), "quant_act")
    assert Xq.intact() and Xs.intact()
    Xq_r, Xs_r = oracle.quant_act(X)
    assert np.array_equal(host(Xq.view(torch.uint8, (M, K // 2))), Xq_r)
    assert np.array_equal(host(Xs.view(torch.float32, (M,))), Xs_r)
    # 8-bit codes
    X8, S8 = Guarded(M * K), Guarded(M * 4)
    _ok(L.qspec_quant_act8(P_(Xd.data_ptr()), M, K, X8.ptr, S8.ptr, _stream()), "quant_act8")
    assert X8.intact() and S8.intact()
    q8, s8 = oracle.quant_act8(X)
    assert np.array_equal(host(X8.view(torch.int8, (M, K))), q8)
    # rotated quantizer and rotations
    Rq, Rs = Guarded(M * K // 2), Guarded(M * 4)
    _ok(L.qspec_quant_act_rot(P_(Xd.data_ptr()), M, K, Rq.ptr, Rs.ptr, _stream()), "quant_act_rot")
    assert Rq.intact() and Rs.intact()
    rq, rs = oracle.quant_act_rot(X)
    assert np.array_equal(host(Rq.view(torch.uint8, (M, K // 2))), rq)
    Xr = Guarded(M * K * 2)
    _ok(L.qspec_rotate_x(P_(Xd.data_ptr()), M, K, Xr.ptr, _stream()), "rotate_x")
    assert Xr.intact()
    assert np.array_equal(host(Xr.view(torch.int16, (M, K))).view(np.uint16),
                          oracle.rotate_x_bf16(X))
    W = synth.weights(synth.make_rng(202), 3, K)
    Wd = dev(W)
    Wr = Guarded(3 * K * 4)
    _ok(L.qspec_rotate_w(P_(Wd.data_ptr()), 3, K, Wr.ptr, _stream()), "rotate_w")
    assert Wr.intact()
    assert np.array_equal(host(Wr.view(torch.float32, (3, K))), oracle.rotate_w(W))
    assert torch.equal(Xd, x_in)


# (M, N, K): ragged M and N, k-split and unsplit shapes
GEMM_SHAPES = [(5, 100, 384), (13, 1001, 2048), (70, 130, 1152), (300, 1001, 256), (1, 17, 128)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemms_exact_buffers(M, N, K):
    L = q.lib()
    G = K // 128
    rng = synth.make_rng(203)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K, n_outliers=1)
    Wq, Ws, Wq_r, Ws_r = _pack(W)
    Xd = dev_bf16(X)
    Xq_r, Xs_r = oracle.quant_act(X)
    Xq_d, Xs_d = dev(Xq_r), dev(Xs_r)
    q8, s8 = oracle.quant_act8(X)
    q8_d, s8_d = dev(q8), dev(s8)
    want4 = oracle.gemm_w4a4(Xq_r, Xs_r, Wq_r, Ws_r)
    want16 = oracle.gemm_w4a16(X, Wq_r, Ws_r)
    want8 = oracle.gemm_w4a8(q8, s8, Wq_r, Ws_r)
    P4 = oracle.w4a4_partials(Xq_r, Wq_r)
    P8 = oracle.w4a8_partials(q8, Wq_r)
    stm = M <= 16
    fam4 = [q.GEMM_AUTO, q.GEMM_SKINNY, q.GEMM_TILED] + ([q.GEMM_STREAM] if stm else [])
    for v in fam4:
        say(f"canary w4a4 M={M} N={N} K={K} variant={v}")
        Y, P, ws = Guarded(M * N * 4), Guarded(M * N * G * 4), _ws(1, M, N, K)
        _ok(L.qspec_gemm_w4a4(P_(Xq_d.data_ptr()), P_(Xs_d.data_ptr()), Wq.ptr, Ws.ptr, M, N, K,
                              128, v, Y.ptr, P.ptr, ws.ptr, ws.n, _stream()), "gemm_w4a4")
        assert Y.intact() and P.intact() and ws.intact(), f"w4a4 variant {v}"
        assert np.array_equal(host(P.view(torch.int32, (M, N, G))), P4)
        assert_close(host(Y.view(torch.float32, (M, N))), want4, what=f"w4a4 variant {v}")
        Yb, ws = Guarded(M * N * 2), _ws(1, M, N, K)
        _ok(L.qspec_gemm_w4a4_bf16(P_(Xq_d.data_ptr()), P_(Xs_d.data_ptr()), Wq.ptr, Ws.ptr, M, N,
                                   K, 128, v, Yb.ptr, ws.ptr, ws.n, _stream()), "gemm_w4a4_bf16")
        assert Yb.intact() and ws.intact(), f"w4a4 bf16 variant {v}"
    fam16 = [q.GEMM_AUTO, q.GEMM_GEMV, q.GEMM_SKINNY, q.GEMM_TILED] + ([q.GEMM_STREAM] if stm else [])
    for v in fam16:
        say(f"canary w4a16 M={M} N={N} K={K} variant={v}")
        Y, ws = Guarded(M * N * 4), _ws(2, M, N, K)
        _ok(L.qspec_gemm_w4a16(P_(Xd.data_ptr()), Wq.ptr, Ws.ptr, M, N, K, 128, v, Y.ptr, ws.ptr,
                               ws.n, _stream()), "gemm_w4a16")
        assert Y.intact() and ws.intact(), f"w4a16 variant {v}"
        assert_close(host(Y.view(torch.float32, (M, N))), want16, what=f"w4a16 variant {v}")
    fam8 = [q.GEMM_AUTO, q.GEMM_SKINNY] + ([q.GEMM_STREAM] if stm else [])
    for v in fam8:
        say(f"canary w4a8 M={M} N={N} K={K} variant={v}")
        Y, P, ws = Guarded(M * N * 4), Guarded(M * N * G * 4), _ws(4, M, N, K)
        _ok(L.qspec_gemm_w4a8(P_(q8_d.data_ptr()), P_(s8_d.data_ptr()), Wq.ptr, Ws.ptr, M, N, K,
                              128, v, Y.ptr, P.ptr, ws.ptr, ws.n, _stream()), "gemm_w4a8")
        assert Y.intact() and P.intact() and ws.intact(), f"w4a8 variant {v}"
        assert np.array_equal(host(P.view(torch.int32, (M, N, G))), P8)
        assert_close(host(Y.view(torch.float32, (M, N))), want8, what=f"w4a8 variant {v}")
    assert torch.equal(Xq_d, dev(Xq_r)) and torch.equal(q8_d, dev(q8))


@pytest.mark.parametrize("B,gamma,V", [(3, 2, 1001), (5, 4, 50257), (1, 16, 8195)])
def test_verify_exact_buffers(B, gamma, V):
    say(f"canary verify B={B} gamma={gamma} V={V}")
    L = q.lib()
    rng = synth.make_rng(204)
    tgt, drf = synth.verify_logits(rng, B, gamma, V)
    d = synth.gumbel_drafts(rng, drf)
    ua = synth.uniforms(rng, (B, gamma))
    us = synth.uniforms(rng, (B,))
    t_d, f_d, d_d, ua_d, us_d = dev(tgt), dev(drf), dev(d), dev(ua), dev(us)
    t_in = t_d.clone()
    for mode in (q.VERIFY_GREEDY, q.VERIFY_SAMPLE):
        n, out, ws = Guarded(B * 4), Guarded(B * (gamma + 1) * 4), _ws(3, B, gamma, V)
        smp = mode == q.VERIFY_SAMPLE
        ptr = lambda t: P_(t.data_ptr()) if smp else None  # noqa: E731
        _ok(L.qspec_verify(mode, B, gamma, V, P_(d_d.data_ptr()), ptr(f_d), P_(t_d.data_ptr()),
                           ptr(ua_d), ptr(us_d), n.ptr, out.ptr, ws.ptr, ws.n, _stream()),
            "verify")
        assert n.intact() and out.intact() and ws.intact(), f"verify mode {mode}"
        got_n = host(n.view(torch.int32, (B,)))
        got_o = host(out.view(torch.int32, (B, gamma + 1)))
        if smp:
            n_r, o_r, flag = oracle.verify_sample(tgt, drf, d, ua, us)
            ok = ~flag
            assert np.array_equal(got_n[ok], n_r[ok]) and np.array_equal(got_o[ok], o_r[ok])
        else:
            n_r, o_r = oracle.verify_greedy(tgt, d)
            assert np.array_equal(got_n, n_r) and np.array_equal(got_o, o_r)
    assert torch.equal(t_d, t_in)
