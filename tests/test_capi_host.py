"""Host-only checks of the C ABI: the library loads without a GPU, exports
every entry point declared in include/qspec.h, and rejects bad arguments with
the documented status codes before touching the device (the pointers passed
here are never dereferenced)."""

import ctypes
import glob
import os
import re

import pytest

import quantization_self_speculation_amd as q
from quantization_self_speculation_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EDEV, EHIP = 0, -1, -2, -3, -4, -5, -6, -7
A = ctypes.c_void_p(0x10000)      # aligned, never dereferenced
MIS = ctypes.c_void_p(0x10004)    # misaligned
NUL = None
S = None                           # null stream


def declared():
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        names |= set(re.findall(r"\b(qspec_[a-z0-9_]+)\s*\(", open(h).read()))
    return sorted(names)


def test_exports_every_declared_symbol():
    L = q.lib()
    names = declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = q.lib()
    for s in (OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EDEV, EHIP):
        assert L.qspec_status_str(s)
    assert L.qspec_status_str(-99) == b"unknown status"


def test_pack_validation():
    L = q.lib()
    assert L.qspec_pack_w4(A, 4, 256, 64, A, A, S) == EUNSUP
    assert L.qspec_pack_w4(A, 4, 200, 128, A, A, S) == ESHAPE
    assert L.qspec_pack_w4(A, 0, 256, 128, A, A, S) == ESHAPE
    assert L.qspec_pack_w4(NUL, 4, 256, 128, A, A, S) == ENULL
    assert L.qspec_pack_w4(A, 4, 256, 128, MIS, A, S) == EALIGN
    assert b"K" in L.qspec_last_error() or True


def test_quant_validation():
    L = q.lib()
    assert L.qspec_quant_act(A, 0, 256, A, A, S) == ESHAPE
    assert L.qspec_quant_act(A, 4, 100, A, A, S) == ESHAPE
    assert L.qspec_quant_act(A, 4, 256, NUL, A, S) == ENULL
    assert L.qspec_quant_act(A, 4, 256, A, MIS, S) == EALIGN


def test_rotation_validation():
    L = q.lib()
    assert L.qspec_rotate_w(A, 0, 256, A, S) == ESHAPE
    assert L.qspec_rotate_w(A, 4, 200, A, S) == ESHAPE
    assert L.qspec_rotate_w(NUL, 4, 256, A, S) == ENULL
    assert L.qspec_rotate_w(A, 4, 256, MIS, S) == EALIGN
    assert L.qspec_rotate_x(A, 0, 256, A, S) == ESHAPE
    assert L.qspec_rotate_x(A, 4, 64, A, S) == ESHAPE
    assert L.qspec_rotate_x(A, 4, 256, NUL, S) == ENULL
    assert L.qspec_quant_act_rot(A, 4, 100, A, A, S) == ESHAPE
    assert L.qspec_quant_act_rot(A, 4, 256, NUL, A, S) == ENULL
    assert L.qspec_quant_act_rot(A, 4, 256, A, MIS, S) == EALIGN


def test_gemm_validation():
    L = q.lib()
    f = L.qspec_gemm_w4a4
    assert f(A, A, A, A, 8, 64, 256, 64, 0, A, NUL, NUL, 0, S) == EUNSUP
    assert f(A, A, A, A, 8, 64, 250, 128, 0, A, NUL, NUL, 0, S) == ESHAPE
    assert f(A, A, A, A, 8, 64, 256, 128, 1, A, NUL, NUL, 0, S) == EUNSUP   # GEMV is W4A16-only
    assert f(A, A, A, A, 8, 64, 256, 128, 9, A, NUL, NUL, 0, S) == EUNSUP
    assert f(NUL, A, A, A, 8, 64, 256, 128, 0, A, NUL, NUL, 0, S) == ENULL
    assert f(A, A, A, A, 8, 64, 256, 128, 0, MIS, NUL, NUL, 0, S) == EALIGN
    assert f(A, A, A, A, 8, 64, 256, 128, 0, A, MIS, NUL, 0, S) == EALIGN
    g = L.qspec_gemm_w4a16
    assert g(A, A, A, 0, 64, 256, 128, 0, A, NUL, 0, S) == ESHAPE
    assert g(A, A, A, 8, 64, 256, 128, 7, A, NUL, 0, S) == EUNSUP
    assert g(A, A, NUL, 8, 64, 256, 128, 0, A, NUL, 0, S) == ENULL
    # a split-K shape needs scratch: NULL / too small workspace is rejected
    need = q.workspace_bytes(b.OP_GEMM_W4A16, 40, 4608, 3584)
    assert need > 0
    assert g(A, A, A, 40, 4608, 3584, 128, 2, A, NUL, 0, S) == EWS
    assert g(A, A, A, 40, 4608, 3584, 128, 2, A, A, need - 1, S) == EWS
    sw = L.qspec_gemm_w4a16_swiglu   # gate|up in pair order, SwiGLU in the epilogue
    assert sw(A, A, A, 8, 72, 256, 128, A, NUL, 0, S) == ESHAPE     # N % 16 != 0
    assert sw(A, A, A, 8, 64, 250, 128, A, NUL, 0, S) == ESHAPE
    assert sw(A, A, A, 8, 64, 256, 64, A, NUL, 0, S) == EUNSUP
    assert sw(A, A, A, 8, 64, 256, 128, NUL, NUL, 0, S) == ENULL
    assert sw(A, A, A, 8, 64, 256, 128, MIS, NUL, 0, S) == EALIGN
    assert sw(A, A, A, 40, 4608, 3584, 128, A, NUL, 0, S) == EWS   # a k-split needs scratch
    for fn in (L.qspec_gemm_w4a4_swiglu, L.qspec_gemm_w4a8_swiglu):  # drafters, STREAM only
        assert fn(A, A, A, A, 8, 72, 256, 128, A, S) == ESHAPE      # N % 16 != 0
        assert fn(A, A, A, A, 8, 64, 250, 128, A, S) == ESHAPE
        assert fn(A, A, A, A, 8, 64, 256, 64, A, S) == EUNSUP
        assert fn(A, A, A, A, 17, 64, 256, 128, A, S) == EUNSUP     # M <= 16
        assert fn(A, A, A, A, 8, 64, 256, 128, NUL, S) == ENULL
        assert fn(A, NUL, A, A, 8, 64, 256, 128, A, S) == ENULL
        assert fn(A, A, A, A, 8, 64, 256, 128, MIS, S) == EALIGN
    fam = L.qspec_gemm_family    # the family a call runs, AUTO resolved, no device work
    W4A4, W4A16, W4A8 = b.OP_GEMM_W4A4, b.OP_GEMM_W4A16, b.OP_GEMM_W4A8
    assert fam(W4A4, 16, 11264, 2048, 0) == b.GEMM_STREAM
    assert fam(W4A8, 16, 11264, 2048, 0) == b.GEMM_STREAM
    assert fam(W4A16, 5, 11264, 2048, 0) == b.GEMM_STREAM
    assert fam(W4A16, 8, 3584, 18944, 0) == b.GEMM_STREAM
    assert fam(W4A16, 9, 3584, 18944, 0) == b.GEMM_SKINNY      # W4A16 STREAM up to 8 rows
    assert fam(W4A4, 16, 3584, 18944, 0) == b.GEMM_STREAM
    assert fam(W4A4, 8, 37888, 3584, 0) == b.GEMM_SKINNY
    assert fam(W4A4, 17, 11264, 2048, 0) == b.GEMM_SKINNY
    assert fam(W4A4, 256, 37888, 3584, 0) == b.GEMM_TILED
    assert fam(W4A8, 256, 37888, 3584, 0) == b.GEMM_SKINNY    # W4A8 has no TILED family
    assert fam(W4A16, 40, 37888, 3584, 1) == b.GEMM_GEMV
    assert fam(W4A4, 8, 64, 256, 3) == b.GEMM_TILED             # an explicit variant stands
    for args in ((W4A4, 8, 64, 256, 1), (W4A8, 8, 64, 256, 3), (W4A16, 17, 64, 256, 4),
                 (W4A16, 8, 64, 250, 0), (b.OP_VERIFY, 8, 64, 256, 0), (W4A4, 0, 64, 256, 0)):
        assert fam(*args) == -1, args
        assert L.qspec_last_error()
    u = L.qspec_gemm_w4a8        # the W4A8 tier: SKINNY and STREAM families; P after Y
    assert u(A, A, A, A, 17, 64, 256, 128, 4, A, NUL, NUL, 0, S) == EUNSUP   # STREAM: M <= 16
    for v in (1, 3, 9):
        assert u(A, A, A, A, 8, 64, 256, 128, v, A, NUL, NUL, 0, S) == EUNSUP
    assert u(A, A, A, A, 8, 64, 250, 128, 0, A, NUL, NUL, 0, S) == ESHAPE
    assert u(NUL, A, A, A, 8, 64, 256, 128, 0, A, NUL, NUL, 0, S) == ENULL
    assert u(A, A, A, A, 8, 64, 256, 128, 2, MIS, NUL, NUL, 0, S) == EALIGN
    assert u(A, A, A, A, 8, 64, 256, 128, 2, A, MIS, NUL, 0, S) == EALIGN
    assert u(A, A, A, A, 8, 1024, 2048, 128, 2, A, NUL, NUL, 0, S) == EWS
    assert q.workspace_bytes(b.OP_GEMM_W4A8, 8, 1024, 2048) == q.workspace_bytes(b.OP_GEMM_W4A4, 8, 1024, 2048)
    qa8 = L.qspec_quant_act8
    assert qa8(A, 0, 256, A, A, S) == ESHAPE
    assert qa8(A, 4, 250, A, A, S) == ESHAPE
    assert qa8(A, 4, 256, NUL, A, S) == ENULL
    assert qa8(A, 4, 256, A, MIS, S) == EALIGN
    h = L.qspec_gemm_w4a4_bf16   # same checks as the fp32 call, bf16 Y
    assert h(A, A, A, A, 8, 64, 256, 64, 0, A, NUL, 0, S) == EUNSUP
    assert h(A, A, A, A, 8, 64, 250, 128, 0, A, NUL, 0, S) == ESHAPE
    assert h(A, A, A, A, 8, 64, 256, 128, 1, A, NUL, 0, S) == EUNSUP
    assert h(A, A, A, A, 17, 64, 256, 128, 4, A, NUL, 0, S) == EUNSUP
    assert h(A, A, A, A, 8, 64, 256, 128, 0, NUL, NUL, 0, S) == ENULL
    assert h(A, A, A, A, 8, 64, 256, 128, 0, MIS, NUL, 0, S) == EALIGN
    need4 = q.workspace_bytes(b.OP_GEMM_W4A4, 8, 1024, 2048)
    assert need4 > 0
    assert h(A, A, A, A, 8, 1024, 2048, 128, 2, A, NUL, 0, S) == EWS


def test_verify_validation():
    L = q.lib()
    f = L.qspec_verify
    assert f(2, 1, 4, 100, A, NUL, A, NUL, NUL, A, A, A, 1 << 20, S) == EUNSUP
    assert f(0, 1, 0, 100, A, NUL, A, NUL, NUL, A, A, A, 1 << 20, S) == ESHAPE
    assert f(0, 1, 17, 100, A, NUL, A, NUL, NUL, A, A, A, 1 << 20, S) == ESHAPE
    assert f(0, 1, 4, 0, A, NUL, A, NUL, NUL, A, A, A, 1 << 20, S) == ESHAPE
    assert f(0, 1, 4, 100, A, A, A, NUL, NUL, A, A, A, 1 << 20, S) == EUNSUP  # greedy + logits
    assert f(1, 1, 4, 100, A, NUL, A, A, A, A, A, A, 1 << 20, S) == ENULL     # sample w/o logits
    assert f(0, 1, 4, 100, A, NUL, A, NUL, NUL, A, A, NUL, 0, S) == EWS
    assert f(0, 4000, 8, 100, A, NUL, A, NUL, NUL, A, A, A, 1 << 30, S) == ESHAPE  # grid limit


def test_workspace_bytes():
    assert q.workspace_bytes(b.OP_VERIFY, 32, 4, 128256) > 0
    assert q.workspace_bytes(b.OP_VERIFY, 32, 0, 128256) == 0
    assert q.workspace_bytes(99, 1, 1, 1) == 0
    # monotone in M (the answer covers every variant of the op)
    assert q.workspace_bytes(b.OP_GEMM_W4A16, 64, 3584, 3584) >= \
        q.workspace_bytes(b.OP_GEMM_W4A16, 8, 3584, 3584)


def test_device_check_without_gpu_is_an_error_not_a_crash():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert q.lib().qspec_device_check() in (EHIP, EDEV)


def test_harness_validation():
    L = q.lib()
    I64, D = ctypes.c_int64, ctypes.c_double
    # embed: d must be a positive multiple of 8; emb 16-byte aligned
    assert L.qspec_embed(A, 10, 12, A, 4, A, S) == ESHAPE
    assert L.qspec_embed(MIS, 10, 16, A, 4, A, S) == EALIGN
    assert L.qspec_embed(A, 10, 16, NUL, 4, A, S) == ENULL
    # add_rmsnorm: d <= 4096, stride >= d, add stride >= d when add is given
    assert L.qspec_add_rmsnorm(A, 8192, NUL, 0, 2, 8192, D(1e-6), A, S) == ESHAPE
    assert L.qspec_add_rmsnorm(A, 100, NUL, 0, 2, 128, D(1e-6), A, S) == ESHAPE
    assert L.qspec_add_rmsnorm(A, 128, A, 64, 2, 128, D(1e-6), A, S) == ESHAPE
    assert L.qspec_add_rmsnorm(A, 128, NUL, 0, 2, 128, D(-1.0), A, S) == ESHAPE
    # rope_kv / attention: heads, cache capacity
    assert L.qspec_rope_kv(A, 4, 6, 4, A, A, D(1e4), A, A, A, 2, 64, S) == ESHAPE
    assert L.qspec_rope_kv(A, 4, 8, 4, A, A, D(1e4), A, A, A, 2, 4000, S) == ESHAPE
    assert L.qspec_rope_kv(A, 4, 8, 4, A, A, D(0.0), A, A, A, 2, 64, S) == ESHAPE
    # the fused RoPE + attention call: the checks of both
    assert L.qspec_rope_attention(A, 4, 6, 4, A, A, D(1e4), A, A, A, 2, 64, A, S) == ESHAPE
    assert L.qspec_rope_attention(A, 4, 8, 4, A, A, D(1e4), A, A, A, 2, 4000, A, S) == ESHAPE
    assert L.qspec_rope_attention(A, 4, 8, 4, A, A, D(0.0), A, A, A, 2, 64, A, S) == ESHAPE
    assert L.qspec_rope_attention(A, 4, 8, 4, A, A, D(1e4), A, A, A, 2, 64, NUL, S) == ENULL
    assert L.qspec_attention(A, A, A, 4, 8, 4, A, A, 2, 0, A, S) == ESHAPE
    assert L.qspec_attention(A, A, A, 4, 8, 3, A, A, 2, 64, A, S) == ESHAPE
    assert L.qspec_attention(A, A, A, 4, 8, 4, NUL, A, 2, 64, A, S) == ENULL
    # the RMSNorm with the drafter's codes: d a multiple of 128, code buffers aligned
    assert L.qspec_add_rmsnorm_quant(A, 200, NUL, 0, 2, 200, D(1e-6), A, A, A, S) == ESHAPE
    assert L.qspec_add_rmsnorm_quant(A, 256, NUL, 0, 2, 256, D(1e-6), A, NUL, A, S) == ENULL
    assert L.qspec_add_rmsnorm_quant(A, 256, NUL, 0, 2, 256, D(1e-6), A, A, MIS, S) == EALIGN
    assert L.qspec_add_rmsnorm_quant8(A, 200, NUL, 0, 2, 200, D(1e-6), A, A, A, S) == ESHAPE
    assert L.qspec_add_rmsnorm_quant8(A, 256, NUL, 0, 2, 256, D(1e-6), A, NUL, A, S) == ENULL
    assert L.qspec_add_rmsnorm_quant8(A, 256, NUL, 0, 2, 256, D(1e-6), A, A, MIS, S) == EALIGN
    assert L.qspec_add_rmsnorm_quant8(A, 128, NUL, 0, 2, 256, D(1e-6), A, A, A, S) == ESHAPE
    # silu, argmax
    assert L.qspec_silu_mul(A, 0, 10, A, S) == ESHAPE
    assert L.qspec_silu_mul_pairs(A, 4, 12, A, S) == ESHAPE       # ffn % 8 != 0
    assert L.qspec_silu_mul_pairs(A, 0, 16, A, S) == ESHAPE
    assert L.qspec_silu_mul_pairs(NUL, 4, 16, A, S) == ENULL
    assert L.qspec_argmax(A, 2, 10, A, 0, S) == ESHAPE
    # round bookkeeping
    assert L.qspec_spec_prepare(2, 4, 2, 0, A, A, A, A, A, A, S) == EUNSUP
    assert L.qspec_spec_prepare(0, 4, 2, 3, A, A, A, A, A, A, S) == ESHAPE
    assert L.qspec_spec_prepare(1, 4, 0, 0, A, A, A, A, A, A, S) == ESHAPE
    assert L.qspec_spec_prepare(1, 4, 2, 0, A, A, NUL, A, A, A, S) == ENULL
    assert L.qspec_spec_commit(4, 17, A, A, A, A, 3, A, 8, A, 5, A, S) == ESHAPE
    assert L.qspec_spec_commit(4, 2, A, A, A, A, 0, A, 8, A, 5, A, S) == ESHAPE
    assert L.qspec_spec_commit(4, 2, A, NUL, A, A, 3, A, 8, A, 5, A, S) == ENULL


def test_stream_variant_limits():
    L = q.lib()
    # the STREAM family (variant 4) takes at most 16 rows
    assert L.qspec_gemm_w4a16(A, A, A, 17, 64, 256, 128, 4, A, NUL, 0, S) == EUNSUP
    assert L.qspec_gemm_w4a4(A, A, A, A, 17, 64, 256, 128, 4, A, NUL, NUL, 0, S) == EUNSUP
    assert L.qspec_gemm_w4a16(A, A, A, 4, 64, 256, 128, 5, A, NUL, 0, S) == EUNSUP
