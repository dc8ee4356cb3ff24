"""ctypes binding of libqspec.so: argument marshalling only.

Each function takes CUDA (HIP) torch tensors, checks dtypes/shapes/contiguity
on the host, allocates outputs and scratch through torch's caching allocator,
and calls the C entry point of the same name on torch's current stream.  All
arithmetic happens in the library's kernels.
"""

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqspec.so")
_lock = threading.Lock()
_lib = None

GEMM_AUTO, GEMM_GEMV, GEMM_SKINNY, GEMM_TILED, GEMM_STREAM = 0, 1, 2, 3, 4
VERIFY_GREEDY, VERIFY_SAMPLE = 0, 1
OP_GEMM_W4A4, OP_GEMM_W4A16, OP_VERIFY, OP_GEMM_W4A8 = 1, 2, 3, 4
GROUP = 128


class QSpecError(RuntimeError):
    def __init__(self, status, name, detail):
        super().__init__(f"{name}: status {status} ({detail})")
        self.status = status


def lib_path():
    return _LIB_PATH


def lib():
    """Load libqspec.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m quantization_self_speculation_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        sig = {
            "qspec_status_str": (ctypes.c_char_p, [I]),
            "qspec_last_error": (ctypes.c_char_p, []),
            "qspec_version": (ctypes.c_char_p, []),
            "qspec_device_check": (I, []),
            "qspec_workspace_bytes": (SZ, [I, I64, I64, I64]),
            "qspec_pack_w4": (I, [P, I64, I64, I, P, P, P]),
            "qspec_quant_act": (I, [P, I64, I64, P, P, P]),
            "qspec_rotate_w": (I, [P, I64, I64, P, P]),
            "qspec_rotate_x": (I, [P, I64, I64, P, P]),
            "qspec_quant_act_rot": (I, [P, I64, I64, P, P, P]),
            "qspec_gemm_w4a4": (I, [P, P, P, P, I64, I64, I64, I, I, P, P, P, SZ, P]),
            "qspec_gemm_w4a4_bf16": (I, [P, P, P, P, I64, I64, I64, I, I, P, P, SZ, P]),
            "qspec_gemm_w4a16": (I, [P, P, P, I64, I64, I64, I, I, P, P, SZ, P]),
            "qspec_gemm_w4a16_swiglu": (I, [P, P, P, I64, I64, I64, I, P, P, SZ, P]),
            "qspec_gemm_family": (I, [I, I64, I64, I64, I]),
            "qspec_gemm_w4a4_swiglu": (I, [P, P, P, P, I64, I64, I64, I, P, P]),
            "qspec_gemm_w4a8_swiglu": (I, [P, P, P, P, I64, I64, I64, I, P, P]),
            "qspec_quant_act8": (I, [P, I64, I64, P, P, P]),
            "qspec_gemm_w4a8": (I, [P, P, P, P, I64, I64, I64, I, I, P, P, P, SZ, P]),
            "qspec_verify": (I, [I, I64, I, I64, P, P, P, P, P, P, P, P, SZ, P]),
            "qspec_verify_noalloc": (I, [I, I64, I, I64, P, P, P, P, P, P, P, P]),
            "qspec_embed": (I, [P, I64, I64, P, I64, P, P]),
            "qspec_add_rmsnorm": (I, [P, I64, P, I64, I64, I64, ctypes.c_double, P, P]),
            "qspec_rope_kv": (I, [P, I64, I, I, P, P, ctypes.c_double, P, P, P, I64, I64, P]),
            "qspec_attention": (I, [P, P, P, I64, I, I, P, P, I64, I64, P, P]),
            "qspec_rope_attention": (I, [P, I64, I, I, P, P, ctypes.c_double, P, P, P, I64, I64, P,
                                         P]),
            "qspec_silu_mul": (I, [P, I64, I64, P, P]),
            "qspec_silu_mul_pairs": (I, [P, I64, I64, P, P]),
            "qspec_add_rmsnorm_quant": (I, [P, I64, P, I64, I64, I64, ctypes.c_double, P, P, P, P]),
            "qspec_add_rmsnorm_quant8": (I, [P, I64, P, I64, I64, I64, ctypes.c_double, P, P, P, P]),
            "qspec_argmax": (I, [P, I64, I64, P, I64, P]),
            "qspec_spec_prepare": (I, [I, I64, I, I, P, P, P, P, P, P, P]),
            "qspec_spec_commit": (I, [I64, I, P, P, P, P, I64, P, I64, P, I, P, P]),
            "qspec_probe_read": (I, [P, I64, I, I, P, P]),
            "qspec_probe_mfma": (I, [I, I, I, P, P]),
            "qspec_probe_empty": (I, [P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
        return L


def _check(status, name):
    if status != 0:
        L = lib()
        raise QSpecError(status, name, f"{L.qspec_status_str(status).decode()}: "
                                       f"{L.qspec_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _out_n(N, Y, Wq):
    if N is not None:
        return int(N)
    if Y is not None:
        return int(Y.shape[1])
    return int(Wq.shape[0])


def workspace_bytes(op, a, b, c):
    return int(lib().qspec_workspace_bytes(op, a, b, c))


def _workspace(nbytes, device, ws):
    """the caller's workspace, or a zero-filled one for this call (a GEMM
    workspace must hold zeros when first used; the calls keep it that way)"""
    if nbytes == 0:
        return None, 0
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws, ws.numel() * ws.element_size()
    w = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return w, nbytes


def padded_rows(N):
    """rows of the tiled weight buffer: N rounded up to a multiple of 16"""
    return -(-N // 16) * 16


def pack_w4(W, Wq=None, Ws=None, N=None):
    """fp32 [N, K] -> (Wq uint8 [Np, K/2], Ws float16 [Np, K/128]), Np =
    ceil(N/16)*16, both in the tiled storage order.  Pass N to the GEMMs."""
    _need(W, "W", torch.float32)
    N, K = W.shape
    if Wq is None:
        Wq = torch.empty((padded_rows(N), K // 2), dtype=torch.uint8, device=W.device)
    if Ws is None:
        Ws = torch.empty((padded_rows(N), max(K // GROUP, 1)), dtype=torch.float16,
                         device=W.device)
    _check(lib().qspec_pack_w4(_ptr(W), N, K, GROUP, _ptr(Wq), _ptr(Ws), _stream()),
           "qspec_pack_w4")
    return Wq, Ws


def quant_act(X, Xq=None, Xs=None):
    """bf16 [M, K] -> (Xq uint8 [M, K/2], Xs float32 [M])."""
    _need(X, "X", torch.bfloat16)
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    if Xs is None:
        Xs = torch.empty((M,), dtype=torch.float32, device=X.device)
    _check(lib().qspec_quant_act(_ptr(X), M, K, _ptr(Xq), _ptr(Xs), _stream()), "qspec_quant_act")
    return Xq, Xs


def rotate_w(W, Wr=None):
    """fp32 [N, K] -> H W / 8 per 128-group, fp32 (then pack_w4)."""
    _need(W, "W", torch.float32)
    N, K = W.shape
    if Wr is None:
        Wr = torch.empty_like(W)
    _need(Wr, "Wr", torch.float32, (N, K))
    _check(lib().qspec_rotate_w(_ptr(W), N, K, _ptr(Wr), _stream()), "qspec_rotate_w")
    return Wr


def rotate_x(X, Xr=None):
    """bf16 [M, K] -> bf16(H x / 16) per 128-group: the verifier's input."""
    _need(X, "X", torch.bfloat16)
    M, K = X.shape
    if Xr is None:
        Xr = torch.empty_like(X)
    _need(Xr, "Xr", torch.bfloat16, (M, K))
    _check(lib().qspec_rotate_x(_ptr(X), M, K, _ptr(Xr), _stream()), "qspec_rotate_x")
    return Xr


def quant_act_rot(X, Xq=None, Xs=None):
    """bf16 [M, K] -> codes and scales of H x / 16 (the drafter's input)."""
    _need(X, "X", torch.bfloat16)
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    if Xs is None:
        Xs = torch.empty((M,), dtype=torch.float32, device=X.device)
    _check(lib().qspec_quant_act_rot(_ptr(X), M, K, _ptr(Xq), _ptr(Xs), _stream()),
           "qspec_quant_act_rot")
    return Xq, Xs


def gemm_w4a4(Xq, Xs, Wq, Ws, variant=GEMM_AUTO, partials=False, Y=None, P=None, ws=None, N=None):
    """Draft-mode linear layer -> Y fp32 [M, N] (and int32 partials [M, N, K/128]).
    Wq, Ws are the tiled buffers of qspec_pack_w4 ([Np, ...], Np = ceil(N/16)*16);
    N defaults to Y's width, else Np."""
    _need(Xq, "Xq", torch.uint8)
    _need(Wq, "Wq", torch.uint8)
    _need(Xs, "Xs", torch.float32)
    _need(Ws, "Ws", torch.float16)
    M, K = Xq.shape[0], 2 * Xq.shape[1]
    N = _out_n(N, Y, Wq)
    _need(Xs, "Xs", torch.float32, (M,))
    _need(Wq, "Wq", torch.uint8, (padded_rows(N), K // 2))
    _need(Ws, "Ws", torch.float16, (padded_rows(N), K // GROUP))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=Xq.device)
    if partials and P is None:
        P = torch.empty((M, N, K // GROUP), dtype=torch.int32, device=Xq.device)
    w, wb = _workspace(workspace_bytes(OP_GEMM_W4A4, M, N, K), Xq.device, ws)
    _check(lib().qspec_gemm_w4a4(_ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws), M, N, K, GROUP, variant,
                                 _ptr(Y), _ptr(P), _ptr(w), wb, _stream()), "qspec_gemm_w4a4")
    return (Y, P) if partials else Y


def gemm_w4a4_bf16(Xq, Xs, Wq, Ws, variant=GEMM_AUTO, Y=None, ws=None, N=None):
    """Draft-mode linear layer with a bf16 output -> Y bf16 [M, N]: the
    round-to-nearest-even of the fp32 result gemm_w4a4 gives (same variant)."""
    _need(Xq, "Xq", torch.uint8)
    M, K = Xq.shape[0], 2 * Xq.shape[1]
    N = _out_n(N, Y, Wq)
    _need(Xs, "Xs", torch.float32, (M,))
    _need(Wq, "Wq", torch.uint8, (padded_rows(N), K // 2))
    _need(Ws, "Ws", torch.float16, (padded_rows(N), K // GROUP))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=Xq.device)
    _need(Y, "Y", torch.bfloat16, (M, N))
    w, wb = _workspace(workspace_bytes(OP_GEMM_W4A4, M, N, K), Xq.device, ws)
    _check(lib().qspec_gemm_w4a4_bf16(_ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws), M, N, K, GROUP,
                                      variant, _ptr(Y), _ptr(w), wb, _stream()),
           "qspec_gemm_w4a4_bf16")
    return Y


def quant_act8(X, Xq=None, Xs=None):
    """bf16 activations [M, K] -> (int8 codes [M, K], fp32 scales [M]): the
    8-bit per-token quantizer of the W4A8 tier."""
    _need(X, "X", torch.bfloat16)
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if Xs is None:
        Xs = torch.empty((M,), dtype=torch.float32, device=X.device)
    _need(Xq, "Xq", torch.int8, (M, K))
    _need(Xs, "Xs", torch.float32, (M,))
    _check(lib().qspec_quant_act8(_ptr(X), M, K, _ptr(Xq), _ptr(Xs), _stream()), "qspec_quant_act8")
    return Xq, Xs


def gemm_w4a8(Xq, Xs, Wq, Ws, variant=GEMM_AUTO, partials=False, Y=None, P=None, ws=None,
              N=None):
    """W4A8 linear layer on the shared buffer -> Y fp32 [M, N] (and int32
    partials [M, N, K/128]); N as for gemm_w4a4."""
    _need(Xq, "Xq", torch.int8)
    M, K = Xq.shape
    N = _out_n(N, Y, Wq)
    _need(Xs, "Xs", torch.float32, (M,))
    _need(Wq, "Wq", torch.uint8, (padded_rows(N), K // 2))
    _need(Ws, "Ws", torch.float16, (padded_rows(N), K // GROUP))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=Xq.device)
    if partials and P is None:
        P = torch.empty((M, N, K // GROUP), dtype=torch.int32, device=Xq.device)
    w, wb = _workspace(workspace_bytes(OP_GEMM_W4A8, M, N, K), Xq.device, ws)
    _check(lib().qspec_gemm_w4a8(_ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws), M, N, K, GROUP, variant,
                                 _ptr(Y), _ptr(P), _ptr(w), wb, _stream()), "qspec_gemm_w4a8")
    return (Y, P) if partials else Y


def gemm_w4a16(X, Wq, Ws, variant=GEMM_AUTO, Y=None, ws=None, N=None):
    """Verify-mode linear layer -> Y fp32 [M, N] (N as for gemm_w4a4)."""
    _need(X, "X", torch.bfloat16)
    M, K = X.shape
    N = _out_n(N, Y, Wq)
    _need(Wq, "Wq", torch.uint8, (padded_rows(N), K // 2))
    _need(Ws, "Ws", torch.float16, (padded_rows(N), K // GROUP))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    w, wb = _workspace(workspace_bytes(OP_GEMM_W4A16, M, N, K), X.device, ws)
    _check(lib().qspec_gemm_w4a16(_ptr(X), _ptr(Wq), _ptr(Ws), M, N, K, GROUP, variant, _ptr(Y),
                                  _ptr(w), wb, _stream()), "qspec_gemm_w4a16")
    return Y


def gemm_w4a16_swiglu(X, Wq, Ws, A=None, ws=None, N=None):
    """Verify-mode gate|up layer with its SwiGLU fused -> A bf16 [M, N/2]:
    Wq, Ws hold the N = 2F gate|up rows in pair order (see pair_rows), the
    SKINNY family's k-split; bitwise silu_mul_pairs of gemm_w4a16(SKINNY)."""
    _need(X, "X", torch.bfloat16)
    M, K = X.shape
    if N is None:
        N = 2 * A.shape[1] if A is not None else Wq.shape[0]
    _need(Wq, "Wq", torch.uint8, (padded_rows(N), K // 2))
    _need(Ws, "Ws", torch.float16, (padded_rows(N), K // GROUP))
    if A is None:
        A = torch.empty((M, N // 2), dtype=torch.bfloat16, device=X.device)
    _need(A, "A", torch.bfloat16, (M, N // 2))
    w, wb = _workspace(workspace_bytes(OP_GEMM_W4A16, M, N, K), X.device, ws)
    _check(lib().qspec_gemm_w4a16_swiglu(_ptr(X), _ptr(Wq), _ptr(Ws), M, N, K, GROUP, _ptr(A),
                                         _ptr(w), wb, _stream()), "qspec_gemm_w4a16_swiglu")
    return A


def gemm_family(op, M, N, K, variant=GEMM_AUTO):
    """The GEMM family (GEMM_GEMV / _SKINNY / _TILED / _STREAM) a call of
    `op` (OP_GEMM_W4A4 / _W4A16 / _W4A8) with these sizes and `variant` runs."""
    f = lib().qspec_gemm_family(op, M, N, K, variant)
    if f < 0:
        raise QSpecError(f, "qspec_gemm_family", lib().qspec_last_error().decode())
    return f


def gemm_w4a4_swiglu(Xq, Xs, Wq, Ws, A=None, N=None):
    """Draft-mode gate|up layer with its SwiGLU fused (STREAM family, M <= 16)
    -> A bf16 [M, N/2]; rows in pair order; bitwise silu_mul_pairs of
    gemm_w4a4(STREAM)."""
    return _int_swiglu("qspec_gemm_w4a4_swiglu", torch.uint8, Xq, Xs, Wq, Ws, A, N)


def gemm_w4a8_swiglu(Xq, Xs, Wq, Ws, A=None, N=None):
    """W4A8 gate|up layer with its SwiGLU fused, as gemm_w4a4_swiglu."""
    return _int_swiglu("qspec_gemm_w4a8_swiglu", torch.int8, Xq, Xs, Wq, Ws, A, N)


def _int_swiglu(fn, code_dtype, Xq, Xs, Wq, Ws, A, N):
    _need(Xq, "Xq", code_dtype)
    M = Xq.shape[0]
    K = Xq.shape[1] * (2 if code_dtype == torch.uint8 else 1)
    if N is None:
        N = 2 * A.shape[1] if A is not None else Wq.shape[0]
    _need(Xs, "Xs", torch.float32, (M,))
    _need(Wq, "Wq", torch.uint8, (padded_rows(N), K // 2))
    _need(Ws, "Ws", torch.float16, (padded_rows(N), K // GROUP))
    if A is None:
        A = torch.empty((M, N // 2), dtype=torch.bfloat16, device=Xq.device)
    _need(A, "A", torch.bfloat16, (M, N // 2))
    _check(getattr(lib(), fn)(_ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws), M, N, K, GROUP, _ptr(A),
                              _stream()), fn)
    return A


def pair_rows(gate_up):
    """[2F, ...] gate|up rows (gate rows first) -> the pair order the fused
    gate|up layer reads: in each block of 16 rows, 8 gate rows then the 8
    matching up rows.  F % 8 == 0; works on numpy arrays and torch tensors."""
    F = gate_up.shape[0] // 2
    if F % 8 != 0 or 2 * F != gate_up.shape[0]:
        raise ValueError("pair order needs 2F rows with F a multiple of 8")
    g = gate_up[:F].reshape(F // 8, 8, *gate_up.shape[1:])
    u = gate_up[F:].reshape(F // 8, 8, *gate_up.shape[1:])
    if isinstance(gate_up, torch.Tensor):
        return torch.stack((g, u), dim=1).reshape(gate_up.shape)
    import numpy as _np
    return _np.stack((g, u), axis=1).reshape(gate_up.shape)


def verify(mode, target_logits, draft_tok, draft_logits=None, u_accept=None, u_sample=None,
           n_accept=None, out_tok=None, ws=None):
    """-> (n_accept int32 [B], out_tok int32 [B, gamma+1] padded with -1)."""
    _need(target_logits, "target_logits", torch.float32)
    B, G1, V = target_logits.shape
    gamma = G1 - 1
    _need(draft_tok, "draft_tok", torch.int32, (B, gamma))
    if mode == VERIFY_SAMPLE:
        _need(draft_logits, "draft_logits", torch.float32, (B, gamma, V))
        _need(u_accept, "u_accept", torch.float32, (B, gamma))
        _need(u_sample, "u_sample", torch.float32, (B,))
    dev = target_logits.device
    if n_accept is None:
        n_accept = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_tok is None:
        out_tok = torch.empty((B, G1), dtype=torch.int32, device=dev)
    w, wb = _workspace(workspace_bytes(OP_VERIFY, B, gamma, V), dev, ws)
    _check(lib().qspec_verify(mode, B, gamma, V, _ptr(draft_tok), _ptr(draft_logits),
                              _ptr(target_logits), _ptr(u_accept), _ptr(u_sample), _ptr(n_accept),
                              _ptr(out_tok), _ptr(w), wb, _stream()), "qspec_verify")
    return n_accept, out_tok


def verify_noalloc(mode, target_logits, draft_tok, draft_logits=None, u_accept=None,
                   u_sample=None, n_accept=None, out_tok=None):
    """verify() on the library's fixed per-device scratch (no workspace);
    the outputs must be given for a call that may not allocate."""
    _need(target_logits, "target_logits", torch.float32)
    B, G1, V = target_logits.shape
    gamma = G1 - 1
    _need(draft_tok, "draft_tok", torch.int32, (B, gamma))
    if mode == VERIFY_SAMPLE:
        _need(draft_logits, "draft_logits", torch.float32, (B, gamma, V))
        _need(u_accept, "u_accept", torch.float32, (B, gamma))
        _need(u_sample, "u_sample", torch.float32, (B,))
    dev = target_logits.device
    if n_accept is None:
        n_accept = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_tok is None:
        out_tok = torch.empty((B, G1), dtype=torch.int32, device=dev)
    _need(n_accept, "n_accept", torch.int32, (B,))
    _need(out_tok, "out_tok", torch.int32, (B, G1))
    _check(lib().qspec_verify_noalloc(mode, B, gamma, V, _ptr(draft_tok), _ptr(draft_logits),
                                      _ptr(target_logits), _ptr(u_accept), _ptr(u_sample),
                                      _ptr(n_accept), _ptr(out_tok), _stream()),
           "qspec_verify_noalloc")
    return n_accept, out_tok


# ---------------------------------------------------------------- decoder kernels
# These take tensors that may be views (row offsets, strided columns): the
# pointer passed is the view's first element; shapes are given explicitly
# where a view cannot carry them.
def _dev(t, name, dtype):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype:
        raise TypeError(f"{name} must be a {dtype} device tensor")


def embed(emb, tok, x):
    """x[m] = float(emb[tok[m]]); emb bf16 [V, d], tok int32 [M], x fp32 [M, d]"""
    _need(emb, "emb", torch.bfloat16)
    _dev(tok, "tok", torch.int32)
    _dev(x, "x", torch.float32)
    V, d = emb.shape
    _check(lib().qspec_embed(_ptr(emb), V, d, _ptr(tok), tok.numel(), _ptr(x), _stream()),
           "qspec_embed")


def add_rmsnorm(x, add, y, eps):
    """x[m] += add[m] (if add is not None); y[m] = bf16(rmsnorm(x[m])).
    x and add are 2-D (row-strided views allowed), y dense bf16 [M, d]."""
    _dev(x, "x", torch.float32)
    _need(y, "y", torch.bfloat16)
    M, d = y.shape
    if x.dim() != 2 or tuple(x.shape) != (M, d) or x.stride(1) != 1:
        raise ValueError("x must be a row-strided [M, d] view")
    a_stride = 0
    if add is not None:
        _dev(add, "add", torch.float32)
        if add.dim() != 2 or tuple(add.shape) != (M, d) or add.stride(1) != 1:
            raise ValueError("add must be a row-strided [M, d] view")
        a_stride = int(add.stride(0))
    _check(lib().qspec_add_rmsnorm(_ptr(x), int(x.stride(0)), _ptr(add), a_stride, M, d,
                                   float(eps), _ptr(y), _stream()), "qspec_add_rmsnorm")


def add_rmsnorm_quant(x, add, y, yq, ys, eps):
    """add_rmsnorm, and the 4-bit codes / scales of y (as quant_act(y) gives
    them) into yq uint8 [M, d/2] and ys fp32 [M] in the same pass."""
    _dev(x, "x", torch.float32)
    _need(y, "y", torch.bfloat16)
    M, d = y.shape
    _need(yq, "yq", torch.uint8, (M, d // 2))
    _need(ys, "ys", torch.float32, (M,))
    if x.dim() != 2 or tuple(x.shape) != (M, d) or x.stride(1) != 1:
        raise ValueError("x must be a row-strided [M, d] view")
    a_stride = 0
    if add is not None:
        _dev(add, "add", torch.float32)
        if add.dim() != 2 or tuple(add.shape) != (M, d) or add.stride(1) != 1:
            raise ValueError("add must be a row-strided [M, d] view")
        a_stride = int(add.stride(0))
    _check(lib().qspec_add_rmsnorm_quant(_ptr(x), int(x.stride(0)), _ptr(add), a_stride, M, d,
                                         float(eps), _ptr(y), _ptr(yq), _ptr(ys), _stream()),
           "qspec_add_rmsnorm_quant")


def add_rmsnorm_quant8(x, add, y, yq, ys, eps):
    """add_rmsnorm, and the 8-bit codes / scales of y (as quant_act8(y) gives
    them) into yq int8 [M, d] and ys fp32 [M] in the same pass."""
    _dev(x, "x", torch.float32)
    _need(y, "y", torch.bfloat16)
    M, d = y.shape
    _need(yq, "yq", torch.int8, (M, d))
    _need(ys, "ys", torch.float32, (M,))
    if x.dim() != 2 or tuple(x.shape) != (M, d) or x.stride(1) != 1:
        raise ValueError("x must be a row-strided [M, d] view")
    a_stride = 0
    if add is not None:
        _dev(add, "add", torch.float32)
        if add.dim() != 2 or tuple(add.shape) != (M, d) or add.stride(1) != 1:
            raise ValueError("add must be a row-strided [M, d] view")
        a_stride = int(add.stride(0))
    _check(lib().qspec_add_rmsnorm_quant8(_ptr(x), int(x.stride(0)), _ptr(add), a_stride, M, d,
                                          float(eps), _ptr(y), _ptr(yq), _ptr(ys), _stream()),
           "qspec_add_rmsnorm_quant8")


def rope_kv(qkv, seq, pos, q_out, kcache, vcache, n_heads, n_kv, rope_base):
    """RoPE on the q and k parts of qkv fp32 [M, (H + 2 Hkv) 128]; q_out fp32
    [M, H 128]; K/V written into the bf16 caches [B, Hkv, cap, 128]"""
    _dev(qkv, "qkv", torch.float32)
    _dev(q_out, "q_out", torch.float32)
    _dev(kcache, "kcache", torch.bfloat16)
    _dev(vcache, "vcache", torch.bfloat16)
    B, _, cap, _ = kcache.shape
    _check(lib().qspec_rope_kv(_ptr(qkv), int(qkv.shape[0]), n_heads, n_kv, _ptr(seq), _ptr(pos),
                               float(rope_base), _ptr(q_out), _ptr(kcache), _ptr(vcache), B, cap,
                               _stream()), "qspec_rope_kv")


def attention(q, kcache, vcache, seq, pos, out, n_heads, n_kv):
    """causal GQA over the cache; q fp32 [M, H 128] -> out bf16 [M, H 128]"""
    _dev(q, "q", torch.float32)
    _dev(out, "out", torch.bfloat16)
    B, _, cap, _ = kcache.shape
    _check(lib().qspec_attention(_ptr(q), _ptr(kcache), _ptr(vcache), int(q.shape[0]), n_heads,
                                 n_kv, _ptr(seq), _ptr(pos), B, cap, _ptr(out), _stream()),
           "qspec_attention")


def rope_attention(qkv, seq, pos, q_out, kcache, vcache, out, n_heads, n_kv, rope_base):
    """rope_kv then attention in one launch; the rows must belong to
    different sequences (one row per sequence)"""
    _dev(qkv, "qkv", torch.float32)
    _dev(q_out, "q_out", torch.float32)
    _dev(kcache, "kcache", torch.bfloat16)
    _dev(vcache, "vcache", torch.bfloat16)
    _dev(out, "out", torch.bfloat16)
    B, _, cap, _ = kcache.shape
    _check(lib().qspec_rope_attention(_ptr(qkv), int(qkv.shape[0]), n_heads, n_kv, _ptr(seq),
                                      _ptr(pos), float(rope_base), _ptr(q_out), _ptr(kcache),
                                      _ptr(vcache), B, cap, _ptr(out), _stream()),
           "qspec_rope_attention")


def silu_mul(gu, a):
    """a = bf16(silu(gate) * up); gu fp32 [M, 2F], a bf16 [M, F]"""
    _dev(gu, "gu", torch.float32)
    _dev(a, "a", torch.bfloat16)
    M, F = a.shape
    _check(lib().qspec_silu_mul(_ptr(gu), M, F, _ptr(a), _stream()), "qspec_silu_mul")


def silu_mul_pairs(gu, a):
    """silu_mul over gate|up outputs in pair order (the columns of a layer
    whose rows are in pair_rows order); gu fp32 [M, 2F], a bf16 [M, F]"""
    _dev(gu, "gu", torch.float32)
    _dev(a, "a", torch.bfloat16)
    M, F = a.shape
    _check(lib().qspec_silu_mul_pairs(_ptr(gu), M, F, _ptr(a), _stream()), "qspec_silu_mul_pairs")


def argmax(x, out, out_stride=1):
    """out[m * out_stride] = first index of the row maximum of x fp32 [M, V]"""
    _need(x, "x", torch.float32)
    _dev(out, "out", torch.int32)
    M, V = x.shape
    _check(lib().qspec_argmax(_ptr(x), M, V, _ptr(out), int(out_stride), _stream()),
           "qspec_argmax")


def spec_prepare(phase, B, gamma, j, len_, vtok, drafts, seq, pos, tok):
    _check(lib().qspec_spec_prepare(int(phase), int(B), int(gamma), int(j), _ptr(len_),
                                    _ptr(vtok), _ptr(drafts), _ptr(seq), _ptr(pos), _ptr(tok),
                                    _stream()), "qspec_spec_prepare")


def spec_commit(B, gamma, n_accept, out_tok, len_, vtok, vtok_stride, gen, n_gen, max_gen, stats):
    _dev(gen, "gen", torch.int32)
    _dev(stats, "stats", torch.int64)
    _check(lib().qspec_spec_commit(int(B), int(gamma), _ptr(n_accept), _ptr(out_tok), _ptr(len_),
                                   _ptr(vtok), int(vtok_stride), _ptr(gen), int(gen.shape[1]),
                                   _ptr(n_gen), int(max_gen), _ptr(stats), _stream()),
           "qspec_spec_commit")


# ---------------------------------------------------------------- ceiling probes
def probe_read(buf, blocks, unroll, sink):
    """read every byte of the device tensor `buf` once (see qspec_probe.h)"""
    _check(lib().qspec_probe_read(_ptr(buf), buf.numel() * buf.element_size(), int(blocks),
                                  int(unroll), _ptr(sink), _stream()), "qspec_probe_read")


def probe_mfma(kind, blocks, iters, sink):
    """independent MFMA chains: kind 0 int8 16x16x64, 1 bf16 16x16x32"""
    _check(lib().qspec_probe_mfma(int(kind), int(blocks), int(iters), _ptr(sink), _stream()),
           "qspec_probe_mfma")


def probe_empty():
    _check(lib().qspec_probe_empty(_stream()), "qspec_probe_empty")
