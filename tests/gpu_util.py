"""Helpers for the GPU parity tests: numpy <-> device tensors and the tolerance."""

import sys

import numpy as np
import torch

DEV = "cuda:0"
FP_REL_TOL = 2e-3   # max|err| <= 2e-3 * max|y| for floating-point outputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev_f16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(DEV)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def host_bits16(t):
    torch.cuda.synchronize()
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def assert_close(got, want, tol=FP_REL_TOL, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    scale = np.abs(want).max()
    err = np.abs(got - want).max()
    assert err <= tol * scale + 1e-30, f"{what}: max|err| {err:.3e} > {tol} * max|y| {scale:.3e}"
    return err / max(scale, 1e-300)
