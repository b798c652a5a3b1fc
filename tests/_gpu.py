"""Helpers for the GPU parity tests (imported only by tests marked gpu)."""
import sys

import numpy as np


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def dev(a: np.ndarray):
    """Copy a numpy array to the current device (uint16 travels as int16 bits)."""
    torch = torch_cuda()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t) -> np.ndarray:
    torch = torch_cuda()
    torch.cuda.synchronize()
    return t.cpu().numpy()


def half_bits(t) -> np.ndarray:
    """A float16/int16 device tensor as uint16 bit patterns on the host."""
    return host(t).view(np.uint16)


def within(y_gpu, y_ref, S, tol, what=""):
    """Assert |y_gpu - y_ref| <= tol * S elementwise (S = 0 forces equality).
    Returns the largest |err| / S seen, for the log."""
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref)
    # written as "not within" so that a NaN or infinite result counts as bad
    bad = ~(err <= tol * S)
    if np.any(bad):
        excess = np.where(bad, np.nan_to_num(err - tol * S, nan=np.inf, posinf=np.inf), -np.inf)
        i = np.unravel_index(np.argmax(excess), err.shape)
        raise AssertionError(
            "%s: %d of %d outputs outside %.1e*S; worst at %s: gpu %.9g ref %.9g S %.6g"
            % (what, int(bad.sum()), bad.size, tol, i, y_gpu[i], y_ref[i], S[i]))
    pos = S > 0
    return float((err[pos] / S[pos]).max()) if np.any(pos) else 0.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
