"""Helpers shared by the GPU parity tests: host<->device copies into the
pitched layouts the ABI wants, and the comparison rules (bit-exact for
integers and quantization scales; relative error <= 1e-6 for fp32 y)."""
import numpy as np
import torch

from bitlinear_matmul_amd import ug

Y_RTOL = 1e-6  # fp32 output tolerance (the stated epilogue is expected exact)


def dev():
    return torch.device("cuda:0")


def pitched(a, align_bytes=16):
    """Copy a 2-D numpy array to the GPU as a [rows, cols] view of a pitched
    allocation (row pitch a multiple of align_bytes)."""
    a = np.ascontiguousarray(a)
    t = ug.empty_pitched(a.shape[0], a.shape[1], getattr(torch, str(a.dtype)), dev(), align_bytes)
    t.copy_(torch.from_numpy(a))
    return t


def vec(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def scalar_dev(v, dtype=np.float32):
    return vec(np.array([v], dtype))


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype.kind == "f":
        eq = got.view(np.uint32 if got.dtype == np.float32 else np.uint64) == \
            want.view(np.uint32 if want.dtype == np.float32 else np.uint64)
    else:
        eq = got == want
    if not eq.all():
        idx = np.argwhere(~eq)
        i = tuple(idx[0])
        raise AssertionError("%s: %d of %d differ; first at %s: got %r want %r"
                             % (what, idx.shape[0], eq.size, i, got[i], want[i]))


def assert_y_close(got, want, what, rtol=Y_RTOL):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape
    err = np.abs(got - want)
    tol = rtol * np.abs(want)
    bad = err > tol
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d elements beyond rel %g; first at %s: got %r want %r"
                             % (what, int(bad.sum()), rtol, i, got[i], want[i]))
