"""Helpers for the GPU parity tests: move seeded 16-bit inputs to the device and compare
with the oracle under the acceptance bound |O - O_ref| <= 2e-2 + 1e-2 |O_ref| (16-bit O)
and |LSE - LSE_ref| <= 1e-3 (fp32 LSE)."""
import numpy as np
import torch

from attn_inputs import BF16, bits_to_f64

O_ATOL, O_RTOL, LSE_ATOL = 2e-2, 1e-2, 1e-3


def tdtype(dtype):
    return torch.bfloat16 if dtype == BF16 else torch.float16


def to_dev(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(tdtype(dtype)).cuda()


def from_dev_f64(t):
    """16-bit device tensor -> float64 numpy (exact widening)."""
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    dt = BF16 if t.dtype == torch.bfloat16 else 1
    return bits_to_f64(bits, dt)


def bits_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_parity(O, O_ref, L=None, L_ref=None, what=""):
    O = np.asarray(O, np.float64)
    O_ref = np.asarray(O_ref, np.float64)
    assert np.all(np.isfinite(O)), f"{what}: non-finite output"
    err = np.abs(O - O_ref)
    bound = O_ATOL + O_RTOL * np.abs(O_ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outputs outside the bound; "
                           f"max err {err.max():.3e}")
    if L is not None:
        L = np.asarray(L, np.float64)
        lerr = np.abs(L - np.asarray(L_ref, np.float64))
        assert np.all(lerr <= LSE_ATOL), f"{what}: LSE max err {lerr.max():.3e}"
    return float(err.max())
