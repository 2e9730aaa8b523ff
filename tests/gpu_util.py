"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

import oracle as O


def dev_bf16(u16, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(device)


def dev(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bits(t):
    """bf16 tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def vals(t):
    """bf16 tensor -> float64 values."""
    return O.bits_to_f64(bits(t))


def host(t):
    return t.detach().cpu().numpy()


def poison_bf16(shape, device="cuda"):
    """Output buffer pre-filled with a signalling-NaN bf16 pattern, so that any
    element a kernel fails to write shows up."""
    return torch.full(shape, 0x7FA0, dtype=torch.int16, device=device).view(torch.bfloat16)


def assert_bf16_close(got, ref, what=""):
    """max|gpu - ref| <= 1e-2 * max|ref| + 1e-3 (fp32 accumulation against the
    float64 oracle)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    tol = 1e-2 * (np.max(np.abs(ref)) if ref.size else 0.0) + 1e-3
    assert err <= tol, f"{what}: max|diff| {err:.3e} > tol {tol:.3e}"


def rel_frobenius(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (n if n > 0 else 1.0)
