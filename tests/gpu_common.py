"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import pytest
import torch

import moe_expert_dispatch_amd as moe

# Output tolerances: fp32 1e-4 relative; bf16 2e-2 relative / 1e-2 absolute,
# applied elementwise as |got - ref| <= atol + rtol * |ref|.
F32_TOL = (1e-4, 1e-5)
BF16_TOL = (2e-2, 1e-2)


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    moe.lib()  # raises if the HIP library is missing: no fallback
    return torch.device("cuda:0")


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def assert_close(got, ref, tol, what=""):
    rtol, atol = tol
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    excess = np.abs(got - ref) - (atol + rtol * np.abs(ref))
    if not (excess <= 0).all():
        i = np.unravel_index(np.nanargmax(np.where(np.isnan(excess), np.inf, excess)), excess.shape)
        raise AssertionError(
            f"{what}: {int((~(excess <= 0)).sum())} of {excess.size} elements out of tolerance; "
            f"worst at {i}: got {got[i]!r}, ref {ref[i]!r}")


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.int32)
