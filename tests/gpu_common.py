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


def assert_close(got, ref, tol, what="", extra=None):
    """|got - ref| <= atol + rtol * |ref| (+ extra, a per-element allowance
    derived elsewhere) for every element."""
    rtol, atol = tol
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    excess = np.abs(got - ref) - (atol + rtol * np.abs(ref))
    if extra is not None:
        excess = excess - np.asarray(extra, dtype=np.float64)
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


# Row tiles of the grouped GEMMs are 256 rows of one slot, counted from the
# slot's first row; each is computed by two 128-row halves (different waves).
TILE_HALF_ROWS = 128


def covering_tokens(offsets, sorted_pairs, pair_row, K, seed=0, block=TILE_HALF_ROWS):
    """Tokens whose pairs put at least one sampled row in every `block`-row
    piece of every slot (counted from the slot's first row), plus the token
    of each slot's last row: a sample that reaches every GEMM work item and
    every ragged tail. Greedy over the pieces in a seeded random order."""
    off = np.asarray(offsets, dtype=np.int64)
    sp = np.asarray(sorted_pairs, dtype=np.int64)
    pr = np.asarray(pair_row, dtype=np.int64)
    rng = np.random.default_rng(seed)
    piece_lo, piece_hi = [], []
    for s in range(off.size - 1):
        for lo in range(int(off[s]), int(off[s + 1]), block):
            piece_lo.append(lo)
            piece_hi.append(min(lo + block, int(off[s + 1])))
    piece_lo = np.asarray(piece_lo, dtype=np.int64)
    piece_hi = np.asarray(piece_hi, dtype=np.int64)
    covered = np.zeros(piece_lo.size, dtype=bool)

    def mark(t):
        rows = pr[t * K:(t + 1) * K]
        rows = rows[rows >= 0]
        covered[np.searchsorted(piece_lo, rows, side="right") - 1] = True

    chosen = set()
    for b in rng.permutation(piece_lo.size):
        if covered[b]:
            continue
        t = int(sp[rng.integers(piece_lo[b], piece_hi[b])] // K)
        chosen.add(t)
        mark(t)
    for s in range(off.size - 1):
        if off[s + 1] > off[s]:
            chosen.add(int(sp[off[s + 1] - 1] // K))
    assert covered.all()
    return np.asarray(sorted(chosen), dtype=np.int64)
