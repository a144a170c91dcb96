"""Comparison rules between the HIP path and the CPU oracle, and a small device
harness used by the GPU tests (uploads synth cases, runs libqsa calls)."""
from __future__ import annotations

import numpy as np

# outputs: |gpu - oracle| <= ATOL + RTOL |oracle|; selections: symmetric difference only
# among blocks whose oracle score lies within SWAP_REL of the oracle's k-th score
ATOL = 1e-2
RTOL = 1e-2
SWAP_REL = 1e-4


def check_close(gpu, ref, what: str):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref) - (ATOL + RTOL * np.abs(ref))
    if np.any(err > 0):
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: {int((err > 0).sum())} of {err.size} outside tolerance; worst at {i}: "
                             f"gpu {gpu[i]} oracle {ref[i]}")


def tol_ratio(gpu, ref) -> float:
    """The largest |gpu - oracle| / (ATOL + RTOL |oracle|) over the finite entries:
    the share of the output tolerance that the GPU result uses (1 = at the bound)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    if not np.any(fin):
        return 0.0
    return float(np.max(np.abs(gpu[fin] - ref[fin]) / (ATOL + RTOL * np.abs(ref[fin]))))


def check_lse(gpu, ref, what: str):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    gi, ri = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(gi, ri), f"{what}: -inf pattern differs ({int(gi.sum())} vs {int(ri.sum())})"
    check_close(gpu[~ri], ref[~ri], what)


def kth_score(scores: np.ndarray, k: int) -> float:
    m = min(k, len(scores))
    return float(np.sort(scores)[::-1][m - 1])


def check_selection(gsel, gcnt: int, osel, ocnt: int, oscores, k: int, what: str) -> bool:
    """True if the sets are equal; False if they differ only by allowed swaps."""
    gsel = np.asarray(gsel)
    assert gcnt == ocnt, f"{what}: count {gcnt} vs oracle {ocnt}"
    g = gsel[:gcnt]
    assert np.all(np.diff(g) > 0), f"{what}: selection not strictly ascending"
    assert np.all(gsel[gcnt:k] == -1), f"{what}: padding is not -1"
    G, O = set(g.tolist()), set(np.asarray(osel)[:ocnt].tolist())
    if G == O:
        return True
    sk = kth_score(np.asarray(oscores), k)
    for b in G ^ O:
        assert abs(oscores[b] - sk) <= SWAP_REL * abs(sk), \
            f"{what}: block {b} score {oscores[b]} vs k-th {sk} beyond the swap window"
    return False


def score_bound(q_group_f64: np.ndarray, ckey: np.ndarray) -> np.ndarray:
    """Forward error bound of an fp32 score: gamma_n * sum_d sum_j |q_jd| |ckey_d|
    with n = g + 256 + 2 and u = 2^-24 (summing the group, then the dot product)."""
    g = q_group_f64.shape[0]
    n = g + ckey.shape[1] + 2
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    return gamma * (np.abs(ckey).astype(np.float64) @ np.abs(q_group_f64).sum(axis=0))
