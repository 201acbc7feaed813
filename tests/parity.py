"""Comparison rules shared by the parity tests (GPU path vs fp64 oracle).

Floating-point outputs: max |gpu - oracle| and mean |gpu - oracle| over the
valid rows and all d; bf16 inputs need max <= 3e-2 and mean <= 3e-3, fp32
inputs <= 1e-4 for both.

Block indices: per query-cube row, let tK and tK1 be the oracle's K-th and
(K+1)-th largest coarse scores and eps = 1e-4 * max(|tK|, |tK1|, 1e-3*rms(row)).
If tK - tK1 > eps the GPU row must equal the oracle row exactly; otherwise it
must hold K distinct ascending indices and every index in which the two rows
differ must score within eps of tK.
"""
from __future__ import annotations

import numpy as np

TOL = {"bf16": (3e-2, 3e-3), "f32": (1e-4, 1e-4)}

# Largest errors measured in this session per (quantity, dtype): the test
# session prints them at its end next to the tolerances.
WORST: dict = {}


def assert_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str, rows=None):
    """gpu/ref: (..., rows, d); rows: optional boolean mask over the row axis."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if rows is not None:
        gpu = gpu[..., rows, :]
        ref = ref[..., rows, :]
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(ref)), f"{what}: reference has non-finite values"
    err = np.abs(gpu - ref)
    if not np.all(np.isfinite(gpu)):
        raise AssertionError(f"{what}: GPU output has non-finite values")
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    tmax, tmean = TOL[dtype]
    key = (what, dtype)
    prev = WORST.get(key, (0.0, 0.0, 0))
    WORST[key] = (max(prev[0], mx), max(prev[1], mean), prev[2] + 1)
    assert mx <= tmax and mean <= tmean, (
        f"{what}: max|err|={mx:.3e} (tol {tmax:g}), mean|err|={mean:.3e} (tol {tmean:g})")
    return mx, mean


def check_idx(gpu_idx: np.ndarray, ref_idx: np.ndarray, scores: np.ndarray, K: int):
    """Applies the near-tie rule row by row.  Returns the number of near-tie rows."""
    C = scores.shape[-1]
    g = gpu_idx.reshape(-1, K)
    r = ref_idx.reshape(-1, K)
    s = scores.reshape(-1, C)
    near = 0
    for row in range(g.shape[0]):
        gi, ri, sc = g[row], r[row], s[row]
        assert np.all((gi >= 0) & (gi < C)), f"row {row}: index out of range {gi}"
        assert np.all(np.diff(gi) > 0), f"row {row}: not strictly ascending {gi}"
        if K == C:
            assert np.array_equal(gi, np.arange(C)), f"row {row}: K = C must keep every cube"
            continue
        srt = np.sort(sc)[::-1]
        tk, tk1 = srt[K - 1], srt[K]
        rms = np.sqrt(np.mean(sc * sc))
        eps = 1e-4 * max(abs(tk), abs(tk1), 1e-3 * rms)
        if tk - tk1 > eps:
            assert np.array_equal(gi, ri), f"row {row}: {gi} != oracle {ri}"
        else:
            near += 1
            diff = np.setxor1d(gi, ri)
            assert np.all(np.abs(sc[diff] - tk) <= eps), (
                f"row {row}: differing indices {diff} are not near-ties of the K-th score")
    return near


def valid_rows(geometry) -> np.ndarray:
    """Boolean mask over cube-order rows: True for real tokens."""
    return geometry["valid"]
