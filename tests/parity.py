"""Acceptance rules for comparing the HIP path with the float64 oracle.

Selection: bit-exact block indices, except where the oracle's k'-th and
(k'+1)-th candidate scores differ by less than a relative 1e-4 (k' = k - |F|
scored picks).  Concretely a row is accepted when it equals the oracle, or when
it has the same size, contains every forced block, and every block in the
symmetric difference scores within a relative 1e-4 of the oracle's k'-th best
candidate score (so a swap can only happen across such a near-tie).

Outputs: |gpu - oracle| <= atol + rtol * |oracle| with (2e-2, 1e-2) for bf16
inputs and (1e-5, 1e-5) for fp32 inputs; the oracle output is evaluated on
the GPU's accepted selection.
"""
from __future__ import annotations

import numpy as np

SELECT_BAND = 1e-4
TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-5, 1e-5)}


def kth_candidate_score(rs) -> float:
    cand = np.nonzero(~rs.forced)[0]
    sc = np.sort(rs.S[cand])[::-1]
    return float(sc[rs.kprime - 1]) if rs.kprime > 0 else float("nan")


def accept_selection(gpu_row: np.ndarray, rs, band: float = SELECT_BAND) -> str:
    """'exact', 'band' (accepted near-tie swap) or a failure description."""
    gpu_row = np.asarray(gpu_row, dtype=np.int64)
    ora = rs.sel
    if np.array_equal(gpu_row, ora):
        return "exact"
    g = gpu_row[gpu_row >= 0]
    o = ora[ora >= 0]
    if g.shape != o.shape or np.any(gpu_row[g.shape[0]:] != -1):
        return f"fail: size/padding gpu={gpu_row.tolist()} oracle={ora.tolist()}"
    if np.any(np.diff(g) <= 0):
        return f"fail: not ascending {g.tolist()}"
    if rs.dense:
        return f"fail: dense row differs gpu={g.tolist()}"
    if np.any(g > rs.S.shape[0] - 1) or np.any(g < 0):
        return f"fail: out-of-range block {g.tolist()}"
    forced = np.nonzero(rs.forced)[0]
    if not set(forced.tolist()) <= set(g.tolist()):
        return "fail: forced block missing"
    t = kth_candidate_score(rs)
    for j in set(g.tolist()) ^ set(o.tolist()):
        sj = rs.S[j]
        if np.isinf(t) or t == 0.0:
            if sj != t:
                return f"fail: block {j} score {sj} vs boundary {t}"
        elif abs(sj - t) > band * abs(t):
            return f"fail: block {j} score {sj} outside band of boundary {t}"
    return "band"


def assert_close(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    atol, rtol = TOL[dtype]
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref) - (atol + rtol * np.abs(ref))
    worst = float(np.max(err)) if err.size else -1.0
    assert worst <= 0.0, f"{what}: allclose violated by {worst:.3e} (max abs err {np.max(np.abs(gpu - ref)):.3e})"
    return float(np.max(np.abs(gpu - ref))) if err.size else 0.0
