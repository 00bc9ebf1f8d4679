"""Tolerances of the parity tests (float results against the float64 oracle).

GEMV: max over outputs of |gpu - ref| / max(|ref|, 1e-3) <= 2e-3 (the 1e-3
floor is on the denominator; the looser reading |gpu - ref| <= 1e-3 +
2e-3 |ref| is reported beside it).  Attention: max |gpu - ref| <= 3e-3.
Logits: max |gpu - ref| <= 5e-2 with identical greedy tokens.
"""
import numpy as np

GEMV_RTOL, GEMV_FLOOR = 2e-3, 1e-3
ATTN_ATOL = 3e-3
LOGIT_ATOL = 5e-2


def gemv_rel_err(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), GEMV_FLOOR))) if r.size else 0.0


def gemv_allclose_err(gpu, ref) -> float:
    """Largest |g - r| / (1e-3 + 2e-3 |r|): <= 1 passes the looser reading."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(g - r) / (GEMV_FLOOR + GEMV_RTOL * np.abs(r)))) if r.size else 0.0


def assert_gemv(gpu, ref, what=""):
    e = gemv_rel_err(gpu, ref)
    assert e <= GEMV_RTOL, f"{what}: GEMV max rel err {e:.3e} > {GEMV_RTOL} (allclose reading {gemv_allclose_err(gpu, ref):.3f})"
    return e


def assert_attn(gpu, ref, what=""):
    e = float(np.max(np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))))
    assert e <= ATTN_ATOL, f"{what}: attention max abs err {e:.3e} > {ATTN_ATOL}"
    return e
