"""Error measures used by the parity tests (no attention arithmetic here)."""

import numpy as np


def max_abs(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.max(np.abs(x - ref))) if x.size else 0.0


def mean_abs(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.mean(np.abs(x - ref))) if x.size else 0.0


def rel_frobenius(x, ref) -> float:
    """||x - ref||_F / ||ref||_F over the whole tensor (all batches and heads)."""
    x = np.asarray(x, dtype=np.float64)
    den = float(np.linalg.norm(np.asarray(ref, dtype=np.float64).ravel()))
    return float(np.linalg.norm((x - ref).ravel())) / den


# Tolerances: fp32 path max-abs 1e-5 (O and LSE); bf16 path O max-abs 1e-2 and
# mean-abs 1e-3, LSE max-abs 1e-3; gradients relative Frobenius 2e-2 (bf16)
# and 1e-5 (fp32 at small sizes).
TOL_F32 = 1e-5
TOL_BF16_O_MAX = 1e-2
TOL_BF16_O_MEAN = 1e-3
TOL_BF16_LSE_MAX = 1e-3
TOL_BF16_GRAD_REL = 2e-2
TOL_F32_GRAD_REL = 1e-5
