"""Helpers shared by the GPU parity tests."""
import numpy as np

from synth.inputs import Inputs, make_inputs  # noqa: F401


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over (row, head) of max|g - r| / max|r| (rows with an all-zero reference use abs)."""
    g = got.reshape(-1, got.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    num = np.abs(g - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())
