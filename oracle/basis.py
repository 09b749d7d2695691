"""Gram matrix of a KV stream, from which the rotation basis is refreshed.  TEST INFRASTRUCTURE ONLY.

The pages (arXiv 2607.00760, section 1, Observation & Approach 1) rotate every KV vector by an SVD basis and
compute it off the decoding path (Observation & Approach 2).  The right singular vectors of a stream X [n][d]
are the eigenvectors of X^T X; the oracle computes X^T X as written, in float64.
"""
from __future__ import annotations

import numpy as np


def gram(x: np.ndarray) -> np.ndarray:
    """X^T X of the exact stored values x [n][d] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    return x.T @ x


def gram_abs(x: np.ndarray) -> np.ndarray:
    """|X|^T |X|: the scale of each entry's summands, for rounding-error bounds of a float32 sum."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    return x.T @ x
