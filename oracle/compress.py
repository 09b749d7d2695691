"""Dynamic two-D compression of one (request, KV head, tensor) stream.  TEST INFRASTRUCTURE ONLY.

Follows the pages (arXiv 2607.00760, section 1, Observation & Approach 1): after an SVD rotation the
importance of elements differs from vector to vector, so each KV vector keeps its own important elements
(per-vector element selection), and the cache is cut into segments that each get their own compression
strategy (dynamic compression strategy).  The pages leave the strategy set, the segment size and the
importance measure open; the readings taken are:

* importance of an element = magnitude of its stored rotated value; equal magnitudes -> lower channel first;
* strategies = kept-channel counts ``policy.keep`` (default 128, 64, 32, i.e. ratios 1, 1/2, 1/4);
* a vector admits keeping c channels when its c largest elements hold at least ``energy_frac`` (0.9) of its
  squared L2 norm (float64 sums, comparison ``E_c >= energy_frac * E_all``); a zero vector admits any c;
* a segment (``seg_len`` = 64 consecutive tokens from token 0; the last one may be shorter) takes the
  smallest c that every vector in it admits;
* each token then stores its c kept channels in ascending channel order together with their values.

Steps are written in that order, each as a small function.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .rounding import rne


@dataclass(frozen=True)
class Policy:
    seg_len: int = 64
    keep: tuple = (128, 64, 32)     # strictly decreasing; keep[0] is the head dimension (nothing dropped)
    energy_frac: float = 0.9


DEFAULT_POLICY = Policy()


@dataclass
class Stream:
    """Logical compressed form of one stream of n vectors of dimension d.

    codes[s]: index into policy.keep of segment s's kept-channel count; c[s] = policy.keep[codes[s]];
    mask[j, i]: channel i of token j is stored; vals[j, i]: its stored value (0 where not stored)."""

    n: int
    d: int
    codes: np.ndarray
    c: np.ndarray
    mask: np.ndarray
    vals: np.ndarray

    def kept_indices(self, j: int) -> np.ndarray:
        return np.nonzero(self.mask[j])[0]

    def segment_of(self, j: int, seg_len: int) -> int:
        return j // seg_len


# step 1: rotation by the SVD basis, rounded to the storage dtype -------------------------------------------
def rotate_round(x: np.ndarray, basis: np.ndarray | None, dtype: str) -> np.ndarray:
    """x_hat = round_dtype(x @ B) with the product in float64; ``basis=None`` means x is already rotated."""
    x = np.asarray(x, dtype=np.float64)
    if basis is None:
        return rne(x, dtype)
    return rne(x @ np.asarray(basis, dtype=np.float64), dtype)


# step 2: per-vector ranking of channels by importance --------------------------------------------------------
def channel_order(xhat: np.ndarray) -> np.ndarray:
    """Row-wise channel indices by decreasing |x_hat|; a stable sort keeps the lower channel first on ties
    (and -0 ties with +0, since abs makes both +0)."""
    return np.argsort(-np.abs(xhat), axis=1, kind="stable")


# step 3: energy kept by the top-c channels ---------------------------------------------------------------------
def kept_energy(xhat: np.ndarray, order: np.ndarray, c: int) -> np.ndarray:
    sq = np.take_along_axis(xhat * xhat, order, axis=1)
    return np.cumsum(sq, axis=1)[:, c - 1]


def vector_min_keep(xhat: np.ndarray, policy: Policy = DEFAULT_POLICY, order=None) -> np.ndarray:
    """For each vector, the smallest c in policy.keep it admits (E_c >= energy_frac * E_all)."""
    if order is None:
        order = channel_order(xhat)
    e_all = np.sum(xhat * xhat, axis=1)
    best = np.full(xhat.shape[0], max(policy.keep), dtype=np.int64)
    for c in sorted(policy.keep, reverse=True):        # later (smaller) admissible c overwrite larger ones
        ok = kept_energy(xhat, order, c) >= policy.energy_frac * e_all
        best = np.where(ok, c, best)
    return best


# step 4 + 5: one strategy per segment, then the kept set of every token ----------------------------------------
def compress_stream(x: np.ndarray, basis: np.ndarray | None, dtype: str,
                    policy: Policy = DEFAULT_POLICY) -> Stream:
    """Compress one stream x [n][d] (exact values of the stored inputs)."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    assert policy.keep[0] == d, "keep[0] must be the head dimension"
    xhat = rotate_round(x, basis, dtype)
    order = channel_order(xhat)
    vmin = vector_min_keep(xhat, policy, order)
    S = (n + policy.seg_len - 1) // policy.seg_len
    codes = np.zeros(S, dtype=np.int64)
    cs = np.zeros(S, dtype=np.int64)
    mask = np.zeros((n, d), dtype=bool)
    for s in range(S):
        lo, hi = s * policy.seg_len, min(n, (s + 1) * policy.seg_len)
        c = int(vmin[lo:hi].max())          # the smallest c every vector of the segment admits
        cs[s] = c
        codes[s] = policy.keep.index(c)
        rows = np.arange(lo, hi)[:, None]
        mask[rows, order[lo:hi, :c]] = True
    vals = np.where(mask, xhat, 0.0)
    return Stream(n, d, codes, cs, mask, vals)


def compress_all(inputs, policy: Policy = DEFAULT_POLICY, units=None) -> dict:
    """Compress every (request, KV head, tensor) stream of a ``workloads.Inputs`` (or the listed
    (r, h) units).  Returns {(r, h, X): Stream} with X = 0 for K, 1 for V."""
    from workloads import to_f64
    out = {}
    B, Hkv = inputs.workload.batch, inputs.workload.n_kv_heads
    cu = inputs.cu_seqlens
    for r in range(B):
        for h in range(Hkv):
            if units is not None and (r, h) not in units:
                continue
            for X, arr in ((0, inputs.K), (1, inputs.V)):
                x = to_f64(arr[cu[r]:cu[r + 1], h, :], inputs.dtype)
                b = None if inputs.basis is None else inputs.basis[r, h, X]
                out[(r, h, X)] = compress_stream(x, b, inputs.dtype, policy)
    return out
