"""One decode step over the compressed store.  TEST INFRASTRUCTURE ONLY.

Follows the pages (arXiv 2607.00760, section 1): sequence compression selects a subset of the historical
tokens per query at run time (the prior-work paragraph, query-aware token selection), MosaicKV keeps both
keys and values two-D compressed through selection and attention (Challenge 1, Observation & Approach 1),
and attention runs directly on the packed sparse K/V without unpacking them to dense form
(Observation & Approach 2, compact sparse attention).  The pages leave the estimator and the budget open;
the readings taken are:

* queries are rotated by the key basis (q' = q @ B_K) so that q'.k_hat estimates q.k;
* the score of token j for a KV group is s_j = sum over its kept channels of Qbar_i * k_hat_j,i, where Qbar
  is the sum of the group's rotated queries;
* the T largest scores (ties -> lower token index) form the selected set, T clamped to the context;
* each query head takes the exact softmax of q'.k_hat_j / sqrt(d) over the selected tokens (dropped channels
  count as 0) and the weighted sum of their sparse values; the result is rotated back by B_V^T.
"""
from __future__ import annotations

import numpy as np

from .compress import Stream


def rotate_queries(q: np.ndarray, basis_k: np.ndarray | None) -> np.ndarray:
    q = np.asarray(q, dtype=np.float64)
    return q if basis_k is None else q @ np.asarray(basis_k, dtype=np.float64)


def scores(qbar: np.ndarray, kstream: Stream) -> np.ndarray:
    """s_j = sum over the kept channels i of token j of Qbar_i * k_hat_j,i (float64)."""
    return np.where(kstream.mask, kstream.vals, 0.0) @ np.asarray(qbar, dtype=np.float64)


def select_top(s: np.ndarray, T: int) -> np.ndarray:
    """Indices of the T largest scores, larger score first and lower index first among equal scores,
    returned in ascending index order.  T is clamped to the number of tokens."""
    n = s.shape[0]
    t = min(int(T), n)
    order = np.lexsort((np.arange(n), -np.asarray(s, dtype=np.float64)))
    return np.sort(order[:t])


def attend(qp: np.ndarray, kvals: np.ndarray, vvals: np.ndarray) -> np.ndarray:
    """Exact softmax attention of the rotated queries qp [G][d] over the rows kvals/vvals [t][d]."""
    d = qp.shape[1]
    logits = (qp @ kvals.T) / np.sqrt(d)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ vvals


def decode_unit(q: np.ndarray, basis_k, basis_v, kstream: Stream, vstream: Stream, T: int) -> dict:
    """Decode step of one (request, KV group): q [G][d] holds the exact query values of the group."""
    qp = rotate_queries(q, basis_k)
    qbar = qp.sum(axis=0)
    s = scores(qbar, kstream)
    sel = select_top(s, T)
    G, d = qp.shape
    if sel.size == 0:
        out = np.zeros((G, d))
    else:
        o = attend(qp, kstream.vals[sel], vstream.vals[sel])
        out = o if basis_v is None else o @ np.asarray(basis_v, dtype=np.float64).T
    return {"out": out, "sel": sel, "scores": s, "qbar": qbar}


def dense_decode_unit(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """The uncompressed baseline the pages compare against (section 1, Observation & Approach 2): exact softmax
    attention of the group's queries q [G][d] over every stored token's full key and value rows k, v [n][d]
    (no rotation, no selection).  An empty context gives zeros."""
    q = np.asarray(q, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros_like(q)
    return attend(q, np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64))


def decode_all(inputs, streams: dict, units=None) -> dict:
    """Decode step for every (request, KV group) of a ``workloads.Inputs`` whose compressed streams are in
    ``streams`` ({(r, h, X): Stream}).  Returns {(r, h): decode_unit result}."""
    from workloads import to_f64
    w = inputs.workload
    G = w.group
    res = {}
    for r in range(w.batch):
        for h in range(w.n_kv_heads):
            if units is not None and (r, h) not in units:
                continue
            q = to_f64(inputs.q[r, h * G:(h + 1) * G, :], inputs.dtype)
            bk = None if inputs.basis is None else inputs.basis[r, h, 0]
            bv = None if inputs.basis is None else inputs.basis[r, h, 1]
            res[(r, h)] = decode_unit(q, bk, bv, streams[(r, h, 0)], streams[(r, h, 1)], int(inputs.T[r]))
    return res
