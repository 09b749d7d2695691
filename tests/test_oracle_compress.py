"""Pins of the oracle's compression steps: brute force on tiny vectors, constructed vectors whose strategy the
energy rule fixes by hand, exact-arithmetic bases, and the stored-bytes closed form."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import (Policy, channel_order, compress_stream, kept_energy, rotate_round, vector_min_keep)
from oracle.sizes import counted_payload_bytes, dense_kv_bytes, stream_payload_bytes

D8 = Policy(seg_len=4, keep=(8, 4, 2), energy_frac=0.9)


def _beats(x, i, j):
    """Channel i ranks before channel j: larger magnitude, or equal magnitude and lower index."""
    return abs(x[i]) > abs(x[j]) or (abs(x[i]) == abs(x[j]) and i < j)


def _brute_topc(x, c):
    d = len(x)
    found = [set(S) for S in itertools.combinations(range(d), c)
             if all(_beats(x, i, j) for i in S for j in range(d) if j not in S)]
    assert len(found) == 1
    return found[0]


def _brute_energy(x, c):
    return max(sum(x[i] * x[i] for i in S) for S in itertools.combinations(range(len(x)), c))


def _tiny_vectors(seed, n):
    rng = np.random.default_rng(seed)
    # small integers (many exact ties, zeros and sign pairs) plus a few continuous rows
    a = rng.integers(-3, 4, size=(n, 8)).astype(np.float64)
    a[: n // 4] = rng.standard_normal((n // 4, 8))
    return a


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topc_set_matches_brute_force(seed):
    xs = _tiny_vectors(seed, 60)
    order = channel_order(xs)
    for x, o in zip(xs, order):
        for c in (1, 2, 3, 4, 5, 8):
            assert set(o[:c].tolist()) == _brute_topc(x, c)


@pytest.mark.parametrize("seed", [3, 4])
def test_kept_energy_is_the_best_subset_energy(seed):
    xs = _tiny_vectors(seed, 60)
    order = channel_order(xs)
    for c in (2, 4, 8):
        e = kept_energy(xs, order, c)
        for x, ec in zip(xs, e):
            assert ec == pytest.approx(_brute_energy(x, c), rel=0, abs=1e-12)


@pytest.mark.parametrize("seed", [5, 6])
def test_vector_min_keep_brute_force(seed):
    xs = _tiny_vectors(seed, 80)
    got = vector_min_keep(xs, D8)
    for x, g in zip(xs, got):
        total = float(np.sum(x * x))
        admissible = [c for c in D8.keep if _brute_energy(x, c) >= 0.9 * total]
        assert g == min(admissible)


def _seg_code(rows, policy=Policy()):
    st = compress_stream(np.asarray(rows, dtype=np.float64), None, "fp32", policy)
    return st


def test_flat_vector_needs_all_channels():
    flat = np.where(np.arange(128) % 2 == 0, 1.0, -1.0)
    # top-64 energy is exactly half the total: below 0.9, so nothing can be dropped
    assert vector_min_keep(flat[None, :])[0] == 128


def test_sparse_and_zero_vectors_take_smallest():
    sparse = np.zeros(128)
    sparse[np.random.default_rng(0).choice(128, 32, replace=False)] = 5.0
    assert vector_min_keep(sparse[None, :])[0] == 32
    assert vector_min_keep(np.zeros((1, 128)))[0] == 32


def test_exact_threshold_is_admissible():
    x = np.zeros(128)
    x[:32] = 3.0
    x[32:64] = 1.0
    # E_32 = 288, E_all = 320, 0.9 * 320 rounds to exactly 288 in float64
    assert 0.9 * 320.0 == 288.0
    assert vector_min_keep(x[None, :])[0] == 32
    y = x.copy()
    y[64] = 2.0 ** -20      # a hair more total energy: 32 no longer admissible
    assert vector_min_keep(y[None, :])[0] == 64


def test_boundary_tie_keeps_lowest_channels():
    rng = np.random.default_rng(7)
    big = rng.choice(128, 31, replace=False)
    rest = np.setdiff1d(np.arange(128), big)
    ties = np.sort(rng.choice(rest, 10, replace=False))
    x = np.zeros(128)
    x[big] = 4.0
    x[ties] = np.where(rng.random(10) < 0.5, 0.5, -0.5)
    st = _seg_code([x])
    assert st.c[0] == 32
    kept = set(np.nonzero(st.mask[0])[0].tolist())
    assert kept == set(big.tolist()) | {int(ties[0])}


def test_one_flat_vector_sets_its_segment_only():
    rng = np.random.default_rng(8)
    n = 64 * 3 + 5
    x = np.zeros((n, 128))
    x[:, :20] = rng.standard_normal((n, 20)) * 10   # 20 strong channels: every vector admits 32
    flat = np.where(np.arange(128) % 2 == 0, 1.0, -1.0)
    x[70] = flat
    st = _seg_code(x)
    assert st.c.tolist() == [32, 128, 32, 32]
    assert st.mask[64:128].all()
    assert st.mask.sum(axis=1)[:64].tolist() == [32] * 64
    assert st.mask.sum(axis=1)[192:].tolist() == [32] * 5     # partial last segment


def test_segment_takes_the_largest_vector_need():
    x = np.zeros((64, 128))
    x[:, 0] = 1.0                       # every vector admits 32 ...
    x[5, :48] = 1.0                     # ... except one that needs 64 (E_32/E_all = 32/48 < 0.9)
    st = _seg_code(x)
    assert st.c.tolist() == [64]


def test_signed_permutation_rotation_is_exact():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((50, 128)).astype(np.float32).astype(np.float64)
    perm = rng.permutation(128)
    sign = rng.choice([-1.0, 1.0], 128)
    b = np.zeros((128, 128))
    b[np.arange(128), perm] = sign
    y = rotate_round(x, b, "fp32")
    expect = np.zeros_like(x)
    expect[:, perm] = x * sign
    np.testing.assert_array_equal(y, expect)


def test_rotation_preserves_dot_products():
    rng = np.random.default_rng(10)
    qmat, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    q = rng.standard_normal((4, 128))
    k = rng.standard_normal((30, 128))
    lhs = (q @ qmat) @ (k @ qmat).T
    np.testing.assert_allclose(lhs, q @ k.T, rtol=0, atol=1e-12)
    # stored values undo to the input within one storage rounding per element
    kh = rotate_round(k, qmat, "bf16")
    back = kh @ qmat.T
    assert np.max(np.abs(back - k)) <= 2.0 ** -8 * np.max(np.abs(k @ qmat)) * 12


def test_payload_closed_form_matches_token_count():
    rng = np.random.default_rng(11)
    for n in (1, 63, 64, 65, 200):
        x = rng.standard_normal((n, 128)) * (np.arange(128) + 1.0) ** -1.5
        x[rng.integers(0, n)] *= 0.0
        for dt, bv in (("bf16", 2), ("fp32", 4)):
            st = compress_stream(x, None, dt)
            assert stream_payload_bytes(st.c, n, 64, 128, bv) == counted_payload_bytes(st, bv, 64)


def test_dense_kv_size_matches_the_pages():
    with open(os.path.join(os.path.dirname(__file__), "golden", "kv_cache_size.json")) as f:
        g = json.load(f)
    m = g["model"]
    for case in g["cases"]:
        got = dense_kv_bytes(case["requests"] * case["tokens_per_request"], m["n_kv_heads"], m["head_dim"],
                             m["bytes_per_value"], layers=m["layers"])
        assert got == case["bytes"]
    # 128 KiB per token across the model: the figure behind both printed totals
    assert dense_kv_bytes(1, 8, 128, 2, 32) == 128 * 1024
