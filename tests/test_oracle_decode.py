"""Pins of the oracle's decode step: brute-force top-T, the dense special case against torch's attention,
the single-token special case, and invariants that hold for any input."""
import itertools

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import (Policy, attend, compress_stream, decode_unit, rne, rotate_queries, scores, select_top)

ALL = Policy(keep=(128,))


def _brute_top(s, T):
    n = len(s)
    t = min(T, n)
    found = []
    for S in itertools.combinations(range(n), t):
        inside = set(S)
        if all((s[i] > s[j]) or (s[i] == s[j] and i < j) for i in inside for j in range(n) if j not in inside):
            found.append(sorted(S))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(6))
def test_select_top_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    for n in range(1, 12):
        s = rng.integers(-3, 4, n).astype(np.float64)
        if seed % 2:
            s = s + 0.25 * rng.standard_normal(n)
        for T in (1, 2, n // 2 + 1, n, n + 3):
            assert select_top(s, T).tolist() == _brute_top(s, T)


def test_select_top_negative_zero_ties_with_zero():
    s = np.array([-0.0, 0.0, -0.0, 1.0])
    assert select_top(s, 2).tolist() == [0, 3]


def _sdpa(q, k, v):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None, None].expand(1, q.shape[0], -1, -1),
        torch.from_numpy(v)[None, None].expand(1, q.shape[0], -1, -1))
    return out[0, :, 0, :].numpy()


@pytest.mark.parametrize("n", [1, 5, 64, 130])
def test_dense_case_equals_textbook_attention(n):
    rng = np.random.default_rng(n)
    k = rng.standard_normal((n, 128)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((n, 128)).astype(np.float32).astype(np.float64)
    q = rng.standard_normal((4, 128)).astype(np.float32).astype(np.float64)
    ks = compress_stream(k, None, "fp32", ALL)
    vs = compress_stream(v, None, "fp32", ALL)
    res = decode_unit(q, None, None, ks, vs, n)
    assert res["sel"].tolist() == list(range(n))
    np.testing.assert_allclose(res["out"], _sdpa(q, k, v), rtol=1e-12, atol=1e-13)


def test_rotated_dense_case_matches_within_storage_rounding():
    rng = np.random.default_rng(3)
    n = 300
    k = rng.standard_normal((n, 128)) * (np.arange(128) + 1.0) ** -0.5
    v = rng.standard_normal((n, 128)) * (np.arange(128) + 1.0) ** -0.5
    q = rng.standard_normal((4, 128))
    bk, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    bv, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    for dt, tol in (("fp32", 1e-5), ("bf16", 2e-2)):
        ks = compress_stream(k, bk, dt, ALL)
        vs = compress_stream(v, bv, dt, ALL)
        out = decode_unit(q, bk, bv, ks, vs, n)["out"]
        ref = _sdpa(q, k, v)
        assert np.linalg.norm(out - ref) <= tol * np.linalg.norm(ref)


def test_single_token_budget_returns_the_argmax_value():
    rng = np.random.default_rng(4)
    n = 200
    k = rng.standard_normal((n, 128))
    v = rng.standard_normal((n, 128))
    q = rng.standard_normal((4, 128))
    bv, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    ks = compress_stream(k, None, "bf16")
    vs = compress_stream(v, bv, "bf16")
    res = decode_unit(q, None, bv, ks, vs, 1)
    j = int(np.argmax(res["scores"]))
    assert res["sel"].tolist() == [j]
    expect = vs.vals[j] @ bv.T
    for g in range(4):
        np.testing.assert_allclose(res["out"][g], expect, rtol=0, atol=1e-14)
    # without the output rotation the result is the stored value row itself, bit for bit
    plain = decode_unit(q, None, None, ks, vs, 1)
    for g in range(4):
        np.testing.assert_array_equal(plain["out"][g], vs.vals[j])


def test_group_of_one_ranks_like_its_logits():
    rng = np.random.default_rng(5)
    n = 500
    k = rng.standard_normal((n, 128))
    q = rng.standard_normal((1, 128))
    ks = compress_stream(k, None, "bf16")
    s = scores(q[0], ks)
    logits = (q @ ks.vals.T)[0] / np.sqrt(128)
    assert select_top(s, 37).tolist() == select_top(logits, 37).tolist()


def test_score_is_the_sum_of_the_group_logits():
    rng = np.random.default_rng(6)
    n = 100
    k = rng.standard_normal((n, 128))
    q = rng.standard_normal((4, 128))
    bk, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    ks = compress_stream(k, bk, "bf16")
    qp = rotate_queries(q, bk)
    s = scores(qp.sum(axis=0), ks)
    per_head = np.array([[sum(qp[h, i] * ks.vals[j, i] for i in ks.kept_indices(j)) for j in range(n)]
                         for h in range(4)])
    np.testing.assert_allclose(s, per_head.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_query_head_order_in_a_group_does_not_change_selection():
    rng = np.random.default_rng(7)
    n = 400
    k = rng.integers(-4, 5, (n, 128)).astype(np.float64)
    v = rng.standard_normal((n, 128))
    q = rng.integers(-3, 4, (4, 128)).astype(np.float64)     # integer data: every sum is exact
    ks = compress_stream(k, None, "bf16")
    vs = compress_stream(v, None, "bf16")
    a = decode_unit(q, None, None, ks, vs, 50)
    b = decode_unit(q[[2, 0, 3, 1]], None, None, ks, vs, 50)
    assert a["sel"].tolist() == b["sel"].tolist()
    np.testing.assert_allclose(b["out"], a["out"][[2, 0, 3, 1]], rtol=1e-14, atol=1e-14)


def test_empty_context_gives_zero_output():
    ks = compress_stream(np.zeros((0, 128)), None, "bf16")
    res = decode_unit(np.ones((4, 128)), None, None, ks, ks, 5)
    assert res["sel"].size == 0 and not res["out"].any()


def test_attention_weights_are_a_softmax():
    rng = np.random.default_rng(8)
    qp = rng.standard_normal((2, 128))
    kv = rng.standard_normal((7, 128))
    o = attend(qp, kv, np.eye(7, 128))
    np.testing.assert_allclose(o[:, :7].sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (o[:, :7] > 0).all() and not o[:, 7:].any()


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 150), T=st.integers(1, 160), seed=st.integers(0, 2 ** 31 - 1),
       dt=st.sampled_from(["bf16", "fp32"]))
def test_selection_and_strategy_invariants(n, T, seed, dt):
    rng = np.random.default_rng(seed)
    scale = (rng.permutation(128) + 1.0) ** -0.5
    k = rng.standard_normal((n, 128)) * scale
    v = rng.standard_normal((n, 128)) * scale
    q = rng.standard_normal((4, 128)) * scale
    ks = compress_stream(k, None, dt)
    vs = compress_stream(v, None, dt)
    res = decode_unit(q, None, None, ks, vs, T)
    s, sel = res["scores"], res["sel"]
    assert len(sel) == min(T, n)
    chosen = np.zeros(n, bool)
    chosen[sel] = True
    if chosen.any() and (~chosen).any():
        worst = min((s[j], -j) for j in np.nonzero(chosen)[0])
        best_out = max((s[j], -j) for j in np.nonzero(~chosen)[0])
        assert worst > best_out
    # strategy: every vector admits its segment's c; one vector in the segment does not admit the next smaller
    pol = Policy()
    for stream in (ks, vs):
        for sgi, c in enumerate(stream.c):
            mask = stream.mask[sgi * 64:(sgi + 1) * 64]
            assert (mask.sum(axis=1) == c).all()
            # kept channels carry the largest magnitudes of the rotated rounded vector
            src = (k if stream is ks else v)[sgi * 64:(sgi + 1) * 64]
            xh = rne(src, dt)
            srt = -np.sort(-(xh * xh), axis=1)
            tot = (xh * xh).sum(axis=1)
            assert (srt[:, :c].sum(axis=1) >= 0.9 * tot * (1 - 1e-15)).all()
            smaller = [x for x in pol.keep if x < c]
            if smaller:
                cs = max(smaller)
                assert (srt[:, :cs].sum(axis=1) < 0.9 * tot * (1 + 1e-15)).any()


@pytest.mark.parametrize("n", [1, 7, 300])
def test_dense_baseline_equals_torch_sdpa(n):
    from oracle import dense_decode_unit
    rng = np.random.default_rng(100 + n)
    k, v = rng.standard_normal((n, 128)), rng.standard_normal((n, 128))
    q = rng.standard_normal((4, 128))
    np.testing.assert_allclose(dense_decode_unit(q, k, v), _sdpa(q, k, v), rtol=1e-12, atol=1e-13)


def test_dense_baseline_special_cases():
    from oracle import dense_decode_unit
    rng = np.random.default_rng(7)
    v = rng.standard_normal((50, 128))
    q = rng.standard_normal((2, 128))
    # one token: its value row, whatever the query
    np.testing.assert_array_equal(dense_decode_unit(q, rng.standard_normal((1, 128)), v[:1]), np.repeat(v[:1], 2, 0))
    # all keys zero: uniform weights, the mean value row
    np.testing.assert_allclose(dense_decode_unit(q, np.zeros((50, 128)), v), np.repeat(v.mean(0)[None], 2, 0),
                               rtol=1e-13, atol=1e-14)
    # empty context: zeros
    assert not dense_decode_unit(q, np.zeros((0, 128)), np.zeros((0, 128))).any()


def test_gram_against_outer_products_and_invariants():
    from oracle import gram, gram_abs
    rng = np.random.default_rng(11)
    x = rng.standard_normal((37, 128))
    g = gram(x)
    brute = np.zeros((128, 128))
    for t in range(x.shape[0]):
        for i in range(128):
            brute[i] += x[t, i] * x[t]
    np.testing.assert_allclose(g, brute, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(g, g.T)
    assert abs(np.trace(g) - np.sum(x * x)) <= 1e-10 * np.sum(x * x)
    assert np.linalg.eigvalsh(g).min() > -1e-9                      # positive semi-definite
    q, _ = np.linalg.qr(rng.standard_normal((128, 128)))             # orthonormal rows: G = I
    np.testing.assert_allclose(gram(q), np.eye(128), atol=1e-12)
    assert np.all(gram_abs(x) >= np.abs(g) - 1e-12)
    # the eigenvectors of X^T X by decreasing eigenvalue are the right singular vectors of X
    w, v = np.linalg.eigh(g)
    _, sv, vt = np.linalg.svd(x, full_matrices=True)
    np.testing.assert_allclose(np.sqrt(np.maximum(w[::-1][:37], 0)), sv, rtol=1e-9)
    np.testing.assert_allclose(np.abs(v[:, ::-1][:, :37].T @ vt[:37].T), np.eye(37), atol=1e-7)
