"""Incremental append into growable stores: after appending tokens one decode step at a time, every segment
holds exactly what compressing the extended context at once gives (codes, channel sets and values, bit for
bit), so decoding it gives bit-identical selections and outputs; with a signed-permutation basis the store also
equals the oracle's compression of the extended inputs bit for bit.  Cases cross segment boundaries (a segment
is sealed when its 64th token arrives), start from empty, partial and full last segments, append to a subset
of the requests, and stop at the capacity."""
import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import inputs_to_torch, read_store

pytestmark = pytest.mark.gpu


def _wl(ctx, seed=61, T=50):
    return W.Workload(f"append{len(ctx)}", len(ctx), 16, 4, tuple(ctx), "bf16", (T,) * len(ctx), "per_request",
                      seed, "append case")


def _grow(mkv, inp, n0, steps, basis, active_of=None):
    """Store from the first n0[r] tokens of each request, then `steps` appends (request r takes part in step k
    when active_of(k)[r]); returns the store and the tokens each request holds."""
    import torch
    K, V, q, _ = inputs_to_torch(inp)
    cu = inp.cu_seqlens
    B = inp.workload.batch
    take = np.concatenate([np.arange(cu[r], cu[r] + n0[r]) for r in range(B)])
    cu0 = np.concatenate([[0], np.cumsum(n0)])
    cap = np.diff(cu)
    st = mkv.mkv_compress(K[take].contiguous(), V[take].contiguous(), cu0, basis, capacity=cap)
    n = np.array(n0)
    for k in range(steps):
        act = np.ones(B, dtype=np.int32) if active_of is None else np.asarray(active_of(k), dtype=np.int32)
        act = act * (n < cap)
        idx = torch.as_tensor(cu[:-1] + np.minimum(n, cap - 1), device="cuda")
        mkv.mkv_append(st, K[idx].contiguous(), V[idx].contiguous(), active=act)
        n = n + act
    torch.cuda.synchronize()
    assert np.array_equal(np.diff(st.cu), n)
    return st, n, q


def _compare(mkv, inp, st, n, q, basis):
    """The grown store against compressing the same tokens at once (GPU) and its decode, bit for bit."""
    import torch
    K, V, _, _ = inputs_to_torch(inp)
    cu = inp.cu_seqlens
    B = inp.workload.batch
    take = np.concatenate([np.arange(cu[r], cu[r] + n[r]) for r in range(B)])
    ref = mkv.mkv_compress(K[take].contiguous(), V[take].contiguous(), np.concatenate([[0], np.cumsum(n)]), basis)
    raw = read_store(st, "bf16")
    assert raw["total"] <= int(st.view().payload_capacity)   # seals never run into the open-segment areas
    g, f = raw["streams"], read_store(ref, "bf16")["streams"]
    for key in f:
        assert np.array_equal(g[key].c, f[key].c), key
        assert np.array_equal(g[key].mask, f[key].mask), key
        assert np.array_equal(g[key].vals, f[key].vals), key
    T = np.asarray(inp.T)
    o1, s1 = mkv.mkv_decode_attn(st, q, T)
    o2, s2 = mkv.mkv_decode_attn(ref, q, T)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(o1, o2)
    return g


@pytest.mark.parametrize("n0,steps", [([64, 100, 0], 70), ([1, 63, 128], 66), ([200, 5, 64], 3)])
def test_append_equals_compressing_the_extended_context(mkv_lib, n0, steps):
    mkv = mkv_lib
    import torch
    inp = W.generate(_wl([max(a + steps, 1) for a in n0]), basis="svd")
    basis = torch.from_numpy(inp.basis).cuda()
    st, n, q = _grow(mkv, inp, n0, steps, basis)
    _compare(mkv, inp, st, n, q, basis)


def test_append_to_a_subset_and_up_to_capacity(mkv_lib):
    mkv = mkv_lib
    import torch
    inp = W.generate(_wl([150, 90, 70]), basis="svd")
    basis = torch.from_numpy(inp.basis).cuda()
    st, n, q = _grow(mkv, inp, [60, 30, 70], 80, basis, active_of=lambda k: [k % 2 == 0, 1, k % 3 == 0])
    assert n.tolist() == [100, 90, 70]        # request 1 stops at its capacity of 90; request 2 starts full
    _compare(mkv, inp, st, n, q, basis)
    K, V, _, _ = inputs_to_torch(inp)
    with pytest.raises(mkv.MkvError):         # every request listed, one of them full: nothing enqueued
        mkv.mkv_append(st, K[:3].contiguous(), V[:3].contiguous())
    assert np.array_equal(np.diff(st.cu), n)


def test_append_matches_the_oracle_bit_for_bit(mkv_lib):
    """Signed-permutation bases make the rotation exact in any order: the grown store equals the oracle's."""
    mkv = mkv_lib
    import torch
    inp = W.generate(_wl([140, 65]), basis="sperm")
    basis = torch.from_numpy(inp.basis).cuda()
    st, n, q = _grow(mkv, inp, [10, 64], 75, basis)
    got = read_store(st, "bf16")["streams"]
    cu = inp.cu_seqlens
    for r in range(2):
        for h in range(4):
            for X, arr in ((0, inp.K), (1, inp.V)):
                ref = oracle.compress_stream(W.to_f64(arr[cu[r]:cu[r] + n[r], h, :], "bf16"), inp.basis[r, h, X], "bf16")
                g = got[(r, h, X)]
                assert np.array_equal(g.c, ref.c) and np.array_equal(g.mask, ref.mask) and np.array_equal(g.vals, ref.vals)


def test_plain_store_refuses_appends(mkv_lib):
    mkv = mkv_lib
    inp = W.generate(_wl([64]), basis="none")
    K, V, _, _ = inputs_to_torch(inp)
    st = mkv.mkv_compress(K, V, inp.cu_seqlens)
    with pytest.raises(mkv.MkvError) as e:
        mkv.mkv_append(st, K[:1].contiguous().view(1, 4, 128), V[:1].contiguous().view(1, 4, 128))
    assert "growable" in str(e.value)


@pytest.fixture(scope="module")
def mkv_lib():
    import kv_cache_compression_svd_amd as m
    m.lib()
    return m


def test_appends_of_constructed_vectors_match_the_oracle(mkv_lib):
    """Appends (no basis, bf16) of the parity tests' constructed vectors (full-range magnitudes, ties, flat,
    zero, exact-threshold, subnormal, out-of-float32-range squares): the grown store equals the oracle's
    compression of the extended context bit for bit."""
    mkv = mkv_lib
    from test_gpu_parity import SEGMENT_KINDS, _crafted_segment
    rng = np.random.default_rng(79)
    ctx = (3 * 64 + 20, 64 + 5)
    tot = sum(ctx)
    wl = W.Workload("append_crafted", 2, 8, 2, ctx, "bf16", (50, 50), "per_request", 79, "append case")
    K = np.zeros((tot, 2, 128), np.uint16)
    V = np.zeros((tot, 2, 128), np.uint16)
    kind_at = 0
    for arr in (K, V):
        for h in range(2):
            for t0 in range(0, tot, 16):
                rows = min(16, tot - t0)
                x = _crafted_segment(rng, SEGMENT_KINDS[kind_at % len(SEGMENT_KINDS)], rows)
                kind_at += 1
                arr[t0:t0 + rows, h, :] = W.f32_to_bf16_bits(x.astype(np.float32))
    q = W.f32_to_bf16_bits(rng.standard_normal((2, 8, 128)).astype(np.float32))
    cu = np.array([0, ctx[0], tot], np.int64)
    inp = W.Inputs(wl, K, V, q, None, cu, np.array([50, 50], np.int32))
    st, n, _ = _grow(mkv, inp, (100, 10), 120, None)
    assert list(n) == list(ctx)
    ref = oracle.compress_all(inp)
    raw = read_store(st, "bf16")
    # every segment keeps all 128 channels here: the sealed segments fill the payload to its capacity
    assert raw["total"] <= int(st.view().payload_capacity)
    got = raw["streams"]
    for key, r in ref.items():
        assert np.array_equal(got[key].c, r.c), key
        assert np.array_equal(got[key].mask, r.mask), key
        assert np.array_equal(got[key].vals, r.vals), key
