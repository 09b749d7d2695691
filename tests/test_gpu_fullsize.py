"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Each workload (one 4096-token fp32 head, one 32768-token layer, 8 x 131072, 1 x 1048576, the 16 ragged
requests) is generated, compressed and decoded whole on the GPU with the calls bench.py makes.  The oracle is
too slow for whole stores at these sizes, so it checks:
  - every segment: the payload size its code implies, the offsets as the running sum of those sizes, and the
    store's recorded total;
  - sampled segments (the first, the last and random ones of sampled streams): the oracle compresses the
    segment's 64 input rows on its own (segments are independent) and the rules of the SVD-basis parity test
    apply: values within one storage ulp, a differing channel set only on a magnitude boundary the rotation
    error can move, a differing code only where some vector's energy ratio is within that error of the target;
  - sampled (request, KV head) units: with the oracle decoding the GPU's own store of that unit (read back
    piecewise), the selection must be one the near-tie rule accepts and the output must match the oracle's
    output for that accepted selection; the uncompressed baseline (bf16 workloads) must match the oracle's
    exact attention over the unit's full rows.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import SEG, StoreReader, check_decode_unit, check_out, inputs_to_torch, seg_counts

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "llama_layer", "batch8_128k", "million", "ragged16"]


@pytest.fixture(scope="module")
def full_inputs():
    """All workloads, generated up front: the generator's worker processes are forked before this process
    has touched the GPU (later, generation runs in-process)."""
    import torch
    workers = 1 if torch.cuda.is_initialized() else min(16, os.cpu_count() or 1)
    return {name: W.generate(W.get(name), basis="svd", workers=workers) for name in NAMES}


@pytest.fixture(scope="module")
def mkv():
    import kv_cache_compression_svd_amd as m
    m.lib()
    return m


def _ulp(x, dtype):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.exp2(e - (7 if dtype == "bf16" else 23))


def _sample_units(w, rng):
    n = np.asarray(w.ctx, dtype=np.int64)
    cand = {(0, 0), (w.batch - 1, w.n_kv_heads - 1), (int(np.argmax(n)), 0),
            (int(rng.integers(w.batch)), int(rng.integers(w.n_kv_heads)))}
    return sorted(u for u in cand if n[u[0]] > 0)


def _check_segment(got, ref_stream, x_rows, basis, dtype, s, key):
    """Sampled-segment rules; returns 1 when the codes differ (allowed only near the energy target)."""
    lo = s * SEG
    ns = x_rows.shape[0]
    g_c = int(got.c[s])
    r_c = int(ref_stream.c[0])
    xhat = oracle.rotate_round(x_rows, basis, dtype)
    if g_c != r_c:
        # some vector must sit within the rotation error of the 0.9 target at the two codes involved
        e_all = np.sum(xhat * xhat, axis=1)
        order = oracle.channel_order(xhat)
        near = False
        for c in (g_c, r_c):
            ratio = oracle.kept_energy(xhat, order, c) / np.where(e_all > 0, e_all, 1.0)
            near |= bool(np.any(np.abs(ratio - 0.9) < 1e-2))
        assert near, f"segment code differs away from the energy target at {key} segment {s}"
        return 1
    gm = got.mask[lo:lo + ns]
    gv = got.vals[lo:lo + ns]
    both = gm & ref_stream.mask
    assert np.all(np.abs(gv[both] - ref_stream.vals[both]) <= _ulp(ref_stream.vals[both], dtype) * 1.0001), key
    for j in np.nonzero(np.any(gm != ref_stream.mask, axis=1))[0]:
        mags = np.abs(xhat[j])
        tc = np.sort(mags)[::-1][r_c - 1]
        swapped = np.nonzero(gm[j] != ref_stream.mask[j])[0]
        assert np.all(np.abs(mags[swapped] - tc) <= 2 * _ulp(np.array([tc]), dtype)[0] + 1e-300), (key, s, j)
    return 0


@pytest.mark.parametrize("name", NAMES)
def test_full_size_sampled_parity(mkv, full_inputs, name):
    import torch
    inp = full_inputs.pop(name)
    w = inp.workload
    rng = np.random.default_rng(1234)
    K, V, q, basis = inputs_to_torch(inp)
    policy = mkv.mkv_default_policy()
    sb, tb = mkv.mkv_compress_bytes(K, V, inp.cu_seqlens, policy)
    store_buf = torch.empty(sb, dtype=torch.uint8, device="cuda")
    scratch = torch.empty(tb, dtype=torch.uint8, device="cuda")
    store = mkv.mkv_compress(K, V, inp.cu_seqlens, basis, policy, store_buf=store_buf, scratch=scratch)
    dense = None
    if inp.dtype == "bf16":   # the uncompressed baseline on the same inputs
        dense = mkv.mkv_dense_decode_attn(K, V, inp.cu_seqlens, q).cpu().numpy().astype(np.float64)
    del K, V, scratch
    T = inp.T
    te = np.minimum(T, np.diff(inp.cu_seqlens))
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.batch, w.n_kv_heads, max(int(te.max()), 1)), dtype=torch.int32, device="cuda")
    ws = torch.empty(mkv.mkv_decode_workspace_bytes(store, w.n_q_heads, T), dtype=torch.uint8, device="cuda")
    mkv.mkv_decode_attn(store, q, T, out=out, sel=sel, ws=ws)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    sel = sel.cpu().numpy()

    # every segment: sizes implied by the codes, offsets as their running sum, the recorded total
    rd = StoreReader(store, inp.dtype)
    bv = 2 if inp.dtype == "bf16" else 4
    assert np.all(rd.codes < len(rd.keep))
    sizes = rd.segment_bytes(bv)
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64)
    np.testing.assert_array_equal(rd.seg_off, offs)
    assert rd.total == int(sizes.sum()) == store.payload_bytes()

    n, S_r, _ = seg_counts(inp.cu_seqlens)
    cu = inp.cu_seqlens
    G = w.group
    code_diff = seg_checked = near_ties = 0
    for (r, h) in _sample_units(w, rng):
        streams = {}
        for X, arr in ((0, inp.K), (1, inp.V)):
            got = rd.stream(r, h, X)
            streams[X] = got
            picks = {0, int(S_r[r]) - 1} | set(int(s) for s in rng.integers(0, int(S_r[r]), 6))
            for s in sorted(picks):
                rows = W.to_f64(arr[cu[r] + s * SEG: cu[r] + min(int(n[r]), (s + 1) * SEG), h, :], inp.dtype)
                ref = oracle.compress_stream(rows, inp.basis[r, h, X], inp.dtype)
                code_diff += _check_segment(got, ref, rows, inp.basis[r, h, X], inp.dtype, s, (r, h, X))
                seg_checked += 1
        # decode of this unit by the oracle, on the GPU's own store
        qg = W.to_f64(inp.q[r, h * G:(h + 1) * G, :], inp.dtype)
        nd = check_decode_unit(sel[r, h], out[r, h * G:(h + 1) * G], qg, inp.basis[r, h, 0], inp.basis[r, h, 1],
                               streams[0], streams[1], int(te[r]))
        assert nd >= 0, f"too many near-tie selections to enumerate at unit {(r, h)}"
        near_ties += nd
        if dense is not None:
            k = W.to_f64(inp.K[cu[r]:cu[r + 1], h, :], inp.dtype)
            v = W.to_f64(inp.V[cu[r]:cu[r + 1], h, :], inp.dtype)
            check_out(dense[r, h * G:(h + 1) * G], oracle.dense_decode_unit(qg, k, v))
    print(f"{name}: {seg_checked} sampled segments, {code_diff} with another code (near the target); "
          f"{near_ties} tokens swapped inside the near-tie band")
    assert code_diff <= 1
