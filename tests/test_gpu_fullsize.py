"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Each workload (one 4096-token fp32 head, one 32768-token layer, 8 x 131072, 1 x 1048576, the 16 ragged
requests) is generated, compressed and decoded whole on the GPU with the calls bench.py makes.  The oracle is
too slow for whole stores at these sizes, so it checks:
  - every segment: the payload size its code implies, offsets that follow the documented placement (runs of
    consecutive segments from a slot's full-size position for bf16, back to back for fp32) with no overlaps
    inside the payload, and the store's recorded total;
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
from _helpers import (SEG, StoreReader, check_run_layout, channel_swap_reason, check_decode_unit, check_out, code_difference_reason,
                      inputs_to_torch, observed_ulps, record_parity, seg_counts)

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


def _sample_units(w, rng):
    n = np.asarray(w.ctx, dtype=np.int64)
    cand = {(0, 0), (w.batch - 1, w.n_kv_heads - 1), (int(np.argmax(n)), 0),
            (int(rng.integers(w.batch)), int(rng.integers(w.n_kv_heads)))}
    return sorted(u for u in cand if n[u[0]] > 0)


def _segment_ulps(got, ref_stream, s, dtype):
    """Observed |GPU - oracle| in ulps over the channels both kept in sampled segment s."""
    lo = s * SEG
    ns = ref_stream.n
    return observed_ulps(got.vals[lo:lo + ns], ref_stream.vals, got.mask[lo:lo + ns] & ref_stream.mask, dtype)


def _check_segment(got, ref_stream, xhat, dtype, s, key, m):
    """Sampled-segment rules with the workload's observed ulps m; returns 1 when the codes differ (each such
    segment must hold a vector whose energy decision the observed rotation error can flip)."""
    lo = s * SEG
    ns = xhat.shape[0]
    g_code = int(got.codes[s])
    r_code = int(ref_stream.codes[0])
    if g_code != r_code:
        why = code_difference_reason(xhat, g_code, r_code, (128, 64, 32), m, dtype)
        assert why is not None, f"segment code differs without a vector near the energy target at {key} segment {s}"
        return 1
    gm = got.mask[lo:lo + ns]
    for j in np.nonzero(np.any(gm != ref_stream.mask, axis=1))[0]:
        assert channel_swap_reason(xhat[j], gm[j], ref_stream.mask[j], int(ref_stream.c[0]), m, dtype), (key, s, j)
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

    # every segment: sizes implied by the codes; the segments of each run of a stream back to back from the run's
    # first slot at full size (64 x 128 values), runs apart, all inside the payload; the recorded total
    rd = StoreReader(store, inp.dtype)
    bv = 2 if inp.dtype == "bf16" else 4
    assert np.all(rd.codes < len(rd.keep))
    sizes = rd.segment_bytes(bv)
    check_run_layout(rd.seg_off, sizes, store, bv)
    assert rd.total == int(sizes.sum()) == store.payload_bytes()

    n, S_r, _ = seg_counts(inp.cu_seqlens)
    cu = inp.cu_seqlens
    G = w.group
    code_diff = seg_checked = near_ties = 0
    sampled = []
    streams_of = {}
    for (r, h) in _sample_units(w, rng):
        for X, arr in ((0, inp.K), (1, inp.V)):
            got = rd.stream(r, h, X)
            streams_of[(r, h, X)] = got
            picks = {0, int(S_r[r]) - 1} | set(int(s) for s in rng.integers(0, int(S_r[r]), 6))
            for s in sorted(picks):
                rows = W.to_f64(arr[cu[r] + s * SEG: cu[r] + min(int(n[r]), (s + 1) * SEG), h, :], inp.dtype)
                ref = oracle.compress_stream(rows, inp.basis[r, h, X], inp.dtype)
                xhat = oracle.rotate_round(rows, inp.basis[r, h, X], inp.dtype)
                sampled.append((got, ref, xhat, s, (r, h, X)))
    # the rotation error bound: the largest value difference observed over every sampled segment
    m = max(_segment_ulps(got, ref, s, inp.dtype) for got, ref, _, s, _ in sampled)
    assert m <= 1.0 + 1e-9, f"stored values differ by {m} ulp"
    for got, ref, xhat, s, key in sampled:
        code_diff += _check_segment(got, ref, xhat, inp.dtype, s, key, m)
        seg_checked += 1
    for (r, h) in sorted({k[:2] for k in streams_of}):
        streams = {X: streams_of[(r, h, X)] for X in (0, 1)}
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
    record_parity("full_size_sampled_parity", name, observed_ulps=m, segments=seg_checked,
                  segments_other_code=code_diff, tokens_swapped_in_band=near_ties)
    assert code_diff <= 1
