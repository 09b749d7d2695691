"""GPU parity of the HIP path against the CPU oracle on the same seeded inputs.

Compression parity modes:
  P1  inputs already rotated and rounded by the oracle, basis = NULL: codes, channel indices, values bit-exact.
  P2  signed-permutation basis (exact in any summation order): the whole path bit-exact.
  P3  SVD basis: stored values within one storage ulp; codes and channel sets equal except where the oracle's
      own decision margin is inside the rotation's rounding error (counted, and checked to be such cases).
Decode parity: selection equal except tokens whose oracle score is within 1e-5 relative of the T-th score;
outputs within 2e-3 relative (per head rel-L2 and elementwise against the row maximum).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import (StoreReader, channel_swap_reason, check_decode_unit, check_out, check_selection,
                      code_difference_reason, inputs_to_torch, observed_ulps, prerotated_inputs, read_store,
                      record_parity, upload_oracle_store)

pytestmark = pytest.mark.gpu

CASES = [("tiny", 8), ("llama_layer", 32), ("ragged16", 64), ("batch8_128k", 256)]
IDS = [f"{n}/{d}" for n, d in CASES]


@pytest.fixture(scope="module")
def mkv():
    import kv_cache_compression_svd_amd as m
    m.lib()
    return m


def _wl(name, div):
    return W.scaled(W.get(name), div)


def _policy(mkv, keep=(128, 64, 32)):
    return mkv.SegPolicy.make(keep)


def _compress_gpu(mkv, inp, keep=(128, 64, 32)):
    import torch
    K, V, q, basis = inputs_to_torch(inp)
    st = mkv.mkv_compress(K, V, inp.cu_seqlens, basis, _policy(mkv, keep))
    torch.cuda.synchronize()
    return st, q


def _assert_streams_equal(got: dict, ref: dict):
    for key, r in ref.items():
        g = got[key]
        np.testing.assert_array_equal(g.c, r.c, err_msg=f"codes differ at {key}")
        np.testing.assert_array_equal(g.mask, r.mask, err_msg=f"channel sets differ at {key}")
        np.testing.assert_array_equal(g.vals, r.vals, err_msg=f"values differ at {key}")


def _closed_form_bytes(streams, dtype):
    bv = 2 if dtype == "bf16" else 4
    return oracle.store_payload_bytes(streams, 64, bv)


@pytest.mark.parametrize("name,div", CASES, ids=IDS)
def test_compress_p1_prerotated_bit_exact(mkv, name, div):
    inp = W.generate(_wl(name, div), basis="svd")
    ref = oracle.compress_all(inp)
    pre = prerotated_inputs(inp, ref)
    st, _ = _compress_gpu(mkv, pre)
    got = read_store(st, inp.dtype)
    _assert_streams_equal(got["streams"], ref)
    assert got["total"] == _closed_form_bytes(ref, inp.dtype) == st.payload_bytes()


@pytest.mark.parametrize("name,div", [("llama_layer", 32), ("ragged16", 64)], ids=["llama_layer/32", "ragged16/64"])
def test_decode_without_basis(mkv, name, div):
    """A store compressed with basis = NULL: decode takes q as already rotated and returns o' unrotated; against
    the oracle run without a basis."""
    inp = W.generate(_wl(name, div), basis="svd")
    pre = prerotated_inputs(inp, oracle.compress_all(inp))
    ref = oracle.compress_all(pre)
    store, q = _compress_gpu(mkv, pre)
    _assert_streams_equal(read_store(store, pre.dtype)["streams"], ref)
    _decode_compare(mkv, pre, store, q, ref)


@pytest.mark.parametrize("name,div", CASES, ids=IDS)
def test_compress_p2_signed_permutation_bit_exact(mkv, name, div):
    inp = W.generate(_wl(name, div), basis="sperm")
    ref = oracle.compress_all(inp)
    st, _ = _compress_gpu(mkv, inp)
    got = read_store(st, inp.dtype)
    _assert_streams_equal(got["streams"], ref)
    assert got["total"] == _closed_form_bytes(ref, inp.dtype)


@pytest.mark.parametrize("name,div", CASES, ids=IDS)
def test_compress_p3_svd_basis(mkv, name, div):
    """SVD basis: stored values within one storage ulp of the oracle's; every segment whose code differs must
    hold a vector whose oracle energy ratio lies within the flip bound implied by the observed value
    differences, on the side that explains the difference; every token whose kept set differs at an equal
    code must swap only channels within 2 m ulp of the oracle's c-th magnitude (m: observed ulps)."""
    inp = W.generate(_wl(name, div), basis="svd")
    keep = (128, 64, 32)
    ref = oracle.compress_all(inp)
    st, _ = _compress_gpu(mkv, inp)
    got = read_store(st, inp.dtype)["streams"]
    m = 0.0
    for key, r in ref.items():
        g = got[key]
        m = max(m, observed_ulps(g.vals, r.vals, g.mask & r.mask, inp.dtype))
    assert m <= 1.0 + 1e-9, f"stored values differ by {m} ulp"
    seg_total = seg_diff = tok_total = tok_diff = 0
    for key, r in ref.items():
        g = got[key]
        rr, hh, X = key
        x = W.to_f64((inp.K if X == 0 else inp.V)[inp.cu_seqlens[rr]:inp.cu_seqlens[rr + 1], hh, :], inp.dtype)
        xhat = oracle.rotate_round(x, inp.basis[rr, hh, X], inp.dtype)
        seg_total += r.c.size
        for s in np.nonzero(g.codes != r.codes)[0]:
            seg_diff += 1
            rows = xhat[64 * s: 64 * s + 64]
            why = code_difference_reason(rows, int(g.codes[s]), int(r.codes[s]), keep, m, inp.dtype)
            assert why is not None, f"segment {s} of {key}: code {g.codes[s]} vs oracle {r.codes[s]} unexplained"
        same_c = np.repeat(g.c == r.c, 64)[: r.n]
        rows = np.nonzero(same_c & np.any(g.mask != r.mask, axis=1))[0]
        tok_total += int(same_c.sum())
        tok_diff += rows.size
        for j in rows:
            c = int(r.c[j // 64])
            assert channel_swap_reason(xhat[j], g.mask[j], r.mask[j], c, m, inp.dtype), (key, j)
    record_parity("compress_p3_svd_basis", f"{name}/{div}", observed_ulps=m, segments=seg_total,
                  segments_other_code=seg_diff, tokens=tok_total, tokens_other_channels=tok_diff)
    # every difference is explained above; these caps only guard against a systematic drift
    assert seg_diff <= max(2, 0.01 * seg_total)
    assert tok_diff <= max(4, 0.02 * tok_total)


def _decode_compare(mkv, inp, store, q, ref_streams):
    """Decodes on the GPU and checks every (request, KV head) unit against the oracle decoding the same
    store: an accepted selection (near ties) and the oracle's output for it.  Returns the number of units
    whose selection differs inside the near-tie band."""
    import torch
    out, sel = mkv.mkv_decode_attn(store, q, inp.T)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    sel = sel.cpu().numpy()
    w = inp.workload
    G = w.group
    ndiff_units = 0
    for r in range(w.batch):
        n = int(inp.cu_seqlens[r + 1] - inp.cu_seqlens[r])
        te = min(int(inp.T[r]), n)
        for h in range(w.n_kv_heads):
            qg = W.to_f64(inp.q[r, h * G:(h + 1) * G, :], inp.dtype)
            bk = None if inp.basis is None else inp.basis[r, h, 0]
            bvv = None if inp.basis is None else inp.basis[r, h, 1]
            nd = check_decode_unit(sel[r, h], out[r, h * G:(h + 1) * G], qg, bk, bvv, ref_streams[(r, h, 0)],
                                   ref_streams[(r, h, 1)], te)
            assert nd >= 0, f"too many near-tie selections to enumerate at unit {(r, h)}"
            ndiff_units += nd > 0
    return ndiff_units


@pytest.mark.parametrize("name,div", CASES, ids=IDS)
def test_decode_on_oracle_store(mkv, name, div):
    """Decode alone: the store is the oracle's, written in the documented layout."""
    inp = W.generate(_wl(name, div), basis="svd")
    ref = oracle.compress_all(inp)
    store = upload_oracle_store(ref, inp, (128, 64, 32))
    _, _, q, _ = inputs_to_torch(inp)
    _decode_compare(mkv, inp, store, q, ref)


@pytest.mark.parametrize("name,div", CASES, ids=IDS)
def test_end_to_end_signed_permutation(mkv, name, div):
    inp = W.generate(_wl(name, div), basis="sperm")
    ref = oracle.compress_all(inp)
    store, q = _compress_gpu(mkv, inp)
    _decode_compare(mkv, inp, store, q, ref)


@pytest.mark.parametrize("name,div", CASES, ids=IDS)
def test_end_to_end_svd(mkv, name, div):
    inp = W.generate(_wl(name, div), basis="svd")
    ref = oracle.compress_all(inp)
    store, q = _compress_gpu(mkv, inp)
    _decode_compare(mkv, inp, store, q, ref)


# ---- edge cases ---------------------------------------------------------------------------------------------
def _custom(ctx, T, Hq=8, Hkv=2, dtype="bf16", seed=5):
    return W.Workload("edge", len(ctx), Hq, Hkv, tuple(ctx), dtype, tuple(T), "single", seed)


EDGE = [
    ("empty_request", _custom([100, 0, 200], [10, 5, 300])),
    ("T_above_n", _custom([130, 64], [1000, 64])),
    ("T_one", _custom([300, 65], [1, 1])),
    ("one_token", _custom([1, 2, 63], [1, 1, 2])),
    ("group1", _custom([500, 129], [50, 7], Hq=2, Hkv=2)),
    ("group8", _custom([260, 70], [33, 70], Hq=16, Hkv=2)),
    ("group2_fp32", _custom([333], [40], Hq=4, Hkv=2, dtype="fp32")),
]


@pytest.mark.parametrize("label,wl", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("basis", ["sperm", "svd"])
def test_edge_cases(mkv, label, wl, basis):
    inp = W.generate(wl, basis=basis)
    ref = oracle.compress_all(inp)
    store, q = _compress_gpu(mkv, inp)
    if basis == "sperm":
        _assert_streams_equal(read_store(store, inp.dtype)["streams"], ref)
        _decode_compare(mkv, inp, store, q, ref)
    else:
        store2 = upload_oracle_store(ref, inp, (128, 64, 32))
        _decode_compare(mkv, inp, store2, q, ref)


def test_many_requests(mkv):
    """130 requests of 0..300 tokens (some empty, most with a ragged last segment) and per-request budgets: the
    per-request tables outgrow the words a kernel launch carries (448), so both calls upload them in several
    launches.  Whole compression bit-exact (signed-permutation basis) and decode against the oracle."""
    rng = np.random.default_rng(31)
    ctx = [int(x) for x in rng.integers(0, 301, 130)]
    ctx[5] = 0
    T = [max(1, int(x)) for x in rng.integers(1, 80, 130)]
    wl = _custom(ctx, T, Hq=4, Hkv=2, seed=31)
    inp = W.generate(wl, basis="sperm")
    ref = oracle.compress_all(inp)
    store, q = _compress_gpu(mkv, inp)
    got = read_store(store, inp.dtype)
    _assert_streams_equal(got["streams"], ref)
    assert got["total"] == _closed_form_bytes(ref, inp.dtype) == store.payload_bytes()
    _decode_compare(mkv, inp, store, q, ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("keep", [(128,), (128, 64), (128, 64, 32, 16)])
def test_other_strategy_sets(mkv, keep, dtype):
    wl = _custom([400, 77], [64, 20], dtype=dtype)
    inp = W.generate(wl, basis="sperm")
    if dtype == "fp32" and len(keep) > 3:   # fp32 stores take at most three kept counts: refused up front
        with pytest.raises(mkv.MkvError) as e:
            _compress_gpu(mkv, inp, keep)
        assert e.value.status == mkv.MKV_E_UNSUPPORTED
        return
    pol = oracle.Policy(keep=keep)
    ref = oracle.compress_all(inp, pol)
    store, q = _compress_gpu(mkv, inp, keep)
    _assert_streams_equal(read_store(store, inp.dtype)["streams"], ref)
    _decode_compare(mkv, inp, store, q, ref)


def test_all_equal_scores_pick_lowest_tokens(mkv):
    """Zero keys give every token the score 0: the selection is the lowest T indices and attention is uniform."""
    import torch
    wl = _custom([300], [37], Hq=4, Hkv=1)
    inp = W.generate(wl, basis="none")
    inp.K[:] = 0
    ref = oracle.compress_all(inp)
    store, q = _compress_gpu(mkv, inp)
    out, sel = mkv.mkv_decode_attn(store, q, inp.T)
    torch.cuda.synchronize()
    assert sel.cpu().numpy()[0, 0, :37].tolist() == list(range(37))
    res = oracle.decode_all(inp, ref)
    check_out(out.cpu().numpy()[0].astype(np.float64), res[(0, 0)]["out"])


def test_repeat_runs_are_bit_identical(mkv):
    import torch
    inp = W.generate(_wl("ragged16", 64), basis="svd")
    K, V, q, basis = inputs_to_torch(inp)
    s1 = mkv.mkv_compress(K, V, inp.cu_seqlens, basis)
    s2 = mkv.mkv_compress(K, V, inp.cu_seqlens, basis)
    torch.cuda.synchronize()
    r1, r2 = read_store(s1, inp.dtype), read_store(s2, inp.dtype)
    assert r1["total"] == r2["total"]
    np.testing.assert_array_equal(r1["codes"], r2["codes"])
    np.testing.assert_array_equal(r1["seg_off"], r2["seg_off"])
    # every segment's bytes (the bytes between runs of segments are never written)
    b1, b2 = s1.buf.cpu().numpy(), s2.buf.cpu().numpy()
    p1 = s1.view().payload - s1.buf.data_ptr()
    p2 = s2.view().payload - s2.buf.data_ptr()
    sizes = StoreReader(s1, inp.dtype).segment_bytes(2 if inp.dtype == "bf16" else 4)
    offs = r1["seg_off"].astype(np.int64)
    live = sizes > 0
    assert int(sizes.sum()) == r1["total"]
    seg1 = np.concatenate([b1[p1 + o:p1 + o + s] for o, s in zip(offs[live], sizes[live])])
    seg2 = np.concatenate([b2[p2 + o:p2 + o + s] for o, s in zip(offs[live], sizes[live])])
    np.testing.assert_array_equal(seg1, seg2)
    o1, q1 = mkv.mkv_decode_attn(s1, q, inp.T)
    o2, q2 = mkv.mkv_decode_attn(s1, q, inp.T)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(q1, q2)


def test_equal_scores_across_emit_tiles(mkv):
    """Every score equal on a stream of several 32768-token emit tiles: the selection is the lowest T indices,
    so the cut among equal keys falls inside a later tile and every tile must count the tokens before it."""
    import torch
    wl = _custom([100_000, 40_000], [70_000, 33_000], Hq=4, Hkv=1, seed=12)
    inp = W.generate(wl, basis="none")
    inp.K[:] = 0
    ref = oracle.compress_all(inp)
    store, q = _compress_gpu(mkv, inp)
    out, sel = mkv.mkv_decode_attn(store, q, inp.T)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    assert np.array_equal(sel[0, 0, :70_000], np.arange(70_000))
    assert np.array_equal(sel[1, 0, :33_000], np.arange(33_000)) and np.all(sel[1, 0, 33_000:] == -1)
    res = oracle.decode_all(inp, ref)
    for r in range(2):
        check_out(out.cpu().numpy()[r].astype(np.float64), res[(r, 0)]["out"])


def test_long_stream_spans_several_bitmap_tiles(mkv):
    """A 300K-token stream spans ten 32768-token bitmap tiles of the selection's emit step."""
    wl = _custom([300_000, 5_000], [5_000, 150], Hq=4, Hkv=1, seed=9)
    inp = W.generate(wl, basis="sperm")
    ref = oracle.compress_all(inp)
    store, q = _compress_gpu(mkv, inp)
    _decode_compare(mkv, inp, store, q, ref)


@pytest.mark.parametrize("frac", ["all", "all_but_one", "half"])
def test_large_budgets_across_bitmap_tiles(mkv, frac):
    """Budgets of every token, all but one, and half of a 70000-token stream (three emit tiles): the selection
    takes whole tiles, leaves a single token out, or cuts in the middle of the candidates."""
    n = 70_000
    T = {"all": n, "all_but_one": n - 1, "half": n // 2}[frac]
    wl = _custom([n, 300], [T, 299], Hq=4, Hkv=1, seed=13)
    inp = W.generate(wl, basis="sperm")
    ref = oracle.compress_all(inp)
    store, q = _compress_gpu(mkv, inp)
    _decode_compare(mkv, inp, store, q, ref)


# ---- constructed vectors for the per-vector threshold search ------------------------------------------------
SEGMENT_KINDS = ["wide", "wide_sparse", "ties", "flat", "zero_mix", "threshold", "denormal", "near_two", "normal",
                 "big_flat", "tiny_sparse"]


def _crafted_segment(rng, kind: str, rows: int) -> np.ndarray:
    """float64 [rows][128] vectors of one kind, exactly representable in bf16 except where rounding is intended."""
    sign = rng.choice([-1.0, 1.0], size=(rows, 128))
    if kind == "wide":          # magnitudes 2^-120 .. 2^100 with 7 random mantissa bits
        x = sign * np.ldexp(1.0 + rng.integers(0, 128, (rows, 128)) / 128.0, rng.integers(-120, 101, (rows, 128)))
    elif kind == "wide_sparse":  # at most 24 non-zeros spanning 2^-120 .. 2^100: every vector admits 32 channels
        x = np.zeros((rows, 128))
        for i in range(rows):
            ch = rng.choice(128, int(rng.integers(1, 25)), replace=False)
            x[i, ch] = sign[i, ch] * np.ldexp(1.0 + rng.integers(0, 128, ch.size) / 128.0,
                                              rng.integers(-120, 101, ch.size))
    elif kind == "ties":        # three magnitudes only: long runs of equal values at every threshold
        x = sign * rng.choice([1.0, 0.5, 0.25], size=(rows, 128), p=[0.2, 0.5, 0.3])
    elif kind == "flat":        # top-64 energy exactly half: only the full vector is admissible
        x = sign.copy()
    elif kind == "zero_mix":    # all-zero vectors (admit every count) between ordinary ones
        x = rng.standard_normal((rows, 128))
        x[::2] = 0.0
    elif kind == "threshold":   # 32 channels of 3, 32 of 1, 64 of 0: E_32 = 288 = 0.9 * 320 exactly
        x = np.zeros((rows, 128))
        for i in range(rows):
            perm = rng.permutation(128)
            x[i, perm[:32]] = 3.0 * sign[i, perm[:32]]
            x[i, perm[32:64]] = sign[i, perm[32:64]]
    elif kind == "denormal":    # bf16 subnormals (below 2^-126) next to small normal values
        x = sign * np.where(rng.random((rows, 128)) < 0.5, np.ldexp(rng.integers(1, 128, (rows, 128)), -133),
                            np.ldexp(1.0 + rng.integers(0, 128, (rows, 128)) / 128.0, -120))
    elif kind == "near_two":    # magnitudes across 2.0, where the top bit of the magnitude pattern flips
        x = sign * rng.uniform(1.9, 2.1, (rows, 128))
    elif kind == "big_flat":    # flat at 2^70: squares beyond the float32 range, only the full vector admissible
        x = sign * 2.0 ** 70
    elif kind == "tiny_sparse":  # at most 24 non-zeros near 2^-100: squares below the float32 range, admits 32
        x = np.zeros((rows, 128))
        for i in range(rows):
            ch = rng.choice(128, int(rng.integers(1, 25)), replace=False)
            x[i, ch] = sign[i, ch] * np.ldexp(1.0 + rng.integers(0, 128, ch.size) / 128.0, -100)
    else:
        x = rng.standard_normal((rows, 128)) * (np.arange(128) + 1.0) ** -0.5
    return x


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_compress_constructed_vectors_bit_exact(mkv, dtype):
    """Pre-rotated (basis NULL) stores of constructed vectors: wide dynamic range (bf16: threshold searches over
    the full 15-bit magnitude range), long ties, flat, zero, exactly-at-threshold, subnormal and 2.0-straddling
    vectors, and vectors whose squares leave the float32 range (the energy rule is float64); codes, channel
    sets and values must equal the oracle's bit for bit."""
    rng = np.random.default_rng(77)
    ctx = (11 * 64 + 17, 200)
    wl = W.Workload("crafted", 2, 4, 2, ctx, dtype, (64, 64), "single", 77)
    tot = sum(ctx)
    store_t = np.uint16 if dtype == "bf16" else np.float32
    K = np.zeros((tot, 2, 128), store_t)
    V = np.zeros((tot, 2, 128), store_t)
    cu = np.array([0, ctx[0], tot], np.int64)
    kind_at = 0
    for r in range(2):
        for h in range(2):
            for arr in (K, V):
                for s0 in range(0, ctx[r], 64):
                    rows = min(64, ctx[r] - s0)
                    x = _crafted_segment(rng, SEGMENT_KINDS[kind_at % len(SEGMENT_KINDS)], rows).astype(np.float32)
                    kind_at += 1
                    arr[cu[r] + s0:cu[r] + s0 + rows, h, :] = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    q = rng.standard_normal((2, 4, 128)).astype(np.float32)
    q = W.f32_to_bf16_bits(q) if dtype == "bf16" else q
    inp = W.Inputs(wl, K, V, q, None, cu, np.array([64, 64], np.int32))
    ref = oracle.compress_all(inp)
    # the data reaches the cases it is meant for: every count, subnormal stored values and, for bf16, a
    # 32-channel segment whose vectors span more than 2^14 magnitude patterns
    codes = np.concatenate([s.c for s in ref.values()])
    assert set(np.unique(codes).tolist()) == {128, 64, 32}
    if dtype == "bf16":
        wide32 = False
        for (r, h, X), s in ref.items():
            arr = K if X == 0 else V
            m = arr[cu[r]:cu[r + 1], h, :] & 0x7FFF
            for si, c in enumerate(s.c):
                seg = m[64 * si:64 * si + 64].astype(np.int64)
                wide32 |= bool(c == 32 and np.any(seg.max(1) - seg.min(1) >= (1 << 14)))
        assert wide32
        assert np.any(((K & 0x7F80) == 0) & ((K & 0x7F) != 0))
    else:
        u = K.view(np.uint32)
        assert np.any(((u & 0x7F800000) == 0) & ((u & 0x7FFFFF) != 0))
    store, _ = _compress_gpu(mkv, inp)
    got = read_store(store, inp.dtype)
    _assert_streams_equal(got["streams"], ref)
    assert got["total"] == _closed_form_bytes(ref, inp.dtype) == store.payload_bytes()


def test_selection_output_is_optional_and_padded(mkv):
    """Decode without the selection output gives the same attention output bit for bit; a selection row wider
    than the budget holds the same ascending tokens followed by -1."""
    import torch
    wl = _custom([700, 150, 0], [90, 150, 5], Hq=8, Hkv=2, seed=23)
    inp = W.generate(wl, basis="svd")
    store, q = _compress_gpu(mkv, inp)
    o1, s1 = mkv.mkv_decode_attn(store, q, inp.T)
    o2, s2 = mkv.mkv_decode_attn(store, q, inp.T, return_sel=False)
    o3, s3 = mkv.mkv_decode_attn(store, q, inp.T, sel_stride=s1.shape[-1] + 37)
    torch.cuda.synchronize()
    assert s2 is None
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    w = s1.shape[-1]
    assert torch.equal(s3[..., :w], s1)
    assert bool((s3[..., w:] == -1).all())
    n = np.diff(inp.cu_seqlens)
    for r in range(wl.batch):   # -1 past each request's own selection in the narrow row too
        te = min(int(inp.T[r]), int(n[r]))
        assert bool((s1[r, :, te:] == -1).all())


def test_calls_on_a_side_stream(mkv):
    """Compression and decode enqueued on a stream other than the current one give the default stream's
    results bit for bit once that stream is synchronised."""
    import torch
    wl = _custom([500, 260], [64, 100], Hq=8, Hkv=2, seed=29)
    inp = W.generate(wl, basis="svd")
    K, V, q, basis = inputs_to_torch(inp)
    a = mkv.mkv_compress(K, V, inp.cu_seqlens, basis)
    oa, sa = mkv.mkv_decode_attn(a, q, inp.T)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b = mkv.mkv_compress(K, V, inp.cu_seqlens, basis, stream=side)
        ob, sb = mkv.mkv_decode_attn(b, q, inp.T, stream=side)
    side.synchronize()
    assert b.payload_bytes(stream=side) == a.payload_bytes()
    assert torch.equal(oa, ob) and torch.equal(sa, sb)
