"""Test-side helpers: moving generator inputs to the GPU, reading a compressed store back into its logical
form, writing an oracle-built store in the library's documented layout, and the parity checks."""
from __future__ import annotations

import numpy as np

import workloads as W
from oracle.compress import Stream

D = 128
SEG = 64


# ---- inputs ------------------------------------------------------------------------------------------------
def storage_to_torch(arr: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def inputs_to_torch(inp: W.Inputs, device="cuda"):
    import torch
    K = storage_to_torch(inp.K, inp.dtype, device)
    V = storage_to_torch(inp.V, inp.dtype, device)
    q = storage_to_torch(inp.q, inp.dtype, device)
    basis = None if inp.basis is None else torch.from_numpy(inp.basis).to(device)
    return K, V, q, basis


def f64_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exactly representable float64 values -> storage array (uint16 bf16 patterns or float32)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        bits = x32.view(np.uint32)
        assert not np.any(bits & 0xFFFF), "value not representable in bf16"
        return (bits >> 16).astype(np.uint16)
    return x32


def prerotated_inputs(inp: W.Inputs, streams: dict) -> W.Inputs:
    """Inputs whose K/V are the oracle's rotated and rounded values (for comparisons with basis = NULL)."""
    from oracle import rotate_round
    K = np.zeros_like(inp.K)
    V = np.zeros_like(inp.V)
    cu = inp.cu_seqlens
    for r in range(inp.workload.batch):
        for h in range(inp.workload.n_kv_heads):
            for X, src, dst in ((0, inp.K, K), (1, inp.V, V)):
                x = W.to_f64(src[cu[r]:cu[r + 1], h, :], inp.dtype)
                xh = rotate_round(x, inp.basis[r, h, X], inp.dtype)
                dst[cu[r]:cu[r + 1], h, :] = f64_to_storage(xh, inp.dtype)
    return W.Inputs(inp.workload, K, V, inp.q, None, inp.cu_seqlens, inp.T, inp.sigma)


# ---- store layout -----------------------------------------------------------------------------------------
def seg_counts(cu):
    n = np.diff(np.asarray(cu, dtype=np.int64))
    S_r = (n + SEG - 1) // SEG
    seg_base = np.concatenate([[0], np.cumsum(S_r)[:-1]]).astype(np.int64)
    return n, S_r, seg_base


def segment_id(X, r, h, s, S, Hkv, seg_base, S_r):
    return X * S + Hkv * seg_base[r] + h * S_r[r] + s


def _parse_segment(payload: np.ndarray, off: int, ns: int, c: int, dtype: str):
    """(channel indices [ns][c], values [ns][c] as float64) of one segment whose bytes start at payload[off]."""
    bv = 2 if dtype == "bf16" else 4
    vb = payload[off:off + ns * c * bv]
    v = W.to_f64(vb.view(np.uint16 if bv == 2 else np.float32).reshape(ns, c), dtype)
    if c < D:
        idx = payload[off + ns * c * bv: off + ns * c * (bv + 1)].reshape(ns, c).astype(np.int64)
        assert np.all(np.diff(idx, axis=1) > 0), "channel indices must ascend"
    else:
        idx = np.broadcast_to(np.arange(D), (ns, D))
    return idx, v


def slot_layout(info):
    """(S_r, seg_base) of a store's segment numbering, as the library reports them."""
    B = int(info.batch)
    S_r = np.array([info.seg_slots[i] for i in range(B)], dtype=np.int64)
    seg_base = np.array([info.seg_base[i] for i in range(B)], dtype=np.int64)
    return S_r, seg_base


def check_run_layout(seg_off, sizes, store, bv: int):
    """Segment offsets of a store built by mkv_compress: no two segments overlap and all lie inside the payload;
    bf16 stores of fixed size (one-pass compression) place each segment at its slot's full-size position
    (64 x 128 values per slot) or right after the previous slot's segment (a run of one workgroup); the others
    (two passes) place them back to back in slot order."""
    info = store.view()
    off = np.asarray(seg_off, dtype=np.int64)
    sz = np.asarray(sizes, dtype=np.int64)
    live = sz > 0
    if bv == 2 and not info.growable:
        g = np.arange(off.size, dtype=np.int64)
        at_slot = off == g * (SEG * D * 2)
        after_prev = np.zeros(off.size, dtype=bool)
        after_prev[1:] = off[1:] == off[:-1] + sz[:-1]
        assert np.all((at_slot | after_prev)[live]), "a segment is neither at its slot nor after its predecessor"
    else:
        np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(sz)[:-1]]))
    lo, hi = off[live], off[live] + sz[live]
    o = np.argsort(lo, kind="stable")
    assert np.all(lo[o][1:] >= hi[o][:-1]), "segments overlap"
    assert hi.max(initial=0) <= int(info.payload_capacity)


def _stream_from(payload, codes, seg_off, pay_base, keep, r, h, X, S, Hkv, cu, dtype, layout=None) -> Stream:
    """Stream (r, h, X) of a store: cu gives the tokens in use, layout = (S_r, seg_base) the segment slots
    (None: slots follow cu)."""
    n, S_use, _ = seg_counts(cu)
    if layout is None:
        _, S_r, seg_base = seg_counts(cu)
    else:
        S_r, seg_base = layout
    nr = int(n[r])
    mask = np.zeros((nr, D), dtype=bool)
    vals = np.zeros((nr, D))
    cs = np.zeros(int(S_use[r]), dtype=np.int64)
    cds = np.zeros(int(S_use[r]), dtype=np.int64)
    for s in range(int(S_use[r])):
        g = segment_id(X, r, h, s, S, Hkv, seg_base, S_r)
        code = int(codes[g])
        c = keep[code]
        cds[s], cs[s] = code, c
        ns = min(SEG, nr - s * SEG)
        idx, v = _parse_segment(payload, int(seg_off[g]) - pay_base, ns, c, dtype)
        rows = np.arange(s * SEG, s * SEG + ns)[:, None]
        mask[rows, idx] = True
        vals[rows, idx] = v
    return Stream(nr, D, cds, cs, mask, vals)


def read_store(store, dtype: str) -> dict:
    """Copies a device store to the host and decodes it into {(r, h, X): Stream}; also returns raw arrays."""
    info = store.view()
    keep = tuple(info.policy.keep[i] for i in range(info.policy.n_keep))
    S = int(info.segments_per_tensor)
    Hkv = int(info.n_kv_heads)
    buf = store.buf.cpu().numpy()
    base = store.buf.data_ptr()
    o_codes = info.codes - base
    o_off = info.seg_off - base
    o_pay = info.payload - base
    codes = buf[o_codes:o_codes + 2 * S].copy()
    seg_off = buf[o_off:o_off + 16 * S].view(np.uint64).copy()
    total = int(buf[0:8].view(np.uint64)[0])
    payload = buf[o_pay:]          # packed segments, then (growable stores) the open-segment areas
    B = int(info.batch)
    cu = np.array([info.cu_seqlens[i] for i in range(B + 1)], dtype=np.int64)
    layout = slot_layout(info)
    n, _, _ = seg_counts(cu)
    out = {}
    for r in range(len(n)):
        for h in range(Hkv):
            for X in (0, 1):
                out[(r, h, X)] = _stream_from(payload, codes, seg_off, 0, keep, r, h, X, S, Hkv, cu, dtype, layout)
    return {"streams": out, "codes": codes, "seg_off": seg_off, "total": total, "S": S}


class StoreReader:
    """Reads a large device store piecewise: its metadata once, then one stream's payload at a time."""

    def __init__(self, store, dtype: str):
        info = store.view()
        self.store, self.dtype = store, dtype
        self.keep = tuple(info.policy.keep[i] for i in range(info.policy.n_keep))
        self.S = int(info.segments_per_tensor)
        self.Hkv = int(info.n_kv_heads)
        base = store.buf.data_ptr()
        self.o_pay = info.payload - base
        o_codes, o_off = info.codes - base, info.seg_off - base
        self.codes = store.buf[o_codes:o_codes + 2 * self.S].cpu().numpy().copy()
        self.seg_off = store.buf[o_off:o_off + 16 * self.S].cpu().numpy().view(np.uint64).copy()
        self.total = int(store.buf[0:8].cpu().numpy().view(np.uint64)[0])
        B = int(info.batch)
        self.cu = np.array([info.cu_seqlens[i] for i in range(B + 1)], dtype=np.int64)
        self.layout = slot_layout(info)

    def segment_bytes(self, bv: int) -> np.ndarray:
        """Payload bytes of every segment slot implied by its code (K slots, then V slots; 0 for unused slots)."""
        n, S_use, _ = seg_counts(self.cu)
        S_r, seg_base = self.layout
        ns = np.zeros(2 * self.S, dtype=np.int64)
        for X in (0, 1):
            for r in range(len(n)):
                per = np.full(int(S_use[r]), SEG, dtype=np.int64)
                if S_use[r]:
                    per[-1] = int(n[r]) - (int(S_use[r]) - 1) * SEG
                for h in range(self.Hkv):
                    g0 = segment_id(X, r, h, 0, self.S, self.Hkv, seg_base, S_r)
                    ns[g0:g0 + int(S_use[r])] = per
        c = np.asarray(self.keep, dtype=np.int64)[self.codes.astype(np.int64) % len(self.keep)]
        return ns * c * (bv + (c < D))

    def stream(self, r: int, h: int, X: int) -> Stream:
        n, S_use, _ = seg_counts(self.cu)
        S_r, seg_base = self.layout
        if S_use[r] == 0:
            return Stream(0, D, np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros((0, D), bool), np.zeros((0, D)))
        g0 = segment_id(X, r, h, 0, self.S, self.Hkv, seg_base, S_r)
        g1 = g0 + int(S_use[r]) - 1
        bv = 2 if self.dtype == "bf16" else 4
        if getattr(self, "_sizes", None) is None:
            self._sizes = self.segment_bytes(bv)
        # the stream's segments lie in one payload range unless appends placed some elsewhere
        offs = self.seg_off[g0:g1 + 1].astype(np.int64)
        lo = int(offs.min())
        hi = int(max(int(o) + int(sz) for o, sz in zip(offs, self._sizes[g0:g1 + 1])))
        payload = self.store.buf[self.o_pay + lo:self.o_pay + hi].cpu().numpy()
        return _stream_from(payload, self.codes, self.seg_off, lo, self.keep, r, h, X, self.S, self.Hkv,
                            self.cu, self.dtype, self.layout)


def pack_oracle_store(streams: dict, cu, Hkv: int, dtype: str, keep: tuple):
    """Lays an oracle store out as the library documents it: (codes [2S], seg_off [2S], payload bytes)."""
    n, S_r, seg_base = seg_counts(cu)
    S = int(S_r.sum()) * Hkv
    bv = 2 if dtype == "bf16" else 4
    codes = np.zeros(2 * S, dtype=np.uint8)
    sizes = np.zeros(2 * S, dtype=np.uint64)
    pieces = {}
    for (r, h, X), st in streams.items():
        for s in range(int(S_r[r])):
            g = segment_id(X, r, h, s, S, Hkv, seg_base, S_r)
            c = int(st.c[s])
            codes[g] = keep.index(c)
            ns = min(SEG, int(n[r]) - s * SEG)
            rows = slice(s * SEG, s * SEG + ns)
            m = st.mask[rows]
            idx = np.nonzero(m)[1].reshape(ns, c)
            vals = np.take_along_axis(st.vals[rows], idx, axis=1)
            blob = f64_to_storage(vals, dtype).tobytes()
            if c < D:
                blob += idx.astype(np.uint8).tobytes()
            pieces[g] = blob
            sizes[g] = len(blob)
    seg_off = np.zeros(2 * S, dtype=np.uint64)
    seg_off[1:] = np.cumsum(sizes)[:-1]
    payload = b"".join(pieces[g] for g in range(2 * S))
    return codes, seg_off, np.frombuffer(payload, dtype=np.uint8)


def upload_oracle_store(streams, inp: W.Inputs, keep, device="cuda"):
    """Writes an oracle store into a fresh store buffer and attaches a library handle to it."""
    import torch
    import kv_cache_compression_svd_amd as mkv
    w = inp.workload
    dt = mkv.MKV_BF16 if inp.dtype == "bf16" else mkv.MKV_FP32
    pol = mkv.SegPolicy.make(keep)
    sb, _ = mkv.mkv_compress_bytes(None, None, inp.cu_seqlens, pol, n_kv_heads=w.n_kv_heads, dtype=dt)
    raw = torch.zeros(sb + 256, dtype=torch.uint8, device=device)
    pad = (-raw.data_ptr()) % 256          # the library wants 256-byte alignment (host buffers may lack it)
    buf = raw[pad:pad + sb]
    store = mkv.mkv_store_attach(inp.cu_seqlens, w.n_kv_heads, dt, pol, inp.basis is not None, buf)
    info = store.view()
    codes, seg_off, payload = pack_oracle_store(streams, inp.cu_seqlens, w.n_kv_heads, inp.dtype, keep)
    base = buf.data_ptr()
    host = np.zeros(sb, dtype=np.uint8)
    host[0:8] = np.frombuffer(np.uint64(payload.size).tobytes(), dtype=np.uint8)
    host[info.codes - base: info.codes - base + codes.size] = codes
    host[info.seg_off - base: info.seg_off - base + seg_off.size * 8] = seg_off.view(np.uint8)
    if inp.basis is not None:
        bb = inp.basis.astype(np.float32).tobytes()
        o_basis = info.basis - base
        host[o_basis:o_basis + len(bb)] = np.frombuffer(bb, dtype=np.uint8)
    host[info.payload - base: info.payload - base + payload.size] = payload
    buf.copy_(torch.from_numpy(host))
    return store


# ---- parity checks ----------------------------------------------------------------------------------------
def kth_score(scores: np.ndarray, t: int) -> float:
    order = np.lexsort((np.arange(scores.size), -scores))
    return float(scores[order[t - 1]])


def check_selection(sel_row: np.ndarray, ref_sel: np.ndarray, scores: np.ndarray, T_eff: int, band=1e-5):
    """GPU selection == oracle selection, except tokens whose oracle score lies within band * |s_T| of the
    T-th score; ascending order; -1 after T_eff.  Returns the number of differing tokens."""
    got = np.asarray(sel_row[:T_eff])
    assert np.all(np.asarray(sel_row[T_eff:]) == -1), "padding after the selection must be -1"
    assert got.size == T_eff
    if T_eff == 0:
        return 0
    assert np.all(np.diff(got) > 0), "selection must be strictly ascending"
    assert got.min() >= 0 and got.max() < scores.size
    diff = np.setxor1d(got, ref_sel)
    if diff.size:
        sT = kth_score(scores, T_eff)
        bad = diff[np.abs(scores[diff] - sT) > band * abs(sT)]
        assert bad.size == 0, f"selection differs outside the near-tie band at tokens {bad[:10]}"
    return int(diff.size)


def valid_selections(scores: np.ndarray, T_eff: int, band=1e-5, cap=64):
    """Every selection the near-tie rule accepts, in ascending order: the tokens scoring above the band around
    the T-th score, plus any choice of the remaining count among the tokens inside it.  The score estimate is
    a sum over the group's heads, so a token at the threshold can still weigh in one head's softmax: each
    accepted selection has its own exact output.  None when there are more than ``cap`` selections."""
    from itertools import combinations
    from math import comb
    if T_eff == 0:
        return [np.zeros(0, dtype=np.int64)]
    sT = kth_score(scores, T_eff)
    tol = band * abs(sT)
    above = np.nonzero(scores > sT + tol)[0]
    inband = np.nonzero(np.abs(scores - sT) <= tol)[0]
    k = T_eff - above.size
    if comb(inband.size, k) > cap:
        return None
    return [np.sort(np.concatenate([above, np.asarray(c, dtype=np.int64)])) for c in combinations(inband, k)]


def check_decode_unit(sel_row, out_rows, q_group, basis_k, basis_v, kstream, vstream, T_eff: int) -> int:
    """One (request, KV head) unit against the oracle on the same store: the selection must be one the
    near-tie rule accepts, and the output must match the oracle's output for that same accepted selection
    (the oracle enumerates the accepted selections itself).  Returns the number of tokens that differ from
    the oracle's own first choice; -1 when the band held too many ties to enumerate (output not compared)."""
    from oracle import attend, decode_unit, rotate_queries
    res = decode_unit(q_group, basis_k, basis_v, kstream, vstream, T_eff)
    nd = check_selection(sel_row, res["sel"], res["scores"], T_eff)
    if nd == 0:
        check_out(out_rows, res["out"])
        return 0
    sels = valid_selections(res["scores"], T_eff)
    if sels is None:
        return -1
    got = np.asarray(sel_row[:T_eff], dtype=np.int64)
    match = [s for s in sels if np.array_equal(s, got)]
    assert match, "selection is not one of the accepted near-tie selections"
    qp = rotate_queries(q_group, basis_k)
    ref = attend(qp, kstream.vals[match[0]], vstream.vals[match[0]])
    if basis_v is not None:
        ref = ref @ np.asarray(basis_v, dtype=np.float64).T
    check_out(out_rows, ref)
    return nd


def check_out(out: np.ndarray, ref: np.ndarray, rel=2e-3):
    """Per query head: relative L2 error <= rel and every element within rel * max|ref row|."""
    for h in range(ref.shape[0]):
        nr = np.linalg.norm(ref[h])
        err = np.linalg.norm(out[h] - ref[h])
        assert err <= rel * max(nr, 1e-30), f"head {h}: rel-L2 {err / max(nr, 1e-30):.3e} > {rel}"
        assert np.max(np.abs(out[h] - ref[h])) <= rel * max(np.max(np.abs(ref[h])), 1e-30), f"head {h}: elementwise"


# ---- SVD-basis compression: every difference from the oracle needs a reason ----------------------------------
# With a true SVD basis the GPU rotates in float32 (MFMA) and the oracle in float64, so a stored value may differ
# by one storage ulp.  A differing segment code or kept set is accepted only where such a difference can move the
# decision: the bound is taken from the value differences actually observed (both sides read back).
def ulp(x, dtype: str) -> np.ndarray:
    """Spacing of the storage dtype at |x| (the spacing at 1.0 for x = 0)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.exp2(e - (7 if dtype == "bf16" else 23))


def observed_ulps(got_vals: np.ndarray, ref_vals: np.ndarray, both: np.ndarray, dtype: str) -> float:
    """Largest |GPU value - oracle value| over the channels both sides kept, in ulps of the oracle value."""
    if not np.any(both):
        return 0.0
    d = np.abs(got_vals[both] - ref_vals[both]) / ulp(ref_vals[both], dtype)
    return float(d.max())


def energy_flip_bound(xhat: np.ndarray, m: float, dtype: str, frac: float = 0.9) -> np.ndarray:
    """Per vector of xhat [n][d]: the largest |E_c/E_all - frac| at which moving every element by at most m ulp
    can flip the decision E_c >= frac * E_all, for any c.  Each square moves by at most 2|x|u + u^2 (u = m ulp);
    E_c (a maximum over c-subsets) and E_all each move by at most the sum of those, so frac * E_all - E_c moves
    by at most (1 + frac) times it."""
    u = m * ulp(xhat, dtype)
    dsq = np.sum(2.0 * np.abs(xhat) * u + u * u, axis=1)
    e_all = np.sum(xhat * xhat, axis=1)
    return (1.0 + frac) * dsq / np.where(e_all > 0, e_all, 1.0)


def code_difference_reason(xhat: np.ndarray, code_got: int, code_ref: int, keep, m: float, dtype: str,
                           frac: float = 0.9):
    """Index of a vector of the segment xhat [ns][d] whose decision at the count that separates the two codes
    lies inside the observed rotation error, on the side that explains the difference; None if there is none.
    GPU code above the oracle's (fewer channels): some vector is inadmissible for the oracle at that count.
    GPU code below: some vector the oracle admits must have been refused by the GPU."""
    import oracle
    c = keep[max(code_got, code_ref)]
    e_all = np.sum(xhat * xhat, axis=1)
    ratio = oracle.kept_energy(xhat, oracle.channel_order(xhat), c) / np.where(e_all > 0, e_all, 1.0)
    bound = energy_flip_bound(xhat, m, dtype, frac)
    side = (ratio < frac) if code_got > code_ref else (ratio >= frac)
    ok = np.nonzero(side & (np.abs(ratio - frac) <= bound) & (e_all > 0))[0]
    return int(ok[0]) if ok.size else None


def channel_swap_reason(xhat_row: np.ndarray, got_mask: np.ndarray, ref_mask: np.ndarray, c: int, m: float,
                        dtype: str) -> bool:
    """A token whose kept set differs at the same count c: every swapped channel's oracle magnitude must lie
    within 2 m ulp of the oracle's c-th largest magnitude (a GPU ranking of a above b with |x_a| <= t <= |x_b|
    needs |x_b| - |x_a| <= m (ulp_a + ulp_b))."""
    mags = np.abs(xhat_row)
    tc = np.sort(mags)[::-1][c - 1]
    swapped = np.nonzero(got_mask != ref_mask)[0]
    return bool(np.all(np.abs(mags[swapped] - tc) <= 2.0 * m * ulp(np.array([tc]), dtype)[0] + 1e-300))


def record_parity(test: str, case: str, **counts):
    """Appends the counts of a parity test to the JSON-lines file named by MKV_PARITY_LOG (if set)."""
    import json
    import os
    path = os.environ.get("MKV_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"test": test, "case": case, **counts}) + "\n")
