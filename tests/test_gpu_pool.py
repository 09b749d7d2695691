"""Paged pools: requests compressed into fixed-size pages of one buffer, removed, and decoded together through
views.  A request in the pool holds exactly the segments a plain store of the same request holds (codes,
channel sets and values, bit for bit), so decoding a view equals decoding a plain store of the listed requests
in that order, bit for bit, wherever the pages lie; with a signed-permutation basis the pool's segments also
equal the oracle's compression, and a view's decode passes the oracle check unit by unit.  Cases: page sizes
that hold one, a few or many segments (segments never straddle pages), ids, slots and pages reused after
removals in a fragmented pool, views in any order and subsets, adds refused for want of pages or of a long
enough run of slots (the pool is left as it was), empty requests, and fp32."""
import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import check_decode_unit, inputs_to_torch, read_store

pytestmark = pytest.mark.gpu

SEG = 64


@pytest.fixture(scope="module")
def mkv_lib():
    import kv_cache_compression_svd_amd as m
    m.lib()
    return m


def _wl(ctx, seed, T=40, dtype="bf16"):
    return W.Workload(f"pool{len(ctx)}", len(ctx), 16, 4, tuple(ctx), dtype, (T,) * len(ctx), "per_request", seed,
                      "pool case")


class Reqs:
    """Generated requests on the GPU, addressable one by one."""

    def __init__(self, ctx, seed, basis="svd", dtype="bf16", T=40):
        import torch
        self.inp = W.generate(_wl(ctx, seed, T, dtype), basis=basis)
        self.K, self.V, self.q, self.basis = inputs_to_torch(self.inp)
        self.cu = self.inp.cu_seqlens
        self.dtype = dtype
        self.T = np.asarray(self.inp.T)
        self.torch = torch

    def pick(self, idx):
        """(K, V, cu, basis, q, T) of the listed requests, in this order."""
        torch = self.torch
        idx = list(idx)
        tok = [np.arange(self.cu[r], self.cu[r + 1]) for r in idx]
        take = torch.as_tensor(np.concatenate(tok) if tok else np.zeros(0, np.int64), device="cuda")
        cu = np.concatenate([[0], np.cumsum([len(t) for t in tok])]).astype(np.int64)
        ii = torch.as_tensor(idx, device="cuda")
        basis = None if self.basis is None else self.basis[ii].contiguous()
        return (self.K[take].contiguous(), self.V[take].contiguous(), cu, basis, self.q[ii].contiguous(),
                self.T[idx])


def _pool(mkv, n_pages, page_bytes, slots, max_req=16, dtype="bf16", has_basis=True, appendable=False):
    code = mkv.MKV_BF16 if dtype == "bf16" else mkv.MKV_FP32
    return mkv.Pool(4, code, max_req, slots, n_pages, page_bytes, has_basis=has_basis, appendable=appendable)


def _same_as_plain(mkv, pool, ids, R, order, dtype="bf16"):
    """View of `ids` against a plain store of requests `order` of R: segments and decode, bit for bit."""
    import torch
    view = pool.view(ids)
    K, V, cu, basis, q, T = R.pick(order)
    ref = mkv.mkv_compress(K, V, cu, basis)
    assert np.array_equal(view.cu, cu)
    g, f = read_store(view, dtype)["streams"], read_store(ref, dtype)["streams"]
    assert g.keys() == f.keys()
    for key in f:
        assert np.array_equal(g[key].c, f[key].c), key
        assert np.array_equal(g[key].mask, f[key].mask), key
        assert np.array_equal(g[key].vals, f[key].vals), key
    o1, s1 = mkv.mkv_decode_attn(view, q, T)
    o2, s2 = mkv.mkv_decode_attn(ref, q, T)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(o1, o2)
    return view


def _check_placement(pool, views, dtype="bf16"):
    """Every segment of the listed views lies inside one page, and no two segments overlap."""
    info = pool.stats()
    pb = int(info.desc.page_bytes)
    bv = 2 if dtype == "bf16" else 4
    spans = []
    for view in views:
        vi = view.view()
        S = int(vi.segments_per_tensor)
        keep = [vi.policy.keep[i] for i in range(vi.policy.n_keep)]
        base = pool.buf.data_ptr()
        codes = pool.buf[vi.codes - base:vi.codes - base + 2 * S].cpu().numpy()
        offs = pool.buf[vi.seg_off - base:vi.seg_off - base + 16 * S].cpu().numpy().view(np.uint64)
        for r in range(int(vi.batch)):
            n = int(vi.cu_seqlens[r + 1] - vi.cu_seqlens[r])
            for X in (0, 1):
                for h in range(int(vi.n_kv_heads)):
                    for s in range((n + SEG - 1) // SEG):
                        g = X * S + vi.n_kv_heads * vi.seg_base[r] + h * vi.seg_slots[r] + s
                        c = keep[int(codes[g])]
                        nb = min(SEG, n - s * SEG) * c * (bv + (c < 128))
                        o = int(offs[g])
                        if o >= int(info.desc.n_pages) * pb:   # an open segment, in its stream's open area
                            assert o + nb <= int(info.pool_bytes)
                        else:
                            assert o // pb == (o + nb - 1) // pb, "segment straddles two pages"
                            assert o + nb <= int(info.desc.n_pages) * pb
                        spans.append((o, o + nb))
    spans = sorted(set(spans))
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0, "segments overlap"


@pytest.mark.parametrize("page_bytes", [16384, 40960, 1 << 20])
def test_pool_holds_what_a_plain_store_holds(mkv_lib, page_bytes):
    mkv = mkv_lib
    R = Reqs([300, 64, 1000, 1], seed=71)
    n_pages = max(40, (16 << 20) // page_bytes)     # every non-empty stream takes at least one page
    pool = _pool(mkv, n_pages=n_pages, page_bytes=page_bytes, slots=64)
    ids = pool.add(*R.pick([0, 1, 2, 3])[:4])
    assert sorted(ids.tolist()) == [0, 1, 2, 3]
    view = _same_as_plain(mkv, pool, ids, R, [0, 1, 2, 3])
    _check_placement(pool, [view])
    # a view lists any subset in any order
    _same_as_plain(mkv, pool, [ids[2], ids[0]], R, [2, 0])
    info = pool.stats()
    used = sum(pool.request(int(i))[1] for i in ids)
    assert info.free_pages == n_pages - used and info.live_requests == 4
    assert view.payload_bytes() == sum(pool.request(int(i))[2] for i in ids)


def test_removal_reuses_ids_slots_and_pages(mkv_lib):
    mkv = mkv_lib
    R = Reqs([500, 260, 130, 700, 64, 900], seed=72)
    # 16 KiB pages hold one uncompressed segment: page counts follow the segment sizes closely
    pool = _pool(mkv, n_pages=700, page_bytes=16384, slots=45, max_req=5)
    a = pool.add(*R.pick([0, 1])[:4])
    b = pool.add(*R.pick([2])[:4])
    c = pool.add(*R.pick([3, 4])[:4])
    free0 = pool.stats().free_pages
    pages_b = pool.request(int(b[0]))[1] + pool.request(int(a[1]))[1]
    pool.remove([b[0], a[1]])
    st = pool.stats()
    assert st.free_pages == free0 + pages_b and st.live_requests == 3
    # 900 tokens need a run of 15 slots: the freed runs of requests 1 and 2 merge into 8, so it takes the tail (17)
    d = pool.add(*R.pick([5])[:4])
    assert d[0] in (int(b[0]), int(a[1]))   # a freed id comes back
    view = _same_as_plain(mkv, pool, [d[0], c[1], a[0], c[0]], R, [5, 4, 0, 3])
    _check_placement(pool, [view])
    # the freed runs are reused by requests that fit them
    e = pool.add(*R.pick([1])[:4])
    _same_as_plain(mkv, pool, [e[0], a[0]], R, [1, 0])


def test_refused_adds_leave_the_pool_unchanged(mkv_lib):
    mkv = mkv_lib
    R = Reqs([640, 640, 200], seed=73)
    # the pages requests 0 and 1 take, measured in a roomy pool; the tight pool holds request 0 and one page
    # less than request 1 needs
    roomy = _pool(mkv, n_pages=400, page_bytes=16384, slots=64)
    p0, p1 = (roomy.request(int(roomy.add(*R.pick([r])[:4])[0]))[1] for r in (0, 1))
    pool = _pool(mkv, n_pages=p0 + p1 - 1, page_bytes=16384, slots=22, max_req=4)
    a = pool.add(*R.pick([0])[:4])
    before = pool.stats()
    snap = (before.free_pages, before.free_segment_slots, before.largest_free_run, before.live_requests)
    # pages: request 1 needs p1 pages, p1 - 1 are free
    with pytest.raises(mkv.MkvError) as ei:
        pool.add(*R.pick([1])[:4])
    assert ei.value.status == mkv.MKV_E_ARG and "pages" in str(ei.value)
    st = pool.stats()
    assert (st.free_pages, st.free_segment_slots, st.largest_free_run, st.live_requests) == snap
    # slots: 200 tokens take 4 of the 12 free slots, then 640 tokens find no run of 10 (that add is undone)
    with pytest.raises(mkv.MkvError) as ei:
        pool.add(*R.pick([2, 1])[:4])
    assert ei.value.status == mkv.MKV_E_ARG and "slots" in str(ei.value)
    st = pool.stats()
    assert (st.free_pages, st.free_segment_slots, st.largest_free_run, st.live_requests) == snap
    # what fits still goes in, and the earlier request is intact
    b = pool.add(*R.pick([2])[:4])
    _same_as_plain(mkv, pool, [a[0], b[0]], R, [0, 2])


def test_empty_requests_and_fp32(mkv_lib):
    mkv = mkv_lib
    R = Reqs([0, 190, 0, 64], seed=74, dtype="fp32")
    pool = _pool(mkv, n_pages=64, page_bytes=32768 * 2, slots=16, dtype="fp32")
    ids = pool.add(*R.pick([0, 1, 2, 3])[:4])
    assert pool.request(int(ids[0]))[:2] == (0, 0)
    view = _same_as_plain(mkv, pool, ids, R, [0, 1, 2, 3], dtype="fp32")
    _check_placement(pool, [view], dtype="fp32")


def test_pool_against_the_oracle(mkv_lib):
    """Signed-permutation basis: the pool's segments equal the oracle's compression bit for bit, and a view's
    decode passes the oracle check for every (request, KV head)."""
    mkv = mkv_lib
    import torch
    R = Reqs([333, 128, 77], seed=75, basis="sperm", T=50)
    pool = _pool(mkv, n_pages=512, page_bytes=20480, slots=32)
    first = pool.add(*R.pick([1])[:4])
    rest = pool.add(*R.pick([0, 2])[:4])
    order = [rest[0], first[0], rest[1]]
    src = [0, 1, 2]
    view = pool.view(order)
    got = read_store(view, "bf16")["streams"]
    inp = R.inp
    cu = inp.cu_seqlens
    for vr, r in enumerate(src):
        for h in range(4):
            for X, arr in ((0, inp.K), (1, inp.V)):
                ref = oracle.compress_stream(W.to_f64(arr[cu[r]:cu[r + 1], h, :], "bf16"), inp.basis[r, h, X], "bf16")
                g = got[(vr, h, X)]
                assert np.array_equal(g.c, ref.c) and np.array_equal(g.mask, ref.mask) and np.array_equal(g.vals, ref.vals)
    _, _, _, _, q, T = R.pick(src)
    out, sel = mkv.mkv_decode_attn(view, q, T)
    torch.cuda.synchronize()
    out, sel = out.cpu().numpy().astype(np.float64), sel.cpu().numpy()
    G = 4
    for vr, r in enumerate(src):
        n = int(cu[r + 1] - cu[r])
        for h in range(4):
            qg = W.to_f64(inp.q[r, h * G:(h + 1) * G, :], "bf16")
            nd = check_decode_unit(sel[vr, h], out[vr, h * G:(h + 1) * G], qg, inp.basis[r, h, 0], inp.basis[r, h, 1],
                                   got[(vr, h, 0)], got[(vr, h, 1)], min(int(T[vr]), n))
            assert nd >= 0


def _grow_in_pool(mkv, R, n0, steps, pool, active_of=None):
    """Adds the first n0[r] tokens of each request of R with their full contexts as capacities, then appends
    `steps` tokens (request r takes part in step k when active_of(k)[r]); returns the ids and token counts."""
    import torch
    cu = R.cu
    B = len(n0)
    take = torch.as_tensor(np.concatenate([np.arange(cu[r], cu[r] + n0[r]) for r in range(B)]), device="cuda")
    cu0 = np.concatenate([[0], np.cumsum(n0)]).astype(np.int64)
    cap = np.diff(cu)
    ids = pool.add(R.K[take].contiguous(), R.V[take].contiguous(), cu0, R.basis, capacity=cap)
    n = np.array(n0)
    for k in range(steps):
        act = np.ones(B, dtype=bool) if active_of is None else np.asarray(active_of(k), dtype=bool)
        act &= n < cap
        rs = np.nonzero(act)[0]
        if rs.size == 0:
            continue
        rows = torch.as_tensor(cu[:-1][rs] + n[rs], device="cuda")
        pool.append(ids[rs], R.K[rows].contiguous(), R.V[rows].contiguous())
        n[rs] += 1
    torch.cuda.synchronize()
    for r in range(B):
        assert pool.request(int(ids[r]))[0] == n[r] and pool.capacity(int(ids[r])) == cap[r]
    return ids, n


def _same_as_plain_prefix(mkv, pool, ids, R, n, dtype="bf16"):
    """A view of the grown requests against compressing their first n[r] tokens at once: segments and decode."""
    import torch
    cu = R.cu
    B = len(n)
    view = pool.view(ids)
    assert np.array_equal(np.diff(view.cu), n)
    take = torch.as_tensor(np.concatenate([np.arange(cu[r], cu[r] + n[r]) for r in range(B)]), device="cuda")
    ref = mkv.mkv_compress(R.K[take].contiguous(), R.V[take].contiguous(), np.concatenate([[0], np.cumsum(n)]),
                           R.basis)
    g, f = read_store(view, dtype)["streams"], read_store(ref, dtype)["streams"]
    for key in f:
        assert np.array_equal(g[key].c, f[key].c), key
        assert np.array_equal(g[key].mask, f[key].mask), key
        assert np.array_equal(g[key].vals, f[key].vals), key
    o1, s1 = mkv.mkv_decode_attn(view, R.q, R.T)
    o2, s2 = mkv.mkv_decode_attn(ref, R.q, R.T)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(o1, o2)
    return view


@pytest.mark.parametrize("n0,steps", [([64, 100, 0], 70), ([1, 63, 128], 66)])
def test_pool_appends_equal_compressing_the_extended_context(mkv_lib, n0, steps):
    mkv = mkv_lib
    R = Reqs([a + steps for a in n0], seed=76)
    pool = _pool(mkv, n_pages=200, page_bytes=40960, slots=64, appendable=True)
    ids, n = _grow_in_pool(mkv, R, n0, steps, pool)
    view = _same_as_plain_prefix(mkv, pool, ids, R, n)
    _check_placement(pool, [view])


def test_pool_appends_to_a_subset_then_removal(mkv_lib):
    mkv = mkv_lib
    R = Reqs([150, 90, 70], seed=77)
    pool = _pool(mkv, n_pages=300, page_bytes=16384, slots=32, max_req=4, appendable=True)
    free0 = pool.stats().free_pages
    ids, n = _grow_in_pool(mkv, R, [60, 20, 63], 80, pool, active_of=lambda k: [k % 2 == 0, True, k < 3])
    _same_as_plain_prefix(mkv, pool, ids, R, n)
    # the request at its capacity refuses one more token, and nothing changes
    full = [r for r in range(3) if n[r] == np.diff(R.cu)[r]]
    assert full
    import torch
    before = pool.stats().free_pages
    with pytest.raises(mkv.MkvError) as ei:
        rows = torch.as_tensor([R.cu[full[0]]], device="cuda")
        pool.append(ids[full[:1]], R.K[rows].contiguous(), R.V[rows].contiguous())
    assert ei.value.status == mkv.MKV_E_ARG and "capacity" in str(ei.value)
    assert pool.stats().free_pages == before and pool.request(int(ids[full[0]]))[0] == n[full[0]]
    pool.remove(ids)
    st = pool.stats()
    assert st.free_pages == free0 and st.live_requests == 0 and st.free_segment_slots == 32


def test_pool_append_refused_without_pages(mkv_lib):
    """An append that would seal segments with no page left fails before anything is enqueued."""
    mkv = mkv_lib
    import torch
    R2 = Reqs([200], seed=78)
    cu0 = np.array([0, 127], dtype=np.int64)
    # the pages the first 127 tokens take, measured in a roomy pool; the tight pool has exactly those, so none is
    # spare for the 8 segments (4 KV heads x 2 tensors) that the 128th token seals
    probe = _pool(mkv, n_pages=64, page_bytes=16384, slots=8, appendable=True)
    p127 = probe.request(int(probe.add(R2.K[:127].contiguous(), R2.V[:127].contiguous(), cu0, R2.basis,
                                       capacity=[200])[0]))[1]
    pool = _pool(mkv, n_pages=p127, page_bytes=16384, slots=8, appendable=True)
    ids = pool.add(R2.K[:127].contiguous(), R2.V[:127].contiguous(), cu0, R2.basis, capacity=[200])
    assert pool.stats().free_pages == 0
    rows = torch.as_tensor([127], device="cuda")
    with pytest.raises(mkv.MkvError) as ei:
        pool.append(ids, R2.K[rows].contiguous(), R2.V[rows].contiguous())
    assert ei.value.status == mkv.MKV_E_ARG and "pages" in str(ei.value)
    assert pool.request(int(ids[0]))[0] == 127
    _same_as_plain_prefix(mkv, pool, ids, R2, np.array([127]))


def test_random_pool_lifecycle(mkv_lib):
    """A seeded sequence of adds (some with capacities), appends to random subsets and removals on a small,
    fragmenting pool: after every few operations each live request still holds exactly what compressing its
    current tokens gives, no two live segments overlap, and the pool's counts add up."""
    mkv = mkv_lib
    import torch
    rng = np.random.default_rng(2024)
    ctx = [int(x) for x in rng.integers(1, 260, size=12)]
    R = Reqs([c + 130 for c in ctx], seed=79)          # each request's full token supply
    n_pages, slots = 400, 96
    pool = _pool(mkv, n_pages=n_pages, page_bytes=20480, slots=slots, max_req=6, appendable=True)
    live = {}                                           # id -> (request index in R, tokens held)
    unused = list(range(12))
    done = {"add": 0, "append": 0, "seal": 0, "remove": 0}

    def check():
        if not live:
            return
        ids = list(live)
        view = pool.view(ids)
        n = np.array([live[i][1] for i in ids])
        rows = [np.arange(R.cu[live[i][0]], R.cu[live[i][0]] + live[i][1]) for i in ids]
        take = torch.as_tensor(np.concatenate(rows), device="cuda")
        ii = torch.as_tensor([live[i][0] for i in ids], device="cuda")
        ref = mkv.mkv_compress(R.K[take].contiguous(), R.V[take].contiguous(), np.concatenate([[0], np.cumsum(n)]),
                               R.basis[ii].contiguous())
        g, f = read_store(view, "bf16")["streams"], read_store(ref, "bf16")["streams"]
        for key in f:
            assert np.array_equal(g[key].c, f[key].c) and np.array_equal(g[key].mask, f[key].mask), key
            assert np.array_equal(g[key].vals, f[key].vals), key
        q = R.q[ii].contiguous()
        T = np.full(len(ids), 40)
        o1, s1 = mkv.mkv_decode_attn(view, q, T)
        o2, s2 = mkv.mkv_decode_attn(ref, q, T)
        torch.cuda.synchronize()
        assert torch.equal(s1, s2) and torch.equal(o1, o2)
        _check_placement(pool, [view])
        st = pool.stats()
        assert st.live_requests == len(live)
        assert st.free_pages + sum(pool.request(i)[1] for i in ids) == n_pages
        assert st.free_segment_slots + sum((pool.capacity(i) + 63) // 64 for i in ids) == slots

    for step in range(40):
        op = rng.choice(["add", "append", "append", "remove"]) if live else "add"
        if op == "add" and unused and len(live) < 6:
            k = min(int(rng.integers(1, 3)), len(unused), 6 - len(live))
            picks = [unused.pop(int(rng.integers(len(unused)))) for _ in range(k)]
            K, V, cu, basis, _, _ = R.pick(picks)
            cap = [ctx[p] + int(rng.integers(0, 131)) for p in picks]
            n0 = [min(ctx[p], c) for p, c in zip(picks, cap)]
            take = torch.as_tensor(np.concatenate([np.arange(R.cu[p], R.cu[p] + a) for p, a in zip(picks, n0)]),
                                   device="cuda")
            try:
                ids = pool.add(R.K[take].contiguous(), R.V[take].contiguous(), np.concatenate([[0], np.cumsum(n0)]),
                               basis, capacity=cap)
            except mkv.MkvError as e:   # out of slots or pages: the pool must be unchanged
                assert e.status == mkv.MKV_E_ARG
                unused += picks
                continue
            for i, p, a in zip(ids, picks, n0):
                live[int(i)] = (p, a)
            done["add"] += len(picks)
        elif op == "append":
            ids = [i for i in live if live[i][1] < pool.capacity(i) and rng.random() < 0.7]
            for _ in range(int(rng.integers(1, 40))):
                ids = [i for i in ids if live[i][1] < pool.capacity(i)]
                if not ids:
                    break
                rows = torch.as_tensor([R.cu[live[i][0]] + live[i][1] for i in ids], device="cuda")
                try:
                    pool.append(ids, R.K[rows].contiguous(), R.V[rows].contiguous())
                except mkv.MkvError as e:   # out of pages for a sealed segment
                    assert e.status == mkv.MKV_E_ARG and "pages" in str(e)
                    break
                for i in ids:
                    live[i] = (live[i][0], live[i][1] + 1)
                    done["append"] += 1
                    done["seal"] += live[i][1] % 64 == 0
        elif op == "remove" and live:
            gone = [i for i in live if rng.random() < 0.4] or [next(iter(live))]
            pool.remove(gone)
            for i in gone:
                unused.append(live.pop(i)[0])
            done["remove"] += len(gone)
        if step % 5 == 4:
            check()
    check()
    assert min(done.values()) > 0, done


@pytest.mark.parametrize("page_bytes", [16384, 40960])
def test_pool_appends_of_constructed_vectors_match_the_oracle(mkv_lib, page_bytes):
    """Appendable pool without bases, grown by appends of the parity tests' constructed vectors (full-range
    magnitudes, ties, flat, zero, exact-threshold, subnormal, out-of-float32-range squares; many segments keep
    all 128 channels, so sealed segments take their full reserved size): every segment of the view equals the
    oracle's compression of the extended contexts bit for bit."""
    import torch
    from _helpers import storage_to_torch
    from test_gpu_parity import SEGMENT_KINDS, _crafted_segment
    mkv = mkv_lib
    rng = np.random.default_rng(81)
    ctx = [2 * 64 + 30, 64 + 3, 40]
    n0 = [70, 10, 0]
    tot = sum(ctx)
    K = np.zeros((tot, 4, 128), np.uint16)
    V = np.zeros((tot, 4, 128), np.uint16)
    kind_at = 0
    for arr in (K, V):
        for h in range(4):
            for t0 in range(0, tot, 16):
                rows = min(16, tot - t0)
                x = _crafted_segment(rng, SEGMENT_KINDS[kind_at % len(SEGMENT_KINDS)], rows)
                kind_at += 1
                arr[t0:t0 + rows, h, :] = W.f32_to_bf16_bits(x.astype(np.float32))
    cu = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int64)
    R = Reqs.__new__(Reqs)
    R.inp = W.Inputs(_wl(tuple(ctx), 81), K, V, None, None, cu, np.full(len(ctx), 40, np.int32))
    R.K, R.V = storage_to_torch(K, "bf16", "cuda"), storage_to_torch(V, "bf16", "cuda")
    R.basis, R.cu, R.dtype, R.torch = None, cu, "bf16", torch
    pool = _pool(mkv, n_pages=160, page_bytes=page_bytes, slots=32, has_basis=False, appendable=True)
    ids, n = _grow_in_pool(mkv, R, n0, max(ctx), pool)
    assert list(n) == ctx
    ref = oracle.compress_all(R.inp)
    got = read_store(pool.view(ids), "bf16")["streams"]
    for key, r in ref.items():
        assert np.array_equal(got[key].c, r.c), key
        assert np.array_equal(got[key].mask, r.mask), key
        assert np.array_equal(got[key].vals, r.vals), key
