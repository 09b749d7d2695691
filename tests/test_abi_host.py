"""C-ABI checks that need no GPU: the library loads, exports every symbol include/mkv.h declares, and rejects
bad arguments on the host before enqueueing anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_compression_svd_amd as mkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = mkv.lib()
    names = _declared()
    assert "mkv_compress" in names and "mkv_decode_attn" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mkv.SIGNATURES), "binding and header disagree"


def test_default_policy():
    p = mkv.mkv_default_policy()
    assert (p.seg_len, p.keeps(), p.energy_frac) == (64, (128, 64, 32), 0.9)


def _desc(batch=1, heads=8, dim=128, dtype=mkv.MKV_BF16, cu=(0, 100)):
    cu = np.asarray(cu, dtype=np.int64)
    d = mkv.KVDesc()
    d.batch, d.n_kv_heads, d.head_dim, d.dtype = batch, heads, dim, dtype
    d.cu_seqlens = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    return d, cu


def _bytes(d, p):
    sb, tb = ctypes.c_size_t(), ctypes.c_size_t()
    return mkv.lib().mkv_compress_bytes(ctypes.byref(d), ctypes.byref(p), ctypes.byref(sb), ctypes.byref(tb)), sb, tb


def test_sizes_match_layout():
    d, cu = _desc(batch=2, cu=(0, 100, 300))
    st, sb, tb = _bytes(d, mkv.mkv_default_policy())
    assert st == mkv.MKV_OK
    S = 8 * (2 + 4)                     # segments per tensor: ceil(100/64) + ceil(200/64) per head
    payload = 2 * S * 64 * 128 * 2      # every segment slot at full size (one-pass bf16 compression)
    basis = 2 * 8 * 2 * 128 * 128 * 4
    align = lambda x: (x + 255) // 256 * 256   # noqa: E731
    codes = 256
    seg_off = align(codes + 2 * S)
    b = align(seg_off + 16 * S)
    p = align(b + basis)
    assert sb.value == p + payload + 256    # slack after the payload
    # scratch of a one-pass (bf16, fixed-size) compression: the request tables only
    assert tb.value == align(4 * (6 * 2 + 1))
    # float32 (two passes): request tables | per-vector thresholds | one payload total per decide workgroup;
    # the payload holds every token at 128 channels
    d32, _ = _desc(batch=2, cu=(0, 100, 300), dtype=mkv.MKV_FP32)
    st, sb32, tb32 = _bytes(d32, mkv.mkv_default_policy())
    assert st == mkv.MKV_OK
    nblk = 8 * (2 + 4)                  # one segment per workgroup at this size
    assert tb32.value == align(align(4 * (6 * 2 + 1)) + 2 * 300 * 8 * 4 * 2) + 2 * nblk * 8
    b32 = align(seg_off + 16 * S)
    assert sb32.value == align(b32 + basis) + 2 * 8 * 300 * 128 * 4 + 256


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, mkv.MKV_E_UNSUPPORTED), ("batch", 0, mkv.MKV_E_ARG), ("n_kv_heads", 0, mkv.MKV_E_ARG),
    ("dtype", 7, mkv.MKV_E_ARG)])
def test_bad_shapes_rejected(field, value, code):
    d, cu = _desc()
    setattr(d, field, value)
    st, _, _ = _bytes(d, mkv.mkv_default_policy())
    assert st == code
    assert mkv.mkv_last_error()


def test_bad_cu_seqlens_rejected():
    d, cu = _desc(batch=2, cu=(0, 100, 50))
    st, _, _ = _bytes(d, mkv.mkv_default_policy())
    assert st == mkv.MKV_E_ARG and "non-decreasing" in mkv.mkv_last_error()
    d, cu = _desc(batch=1, cu=(5, 100))
    assert _bytes(d, mkv.mkv_default_policy())[0] == mkv.MKV_E_ARG


@pytest.mark.parametrize("keep,frac,seg,code", [
    ((64, 32), 0.9, 64, mkv.MKV_E_ARG), ((128, 64, 64), 0.9, 64, mkv.MKV_E_ARG),
    ((128, 48), 0.9, 64, mkv.MKV_E_UNSUPPORTED), ((128, 64), 0.0, 64, mkv.MKV_E_ARG),
    ((128, 64), 1.5, 64, mkv.MKV_E_ARG), ((128, 64), 0.9, 32, mkv.MKV_E_UNSUPPORTED)])
def test_bad_policies_rejected(keep, frac, seg, code):
    d, cu = _desc()
    p = mkv.SegPolicy.make(keep, frac, seg)
    assert _bytes(d, p)[0] == code


def test_compress_rejects_missing_buffers_before_any_launch():
    d, cu = _desc()
    d.K = ctypes.c_void_p(256)     # never dereferenced: the call must fail on its host checks first
    d.V = ctypes.c_void_p(512)
    p = mkv.mkv_default_policy()
    h = ctypes.c_void_p()
    st = mkv.lib().mkv_compress(ctypes.byref(d), None, ctypes.byref(p), None, 0, None, 0, None, ctypes.byref(h))
    assert st == mkv.MKV_E_ARG and not h.value
    # undersized store buffer
    st = mkv.lib().mkv_compress(ctypes.byref(d), None, ctypes.byref(p), ctypes.c_void_p(4096), 10,
                                ctypes.c_void_p(8192), 1 << 30, None, ctypes.byref(h))
    assert st == mkv.MKV_E_ARG and "store_bytes" in mkv.mkv_last_error()
    # misaligned
    st = mkv.lib().mkv_compress(ctypes.byref(d), None, ctypes.byref(p), ctypes.c_void_p(4100), 1 << 40,
                                ctypes.c_void_p(8192), 1 << 30, None, ctypes.byref(h))
    assert st == mkv.MKV_E_ARG and "aligned" in mkv.mkv_last_error()


def _attached(cu=(0, 100, 0 + 100), heads=2):
    d, cu = _desc(batch=len(cu) - 1, heads=heads, cu=cu)
    p = mkv.mkv_default_policy()
    st, sb, _ = _bytes(d, p)
    h = ctypes.c_void_p()
    # attach only records pointers: a fake aligned address is never touched by the host checks below
    st = mkv.lib().mkv_store_attach(ctypes.byref(d), ctypes.byref(p), 0, ctypes.c_void_p(1 << 20), sb, ctypes.byref(h))
    assert st == mkv.MKV_OK
    return h, cu


def test_decode_argument_checks():
    h, cu = _attached(cu=(0, 100, 200), heads=2)
    L = mkv.lib()
    T = (ctypes.c_int32 * 2)(10, 0)
    ws = ctypes.c_size_t()
    assert L.mkv_decode_workspace_bytes(h, 8, T, ctypes.byref(ws)) == mkv.MKV_E_ARG      # T[1] = 0
    T[1] = 5
    assert L.mkv_decode_workspace_bytes(h, 8, T, ctypes.byref(ws)) == mkv.MKV_OK
    assert L.mkv_decode_workspace_bytes(h, 7, T, ctypes.byref(ws)) == mkv.MKV_E_ARG      # not a multiple
    assert L.mkv_decode_workspace_bytes(h, 6, T, ctypes.byref(ws)) == mkv.MKV_E_UNSUPPORTED  # group 3
    assert L.mkv_decode_workspace_bytes(None, 8, T, ctypes.byref(ws)) == mkv.MKV_E_ARG
    need = ws.value
    fake = ctypes.c_void_p(1 << 24)
    assert L.mkv_decode_attn(h, fake, 8, T, fake, None, 0, fake, need - 1, None) == mkv.MKV_E_ARG
    assert "ws_bytes" in mkv.mkv_last_error()
    assert L.mkv_decode_attn(h, fake, 8, T, fake, fake, 4, fake, need, None) == mkv.MKV_E_ARG   # stride < 10
    assert "sel_stride" in mkv.mkv_last_error()
    assert L.mkv_decode_attn(h, None, 8, T, fake, None, 0, fake, need, None) == mkv.MKV_E_ARG
    assert L.mkv_store_destroy(h) == mkv.MKV_OK


def test_view_reports_layout():
    h, cu = _attached(cu=(0, 100, 300), heads=2)
    info = mkv.StoreInfo()
    assert mkv.lib().mkv_store_view(h, ctypes.byref(info)) == mkv.MKV_OK
    assert info.segments_per_tensor == 2 * (2 + 4) and info.total_tokens == 300
    assert info.codes == (1 << 20) + 256 and info.basis is None
    assert [info.cu_seqlens[i] for i in range(3)] == [0, 100, 300]
    mkv.lib().mkv_store_destroy(h)


def test_kernel_names():
    names = [mkv.mkv_kernel_name(i) for i in range(mkv.PROFILE_KERNELS)]
    assert "score" in names and "attend" in names and names[-1] is None


def test_growable_sizes_and_argument_checks():
    L = mkv.lib()
    d, cu = _desc(batch=2, cu=(0, 100, 300))
    p = mkv.mkv_default_policy()
    cap = np.array([164, 200], dtype=np.int64)
    sb, tb = ctypes.c_size_t(), ctypes.c_size_t()
    capp = cap.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    assert L.mkv_compress_bytes_growable(ctypes.byref(d), ctypes.byref(p), capp, ctypes.byref(sb), ctypes.byref(tb)) == mkv.MKV_OK
    plain = _bytes(d, p)[1].value
    assert sb.value > plain                       # room for 64 more tokens of request 0 and the open areas
    small = np.array([99, 300], dtype=np.int64)   # below request 0's context
    assert L.mkv_compress_bytes_growable(ctypes.byref(d), ctypes.byref(p), small.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                         ctypes.byref(sb), ctypes.byref(tb)) == mkv.MKV_E_ARG
    d.dtype = mkv.MKV_FP32
    assert L.mkv_compress_bytes_growable(ctypes.byref(d), ctypes.byref(p), capp, ctypes.byref(sb), ctypes.byref(tb)) == mkv.MKV_E_UNSUPPORTED
    assert L.mkv_append(None, ctypes.c_void_p(256), ctypes.c_void_p(512), None, ctypes.c_void_p(1024), 4096, None) == mkv.MKV_E_ARG
    h, _ = _attached(cu=(0, 100, 200), heads=2)   # a plain store refuses appends before enqueueing anything
    assert L.mkv_append(h, ctypes.c_void_p(256), ctypes.c_void_p(512), None, ctypes.c_void_p(1 << 20), 4096, None) == mkv.MKV_E_ARG
    assert "growable" in mkv.mkv_last_error()
    L.mkv_store_destroy(h)


def _pool_desc(heads=2, dtype=mkv.MKV_BF16, max_req=4, slots=10, pages=8, page_bytes=16384, has_basis=1):
    d = mkv.PoolDesc()
    d.n_kv_heads, d.dtype, d.has_basis, d.max_requests = heads, dtype, has_basis, max_req
    d.segment_slots, d.n_pages, d.page_bytes = slots, pages, page_bytes
    return d


def test_pool_layout_and_host_checks():
    L = mkv.lib()
    d = _pool_desc()
    nb = ctypes.c_size_t()
    assert L.mkv_pool_bytes(ctypes.byref(d), ctypes.byref(nb)) == mkv.MKV_OK
    align = lambda x: (x + 255) // 256 * 256   # noqa: E731
    S = 2 * 10
    seg_off = align(256 + 2 * S)
    basis = align(seg_off + 16 * S)
    payload = align(basis + 4 * 2 * 2 * 128 * 128 * 4)
    assert nb.value == payload + 8 * 16384 + 256
    for field, value in (("page_bytes", 8192), ("page_bytes", 16384 + 128), ("n_pages", 0), ("max_requests", 0),
                         ("n_kv_heads", 0), ("segment_slots", -1)):
        bad = _pool_desc()
        setattr(bad, field, value)
        assert L.mkv_pool_bytes(ctypes.byref(bad), ctypes.byref(nb)) == mkv.MKV_E_ARG, field
    assert L.mkv_pool_bytes(ctypes.byref(_pool_desc(dtype=mkv.MKV_FP32)), ctypes.byref(nb)) == mkv.MKV_E_ARG  # < 32 KiB
    # create only records pointers: a fake aligned address is never touched by the host-side calls below
    p = mkv.mkv_default_policy()
    h = ctypes.c_void_p()
    assert L.mkv_pool_create(ctypes.byref(d), ctypes.byref(p), ctypes.c_void_p(1 << 20), nb.value - 1, ctypes.byref(h)) == mkv.MKV_E_ARG
    assert L.mkv_pool_create(ctypes.byref(d), ctypes.byref(p), ctypes.c_void_p((1 << 20) + 64), 1 << 30, ctypes.byref(h)) == mkv.MKV_E_ARG
    L.mkv_pool_bytes(ctypes.byref(d), ctypes.byref(nb))
    assert L.mkv_pool_create(ctypes.byref(d), ctypes.byref(p), ctypes.c_void_p(1 << 20), nb.value, ctypes.byref(h)) == mkv.MKV_OK
    info = mkv.PoolInfo()
    assert L.mkv_pool_stats(h, ctypes.byref(info)) == mkv.MKV_OK
    assert (info.free_pages, info.free_segment_slots, info.largest_free_run, info.live_requests) == (8, 10, 10, 0)
    assert info.payload == (1 << 20) + payload and info.pool_bytes == nb.value
    ids = (ctypes.c_int32 * 2)(0, 1)
    out = ctypes.c_void_p()
    assert L.mkv_pool_view(h, 1, ids, ctypes.byref(out)) == mkv.MKV_E_ARG and "not in the pool" in mkv.mkv_last_error()
    assert L.mkv_pool_remove(h, 1, ids) == mkv.MKV_E_ARG
    assert L.mkv_pool_request(h, 0, None, None, None, None) == mkv.MKV_E_ARG
    # adds whose shape or basis does not match the pool fail before anything is enqueued
    kd, cu = _desc(batch=1, heads=3, cu=(0, 100))
    kd.K, kd.V = ctypes.c_void_p(256), ctypes.c_void_p(512)
    got = (ctypes.c_int32 * 1)()
    fake = ctypes.c_void_p(1 << 24)
    assert L.mkv_pool_add(h, ctypes.byref(kd), fake, None, fake, 1 << 30, None, got) == mkv.MKV_E_ARG
    assert "n_kv_heads" in mkv.mkv_last_error()
    kd, cu = _desc(batch=1, heads=2, cu=(0, 100))
    kd.K, kd.V = ctypes.c_void_p(256), ctypes.c_void_p(512)
    assert L.mkv_pool_add(h, ctypes.byref(kd), None, None, fake, 1 << 30, None, got) == mkv.MKV_E_ARG
    assert "basis" in mkv.mkv_last_error()
    cap = (ctypes.c_int64 * 1)(200)
    assert L.mkv_pool_add(h, ctypes.byref(kd), fake, cap, fake, 1 << 30, None, got) == mkv.MKV_E_ARG
    assert "appendable" in mkv.mkv_last_error()
    ws = ctypes.c_size_t()
    assert L.mkv_pool_append_workspace_bytes(h, 2, ctypes.byref(ws)) == mkv.MKV_OK
    assert L.mkv_pool_append(h, 1, got, fake, fake, fake, ws.value, None) == mkv.MKV_E_ARG
    assert "appendable" in mkv.mkv_last_error()
    sb = ctypes.c_size_t()
    assert L.mkv_pool_add_scratch_bytes(h, ctypes.byref(kd), ctypes.byref(sb)) == mkv.MKV_OK
    assert L.mkv_pool_add(h, ctypes.byref(kd), fake, None, fake, sb.value - 1, None, got) == mkv.MKV_E_ARG
    # more requests than free ids
    kd, cu = _desc(batch=5, heads=2, cu=(0, 1, 2, 3, 4, 5))
    kd.K, kd.V = ctypes.c_void_p(256), ctypes.c_void_p(512)
    got5 = (ctypes.c_int32 * 5)()
    assert L.mkv_pool_add(h, ctypes.byref(kd), fake, None, fake, 1 << 30, None, got5) == mkv.MKV_E_ARG
    assert "ids" in mkv.mkv_last_error()
    assert L.mkv_pool_stats(h, ctypes.byref(info)) == mkv.MKV_OK
    assert (info.free_pages, info.free_segment_slots, info.live_requests) == (8, 10, 0)
    assert L.mkv_pool_destroy(h) == mkv.MKV_OK


def test_appendable_pool_layout_and_refusals():
    L = mkv.lib()
    align = lambda x: (x + 255) // 256 * 256   # noqa: E731
    plain, grow = _pool_desc(has_basis=0), _pool_desc(has_basis=0)
    grow.appendable = 1
    nb0, nb1 = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.mkv_pool_bytes(ctypes.byref(plain), ctypes.byref(nb0)) == mkv.MKV_OK
    assert L.mkv_pool_bytes(ctypes.byref(grow), ctypes.byref(nb1)) == mkv.MKV_OK
    # per request id, KV head and tensor: a packed open segment and its original rows, 64 x 128 bf16 each
    assert nb1.value - nb0.value == 2 * (4 * 2 * 2) * 64 * 128 * 2
    bad = _pool_desc(dtype=mkv.MKV_FP32, page_bytes=32768)
    bad.appendable = 1
    assert L.mkv_pool_bytes(ctypes.byref(bad), ctypes.byref(nb0)) == mkv.MKV_E_UNSUPPORTED
    p = mkv.mkv_default_policy()
    h = ctypes.c_void_p()
    assert L.mkv_pool_create(ctypes.byref(grow), ctypes.byref(p), ctypes.c_void_p(1 << 20), nb1.value, ctypes.byref(h)) == mkv.MKV_OK
    fake = ctypes.c_void_p(1 << 24)
    ws = ctypes.c_size_t()
    assert L.mkv_pool_append_workspace_bytes(h, 3, ctypes.byref(ws)) == mkv.MKV_OK
    assert ws.value == align(20 * 3) + align(16 * 3 * 2)
    ids = (ctypes.c_int32 * 1)(0)
    assert L.mkv_pool_append(h, 1, ids, fake, fake, fake, ws.value, None) == mkv.MKV_E_ARG   # id 0 not live
    assert "not in the pool" in mkv.mkv_last_error()
    assert L.mkv_pool_append(h, 0, None, None, None, None, 0, None) == mkv.MKV_OK            # nothing to do
    kd, cu = _desc(batch=1, heads=2, cu=(0, 100))
    kd.K, kd.V = ctypes.c_void_p(256), ctypes.c_void_p(512)
    cap = (ctypes.c_int64 * 1)(99)                                                          # below the context
    got = (ctypes.c_int32 * 1)()
    assert L.mkv_pool_add(h, ctypes.byref(kd), None, cap, fake, 1 << 30, None, got) == mkv.MKV_E_ARG
    assert "capacity" in mkv.mkv_last_error()
    cap[0] = 64 * 11                                                                        # 11 slots > 10
    assert L.mkv_pool_add(h, ctypes.byref(kd), None, cap, fake, 1 << 30, None, got) == mkv.MKV_E_ARG
    assert "slots" in mkv.mkv_last_error()
    info = mkv.PoolInfo()
    L.mkv_pool_stats(h, ctypes.byref(info))
    assert (info.free_pages, info.free_segment_slots, info.live_requests) == (8, 10, 0)
    L.mkv_pool_destroy(h)


def test_noalloc_decode_refuses_workspaces_above_its_maximum():
    """A decode whose workspace would exceed the device-resident array is refused on the host, before anything is
    enqueued: the store is only attached (its buffer address is recorded, never read), so no GPU is needed."""
    L = mkv.lib()
    cap = int(L.mkv_decode_noalloc_max_bytes())
    assert cap == 128 << 20
    n = 1 << 22                                   # 4M tokens x 8 KV heads: keys and lists far above the maximum
    d, cu = _desc(batch=1, heads=8, cu=(0, n))
    p = mkv.mkv_default_policy()
    st, sb, tb = _bytes(d, p)
    assert st == mkv.MKV_OK
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 40)               # an aligned address that is never dereferenced here
    assert L.mkv_store_attach(ctypes.byref(d), ctypes.byref(p), 0, fake, sb, ctypes.byref(h)) == mkv.MKV_OK
    T = (ctypes.c_int32 * 1)(4096)
    ws = ctypes.c_size_t()
    assert L.mkv_decode_workspace_bytes(h, 32, T, ctypes.byref(ws)) == mkv.MKV_OK
    assert ws.value > cap
    st = L.mkv_decode_attn_noalloc(h, fake, 32, T, fake, None, 0, None)
    assert st == mkv.MKV_E_ARG
    assert "workspace" in mkv.mkv_last_error()
    assert L.mkv_store_destroy(h) == mkv.MKV_OK
