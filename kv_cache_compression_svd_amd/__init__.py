"""Python binding of libmkv, a MosaicKV-style compressed KV cache for AMD MI355X (gfx950).

Method: arXiv 2607.00760, "MosaicKV: Serving Long-Context LLM with Dynamic Two-D KV Cache Compression"
(section 1: dynamic two-D compression; compact sparse attention; query-aware token selection).

The functions carry the names of the C entry points declared in include/mkv.h and only marshal arguments:
torch supplies device memory (the store, scratch and workspace buffers are uint8 CUDA tensors) and the current
stream; every step of compression and decode runs in the library's HIP kernels.  If libmkv.so is missing the
first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_double, c_int32, c_int64, c_size_t, c_uint32, c_uint64, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmkv.so")

MKV_OK, MKV_E_ARG, MKV_E_UNSUPPORTED, MKV_E_DEVICE = 0, 1, 2, 3
MKV_FP32, MKV_BF16 = 0, 1
HEAD_DIM = 128
SEG_LEN = 64
PROFILE_KERNELS = 32


class MkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"mkv status {status}: {msg}")
        self.status = status


class SegPolicy(ctypes.Structure):
    _fields_ = [("seg_len", c_int32), ("n_keep", c_int32), ("keep", c_int32 * 4), ("energy_frac", c_double)]

    @classmethod
    def make(cls, keep=(128, 64, 32), energy_frac=0.9, seg_len=SEG_LEN):
        p = cls()
        p.seg_len = seg_len
        p.n_keep = len(keep)
        for i, c in enumerate(keep):
            p.keep[i] = int(c)
        p.energy_frac = float(energy_frac)
        return p

    def keeps(self):
        return tuple(self.keep[i] for i in range(self.n_keep))


class KVDesc(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32), ("dtype", c_int32),
                ("cu_seqlens", POINTER(c_int64)), ("K", c_void_p), ("V", c_void_p)]


class StoreInfo(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32), ("dtype", c_int32),
                ("policy", SegPolicy), ("has_basis", c_int32), ("total_tokens", c_int64),
                ("segments_per_tensor", c_int64), ("cu_seqlens", POINTER(c_int64)), ("codes", c_void_p),
                ("seg_off", c_void_p), ("basis", c_void_p), ("payload", c_void_p), ("payload_total", c_void_p),
                ("payload_capacity", c_uint64), ("store_bytes", c_uint64), ("cu_capacity", POINTER(c_int64)),
                ("growable", c_int32), ("seg_base", POINTER(c_int32)), ("seg_slots", POINTER(c_int32)),
                ("basis_slot", POINTER(c_int32)), ("pool_view", c_int32)]


class PoolDesc(ctypes.Structure):
    _fields_ = [("n_kv_heads", c_int32), ("dtype", c_int32), ("has_basis", c_int32), ("max_requests", c_int32),
                ("segment_slots", c_int64), ("n_pages", c_int64), ("page_bytes", c_int64), ("appendable", c_int32)]


class PoolInfo(ctypes.Structure):
    _fields_ = [("desc", PoolDesc), ("live_requests", c_int32), ("free_pages", c_int64),
                ("free_segment_slots", c_int64), ("largest_free_run", c_int64), ("codes", c_void_p),
                ("seg_off", c_void_p), ("basis", c_void_p), ("payload", c_void_p), ("pool_bytes", c_uint64)]


# Every symbol include/mkv.h declares, with its ctypes signature.
SIGNATURES = {
    "mkv_default_policy": (None, [POINTER(SegPolicy)]),
    "mkv_compress_bytes": (c_int32, [POINTER(KVDesc), POINTER(SegPolicy), POINTER(c_size_t), POINTER(c_size_t)]),
    "mkv_compress": (c_int32, [POINTER(KVDesc), c_void_p, POINTER(SegPolicy), c_void_p, c_size_t, c_void_p, c_size_t,
                               c_void_p, POINTER(c_void_p)]),
    "mkv_store_attach": (c_int32, [POINTER(KVDesc), POINTER(SegPolicy), c_int32, c_void_p, c_size_t,
                                   POINTER(c_void_p)]),
    "mkv_compress_bytes_growable": (c_int32, [POINTER(KVDesc), POINTER(SegPolicy), POINTER(c_int64),
                                              POINTER(c_size_t), POINTER(c_size_t)]),
    "mkv_compress_growable": (c_int32, [POINTER(KVDesc), c_void_p, POINTER(SegPolicy), POINTER(c_int64), c_void_p,
                                        c_size_t, c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]),
    "mkv_append_workspace_bytes": (c_int32, [c_void_p, POINTER(c_size_t)]),
    "mkv_append": (c_int32, [c_void_p, c_void_p, c_void_p, POINTER(c_int32), c_void_p, c_size_t, c_void_p]),
    "mkv_store_view": (c_int32, [c_void_p, POINTER(StoreInfo)]),
    "mkv_store_payload_bytes": (c_int32, [c_void_p, c_void_p, POINTER(c_uint64)]),
    "mkv_store_destroy": (c_int32, [c_void_p]),
    "mkv_decode_workspace_bytes": (c_int32, [c_void_p, c_int32, POINTER(c_int32), POINTER(c_size_t)]),
    "mkv_decode_attn": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32), c_void_p, c_void_p, c_int32,
                                  c_void_p, c_size_t, c_void_p]),
    "mkv_decode_noalloc_max_bytes": (c_size_t, []),
    "mkv_decode_attn_noalloc": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32), c_void_p, c_void_p,
                                          c_int32, c_void_p]),
    "mkv_dense_decode_workspace_bytes": (c_int32, [c_void_p, c_int32, POINTER(c_size_t)]),
    "mkv_dense_decode_attn": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mkv_gram_workspace_bytes": (c_int32, [c_void_p, POINTER(c_size_t)]),
    "mkv_gram": (c_int32, [c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mkv_pool_bytes": (c_int32, [POINTER(PoolDesc), POINTER(c_size_t)]),
    "mkv_pool_create": (c_int32, [POINTER(PoolDesc), POINTER(SegPolicy), c_void_p, c_size_t, POINTER(c_void_p)]),
    "mkv_pool_add_scratch_bytes": (c_int32, [c_void_p, POINTER(KVDesc), POINTER(c_size_t)]),
    "mkv_pool_add": (c_int32, [c_void_p, POINTER(KVDesc), c_void_p, POINTER(c_int64), c_void_p, c_size_t, c_void_p,
                               POINTER(c_int32)]),
    "mkv_pool_append_workspace_bytes": (c_int32, [c_void_p, c_int32, POINTER(c_size_t)]),
    "mkv_pool_append": (c_int32, [c_void_p, c_int32, POINTER(c_int32), c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mkv_pool_remove": (c_int32, [c_void_p, c_int32, POINTER(c_int32)]),
    "mkv_pool_view": (c_int32, [c_void_p, c_int32, POINTER(c_int32), POINTER(c_void_p)]),
    "mkv_pool_stats": (c_int32, [c_void_p, POINTER(PoolInfo)]),
    "mkv_pool_request": (c_int32, [c_void_p, c_int32, POINTER(c_int64), POINTER(c_int64), POINTER(c_int64),
                                   POINTER(c_uint64)]),
    "mkv_pool_destroy": (c_int32, [c_void_p]),
    "mkv_last_error": (c_char_p, []),
    "mkv_profile_start": (c_int32, [c_int32, c_uint32]),
    "mkv_profile_stop": (c_int32, [POINTER(c_double), POINTER(c_int32)]),
    "mkv_kernel_name": (c_char_p, [c_int32]),
}

_lib = None


def lib():
    """The loaded libmkv (torch is imported first so that both use torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (or python "
                               f"kv_cache_compression_svd_amd/build.py) first")
        import torch  # noqa: F401  (loads the HIP runtime libmkv links against)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def mkv_last_error() -> str:
    return lib().mkv_last_error().decode()


def _check(status: int):
    if status != MKV_OK:
        raise MkvError(status, mkv_last_error())


def mkv_default_policy() -> SegPolicy:
    p = SegPolicy()
    lib().mkv_default_policy(byref(p))
    return p


# ---- torch marshalling helpers ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MKV_BF16
    if t.dtype == torch.float32:
        return MKV_FP32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or float32")


def _ptr(t):
    return c_void_p(0 if t is None else t.data_ptr())


def _kv_desc(K, V, cu_seqlens, n_kv_heads=None, dtype=None):
    import numpy as np
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    d = KVDesc()
    d.batch = len(cu) - 1
    if K is not None:
        if K.dim() != 3 or K.shape[2] != HEAD_DIM or not K.is_contiguous() or not K.is_cuda:
            raise ValueError("K must be a contiguous CUDA tensor [tokens][n_kv_heads][128]")
        if V is None or V.shape != K.shape or V.dtype != K.dtype or not V.is_contiguous() or not V.is_cuda:
            raise ValueError("V must be a contiguous CUDA tensor shaped and typed like K")
        d.n_kv_heads = K.shape[1]
        d.dtype = _dtype_code(K)
        if K.shape[0] != int(cu[-1]):
            raise ValueError(f"K has {K.shape[0]} tokens but cu_seqlens ends at {int(cu[-1])}")
    else:
        d.n_kv_heads = int(n_kv_heads)
        d.dtype = int(dtype)
    d.head_dim = HEAD_DIM
    d.cu_seqlens = cu.ctypes.data_as(POINTER(c_int64))
    d.K = _ptr(K)
    d.V = _ptr(V)
    return d, cu


class Store:
    """A compressed store: the device buffer (a uint8 tensor), its host handle and shape metadata."""

    def __init__(self, handle: c_void_p, buf, cu, n_kv_heads: int, dtype: int, policy: SegPolicy, keep_alive=()):
        self.handle = handle
        self.buf = buf
        self.cu = cu
        self.n_kv_heads = n_kv_heads
        self.dtype = dtype
        self.policy = policy
        self._keep = keep_alive

    @property
    def batch(self):
        return len(self.cu) - 1

    def view(self) -> StoreInfo:
        info = StoreInfo()
        _check(lib().mkv_store_view(self.handle, byref(info)))
        return info

    def payload_bytes(self, stream=None) -> int:
        v = c_uint64()
        _check(lib().mkv_store_payload_bytes(self.handle, _stream_ptr(stream), byref(v)))
        return int(v.value)

    def close(self):
        if self.handle is not None and self.handle.value:
            lib().mkv_store_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mkv_compress_bytes(K, V, cu_seqlens, policy: SegPolicy | None = None, n_kv_heads=None, dtype=None):
    policy = policy or mkv_default_policy()
    d, _ = _kv_desc(K, V, cu_seqlens, n_kv_heads, dtype)
    sb, tb = c_size_t(), c_size_t()
    _check(lib().mkv_compress_bytes(byref(d), byref(policy), byref(sb), byref(tb)))
    return int(sb.value), int(tb.value)


def mkv_compress(K, V, cu_seqlens, basis=None, policy: SegPolicy | None = None, stream=None, store_buf=None,
                 scratch=None, capacity=None) -> Store:
    """Compress K, V ([tokens][n_kv_heads][128], bf16 or float32, CUDA) with the per-(request, KV head, tensor)
    bases ``basis`` (float32 [batch][n_kv_heads][2][128][128] CUDA, or None for already-rotated inputs).
    ``capacity`` (per-request token counts >= the contexts) builds a growable store that mkv_append extends."""
    import numpy as np
    torch = _torch()
    policy = policy or mkv_default_policy()
    d, cu = _kv_desc(K, V, cu_seqlens)
    sb, tb = c_size_t(), c_size_t()
    cap = None
    if capacity is not None:
        cap = np.ascontiguousarray(np.asarray(capacity, dtype=np.int64))
        if cap.shape != (d.batch,):
            raise ValueError("capacity must hold one token count per request")
        _check(lib().mkv_compress_bytes_growable(byref(d), byref(policy), cap.ctypes.data_as(POINTER(c_int64)),
                                                 byref(sb), byref(tb)))
    else:
        _check(lib().mkv_compress_bytes(byref(d), byref(policy), byref(sb), byref(tb)))
    if basis is not None:
        if basis.dtype != torch.float32 or not basis.is_contiguous() or not basis.is_cuda or \
                tuple(basis.shape) != (d.batch, d.n_kv_heads, 2, HEAD_DIM, HEAD_DIM):
            raise ValueError("basis must be a contiguous CUDA float32 tensor [batch][n_kv_heads][2][128][128]")
    if store_buf is None:
        store_buf = torch.empty(sb.value, dtype=torch.uint8, device=K.device)
    if scratch is None:
        scratch = torch.empty(max(tb.value, 1), dtype=torch.uint8, device=K.device)
    h = c_void_p()
    if cap is not None:
        _check(lib().mkv_compress_growable(byref(d), _ptr(basis), byref(policy), cap.ctypes.data_as(POINTER(c_int64)),
                                           _ptr(store_buf), c_size_t(store_buf.numel()), _ptr(scratch),
                                           c_size_t(scratch.numel()), _stream_ptr(stream), byref(h)))
    else:
        _check(lib().mkv_compress(byref(d), _ptr(basis), byref(policy), _ptr(store_buf), c_size_t(store_buf.numel()),
                                  _ptr(scratch), c_size_t(scratch.numel()), _stream_ptr(stream), byref(h)))
    # scratch must outlive the asynchronous kernels: keep it until the store is dropped
    return Store(h, store_buf, cu, d.n_kv_heads, d.dtype, policy, keep_alive=(scratch,))


def mkv_append(store: Store, K_new, V_new, active=None, ws=None, stream=None):
    """Appends one token per active request (all when ``active`` is None) to a growable store: K_new, V_new are
    [batch][n_kv_heads][128] CUDA tensors of the store's dtype.  Updates ``store.cu``."""
    import numpy as np
    torch = _torch()
    B, H = len(store.cu) - 1, store.n_kv_heads
    for t in (K_new, V_new):
        if tuple(t.shape) != (B, H, HEAD_DIM) or not t.is_contiguous() or not t.is_cuda or _dtype_code(t) != store.dtype:
            raise ValueError("K_new and V_new must be contiguous CUDA tensors [batch][n_kv_heads][128] of the store's dtype")
    act = None
    if active is not None:
        act = np.ascontiguousarray(np.asarray(active, dtype=np.int32))
        if act.shape != (B,):
            raise ValueError("active must hold one flag per request")
    if ws is None:
        v = c_size_t()
        _check(lib().mkv_append_workspace_bytes(store.handle, byref(v)))
        ws = torch.empty(v.value, dtype=torch.uint8, device=K_new.device)
    _check(lib().mkv_append(store.handle, _ptr(K_new), _ptr(V_new),
                            None if act is None else act.ctypes.data_as(POINTER(c_int32)), _ptr(ws),
                            c_size_t(ws.numel()), _stream_ptr(stream)))
    info = store.view()
    store.cu = np.array([info.cu_seqlens[i] for i in range(B + 1)], dtype=np.int64)
    return store


def mkv_store_attach(cu_seqlens, n_kv_heads: int, dtype: int, policy: SegPolicy, has_basis: bool, store_buf) -> Store:
    d, cu = _kv_desc(None, None, cu_seqlens, n_kv_heads, dtype)
    h = c_void_p()
    _check(lib().mkv_store_attach(byref(d), byref(policy), int(bool(has_basis)), _ptr(store_buf),
                                  c_size_t(store_buf.numel()), byref(h)))
    return Store(h, store_buf, cu, n_kv_heads, dtype, policy)


class Pool:
    """A paged pool of compressed requests in one device buffer (a uint8 tensor) with its host handle."""

    def __init__(self, n_kv_heads: int, dtype: int, max_requests: int, segment_slots: int, n_pages: int,
                 page_bytes: int, has_basis: bool = True, policy: SegPolicy | None = None, device="cuda", buf=None,
                 appendable: bool = False):
        torch = _torch()
        self.policy = policy or mkv_default_policy()
        d = PoolDesc()
        d.n_kv_heads, d.dtype, d.has_basis, d.max_requests = int(n_kv_heads), int(dtype), int(bool(has_basis)), int(max_requests)
        d.segment_slots, d.n_pages, d.page_bytes = int(segment_slots), int(n_pages), int(page_bytes)
        d.appendable = int(bool(appendable))
        self.desc = d
        nb = c_size_t()
        _check(lib().mkv_pool_bytes(byref(d), byref(nb)))
        self.buf = torch.empty(nb.value, dtype=torch.uint8, device=device) if buf is None else buf
        self.handle = c_void_p()
        _check(lib().mkv_pool_create(byref(d), byref(self.policy), _ptr(self.buf), c_size_t(self.buf.numel()),
                                     byref(self.handle)))
        self.n_kv_heads, self.dtype = int(n_kv_heads), int(dtype)
        self._keep = []

    def add(self, K, V, cu_seqlens, basis=None, stream=None, scratch=None, capacity=None):
        """Compresses the requests of (K, V, cu_seqlens) into the pool; returns their ids (numpy int32).
        ``capacity``: per-request token capacities for later appends (appendable pools).  Synchronises the
        stream."""
        import numpy as np
        torch = _torch()
        d, cu = _kv_desc(K, V, cu_seqlens)
        if basis is not None and (basis.dtype != torch.float32 or not basis.is_contiguous() or not basis.is_cuda or
                                  tuple(basis.shape) != (d.batch, d.n_kv_heads, 2, HEAD_DIM, HEAD_DIM)):
            raise ValueError("basis must be a contiguous CUDA float32 tensor [batch][n_kv_heads][2][128][128]")
        if scratch is None:
            v = c_size_t()
            _check(lib().mkv_pool_add_scratch_bytes(self.handle, byref(d), byref(v)))
            scratch = torch.empty(max(v.value, 1), dtype=torch.uint8, device=self.buf.device)
        ids = np.zeros(d.batch, dtype=np.int32)
        cap = None
        if capacity is not None:
            cap = np.ascontiguousarray(np.asarray(capacity, dtype=np.int64))
            if cap.shape != (d.batch,):
                raise ValueError("capacity must hold one token count per request")
        _check(lib().mkv_pool_add(self.handle, byref(d), _ptr(basis),
                                  None if cap is None else cap.ctypes.data_as(POINTER(c_int64)), _ptr(scratch),
                                  c_size_t(scratch.numel()), _stream_ptr(stream), ids.ctypes.data_as(POINTER(c_int32))))
        return ids

    def append(self, ids, K_new, V_new, ws=None, stream=None):
        """One token for each listed request: K_new, V_new are [len(ids)][n_kv_heads][128] bf16 CUDA tensors."""
        import numpy as np
        torch = _torch()
        a = np.ascontiguousarray(np.atleast_1d(np.asarray(ids, dtype=np.int32)))
        for t in (K_new, V_new):
            if tuple(t.shape) != (len(a), self.n_kv_heads, HEAD_DIM) or not t.is_contiguous() or not t.is_cuda \
                    or _dtype_code(t) != self.dtype:
                raise ValueError("K_new and V_new must be contiguous CUDA tensors [len(ids)][n_kv_heads][128] of "
                                 "the pool's dtype")
        if ws is None:
            v = c_size_t()
            _check(lib().mkv_pool_append_workspace_bytes(self.handle, len(a), byref(v)))
            ws = torch.empty(max(v.value, 1), dtype=torch.uint8, device=self.buf.device)
        _check(lib().mkv_pool_append(self.handle, len(a), a.ctypes.data_as(POINTER(c_int32)), _ptr(K_new),
                                     _ptr(V_new), _ptr(ws), c_size_t(ws.numel()), _stream_ptr(stream)))
        self._keep = [ws]   # the enqueued kernel reads it

    def remove(self, ids):
        import numpy as np
        a = np.ascontiguousarray(np.atleast_1d(np.asarray(ids, dtype=np.int32)))
        _check(lib().mkv_pool_remove(self.handle, len(a), a.ctypes.data_as(POINTER(c_int32))))

    def view(self, ids) -> Store:
        """A Store over the listed live requests (in this order) for mkv_decode_attn."""
        import numpy as np
        a = np.ascontiguousarray(np.atleast_1d(np.asarray(ids, dtype=np.int32)))
        h = c_void_p()
        _check(lib().mkv_pool_view(self.handle, len(a), a.ctypes.data_as(POINTER(c_int32)), byref(h)))
        st = Store(h, self.buf, None, self.n_kv_heads, self.dtype, self.policy, keep_alive=(self,))
        info = st.view()
        st.cu = np.array([info.cu_seqlens[i] for i in range(len(a) + 1)], dtype=np.int64)
        return st

    def stats(self) -> PoolInfo:
        info = PoolInfo()
        _check(lib().mkv_pool_stats(self.handle, byref(info)))
        return info

    def request(self, rid: int):
        """(tokens, pages, payload bytes) of a live request."""
        n, cap, pg, pb = c_int64(), c_int64(), c_int64(), c_uint64()
        _check(lib().mkv_pool_request(self.handle, int(rid), byref(n), byref(cap), byref(pg), byref(pb)))
        return int(n.value), int(pg.value), int(pb.value)

    def capacity(self, rid: int) -> int:
        cap = c_int64()
        _check(lib().mkv_pool_request(self.handle, int(rid), None, byref(cap), None, None))
        return int(cap.value)

    def close(self):
        if self.handle is not None and self.handle.value:
            lib().mkv_pool_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _T_array(T, batch):
    import numpy as np
    t = np.ascontiguousarray(np.broadcast_to(np.asarray(T, dtype=np.int32), (batch,)))
    return t, t.ctypes.data_as(POINTER(c_int32))


def mkv_decode_workspace_bytes(store: Store, n_q_heads: int, T) -> int:
    t, tp = _T_array(T, store.batch)
    v = c_size_t()
    _check(lib().mkv_decode_workspace_bytes(store.handle, int(n_q_heads), tp, byref(v)))
    return int(v.value)


def mkv_decode_attn(store: Store, q, T, out=None, sel=None, sel_stride=None, ws=None, stream=None,
                    return_sel: bool = True):
    """One decode step for q [batch][n_q_heads][128] (the store's dtype, CUDA).  Returns (out, sel):
    out float32 [batch][n_q_heads][128]; sel int32 [batch][n_kv_heads][sel_stride] (or None)."""
    torch = _torch()
    import numpy as np
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q must be a contiguous CUDA tensor [batch][n_q_heads][128]")
    if _dtype_code(q) != store.dtype:
        raise TypeError("q must have the store's dtype")
    B, Hq = q.shape[0], q.shape[1]
    if B != store.batch:
        raise ValueError(f"q has batch {B}, the store {store.batch}")
    t, tp = _T_array(T, B)
    n = np.diff(store.cu)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if return_sel and sel is None:
        stride = int(sel_stride) if sel_stride is not None else max(1, int(np.minimum(t, n).max(initial=0)))
        sel = torch.empty((B, store.n_kv_heads, stride), dtype=torch.int32, device=q.device)
    stride = sel.shape[-1] if sel is not None else 0
    if ws is None:
        ws = torch.empty(mkv_decode_workspace_bytes(store, Hq, t), dtype=torch.uint8, device=q.device)
    _check(lib().mkv_decode_attn(store.handle, _ptr(q), int(Hq), tp, _ptr(out), _ptr(sel), int(stride), _ptr(ws),
                                 c_size_t(ws.numel()), _stream_ptr(stream)))
    return out, sel


def mkv_decode_noalloc_max_bytes() -> int:
    return int(lib().mkv_decode_noalloc_max_bytes())


def mkv_decode_attn_noalloc(store: Store, q, T, out, sel=None, stream=None):
    """mkv_decode_attn on the library's device-resident workspace: no device memory is allocated by this call
    (out, and sel if given, are the caller's).  Returns (out, sel)."""
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q must be a contiguous CUDA tensor [batch][n_q_heads][128]")
    if _dtype_code(q) != store.dtype:
        raise TypeError("q must have the store's dtype")
    B, Hq = q.shape[0], q.shape[1]
    if B != store.batch:
        raise ValueError(f"q has batch {B}, the store {store.batch}")
    _, tp = _T_array(T, B)
    stride = sel.shape[-1] if sel is not None else 0
    _check(lib().mkv_decode_attn_noalloc(store.handle, _ptr(q), int(Hq), tp, _ptr(out), _ptr(sel), int(stride),
                                         _stream_ptr(stream)))
    return out, sel


def mkv_dense_decode_workspace_bytes(K, V, cu_seqlens, n_q_heads: int) -> int:
    d, cu = _kv_desc(K, V, cu_seqlens)
    v = c_size_t()
    _check(lib().mkv_dense_decode_workspace_bytes(byref(d), int(n_q_heads), byref(v)))
    return int(v.value)


def mkv_dense_decode_attn(K, V, cu_seqlens, q, out=None, ws=None, stream=None):
    """Uncompressed decode attention (the baseline): out float32 [batch][n_q_heads][128] for bf16 K, V
    [tokens][n_kv_heads][128] and q [batch][n_q_heads][128] (all CUDA)."""
    torch = _torch()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q must be a contiguous CUDA tensor [batch][n_q_heads][128]")
    d, cu = _kv_desc(K, V, cu_seqlens)
    B, Hq = q.shape[0], q.shape[1]
    if B != d.batch:
        raise ValueError(f"q has batch {B}, cu_seqlens {d.batch}")
    if _dtype_code(q) != d.dtype:
        raise TypeError("q must have the dtype of K and V")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(mkv_dense_decode_workspace_bytes(K, V, cu_seqlens, Hq), dtype=torch.uint8, device=q.device)
    _check(lib().mkv_dense_decode_attn(byref(d), _ptr(q), int(Hq), _ptr(out), _ptr(ws), c_size_t(ws.numel()),
                                       _stream_ptr(stream)))
    return out


def mkv_gram(K, V, cu_seqlens, out=None, ws=None, stream=None):
    """X^T X (float32 [batch][n_kv_heads][2][128][128]) of every (request, KV head, tensor) stream of bf16 K, V."""
    torch = _torch()
    d, cu = _kv_desc(K, V, cu_seqlens)
    if out is None:
        out = torch.empty((d.batch, d.n_kv_heads, 2, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=K.device)
    if ws is None:
        v = c_size_t()
        _check(lib().mkv_gram_workspace_bytes(byref(d), byref(v)))
        ws = torch.empty(v.value, dtype=torch.uint8, device=K.device)
    _check(lib().mkv_gram(byref(d), _ptr(out), _ptr(ws), c_size_t(ws.numel()), _stream_ptr(stream)))
    return out


def svd_basis_from_gram(gram):
    """Rotation bases from Gram matrices (any [..., 128, 128] tensor or array): the eigenvectors by decreasing
    eigenvalue, as float32 columns, computed in float64 on the host.  Returns a CPU float32 tensor."""
    import numpy as np
    torch = _torch()
    g = gram.detach().cpu().numpy().astype(np.float64) if hasattr(gram, "detach") else np.asarray(gram, np.float64)
    w, vecs = np.linalg.eigh(g)
    order = np.argsort(-w, axis=-1, kind="stable")
    vecs = np.take_along_axis(vecs, order[..., None, :], axis=-1)
    return torch.from_numpy(np.ascontiguousarray(vecs.astype(np.float32)))


def mkv_profile_start(max_launches: int = 1 << 20, kernels=None):
    """Times the library's kernel launches until mkv_profile_stop; kernels: names to time (default: all)."""
    if kernels is None:
        mask = 0xFFFFFFFF
    else:
        names = [mkv_kernel_name(i) for i in range(PROFILE_KERNELS)]
        mask = 0
        for k in kernels:
            if k not in names:
                raise ValueError(f"unknown kernel {k!r}")
            mask |= 1 << names.index(k)
    _check(lib().mkv_profile_start(int(max_launches), c_uint32(mask)))


def mkv_profile_stop():
    """Returns {kernel name: (total ms, launches)} for the kernels launched since mkv_profile_start."""
    ms = (c_double * PROFILE_KERNELS)()
    cnt = (c_int32 * PROFILE_KERNELS)()
    _check(lib().mkv_profile_stop(ms, cnt))
    res = {}
    for i in range(PROFILE_KERNELS):
        name = lib().mkv_kernel_name(i)
        if name is not None and cnt[i] > 0:
            res[name.decode()] = (float(ms[i]), int(cnt[i]))
    return res


def mkv_kernel_name(kernel_id: int):
    n = lib().mkv_kernel_name(int(kernel_id))
    return None if n is None else n.decode()
