"""Decode on the library's device-resident workspace (mkv_decode_attn_noalloc, for callers that cannot allocate
device memory) against the same call with a caller workspace (mkv_decode_attn): the same kernels on the same
store, so outputs and selections must be identical bit for bit.  Two calls in a row, the second on a smaller
store, so the array's leftovers from the first call cannot leak into the second."""
import numpy as np
import pytest

import workloads as W
from _helpers import inputs_to_torch

pytestmark = pytest.mark.gpu


def _store(mkv, ctx, T, seed):
    import torch
    wl = W.Workload("noalloc", len(ctx), 32, 8, tuple(ctx), "bf16", tuple(T), "single", seed)
    inp = W.generate(wl, basis="svd")
    K, V, q, basis = inputs_to_torch(inp)
    st = mkv.mkv_compress(K, V, inp.cu_seqlens, basis)
    torch.cuda.synchronize()
    return st, q, inp.T


def test_noalloc_decode_equals_workspace_decode():
    import torch
    import kv_cache_compression_svd_amd as mkv
    cases = [((9000, 3000, 700, 0), (400, 128, 700, 5), 61),   # larger first
             ((1500,), (90,), 62)]                              # then smaller
    for ctx, T, seed in cases:
        st, q, t = _store(mkv, ctx, T, seed)
        need = mkv.mkv_decode_workspace_bytes(st, q.shape[1], t)
        assert need <= mkv.mkv_decode_noalloc_max_bytes()
        ref_out, ref_sel = mkv.mkv_decode_attn(st, q, t)
        out = torch.full_like(ref_out, float("nan"))
        sel = torch.full_like(ref_sel, -7)
        mkv.mkv_decode_attn_noalloc(st, q, t, out, sel)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), ctx
        assert torch.equal(sel, ref_sel), ctx
        # and without the selection output
        out2 = torch.full_like(ref_out, float("nan"))
        mkv.mkv_decode_attn_noalloc(st, q, t, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref_out), ctx
        n = np.diff(st.cu)
        assert bool(np.all(n >= 0))
