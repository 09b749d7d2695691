"""Decode results do not depend on where the segments sit in the payload.

A store built by mkv_compress is copied to the host, its segments are laid out again back to back in reverse
slot order (a placement the compressor never makes), every other payload byte is set to 0xFF (a NaN pattern in
bf16 and float32, so that any read past a segment that reached the results would show), and the copy is
attached as a store.  Decoding both must give bit-identical outputs and selections.
"""
import numpy as np
import pytest

import workloads as W
from _helpers import StoreReader, inputs_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mkv():
    import kv_cache_compression_svd_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("name,div", [("ragged16", 64), ("llama_layer", 32), ("tiny", 8)],
                         ids=["ragged16/64", "llama_layer/32", "tiny/8"])
def test_decode_is_independent_of_segment_placement(mkv, name, div):
    import torch
    w = W.scaled(W.get(name), div)
    inp = W.generate(w, basis="svd")
    K, V, q, basis = inputs_to_torch(inp)
    s1 = mkv.mkv_compress(K, V, inp.cu_seqlens, basis)
    torch.cuda.synchronize()
    info = s1.view()
    base = s1.buf.data_ptr()
    S2 = 2 * int(info.segments_per_tensor)
    o_off, o_pay = info.seg_off - base, info.payload - base
    sizes = StoreReader(s1, inp.dtype).segment_bytes(2 if inp.dtype == "bf16" else 4)
    host = s1.buf.cpu().numpy()
    offs = host[o_off:o_off + 8 * S2].view(np.uint64).astype(np.int64)
    out = host.copy()
    out[o_pay:] = 0xFF
    new = offs.copy()
    pos = 0
    for g in range(S2 - 1, -1, -1):
        sz = int(sizes[g])
        if sz == 0:
            continue
        new[g] = pos
        out[o_pay + pos:o_pay + pos + sz] = host[o_pay + offs[g]:o_pay + offs[g] + sz]
        pos += sz
    assert pos == s1.payload_bytes()
    out[o_off:o_off + 8 * S2] = new.astype(np.uint64).view(np.uint8)
    buf2 = torch.from_numpy(out).to("cuda")
    s2 = mkv.mkv_store_attach(inp.cu_seqlens, w.n_kv_heads, s1.dtype, s1.policy, basis is not None, buf2)
    o1, sel1 = mkv.mkv_decode_attn(s1, q, inp.T)
    o2, sel2 = mkv.mkv_decode_attn(s2, q, inp.T)
    torch.cuda.synchronize()
    assert torch.equal(sel1, sel2)
    assert torch.equal(o1, o2)
    assert not torch.isnan(o2).any()
