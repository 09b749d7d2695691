"""Layer-batched decode: one store whose requests are the layers of a model compresses and decodes exactly like
the layers one call at a time: the same stored segments (codes, channel sets, values) and bit-identical
selections and outputs, since every (request, KV head) unit is computed independently of the grid around it."""
import numpy as np
import pytest

import workloads as W
from _helpers import inputs_to_torch, read_store

pytestmark = pytest.mark.gpu


def test_layers_in_one_call_equal_layers_one_by_one():
    import torch
    import kv_cache_compression_svd_amd as mkv
    L, n, T = 3, 3000, 200
    wl = W.Workload("layers", L, 32, 8, (n,) * L, "bf16", (T,) * L, "per_request", 40, "3 layers of one request")
    inp = W.generate(wl, basis="svd")
    K, V, q, basis = inputs_to_torch(inp)
    st = mkv.mkv_compress(K, V, inp.cu_seqlens, basis)
    out, sel = mkv.mkv_decode_attn(st, q, inp.T)
    torch.cuda.synchronize()
    whole = read_store(st, "bf16")["streams"]
    for layer in range(L):
        sl = slice(layer * n, (layer + 1) * n)
        st1 = mkv.mkv_compress(K[sl].contiguous(), V[sl].contiguous(), np.array([0, n]), basis[layer:layer + 1].contiguous())
        o1, s1 = mkv.mkv_decode_attn(st1, q[layer:layer + 1].contiguous(), inp.T[layer:layer + 1])
        torch.cuda.synchronize()
        one = read_store(st1, "bf16")["streams"]
        for h in range(8):
            for X in (0, 1):
                a, b = whole[(layer, h, X)], one[(0, h, X)]
                assert np.array_equal(a.c, b.c) and np.array_equal(a.mask, b.mask) and np.array_equal(a.vals, b.vals)
        assert torch.equal(out[layer:layer + 1], o1) and torch.equal(sel[layer:layer + 1], s1), layer


def test_one_layer_of_a_batched_store_matches_the_oracle():
    """The middle layer of a 3-layer store against the oracle itself: with a signed-permutation basis (exact in
    any summation order) its segments equal the oracle's bit for bit, and its decode units pass the decode
    parity rules (accepted near-tie selection, output within 2e-3 of the oracle's for that selection)."""
    import torch
    import kv_cache_compression_svd_amd as mkv
    import oracle
    from _helpers import check_decode_unit
    L, n, T = 3, 2500, 150
    wl = W.Workload("layers", L, 32, 8, (n,) * L, "bf16", (T,) * L, "per_request", 41, "3 layers of one request")
    inp = W.generate(wl, basis="sperm")
    K, V, q, basis = inputs_to_torch(inp)
    st = mkv.mkv_compress(K, V, inp.cu_seqlens, basis)
    out, sel = mkv.mkv_decode_attn(st, q, inp.T)
    torch.cuda.synchronize()
    whole = read_store(st, "bf16")["streams"]
    layer = 1
    ref = oracle.compress_all(inp, units=[(layer, h) for h in range(8)])
    out = out.cpu().numpy().astype(np.float64)
    sel = sel.cpu().numpy()
    G = 4
    for h in range(8):
        for X in (0, 1):
            a, b = whole[(layer, h, X)], ref[(layer, h, X)]
            assert np.array_equal(a.c, b.c) and np.array_equal(a.mask, b.mask) and np.array_equal(a.vals, b.vals)
        qg = W.to_f64(inp.q[layer, h * G:(h + 1) * G, :], "bf16")
        nd = check_decode_unit(sel[layer, h], out[layer, h * G:(h + 1) * G], qg, inp.basis[layer, h, 0],
                               inp.basis[layer, h, 1], ref[(layer, h, 0)], ref[(layer, h, 1)], T)
        assert nd >= 0
