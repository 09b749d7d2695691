"""GPU parity of the uncompressed decode-attention baseline against the oracle's exact softmax attention over
every token's full rows (float64).  No selection is involved, so every output is unique: per query head
rel-L2 <= 2e-3 and elementwise <= 2e-3 of the row maximum.  Scaled workloads cover several 512-token chunks
and ragged tails; the full sizes are checked on sampled units with the full-size parity tests."""
import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import check_out, inputs_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mkv():
    import kv_cache_compression_svd_amd as m
    m.lib()
    return m


def _custom(ctx, Hq=32, Hkv=8, seed=5):
    return W.Workload(f"dense{len(ctx)}", len(ctx), Hq, Hkv, tuple(ctx), "bf16", (1,) * len(ctx), "per_request",
                      seed, "dense-baseline case")


def _check_units(mkv, inp, units=None):
    import torch
    K, V, q, _ = inputs_to_torch(inp)
    out = mkv.mkv_dense_decode_attn(K, V, inp.cu_seqlens, q)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    w = inp.workload
    G = w.group
    cu = inp.cu_seqlens
    for r in range(w.batch):
        for h in range(w.n_kv_heads):
            if units is not None and (r, h) not in units:
                continue
            k = W.to_f64(inp.K[cu[r]:cu[r + 1], h, :], inp.dtype)
            v = W.to_f64(inp.V[cu[r]:cu[r + 1], h, :], inp.dtype)
            qg = W.to_f64(inp.q[r, h * G:(h + 1) * G, :], inp.dtype)
            check_out(out[r, h * G:(h + 1) * G], oracle.dense_decode_unit(qg, k, v))


@pytest.mark.parametrize("name,div", [("llama_layer", 32), ("ragged16", 64), ("batch8_128k", 256)])
def test_dense_scaled(mkv, name, div):
    _check_units(mkv, W.generate(W.scaled(W.get(name), div), basis="none"))


@pytest.mark.parametrize("ctx,Hq,Hkv", [([0, 1, 513, 1500], 32, 8), ([2048], 8, 8), ([777, 5], 16, 2),
                                        ([1030], 64, 8)])
def test_dense_edges(mkv, ctx, Hq, Hkv):
    """Empty request, one token, ragged chunk tails, groups of 1, 8 and 8 with 64 heads."""
    _check_units(mkv, W.generate(_custom(ctx, Hq, Hkv), basis="none"))


def test_dense_rejects_fp32(mkv):
    import torch
    inp = W.generate(W.scaled(W.get("tiny"), 8), basis="none")
    K, V, q, _ = inputs_to_torch(inp)
    with pytest.raises(mkv.MkvError) as e:
        mkv.mkv_dense_decode_attn(K, V, inp.cu_seqlens, q)
    assert e.value.status == mkv.MKV_E_UNSUPPORTED and "bf16" in str(e.value)
    del torch
