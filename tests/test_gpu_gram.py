"""GPU parity of the Gram matrices X^T X (basis refresh) against the oracle's float64 product.

Products of bf16 values are exact in float32 and the GPU sums them in float32: within one 32-token MFMA step,
then over the 512 steps of a 16384-token chunk, then over the chunks.  A float32 sum of m terms is within
(m - 1) * 2^-24 of the sum of the terms' magnitudes, so each entry must lie within 4e-5 * (|X|^T |X|)_ij of
the exact value (the bound for ~600 sequential additions).  Cases cover chunk tails, several chunks per stream,
empty requests, and sampled streams of the full workloads; the basis a Gram matrix yields, used by the
compressor, gives the oracle's compression of the same inputs with that basis."""
import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import inputs_to_torch, read_store

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mkv():
    import kv_cache_compression_svd_amd as m
    m.lib()
    return m


def _custom(ctx, Hkv=8, seed=21):
    return W.Workload(f"gram{len(ctx)}", len(ctx), 4 * Hkv, Hkv, tuple(ctx), "bf16", (1,) * len(ctx),
                      "per_request", seed, "gram case")


def _check(mkv, inp, units=None):
    import torch
    K, V, _, _ = inputs_to_torch(inp)
    g = mkv.mkv_gram(K, V, inp.cu_seqlens)
    torch.cuda.synchronize()
    g = g.cpu().numpy().astype(np.float64)
    cu = inp.cu_seqlens
    w = inp.workload
    for r in range(w.batch):
        for h in range(w.n_kv_heads):
            if units is not None and (r, h) not in units:
                continue
            for X, arr in ((0, inp.K), (1, inp.V)):
                x = W.to_f64(arr[cu[r]:cu[r + 1], h, :], inp.dtype)
                ref = oracle.gram(x)
                bound = 4e-5 * oracle.gram_abs(x)
                err = np.abs(g[r, h, X] - ref)
                assert np.all(err <= bound), (r, h, X, float((err / np.maximum(bound, 1e-300)).max()))
    return g


@pytest.mark.parametrize("ctx", [[100, 0, 64, 1], [40_000], [16_384, 16_385]])
def test_gram_tails_chunks_and_empty(mkv, ctx):
    _check(mkv, W.generate(_custom(ctx), basis="none"))


@pytest.mark.parametrize("name,div", [("llama_layer", 1), ("ragged16", 16), ("batch8_128k", 8)])
def test_gram_workloads(mkv, name, div):
    w = W.get(name) if div == 1 else W.scaled(W.get(name), div)
    _check(mkv, W.generate(w, basis="none"), units={(0, 0), (w.batch - 1, w.n_kv_heads - 1)})


def test_basis_from_gram_drives_the_compressor(mkv):
    """The eigenvectors of the GPU's Gram matrices, as the rotation basis of both the GPU compressor and the
    oracle: the stores agree under the SVD-basis rules (values within one ulp; identical codes here)."""
    import torch
    inp = W.generate(W.scaled(W.get("llama_layer"), 16), basis="none")
    K, V, q, _ = inputs_to_torch(inp)
    basis = mkv.svd_basis_from_gram(mkv.mkv_gram(K, V, inp.cu_seqlens))
    inp = W.Inputs(inp.workload, inp.K, inp.V, inp.q, basis.numpy(), inp.cu_seqlens, inp.T, inp.sigma)
    st = mkv.mkv_compress(K, V, inp.cu_seqlens, basis.cuda())
    torch.cuda.synchronize()
    got = read_store(st, inp.dtype)["streams"]
    ref = oracle.compress_all(inp)
    diff = 0
    for key, r in ref.items():
        diff += int(np.sum(got[key].c != r.c))
        both = got[key].mask & r.mask
        ax = np.abs(r.vals[both])
        ulp = np.exp2(np.floor(np.log2(np.where(ax > 0, ax, 1.0))) - 7)
        assert np.all(np.abs(got[key].vals[both] - r.vals[both]) <= ulp * 1.0001), key
    assert diff <= 2
