"""Seeded synthetic inputs for MosaicKV-style compressed decode attention.

This module only draws inputs: keys, values, queries, per-(request, KV head, tensor) orthonormal bases,
context lengths and token budgets. It holds no step of the compression or attention method, so both the
CPU oracle and the GPU path can take their inputs from it.

The recipe (one per workload, all seeded with numpy's default_rng):

* For each request, for each KV head in order: ``perm = rng.permutation(128)`` gives channel j the scale
  ``sigma_j = (perm_j + 1) ** -0.5``; ``rng.choice(128, 4, replace=False)`` picks 4 outlier channels whose
  scale is multiplied by 10; then K = standard_normal((n, 128)) * sigma, V likewise, then the G query
  heads of that KV group likewise.  K, V and q of one (request, KV head) share sigma.
* Draws are float64, rounded to float32 (round-to-nearest-even), and for bf16 storage rounded once more
  from float32 to bf16 (round-to-nearest-even).  The rounded values are the inputs.
* The basis of (request, KV head, X) for X in {K, V} holds the right singular vectors of the rounded X as
  columns, ordered by decreasing singular value: eigenvectors of X^T X computed in float64, handed over as
  float32.  Other basis kinds exist for exact-arithmetic tests: a signed permutation ("sperm") and none.

The MosaicKV pages (arXiv 2607.00760, "MosaicKV: Serving Long-Context LLM with Dynamic Two-D KV Cache
Compression", section 1, Observation & Approach 1) describe the rotation as an SVD rotation of KV vectors; the
basis itself is computed outside the kernel path, so here it is an input.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
_N_OUTLIERS = 4
_OUTLIER_GAIN = 10.0


@dataclass(frozen=True)
class Workload:
    """Shape, dtype, budget and seeding of one synthetic workload."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    ctx: tuple            # context length per request
    dtype: str            # "bf16" or "fp32": storage dtype of K, V, q and packed values
    T: tuple              # token budget per request (per KV head)
    seeding: str          # "single" (one rng for all requests), "per_request" (rng seed_base + r)
    seed: int
    note: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def total_tokens(self) -> int:
        return int(sum(self.ctx))


def _ragged_contexts(seed: int, count: int, lo: int, hi: int) -> tuple:
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(lo), math.log(hi), count)
    return tuple(int(math.floor(math.exp(x))) for x in u)


def _three_percent(ctx):
    return tuple(max(1, (3 * n) // 100) for n in ctx)


_RAGGED_CTX = _ragged_contexts(11, 16, 4096, 262144)

WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 1, (4096,), "fp32", (256,), "single", 0,
                     "1 request, 4 q heads share 1 KV head, context 4096, fp32"),
    "llama_layer": Workload("llama_layer", 1, 32, 8, (32768,), "bf16", (2048,), "single", 1,
                            "Llama-3.1-8B single-layer decode shape: 32 q / 8 KV heads, context 32768"),
    "batch8_128k": Workload("batch8_128k", 8, 32, 8, (131072,) * 8, "bf16", (4096,) * 8, "per_request", 2,
                            "8 requests x 131072 tokens, per-request seeds 2..9"),
    "million": Workload("million", 1, 32, 8, (1048576,), "bf16", (8192,), "single", 10,
                        "one request of 1048576 tokens"),
    "ragged16": Workload("ragged16", 16, 32, 8, _RAGGED_CTX, "bf16", _three_percent(_RAGGED_CTX), "ragged", 11,
                         "16 requests, contexts log-uniform in [4096, 262144], T = 3% of each context"),
}
ORDER = ["tiny", "llama_layer", "batch8_128k", "million", "ragged16"]


def scaled(w: Workload, ctx_div: int = 1, ctx=None, T=None, name=None) -> Workload:
    """The same recipe at smaller contexts: each context is divided by ``ctx_div`` (at least 1 token kept),
    or replaced by ``ctx``.  T keeps its rule: 3% of each context for the ragged mix, otherwise the fixed
    budget divided by ``ctx_div`` (at least 1), unless ``T`` is given."""
    if ctx is None:
        ctx = tuple(max(1, n // ctx_div) for n in w.ctx)
    ctx = tuple(int(n) for n in ctx)
    if T is None:
        if w.name == "ragged16":
            T = _three_percent(ctx)
        else:
            T = (max(1, w.T[0] // ctx_div),) * len(ctx)
    elif np.isscalar(T):
        T = (int(T),) * len(ctx)
    return Workload(name or f"{w.name}/{ctx_div}", len(ctx), w.n_q_heads, w.n_kv_heads, ctx, w.dtype,
                    tuple(int(t) for t in T), w.seeding, w.seed, w.note)


# --------------------------------------------------------------------------------------------------
# storage rounding of the drawn inputs
# --------------------------------------------------------------------------------------------------

def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns the 16-bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))   # no overflow for finite values
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a storage array (uint16 bf16 patterns, or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


# --------------------------------------------------------------------------------------------------
# generation
# --------------------------------------------------------------------------------------------------

@dataclass
class Inputs:
    """One batch of inputs.  K, V: [sum n][Hkv][128] in storage form (uint16 bf16 patterns or float32),
    token-major (NHD); q: [B][Hq][128] storage form; basis: float32 [B][Hkv][2][128][128] or None;
    cu_seqlens: int64 [B+1]; T: int32 [B]."""

    workload: Workload
    K: np.ndarray
    V: np.ndarray
    q: np.ndarray
    basis: np.ndarray | None
    cu_seqlens: np.ndarray
    T: np.ndarray
    sigma: np.ndarray = field(default=None)   # [B][Hkv][128] channel scales used

    @property
    def dtype(self) -> str:
        return self.workload.dtype


def _svd_basis(x64: np.ndarray) -> np.ndarray:
    g = x64.T @ x64
    w, v = np.linalg.eigh(g)
    order = np.argsort(-w, kind="stable")
    return v[:, order].astype(np.float32)


def _sperm_basis(rng: np.random.Generator) -> np.ndarray:
    p = rng.permutation(HEAD_DIM)
    s = rng.choice(np.array([-1.0, 1.0]), HEAD_DIM)
    b = np.zeros((HEAD_DIM, HEAD_DIM), dtype=np.float32)
    b[np.arange(HEAD_DIM), p] = s
    return b


def _draw_request(w: Workload, rng, r: int, t0: int, n: int, K, V, q, sig, bas, basis: str, brng, heads):
    """Draws request r's K, V, q (and bases) from ``rng`` in the recipe's order, writing into the arrays."""
    G = w.group
    for h in range(w.n_kv_heads):
        perm = rng.permutation(HEAD_DIM)
        sigma = (perm + 1.0) ** -0.5
        out = rng.choice(HEAD_DIM, _N_OUTLIERS, replace=False)
        sigma[out] *= _OUTLIER_GAIN
        sig[r, h] = sigma
        for slot, dst in ((0, K), (1, V)):
            x = rng.standard_normal((n, HEAD_DIM)) * sigma
            xs = _store(x, w.dtype)
            if heads is None or h in heads:
                dst[t0:t0 + n, h, :] = xs
            if bas is not None:
                if basis == "svd":
                    bas[r, h, slot] = _svd_basis(to_f64(xs, w.dtype)) if (heads is None or h in heads) \
                        else np.eye(HEAD_DIM, dtype=np.float32)
                elif basis == "sperm":
                    bas[r, h, slot] = _sperm_basis(brng)
                else:
                    raise ValueError(basis)
        qq = rng.standard_normal((G, HEAD_DIM)) * sigma
        q[r, h * G:(h + 1) * G, :] = _store(qq, w.dtype)


def _shared_array(shape, dtype):
    import mmap
    nbytes = int(np.prod(shape)) * np.dtype(dtype).itemsize
    buf = mmap.mmap(-1, max(nbytes, 1))   # anonymous shared mapping: forked workers write into it
    return np.frombuffer(buf, dtype=dtype, count=int(np.prod(shape))).reshape(shape)


_FORK_STATE = None


def _fork_worker(r):
    from threadpoolctl import threadpool_limits
    w, cu, K, V, q, sig, bas, basis, heads = _FORK_STATE
    rng = np.random.default_rng(w.seed + r)
    brng = np.random.default_rng([w.seed, 7, r])
    with threadpool_limits(1):
        _draw_request(w, rng, r, int(cu[r]), int(cu[r + 1] - cu[r]), K, V, q, sig, bas, basis, brng, heads)
    return r


def generate(w: Workload, basis: str = "svd", heads=None, workers: int = 1) -> Inputs:
    """Draw the inputs of workload ``w``.  ``basis`` is "svd", "sperm" or "none".  ``heads`` restricts the
    draw of K/V to a subset of KV heads (other heads are left zero; the rng stream is unchanged).
    ``workers`` > 1 draws the requests of a per-request-seeded workload in forked processes (same values);
    call it before the process touches a GPU."""
    global _FORK_STATE
    B = w.batch
    ctx = np.asarray(w.ctx, dtype=np.int64)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(ctx)
    total = int(cu[-1])
    sdt = np.uint16 if w.dtype == "bf16" else np.float32
    par = workers > 1 and w.seeding == "per_request" and B > 1
    alloc = _shared_array if par else (lambda shape, dt: np.zeros(shape, dtype=dt))
    K = alloc((total, w.n_kv_heads, HEAD_DIM), sdt)
    V = alloc((total, w.n_kv_heads, HEAD_DIM), sdt)
    q = alloc((B, w.n_q_heads, HEAD_DIM), sdt)
    sig = alloc((B, w.n_kv_heads, HEAD_DIM), np.float64)
    bas = None if basis == "none" else alloc((B, w.n_kv_heads, 2, HEAD_DIM, HEAD_DIM), np.float32)
    if par:
        import multiprocessing as mp
        _FORK_STATE = (w, cu, K, V, q, sig, bas, basis, heads)
        pool = mp.get_context("fork").Pool(min(workers, B))
        try:
            list(pool.imap_unordered(_fork_worker, range(B)))
            pool.close()    # workers exit on their own: no termination signal reaches them
            pool.join()
        except BaseException:
            pool.terminate()
            raise
        finally:
            _FORK_STATE = None
    else:
        rng = np.random.default_rng(w.seed)
        if w.seeding == "ragged":
            rng.uniform(0.0, 1.0, B)   # the context draw comes first on this stream (see _ragged_contexts)
        for r in range(B):
            if w.seeding == "per_request":
                rng = np.random.default_rng(w.seed + r)
                brng = np.random.default_rng([w.seed, 7, r])
            else:
                brng = np.random.default_rng([w.seed, 7, r])
            _draw_request(w, rng, r, int(cu[r]), int(ctx[r]), K, V, q, sig, bas, basis, brng, heads)
    T = np.asarray(w.T, dtype=np.int32)
    return Inputs(w, K, V, q, bas, cu, T, sig)


def get(name: str) -> Workload:
    return WORKLOADS[name]
