"""Byte counts of the compressed store and of the dense KV cache.  TEST INFRASTRUCTURE ONLY.

Dense size: the pages (arXiv 2607.00760, section 1 and section 2.1) state that 8 concurrent LLaMA-3.1-8B
requests of 128K tokens need 128 GB of KV cache and 1M-token requests 1 TB: 32 layers x 8 KV heads x 128
channels x 2 tensors x 2 bytes per token.

Compressed payload: a segment of n_s tokens that keeps c channels stores n_s * c values of b_v bytes, plus
n_s * c one-byte channel indices when c is below the head dimension (at full width the indices are implicit).
Each segment of each tensor also carries 9 bytes of metadata: a one-byte strategy code and an 8-byte offset.
"""
from __future__ import annotations

import numpy as np


def stream_payload_bytes(c: np.ndarray, n: int, seg_len: int, d: int, b_v: int) -> int:
    """Closed form over the per-segment kept counts c[s] of one stream of n tokens."""
    total = 0
    for s, cs in enumerate(np.asarray(c).tolist()):
        n_s = min(seg_len, n - s * seg_len)
        total += n_s * cs * (b_v + (1 if cs < d else 0))
    return total


def store_payload_bytes(streams: dict, seg_len: int, b_v: int) -> int:
    return sum(stream_payload_bytes(st.c, st.n, seg_len, st.d, b_v) for st in streams.values())


def counted_payload_bytes(stream, b_v: int, seg_len: int) -> int:
    """Payload bytes counted token by token from the logical store (kept channels of every token)."""
    total = 0
    for j in range(stream.n):
        k = int(stream.mask[j].sum())
        c = int(stream.c[j // seg_len])
        total += k * (b_v + (1 if c < stream.d else 0))
    return total


def segment_meta_bytes(n_segments: int) -> int:
    return 9 * int(n_segments)


def dense_kv_bytes(tokens: int, n_kv_heads: int, head_dim: int, b_v: int, layers: int = 1) -> int:
    """Uncompressed K + V bytes: tokens x layers x KV heads x head_dim x 2 tensors x b_v."""
    return int(tokens) * int(layers) * int(n_kv_heads) * int(head_dim) * 2 * int(b_v)
