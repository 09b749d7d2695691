"""CPU oracle of MosaicKV-style compressed decode attention: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.  The product
(the HIP library and its Python binding) never calls it and shares no code with it.

It is a plain, slow implementation in float64 numpy of what the pages describe (arXiv 2607.00760,
"MosaicKV: Serving Long-Context LLM with Dynamic Two-D KV Cache Compression"):

* ``rounding``  -- round-to-nearest-even to the storage dtype (bf16 or fp32).
* ``compress``  -- dynamic two-D compression of one (request, KV head, tensor) stream: SVD rotation, per-vector
  element selection, one compression strategy (kept-channel count) per KV-cache segment
  (section 1, Observation & Approach 1).
* ``decode``    -- one decode step: query-aware token selection by a score estimate over the compressed keys
  (section 1, prior-work paragraph on query-aware selection, and Challenge 1 on keeping both dimensions
  compressed through selection and attention), then exact softmax attention over the selected sparse
  keys/values (section 1, Observation & Approach 2, compact sparse attention).
* ``sizes``     -- byte counts: the compressed store's closed form and the dense KV-cache size
  (section 1 and section 2.1 give the dense size of 8 LLaMA-3.1-8B requests).

Every function is pinned by tests under ``tests/`` against values the mathematics fixes (closed forms, brute
force on tiny inputs, library routines for the special cases that reduce to them).
"""
from .rounding import rne, rne_bf16, rne_f32  # noqa: F401
from .compress import (Policy, DEFAULT_POLICY, Stream, rotate_round, channel_order, kept_energy,  # noqa: F401
                       vector_min_keep, compress_stream, compress_all)
from .decode import (rotate_queries, scores, select_top, attend, decode_unit, decode_all,  # noqa: F401
                     dense_decode_unit)
from .sizes import stream_payload_bytes, store_payload_bytes, dense_kv_bytes, segment_meta_bytes  # noqa: F401
from .basis import gram, gram_abs  # noqa: F401
