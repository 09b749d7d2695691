"""Test helpers checked on the CPU.

The piecewise store reader of the full-size GPU tests: an oracle store laid out in the library's documented
format (in host memory; attaching only records pointers) reads back stream by stream as the oracle's own
streams, and the segment sizes and offsets it derives match the layout.  The near-tie selection enumerator:
the selections it accepts on constructed scores."""
import numpy as np

import oracle
import workloads as W
from _helpers import StoreReader, upload_oracle_store, valid_selections


def test_reader_round_trips_an_oracle_store():
    import kv_cache_compression_svd_amd as mkv
    w = W.scaled(W.get("ragged16"), 64)
    inp = W.generate(w, basis="svd")
    keep = (128, 64, 32)
    ref = oracle.compress_all(inp)
    store = upload_oracle_store(ref, inp, keep, device="cpu")
    rd = StoreReader(store, inp.dtype)
    sizes = rd.segment_bytes(2)
    np.testing.assert_array_equal(rd.seg_off, np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64))
    assert rd.total == int(sizes.sum()) == oracle.store_payload_bytes(ref, 64, 2)
    for (r, h, X), st in ref.items():
        got = rd.stream(r, h, X)
        np.testing.assert_array_equal(got.c, st.c)
        np.testing.assert_array_equal(got.mask, st.mask)
        np.testing.assert_array_equal(got.vals, st.vals)
    del mkv


def test_valid_selections_enumerates_the_tie_band():
    s = np.array([5.0, 4.0, 3.0, 3.0 + 1e-7, 3.0 - 1e-7, 1.0, 3.1])
    # T = 4: 5, 4 and 3.1 are above the band around the 4th score (3 + 1e-7); one more from {2, 3, 4}
    sels = valid_selections(s, 4)
    assert [x.tolist() for x in sels] == [[0, 1, 2, 6], [0, 1, 3, 6], [0, 1, 4, 6]]
    assert [x.tolist() for x in valid_selections(s, 3)] == [[0, 1, 6]]      # the 3rd score stands alone
    assert valid_selections(np.zeros(100), 50) is None                       # C(100, 50) selections
    assert valid_selections(s, 0)[0].size == 0
