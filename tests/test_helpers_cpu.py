"""Test helpers checked on the CPU.

The piecewise store reader of the full-size GPU tests: an oracle store laid out in the library's documented
format (in host memory; attaching only records pointers) reads back stream by stream as the oracle's own
streams, and the segment sizes and offsets it derives match the layout.  The near-tie selection enumerator:
the selections it accepts on constructed scores.  The placement check of the full-size tests: constructed
offsets it accepts and rejects."""
import types

import numpy as np
import pytest

import oracle
import workloads as W
from _helpers import StoreReader, check_run_layout, upload_oracle_store, valid_selections


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


def _near_threshold_segment(rng, target_gap):
    """64 bf16-exact vectors that keep 64 channels comfortably, except vector 5 whose 64-channel energy ratio
    sits target_gap away from 0.9 (positive: admissible)."""
    x = np.zeros((64, 128))
    x[:, :16] = rng.choice([-1.0, 1.0], (64, 16)) * 4.0       # big channels: ratio well above 0.9 at 32 and 64
    x[:, 16:] = rng.choice([-1.0, 1.0], (64, 112)) * 0.0625
    # vector 5: 64 channels of a, 64 of b with 64 a^2 / (64 a^2 + 64 b^2) = 0.9 + gap
    a = 1.0
    b2 = a * a * (1.0 / (0.9 + target_gap) - 1.0)
    x[5, :64] = a
    x[5, 64:] = np.sqrt(b2)
    return oracle.rne(x, "bf16")


def test_code_difference_needs_a_vector_inside_the_flip_bound():
    """The P3 justification accepts a differing code only with a vector near the energy target on the side that
    explains it: vector 5 sits just below 0.9 at 64 channels, so a GPU that kept 64 (code 1) where the oracle
    kept 128 (code 0) is explained at m = 1 ulp but not at m = 0, and never the other way round."""
    from _helpers import code_difference_reason, energy_flip_bound
    rng = np.random.default_rng(3)
    seg = _near_threshold_segment(rng, -2e-4)
    order = oracle.channel_order(seg)
    ratio = oracle.kept_energy(seg, order, 64)[5] / np.sum(seg[5] ** 2)
    assert ratio < 0.9 and abs(ratio - 0.9) <= energy_flip_bound(seg, 1.0, "bf16")[5]
    assert oracle.vector_min_keep(seg)[5] == 128
    assert code_difference_reason(seg, 1, 0, (128, 64, 32), 1.0, "bf16") == 5
    assert code_difference_reason(seg, 1, 0, (128, 64, 32), 0.0, "bf16") is None
    assert code_difference_reason(seg, 0, 1, (128, 64, 32), 1.0, "bf16") is None   # wrong side of the target
    far = _near_threshold_segment(rng, -0.05)
    assert code_difference_reason(far, 1, 0, (128, 64, 32), 1.0, "bf16") is None


def test_channel_swap_needs_magnitudes_at_the_cut():
    from _helpers import channel_swap_reason
    x = oracle.rne(np.linspace(1.0, 3.0, 128), "bf16")[::-1].copy()   # descending, bf16-exact
    ref = np.zeros(128, bool)
    ref[np.argsort(-np.abs(x), kind="stable")[:64]] = True
    got = ref.copy()
    i_in, i_out = 63, 64          # swap the channels on either side of the cut
    got[i_in], got[i_out] = False, True
    assert channel_swap_reason(x, got, ref, 64, 1.0, "bf16") == (abs(x[i_in] - x[i_out]) <= 2 * 2.0 ** -6)
    got2 = ref.copy()
    got2[0], got2[127] = False, True   # swap the largest for the smallest: never explained
    assert not channel_swap_reason(x, got2, ref, 64, 1.0, "bf16")


class _InfoOnly:
    """Stands in for a store: check_run_layout reads only view().growable and view().payload_capacity."""

    def __init__(self, growable, capacity):
        self._info = types.SimpleNamespace(growable=growable, payload_capacity=capacity)

    def view(self):
        return self._info


def test_run_layout_check():
    slot = 64 * 128 * 2
    sizes = np.array([12288, 12288, 6144, 0, 12288, 12288])
    # one run from slot 0 (three segments back to back), slot 3 unused, a second run from slot 4
    offs = np.array([0, 12288, 24576, 0, 4 * slot, 4 * slot + 12288])
    store = _InfoOnly(0, 6 * slot)
    check_run_layout(offs, sizes, store, 2)
    ok = offs.copy()
    ok[5] = 5 * slot                    # a run may start at any slot
    check_run_layout(ok, sizes, store, 2)
    bad = offs.copy()
    bad[1] = 6000                       # neither at its slot nor after its predecessor (and overlapping)
    with pytest.raises(AssertionError):
        check_run_layout(bad, sizes, store, 2)
    with pytest.raises(AssertionError):  # past the payload
        check_run_layout(offs, sizes, _InfoOnly(0, 5 * slot), 2)
    # two-pass stores (float32 or growable): back to back in slot order
    packed = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    check_run_layout(packed, sizes, _InfoOnly(1, 6 * slot), 2)
    check_run_layout(packed, sizes, store, 4)
    with pytest.raises(AssertionError):
        check_run_layout(offs, sizes, store, 4)
