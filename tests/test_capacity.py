"""Memory-per-request model of the three decode routes (host arithmetic): the
ring sizes agree with what the library's rssm_ring_sizes reports, and the
capacity ratios follow from the slot counts."""
import ctypes

import pytest

from ssm_recurrent_decode_amd import _lib, capacity


@pytest.mark.parametrize("B,H,d,n,G,L,gdn", [(256, 32, 64, 128, 8, 16, False), (512, 32, 64, 128, 1, 16, False),
                                             (256, 32, 128, 128, 32, 16, True), (3, 8, 64, 128, 2, 30, True)])
def test_ring_bytes_match_library(B, H, d, n, G, L, gdn):
    out = (ctypes.c_size_t * 4)()
    dims = _lib.rssm_dims(B, H, d, n, G, L)
    assert _lib.load().rssm_ring_sizes(ctypes.byref(dims), int(gdn), out) == 0
    assert sum(out) == B * capacity.ring_bytes_per_request(H, d, n, G, L, gdn) + 4


def test_route_ratios():
    H, d, n, G, L, T = 32, 64, 128, 1, 16, 4
    st = capacity.state_bytes(H, d, n)
    assert st == 1 << 20
    assert capacity.bytes_per_request("snapshot", H, d, n, G, L, T) == 5 * st + 4
    tab = capacity.concurrency_table(H, d, n, G, L, T, False, 288 * 10**9)
    mb = tab["max_batch"]
    assert mb["standard"] == 288 * 10**9 // st
    assert mb["snapshot"] == 288 * 10**9 // (5 * st + 4)
    # the ring (16 entries of 4.4 KB + records) costs under 7% of the state, so
    # ReplaySSM keeps over 4.6x the snapshot route's batch at T = 4
    assert 4.6 < tab["replay_over_snapshot"] < 5.0
    assert abs(tab["snapshot_over_standard"] - 0.2) < 1e-3
    with pytest.raises(ValueError):
        capacity.bytes_per_request("other", H, d, n, G)
