"""The traffic model (algorithmic bytes per launch) against per-request byte counts
derived independently from the method page's traffic paragraph for the five
workloads, and against the page's own per-head formula.

Two differences are by design and are checked as exact offsets: the ring keeps
the step size Delta but not the decay a = exp(A Delta) (recomputed in the
kernel), 4 bytes per head and cached entry fewer; and the packed pointer word of
a request is read and written once per call, 16 bytes more (8 bytes per call for
the snapshot route's slot index: read only, 4 bytes).  Per-head parameters (A,
dt_bias) are shared by the batch, so per-request figures are differences
between batch sizes B and B - 1."""
from ssm_recurrent_decode_amd import traffic as tr

MiB = 1 << 20


def per_request(fn, *args, **kw):
    return fn(2, *args, **kw) - fn(1, *args, **kw)


def test_standard_step_nemotron_shape():
    # 2 x 1 MiB state + 4,096 v + 2 x 2,048 k/q + 128 dt + 8,192 y
    assert per_request(tr.standard_step, 32, 64, 128, 8) == 2 * MiB + 4096 + 2 * 2048 + 128 + 8192
    assert tr.standard_step(256, 32, 64, 128, 8) == 541_098_240


def test_replay_append_nemotron_shape():
    # page count with (v, k, Delta, a) per cached entry: 1,071,488 + 6,400 h,
    # +1 MiB instead of the new entry's 6,400 on the flush step
    decay, ptr = 4 * 32, 16
    for h in range(16):
        page = 1_071_488 + 6_400 * h
        assert per_request(tr.replay_append, 32, 64, 128, 8, h, False) == page - decay * (h + 1) + ptr
    page_flush = 1_071_488 + 6_400 * 15 - 6_400 + MiB
    assert per_request(tr.replay_append, 32, 64, 128, 8, 15, True) == page_flush - decay * 15 + ptr
    # the L = 16 cycle average the roofline uses: 303.0 MB per launch at B = 256
    avg = sum(tr.replay_append(256, 32, 64, 128, 8, h, h == 15) for h in range(16)) / 16
    assert round(avg) == 302_991_616


def test_replay_verify_spec_shape():
    # G = 1: 1 MiB + T (4,736 in + 8,192 y + 4,608 slot) + 4,608 c, +1 MiB on a flush round
    decay, ptr, T = 4 * 32, 16, 4
    for c in range(13):
        for flush in (False, True):
            page = MiB + T * (4_736 + 8_192 + 4_608) + 4_608 * c + (MiB if flush else 0)
            got = per_request(tr.replay_verify, 32, 64, 128, 1, T, c, flush)
            assert got == page - decay * (T + c) + ptr, (c, flush)


def test_gdn_verify_shape():
    # 2 MiB + T (24,832 in + 16,384 y + 24,704 slot) + 24,704 c, +2 MiB on a flush round
    T = 4
    for c in range(13):
        for flush in (False, True):
            page = 2 * MiB + T * (24_832 + 16_384 + 24_704) + 24_704 * c + (2 * MiB if flush else 0)
            assert per_request(tr.gdn_verify, 32, 128, 128, 32, T, c, flush) == page + 16, (c, flush)


def test_snapshot_route():
    # Mamba-2 (d = 64, G = 1, T = 4): state read + 4 snapshots + drafts + y = 5,294,592
    assert per_request(tr.snapshot_verify, 32, 64, 128, 1, 4) == 5_294_592 + 4
    # GDN (d = 128, G = 32, T = 4): 10,650,624
    assert per_request(tr.snapshot_verify, 32, 128, 128, 32, 4, gdn=True) == 10_650_624 + 4


def test_conv_update():
    # 3,072 channels: state read + write (2 x 3 x 2 B), x (2 B), out (4 B) = 18 B per channel
    assert per_request(tr.conv1d, 3072, 4) == 3072 * 18


def test_pages_formula_matches_the_model_with_two_byte_scalars():
    # with every scalar at 2 bytes, no pointer word and k/q per head (G = H),
    # one head's replay read + new entry is the page's 4dn + 2h(d+n+1) + ... form
    d, n = 64, 128
    for h in (0, 5, 15):
        slot = 2 * d + 2 * n + 2                     # v, k, Delta at 2 bytes
        model = 4 * d * n + h * slot + (2 * d + 2 * 2 * n + 2) + slot
        assert tr.pages_traffic_per_head(d, n, h) == model
    assert tr.pages_traffic_per_head(d, n) == 8 * d * n + 2 * (d + 2 * n + 1)
