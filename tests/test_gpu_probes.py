"""The streaming HBM probes (the bandwidth ceilings the bench reports, and the
kernel whose counters calibrate the traffic summaries) through the C ABI: the
copy is exact, and the read probe's per-work-group checksums add up to the sum of
the data, at sizes that leave a ragged last pass and at the 4096-work-group cap."""
import ctypes

import pytest
import torch

from ssm_recurrent_decode_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 1040, 1 << 20, (64 << 20) + 48])
def test_probe_copy_and_read(nbytes):
    lib = _lib.load()
    n = nbytes // 4
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    src = torch.randint(-8, 8, (n,), generator=g, device="cuda").float()  # small integers: exact sums
    dst = torch.full_like(src, float("nan"))
    assert lib.rssm_probe_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                               ctypes.c_size_t(nbytes), None) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    nsink = lib.rssm_probe_read_sink_floats(ctypes.c_size_t(nbytes))
    assert 1 <= nsink <= 4096
    sink = torch.full((nsink,), float("nan"), device="cuda")
    assert lib.rssm_probe_read(ctypes.c_void_p(src.data_ptr()), ctypes.c_size_t(nbytes),
                               ctypes.c_void_p(sink.data_ptr()), None) == 0
    torch.cuda.synchronize()
    assert not torch.isnan(sink).any()
    assert float(sink.double().sum()) == float(src.double().sum())
