"""The C ABI without a GPU: the library loads, exports every function the header
declares (and the binding prototypes exactly those), and rejects bad arguments on
the host with the documented codes before anything is launched."""
import ctypes
import os
import re

import pytest

from ssm_recurrent_decode_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_recurrent_decode.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation returns first
FAKE2 = ctypes.c_void_p(0x2000)  # a second distinct fake pointer (outputs that must not alias)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_0-9]+\s*\**\s*([A-Za-z_0-9]+)\s*\(", text, re.M)))


def test_every_declared_function_is_exported_and_prototyped():
    names = _declared()
    assert "replay_append_decode" in names and "gdn_replay_verify_T" in names
    lib = _lib.load()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)


def test_abi_version_and_strerror():
    lib = _lib.load()
    assert lib.rssm_abi_version() == _lib.ABI_VERSION == 11
    assert "invalid" in _lib.strerror(_lib.RSSM_EINVAL)
    assert "not compiled" in _lib.strerror(_lib.RSSM_ENOTSUP)


def _dims(B=4, H=8, d=64, n=128, G=1, L=8):
    return _lib.rssm_dims(B, H, d, n, G, L)


def _ring():
    return _lib.rssm_ring(*([FAKE.value] * 4), None, 0)


def test_ring_sizes():
    lib = _lib.load()
    out = (ctypes.c_size_t * 4)()
    d = _dims(B=256, H=32, d=64, n=128, G=8, L=16)
    assert lib.rssm_ring_sizes(ctypes.byref(d), 0, out) == 0
    assert list(out) == [256 * 32 * 16 * 64 * 2, 256 * 8 * 16 * 128 * 2, 256 * 32 * 32 * 4, 4]
    assert lib.rssm_ring_sizes(ctypes.byref(d), 1, out) == 0
    assert out[0] == 256 * 32 * 16 * 64 * 4
    # a record is one 128-byte line up to L = 29, two lines above
    for L, words in ((29, 32), (30, 64), (32, 64)):
        d = _dims(B=2, H=4, L=L)
        assert lib.rssm_ring_sizes(ctypes.byref(d), 0, out) == 0
        assert out[2] == 2 * 4 * words * 4
    assert lib.rssm_ring_sizes(ctypes.byref(_dims(L=33)), 0, out) == _lib.RSSM_ENOTSUP


def test_host_validation_codes():
    lib = _lib.load()
    P = FAKE
    d = _dims()
    r = _ring()
    EINVAL, ENOTSUP = _lib.RSSM_EINVAL, _lib.RSSM_ENOTSUP
    # null pointers
    assert lib.ssm_decode_step(ctypes.byref(d), None, P, P, P, P, P, P, P, None) == EINVAL
    assert lib.replay_append_decode(ctypes.byref(d), P, None, P, P, P, P, P, P, P, None, None) == EINVAL
    # H % G != 0
    bad = _dims(H=6, G=4)
    assert lib.ssm_decode_step(ctypes.byref(bad), P, P, P, P, P, P, P, P, None) == EINVAL
    # unsupported head/state dims (every call: d in {64, 128}, n in {64, 128, 256})
    for dd in (_dims(d=96), _dims(n=96), _dims(n=32), _dims(n=512), _dims(d=256)):
        assert lib.ssm_decode_step(ctypes.byref(dd), P, P, P, P, P, P, P, P, None) == ENOTSUP
        assert lib.replay_append_decode(ctypes.byref(dd), P, ctypes.byref(r), P, P, P, P, P, P, P,
                                        None, None) == ENOTSUP
        assert lib.replay_verify_T(ctypes.byref(dd), 2, P, ctypes.byref(r), P, P, P, P, P, P, P,
                                   None, None) == ENOTSUP
        assert lib.replay_flush(ctypes.byref(dd), P, ctypes.byref(r), None, None) == ENOTSUP
        assert lib.ssm_snapshot_verify_T(ctypes.byref(dd), 2, 3, P, P, P, P, P, P, P, P, P, P,
                                         None) == ENOTSUP
        assert lib.gdn_decode_step(ctypes.byref(dd), P, P, P, P, P, P, P, None) == ENOTSUP
        assert lib.gdn_replay_verify_T(ctypes.byref(dd), 2, P, ctypes.byref(r), P, P, P, P, P, P,
                                       None, None) == ENOTSUP
        assert lib.gdn_replay_flush(ctypes.byref(dd), P, ctypes.byref(r), None, None) == ENOTSUP
        assert lib.gdn_replay_append_decode(ctypes.byref(dd), P, ctypes.byref(r), P, P, P, P, P, P,
                                            None, None) == ENOTSUP
        assert lib.gdn_snapshot_verify_T(ctypes.byref(dd), 2, 3, P, P, P, P, P, P, P, P, P,
                                         None) == ENOTSUP
    # the fused front-end takes the same shapes as every other call
    for hd, sn in ((64, 96), (96, 128), (128, 32)):
        dd = _dims(d=hd, n=sn)
        assert lib.replay_append_decode_conv(ctypes.byref(dd), P, ctypes.byref(r), P, FAKE2, P, P, P, P,
                                             P, P, None, None) == ENOTSUP
    # capacity limits
    assert lib.replay_append_decode(ctypes.byref(_dims(L=0)), P, ctypes.byref(r), P, P, P, P, P, P,
                                    P, None, None) == EINVAL
    assert lib.replay_append_decode(ctypes.byref(_dims(L=33)), P, ctypes.byref(r), P, P, P, P, P,
                                    P, P, None, None) == ENOTSUP
    # verify window: T < 1, L < 2T, T > 8
    for T, L, code in ((0, 8, EINVAL), (5, 8, EINVAL), (9, 32, ENOTSUP)):
        dd = _dims(L=L)
        assert lib.replay_verify_T(ctypes.byref(dd), T, P, ctypes.byref(r), P, P, P, P, P, P, P,
                                   None, None) == code
        assert lib.gdn_replay_verify_T(ctypes.byref(dd), T, P, ctypes.byref(r), P, P, P, P, P, P,
                                       None, None) == code
    # ring records must be present and 128-byte aligned
    r_nometa = _ring()
    r_nometa.meta = None
    assert lib.replay_flush(ctypes.byref(d), P, ctypes.byref(r_nometa), None, None) == EINVAL
    # conv1d: only W = 4 and an even channel count
    assert lib.causal_conv1d_update(4, 3072, 3, P, P, P, P, None) == ENOTSUP
    assert lib.causal_conv1d_update(4, 3071, 4, P, P, P, P, None) == ENOTSUP
    assert lib.causal_conv1d_update(0, 3072, 4, P, P, P, P, None) == EINVAL
    # rollback needs accepted, and so does commit-and-verify
    assert lib.replay_rollback(ctypes.byref(d), ctypes.byref(r), None, None) == EINVAL
    assert lib.replay_commit_verify_T(ctypes.byref(d), 2, P, ctypes.byref(r), None, P, P, P, P, P, P, P,
                                      None, None) == EINVAL
    assert lib.gdn_replay_commit_verify_T(ctypes.byref(d), 2, P, ctypes.byref(r), None, P, P, P, P, P, P,
                                          None, None) == EINVAL
    assert lib.replay_commit_verify_T(ctypes.byref(d), 5, P, ctypes.byref(r), P, P, P, P, P, P, P, P,
                                      None, None) == EINVAL       # L < 2T
    r_odd = _ring()
    r_odd.meta = FAKE.value + 64
    assert lib.replay_rollback(ctypes.byref(d), ctypes.byref(r_odd), P, None) == EINVAL
    # every array 16-byte aligned: a misaligned input, output, ring array or flag
    # array is rejected before any launch
    M = ctypes.c_void_p(FAKE.value + 8)
    assert lib.ssm_decode_step(ctypes.byref(d), P, M, P, P, P, P, P, P, None) == EINVAL
    assert lib.replay_append_decode(ctypes.byref(d), P, ctypes.byref(r), P, P, P, P, P, P, M, None, None) == EINVAL
    assert lib.replay_append_decode(ctypes.byref(d), P, ctypes.byref(r), P, P, P, P, P, P, P, M, None) == EINVAL
    assert lib.replay_verify_T(ctypes.byref(d), 2, M, ctypes.byref(r), P, P, P, P, P, P, P, None, None) == EINVAL
    assert lib.replay_commit_verify_T(ctypes.byref(d), 2, P, ctypes.byref(r), M, P, P, P, P, P, P, P,
                                      None, None) == EINVAL
    assert lib.gdn_replay_verify_T(ctypes.byref(d), 2, P, ctypes.byref(r), P, P, M, P, P, P, None, None) == EINVAL
    assert lib.gdn_replay_append_decode(ctypes.byref(d), P, ctypes.byref(r), P, P, P, P, M, P, None, None) == EINVAL
    assert lib.replay_flush(ctypes.byref(d), P, ctypes.byref(r), M, None) == EINVAL
    assert lib.replay_rollback(ctypes.byref(d), ctypes.byref(r), M, None) == EINVAL
    assert lib.causal_conv1d_update(4, 3072, 4, P, P, M, P, None) == EINVAL
    assert lib.snapshot_commit(4, 2, 3, M, P, None, None) == EINVAL
    r_vu = _ring()
    r_vu.vu = FAKE.value + 4
    assert lib.replay_append_decode(ctypes.byref(d), P, ctypes.byref(r_vu), P, P, P, P, P, P, P, None,
                                    None) == EINVAL
    r_err = _ring()
    r_err.err = FAKE.value + 2
    assert lib.replay_rollback(ctypes.byref(d), ctypes.byref(r_err), P, None) == EINVAL
    for fn, args in (("rssm_ring_pointers", (M, None, None)), ("rssm_ring_reset", (M,))):
        assert getattr(lib, fn)(ctypes.byref(d), ctypes.byref(r), *args, None) == EINVAL
    assert lib.rssm_probe_copy(M, P, 64, None) == EINVAL
    assert lib.rssm_ring_reset(ctypes.byref(d), ctypes.byref(r_odd), None, None) == EINVAL
    # the pointer view: an aligned record array, L within the build
    assert lib.rssm_ring_pointers(ctypes.byref(d), ctypes.byref(r_odd), P, P, P, None) == EINVAL
    assert lib.rssm_ring_pointers(ctypes.byref(d), None, P, P, P, None) == EINVAL
    assert lib.rssm_ring_pointers(ctypes.byref(_dims(L=33)), ctypes.byref(r), P, P, P, None) == ENOTSUP

    # fused front-end: both conv buffers present and distinct
    assert lib.replay_append_decode_conv(ctypes.byref(d), P, ctypes.byref(r), P, P, P, P, P, P, P, P,
                                         None, None) == EINVAL
    Q = ctypes.c_void_p(0x2000)
    assert lib.replay_append_decode_conv(ctypes.byref(d), P, ctypes.byref(r), None, Q, P, P, P, P, P, P,
                                         None, None) == EINVAL
    assert lib.replay_append_decode_conv(ctypes.byref(_dims(d=96)), P, ctypes.byref(r), P, Q, P, P, P, P,
                                         P, P, None, None) == ENOTSUP

    # a pooled ring needs at least one row
    r_pool = _ring()
    r_pool.slots, r_pool.rows = FAKE.value, 0
    assert lib.replay_append_decode(ctypes.byref(d), P, ctypes.byref(r_pool), P, P, P, P, P, P, P,
                                    None, None) == EINVAL
    assert lib.replay_rollback(ctypes.byref(d), ctypes.byref(r_pool), P, None) == EINVAL
    r_pool.rows = 3
    assert lib.replay_append_decode(ctypes.byref(_dims(d=96)), P, ctypes.byref(r_pool), P, P, P, P, P,
                                    P, P, None, None) == ENOTSUP

    # storage-precision flags: unknown bits rejected; bf16 y only where honoured
    bad_flags = _dims()
    bad_flags.flags = 4
    assert lib.ssm_decode_step(ctypes.byref(bad_flags), P, P, P, P, P, P, P, P, None) == EINVAL
    # one 256-thread work-group per (request, head): B * H beyond 2^24 - 1 is refused
    huge = _lib.rssm_dims(1 << 23, 2, 64, 128, 1, 8, 0)
    assert lib.ssm_decode_step(ctypes.byref(huge), P, P, P, P, P, P, P, P, None) == EINVAL
    assert lib.replay_append_decode(ctypes.byref(huge), P, ctypes.byref(r), P, P, P, P, P, P, P, None,
                                    None) == EINVAL
    ybf = _dims()
    ybf.flags = _lib.RSSM_F_Y_BF16
    assert lib.ssm_decode_step(ctypes.byref(ybf), P, P, P, P, P, P, P, P, None) == ENOTSUP
    assert lib.gdn_decode_step(ctypes.byref(ybf), P, P, P, P, P, P, P, None) == ENOTSUP
    assert lib.ssm_snapshot_verify_T(ctypes.byref(ybf), 2, 3, P, P, P, P, P, P, P, P, P, None, None) == ENOTSUP
    out = (ctypes.c_size_t * 4)()
    ubf = _dims(B=2, H=4, d=64, L=8)
    ubf.flags = _lib.RSSM_F_U_BF16
    assert lib.rssm_ring_sizes(ctypes.byref(ubf), 1, out) == 0 and out[0] == 2 * 4 * 8 * 64 * 2

    # GDN append-decode: ring required, L in [1, 32], supported (d, n)
    assert lib.gdn_replay_append_decode(ctypes.byref(d), P, None, P, P, P, P, P, P, None, None) == EINVAL
    assert lib.gdn_replay_append_decode(ctypes.byref(_dims(L=0)), P, ctypes.byref(r), P, P, P, P, P, P,
                                        None, None) == EINVAL
    assert lib.gdn_replay_append_decode(ctypes.byref(_dims(L=33)), P, ctypes.byref(r), P, P, P, P, P, P,
                                        None, None) == ENOTSUP
    assert lib.gdn_replay_append_decode(ctypes.byref(_dims(d=96)), P, ctypes.byref(r), P, P, P, P, P, P,
                                        None, None) == ENOTSUP

    # snapshot route: T in [1, 8], nslots >= T + 1, slot and pool present
    for T, nslots, code in ((0, 4, EINVAL), (4, 4, EINVAL), (9, 10, ENOTSUP), (4, 5, ENOTSUP)):
        dd = _dims(d=96) if code == ENOTSUP and T == 4 else d
        assert lib.ssm_snapshot_verify_T(ctypes.byref(dd), T, nslots, P, P, P, P, P, P, P, P, P,
                                         None, None) == code
        assert lib.gdn_snapshot_verify_T(ctypes.byref(dd), T, nslots, P, P, P, P, P, P, P, P,
                                         None, None) == code
    assert lib.ssm_snapshot_verify_T(ctypes.byref(d), 2, 3, P, None, P, P, P, P, P, P, P,
                                     None, None) == EINVAL
    assert lib.snapshot_commit(4, 2, 2, P, P, None, None) == EINVAL
    assert lib.snapshot_commit(4, 2, 3, P, None, None, None) == EINVAL
    assert lib.snapshot_commit(0, 2, 3, P, P, None, None) == EINVAL

    # probes
    assert lib.rssm_probe_copy(P, P, 15, None) == EINVAL


def test_binding_rejects_host_tensors_and_wrong_shapes():
    torch = pytest.importorskip("torch")
    from ssm_recurrent_decode_amd import binding
    dims = binding.Dims(2, 4, 64, 128, 2, 8)
    st = torch.zeros(2, 4, 64, 128)
    with pytest.raises(ValueError):
        binding._p(st, "state", binding._F32, (2, 4, 64, 128))        # host tensor
    with pytest.raises(ValueError):
        binding._p(torch.zeros(3), "x", binding._F32, (2,))
    with pytest.raises(TypeError):
        binding._p(torch.zeros(2, dtype=torch.float64), "x", binding._F32, (2,))
    assert dims.c().capacity == 8


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "nope.so"))
