"""ctypes view of the C ABI in include/ssm_recurrent_decode.h.

Loading fails loudly (ImportError) when the shared library has not been built:
there is no fallback implementation of any entry point."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int, c_int32, c_size_t, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libssm_recurrent_decode.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

RSSM_OK = 0
RSSM_EINVAL = -22
RSSM_ENOTSUP = -95
RSSM_ELAUNCH = -5
RSSM_ERR_POINTERS = 1
RSSM_ERR_ACCEPTED = 2
RSSM_ERR_PENDING = 4
RSSM_ERR_SLOT = 8
RSSM_ERR_DIVERGED = 16
RSSM_F_Y_BF16 = 1
RSSM_F_U_BF16 = 2
ABI_VERSION = 11  # RSSM_ABI_VERSION of the header this binding follows


class rssm_dims(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("nheads", c_int32), ("head_dim", c_int32),
                ("state_dim", c_int32), ("ngroups", c_int32), ("capacity", c_int32), ("flags", c_int32)]


class rssm_ring(ctypes.Structure):
    _fields_ = [("vu", c_void_p), ("k", c_void_p), ("meta", c_void_p), ("err", c_void_p),
                ("slots", c_void_p), ("rows", c_int32)]


_D = POINTER(rssm_dims)
_R = POINTER(rssm_ring)
_P = c_void_p

# name -> (restype, argtypes); the exported symbols declared in the header
SIGNATURES = {
    "rssm_abi_version": (c_int, []),
    "rssm_strerror": (c_char_p, [c_int]),
    "rssm_ring_sizes": (c_int, [_D, c_int, POINTER(c_size_t)]),
    "rssm_ring_reset": (c_int, [_D, _R, _P, _P]),
    "rssm_ring_pointers": (c_int, [_D, _R, _P, _P, _P, _P]),
    "ssm_decode_step": (c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "replay_append_decode": (c_int, [_D, _P, _R, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "replay_append_decode_conv": (c_int, [_D, _P, _R, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "replay_flush": (c_int, [_D, _P, _R, _P, _P]),
    "replay_verify_T": (c_int, [_D, c_int32, _P, _R, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "replay_rollback": (c_int, [_D, _R, _P, _P]),
    "replay_commit_verify_T": (c_int, [_D, c_int32, _P, _R, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdn_replay_commit_verify_T": (c_int, [_D, c_int32, _P, _R, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdn_decode_step": (c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdn_replay_verify_T": (c_int, [_D, c_int32, _P, _R, _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdn_replay_append_decode": (c_int, [_D, _P, _R, _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdn_replay_flush": (c_int, [_D, _P, _R, _P, _P]),
    "ssm_snapshot_verify_T": (c_int, [_D, c_int32, c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdn_snapshot_verify_T": (c_int, [_D, c_int32, c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "snapshot_commit": (c_int, [c_int32, c_int32, c_int32, _P, _P, _P, _P]),
    "causal_conv1d_update": (c_int, [c_int32, c_int32, c_int32, _P, _P, _P, _P, _P]),
    "rssm_probe_copy": (c_int, [_P, _P, c_size_t, _P]),
    "rssm_probe_read": (c_int, [_P, c_size_t, _P, _P]),
    "rssm_probe_read_sink_floats": (c_size_t, [c_size_t]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load the library once and attach prototypes to every exported symbol."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    try:
        # Load torch's HIP runtime first so this library binds to the same one
        # (one runtime per process: torch's streams are passed straight through).
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m ssm_recurrent_decode_amd.build` "
            "(the decode path has no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.rssm_abi_version() != ABI_VERSION:
        raise ImportError("libssm_recurrent_decode.so ABI version mismatch")
    if path == LIB_PATH:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().rssm_strerror(code).decode()


def check(code: int, what: str) -> None:
    if code != RSSM_OK:
        raise RuntimeError(f"{what} failed: {strerror(code)} (code {code})")
