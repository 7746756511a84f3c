"""MI355X (gfx950) batched single-token SSM decode: standard Mamba-2, ReplaySSM
(append-decode, flush, speculative verify, rollback), Gated DeltaNet ReplaySSM
verify/flush, the per-draft snapshot route that speculative decoding uses without
ReplaySSM (the comparator), and the causal conv1d state update.

The compute lives in hand-written HIP kernels behind the C ABI declared in
include/ssm_recurrent_decode.h (libssm_recurrent_decode.so, built in-tree by
``python -m ssm_recurrent_decode_amd.build``).  The names exported here are the
thin PyTorch binding of that ABI; they are loaded lazily so that the input
generators in ``synth`` can be used without torch or a GPU.
"""

_BINDING_NAMES = (
    "Dims", "Ring", "ring_sizes", "rssm_ring_reset", "rssm_ring_pointers", "ssm_decode_step", "replay_append_decode",
    "replay_append_decode_conv", "replay_flush", "replay_verify_T", "replay_commit_verify_T", "replay_rollback",
    "gdn_decode_step", "gdn_replay_commit_verify_T",
    "gdn_replay_verify_T", "gdn_replay_append_decode", "gdn_replay_flush", "ssm_snapshot_verify_T", "gdn_snapshot_verify_T",
    "snapshot_commit", "causal_conv1d_update", "rssm_probe_copy",
    "rssm_probe_read", "probe_read_sink_floats", "Prepared", "prepare_replay_append_decode",
    "prepare_ssm_decode_step", "prepare_causal_conv1d_update",
)

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
