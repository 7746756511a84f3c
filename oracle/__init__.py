"""CPU oracle for batched single-token SSM decode -- TEST INFRASTRUCTURE ONLY.

Plain, slow float64 numpy implementations of what the decode path computes, written
from the ReplaySSM page ("ReplaySSM: Cache SSM Inputs, Not State", a summary of
Tri Dao's blog post) and checked against brute force, closed forms and invariants in
``tests/test_oracle_*.py``.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path (the HIP library and its Python binding)
never calls it, and this package shares no code with that path: inputs come in as
float64 arrays that the caller converted from the exact bf16/fp32 values the GPU
receives.

Modules
-------
mamba2   the standard Mamba-2 recurrence (the definition) and the per-draft
         snapshot semantics of speculative decoding.
replay   ReplaySSM bookkeeping written out on its own: a ring of recent inputs, an
         untouched checkpoint, output-only decode, flush when full, speculative
         verify with the early-flush rule, rollback by pointer move.
gdn      Gated DeltaNet: the Householder-form recurrence, its snapshot semantics,
         the ReplaySSM route that caches the corrections u, and the chunk-wise
         lower-triangular solve for a draft window.
conv1d   the causal depthwise conv1d state update with SiLU, and the split of a
         Mamba-2 layer's xBC channels into v, k, q.
rounding rounding to the bf16 grid, where a vector is handed on in bf16.

Every function's docstring names the passage it follows, and states the reading
taken where the page leaves a step open.  Nothing here is "parity unpinned": each
function has at least one pin that does not reuse its own formula.
"""
