"""CPU oracle for packed segment-id masked attention (TEST INFRASTRUCTURE).

Plain, slow, fp64 NumPy code that states what the hot path computes.  Only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it; the product path (the HIP library and its binding) never does
and shares no code with it.

Pages cited (by title and section):
  * "LingBot-VA packing" report -- section 2.1 (packing module: pad to a
    multiple of 8 frames, ``valid_frames``, frames past ``valid_frames`` get
    seq id -1 in both the self- and cross-attention masks), section 2.2 (the
    packed-vs-single verification) and the section 3.1 table (no NaN in
    fully masked padding rows, finite gradients).
  * "Furniture packing, variable length" report -- implementation part: a
    seq id of -1 removes a token from attention as both query and key, and
    tokens only attend to tokens with the same seq id.
  * AdaptiveLoad summary -- section 2A: dual-constraint batch sizing and the
    step-cost fit; section 2B: the fused LayerNorm-Modulate (AdaLN)
    operation and its modulation-gradient reduction over the sequence.
  * "LingBot-VA attention profiling" report -- next steps: the document-id
    mask predicate ``doc_id[q] == doc_id[k]``; conclusion: several episodes
    concatenated per GPU up to its token budget.

Modules:
  seqids     -- per-token seq ids from valid frames or from episode lengths
  packing    -- next-fit assignment of episodes to packs under a token budget
  loss       -- frame-valid masked squared-error loss and its gradient
  adaln      -- LayerNorm with per-segment modulation, forward and backward
  sampler    -- length-bucket batch sampler, dual-constraint batch sizing, cost fit
  blockmask  -- per tile-pair valid-pair counts, classes and CSR lists
  attention  -- per-episode dense softmax attention and its gradients

Every function here is pinned by ``tests/test_oracle_*.py`` against brute
force, torch's fp64 attention with autograd, finite differences, closed forms
and the pages' invariants; none is marked "parity unpinned".
"""
from . import seqids, blockmask, attention, loss, packing, adaln, sampler  # noqa: F401
