"""fp64 CPU oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path (the HIP
library under ``exact_attention_13_amd``) never imports, links or calls it,
and the two share no code.

Contents:
  * ``reference.fwd``       -- three-pass fp64 attention (C, ``fa_oracle.c``),
                               the plain definition of what the method computes;
  * ``reference.fwd_gqa``   -- the same with grouped K/V heads and separate
                               query / key lengths (decoding);
  * ``reference.combine``   -- fp64 merge of results over disjoint key ranges;
  * ``reference.bwd``       -- fp64 gradients of sum(dO * O) w.r.t. Q, K, V,
                               grouped K/V heads and N_q != N_kv included
                               (``bwd_dq_rows``: dQ of sampled rows only);
  * ``online_ref``          -- the tile-by-tile online-softmax recurrence in
                               numpy fp64, in the deferred-normalisation form and
                               in the per-step-normalised form, used only to pin
                               the method's claim that it equals the plain
                               definition.
"""
from .reference import (build, fwd, fwd_gqa, combine, bwd, bwd_dq_rows, widen,  # noqa: F401
                        FLAT_ROWS_ALL)
