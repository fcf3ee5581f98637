"""Plain, slow fp64 CPU oracle for one rank's share of Ring Attention.

TEST INFRASTRUCTURE ONLY. Nothing but ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It imports nothing from
``blockwise_ring_attention_amd`` (the HIP product path) and shares no code with it; the
two meet only in the seeded input generator, which holds none of the method's arithmetic.

Functions and their pins (the tests that tie each one to something other than itself):

* ``attention.rank_forward`` -- full-row softmax attention, the definition the ring
  reaches exactly. Pinned by: 50-digit brute force on tiny inputs; the independent
  blockwise combination of per-block partials in any block order; torch's fp64 scaled-dot-product attention with
  ``enable_gqa`` on the full sequence; gathering rank rows out of full-sequence causal
  attention; closed forms (Q = 0, constant V, key shift).
* ``attention.rank_forward(..., doc_start=...)`` -- the document mask of packed
  sequences. Pinned by: torch's fp64 causal attention run separately on every document
  span; 50-digit brute force; all-zero starts reduce to the causal mask; shares gathered
  out of the full sequence; the Q = 0 closed form (lse = ln of the document prefix).
* ``attention.merge`` -- combination of two partial results. Pinned by: merging results
  over disjoint key sets equals the oracle over their union; identity and symmetry.
* ``fold.blockwise_attention`` -- attention rebuilt from each key block's own partial
  result (out_i, lse_i), combined two at a time with logaddexp weights in a given order;
  a second implementation used only to pin the first. Pinned by: the same brute force,
  the page's worked example, and equality with the full row in every order.
* ``attention.chunk_positions``, ``attention.ring_blocks``, ``attention.allowed_count``,
  ``attention.chunk_units`` -- ownership and counting. Pinned by: the load-balance
  figures the pages print (i+1 units per rank contiguous, 2c+1 zigzag) and exact
  closed-form counts checked by brute force.

No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    allowed_count,
    chunk_positions,
    chunk_units,
    document_allowed,
    kv_head,
    merge,
    rank_forward,
    ring_blocks,
)
from .fold import blockwise_attention, block_partial, combine_partials  # noqa: F401
