"""Float64 CPU oracle for one rank's share of context-parallel Pass-KV ring attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library or its Python binding; the only common module is the seeded input
generator (``context_long_attention_amd.inputs``), which holds no attention
arithmetic and which this package does not import either.

Every function is written from the pages' statement of the method and from the
plain definition of softmax attention, slowly and in float64:

* zigzag partition -- "Context Parallelism for Scalable Million-Token
  Inference", section "Load Balancing in CP";
* ring order and Pass-KV -- same page, section "Ring Attention Algorithms";
  "Announcing Long-Context Training on TPUs with MaxText Context Parallelism",
  section "Context Parallelism in MaxText" (P2P paragraph, Figure 3);
* causal visibility -- "Context Parallelism for Scalable Million-Token
  Inference", section "Attention Compute Patterns in Multi-Turn Chat" (full
  prefill);
* packed documents and skipping of fully masked blocks -- "Announcing
  Long-Context Training ...", section "Built on a fast attention kernel";
* merge of partial outputs -- "Context Parallelism for Scalable Million-Token
  Inference", section "Ring Attention Algorithms" (final output of Pass KV);
* sliding-window visibility -- "Announcing Long-Context Training ...", closing
  section (window layers of models such as Gemma, run with a short exchange
  between neighbouring chips).

Pins: every function is checked by ``tests/test_oracle_*.py`` against the
pages' worked example, closed forms, library routines and brute force.  The
FLOP-counting convention (``causal_flops``) and the GPU rounding tolerance are
the only parts with no pin ("parity unpinned").
"""
from .ring import (  # noqa: F401
    CLS_DIAG, CLS_DOC, CLS_FULL, CLS_SKIP, TILE_FULL, TILE_PARTIAL, TILE_SKIP,
    attention_backward_partial, attention_partial, causal_flops, chunk_pair_class,
    delta_rows, document_index, merge, rank_backward, rank_forward, ring_source,
    tile_map, visibility, zigzag_chunks, zigzag_positions,
)
