"""CPU oracle for tree verification — TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy statement of what the verification path computes,
written from the pages that describe tree-based speculative decoding:

* tree-masked verify attention: every flattened draft-tree node attends to the
  whole committed prefix plus its own ancestors and itself ("Report: Support
  nextn speculative decoding", section "Tree-based Speculative Decoding (EAGLE)
  Implementation Summary", step 3, and the tree_mask discussion above it);
* speculative rejection sampling with residual resampling and a bonus token
  ("Speculative Decoding" notes, section "Draft Token Validation"), tried over
  the siblings of a node in turn, with the Sequoia without-replacement variant
  ("Sequoia: Scalable and Robust Speculative Decoding" summary, "Robust
  Sampling");
* selective KV-cache compaction to the accepted path (the EAGLE report's
  "Important Implementation Detail" and "Issue: Speculative Decoding on vLLM";
  the SGLang "SpeculativeDecoding" doc, "Prefix Match");
* the step before attention: rotary positions that follow the tree and the
  write of the tree's K/V rows into the paged cache (``rope.py``);
* top-k / top-p truncation of the target logits before the acceptance tests
  (``truncate.py``);
* the Sequoia tree-construction dynamic program over a positional acceptance
  vector (``sequoia.py``; the objective and recurrence come from the published
  Sequoia paper, the pages only name the method).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and the library never calls it.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, brute force, library routines, exact enumeration, the worked
example of the SGLang doc); the one exception is the absolute bit pattern of
Philox4x32-10, which is pinned only to the known-answer vectors of its
published reference implementation (see ``philox.py``).
"""
from .philox import philox4x32_10, uniform_draw, draw_counter  # noqa: F401
from .tree import Tree, tree_structure  # noqa: F401
from .attention import tree_attention, tree_attention_rows  # noqa: F401
from .reject import (  # noqa: F401
    PhiloxDraws,
    accept_draw,
    accept_margin,
    final_margin,
    accept_flag_probability,
    final_flag_probability,
    final_draw_candidates,
    inverse_cdf,
    residual_update,
    without_replacement_update,
    softmax64,
    reject_sequence,
    tree_reject,
    FLAG_MARGIN,
)
from .compact import kv_compact  # noqa: F401
from .rope import rope, tree_kv_write, tree_positions  # noqa: F401
from .truncate import truncate_logits, truncate_row  # noqa: F401
from .sequoia import expected_tokens, sequoia_tree  # noqa: F401
