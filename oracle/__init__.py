"""Plain, slow, obviously correct CPU oracle for document-masked attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path: it shares
no code with it.  The only module both sides use is the seeded input
generator, which holds no attention arithmetic.

All arithmetic is float64 numpy.  Sources (web pages on context parallelism):

* "FlashCP: Load-Balanced Communication-Efficient Context Parallelism for LLM
  Training" (FlashCP paper): section 2.1 and Figure 1(a) define the document
  mask (intra-document causal attention over a packed sequence); section 3.1
  gives the shard workload W = (2p + s + 1) * s / 2 (diagonal included);
  section 2.2 gives the 2 x CP chunking; section 3.2 and Eq. 4 / Eq. 5 the
  sharding-aware KV exchange (only shards that are not their document's last
  shard travel, compacted into one buffer); section 3.3 and Algorithm 1 the
  Whole-Doc / Per-Doc heuristic planner.
* "LLM Context Parallel in Production" (production guide): the online-softmax
  combination of per-KV-block partial results keeps the row maximum and the
  exponential sum ("Core Principle: Split Q, Circulate KV"); block skipping and
  the effective QK block count ("Causal Attention Creates Rank Load
  Imbalance"); cumulative-length arrays for variable-length attention.
* The CP-variance article (liuch.name): causal pair count L(L+1)/2 ("Theory").

The pages never write the backward pass; ``attention_backward`` is the exact
gradient of <dO, O> by plain calculus.  Readings where the pages are silent are
listed in each function's docstring.

Pins: every function here is checked against things other than itself in
``tests/test_oracle_*.py`` (library routines, closed forms, invariants, brute
force, finite differences, hand-derived fixtures in ``tests/golden/``).
"""
from .attention import (doc_index, local_positions, allowed_mask, attention_forward,
                        attention_backward, lse_merge)
from .convert import round_to_bf16_bits
from .exchange import (document_shards, is_last_shard, sent_rows, eq4_elements, eq5_elements,
                       packed_send_buffer, needed_positions, received_kv)
from .planner import shard_workload, flashcp_plan, plan_chunks, imbalance_ratio
from .schedule import (q_tiles, kv_tiles, tile_pair_counts_bruteforce, tile_pair_counts,
                       classify, schedule, need_intervals, useful_pairs, lpt_order)

__all__ = [
    "doc_index", "local_positions", "allowed_mask", "attention_forward", "attention_backward",
    "lse_merge", "q_tiles", "kv_tiles", "tile_pair_counts_bruteforce", "tile_pair_counts",
    "classify", "schedule", "need_intervals", "useful_pairs", "lpt_order", "round_to_bf16_bits",
    "document_shards", "is_last_shard", "sent_rows", "eq4_elements", "eq5_elements", "packed_send_buffer",
    "needed_positions", "received_kv", "shard_workload", "flashcp_plan", "plan_chunks", "imbalance_ratio",
]
