"""Plain fp64 CPU oracle for the speculative-decoding attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or calls this
package; only the test-suite, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP path: it reads the same seeded inputs
(bf16 bit patterns or float32 arrays) and computes every result from the plain
definitions, in float64, with NumPy.

Sources (page title, then the passage):

* "Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
  Context" (Pith review) -- "What carries the argument": the draft attends
  only to the first ``n_sink`` tokens plus the last ``W`` tokens; RoPE is
  already inside the cached keys, so scores are plain dot products; the
  draft KV pool can be compacted into a ring buffer.
* "BudgetDraft: Acceptance-Aware Multi-View Training for Sparse-KV Speculative
  Decoding" (Pith review) -- abstract and Figure 2: the drafter reads a sparse
  KV view under a fixed budget, the verifier reads the full cache and produces
  greedy targets.
* "SpecMemo: Speculative Decoding is in Your Pocket" (Pith review) -- "What
  carries the argument" and Figure 9: tree attention mask over N speculated
  nodes; batched verification pads accepted tokens, remaps position IDs to
  ignore padding and gives cached padding slots -inf.
* "SpecPV: Improving Self-Speculative Decoding for Long-Context Generation via
  Partial Verification" -- section 4.1 "Metrics": the accept length may be 0;
  section 3.3: candidates that were not accepted leave the cache once
  verification is done, and full verification refreshes the partial cache;
  section 3.2 and 4.1: the partial cache is chosen block by block with mean
  reduction and is one contiguous KV segment.

Pin status: every public function here is pinned by ``tests/test_oracle_*.py``
against something other than itself (library SDPA, closed forms, brute force,
values fixed by construction, hand-enumerated fixtures under
``tests/golden/``).  No function is "parity unpinned".
"""
from .bf16 import decode_bf16, as_f64
from .attention import (draft_view, draft_attn_ref, tree_depths, tree_ancestors,
                        position_ids, verify_attn_ref)
from .accept import argmax_ref, accept_ref, accept_bruteforce
from .commit import commit_ref, compact_ref
from .select import block_means_ref, block_scores_ref, select_blocks_ref
from .partial import gather_ref, verify_mode_ref
from .ring import ring_draft_ref, ring_from_logical, ring_slot

__all__ = ["decode_bf16", "as_f64", "draft_view", "draft_attn_ref", "tree_depths",
           "tree_ancestors", "position_ids", "verify_attn_ref",
           "argmax_ref", "accept_ref", "accept_bruteforce", "commit_ref",
           "block_means_ref", "block_scores_ref", "select_blocks_ref", "gather_ref",
           "verify_mode_ref", "ring_draft_ref", "ring_from_logical", "ring_slot"]
