"""Plain, slow, obviously-correct fp64 CPU oracle for document-masked causal attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (no common helpers, tables or generators); the two meet only in the
seeded input module ``workloads``.

What it computes, and the passage each part follows:

* ``attention.allowed``      -- the document-causal mask. HSAP summary page
  (gptget.net/papers/2606.30460), original abstract: causal attention over
  packed (hybrid-context) sequences must not let one document's tokens see
  another's. AutoSP page (gist.science/zh/paper/2604.27089), section 2.A step 4
  (index recomputation): masks follow the tokens' global positions after the
  sequence is sharded.
* ``attention.forward``      -- softmax attention restricted to that mask, over
  whatever KV rows one call holds, giving O and the log-sum-exp.
* ``attention.merge``        -- exact combination of two partial results over
  disjoint KV sets. SP blog page (bmjup.com/post/14448.html), FAQ Q1: sequence
  parallelism is a computation-equivalent transform of single-device
  attention; its core-principles section: a ring of KV chunks gives every rank
  the full-sequence result. The pages give no formula: the log-sum-exp merge
  is the plain reading of "exact".
* ``attention.backward``     -- gradients of the same function, computed from
  the saved final O and LSE (recompute form; the attention-level echo of the
  AutoSP page's section 2.B, which keeps attention and recomputes the rest).
* ``planner.plan``           -- which (Q-tile, KV-tile) pairs hold any allowed
  pair, and whether each is FULL, DIAGONAL or PARTIAL. This is the one-device
  analogue of the HSAP summary page's method section: schedules are generated
  ahead of time for incomplete tensors and irregular attention.
* ``balance.balance``        -- which rank holds each chunk of query rows, so
  that ranks with equal token counts get nearly equal attention work. HSAP
  summary page, technical contributions (load balance across devices by
  scheduling); SP blog page, future trends and challenges (uneven lengths
  leave GPUs idle). The rule itself is a reading: heaviest chunk first to the
  least-loaded rank with room.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
closed forms, hand-worked examples, a library routine (torch's scaled_dot_product_attention in
float64 on each document alone, torch.autograd) and invariants.
"""
