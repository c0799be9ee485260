"""fp64 CPU oracle for causal ring attention under HeadTail sharding.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only the tests, the smoke check of ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import or run it. It shares no code with the HIP library.

Modules
  shard      HeadTail shard map (integer, exact)
  attention  full-sequence causal softmax attention and block attention at
             global positions, forward (O, LSE) and analytic backward
  merge      log-sum-exp merge of two partial results
  rope       rotary position embedding at global positions, and the backward
             through it (the transposed rotation)
  gqa        grouped-query attention: KV heads shared by groups of query heads
  brute      pure-Python loop versions for tiny inputs (independent cross-check)
  ring       the ring schedule assembled from the pieces above (used by the
             invariant tests: any chunk partition, any ring order)

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (a worked example from the pages, a closed form, an invariant,
brute force, or finite differences). No function here is "parity unpinned".
"""
