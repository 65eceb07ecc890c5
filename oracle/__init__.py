"""CPU oracle for the Medusa tree-verify step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy implementation of what one Medusa decoding step
computes, written from the method's description (Medusa paper digest,
"Method" items 1-5 and "Algorithm: Medusa decoding step"; wq-win lecture note
on Medusa, sections 二 and 三).  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the GPU library never calls
it and shares no code with it.

Modules:
  tree    -- flattening a prefix-closed path list into parent/depth/rank and
             ancestor sets (Method 3, Algorithm step 2)
  model   -- Llama-style backbone: causal forward and tree-verify forward
             (Method 3, Algorithm step 3)
  heads   -- Medusa heads and per-head top-s (Method 1-2, Algorithm step 1)
  accept  -- root selection, greedy and typical acceptance, best candidate
             (Method 5, Algorithm steps 4-5)
  decode  -- KV compaction, one full step, prefill, vanilla greedy decoding
             (Algorithm step 6)
  metrics -- the speedup identity (Results, app. B.1)
  train   -- the Medusa-1 head loss and its gradients (Method 6, eq. 1)

Every function here is pinned by a `-m "not gpu"` test against something other
than itself (a library implementation, a closed form, a brute force, or a
worked example from the pages); see tests/test_oracle_*.py.
"""
from . import accept, decode, heads, metrics, model, train, tree  # noqa: F401
