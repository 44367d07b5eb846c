"""CPU oracle for the streaming frame-to-cache attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only the tests, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants) and never reads anything
the HIP path produced.

The oracle is plain and slow on purpose: numpy in float64 plus Python
integers, one definition per function, written from the pages:

* ``window``    -- keyframe rule, sliding-window eviction with never-evicted
                   scale frames, and the page allocator that the page tables
                   are compared against (GCTStream explainer, "KV Cache
                   Lifecycle Management", "Streaming Inference Pipeline",
                   "Sliding Window Eviction"; LingBot-Map 20 FPS explainer,
                   "Sliding-Window Eviction Strategy", "Keyframe Interval
                   Configuration").
* ``attention`` -- softmax attention of a frame's queries over an explicit list
                   of retained keys/values (GCTStream explainer, "Frame-by-
                   Frame Causal Processing" and "Scale-Frame Phase").
* ``clces``     -- cross-layer rank-consistency score, fused score, top-k
                   keep and page-local compaction (StreamCacheVGGT article,
                   section 2.1 and its sub-sections 2.1.1-2.1.4; InfiniteVGGT
                   explainer, "Rolling Memory" and "Prune and roll the memory").
* ``budget``    -- the per-layer token-budget policy that runs the CLCES step
                   after every frame (the two pages above combined).

Every function states whether it is pinned by a test against something other
than itself; see the tests under ``tests/test_oracle_*.py``.
"""

from . import window, attention, clces, budget  # noqa: F401
