"""CPU oracle for attention over a per-KV-head mixed (retrieval / streaming) KV cache.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy / pure-Python code that
states what the hot path must compute, written from the DuoAttention pages:

  * "DuoAttention: Dual Retrieval & Streaming Heads Guide" -- the head split,
    the cache partition (full buffer per retrieval head, sink + rolling window
    per streaming head), the KV-size formulas and the head-separation simulation;
  * "Attention Variants and KV-Cache Compression" -- the KV-size formula with its
    512 MiB example and, in "When Is Reuse Exact?", the rule that chunk row i
    attends through absolute key position (cached + i) with original positions
    preserved after eviction;
  * "Attention Variants and Memory Efficiency" -- repeat_kv head mapping for
    GQA, and in "Sliding-Window and Mixed Attention" the window of query t and
    the ring-buffer slot rule with its printed example.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
under ``head_wise_kv_amd/`` and never imports it.

Parity status: every function here is pinned by a test in ``tests/`` against a
value printed on the pages, a closed form, a library routine on a special case,
or brute force on tiny inputs (see each module's docstring).  None is
"parity unpinned".
"""
from . import sizes, cache, attention  # noqa: F401
