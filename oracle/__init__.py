"""Oracle for the paged KV cache: a plain, slow, CPU statement of what the method computes.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything here; the
library (``paged_kv_cache_53_amd``) never does, and it shares no code,
header, table or helper with this package.

Parts (each file's docstring cites the passages it follows):

* ``memory_math``  -- the byte and utilisation arithmetic of the pages (O1)
* ``allocator``    -- the block manager as plain lists and dicts (O2)
* ``scatter``      -- writing token rows into physical slots, and reading a
                      sequence's logical K/V back through its block table (O3)
* ``attention``    -- decode attention over the gathered K/V, in fp64 (O4)
* ``fp8``          -- the FP8 E4M3 codes of a quantised cache, with per-tensor
                      scales (the quantised-KV extension)

Source pages (cited by title and section):

* "Contiguous vs Paged KV Cache on RDNA4: Why an Agent Swarm Runs Out of VRAM
  Early" (zolotukhin.ai blog)
* "KV-Cache Optimization & PagedAttention for Long-Context Agents"
  (akmalkhaniub.github.io blog)
* "Reserve for the worst case, or page" (inference.academy explainer)
* "KV-cache paging in vLLM" (zhanyl-tech.github.io blog post of 2026-01-15)
* "PagedAttention -- Math + Memory Model" (aicassindra.com transformer math)

Every function here is pinned by tests under ``tests/`` against values the
pages print, closed forms, brute force or library routines; none is marked
"parity unpinned".
"""
from . import memory_math, allocator, scatter, attention, fp8  # noqa: F401
