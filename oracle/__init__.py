"""CPU oracle for paged attention: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and this
package never imports the product: the two share no code.  The only module
both sides use is ``paged_kv_cache_19_amd.workloads``, which draws seeded
inputs and holds none of the method's arithmetic.

What the oracle computes, and the passage each part follows:

* ``block_manager`` -- the host block allocator (FIFO free list, reference
  counts, on-demand append, zero-copy fork, copy-on-write, free), after the
  block-manager code in "Inside vLLM: Anatomy of a High-Throughput LLM
  Inference System (2025)" (section "Code Architecture: Custom Block Manager
  and Scheduler Implementation") and the worked example in "03 --
  PagedAttention & the vLLM V1 Architecture" (section "The block table
  walkthrough").
* ``paged_attention`` -- slot computation, the cache write, the block-table
  gather and textbook softmax attention in float64 ("03 -- PagedAttention &
  the vLLM V1 Architecture", section "The attention kernel side"; "Inside
  vLLM", section "Physical Block Mapping and Kernel Invocation").
* ``block_ops`` -- whole-block copies between pools: copy-on-write inside
  a pool and swapping to and from a host pool ("03 -- PagedAttention & the
  vLLM V1 Architecture", sections "The block table walkthrough" and
  "Preemption & eviction").
* ``fp8`` -- the e4m3 KV cache: per-(block, KV head) scales, quantisation
  on the cache write (float32 division, clamp, round to nearest even) and
  attention over the dequantised pools ("Tech Radar: vLLM v1 Production
  Engine Architecture ...", section "Hopper TMA Warp Specialization & FP8
  Kernel Integration", item "FP8 Block-Quantized Caching").
* ``scheduler`` -- the host batch builder: the chunked-prefill token budget
  ("Tech Radar: vLLM v1 ...", section "The Dynamic Chunked Prefill
  Scheduler Formulation"), the schedule() step ("03 -- PagedAttention & the
  vLLM V1 Architecture", section "The scheduler's schedule() step"),
  hash-chained prefix reuse and preemption by recomputation; it emits the
  tables, lengths, query offsets and slots the attention calls take.
* ``sizes`` -- the closed forms for block counts, KV bytes and internal
  fragmentation ("Tech Radar: vLLM v1 Production Engine Architecture ...",
  section "Mathematical Modeling of PagedAttention v3 Memory Bounds").

Every function is pinned by ``tests/test_oracle_*.py`` to values the pages
print, closed forms, special cases and brute force; none is "parity
unpinned".
"""

from . import block_manager, block_ops, fp8, paged_attention, scheduler, sizes  # noqa: F401
