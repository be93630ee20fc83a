"""Whole-block copy and swap (oracle; test infrastructure only).

What the method does, restated from the pages:

* Copy-on-write: before a sequence writes into a block it shares, the block
  is copied into a fresh one, whole blocks at a time ("03 -- PagedAttention
  & the vLLM V1 Architecture", section "The block table walkthrough";
  "High-Throughput Local LLM Infrastructure ...", section "Reference
  Counting & Copy-on-Write (CoW)").
* Preemption by swapping: a sequence's blocks are written out to pinned host
  memory and later brought back into (possibly other) GPU blocks ("03 --
  PagedAttention & the vLLM V1 Architecture", section "Preemption &
  eviction"; "Inside vLLM", section "Preemption Mechanics: Swapping vs.
  Recomputation").

Both are one operation: for every pair (src, dst) of the mapping, block dst
of the destination pool becomes a bit copy of block src of the source pool.
A pool is any tensor whose first dimension is the block id (K and V pools,
and the per-block scales of an fp8 cache, alike).

Readings: destination blocks of one call are distinct; within one pool no
destination is also a source of the same call (otherwise the result would
depend on the order of the copies).
"""

from __future__ import annotations

import torch

from .paged_attention import _as_cpu_long


def _pairs(block_mapping):
    m = _as_cpu_long(block_mapping).reshape(-1, 2)
    return [(int(s), int(d)) for s, d in m.tolist()]


def copy_blocks(dst_pool: torch.Tensor, src_pool: torch.Tensor, block_mapping,
                same_pool: bool = False) -> torch.Tensor:
    """Return a copy of ``dst_pool`` with block d replaced by block s of
    ``src_pool`` for every (s, d) in ``block_mapping`` ([n, 2])."""
    pairs = _pairs(block_mapping)
    dsts = [d for _, d in pairs]
    assert len(set(dsts)) == len(dsts), "a destination block appears twice"
    if same_pool:
        assert not (set(dsts) & {s for s, _ in pairs}), "a block is both source and destination"
    out = dst_pool.clone()
    for s, d in pairs:
        assert 0 <= s < src_pool.shape[0] and 0 <= d < dst_pool.shape[0]
        out[d] = src_pool[s]
    return out


def copy_blocks_in_pool(pool: torch.Tensor, block_mapping) -> torch.Tensor:
    """Copy-on-write copies inside one pool."""
    return copy_blocks(pool, pool, block_mapping, same_pool=True)
