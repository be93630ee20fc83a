"""Host block allocator with reference counts (oracle; test infrastructure only).

Follows the block-manager code of "Inside vLLM: Anatomy of a High-Throughput
LLM Inference System (2025)", section "Code Architecture: Custom Block Manager
and Scheduler Implementation", restated here in my own structure:

* the pool is a FIFO list of free block ids; ``allocate`` takes the front id
  and gives it reference count 1, and fails with ``MemoryError`` when the list
  is empty; ``free`` lowers the count and returns the id to the back of the
  list when it reaches 0;
* a sequence appends one token at a time: a fresh block when its token count
  is a multiple of the block size, otherwise, if its last block is shared
  (count > 1), a copy-on-write into a fresh block;
* ``fork`` copies the parent's table and raises the count of every block;
* ``free_sequence`` releases every block of the table.

Reading taken where the pages differ: the listing replaces the shared block
without moving any data, while "03 -- PagedAttention & the vLLM V1
Architecture" (section "The block table walkthrough") says the whole block is
copied when a write would diverge.  Without the copy the sequence would lose
the tokens already in that block, so ``append_token`` copies the block's
valid prefix (its first ``count mod B`` slots) through ``copy_hook``.

The same section's allocation lifecycle in "High-Throughput Local LLM
Infrastructure ..." (section "2.1 PagedAttention Memory Allocation
Life-Cycle") gives the on-demand rule (a new block once the offset reaches the
block size) and the release on completion.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence


class BlockAllocator:
    """FIFO pool of physical block ids with reference counts."""

    def __init__(self, free_order: Sequence[int]):
        ids = [int(b) for b in free_order]
        if len(set(ids)) != len(ids):
            raise ValueError("free_order holds a block id twice")
        self.num_blocks = len(ids)
        self.free_list: List[int] = list(ids)
        self.ref_count: Dict[int, int] = {b: 0 for b in ids}

    def allocate(self) -> int:
        if not self.free_list:
            raise MemoryError("no free physical block left in the pool")
        block = self.free_list.pop(0)
        assert self.ref_count[block] == 0
        self.ref_count[block] = 1
        return block

    def incref(self, block: int) -> None:
        assert self.ref_count[block] >= 1, "incref of a free block"
        self.ref_count[block] += 1

    def free(self, block: int) -> None:
        assert self.ref_count[block] >= 1, "reference count underflow"
        self.ref_count[block] -= 1
        if self.ref_count[block] == 0:
            self.free_list.append(block)

    def used_blocks(self) -> List[int]:
        return sorted(b for b, rc in self.ref_count.items() if rc > 0)


@dataclass
class Sequence_:
    """One sequence: its token count and its block table."""

    seq_id: int
    num_tokens: int = 0
    block_table: List[int] = field(default_factory=list)


CopyHook = Callable[[int, int, int], None]  # (src_block, dst_block, n_slots)


class BlockManager:
    """Sequence-to-block translation with fork and copy-on-write."""

    def __init__(self, free_order: Sequence[int], block_size: int,
                 copy_hook: Optional[CopyHook] = None):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.block_size = block_size
        self.allocator = BlockAllocator(free_order)
        self.copy_hook = copy_hook
        self.seqs: Dict[int, Sequence_] = {}

    # -- sequence lifecycle -------------------------------------------------
    def add_sequence(self, seq_id: int) -> Sequence_:
        if seq_id in self.seqs:
            raise KeyError(f"sequence {seq_id} exists")
        seq = Sequence_(seq_id)
        self.seqs[seq_id] = seq
        return seq

    def append_token(self, seq_id: int) -> int:
        """Make room for one more token; return the slot it must be written to.

        The slot is ``table[pos // B] * B + pos % B`` for the new position.
        """
        seq = self.seqs[seq_id]
        B = self.block_size
        offset = seq.num_tokens % B
        if offset == 0:
            seq.block_table.append(self.allocator.allocate())
        else:
            last = seq.block_table[-1]
            if self.allocator.ref_count[last] > 1:
                fresh = self.allocator.allocate()
                if self.copy_hook is not None:
                    self.copy_hook(last, fresh, offset)
                self.allocator.free(last)  # the other holders keep it
                seq.block_table[-1] = fresh
        pos = seq.num_tokens
        seq.num_tokens += 1
        return slot_for(seq.block_table, pos, B)

    def append_tokens(self, seq_id: int, n: int) -> List[int]:
        return [self.append_token(seq_id) for _ in range(n)]

    def fork(self, parent_id: int, child_id: int) -> Sequence_:
        parent = self.seqs[parent_id]
        child = self.add_sequence(child_id)
        child.block_table = list(parent.block_table)
        child.num_tokens = parent.num_tokens
        for b in child.block_table:
            self.allocator.incref(b)
        return child

    def free_sequence(self, seq_id: int) -> None:
        seq = self.seqs.pop(seq_id)
        for b in seq.block_table:
            self.allocator.free(b)
        seq.block_table.clear()

    # -- views ----------------------------------------------------------------
    def table(self, seq_id: int) -> List[int]:
        return list(self.seqs[seq_id].block_table)

    def check_invariants(self) -> None:
        """Refcounts equal table references; free and used blocks partition
        the pool; no free block is referenced; each table covers its tokens."""
        refs: Dict[int, int] = {}
        for seq in self.seqs.values():
            assert len(seq.block_table) == -(-seq.num_tokens // self.block_size)
            for b in seq.block_table:
                refs[b] = refs.get(b, 0) + 1
        alloc = self.allocator
        for b, rc in alloc.ref_count.items():
            assert rc == refs.get(b, 0), f"block {b}: rc {rc} != refs {refs.get(b, 0)}"
        free = set(alloc.free_list)
        assert len(free) == len(alloc.free_list), "free list holds a duplicate"
        used = set(alloc.used_blocks())
        assert not (free & used)
        assert len(free) + len(used) == alloc.num_blocks


def slot_for(block_table: Sequence[int], pos: int, block_size: int) -> int:
    """Physical slot of logical position ``pos``: block id times B plus offset.

    The logical block index is floor(pos / B) and the offset pos mod B
    ("High-Throughput Local LLM Infrastructure ...", section "1.2
    PagedAttention Mechanics & Virtual Page Tables"; "Inside vLLM", section
    "Physical Block Mapping and Kernel Invocation").
    """
    return int(block_table[pos // block_size]) * block_size + pos % block_size
