"""Host batch builder: chunked-prefill scheduling with prefix reuse (oracle;
test infrastructure only).

What the method does, restated from the pages:

* Token budget per step ("Tech Radar: vLLM v1 Production Engine
  Architecture ...", section "The Dynamic Chunked Prefill Scheduler
  Formulation", equations 1-3): every active decode stream gets its one token
  first, N_decode = |R_decode|; what is left for prompt chunks is
  C_avail = max(0, T_budget - N_decode); a pending prompt p with U_p
  uncomputed tokens gets c_p = min(U_p, C_chunk, C_avail).
* The step itself ("03 -- PagedAttention & the vLLM V1 Architecture",
  section "The scheduler's schedule() step"): running requests first (a
  request whose next tokens cannot get KV blocks is preempted), then waiting
  requests are admitted in arrival order while budget is left, after a
  prefix-cache lookup; admission stops at the first request that cannot be
  allocated.
* Prefix reuse: full blocks are keyed by a hash of their tokens chained to
  the previous block's key, so a key names a whole prefix; a request whose
  leading full blocks match cached keys reuses those physical blocks
  (reference count + 1) and skips their prefill ("Inside vLLM ...", section
  "Zero-Copy Branching and Parallel Sampling", prefix caching; "Tech Radar
  ...", section "Prefix Caching: Radix Tree vs. Hash-Based Indexing").
* Preemption by recomputation: the request's blocks are released and it
  returns to the front of the waiting queue, to be prefilled again ("03 --
  ...", section "Preemption & eviction").
* Preemption by swapping: the request's blocks are copied to host swap
  space and released on the device; later its blocks are copied back into
  fresh device blocks and it continues where it stopped, without recomputing
  ("03 -- ...", section "Preemption & eviction"; "Inside vLLM ...", section
  "Preemption Mechanics: Swapping vs. Recomputation").

Readings where the pages are silent (each is listed in the design notes):

* C_avail is consumed in order: running prefill chunks first (in running
  order), then admissions; equation 3 is applied to each with what is left.
* Decode tokens are always scheduled (they are reserved before the budget
  is split), even past T_budget.
* The batch is packed in the order decodes, running prefills, admissions.
* A cache hit covers at most (len(tokens) - 1) // B full blocks, so at
  least one token is computed (its logits are needed) and it falls in a
  block the request owns.
* Freed blocks go to the back of the free list and keep their key until the
  allocator hands them out again (then the key is dropped); a hit on such a
  block takes it out of the free list.  A full block's key is registered
  when the step that computes its last token is scheduled, unless the key
  is already taken.
* Keys: 64-bit FNV-1a over the parent key's 8 bytes (little-endian) and the
  block's tokens as 4-byte little-endian integers; the first block's parent
  key is the FNV offset basis.
* Preemption takes the request that cannot allocate (the page's code); its
  prompt becomes all its tokens so far.  A step that preempted admits no
  waiting request (memory is short).
* A request ends when a step computed all its tokens and it has generated
  max_new_tokens; otherwise the caller appends the token it sampled.
* Swapping (pages name both modes but no rule to choose): with a host swap
  space of ``num_host_blocks`` blocks, a preempted request is swapped out
  when the swap space has a host block for each of its device blocks, else
  recomputed.  Host blocks come from a FIFO free list.  Swapped requests
  wait in a FIFO of their own; a step that preempted nobody swaps them back
  in, in order, after the running requests and before any admission, each
  while budget is left and the device has blocks for all of its tokens plus
  this step's (a decode token takes one unit of budget here, as its row is
  not among the step's first reserved decodes).  A swapped-in request gets
  fresh device blocks, its full blocks are keyed again (unless the keys are
  taken), and it is scheduled in the same step.  No request is admitted
  while any is swapped out.  The step reports the copies: swap_out pairs
  (device block, host block), swap_in pairs (host block, device block); the
  caller runs the swap-outs before the swap-ins and both before the step's
  cache write.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    for b in data:
        h ^= b
        h = (h * FNV_PRIME) & MASK64
    return h


def block_key(parent: int, tokens: Sequence[int]) -> int:
    data = parent.to_bytes(8, "little") + b"".join(
        (t & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    return fnv1a64(data)


@dataclass
class Request:
    req_id: int
    tokens: List[int]
    prompt_len: int
    max_new_tokens: int
    generated: int = 0
    num_computed: int = 0
    table: List[int] = field(default_factory=list)
    keys: List[int] = field(default_factory=list)   # keys of the table's full blocks
    host_table: List[int] = field(default_factory=list)  # swap-space blocks while swapped out

    @property
    def pending(self) -> int:
        return len(self.tokens) - self.num_computed


@dataclass
class Scheduled:
    req_id: int
    q_len: int
    seq_len: int          # tokens in the cache after this step
    table: List[int]
    slots: List[int]      # slots of the q_len new tokens


@dataclass
class Batch:
    entries: List[Scheduled]
    preempted: List[int]                      # every request preempted in this step
    swapped_out: List[int] = field(default_factory=list)   # those of them swapped out
    swap_out: List[tuple] = field(default_factory=list)    # (device block, host block)
    swap_in: List[tuple] = field(default_factory=list)     # (host block, device block)

    @property
    def num_tokens(self) -> int:
        return sum(e.q_len for e in self.entries)

    def query_start_loc(self) -> List[int]:
        out = [0]
        for e in self.entries:
            out.append(out[-1] + e.q_len)
        return out


class Scheduler:
    def __init__(self, num_blocks: int, block_size: int, token_budget: int, chunk_tokens: int,
                 free_order: Optional[Sequence[int]] = None, num_host_blocks: int = 0):
        self.B = block_size
        self.token_budget = token_budget
        self.chunk_tokens = chunk_tokens
        ids = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        assert sorted(ids) == list(range(num_blocks))
        self.free: deque = deque(ids)
        self.rc: Dict[int, int] = {b: 0 for b in ids}
        self.key_of_block: Dict[int, int] = {}
        self.block_of_key: Dict[int, int] = {}
        self.waiting: deque = deque()
        self.running: List[Request] = []
        self.finished: List[int] = []
        self.num_host_blocks = num_host_blocks
        self.host_free: deque = deque(range(num_host_blocks))
        self.swapped: deque = deque()

    # -- blocks ----------------------------------------------------------------
    def _allocate(self) -> int:
        b = self.free.popleft()
        assert self.rc[b] == 0
        k = self.key_of_block.pop(b, None)
        if k is not None:
            del self.block_of_key[k]
        self.rc[b] = 1
        return b

    def _release(self, req: Request) -> None:
        for b in req.table:
            self.rc[b] -= 1
            assert self.rc[b] >= 0
            if self.rc[b] == 0:
                self.free.append(b)
        req.table = []
        req.keys = []

    def _lookup(self, req: Request) -> List[int]:
        """Leading full blocks of the request's tokens with a cached key."""
        hits, parent = [], FNV_OFFSET
        for i in range((len(req.tokens) - 1) // self.B):
            k = block_key(parent, req.tokens[i * self.B:(i + 1) * self.B])
            b = self.block_of_key.get(k)
            if b is None:
                break
            hits.append((b, k))
            parent = k
        return hits

    def _register_full_blocks(self, req: Request, upto: int) -> None:
        """Key every full block of positions < upto that has no key yet."""
        while len(req.keys) < upto // self.B:
            i = len(req.keys)
            parent = req.keys[-1] if req.keys else FNV_OFFSET
            k = block_key(parent, req.tokens[i * self.B:(i + 1) * self.B])
            req.keys.append(k)
            b = req.table[i]
            if k not in self.block_of_key and b not in self.key_of_block:
                self.block_of_key[k] = b
                self.key_of_block[b] = k

    def _blocks_needed(self, req: Request, c: int) -> int:
        return -(-(req.num_computed + c) // self.B) - len(req.table)

    def _schedule(self, req: Request, c: int) -> Scheduled:
        for _ in range(self._blocks_needed(req, c)):
            req.table.append(self._allocate())
        start = req.num_computed
        slots = [req.table[p // self.B] * self.B + p % self.B for p in range(start, start + c)]
        req.num_computed += c
        self._register_full_blocks(req, req.num_computed)
        return Scheduled(req.req_id, c, req.num_computed, list(req.table), slots)

    def _preempt(self, req: Request, swap_out: List[tuple]) -> bool:
        """Swap the request out when the swap space holds all its blocks,
        else release them for recomputation.  True when swapped."""
        if self.num_host_blocks and len(self.host_free) >= len(req.table):
            for b in req.table:
                h = self.host_free.popleft()
                swap_out.append((b, h))
                req.host_table.append(h)
            self._release(req)
            self.swapped.append(req)
            return True
        self._release(req)
        req.num_computed = 0
        req.prompt_len = len(req.tokens)
        return False

    def _swap_in(self, req: Request, swap_in: List[tuple]) -> None:
        for h in req.host_table:
            b = self._allocate()
            swap_in.append((h, b))
            req.table.append(b)
            self.host_free.append(h)
        req.host_table = []
        self._register_full_blocks(req, req.num_computed)

    # -- the public steps --------------------------------------------------------
    def add_request(self, req_id: int, prompt: Sequence[int], max_new_tokens: int) -> None:
        assert len(prompt) >= 1 and max_new_tokens >= 1
        self.waiting.append(Request(req_id, [int(t) for t in prompt], len(prompt),
                                    max_new_tokens))

    def step(self) -> Batch:
        entries: List[Scheduled] = []
        preempted: List[int] = []
        swapped_out: List[int] = []
        swap_out: List[tuple] = []
        swap_in: List[tuple] = []
        decodes = [r for r in self.running if r.num_computed >= r.prompt_len]
        prefills = [r for r in self.running if r.num_computed < r.prompt_len]
        still: List[Request] = []

        def preempt(r):
            preempted.append(r.req_id)
            if self._preempt(r, swap_out):
                swapped_out.append(r.req_id)

        # 1. decode streams: one token each, reserved before the budget is split
        for r in decodes:
            if self._blocks_needed(r, 1) > len(self.free):
                preempt(r)
                continue
            entries.append(self._schedule(r, 1))
            still.append(r)
        avail = max(0, self.token_budget - len(entries))
        # 2. running prompts resume their chunks
        for r in prefills:
            c = min(r.pending, self.chunk_tokens, avail)
            if c == 0:
                still.append(r)
                continue
            if self._blocks_needed(r, c) > len(self.free):
                preempt(r)
                continue
            entries.append(self._schedule(r, c))
            avail -= c
            still.append(r)
        # requests preempted for recomputation go back to the front of the
        # queue, in order
        for rid in reversed([x for x in preempted if x not in swapped_out]):
            req = next(x for x in self.running if x.req_id == rid)
            self.waiting.appendleft(req)
        # 3. swapped-out requests come back, in order, when nobody was
        #    preempted in this step
        while self.swapped and avail > 0 and not preempted:
            r = self.swapped[0]
            c = 1 if r.num_computed >= r.prompt_len else min(r.pending, self.chunk_tokens, avail)
            if -(-(r.num_computed + c) // self.B) > len(self.free):
                break
            self.swapped.popleft()
            self._swap_in(r, swap_in)
            entries.append(self._schedule(r, c))
            avail -= c
            still.append(r)
        # 4. admissions in arrival order while budget is left (none after a
        #    preemption, none while a request is swapped out)
        while self.waiting and avail > 0 and not preempted and not self.swapped:
            r = self.waiting[0]
            hits = self._lookup(r)
            n_cached = len(hits) * self.B
            c = min(len(r.tokens) - n_cached, self.chunk_tokens, avail)
            revive = sum(1 for b, _ in hits if self.rc[b] == 0)
            new_blocks = -(-(n_cached + c) // self.B) - len(hits)
            if new_blocks > len(self.free) - revive:
                break
            self.waiting.popleft()
            for b, k in hits:
                if self.rc[b] == 0:
                    self.free.remove(b)
                self.rc[b] += 1
                r.table.append(b)
                r.keys.append(k)
            r.num_computed = n_cached
            entries.append(self._schedule(r, c))
            avail -= c
            still.append(r)
        self.running = still
        return Batch(entries, preempted, swapped_out, swap_out, swap_in)

    def update(self, batch: Batch, sampled: Dict[int, int]) -> None:
        """After the step ran: requests with every token computed either end
        (max_new_tokens generated) or take the caller's sampled token."""
        by_id = {r.req_id: r for r in self.running}
        for e in batch.entries:
            r = by_id[e.req_id]
            if r.num_computed < len(r.tokens):
                continue
            if r.generated >= r.max_new_tokens:
                self._release(r)
                self.running.remove(r)
                self.finished.append(r.req_id)
                continue
            r.tokens.append(int(sampled[r.req_id]))
            r.generated += 1

    def check_invariants(self) -> None:
        refs: Dict[int, int] = {}
        for r in self.running:
            assert len(r.table) == -(-r.num_computed // self.B)
            for b in r.table:
                refs[b] = refs.get(b, 0) + 1
        for b, n in self.rc.items():
            assert n == refs.get(b, 0), (b, n, refs.get(b, 0))
        assert len(set(self.free)) == len(self.free)
        assert all(self.rc[b] == 0 for b in self.free)
        assert len(self.free) + sum(1 for n in self.rc.values() if n > 0) == len(self.rc)
        for k, b in self.block_of_key.items():
            assert self.key_of_block[b] == k
        held = [h for r in self.swapped for h in r.host_table]
        assert len(set(held)) == len(held) and not set(held) & set(self.host_free)
        assert len(held) + len(self.host_free) == self.num_host_blocks
        for r in self.swapped:
            assert not r.table and len(r.host_table) == -(-r.num_computed // self.B)
            assert r not in self.running
