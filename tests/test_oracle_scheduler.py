"""Pins of the host batch builder oracle (``oracle/scheduler.py``).

* The chunked-prefill numbers of "Tech Radar: vLLM v1 ...", section "3.
  Dynamic Chunked Prefill" (``tests/golden/chunked_prefill_schedule.json``):
  64 decode streams, a 32K prompt, budget 2048, 1024-token chunks -> chunk 1
  is tokens 0..1023 and the prompt takes 32 chunks; C_avail = 1984.
* The block-table walkthrough of "03 -- PagedAttention & the vLLM V1
  Architecture" reached through prefix reuse instead of fork: the end state
  (tables [0, 1, 3] / [0, 2, 4], block 0 shared with reference count 2) is
  the page's.
* FNV-1a 64-bit against its published test vectors.
* A fuzz run that writes, through the emitted slots, what a slot's K/V
  depends on -- the token and every token before it in its sequence -- into
  a simulated pool: every scheduled sequence reads back exactly its own
  prefixes through its table (prefix hits included), budgets hold,
  invariants hold.  One stream draws prompts from a few whole blocks, so
  that equal blocks after different earlier blocks are common.
* Prefix reuse keys a block by everything before it ("Tech Radar ...",
  section "Prefix Caching: Radix Tree vs. Hash-Based Indexing": a tree node
  is reached only through its ancestors): a block whose tokens match a
  cached block that follows different earlier blocks is not reused.  A
  prompt whose every block is cached still computes its last token (its
  logits are needed), in a block of its own.
* Preemption by swapping ("03 -- ...", section "Preemption & eviction";
  "Inside vLLM ...", section "Preemption Mechanics: Swapping vs.
  Recomputation"): the swap-out and swap-in copies a step reports, applied to
  the simulated pool and a simulated swap space, keep every token readable
  through the tables, and a request swapped back in resumes where it
  stopped; a small walkthrough pins the exact copies.
Planted mistakes (budget not reduced by decode rows, a hit on a partial
block, a wrong slot offset, a key without its parent, a hit on the block
holding the last token, swap-in pairs reversed, swap-outs not reported, a
swapped-in request recomputed) fail.
"""
import json
import os
import random

import pytest

import oracle.scheduler as sch
from tests.conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_fnv1a64_published_vectors():
    assert sch.fnv1a64(b"") == 0xCBF29CE484222325
    assert sch.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert sch.fnv1a64(b"foobar") == 0x85944171F73967E8


def _sample(req_id, pos):
    return (req_id * 7919 + pos * 104729 + 13) % 32000


def apply_swaps(batch, pool, host, B):
    """The copies a step asks for, in the stated order: swap-outs (device
    block -> host block), then swap-ins (host block -> device block)."""
    for b, h in batch.swap_out:
        for o in range(B):
            host[(h, o)] = pool.get(b * B + o)
    for h, b in batch.swap_in:
        for o in range(B):
            pool[b * B + o] = host.get((h, o))


def run(s, steps, pool=None, B=None, check=True, host=None):
    """Drive ``steps`` steps; with ``pool`` (dict slot -> the tokens its K/V
    was computed from), write through the slots and check reads through
    tables; ``host`` is the swap space's content."""
    out = []
    for _ in range(steps):
        batch = s.step()
        out.append(batch)
        if pool is not None and host is not None:
            apply_swaps(batch, pool, host, B)
        by_id = {r.req_id: r for r in s.running}
        for e in batch.entries:
            r = by_id[e.req_id]
            first = e.seq_len - e.q_len
            if pool is not None:
                # a slot's K/V is a function of its token and all earlier ones
                for j, slot in enumerate(e.slots):
                    pool[slot] = tuple(r.tokens[:first + j + 1])
                for p in range(e.seq_len):
                    blk = e.table[p // B]
                    assert pool.get(blk * B + p % B) == tuple(r.tokens[:p + 1]), (e.req_id, p)
        sampled = {e.req_id: _sample(e.req_id, e.seq_len) for e in batch.entries}
        s.update(batch, sampled)
        if check:
            s.check_invariants()
    return out


def test_chunk_formula_worked_example():
    g = _load("chunked_prefill_schedule.json")
    n_dec, budget, chunk = g["decode_streams"], g["token_budget"], g["chunk_tokens"]
    s = sch.Scheduler(num_blocks=4096, block_size=16, token_budget=budget, chunk_tokens=chunk)
    for i in range(n_dec):
        s.add_request(i, [i + 1], max_new_tokens=1000)
    run(s, 1)                                         # the 64 one-token prompts
    s.add_request(999, list(range(g["prompt_tokens"])), max_new_tokens=4)
    chunks = []
    for _ in range(g["num_chunks"] + 2):
        batch = run(s, 1)[0]
        dec = [e for e in batch.entries if e.q_len == 1 and e.req_id != 999]
        assert len(dec) == n_dec                       # every decode stream served first
        pre = [e for e in batch.entries if e.req_id == 999]
        if pre and pre[0].q_len > 1:
            chunks.append((pre[0].seq_len - pre[0].q_len, pre[0].seq_len - 1))
            assert sum(e.q_len for e in batch.entries) <= budget
    assert chunks[0] == tuple(g["first_chunk"])
    assert len(chunks) == g["num_chunks"]
    assert chunks[-1][1] == g["prompt_tokens"] - 1
    # equation 3 with C_chunk above C_avail: the chunk is C_avail
    s2 = sch.Scheduler(4096, 16, budget, 2048)
    for i in range(n_dec):
        s2.add_request(i, [i + 1], max_new_tokens=1000)
    run(s2, 1)
    s2.add_request(999, list(range(g["prompt_tokens"])), max_new_tokens=4)
    e = [e for e in run(s2, 1)[0].entries if e.req_id == 999][0]
    assert e.q_len == g["c_avail"]


def test_walkthrough_reached_by_prefix_reuse():
    g = _load("walkthrough.json")
    B = g["block_size"]
    s = sch.Scheduler(num_blocks=16, block_size=B, token_budget=64, chunk_tokens=64)
    shared = [101, 102, 103, 104, 105, 106]            # the six tokens both agree on
    a_tokens = shared + [7]                            # A's prompt reaches position 6 ("and")
    s.add_request(0, a_tokens, max_new_tokens=100)
    sampled_a = iter([8, 9, 10, 11, 12])
    sampled_b = iter([70, 71, 72, 73])                 # B diverges at position 6 ("but")
    pool = {}
    for step in range(6):
        if step == 1:
            s.add_request(1, shared, max_new_tokens=100)
        batch = s.step()
        by_id = {r.req_id: r for r in s.running}
        for e in batch.entries:
            r = by_id[e.req_id]
            for j, slot in enumerate(e.slots):
                pool[slot] = r.tokens[e.seq_len - e.q_len + j]
        s.update(batch, {0: next(sampled_a, 0), 1: next(sampled_b, 0)})
        s.check_invariants()
    A, Bq = (next(r for r in s.running if r.req_id == i) for i in (0, 1))
    assert A.table == g["block_tables"]["A"] and Bq.table == g["block_tables"]["B"]
    assert A.num_computed == g["seq_lens"]["A"] and Bq.num_computed == g["seq_lens"]["B"]
    for entry in g["pool"]:
        assert s.rc[entry["block"]] == entry["refcount"]
    # block 0 holds the shared tokens once; B's own block 2 holds positions 4..7
    assert [pool[p] for p in range(4)] == shared[:4]
    assert [pool[2 * B + o] for o in range(4)] == Bq.tokens[4:8]


def block_prompt(rng, vocab_blocks, B):
    """A prompt of 1-4 whole blocks drawn from ``vocab_blocks`` plus 0-B
    loose tokens: the same block often follows different earlier blocks."""
    prompt = []
    for _ in range(rng.randrange(1, 5)):
        prompt += rng.choice(vocab_blocks)
    return prompt + [rng.randrange(50) for _ in range(rng.randrange(0, B + 1))]


def _fuzz(seed, steps=60, num_blocks=48, max_new=10, block_vocab=False, host_blocks=0):
    rng = random.Random(seed)
    B = 4
    s = sch.Scheduler(num_blocks=num_blocks, block_size=B, token_budget=24, chunk_tokens=8,
                      free_order=rng.sample(range(num_blocks), num_blocks),
                      num_host_blocks=host_blocks)
    prefixes = [[rng.randrange(50) for _ in range(rng.randrange(1, 14))] for _ in range(3)]
    vocab_blocks = [[rng.randrange(50) for _ in range(B)] for _ in range(3)]
    pool, host = {}, {}
    s.swap_ins = s.swap_outs = 0
    at_swap_out = {}   # request -> tokens computed when it was swapped out
    nid = 0
    for _ in range(steps):
        for _ in range(rng.randrange(0, 3)):
            if block_vocab:
                prompt = block_prompt(rng, vocab_blocks, B)
            else:
                pre = rng.choice(prefixes) if rng.random() < 0.6 else []
                prompt = pre + [rng.randrange(50) for _ in range(rng.randrange(1, 12))]
            s.add_request(nid, prompt, max_new_tokens=rng.randrange(1, max_new))
            nid += 1
        batch = run(s, 1, pool, B, host=host)[0]
        s.preemptions = getattr(s, "preemptions", 0) + len(batch.preempted)
        s.swap_outs += len(batch.swapped_out)
        s.swap_ins += len(batch.swap_in) > 0
        for r in s.swapped:
            at_swap_out.setdefault(r.req_id, r.num_computed)
        for e in batch.entries:      # a swapped-in request resumes, not recomputes
            if e.req_id in at_swap_out and e.req_id not in [r.req_id for r in s.swapped]:
                assert e.seq_len - e.q_len == at_swap_out.pop(e.req_id), e.req_id
        n_dec = sum(1 for e in batch.entries if e.q_len == 1)
        assert sum(e.q_len for e in batch.entries if e.q_len > 1) <= max(0, 24 - n_dec) + 0
    return s


@pytest.mark.parametrize("seed", range(6))
def test_fuzz_tokens_read_back_through_tables(seed):
    _fuzz(seed)


@pytest.mark.parametrize("seed", range(6))
def test_fuzz_repeated_blocks_read_back_their_prefixes(seed):
    _fuzz(seed, block_vocab=True)


X, Y, Z = [1, 2, 3, 4], [5, 6, 7, 8], [9, 10, 11, 12]


def _admit_alone(s, req_id, prompt):
    """Admit one request and run its prefill to the end (one step each)."""
    s.add_request(req_id, prompt, max_new_tokens=1)
    first = None
    while True:
        batch = s.step()
        e = next(e for e in batch.entries if e.req_id == req_id)
        first = first or e
        r = next(r for r in s.running if r.req_id == req_id)
        s.update(batch, {x.req_id: 0 for x in batch.entries})
        s.check_invariants()
        if r.num_computed >= r.prompt_len:
            return first, list(r.table)


def prefix_key_chain_case(s):
    """Three prompts share block Y after different first blocks (X, then Z,
    then Z again).  Returns the tables and first entries."""
    a_entry, a = _admit_alone(s, 0, X + Y + [13])
    c_entry, c = _admit_alone(s, 1, Z + Y + [14])
    d_entry, d = _admit_alone(s, 2, Z + Y + [15])
    e_entry, e = _admit_alone(s, 3, X + Y + [16])
    return (a_entry, a), (c_entry, c), (d_entry, d), (e_entry, e)


def check_prefix_key_chain(results, B=4):
    (a_entry, a), (c_entry, c), (d_entry, d), (e_entry, e) = results
    # Z + Y: block Y follows Z, not X -- no hit at all, every token computed
    assert c_entry.q_len == 2 * B + 1 and c[1] != a[1]
    # Z + Y again: both blocks are the ones computed after Z
    assert d_entry.q_len == 1 and d[:2] == c[:2] and d[1] != a[1]
    # X + Y again: the blocks computed after X
    assert e_entry.q_len == 1 and e[:2] == a[:2]


def test_prefix_key_names_the_whole_prefix():
    s = sch.Scheduler(num_blocks=32, block_size=4, token_budget=64, chunk_tokens=64)
    check_prefix_key_chain(prefix_key_chain_case(s))


def full_prompt_case(s):
    """A prompt of exactly two blocks, cached, then asked for again."""
    _, a = _admit_alone(s, 0, X + Y)
    b_entry, b = _admit_alone(s, 1, X + Y)
    return a, b_entry, b


def check_full_prompt(a, b_entry, b, B=4):
    # the block holding the last token is computed again, in a block of its own
    assert b_entry.q_len == B and b_entry.seq_len == 2 * B
    assert b[0] == a[0] and b[1] != a[1]


def test_fully_cached_prompt_computes_its_last_token():
    s = sch.Scheduler(num_blocks=32, block_size=4, token_budget=64, chunk_tokens=64)
    check_full_prompt(*full_prompt_case(s))


@pytest.mark.parametrize("seed", range(6))
def test_fuzz_swapping_restores_every_token(seed):
    """Memory pressure with a swap space: preempted requests are swapped out
    and back, every token still reads back through the tables after the
    copies the steps asked for, and resumed requests are not recomputed."""
    s = _fuzz(seed, steps=80, num_blocks=14, max_new=40, host_blocks=24)
    assert s.swap_outs > 0 and s.swap_ins > 0


def test_swap_walkthrough():
    """Four device blocks of 4 tokens, a swap space of 2: B is swapped out
    when A takes the last block, and swapped back into fresh blocks once A
    has finished; B resumes at token 5 (the exact copies follow from the FIFO
    free lists)."""
    s = sch.Scheduler(num_blocks=4, block_size=4, token_budget=64, chunk_tokens=64,
                      num_host_blocks=2)
    s.add_request(0, list(range(1, 9)), max_new_tokens=3)    # A: 8 tokens, blocks 0, 1
    s.add_request(1, [11, 12, 13, 14], max_new_tokens=8)     # B: 4 tokens, block 2
    pool, host = {}, {}
    batches = run(s, 5, pool, 4, host=host)
    b1, b2, b3, b4, b5 = batches
    assert [e.table for e in b1.entries] == [[0, 1], [2]]
    assert b2.preempted == [1] and b2.swapped_out == [1] and b2.swap_out == [(2, 0)]
    assert [e.table for e in b2.entries] == [[0, 1, 3]]
    assert not b3.swap_in and not b4.swap_in          # A still holds three blocks
    assert b5.swap_in == [(0, 2)]
    (e,) = b5.entries
    assert (e.req_id, e.q_len, e.seq_len, e.table) == (1, 1, 5, [2, 0])
    assert e.slots == [0]


def test_fuzz_under_memory_pressure_preempts_and_recovers():
    n = 0
    for seed in range(6):
        s = _fuzz(seed, steps=80, num_blocks=14, max_new=40)
        n += s.preemptions
    assert n > 0


def test_fuzz_exercises_hits_and_preemption():
    hits = preempts = 0
    orig = sch.Scheduler._lookup

    def counting(self, req):
        nonlocal hits
        h = orig(self, req)
        hits += len(h)
        return h
    sch.Scheduler._lookup = counting
    try:
        for seed in range(6):
            s = _fuzz(seed)
    finally:
        sch.Scheduler._lookup = orig
    assert hits > 0


def _bad_budget(self):
    self.token_budget += 64          # decode rows not taken out of the budget
    try:
        return _orig_step(self)
    finally:
        self.token_budget -= 64


def _bad_lookup(self, req):
    hits = _orig_lookup(self, req)
    if hits:
        return hits
    # a hit on the first block even when only part of it matches
    parent = sch.FNV_OFFSET
    for k, b in self.block_of_key.items():
        return [(b, k)] if len(req.tokens) > self.B else []
    return []


def _bad_slots(self, req, c):
    e = _orig_schedule(self, req, c)
    e.slots = [x + 1 if i == 0 else x for i, x in enumerate(e.slots)]
    return e


def _lookup_uncapped(self, req):
    """Hits may cover the block holding the prompt's last token."""
    hits, parent = [], sch.FNV_OFFSET
    for i in range(len(req.tokens) // self.B):
        k = sch.block_key(parent, req.tokens[i * self.B:(i + 1) * self.B])
        b = self.block_of_key.get(k)
        if b is None:
            break
        hits.append((b, k))
        parent = k
    return hits


def _flat_key(parent, tokens):
    """A block keyed by its own tokens only (parent dropped)."""
    return _orig_block_key(sch.FNV_OFFSET, tokens)


_orig_step = sch.Scheduler.step
_orig_lookup = sch.Scheduler._lookup
_orig_schedule = sch.Scheduler._schedule
_orig_block_key = sch.block_key


def _all_pins():
    test_chunk_formula_worked_example()
    for seed in range(6):
        _fuzz(seed)
        _fuzz(seed, block_vocab=True)
    test_prefix_key_names_the_whole_prefix()
    test_fully_cached_prompt_computes_its_last_token()


def _swap_in_reversed(self, req, swap_in):
    n = len(swap_in)
    _orig_swap_in(self, req, swap_in)
    swap_in[n:] = [(b, h) for h, b in swap_in[n:]]


def _swap_out_not_reported(self, req, swap_out):
    out = _orig_preempt(self, req, [])
    return out


def _swapped_request_recomputed(self, req, swap_in):
    _orig_swap_in(self, req, swap_in)
    req.num_computed = 0


_orig_swap_in = sch.Scheduler._swap_in
_orig_preempt = sch.Scheduler._preempt


@pytest.mark.parametrize("name,bad", [("_swap_in", _swap_in_reversed),
                                      ("_preempt", _swap_out_not_reported),
                                      ("_swap_in", _swapped_request_recomputed)])
def test_planted_swap_mistake_fails(monkeypatch, name, bad):
    monkeypatch.setattr(sch.Scheduler, name, bad)
    with pytest.raises((AssertionError, KeyError, IndexError, StopIteration)):
        test_swap_walkthrough()
        for seed in range(6):
            _fuzz(seed, steps=80, num_blocks=14, max_new=40, host_blocks=24)


@pytest.mark.parametrize("name,bad", [("step", _bad_budget), ("_lookup", _bad_lookup),
                                      ("_schedule", _bad_slots),
                                      ("_lookup", _lookup_uncapped)])
def test_planted_scheduler_mistake_fails(monkeypatch, name, bad):
    monkeypatch.setattr(sch.Scheduler, name, bad)
    with pytest.raises((AssertionError, KeyError, IndexError, StopIteration)):
        _all_pins()


def test_planted_flat_block_key_fails(monkeypatch):
    monkeypatch.setattr(sch, "block_key", _flat_key)
    with pytest.raises(AssertionError):
        test_prefix_key_names_the_whole_prefix()
    with pytest.raises(AssertionError):
        for seed in range(6):
            _fuzz(seed, block_vocab=True)


def test_pins_pass_unmutated():
    _all_pins()
