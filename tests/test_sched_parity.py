"""The native batch builder (libpa, ``include/pa_sched.h``) against the
oracle (``oracle/scheduler.py``): identical batches -- request order, query
lengths, sequence lengths, block tables, slots, preemptions -- and identical
block reference counts after every step, on the pages' worked examples and
on seeded random request streams (with shared prefixes and memory pressure).
Host code only: runs without a GPU."""
import json
import os
import random

import numpy as np
import pytest

import oracle.scheduler as sch
from paged_kv_cache_19_amd import binding
from tests.conftest import GOLDEN

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH), reason="libpa.so not built")


def _sample(req_id, pos):
    return (req_id * 7919 + pos * 104729 + 13) % 32000


def _compare_step(ref, nat):
    b = ref.step()
    n = nat.step()
    assert list(n["req_ids"]) == [e.req_id for e in b.entries]
    assert list(n["query_start_loc"]) == b.query_start_loc()
    assert list(n["seq_lens"]) == [e.seq_len for e in b.entries]
    assert list(n["slot_mapping"]) == [x for e in b.entries for x in e.slots]
    for i, e in enumerate(b.entries):
        assert list(n["block_tables"][i, :len(e.table)]) == e.table
    assert list(n["preempted"]) == b.preempted
    assert list(n["swapped_out"]) == b.swapped_out
    assert [tuple(x) for x in n["swap_out"].tolist()] == [tuple(x) for x in b.swap_out]
    assert [tuple(x) for x in n["swap_in"].tolist()] == [tuple(x) for x in b.swap_in]
    sampled = {e.req_id: _sample(e.req_id, e.seq_len) for e in b.entries}
    ref.update(b, sampled)
    nat.update(sampled)
    ref.check_invariants()
    want_rc = np.array([ref.rc[i] for i in range(len(ref.rc))], np.int32)
    assert np.array_equal(nat.block_refcounts(), want_rc)
    return b


def _pair(num_blocks, B, budget, chunk, free_order=None, host_blocks=0):
    return (sch.Scheduler(num_blocks, B, budget, chunk, free_order, num_host_blocks=host_blocks),
            binding.BatchBuilder(num_blocks, B, budget, chunk, free_order,
                                 num_host_blocks=host_blocks))


def test_chunk_formula_example_native():
    with open(os.path.join(GOLDEN, "chunked_prefill_schedule.json")) as f:
        g = json.load(f)
    ref, nat = _pair(4096, 16, g["token_budget"], g["chunk_tokens"])
    for i in range(g["decode_streams"]):
        ref.add_request(i, [i + 1], 1000)
        nat.add_request(i, [i + 1], 1000)
    _compare_step(ref, nat)
    prompt = list(range(g["prompt_tokens"]))
    ref.add_request(999, prompt, 4)
    nat.add_request(999, prompt, 4)
    chunks = 0
    for _ in range(g["num_chunks"] + 2):
        b = _compare_step(ref, nat)
        chunks += sum(1 for e in b.entries if e.req_id == 999 and e.q_len > 1)
    assert chunks == g["num_chunks"]


def test_walkthrough_native():
    with open(os.path.join(GOLDEN, "walkthrough.json")) as f:
        g = json.load(f)
    ref, nat = _pair(16, 4, 64, 64)
    shared = [101, 102, 103, 104, 105, 106]
    for s in (ref, nat):
        s.add_request(0, shared + [7], 100)
    for step in range(6):
        if step == 1:
            ref.add_request(1, shared, 100)
            nat.add_request(1, shared, 100)
        _compare_step(ref, nat)
    rc = nat.block_refcounts()
    for entry in g["pool"]:
        assert rc[entry["block"]] == entry["refcount"]


@pytest.mark.parametrize("seed,num_blocks,max_new", [(s, 48, 10) for s in range(4)] +
                         [(s, 14, 40) for s in range(4)] + [(s, 200, 30) for s in range(2)])
def test_random_streams_match(seed, num_blocks, max_new):
    rng = random.Random(seed)
    B = 4
    order = rng.sample(range(num_blocks), num_blocks)
    ref, nat = _pair(num_blocks, B, 24, 8, order)
    prefixes = [[rng.randrange(50) for _ in range(rng.randrange(1, 14))] for _ in range(3)]
    nid = 0
    preempted = 0
    for _ in range(80):
        for _ in range(rng.randrange(0, 3)):
            pre = rng.choice(prefixes) if rng.random() < 0.6 else []
            prompt = pre + [rng.randrange(50) for _ in range(rng.randrange(1, 12))]
            mn = rng.randrange(1, max_new)
            ref.add_request(nid, prompt, mn)
            nat.add_request(nid, prompt, mn)
            nid += 1
        preempted += len(_compare_step(ref, nat).preempted)
    w, r, f = nat.counts()
    assert (w, r, f) == (len(ref.waiting), len(ref.running), len(ref.finished))


def _admit_pair(ref, nat, req_id, prompt):
    """Admit one request on both builders and run its prefill to the end;
    returns the oracle's first entry and the request's table."""
    ref.add_request(req_id, prompt, 1)
    nat.add_request(req_id, prompt, 1)
    first = None
    while True:
        b = _compare_step(ref, nat)
        e = next(e for e in b.entries if e.req_id == req_id)
        first = first or e
        r = next(r for r in ref.running if r.req_id == req_id)
        if r.num_computed >= r.prompt_len:
            return first, list(r.table)


def test_prefix_key_chain_native():
    """Equal blocks after different first blocks are not shared, on both
    builders (the oracle's pin of the chained key, replayed natively)."""
    from tests.test_oracle_scheduler import X, Y, Z, check_prefix_key_chain
    ref, nat = _pair(32, 4, 64, 64)
    res = [_admit_pair(ref, nat, i, p)
           for i, p in enumerate([X + Y + [13], Z + Y + [14], Z + Y + [15], X + Y + [16]])]
    check_prefix_key_chain(res)


def test_fully_cached_prompt_native():
    from tests.test_oracle_scheduler import X, Y, check_full_prompt
    ref, nat = _pair(32, 4, 64, 64)
    _, a = _admit_pair(ref, nat, 0, X + Y)
    b_entry, b = _admit_pair(ref, nat, 1, X + Y)
    check_full_prompt(a, b_entry, b)


@pytest.mark.parametrize("seed,num_blocks", [(s, 48) for s in range(3)] + [(s, 14) for s in range(3)])
def test_repeated_block_streams_match(seed, num_blocks):
    """Prompts built from a few whole blocks: the same block after different
    earlier blocks is common, so a key that ignored its parent would show."""
    from tests.test_oracle_scheduler import block_prompt
    rng = random.Random(100 + seed)
    B = 4
    ref, nat = _pair(num_blocks, B, 24, 8, rng.sample(range(num_blocks), num_blocks))
    vocab_blocks = [[rng.randrange(50) for _ in range(B)] for _ in range(3)]
    nid = 0
    for _ in range(80):
        for _ in range(rng.randrange(0, 3)):
            prompt = block_prompt(rng, vocab_blocks, B)
            mn = rng.randrange(1, 30)
            ref.add_request(nid, prompt, mn)
            nat.add_request(nid, prompt, mn)
            nid += 1
        _compare_step(ref, nat)


def test_swap_walkthrough_native():
    ref, nat = _pair(4, 4, 64, 64, host_blocks=2)
    for s in (ref, nat):
        s.add_request(0, list(range(1, 9)), 3)
        s.add_request(1, [11, 12, 13, 14], 8)
    swaps = []
    for _ in range(8):
        b = _compare_step(ref, nat)
        swaps.append((b.swap_out, b.swap_in))
    assert swaps[1] == ([(2, 0)], []) and swaps[4] == ([], [(0, 2)])


@pytest.mark.parametrize("seed,num_blocks,host_blocks", [(s, 14, 24) for s in range(4)] +
                         [(s, 10, 6) for s in range(2)] + [(s, 20, 64) for s in range(2)])
def test_random_streams_with_swapping_match(seed, num_blocks, host_blocks):
    """Memory pressure with a swap space (large enough, or too small for some
    requests so that recomputation stays the fallback)."""
    rng = random.Random(300 + seed)
    B = 4
    order = rng.sample(range(num_blocks), num_blocks)
    ref, nat = _pair(num_blocks, B, 24, 8, order, host_blocks)
    prefixes = [[rng.randrange(50) for _ in range(rng.randrange(1, 14))] for _ in range(3)]
    nid = swaps = 0
    for _ in range(80):
        for _ in range(rng.randrange(0, 3)):
            pre = rng.choice(prefixes) if rng.random() < 0.6 else []
            prompt = pre + [rng.randrange(50) for _ in range(rng.randrange(1, 12))]
            mn = rng.randrange(1, 40)
            ref.add_request(nid, prompt, mn)
            nat.add_request(nid, prompt, mn)
            nid += 1
        swaps += len(_compare_step(ref, nat).swapped_out)
    assert swaps > 0


def test_native_argument_errors():
    lib = binding.lib()
    assert not lib.pa_sched_create(0, 16, 64, 64, None)
    bad_order = np.array([0, 0, 1], np.int32)
    assert not lib.pa_sched_create(3, 16, 64, 64, bad_order.ctypes.data_as(binding.ctypes.c_void_p))
    b = binding.BatchBuilder(8, 4, 16, 16)
    with pytest.raises(binding.PAError):
        b.add_request(1, [], 3)
    b.add_request(1, [5, 6], 3)
    with pytest.raises(binding.PAError) as e:
        b.add_request(1, [7], 3)                      # id in use
    assert e.value.status == -6
    out = b.step()
    with pytest.raises(binding.PAError) as e:
        b.update({})                                  # request 1 needs its sampled token
    assert e.value.status == -6
    b.update({1: 9})
    assert list(out["seq_lens"]) == [2]
    assert lib.pa_sched_enable_swap(b._h, 4) == -6        # requests already queued
    fresh = binding.BatchBuilder(8, 4, 16, 16)
    assert lib.pa_sched_enable_swap(fresh._h, -1) == -2
    assert lib.pa_sched_enable_swap(fresh._h, 4) == 0
    assert lib.pa_sched_enable_swap(fresh._h, 4) == -6    # once
