"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Slot mapping and the cache write must match bit for bit; attention outputs
must match within 1e-4 (fp32) / 2e-2 (bf16) max-abs error on every row of
every sequence, full-size workloads included.  Every slot that does not hold a cached position (block tails, spare
blocks, this step's slots before the write) is NaN-poisoned first, and table
padding points at a poisoned spare block: a finite output proves none of it
was read.
"""
import math

import pytest
import torch

from paged_kv_cache_19_amd import binding, workloads
from tests.gpu_common import TOL, log, run_and_compare

pytestmark = pytest.mark.gpu

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6, 7])
def test_workload_parity(cfg):
    log(f"[parity] workload {cfg}: {workloads.SHAPES[cfg].name}")
    wl = workloads.make_workload(cfg, device="cuda")
    out, err = run_and_compare(wl)
    log(f"[parity] workload {cfg}: max abs err {err:.3e}")
    assert err <= TOL[wl.shape.dtype]
    del wl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg,tp", [(3, 8), (5, 8), (2, 2)], ids=["70b-tp8", "mix-tp8", "8b-tp2"])
def test_tensor_parallel_rank_shape(cfg, tp):
    """One tensor-parallel rank's share of a workload (bench.py --tp): the
    same sequences with H_q / tp query and H_kv / tp KV heads (at tp = 8 a
    single KV head); every row."""
    base = workloads.SHAPES[cfg]
    shape = workloads.Shape(base.name + f"-tp{tp}", base.dtype, base.num_q_heads // tp,
                            base.num_kv_heads // tp, base.head_dim, base.block_size)
    log(f"[tp rank] workload {cfg} at tp={tp}: H_q={shape.num_q_heads} H_kv={shape.num_kv_heads}")
    wl = workloads.make_workload(cfg, device="cuda", shape=shape)
    out, err = run_and_compare(wl)
    log(f"[tp rank] max abs err {err:.3e}")
    assert err <= TOL[wl.shape.dtype]
    del wl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("split", [64, 128, 512, 1024])
def test_split_counts_agree(split):
    wl = workloads.make_workload(2, device="cuda", seq_lens=[1, 63, 64, 65, 700, 2048, 4000, 4096],
                                 q_lens=[1] * 8)
    log(f"[split] kv_split_tokens={split}")
    out, err = run_and_compare(wl, kv_split_tokens=split)
    assert err <= TOL[wl.shape.dtype]


@pytest.mark.parametrize("split", [64, 256, 1024])
def test_chunk_ranges_agree(split):
    """Fixed ranges of `split` keys cut every row tile into many pieces; the
    merged rows must agree with the oracle like the balanced default."""
    shape = workloads.Shape("chunks", "bf16", 32, 8, 128, 16)
    wl = workloads.make_workload(2, seed=91, device="cuda", seq_lens=[2100, 700, 5, 1300],
                                 q_lens=[600, 700, 1, 64], shape=shape)
    log(f"[chunk ranges] kv_split_tokens={split}")
    out, err = run_and_compare(wl, kv_split_tokens=split, force_chunked=True)
    log(f"[chunk ranges] max abs err {err:.3e}")
    assert err <= TOL["bf16"]


def test_merge_finds_sequences_among_thousands():
    """The merge finds each row's sequence by a 64-way search over the query
    offsets: with 5,000 sequences it takes three rounds (beyond 4,096), and
    fixed 64-key splits send every row through it (fp32, vector-ALU path)."""
    import random
    rng = random.Random(95)
    n = 5000
    lens = [rng.randint(65, 200) for _ in range(n)]
    qls = [rng.choice([1, 1, 1, 2, 3]) for _ in range(n)]
    shape = workloads.Shape("many-seqs", "f32", 8, 2, 64, 4)
    wl = workloads.make_workload(2, seed=95, device="cuda", seq_lens=lens, q_lens=qls, shape=shape)
    log(f"[merge search] {n} sequences, {sum(qls)} query rows")
    out, err = run_and_compare(wl, kv_split_tokens=64, force_chunked=True)
    log(f"[merge search] max abs err {err:.3e}")
    assert err <= TOL["f32"]


def test_chunks_beyond_one_launch():
    """More sequences than the fused chunk + decode launch takes (1,024): the
    chunk units and the decode rows then run as two launches."""
    shape = workloads.Shape("many", "bf16", 32, 8, 128, 16)
    n_chunk, n_dec = 12, 1088
    lens = [300 + 25 * i for i in range(n_chunk)] + [20 + (7 * i) % 100 for i in range(n_dec)]
    qls = [40 + 5 * i for i in range(n_chunk)] + [1] * n_dec
    wl = workloads.make_workload(2, seed=93, device="cuda", seq_lens=lens, q_lens=qls, shape=shape)
    log(f"[many] {len(lens)} sequences, {n_chunk} chunks")
    out, err = run_and_compare(wl, force_chunked=True)
    log(f"[many] max abs err {err:.3e}")
    assert err <= TOL["bf16"]


EDGE = [
    # dtype, Hq, Hkv, D, B, seq_lens, q_lens
    ("bf16", 32, 8, 128, 16, [1, 2, 15, 16, 17, 31, 32, 33], None),
    ("bf16", 16, 16, 128, 16, [100, 37], None),                  # G = 1
    ("bf16", 16, 1, 128, 16, [300, 5], None),                    # G = 16
    ("bf16", 8, 2, 64, 16, [129, 64, 1], None),                  # head_dim 64
    ("bf16", 8, 2, 128, 8, [77, 8, 9], None),                    # B = 8
    ("bf16", 8, 2, 128, 32, [77, 32, 33, 1000], None),           # B = 32
    ("bf16", 8, 2, 128, 64, [3000, 64, 65], None),               # B = 64
    ("bf16", 8, 2, 128, 4, [77, 5, 4], None),                    # B = 4: vector-ALU path
    ("bf16", 8, 2, 64, 1, [9, 1], None),                         # B = 1
    ("f32", 8, 2, 128, 16, [100, 1, 530], None),                 # fp32 with B = 16
    ("f32", 8, 4, 64, 2, [7, 40], None),
    ("bf16", 32, 8, 128, 16, [600, 17, 9], [600, 5, 1]),         # pure prefill + chunk + decode
    ("bf16", 8, 2, 128, 16, [40, 2000, 1], [33, 130, 1]),        # ragged chunks
    ("bf16", 16, 1, 64, 32, [300, 260], [100, 3]),               # G = 16 chunks
    ("f32", 8, 2, 64, 4, [50, 12, 64], [20, 12, 1]),             # fp32 chunks
    ("bf16", 8, 2, 128, 4, [50, 12], [20, 1]),                   # bf16 chunks, B = 4
    ("bf16", 8, 1, 128, 16, [1] * 300, None),                    # many one-token sequences
    ("bf16", 64, 8, 128, 16, [32768], None),                     # one long context, many pieces
    ("bf16", 32, 8, 128, 16, [5, 9000, 3, 1, 17000], None),      # ragged mix
    ("bf16", 32, 8, 64, 32, [4000, 70, 2500], None),             # head_dim 64, B = 32
    ("bf16", 8, 2, 128, 8, [300, 90], [150, 2]),                 # chunks, B = 8
    ("bf16", 8, 2, 128, 64, [700, 130], [300, 64]),              # chunks, B = 64
    ("bf16", 8, 2, 128, 32, [700, 130, 9], [300, 32, 1]),        # chunks, B = 32
    ("bf16", 8, 2, 64, 16, [500, 33], [257, 33]),                # chunks, head_dim 64, B = 16
    ("bf16", 32, 8, 128, 16, [3000, 2500, 7], [1000, 700, 1]),   # long chunks, many row tiles
    ("bf16", 8, 2, 64, 8, [300, 90], [150, 2]),                  # chunks, head_dim 64, B = 8
    ("bf16", 8, 2, 64, 64, [700, 130], [300, 64]),               # chunks, head_dim 64, B = 64
]


@pytest.mark.parametrize("qscale", [4.0, 16.0])
def test_chunk_rows_rescale_on_large_logits(qscale):
    """Queries scaled up (by a power of two, exact in bf16) spread the scores
    so that a row's maximum keeps rising over its keys: the chunk kernel's
    rescale of o and l (taken when a step's probabilities grow past 2^8)
    runs many times per row and must still match the oracle."""
    shape = workloads.Shape("big-logits", workloads.BF16, 8, 2, 128, 16)
    wl = workloads.make_workload(2, seed=97, device="cuda", seq_lens=[3000, 1200, 700, 90],
                                 q_lens=[400, 300, 1, 90], shape=shape)
    wl.tensors["query"].mul_(qscale)
    log(f"[rescale] query x {qscale}")
    out, err = run_and_compare(wl, force_chunked=True)
    log(f"[rescale] max abs err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("case", EDGE, ids=[f"edge{i}" for i in range(len(EDGE))])
def test_edge_shapes(case):
    dtype, Hq, Hkv, D, B, lens, qls = case
    shape = workloads.Shape("edge", dtype, Hq, Hkv, D, B)
    wl = workloads.make_workload(2, seed=77, device="cuda", seq_lens=lens, q_lens=qls, shape=shape)
    log(f"[edge] {case}")
    out, err = run_and_compare(wl, force_chunked=qls is not None)
    log(f"[edge] max abs err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("cfg", [1, 4])
def test_refcount_hint_changes_nothing(cfg):
    """The reference counts steer only the cache policy: outputs with and
    without them are bit-identical."""
    wl = workloads.make_workload(cfg, device="cuda")
    t = wl.tensors
    bt = wl.block_tables_tensor("cuda")
    lens = wl.seq_lens_tensor("cuda")
    rc = wl.block_refcounts_tensor("cuda")
    if cfg == 4:
        assert int(rc.max()) == wl.num_seqs
    a = binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, lens, wl.max_seq_len, wl.scale)
    b = binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, lens, wl.max_seq_len, wl.scale,
                       block_refcounts=rc)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int32),
                       b.view(torch.int16) if b.element_size() == 2 else b.view(torch.int32))


def test_workspace_reuse():
    """Consecutive calls on one workspace match calls on fresh workspaces bit
    for bit (nothing in the workspace carries over between calls)."""
    wl = workloads.make_workload(3, device="cuda", seq_lens=[8000, 3000, 20000, 77, 4096],
                                 q_lens=[1] * 5)
    t = wl.tensors
    bt = wl.block_tables_tensor("cuda")
    S, Hq, D = t["query"].shape
    B = wl.shape.block_size
    ws = torch.full((binding.decode_workspace_bytes(S, Hq, D, 20000, B),), 0x7F, dtype=torch.uint8,
                    device="cuda")
    for lens in ([8000, 3000, 20000, 77, 4096], [100, 3000, 19000, 77, 1], [8000, 3000, 20000, 77, 4096]):
        lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
        got = binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, lt, 20000, wl.scale,
                             workspace=ws)
        ref = binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, lt, 20000, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_decode_through_chunked_entry_point():
    """q_len = 1 rows give the same result through pa_chunked_prefill."""
    wl = workloads.make_workload(2, device="cuda", seq_lens=[300, 1, 4096, 17], q_lens=[1] * 4)
    out, err = run_and_compare(wl, force_chunked=True)
    assert err <= 2e-2


def test_block_relabelling_gives_bit_identical_output():
    wl = workloads.make_workload(2, device="cuda", seq_lens=[513, 2048, 33, 4000, 1000, 16],
                                 q_lens=[1] * 6)
    t = wl.tensors
    bt = wl.block_tables_tensor("cuda")
    lens = wl.seq_lens_tensor("cuda")
    out1 = binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, lens, wl.max_seq_len, wl.scale)
    perm = torch.randperm(wl.num_blocks, generator=torch.Generator().manual_seed(5)).cuda()
    kc = torch.empty_like(t["k_cache"]); vc = torch.empty_like(t["v_cache"])
    kc[perm] = t["k_cache"]; vc[perm] = t["v_cache"]
    out2 = binding.decode(t["query"], kc, vc, perm[bt.long()].int().contiguous(), lens,
                          wl.max_seq_len, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("where", ["first", "boundary", "tail"])
def test_needle_is_found(where):
    """One key per sequence is made to dominate; the output must be that
    key's value row (an O(1) error if the block holding it were missed)."""
    lens = [1000, 257, 4096, 33]
    wl = workloads.make_workload(2, device="cuda", seq_lens=lens, q_lens=[1] * 4)
    t = wl.tensors
    B = wl.shape.block_size
    G = wl.shape.num_q_heads // wl.shape.num_kv_heads
    needles = []
    for s, L in enumerate(lens):
        p = {"first": 0, "boundary": (L // 2) // B * B, "tail": L - 2}[where]
        blk = wl.block_tables[s][p // B]
        for h in range(wl.shape.num_kv_heads):
            qvec = t["query"][s, h * G:(h + 1) * G].float().sum(0)
            t["k_cache"][blk, h, p % B] = (qvec / qvec.norm() * 60).to(torch.bfloat16)
        needles.append((s, blk, p))
    bt = wl.block_tables_tensor("cuda")
    out = binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, wl.seq_lens_tensor("cuda"),
                         wl.max_seq_len, wl.scale)
    torch.cuda.synchronize()
    for s, blk, p in needles:
        for h in range(wl.shape.num_kv_heads):
            v = t["v_cache"][blk, h, :, p % B].float()
            got = out[s, h * G:(h + 1) * G].float()
            assert (got - v).abs().max().item() < 0.1, (s, h, where)


def test_pa_check_reports_bad_metadata(monkeypatch):
    monkeypatch.setenv("PA_CHECK", "1")
    wl = workloads.make_workload(2, device="cuda", seq_lens=[40, 20], q_lens=[1, 1])
    t = wl.tensors
    bt = wl.block_tables_tensor("cuda")
    lens = wl.seq_lens_tensor("cuda")
    binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, lens, wl.max_seq_len, wl.scale)
    bad = bt.clone()
    bad[0, 1] = wl.num_blocks + 5
    with pytest.raises(binding.PAError) as e:
        binding.decode(t["query"], t["k_cache"], t["v_cache"], bad, lens, wl.max_seq_len, wl.scale)
    assert e.value.status == -6
    with pytest.raises(binding.PAError) as e:       # a length beyond max_seq_len
        binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, lens, 30, wl.scale)
    assert e.value.status == -6
    dup = torch.tensor([5, 5], dtype=torch.int64, device="cuda")
    with pytest.raises(binding.PAError) as e:
        binding.reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"], dup)
    assert e.value.status == -6


def test_negative_slots_are_skipped():
    wl = workloads.make_workload(2, device="cuda", seq_lens=[40, 20], q_lens=[1, 1])
    t = wl.tensors
    before_k = t["k_cache"].clone()
    before_v = t["v_cache"].clone()
    slots = torch.tensor([-1, -7], dtype=torch.int64, device="cuda")
    binding.reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"], slots)
    torch.cuda.synchronize()
    assert torch.equal(before_k.view(torch.int16), t["k_cache"].view(torch.int16))
    assert torch.equal(before_v.view(torch.int16), t["v_cache"].view(torch.int16))
