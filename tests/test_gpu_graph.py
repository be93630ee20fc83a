"""The hot path inside a HIP graph (torch.cuda.CUDAGraph).

The entry points enqueue kernels on the caller's stream and make no host
synchronisation, allocation or memset of their own (outside PA_CHECK=1), so
a caller can capture a step -- the cache write and the attention, with the
output and workspace allocated beforehand -- and replay it.  Each test runs
the step eagerly, captures it, then replays the graph three times with eager
work in between (the output overwritten with NaN, an unrelated kernel, a
synchronisation) and requires every replay to reproduce the eager output bit
for bit.  The eager output itself is checked against the oracle elsewhere."""
import math

import pytest
import torch

from paged_kv_cache_19_amd import binding, workloads
from tests.gpu_common import bits, log

pytestmark = pytest.mark.gpu


def _replays_match(step, out, name):
    """step() enqueues the work and writes ``out``."""
    step()
    torch.cuda.synchronize()
    expect = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up on a side stream before the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    scratch = torch.empty(1 << 20, device="cuda")
    for r in range(3):
        out.fill_(math.nan)
        scratch.uniform_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(expect)), f"{name}: replay {r} differs from eager"
    log(f"[graph] {name}: 3 replays bit-identical to the eager step")


def _decode_batch(fp8=False):
    shape = workloads.Shape("graph", workloads.BF16, 32, 8, 128, 16)
    return workloads.make_workload(2, seed=31, device="cuda", seq_lens=[700, 33, 2100, 5, 512],
                                   shape=shape, kv_fp8=fp8)


def _chunk_batch(fp8=False):
    shape = workloads.Shape("graph-chunks", workloads.BF16, 32, 8, 128, 16)
    return workloads.make_workload(2, seed=32, device="cuda", seq_lens=[600, 17, 900, 300],
                                   q_lens=[64, 5, 1, 1], shape=shape, kv_fp8=fp8)


def test_graph_decode():
    wl = _decode_batch()
    t = wl.tensors
    B, D, S, Hq = 16, 128, wl.num_seqs, 32
    bt, lens = wl.block_tables_tensor("cuda"), wl.seq_lens_tensor("cuda")
    slots = binding.compute_slot_mapping(bt, lens, None, B)
    out = torch.empty_like(t["query"])
    ws = torch.empty(binding.decode_workspace_bytes(S, Hq, D, wl.max_seq_len, B),
                     dtype=torch.uint8, device="cuda")

    def step():
        binding.reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"], slots)
        binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, lens, wl.max_seq_len,
                       wl.scale, out=out, workspace=ws)
    _replays_match(step, out, "pa_reshape_and_cache + pa_decode")


def test_graph_decode_noalloc():
    wl = _decode_batch()
    t = wl.tensors
    bt, lens = wl.block_tables_tensor("cuda"), wl.seq_lens_tensor("cuda")
    out = torch.empty_like(t["query"])

    def step():
        binding.decode_noalloc(t["query"], t["k_cache"], t["v_cache"], bt, lens,
                               wl.max_seq_len, wl.scale, out=out)
    _replays_match(step, out, "pa_decode_noalloc")


def test_graph_decode_fp8():
    wl = _decode_batch(fp8=True)
    t = wl.tensors
    B, D, S, Hq = 16, 128, wl.num_seqs, 32
    bt, lens = wl.block_tables_tensor("cuda"), wl.seq_lens_tensor("cuda")
    slots = binding.compute_slot_mapping(bt, lens, None, B)
    out = torch.empty_like(t["query"])
    ws = torch.empty(binding.decode_fp8_workspace_bytes(S, Hq, D, wl.max_seq_len, B),
                     dtype=torch.uint8, device="cuda")

    def step():
        binding.reshape_and_cache_fp8(t["key"], t["value"], t["k_cache8"], t["v_cache8"],
                                      t["k_scales"], t["v_scales"], slots)
        binding.decode_fp8(t["query"], t["k_cache8"], t["v_cache8"], t["k_scales"],
                           t["v_scales"], bt, lens, wl.max_seq_len, wl.scale, out=out,
                           workspace=ws)
    _replays_match(step, out, "pa_reshape_and_cache_fp8 + pa_decode_fp8")


def test_graph_chunked_prefill():
    wl = _chunk_batch()
    t = wl.tensors
    B, D, S, Hq = 16, 128, wl.num_seqs, 32
    bt, lens = wl.block_tables_tensor("cuda"), wl.seq_lens_tensor("cuda")
    qsl = wl.query_start_loc_tensor("cuda")
    T = wl.num_tokens
    slots = binding.compute_slot_mapping(bt, lens, qsl, B, num_tokens=T)
    out = torch.empty_like(t["query"])
    ws = torch.empty(binding.chunked_prefill_workspace_bytes(S, T, Hq, D, wl.max_seq_len, B, 0),
                     dtype=torch.uint8, device="cuda")

    def step():
        binding.reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"], slots)
        binding.chunked_prefill(t["query"], t["k_cache"], t["v_cache"], bt, lens, qsl,
                                wl.max_seq_len, wl.max_query_len, wl.scale, out=out,
                                workspace=ws)
    _replays_match(step, out, "pa_reshape_and_cache + pa_chunked_prefill")


def test_graph_chunked_prefill_fp8():
    wl = _chunk_batch(fp8=True)
    t = wl.tensors
    B, D, S, Hq, Hkv = 16, 128, wl.num_seqs, 32, 8
    bt, lens = wl.block_tables_tensor("cuda"), wl.seq_lens_tensor("cuda")
    qsl = wl.query_start_loc_tensor("cuda")
    T = wl.num_tokens
    slots = binding.compute_slot_mapping(bt, lens, qsl, B, num_tokens=T)
    cap = binding.chunk_context_blocks(wl.seq_lens, wl.query_start_loc(), B)
    out = torch.empty_like(t["query"])
    ws = torch.empty(binding.chunked_prefill_fp8_workspace_bytes(
        S, T, Hq, Hkv, D, wl.max_seq_len, bt.shape[1], B, cap), dtype=torch.uint8, device="cuda")

    def step():
        binding.reshape_and_cache_fp8(t["key"], t["value"], t["k_cache8"], t["v_cache8"],
                                      t["k_scales"], t["v_scales"], slots)
        binding.chunked_prefill_fp8(t["query"], t["k_cache8"], t["v_cache8"], t["k_scales"],
                                    t["v_scales"], bt, lens, qsl, wl.max_seq_len,
                                    wl.max_query_len, wl.scale, cap, out=out, workspace=ws)
    _replays_match(step, out, "pa_reshape_and_cache_fp8 + pa_chunked_prefill_fp8")


def test_graph_decode_shared_prefix():
    shape = workloads.Shape("graph-sp", workloads.BF16, 32, 8, 128, 16)
    wl = workloads.make_workload(2, seed=33, device="cuda",
                                 seq_lens=[600, 513, 1400, 777, 530, 900], shape=shape,
                                 shared_prefix_tokens=512)
    t = wl.tensors
    B, D, S, Hq, pb = 16, 128, wl.num_seqs, 32, 512 // 16
    bt, lens = wl.block_tables_tensor("cuda"), wl.seq_lens_tensor("cuda")
    rc = wl.block_refcounts_tensor("cuda")
    slots = binding.compute_slot_mapping(bt, lens, None, B)
    out = torch.empty_like(t["query"])
    ws = torch.empty(binding.decode_shared_prefix_workspace_bytes(S, Hq, D, wl.max_seq_len, B,
                                                                  pb),
                     dtype=torch.uint8, device="cuda")

    def step():
        binding.reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"], slots)
        binding.decode_shared_prefix(t["query"], t["k_cache"], t["v_cache"], bt, lens,
                                     wl.max_seq_len, wl.scale, pb, block_refcounts=rc,
                                     out=out, workspace=ws)
    _replays_match(step, out, "pa_reshape_and_cache + pa_decode_shared_prefix")


def test_graph_decode_append():
    """The appending decode (slot computation, cache write and attention in
    one call) captured and replayed: every replay writes the same new tokens
    and reproduces the eager output and pools."""
    wl = _decode_batch()
    t = wl.tensors
    B, D, S, Hq = 16, 128, wl.num_seqs, 32
    bt, lens = wl.block_tables_tensor("cuda"), wl.seq_lens_tensor("cuda")
    out = torch.empty_like(t["query"])
    ws = torch.empty(binding.decode_workspace_bytes(S, Hq, D, wl.max_seq_len, B),
                     dtype=torch.uint8, device="cuda")

    def step():
        binding.decode_append(t["query"], t["key"], t["value"], t["k_cache"], t["v_cache"], bt,
                              lens, wl.max_seq_len, wl.scale, out=out, workspace=ws)
    _replays_match(step, out, "pa_decode_append")


def test_graph_decode_fp8_append():
    wl = _decode_batch(fp8=True)
    t = wl.tensors
    B, D, S, Hq = 16, 128, wl.num_seqs, 32
    bt, lens = wl.block_tables_tensor("cuda"), wl.seq_lens_tensor("cuda")
    out = torch.empty_like(t["query"])
    ws = torch.empty(binding.decode_fp8_workspace_bytes(S, Hq, D, wl.max_seq_len, B),
                     dtype=torch.uint8, device="cuda")

    def step():
        binding.decode_fp8_append(t["query"], t["key"], t["value"], t["k_cache8"],
                                  t["v_cache8"], t["k_scales"], t["v_scales"], bt, lens,
                                  wl.max_seq_len, wl.scale, out=out, workspace=ws)
    _replays_match(step, out, "pa_decode_fp8_append")


def test_graph_decode_shared_prefix_append():
    shape = workloads.Shape("graph-sp-append", workloads.BF16, 32, 8, 128, 16)
    wl = workloads.make_workload(2, seed=34, device="cuda",
                                 seq_lens=[600, 513, 1400, 777, 530, 900], shape=shape,
                                 shared_prefix_tokens=512)
    t = wl.tensors
    B, D, S, Hq, pb = 16, 128, wl.num_seqs, 32, 512 // 16
    bt, lens = wl.block_tables_tensor("cuda"), wl.seq_lens_tensor("cuda")
    rc = wl.block_refcounts_tensor("cuda")
    out = torch.empty_like(t["query"])
    ws = torch.empty(binding.decode_shared_prefix_workspace_bytes(S, Hq, D, wl.max_seq_len, B,
                                                                  pb),
                     dtype=torch.uint8, device="cuda")

    def step():
        binding.decode_shared_prefix_append(t["query"], t["key"], t["value"], t["k_cache"],
                                            t["v_cache"], bt, lens, wl.max_seq_len, wl.scale, pb,
                                            block_refcounts=rc, out=out, workspace=ws)
    _replays_match(step, out, "pa_decode_shared_prefix_append")
