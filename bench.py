#!/usr/bin/env python3
"""Paged-attention benchmark on one MI355X.

One step = the whole hot path over one synthetic batch, through the C ABI:
slot mapping for the new tokens, the cache write of their K/V, and paged
attention.  For the decode workloads that is one pa_decode_append call
(pa_decode_fp8_append on the e4m3 cache), which computes each sequence's
new slot, writes its K/V and attends in one launch, then merges; with
``--no-append``, and always for the prefill + decode mix (pa_chunked_prefill)
the three calls pa_compute_slot_mapping, pa_reshape_and_cache and the
attention call (the shared-prefix decode has its own appending call,
pa_decode_shared_prefix_append).  The separate calls are timed
in every run (``cache_write``, and ``separate_calls`` beside an appending
step).  Inputs are resident in HBM before the timed region.

Workload (default 3): one Llama-3-70B attention layer in bf16 -- 128
sequences of U[2048, 8192] tokens, 64 query / 8 KV heads, head_dim 128,
block size 16, blocks scattered by a seeded permutation of the pool.
``--workload`` picks another of the seeded workloads (2: Llama-3-8B layer,
4: shared prefix, 5: chunked prefill + decode mix, 6: long context
U[32K, 128K], 7: workload 3 with 32-token blocks); ``--kv-dtype fp8`` runs
the decode workloads on the e4m3 cache (cache write and decode of the fp8
entry points).

Prints ONE JSON line.  ``value`` is the step's KV-read throughput in GB/s
(algorithmic KV bytes / step time); tokens/s and the fraction of the 8 TB/s
HBM peak ride along.  The K timed steps carry no event between their
kernels; a second pass of K steps under the same conditions times the
parts.  ``roofline`` covers the attention call (the dominant one), timed
there with HIP events on the stream its kernels run on: HBM-bound for
decode, MFMA-bound (bf16 dense peak) for the chunked-prefill mix.
``roofline.ceiling`` is the second denominator, measured in the same run:
for decode the read rate of a probe that gathers random 4 KiB tiles (one K
or V tile of a block and KV head) from a 4 GiB pool with the decode's loads;
for the chunked-prefill mix the rate of back-to-back
v_mfma_f32_32x32x16_bf16, the chunk kernel's instruction.  ``--tp N`` runs
one tensor-parallel rank's share of a workload: the same sequences with
H_q / N query and H_kv / N KV heads.
``cache_write`` times pa_reshape_and_cache (and the slot mapping) on their
own.  By default the 256 MB Infinity Cache is flushed before every step,
outside the timed events, so no step reads what the step before left there
(a serving loop's next call on a layer comes after every other layer).
``cpu_baseline`` is the CPU oracle timed on a bounded sample of the same
batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attention decode KV-read GB/s (% of HBM peak) and tokens/s, 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "paged_kv_cache_19_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_19_amd", "libpa_probe.so")
CEILING_TILE_BYTES = 4096
CEILING_POOL_BYTES = 4 << 30

SEQ_LENS = {
    2: "U[512,4096]",
    3: "U[2048,8192]",
    4: "512 shared + U[64,1024]",
    5: "4 x (ctx U[1024,8192] + 512-token chunk) + 60 decode U[256,4096]",
    6: "U[32768,131072]",
    7: "U[2048,8192]",
}


def kernel_source_digest() -> str:
    """sha256 over the HIP/C++ sources of libpa (ties counter data to code)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        path = os.path.join(CSRC, name)
        if not os.path.isfile(path):
            continue
        with open(path, "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _summary_fields(path):
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip()] = v.strip().strip("`")
    return fields


def measured_traffic(workload_name: str, call: str):
    """HBM bytes per attention call from the committed rocprofv3 counter
    summary of this workload and call (``profiles/*_hbm_counters.md``), or
    None when there is none or it was taken on different kernel sources."""
    if not os.path.isdir(PROFILES):
        return None
    digest = kernel_source_digest()
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith("_hbm_counters.md"):
            continue
        fields = _summary_fields(os.path.join(PROFILES, name))
        if fields.get("workload") != workload_name or fields.get("call") != call:
            continue
        if fields.get("kernel_source_sha256") != digest:
            return None
        try:
            return int(fields["traffic_bytes_per_call"])
        except (KeyError, ValueError):
            return None
    return None


def read_ceiling(dev, reps=5):
    """GB/s of the random-tile read probe (libpa_probe.so): a permutation of
    the 4 KiB tiles of a 4 GiB pool, 2,048 waves, non-temporal 16-byte loads.
    Returns (median GB/s, description) or (None, reason)."""
    import ctypes

    import torch
    if not os.path.exists(PROBE_LIB):
        return None, "libpa_probe.so not built"
    lib = ctypes.CDLL(PROBE_LIB)
    fn = lib.pa_probe_read_tiles
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    n_tiles = CEILING_POOL_BYTES // CEILING_TILE_BYTES
    waves = 2048
    pool = torch.empty(CEILING_POOL_BYTES, dtype=torch.uint8, device=dev)
    ids = torch.randperm(n_tiles, dtype=torch.int32, device=dev,
                         generator=torch.Generator(device=dev).manual_seed(7))
    sink = torch.empty(waves * 64, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    rates = []
    for k in range(reps + 1):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rc = fn(pool.data_ptr(), CEILING_POOL_BYTES, ids.data_ptr(), n_tiles, CEILING_TILE_BYTES,
                sink.data_ptr(), waves, ctypes.c_void_p(stream.cuda_stream))
        b.record(stream)
        if rc != 0:
            return None, f"probe returned {rc}"
        torch.cuda.synchronize()
        if k > 0:
            rates.append(CEILING_POOL_BYTES / (a.elapsed_time(b) * 1e-3) / 1e9)
    del pool, ids, sink
    torch.cuda.empty_cache()
    return percentile(rates, 50), (f"random {CEILING_TILE_BYTES // 1024} KiB tiles of a "
                                   f"{CEILING_POOL_BYTES >> 30} GiB pool, {waves} waves, "
                                   f"non-temporal 16-byte loads; median of {reps} reads")


def mfma_ceiling(dev, reps=5):
    """TFLOP/s of back-to-back v_mfma_f32_32x32x16_bf16 (libpa_probe.so):
    two workgroups of four waves per CU, four independent accumulators per
    wave.  Returns (median TFLOP/s, description) or (None, reason)."""
    import ctypes

    import torch
    if not os.path.exists(PROBE_LIB):
        return None, "libpa_probe.so not built"
    lib = ctypes.CDLL(PROBE_LIB)
    fn = lib.pa_probe_mfma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    wgs = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 8192
    flops = wgs * 4 * iters * 4 * 2 * 32 * 32 * 16
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    warm = 20  # about 20 ms of matrix work first: the clock ramps up under it
    rates = []
    for k in range(warm + reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rc = fn(sink.data_ptr(), wgs, iters, ctypes.c_void_p(stream.cuda_stream))
        b.record(stream)
        if rc != 0:
            return None, f"probe returned {rc}"
        if k >= warm:
            torch.cuda.synchronize()
            rates.append(flops / (a.elapsed_time(b) * 1e-3) / 1e12)
    torch.cuda.synchronize()
    del sink
    return percentile(rates, 50), (f"back-to-back v_mfma_f32_32x32x16_bf16, {wgs} workgroups "
                                   f"of 4 waves, 4 accumulators per wave, after {warm} untimed "
                                   f"runs; median of {reps} runs")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=50,
                   help="untimed steps first (the first ~90 calls of the chunked-prefill mix run up to 18% slower)")
    p.add_argument("--workload", type=int, default=3, choices=sorted(SEQ_LENS))
    p.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"])
    p.add_argument("--kv-split", type=int, default=0, help="keys per split (0: library default)")
    p.add_argument("--shared-prefix", action="store_true",
                   help="decode through pa_decode_shared_prefix, which reads the blocks every "
                        "table starts with once per group of sequences (workload 4)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget for the oracle baseline")
    p.add_argument("--flush", action=argparse.BooleanOptionalAction, default=True,
                   help="write a 1 GiB scratch buffer before every step, outside the timed "
                        "events, so that no step reads K/V left in the 256 MB Infinity Cache "
                        "by the step before; ms_per_step is then the mean of per-step events "
                        "(default on; --no-flush times back-to-back steps)")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the ceiling probe (the roofline's second denominator)")
    p.add_argument("--tp", type=int, default=1,
                   help="one tensor-parallel rank's share: H_q / tp query and H_kv / tp KV "
                        "heads of the workload (tp divides H_kv)")
    p.add_argument("--append", action=argparse.BooleanOptionalAction, default=True,
                   help="decode workloads: the step is one pa_decode_append (or "
                        "pa_decode_fp8_append, or with --shared-prefix "
                        "pa_decode_shared_prefix_append) call, which computes the new tokens' "
                        "slots, writes them and attends in one launch plus the merge "
                        "(default); --no-append times the three separate calls instead.  The "
                        "separate calls are timed either way")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="also run one plain device copy of BYTES bytes (a reference for "
                        "hardware byte counters)")
    return p.parse_args()


def kv_bytes_per_token(shp, kv_dtype):
    e = 1 if kv_dtype == "fp8" else (2 if shp.dtype == "bf16" else 4)
    return 2 * shp.num_kv_heads * shp.head_dim * e


def algorithmic_bytes(wl, kv_dtype="bf16"):
    """Bytes the attention call must move: every sequence's K and V
    (token-exact), the query and output rows, the block-table entries it
    reads and seq_lens (and, for fp8, one K and one V scale per block and KV
    head).  For a shared prefix the shared blocks count once (unique
    bytes).  Returns (KV bytes, all bytes)."""
    shp = wl.shape
    e = 2 if shp.dtype == "bf16" else 4
    shared_tokens = len(wl.shared_blocks) * shp.block_size
    kv_tokens = sum(wl.seq_lens) - shared_tokens * (wl.num_seqs - 1)
    kv = kv_tokens * kv_bytes_per_token(shp, kv_dtype)
    qo = 2 * wl.num_tokens * shp.num_q_heads * shp.head_dim * e
    nblk = sum(-(-L // shp.block_size) for L in wl.seq_lens)
    tables = nblk * 4 + wl.num_seqs * 4
    scales = nblk * shp.num_kv_heads * 8 if kv_dtype == "fp8" else 0
    return kv, kv + qo + tables + scales


def algorithmic_flops(wl):
    """4 * H_q * D flops (QK^T and PV multiply-adds) per key each query row
    attends to (causal: row j of a q_len chunk sees L - q_len + j + 1 keys).
    Returns (query-chunk flops, single-row flops)."""
    shp = wl.shape
    chunk = single = 0
    for L, n in zip(wl.seq_lens, wl.q_lens):
        keys = n * (L - n) + n * (n + 1) // 2
        f = 4 * shp.num_q_heads * shp.head_dim * keys
        if n > 1:
            chunk += f
        else:
            single += f
    return chunk, single


def cpu_baseline(wl, budget_s, kv_dtype):
    """The oracle (gather through the block table + float64 softmax attention)
    on whole sequences of the same batch, cycling through it until about
    ``budget_s`` seconds of CPU work are done."""
    import torch

    import oracle.paged_attention as ref
    import oracle.fp8 as ref8

    t = wl.tensors
    q = t["query"].cpu()
    bt = wl.block_tables_tensor("cpu")
    qsl = wl.query_start_loc()
    if kv_dtype == "fp8":
        pools = (t["k_cache8"].cpu(), t["v_cache8"].cpu(), t["k_scales"].cpu(),
                 t["v_scales"].cpu())
    else:
        pools = (t["k_cache"].cpu(), t["v_cache"].cpu())
    affinity = len(os.sched_getaffinity(0))
    threads = affinity
    env_threads = os.environ.get("OMP_NUM_THREADS", "")
    if env_threads.isdigit() and int(env_threads) > 0:
        threads = min(threads, int(env_threads))   # the process's CPU share on a shared host
    torch.set_num_threads(threads)
    n_seqs = n_rows = n_tok = kv_bytes = 0
    per_tok = kv_bytes_per_token(wl.shape, kv_dtype)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        s = n_seqs % wl.num_seqs
        if kv_dtype == "fp8":
            ref8.paged_attention_fp8(q, *pools, bt, wl.seq_lens, qsl, wl.scale, seq_ids=[s])
        else:
            ref.paged_attention(q, *pools, bt, wl.seq_lens, qsl, wl.scale, seq_ids=[s])
        n_seqs += 1
        n_rows += wl.q_lens[s]
        n_tok += wl.seq_lens[s]
        kv_bytes += wl.seq_lens[s] * per_tok
    dt = time.perf_counter() - t0
    return {
        "value": round(n_rows / dt, 3),
        "unit": "tokens/s",
        "kv_gbs": round(kv_bytes / dt / 1e9, 4),
        "cores": torch.get_num_threads(),
        "affinity_cpus": affinity,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{n_seqs} sequences of the same batch (cycled; {n_rows} query rows, {n_tok} "
                  f"cached tokens, all {wl.shape.num_q_heads} heads each) in {dt:.1f} s",
    }


def percentile(xs, p):
    xs = sorted(xs)
    k = min(len(xs) - 1, max(0, int(round(p / 100 * (len(xs) - 1)))))
    return xs[k]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    fp8 = args.kv_dtype == "fp8"
    if fp8 and args.kv_split:
        print("the fp8 cache runs the balanced decode only (no fixed split)", file=sys.stderr)
        sys.exit(2)

    if args.shared_prefix and (args.workload == 5 or args.kv_split):
        print("--shared-prefix is a decode of the balanced kind (no chunked prefill, no fixed "
              "split)", file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_kv_cache_19_amd import binding, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()  # raises if libpa.so is missing
    dev = "cuda"
    shape = None
    if args.tp != 1:
        base = workloads.SHAPES[args.workload]
        if args.tp < 1 or base.num_kv_heads % args.tp:
            print(f"--tp must divide the workload's {base.num_kv_heads} KV heads", file=sys.stderr)
            sys.exit(2)
        shape = workloads.Shape(base.name.replace("-bf16", f"-tp{args.tp}-rank-bf16"),
                                base.dtype, base.num_q_heads // args.tp,
                                base.num_kv_heads // args.tp, base.head_dim, base.block_size)
    wl = workloads.make_workload(args.workload, device=dev, kv_fp8=fp8, shape=shape)
    shp = wl.shape
    t = wl.tensors
    bt = wl.block_tables_tensor(dev)
    lens = wl.seq_lens_tensor(dev)
    refcounts = wl.block_refcounts_tensor(dev)
    chunked = args.workload == 5
    qsl = wl.query_start_loc_tensor(dev) if chunked else None
    T, Hq, D = t["query"].shape
    S = wl.num_seqs
    prefix_blocks = len(wl.shared_blocks)
    if args.shared_prefix and prefix_blocks == 0:
        print("--shared-prefix: this workload's tables share no prefix", file=sys.stderr)
        sys.exit(2)
    if args.shared_prefix:
        ws_bytes = binding.decode_shared_prefix_workspace_bytes(S, Hq, D, wl.max_seq_len,
                                                                shp.block_size, prefix_blocks)
    elif chunked and fp8:
        cap = binding.chunk_context_blocks(wl.seq_lens, wl.query_start_loc(), shp.block_size)
        ws_bytes = binding.chunked_prefill_fp8_workspace_bytes(
            S, T, Hq, shp.num_kv_heads, D, wl.max_seq_len, bt.shape[1], shp.block_size, cap)
    elif chunked:
        ws_bytes = binding.chunked_prefill_workspace_bytes(S, T, Hq, D, wl.max_seq_len,
                                                           shp.block_size, args.kv_split)
    elif fp8:
        ws_bytes = binding.decode_fp8_workspace_bytes(S, Hq, D, wl.max_seq_len, shp.block_size)
    else:
        ws_bytes = binding.decode_workspace_bytes(S, Hq, D, wl.max_seq_len, shp.block_size,
                                                  args.kv_split)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(t["query"])
    slots = torch.empty(T, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    def attention():
        if args.shared_prefix:
            kc, vc = (t["k_cache8"], t["v_cache8"]) if fp8 else (t["k_cache"], t["v_cache"])
            scales = dict(k_scales=t["k_scales"], v_scales=t["v_scales"]) if fp8 else {}
            binding.decode_shared_prefix(t["query"], kc, vc, bt, lens, wl.max_seq_len, wl.scale,
                                         prefix_blocks, block_refcounts=refcounts, out=out,
                                         workspace=ws, **scales)
        elif chunked and fp8:
            binding.chunked_prefill_fp8(t["query"], t["k_cache8"], t["v_cache8"], t["k_scales"],
                                        t["v_scales"], bt, lens, qsl, wl.max_seq_len,
                                        wl.max_query_len, wl.scale, cap,
                                        block_refcounts=refcounts, out=out, workspace=ws)
        elif chunked:
            binding.chunked_prefill(t["query"], t["k_cache"], t["v_cache"], bt, lens, qsl,
                                    wl.max_seq_len, wl.max_query_len, wl.scale,
                                    kv_split_tokens=args.kv_split, block_refcounts=refcounts,
                                    out=out, workspace=ws)
        elif fp8:
            binding.decode_fp8(t["query"], t["k_cache8"], t["v_cache8"], t["k_scales"],
                               t["v_scales"], bt, lens, wl.max_seq_len, wl.scale,
                               block_refcounts=refcounts, out=out, workspace=ws)
        else:
            binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, lens, wl.max_seq_len,
                           wl.scale, kv_split_tokens=args.kv_split, block_refcounts=refcounts,
                           out=out, workspace=ws)

    append = args.append and not chunked

    def attention_append():
        if args.shared_prefix:
            kc, vc = (t["k_cache8"], t["v_cache8"]) if fp8 else (t["k_cache"], t["v_cache"])
            scales = dict(k_scales=t["k_scales"], v_scales=t["v_scales"]) if fp8 else {}
            binding.decode_shared_prefix_append(t["query"], t["key"], t["value"], kc, vc, bt, lens,
                                                wl.max_seq_len, wl.scale, prefix_blocks,
                                                block_refcounts=refcounts, out=out, workspace=ws,
                                                **scales)
        elif fp8:
            binding.decode_fp8_append(t["query"], t["key"], t["value"], t["k_cache8"],
                                      t["v_cache8"], t["k_scales"], t["v_scales"], bt, lens,
                                      wl.max_seq_len, wl.scale, block_refcounts=refcounts,
                                      out=out, workspace=ws)
        else:
            binding.decode_append(t["query"], t["key"], t["value"], t["k_cache"], t["v_cache"],
                                  bt, lens, wl.max_seq_len, wl.scale,
                                  kv_split_tokens=args.kv_split, block_refcounts=refcounts,
                                  out=out, workspace=ws)

    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if args.flush else None

    def step(ev=None, sev=None, wev=None, fused=append):
        if scratch is not None:
            scratch.fill_(1)  # evicts the Infinity Cache; outside every timed event
        if sev is not None:
            sev[0].record(stream)
        if fused:  # slot computation, cache write and attention in one call
            attention_append()
            if sev is not None:
                sev[1].record(stream)
            return
        binding.compute_slot_mapping(bt, lens, qsl, shp.block_size, num_tokens=T, out=slots)
        if wev is not None:
            wev.record(stream)
        if fp8:
            binding.reshape_and_cache_fp8(t["key"], t["value"], t["k_cache8"], t["v_cache8"],
                                          t["k_scales"], t["v_scales"], slots)
        else:
            binding.reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"], slots)
        if ev is not None:
            ev[0].record(stream)
        attention()
        if ev is not None:
            ev[1].record(stream)
        if sev is not None:
            sev[1].record(stream)

    if args.copy_probe:
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    def pairs():
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
    # The timed region: exactly K steps, each bracketed by its own two events
    # (so that the flushes between steps can be left out) and nothing inside
    # it, so that no event record sits between the step's kernels.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    sevs = pairs()
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        step(sev=sevs[k])
    stop.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    if args.flush:  # the flushes are not part of the step
        ms_step = sum(a.elapsed_time(b) for a, b in sevs) / args.steps
    fused_ms = [a.elapsed_time(b) for a, b in sevs]  # the step is one call when appending
    # The parts of the step: K more steps of the separate calls under the
    # same conditions, with events around the attention call, the cache
    # write and the slot mapping.
    evs, sevs2 = pairs(), pairs()
    wevs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(evs[k], sevs2[k], wevs[k], fused=False)
    torch.cuda.synchronize()
    attn_ms = sep_attn_ms = [a.elapsed_time(b) for a, b in evs]
    slot_ms = [a[0].elapsed_time(w) for a, w in zip(sevs2, wevs)]
    write_ms = [w.elapsed_time(e[0]) for w, e in zip(wevs, evs)]
    separate_ms = None
    if append:
        # the three separate calls again, with only the bracketing events
        sevs3 = pairs()
        torch.cuda.synchronize()
        for k in range(args.steps):
            step(sev=sevs3[k], fused=False)
        torch.cuda.synchronize()
        separate_ms = sum(a.elapsed_time(b) for a, b in sevs3) / args.steps
    call = ("pa_chunked_prefill" + ("_fp8" if fp8 else "")) if chunked else (
        "pa_decode_fp8" if fp8 else "pa_decode")
    if args.shared_prefix:
        call = "pa_decode_shared_prefix"
    separate_call = call
    if append:  # the roofline covers the appending call, which is the whole step
        call = "pa_decode_fp8_append" if fp8 else "pa_decode_append"
        if args.shared_prefix:
            call = "pa_decode_shared_prefix_append"
        attn_ms = fused_ms
    attn_avg = sum(attn_ms) / len(attn_ms)
    print(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step, {call} avg "
          f"{attn_avg:.4f} ms (p10 {percentile(attn_ms, 10):.4f}, median "
          f"{percentile(attn_ms, 50):.4f}, p90 {percentile(attn_ms, 90):.4f})",
          file=sys.stderr, flush=True)

    # cache write: K and V rows read from the step's tensors and written to
    # their slots (the fp8 write reads bf16 and writes one byte per element)
    e_in = 2 if shp.dtype == "bf16" else 4
    e_out = 1 if fp8 else e_in
    write_bytes = 2 * T * shp.num_kv_heads * shp.head_dim * (e_in + e_out) + 8 * T
    if args.no_ceiling:
        ceiling, ceiling_how = None, "skipped"
    elif chunked:
        ceiling, ceiling_how = mfma_ceiling(dev)
        if ceiling is not None:
            print(f"[bench] MFMA ceiling {ceiling:.1f} TFLOP/s ({ceiling_how})", file=sys.stderr,
                  flush=True)
    else:
        ceiling, ceiling_how = read_ceiling(dev)
        if ceiling is not None:
            print(f"[bench] read ceiling {ceiling:.1f} GB/s ({ceiling_how})", file=sys.stderr,
                  flush=True)
    kv_bytes, call_bytes = algorithmic_bytes(wl, args.kv_dtype)
    if append:  # the new tokens' K and V, read and written inside the call
        call_bytes += 2 * T * shp.num_kv_heads * shp.head_dim * (e_in + e_out)
    gbs = kv_bytes / (ms_step * 1e-3) / 1e9
    workload_name = shp.name if not fp8 else shp.name.replace("-bf16", "-fp8kv")
    if chunked:
        f_chunk, f_single = algorithmic_flops(wl)
        achieved = (f_chunk + f_single) / (attn_avg * 1e-3) / 1e12
        roofline = {
            "kernel": ("pa_chunked_prefill_fp8: the query-chunk sequences' blocks staged as "
                       "bf16, then one persistent launch splitting the CUs between the "
                       "query-chunk units (MFMA, on the staged blocks) and the e4m3 balanced "
                       "decode of the single-token rows, then the merges") if fp8 else
                      ("pa_chunked_prefill: one persistent launch splitting the CUs between "
                       "the query-chunk units (MFMA) and the balanced decode of the "
                       "single-token rows, then the merges"),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_launch": f_chunk + f_single,
            "avg_launch_ms": round(attn_avg, 5),
            "traffic": measured_traffic(workload_name, call),
            "ceiling": None if ceiling is None else {
                "what": ceiling_how,
                "achieved_over_ceiling": round(achieved / ceiling, 4),
                "tflops": round(ceiling, 1),
            },
        }
    else:
        achieved = call_bytes / (attn_avg * 1e-3) / 1e9
        roofline = {
            "kernel": (f"{call}: balanced split-K attention kernel (the wave reading a "
                       "sequence's last key step first writes its new token) + merge kernel")
                      if append else f"{call}: balanced split-K attention kernel + merge kernel",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "bytes_per_launch": call_bytes,
            "avg_launch_ms": round(attn_avg, 5),
            "traffic": measured_traffic(workload_name, call),
            "ceiling": None if ceiling is None else {
                "what": ceiling_how,
                "achieved_over_ceiling": round(achieved / ceiling, 4),
                "gbs": round(ceiling, 1),
            },
        }
    roofline["p10_ms"] = round(percentile(attn_ms, 10), 5)
    roofline["median_ms"] = round(percentile(attn_ms, 50), 5)
    roofline["p90_ms"] = round(percentile(attn_ms, 90), 5)
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 cache, bf16 q/out" if fp8 else shp.dtype,
        "data": "synthetic",
        "config": {
            "workload": workload_name,
            "num_seqs": wl.num_seqs,
            "num_query_tokens": T,
            "num_q_heads": shp.num_q_heads,
            "num_kv_heads": shp.num_kv_heads,
            "head_dim": shp.head_dim,
            "block_size": shp.block_size,
            "kv_cache": args.kv_dtype,
            "seq_lens": SEQ_LENS[args.workload],
            "tensor_parallel_rank_of": args.tp,
            "seed": wl.seed,
            "total_tokens": sum(wl.seq_lens),
            "kv_bytes": kv_bytes,
            "kv_split_tokens": args.kv_split,
            "step": (f"{call} (slot computation, cache write and attention in one launch, "
                     "then the merge)") if append else
                    f"slot mapping + reshape_and_cache{'_fp8' if fp8 else ''} + {call}",
            "shared_prefix_blocks": prefix_blocks if args.shared_prefix else 0,
            "infinity_cache_flushed": bool(args.flush),
        },
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "cache_write": {
            "call": "pa_reshape_and_cache_fp8" if fp8 else "pa_reshape_and_cache",
            "avg_us": round(1e3 * sum(write_ms) / len(write_ms), 2),
            "median_us": round(1e3 * percentile(write_ms, 50), 2),
            "bytes": write_bytes,
            "slot_mapping_avg_us": round(1e3 * sum(slot_ms) / len(slot_ms), 2),
        },
    }
    if append:
        result["separate_calls"] = {
            "step": f"slot mapping + reshape_and_cache{'_fp8' if fp8 else ''} + {separate_call}",
            "ms_per_step": round(separate_ms, 5),
            "attention_avg_ms": round(sum(sep_attn_ms) / len(sep_attn_ms), 5),
        }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, args.kv_dtype)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
