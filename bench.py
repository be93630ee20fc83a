#!/usr/bin/env python3
"""Paged-attention decode benchmark on one MI355X.

One step = the whole hot path over one synthetic decode batch, through the C
ABI: slot mapping for the new tokens, the cache write of their K/V, and
split-K paged decode attention (attention pass + log-sum-exp merge).  Inputs
are resident in HBM before the timed region.

Workload (default): one Llama-3-70B attention layer in bf16 -- 128 sequences
of U[2048, 8192] tokens, 64 query / 8 KV heads, head_dim 128, block size 16,
blocks scattered by a seeded permutation of the pool.

Prints ONE JSON line.  ``value`` is the step's KV-read throughput in GB/s
(algorithmic KV bytes / step time); tokens/s and the fraction of the 8 TB/s
HBM peak ride along.  ``roofline`` covers pa_decode (the dominant call),
timed with HIP events on the stream its kernels run on.  ``cpu_baseline`` is
the CPU oracle timed on a bounded sample of the same batch.
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
CSRC = os.path.join(ROOT, "paged_kv_cache_19_amd", "csrc")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pa_decode_llama3-70b-layer_hbm_counters.md")


def kernel_source_digest() -> str:
    """sha256 over the HIP/C++ sources of libpa (ties counter data to code)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: int):
    """HBM bytes per pa_decode call from the committed rocprofv3 counter
    summary, or None when the summary is missing, is for another workload, or
    was taken on different kernel sources."""
    if workload != 3 or not os.path.exists(PMC_SUMMARY):
        return None
    fields = {}
    with open(PMC_SUMMARY) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", type=int, default=3, choices=[2, 3, 4])
    p.add_argument("--kv-split", type=int, default=0, help="keys per split (0: library default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget for the oracle baseline")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="also run one plain device copy of BYTES bytes (a reference for "
                        "hardware byte counters)")
    return p.parse_args()


def algorithmic_bytes(wl):
    """Bytes pa_decode must move: every sequence's K and V (token-exact),
    the query and output rows, the block-table entries it reads and seq_lens.
    For a shared prefix the shared blocks count once (unique bytes)."""
    shp = wl.shape
    e = 2 if shp.dtype == "bf16" else 4
    per_tok = 2 * shp.num_kv_heads * shp.head_dim * e
    shared_tokens = len(wl.shared_blocks) * shp.block_size
    kv_tokens = sum(wl.seq_lens) - shared_tokens * (wl.num_seqs - 1)
    kv = kv_tokens * per_tok
    qo = 2 * wl.num_tokens * shp.num_q_heads * shp.head_dim * e
    tables = sum(-(-L // shp.block_size) for L in wl.seq_lens) * 4 + wl.num_seqs * 4
    return kv, kv + qo + tables


def cpu_baseline(wl, budget_s):
    """The oracle (gather through the block table + float64 softmax attention)
    on whole sequences of the same batch, cycling through it until about
    ``budget_s`` seconds of CPU work are done."""
    import torch

    import oracle.paged_attention as ref

    kc = wl.tensors["k_cache"].cpu()
    vc = wl.tensors["v_cache"].cpu()
    q = wl.tensors["query"].cpu()
    bt = wl.block_tables_tensor("cpu")
    n_seqs, n_tok, kv_bytes = 0, 0, 0
    per_tok = 2 * wl.shape.num_kv_heads * wl.shape.head_dim * 2
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        s = n_seqs % wl.num_seqs
        ref.decode(q, kc, vc, bt, wl.seq_lens, wl.scale, seq_ids=[s])
        n_seqs += 1
        n_tok += wl.seq_lens[s]
        kv_bytes += wl.seq_lens[s] * per_tok
    dt = time.perf_counter() - t0
    return {
        "value": round(n_seqs / dt, 3),
        "unit": "tokens/s",
        "kv_gbs": round(kv_bytes / dt / 1e9, 4),
        "cores": torch.get_num_threads(),
        "kind": "oracle",
        "sample": f"{n_seqs} decode rows (sequences of the same batch, cycled; {n_tok} cached "
                  f"tokens, all 64 heads each) in {dt:.1f} s",
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_kv_cache_19_amd import binding, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()  # raises if libpa.so is missing
    dev = "cuda"
    wl = workloads.make_workload(args.workload, device=dev)
    shp = wl.shape
    t = wl.tensors
    bt = wl.block_tables_tensor(dev)
    lens = wl.seq_lens_tensor(dev)
    refcounts = wl.block_refcounts_tensor(dev)
    S, Hq, D = t["query"].shape
    ws = torch.zeros(binding.decode_workspace_bytes(S, Hq, D, wl.max_seq_len, shp.block_size,
                                                    args.kv_split), dtype=torch.uint8, device=dev)
    out = torch.empty_like(t["query"])
    slots = torch.empty(S, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        binding.compute_slot_mapping(bt, lens, None, shp.block_size, out=slots)
        binding.reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"], slots)
        if ev is not None:
            ev[0].record(stream)
        binding.decode(t["query"], t["k_cache"], t["v_cache"], bt, lens, wl.max_seq_len, wl.scale,
                       kv_split_tokens=args.kv_split, block_refcounts=refcounts, out=out,
                       workspace=ws)
        if ev is not None:
            ev[1].record(stream)

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

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        step(evs[k])
    stop.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    decode_ms = sorted(a.elapsed_time(b) for a, b in evs)
    decode_avg = sum(decode_ms) / len(decode_ms)
    print(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step, pa_decode avg "
          f"{decode_avg:.4f} ms (min {decode_ms[0]:.4f}, max {decode_ms[-1]:.4f})",
          file=sys.stderr, flush=True)

    kv_bytes, decode_bytes = algorithmic_bytes(wl)
    gbs = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = decode_bytes / (decode_avg * 1e-3) / 1e9
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
        "dtype": shp.dtype,
        "data": "synthetic",
        "config": {
            "workload": shp.name,
            "num_seqs": wl.num_seqs,
            "num_q_heads": shp.num_q_heads,
            "num_kv_heads": shp.num_kv_heads,
            "head_dim": shp.head_dim,
            "block_size": shp.block_size,
            "seq_lens": {2: "U[512,4096]", 3: "U[2048,8192]", 4: "512 shared + U[64,1024]"}[
                args.workload],
            "seed": wl.seed,
            "total_tokens": sum(wl.seq_lens),
            "kv_bytes": kv_bytes,
            "kv_split_tokens": args.kv_split,
            "step": "slot mapping + reshape_and_cache + pa_decode",
        },
        "tokens_per_s": round(wl.num_seqs / (ms_step * 1e-3), 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {
            "kernel": "pa_decode: balanced split-K attention kernel + merge kernel",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "bytes_per_launch": decode_bytes,
            "avg_launch_ms": round(decode_avg, 5),
            "traffic": measured_traffic(args.workload),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
