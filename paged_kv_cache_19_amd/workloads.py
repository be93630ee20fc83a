"""Seeded synthetic workloads for paged attention.

This module only draws inputs: sequence lengths, a scattered assignment of
physical block ids to each sequence's logical blocks (shared prefixes point at
the same ids), and N(0, 1) values for the query, the new K/V and the cache
pools.  It holds none of the method's arithmetic (no slot computation, no
cache write, no attention); the HIP library and the CPU oracle both take
their inputs from here and from nowhere else.

Block ids are handed out in sequence order from a seeded permutation of the
pool, one id per logical block, with every block of a shared prefix taken
from the sequence that owns it.  That is the order a first-in first-out
allocator produces when the owner writes the prefix, the other sequences
fork from it and each sequence then appends its own tokens; the tests replay
exactly that with the oracle's allocator and require identical tables.

Workload shapes (one attention layer; "G" = query heads per KV head):

1. tiny decode, fp32: 4 sequences of 12/10/33/64 tokens, 8/2 heads, head dim
   64, block size 4, a 64-block pool; sequences 0 and 1 share their first
   block.
2. Llama-3-8B layer decode, bf16: 64 sequences, lengths U[512, 4096],
   32/8 heads, head dim 128, block size 16.
3. Llama-3-70B layer decode, bf16: 128 sequences, lengths U[2048, 8192],
   64/8 heads, head dim 128, block size 16.
4. shared-prefix decode, bf16: 256 sequences sharing one 512-token prefix
   (32 blocks) plus a private suffix of U[64, 1024] tokens, 32/8 heads.
5. chunked prefill + decode mix, bf16: 4 requests with a 512-token query
   chunk after U[1024, 8192] cached tokens, then 60 decode sequences of
   U[256, 4096] tokens; 32/8 heads, head dim 128, block size 16.
6. long-context decode, bf16: 8 sequences of U[32768, 131072] tokens at the
   Llama-3-70B layer shape (64/8 heads, head dim 128, block size 16).
7. Llama-3-70B layer decode with 32-token blocks: workload 3's batch shape
   (128 sequences of U[2048, 8192] tokens, 64/8 heads) at block size 32.

With ``kv_fp8`` the workload also carries an e4m3 KV cache: uint8 pools
``k_cache8`` / ``v_cache8`` (same layouts as the bf16 pools) of uniformly
drawn codes, the two NaN codes left out, and float32 scales ``k_scales`` /
``v_scales`` of shape ``[NB, H_kv]`` drawn uniformly from [2/448, 4/448]
(what an amax of 2 to 4 would give), so the dequantised values stay within
+-4 like the N(0, 1) values of the bf16 pools.  They come from a generator of their
own, so the bf16 tensors are the same with or without them.

Lengths are inclusive uniform integers.  ``seq_lens`` counts every token
including this step's new ones; the query rows of sequence s are its last
``q_len`` positions.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Shape:
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int


SHAPES: Dict[int, Shape] = {
    1: Shape("tiny-decode-fp32", F32, 8, 2, 64, 4),
    2: Shape("llama3-8b-layer-decode-bf16", BF16, 32, 8, 128, 16),
    3: Shape("llama3-70b-layer-decode-bf16", BF16, 64, 8, 128, 16),
    4: Shape("shared-prefix-decode-bf16", BF16, 32, 8, 128, 16),
    5: Shape("chunked-prefill-mix-bf16", BF16, 32, 8, 128, 16),
    6: Shape("long-context-decode-bf16", BF16, 64, 8, 128, 16),
    7: Shape("llama3-70b-layer-decode-b32-bf16", BF16, 64, 8, 128, 32),
}


@dataclass
class Workload:
    config: int
    shape: Shape
    seed: int
    seq_lens: List[int]
    q_lens: List[int]
    block_tables: List[List[int]]        # valid entries only, per sequence
    shared_blocks: List[int]             # logical blocks borrowed from seq 0
    num_blocks: int
    spare_blocks: List[int]              # pool ids no sequence uses
    pad_block: int                       # id written into unused table cells
    max_blocks_per_seq: int
    device: str = "cpu"
    tensors: Dict[str, torch.Tensor] = field(default_factory=dict)

    # -- derived views (shapes only) ------------------------------------------
    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def num_tokens(self) -> int:
        return int(sum(self.q_lens))

    @property
    def max_seq_len(self) -> int:
        return int(max(self.seq_lens))

    @property
    def max_query_len(self) -> int:
        return int(max(self.q_lens))

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.shape.head_dim)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.shape.dtype == F32 else torch.bfloat16

    def query_start_loc(self) -> List[int]:
        out = [0]
        for n in self.q_lens:
            out.append(out[-1] + n)
        return out

    def block_tables_tensor(self, device=None) -> torch.Tensor:
        S, M = self.num_seqs, self.max_blocks_per_seq
        bt = torch.full((S, M), self.pad_block, dtype=torch.int32)
        for s, row in enumerate(self.block_tables):
            bt[s, :len(row)] = torch.tensor(row, dtype=torch.int32)
        return bt.to(device or self.device)

    def block_refcounts_tensor(self, device=None) -> torch.Tensor:
        """int32 [num_blocks]: how many block tables hold each physical block
        (the block manager's reference count; 0 for spare blocks)."""
        rc = torch.zeros(self.num_blocks, dtype=torch.int32)
        for row in self.block_tables:
            rc[torch.tensor(row, dtype=torch.long)] += 1
        return rc.to(device or self.device)

    def seq_lens_tensor(self, device=None) -> torch.Tensor:
        return torch.tensor(self.seq_lens, dtype=torch.int32,
                            device=device or self.device)

    def query_start_loc_tensor(self, device=None) -> torch.Tensor:
        return torch.tensor(self.query_start_loc(), dtype=torch.int32,
                            device=device or self.device)


def _draw_lengths(cfg: int, rng: np.random.Generator):
    """Return (seq_lens, q_lens, shared_prefix_tokens)."""
    if cfg == 1:
        return [12, 10, 33, 64], [1, 1, 1, 1], 4
    if cfg == 2:
        lens = rng.integers(512, 4096 + 1, size=64)
        return lens.tolist(), [1] * 64, 0
    if cfg == 3:
        lens = rng.integers(2048, 8192 + 1, size=128)
        return lens.tolist(), [1] * 128, 0
    if cfg == 4:
        suffix = rng.integers(64, 1024 + 1, size=256)
        return (512 + suffix).tolist(), [1] * 256, 512
    if cfg == 5:
        ctx = rng.integers(1024, 8192 + 1, size=4)
        dec = rng.integers(256, 4096 + 1, size=60)
        lens = (ctx + 512).tolist() + dec.tolist()
        return lens, [512] * 4 + [1] * 60, 0
    if cfg == 6:
        lens = rng.integers(32768, 131072 + 1, size=8)
        return lens.tolist(), [1] * 8, 0
    if cfg == 7:
        lens = rng.integers(2048, 8192 + 1, size=128)
        return lens.tolist(), [1] * 128, 0
    raise ValueError(f"unknown workload {cfg}")


def make_workload(cfg: int, seed: Optional[int] = None, device: str = "cpu",
                  materialize: bool = True, seq_lens: Optional[List[int]] = None,
                  q_lens: Optional[List[int]] = None,
                  shape: Optional[Shape] = None,
                  shared_prefix_tokens: Optional[int] = None,
                  num_blocks: Optional[int] = None, kv_fp8: bool = False) -> Workload:
    """Draw workload ``cfg`` (1..7) with ``seed`` (default 1000 + cfg).

    ``seq_lens``/``q_lens``/``shape``/``shared_prefix_tokens``/``num_blocks``
    override the named workload to build custom cases (ragged tails, tiny
    brute-force cases, other block sizes).  With ``materialize`` False only
    the integer structure is drawn.
    """
    seed = 1000 + cfg if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    shp = shape or SHAPES.get(cfg, SHAPES[2])
    if seq_lens is None:
        lens, qls, prefix = _draw_lengths(cfg, rng)
    else:
        lens = list(seq_lens)
        qls = list(q_lens) if q_lens is not None else [1] * len(lens)
        prefix = 0
    if shared_prefix_tokens is not None:
        prefix = shared_prefix_tokens
    B = shp.block_size
    if prefix % B:
        raise ValueError("a shared prefix must end on a block boundary")
    shared = list(range(prefix // B))
    if any(L < prefix for L in lens[1:]) and prefix:
        raise ValueError("every sequence must hold the shared prefix")
    blocks_per_seq = [-(-L // B) for L in lens]
    distinct = blocks_per_seq[0] + sum(n - len(shared) for n in blocks_per_seq[1:])
    if num_blocks is None:
        num_blocks = 64 if cfg == 1 and seq_lens is None else distinct + max(64, distinct // 16)
    if num_blocks <= distinct:
        raise ValueError("pool too small: need at least one spare block")
    perm = rng.permutation(num_blocks).tolist()
    nxt = 0
    tables: List[List[int]] = []
    for s, nb in enumerate(blocks_per_seq):
        row = []
        for lb in range(nb):
            if s > 0 and lb < len(shared):
                row.append(tables[0][lb])
            else:
                row.append(perm[nxt])
                nxt += 1
        tables.append(row)
    spare = perm[nxt:]
    wl = Workload(cfg, shp, seed, [int(x) for x in lens], [int(x) for x in qls],
                  tables, shared, num_blocks, spare, spare[0],
                  max(blocks_per_seq) + 1, device)
    if materialize:
        _draw_values(wl)
        if kv_fp8:
            _draw_fp8_cache(wl)
    return wl


def _draw_values(wl: Workload) -> None:
    """N(0, 1) values, drawn in float32 and rounded (RNE) to the dtype."""
    shp = wl.shape
    gen = torch.Generator(device=wl.device)
    gen.manual_seed(wl.seed)
    NB, H, B, D, Hq = wl.num_blocks, shp.num_kv_heads, shp.block_size, shp.head_dim, shp.num_q_heads
    T = wl.num_tokens
    dt = wl.torch_dtype

    def randn(*size):
        return torch.randn(*size, generator=gen, device=wl.device,
                           dtype=torch.float32).to(dt)

    wl.tensors["k_cache"] = randn(NB, H, B, D)
    wl.tensors["v_cache"] = randn(NB, H, D, B)
    wl.tensors["key"] = randn(T, H, D)
    wl.tensors["value"] = randn(T, H, D)
    wl.tensors["query"] = randn(T, Hq, D)


def _draw_fp8_cache(wl: Workload) -> None:
    """Uniform e4m3 codes (NaN codes 0x7F/0xFF excluded) and uniform scales."""
    shp = wl.shape
    gen = torch.Generator(device=wl.device)
    gen.manual_seed(wl.seed + 7919)
    NB, H, B, D = wl.num_blocks, shp.num_kv_heads, shp.block_size, shp.head_dim

    def codes(*size):
        c = torch.randint(0, 254, size, generator=gen, device=wl.device, dtype=torch.int32)
        return (c + (c >= 127).to(torch.int32)).to(torch.uint8)   # skip 0x7F; 0xFF unreachable

    def scales():
        return torch.rand(NB, H, generator=gen, device=wl.device,
                          dtype=torch.float32) * (2.0 / 448) + 2.0 / 448

    wl.tensors["k_cache8"] = codes(NB, H, B, D)
    wl.tensors["v_cache8"] = codes(NB, H, D, B)
    wl.tensors["k_scales"] = scales()
    wl.tensors["v_scales"] = scales()
