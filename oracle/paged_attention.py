"""Paged attention, computed plainly on the CPU (oracle; test infrastructure only).

What the method computes, restated from the pages:

* Attention for a query is softmax(q K^T / sqrt(d)) V over all of the
  sequence's past keys and values ("03 -- PagedAttention & the vLLM V1
  Architecture", section "The attention kernel side"; "Inside vLLM: Anatomy
  of a High-Throughput LLM Inference System (2025)", section "Physical Block
  Mapping and Kernel Invocation", attention equation).
* Paging changes only where K and V live: position i of a sequence sits in
  the physical block its block table names for logical block floor(i / B), at
  offset i mod B (same sections; "High-Throughput Local LLM Infrastructure
  ...", section "1.2 PagedAttention Mechanics & Virtual Page Tables", index
  and offset equations).  So the oracle materialises each sequence's
  contiguous K and V from its table and then runs dense attention.
* New K/V are written into the slots the block table assigns ("High-Throughput
  Local LLM Infrastructure ...", section "2.1 PagedAttention Memory Allocation
  Life-Cycle", step 4).

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* one layer per call, K and V in separate pools; K pool ``[NB, H_kv, B, D]``
  (token rows, head_dim contiguous) and V pool ``[NB, H_kv, D, B]`` (each
  head_dim row holds the block's B tokens contiguously);
* slot = block id * B + offset; a negative slot means "write nothing";
* query head h reads KV head h // G with G = H_q / H_kv (contiguous groups);
* ``seq_lens`` counts the tokens after this step's K/V are written; the
  query rows of a sequence are its last ``q_len`` positions, and a query at
  position P sees keys 0..P (causal, inclusive);
* the scale is an explicit argument (1/sqrt(D) in every workload).

All arithmetic is float64 on torch CPU tensors.  Pools are indexed only
through :func:`gather_kv` and written only through :func:`reshape_and_cache`.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import torch

from .block_manager import slot_for


def _as_cpu_long(x) -> torch.Tensor:
    return torch.as_tensor(x).to("cpu", torch.int64)


def compute_slot_mapping(block_tables, seq_lens, query_start_loc,
                         block_size: int) -> torch.Tensor:
    """Slot of every query token: its sequence's last q_len positions.

    ``query_start_loc`` is ``[S+1]``; ``None`` means one query token per
    sequence (decode).  Returns int64 ``[T]``.
    """
    bt = _as_cpu_long(block_tables)
    lens = _as_cpu_long(seq_lens)
    S = lens.numel()
    qsl = (torch.arange(S + 1) if query_start_loc is None
           else _as_cpu_long(query_start_loc))
    out = torch.empty(int(qsl[-1]), dtype=torch.int64)
    for s in range(S):
        q_len = int(qsl[s + 1] - qsl[s])
        L = int(lens[s])
        for j in range(q_len):
            pos = L - q_len + j
            out[int(qsl[s]) + j] = slot_for(bt[s].tolist(), pos, block_size)
    return out


def reshape_and_cache(k_cache: torch.Tensor, v_cache: torch.Tensor,
                      key: torch.Tensor, value: torch.Tensor,
                      slot_mapping) -> Tuple[torch.Tensor, torch.Tensor]:
    """Return copies of the pools with token t's K/V stored at slot_mapping[t].

    ``key``/``value`` are ``[T, H_kv, D]``; pools as in the module docstring.
    Values are copied bit for bit.  Negative slots are skipped; two tokens
    aiming at one slot is an error.
    """
    k_out = k_cache.clone()
    v_out = v_cache.clone()
    B = k_cache.shape[2]
    slots = _as_cpu_long(slot_mapping).tolist()
    valid = [s for s in slots if s >= 0]
    assert len(set(valid)) == len(valid), "duplicate slot in slot_mapping"
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = divmod(slot, B)
        k_out[blk, :, off, :] = key[t]
        v_out[blk, :, :, off] = value[t]
    return k_out, v_out


def gather_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, table_row,
              length: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Materialise positions 0..length-1 of one sequence as ``[L, H_kv, D]``.

    Position p comes from block ``table_row[p // B]`` at offset ``p % B``.
    """
    B = k_cache.shape[2]
    pos = torch.arange(length)
    row = _as_cpu_long(table_row)
    blocks = row[pos // B]
    offs = pos % B
    K = k_cache[blocks, :, offs, :]                    # [L, H_kv, D]
    V = v_cache[blocks, :, :, offs]                    # [L, H_kv, D]
    return K, V


def attention(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
              positions: Sequence[int], scale: float) -> torch.Tensor:
    """Textbook causal softmax attention for one sequence, in float64.

    ``q`` is ``[n, H_q, D]`` (row j at absolute position ``positions[j]``),
    ``K``/``V`` are ``[L, H_kv, D]``.  Row j, head h attends to keys
    0..positions[j] of KV head h // (H_q / H_kv).
    """
    q = q.to(torch.float64)
    K = K.to(torch.float64)
    V = V.to(torch.float64)
    n, Hq, D = q.shape
    Hkv = K.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = torch.empty((n, Hq, D), dtype=torch.float64)
    for j in range(n):
        P = int(positions[j])
        for h in range(Hq):
            kvh = h // G
            z = scale * (K[:P + 1, kvh, :] @ q[j, h, :])    # [P+1]
            w = torch.exp(z - z.max())
            w = w / w.sum()
            out[j, h, :] = w @ V[:P + 1, kvh, :]
    return out


def paged_attention(q: torch.Tensor, k_cache: torch.Tensor,
                    v_cache: torch.Tensor, block_tables, seq_lens,
                    query_start_loc, scale: float,
                    seq_ids: Optional[Sequence[int]] = None,
                    rows: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Attention for packed query rows against each sequence's paged K/V.

    ``q`` is ``[T, H_q, D]``; sequence s owns rows
    ``query_start_loc[s] .. query_start_loc[s+1]-1`` (``None``: one row per
    sequence), which sit at positions ``L_s - q_len .. L_s - 1``.  Returns
    float64 ``[T, H_q, D]``.  When ``seq_ids`` and/or ``rows`` (packed row
    indices) are given, only those sequences / rows are computed and every
    other row is left as NaN.
    """
    lens = _as_cpu_long(seq_lens)
    S = lens.numel()
    qsl = (torch.arange(S + 1) if query_start_loc is None
           else _as_cpu_long(query_start_loc))
    bt = _as_cpu_long(block_tables)
    out = torch.full((q.shape[0], q.shape[1], q.shape[2]), math.nan,
                     dtype=torch.float64)
    wanted = None if rows is None else set(int(r) for r in rows)
    for s in (range(S) if seq_ids is None else seq_ids):
        r0, r1 = int(qsl[s]), int(qsl[s + 1])
        L = int(lens[s])
        q_len = r1 - r0
        picked = [r for r in range(r0, r1) if wanted is None or r in wanted]
        if not picked:
            continue
        K, V = gather_kv(k_cache, v_cache, bt[s], L)
        positions = [L - q_len + (r - r0) for r in picked]
        out[picked] = attention(q[picked], K, V, positions, scale)
    return out


def decode(q, k_cache, v_cache, block_tables, seq_lens, scale, seq_ids=None):
    """One query token per sequence, at position L_s - 1."""
    return paged_attention(q, k_cache, v_cache, block_tables, seq_lens, None,
                           scale, seq_ids=seq_ids)


def chunked_prefill(q, k_cache, v_cache, block_tables, seq_lens,
                    query_start_loc, scale, seq_ids=None, rows=None):
    """Query chunks (and single decode rows) against paged context."""
    return paged_attention(q, k_cache, v_cache, block_tables, seq_lens,
                           query_start_loc, scale, seq_ids=seq_ids, rows=rows)
