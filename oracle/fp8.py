"""FP8 (e4m3) KV cache, computed plainly on the CPU (oracle; test infrastructure only).

What the method computes, restated from the pages:

* K and V may be kept in the cache as 8-bit floats (e4m3), one byte per
  element instead of two, quantised per block ("Tech Radar: vLLM v1
  Production Engine Architecture & Distributed KV Cache Optimization",
  section "Hopper TMA Warp Specialization & FP8 Kernel Integration", item
  "FP8 Block-Quantized Caching"; "High-Throughput Local LLM Infrastructure
  ...", FAQ "Q5", memory footprint).  Attention then runs on the stored
  values scaled back.

Readings taken where the pages are silent:

* Format: e4m3 as the OCP 8-bit floating point specification defines it
  (the variant without infinities): sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; the codes
  0x7F and 0xFF are NaN; the largest finite magnitude is 448.
* Scale granularity: one float32 scale per (physical block, KV head), for K
  and for V separately ("block-quantized").  The pages do not say how a
  block's scale is chosen; the caller owns the scales (set, for example,
  when a block is allocated) and the cache write and attention only apply
  them.
* Quantisation of an element x (bf16 or fp32) with scale s: y = x / s
  computed in float32 (one correctly rounded division), clamped to
  [-448, 448], then rounded to the nearest e4m3 value, ties to the even code
  (even mantissa).  The sign of y is kept (a tiny negative y gives -0).
  Float32 is the precision the quantised code is decided in on both sides.
* Dequantisation: value(code) * s, exactly (in float64 here).

Pools are ``uint8`` tensors laid out like the bf16 pools (K ``[NB, H_kv, B,
D]``, V ``[NB, H_kv, D, B]``); scales are float32 ``[NB, H_kv]``.
"""

from __future__ import annotations

import math

import torch

from .paged_attention import _as_cpu_long, attention, gather_kv

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one e4m3 code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def decode_table() -> torch.Tensor:
    """float64 [256]: the value of every code."""
    return torch.tensor([e4m3_value(c) for c in range(256)], dtype=torch.float64)


def encode(y: torch.Tensor) -> torch.Tensor:
    """Round finite values with |y| <= 448 to e4m3 codes (uint8), nearest,
    ties to the even code; the sign bit follows the sign of y (also for 0)."""
    y = y.to(torch.float64).reshape(-1)
    assert torch.isfinite(y).all() and (y.abs() <= E4M3_MAX).all()
    pos = decode_table()[:127]                    # codes 0..126: 0 .. 448, increasing
    mag = y.abs()
    hi = torch.searchsorted(pos, mag).clamp(max=126)   # first value >= mag
    lo = (hi - 1).clamp(min=0)
    d_lo = mag - pos[lo]
    d_hi = pos[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = torch.where(pick_hi, hi, lo)
    code = torch.where(mag == pos[hi], hi, code)       # exact values
    sign = torch.signbit(y).to(torch.int64) << 7
    return (code | sign).to(torch.uint8)


def quantize(x: torch.Tensor, scale) -> torch.Tensor:
    """e4m3 codes of x / scale (float32 division, clamp to +-448, RNE)."""
    x32 = x.to(torch.float32)
    s32 = torch.as_tensor(scale, dtype=torch.float32)
    y = torch.clamp(x32 / s32, -E4M3_MAX, E4M3_MAX)
    return encode(y).reshape(x.shape)


def reshape_and_cache_fp8(k_cache: torch.Tensor, v_cache: torch.Tensor,
                          k_scales: torch.Tensor, v_scales: torch.Tensor,
                          key: torch.Tensor, value: torch.Tensor, slot_mapping):
    """Return copies of the uint8 pools with token t's K/V quantised into
    slot_mapping[t] with the scales of that (block, KV head).  Negative slots
    are skipped; two tokens aiming at one slot is an error."""
    k_out = k_cache.clone()
    v_out = v_cache.clone()
    B = k_cache.shape[2]
    H = k_cache.shape[1]
    slots = _as_cpu_long(slot_mapping).tolist()
    valid = [s for s in slots if s >= 0]
    assert len(set(valid)) == len(valid), "duplicate slot in slot_mapping"
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = divmod(slot, B)
        for h in range(H):
            k_out[blk, h, off, :] = quantize(key[t, h], k_scales[blk, h])
            v_out[blk, h, :, off] = quantize(value[t, h], v_scales[blk, h])
    return k_out, v_out


def dequantize_pool(cache: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """float64 pool: value(code) * scale of the element's (block, KV head)."""
    vals = decode_table()[cache.to(torch.int64)]
    s = scales.to(torch.float64)[:, :, None, None]
    return vals * s


def gather_dequantized(k_cache, v_cache, k_scales, v_scales, table_row, length):
    """Positions 0..length-1 of one sequence as float64 ``[L, H_kv, D]``:
    the codes gathered through the table, times their block's scale."""
    B = k_cache.shape[2]
    K8, V8 = gather_kv(k_cache, v_cache, table_row, length)
    pos = torch.arange(length)
    blocks = _as_cpu_long(table_row)[pos // B]
    table = decode_table()
    K = table[K8.to(torch.int64)] * k_scales.to(torch.float64)[blocks][:, :, None]
    V = table[V8.to(torch.int64)] * v_scales.to(torch.float64)[blocks][:, :, None]
    return K, V


def paged_attention_fp8(q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                        query_start_loc, scale, seq_ids=None, rows=None) -> torch.Tensor:
    """Paged attention over the dequantised values (float64); rows and
    sequences are chosen as in ``paged_attention`` (others stay NaN).  Each
    sequence is dequantised after its gather, which is the same arithmetic
    as dequantising the whole pools first."""
    lens = _as_cpu_long(seq_lens)
    S = lens.numel()
    qsl = (torch.arange(S + 1) if query_start_loc is None
           else _as_cpu_long(query_start_loc))
    bt = _as_cpu_long(block_tables)
    out = torch.full(tuple(q.shape), math.nan, dtype=torch.float64)
    wanted = None if rows is None else set(int(r) for r in rows)
    for s in (range(S) if seq_ids is None else seq_ids):
        r0, r1 = int(qsl[s]), int(qsl[s + 1])
        L = int(lens[s])
        picked = [r for r in range(r0, r1) if wanted is None or r in wanted]
        if not picked:
            continue
        K, V = gather_dequantized(k_cache, v_cache, k_scales, v_scales, bt[s], L)
        positions = [L - (r1 - r0) + (r - r0) for r in picked]
        out[picked] = attention(q[picked], K, V, positions, scale)
    return out


def decode_fp8(q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, scale,
               seq_ids=None):
    """One query token per sequence against the fp8 pools."""
    return paged_attention_fp8(q, k_cache, v_cache, k_scales, v_scales, block_tables,
                               seq_lens, None, scale, seq_ids=seq_ids)
