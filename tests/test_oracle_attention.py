"""Pins of the oracle's paged attention (oracle/paged_attention.py).

Attention is softmax(q K^T / sqrt(d)) V over a sequence's past keys ("03 --
PagedAttention & the vLLM V1 Architecture", section "The attention kernel
side"); paging only moves where K and V live.  The oracle is checked against
things other than itself:

* brute force: scalar Python loops over dense per-position K/V that never
  went through a pool, on tiny cases whose pools were filled through the
  allocator's slots and the oracle's cache write;
* torch's scaled_dot_product_attention in float64 (a library routine the
  definition reduces to once heads are expanded and the causal offset is
  written as a mask);
* closed forms: one key gives its value exactly; equal logits give the mean
  of the values; a dominant needle key gives its value;
* invariance of the result under any relabelling of physical blocks.
"""
import math
import random

import pytest
import torch

from oracle import paged_attention as pa
from oracle.block_manager import BlockManager
from paged_kv_cache_19_amd import workloads


def _dense_case(lens, q_lens, Hq, Hkv, D, B, seed, shared_prefix=0, extra_blocks=7):
    """Dense per-position K/V and q, plus a pool filled via the allocator."""
    g = torch.Generator().manual_seed(seed)
    S = len(lens)
    dense_k = [torch.randn(L, Hkv, D, generator=g, dtype=torch.float64) for L in lens]
    dense_v = [torch.randn(L, Hkv, D, generator=g, dtype=torch.float64) for L in lens]
    if shared_prefix:
        for s in range(1, S):
            dense_k[s][:shared_prefix] = dense_k[0][:shared_prefix]
            dense_v[s][:shared_prefix] = dense_v[0][:shared_prefix]
    nb = sum(-(-L // B) for L in lens) + extra_blocks
    order = list(range(nb))
    random.Random(seed).shuffle(order)
    bm = BlockManager(order, B)
    kc = torch.full((nb, Hkv, B, D), math.nan, dtype=torch.float64)
    vc = torch.full((nb, Hkv, D, B), math.nan, dtype=torch.float64)
    slots_all, keys, vals = [], [], []
    bm.add_sequence(0)
    for p in range(shared_prefix):
        slots_all.append(bm.append_token(0)); keys.append(dense_k[0][p]); vals.append(dense_v[0][p])
    for s in range(1, S):
        if shared_prefix:
            bm.fork(0, s)
        else:
            bm.add_sequence(s)
    for s in range(S):
        for p in range(shared_prefix, lens[s]):
            slots_all.append(bm.append_token(s)); keys.append(dense_k[s][p]); vals.append(dense_v[s][p])
    kc, vc = pa.reshape_and_cache(kc, vc, torch.stack(keys), torch.stack(vals), slots_all)
    maxb = max(len(bm.table(s)) for s in range(S)) + 1
    bt = torch.full((S, maxb), order[-1], dtype=torch.int64)
    for s in range(S):
        bt[s, :len(bm.table(s))] = torch.tensor(bm.table(s))
    T = sum(q_lens)
    q = torch.randn(T, Hq, D, generator=g, dtype=torch.float64)
    qsl = [0]
    for n in q_lens:
        qsl.append(qsl[-1] + n)
    return dense_k, dense_v, kc, vc, bt, q, qsl


def _brute_force(dense_k, dense_v, q, qsl, lens, scale):
    T, Hq, D = q.shape
    Hkv = dense_k[0].shape[1]
    G = Hq // Hkv
    out = torch.zeros(T, Hq, D, dtype=torch.float64)
    for s in range(len(lens)):
        qn = qsl[s + 1] - qsl[s]
        for j in range(qn):
            P = lens[s] - qn + j
            for h in range(Hq):
                kv = h // G
                logits = []
                for t in range(P + 1):
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[qsl[s] + j, h, d]) * float(dense_k[s][t, kv, d])
                    logits.append(acc * scale)
                mx = max(logits)
                ws = [math.exp(x - mx) for x in logits]
                tot = sum(ws)
                for d in range(D):
                    out[qsl[s] + j, h, d] = sum(ws[t] * float(dense_v[s][t, kv, d]) for t in range(P + 1)) / tot
    return out


@pytest.mark.parametrize("case", [
    dict(lens=[12, 10, 33, 9], q_lens=[1, 1, 1, 1], Hq=4, Hkv=2, D=8, B=4, prefix=4),
    dict(lens=[7, 20], q_lens=[3, 5], Hq=6, Hkv=2, D=5, B=2, prefix=0),
    dict(lens=[1, 17, 16], q_lens=[1, 17, 2], Hq=2, Hkv=1, D=4, B=8, prefix=0),
])
def test_brute_force(case):
    dk, dv, kc, vc, bt, q, qsl = _dense_case(case["lens"], case["q_lens"], case["Hq"],
                                             case["Hkv"], case["D"], case["B"], 11,
                                             shared_prefix=case["prefix"])
    scale = 1 / math.sqrt(case["D"])
    ref = _brute_force(dk, dv, q, qsl, case["lens"], scale)
    got = pa.chunked_prefill(q, kc, vc, bt, case["lens"], qsl, scale)
    assert torch.allclose(got, ref, rtol=0, atol=1e-12)


def _sdpa(q, dense_k, dense_v, qsl, lens, scale):
    T, Hq, D = q.shape
    out = torch.empty(T, Hq, D, dtype=torch.float64)
    for s, L in enumerate(lens):
        qs = q[qsl[s]:qsl[s + 1]]
        n = qs.shape[0]
        G = Hq // dense_k[s].shape[1]
        K = dense_k[s].repeat_interleave(G, dim=1).permute(1, 0, 2)   # [Hq, L, D]
        V = dense_v[s].repeat_interleave(G, dim=1).permute(1, 0, 2)
        rowpos = torch.arange(L - n, L).unsqueeze(1)
        mask = torch.arange(L).unsqueeze(0) <= rowpos               # [n, L]
        o = torch.nn.functional.scaled_dot_product_attention(
            qs.permute(1, 0, 2), K, V, attn_mask=mask, scale=scale)
        out[qsl[s]:qsl[s + 1]] = o.permute(1, 0, 2)
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_matches_torch_sdpa_float64(seed):
    lens = [130, 47, 300, 16]
    q_lens = [1, 20, 64, 16]
    dk, dv, kc, vc, bt, q, qsl = _dense_case(lens, q_lens, 8, 2, 32, 16, seed)
    got = pa.chunked_prefill(q, kc, vc, bt, lens, qsl, 0.17)
    ref = _sdpa(q, dk, dv, qsl, lens, 0.17)
    assert torch.allclose(got, ref, rtol=0, atol=1e-12)


def test_gqa_grouping_is_contiguous():
    """Query head h reads KV head h // G: with KV head 1 zeroed in V, query
    heads G..2G-1 give exactly zero and heads 0..G-1 do not."""
    lens = [9]
    dk, dv, kc, vc, bt, q, qsl = _dense_case(lens, [1], 4, 2, 8, 4, 3)
    vc = vc.clone()
    vc[:, 1] = 0.0
    out = pa.decode(q, kc, vc, bt, lens, 0.3)
    assert torch.all(out[0, 2:] == 0)
    assert torch.all(out[0, :2].abs().sum(-1) > 0)


def test_single_key_returns_its_value():
    dk, dv, kc, vc, bt, q, qsl = _dense_case([1, 1], [1, 1], 4, 2, 16, 4, 5)
    out = pa.decode(q, kc, vc, bt, [1, 1], 0.25)
    for s in range(2):
        for h in range(4):
            assert torch.equal(out[s, h], dv[s][0, h // 2])


def test_zero_query_gives_mean_of_values():
    dk, dv, kc, vc, bt, q, qsl = _dense_case([23], [1], 2, 1, 8, 4, 6)
    q = torch.zeros_like(q)
    out = pa.decode(q, kc, vc, bt, [23], 0.5)
    assert torch.allclose(out[0, 0], dv[0][:, 0].mean(0), atol=1e-14)


def test_needle_key_dominates():
    dk, dv, kc, vc, bt, q, qsl = _dense_case([40], [1], 1, 1, 8, 4, 7)
    # make key 17 parallel to q with a huge logit: weight ~ 1 on value 17
    B = 4
    blk = int(bt[0, 17 // B])
    kc = kc.clone()
    kc[blk, 0, 17 % B] = q[0, 0] * 1e3
    out = pa.decode(q, kc, vc, bt, [40], 1.0)
    assert torch.allclose(out[0, 0], dv[0][17, 0], atol=1e-9)


def test_causal_row_limits():
    """Row j of a chunk sees exactly keys 0..L-q_len+j: changing key P+1 leaves
    row j unchanged and changes row j+1."""
    lens, q_lens = [20], [6]
    dk, dv, kc, vc, bt, q, qsl = _dense_case(lens, q_lens, 2, 1, 8, 4, 8)
    base = pa.chunked_prefill(q, kc, vc, bt, lens, qsl, 0.3)
    B = 4
    for j in range(5):
        P = 20 - 6 + j
        vc2 = vc.clone()
        vc2[int(bt[0, (P + 1) // B]), :, :, (P + 1) % B] += 5.0
        out = pa.chunked_prefill(q, kc, vc2, bt, lens, qsl, 0.3)
        assert torch.equal(out[j], base[j])
        assert not torch.equal(out[j + 1], base[j + 1])


def test_block_relabelling_is_exactly_invariant():
    wl = workloads.make_workload(5, seq_lens=[37, 64, 5], q_lens=[4, 1, 5],
                                 shape=workloads.Shape("t", "f32", 4, 2, 16, 8))
    t = wl.tensors
    bt = wl.block_tables_tensor()
    qsl = wl.query_start_loc()
    ref = pa.chunked_prefill(t["query"], t["k_cache"], t["v_cache"], bt, wl.seq_lens, qsl, wl.scale)
    perm = torch.randperm(wl.num_blocks, generator=torch.Generator().manual_seed(3))
    kc = torch.empty_like(t["k_cache"]); vc = torch.empty_like(t["v_cache"])
    kc[perm] = t["k_cache"]; vc[perm] = t["v_cache"]
    out = pa.chunked_prefill(t["query"], kc, vc, perm[bt.long()], wl.seq_lens, qsl, wl.scale)
    assert torch.equal(out, ref)


def test_slot_mapping_of_decode_and_chunks():
    bt = torch.tensor([[42, 108, 17], [5, 6, 7]])
    slots = pa.compute_slot_mapping(bt, [40, 33], [0, 3, 5], 16)
    # seq 0: positions 37..39 in logical block 2 (id 17); seq 1: 31, 32
    assert slots.tolist() == [17 * 16 + 5, 17 * 16 + 6, 17 * 16 + 7, 6 * 16 + 15, 7 * 16 + 0]
    assert pa.compute_slot_mapping(bt, [1, 48], None, 16).tolist() == [42 * 16, 7 * 16 + 15]


def test_cache_write_is_a_bit_copy_and_skips_negative_slots():
    NB, H, B, D = 4, 2, 4, 3
    kc = torch.full((NB, H, B, D), math.nan, dtype=torch.bfloat16)
    vc = torch.full((NB, H, D, B), math.nan, dtype=torch.bfloat16)
    key = torch.randn(3, H, D).to(torch.bfloat16)
    val = torch.randn(3, H, D).to(torch.bfloat16)
    k2, v2 = pa.reshape_and_cache(kc, vc, key, val, [9, -1, 2])
    assert torch.equal(k2[2, :, 1, :].view(torch.int16), key[0].view(torch.int16))
    assert torch.equal(v2[2, :, :, 1].view(torch.int16), val[0].view(torch.int16))
    assert torch.equal(k2[0, :, 2, :].view(torch.int16), key[2].view(torch.int16))
    assert torch.equal(v2[0, :, :, 2].view(torch.int16), val[2].view(torch.int16))
    written = torch.zeros(NB, B, dtype=torch.bool)
    written[2, 1] = written[0, 2] = True
    assert torch.isnan(k2.float().permute(0, 2, 1, 3)[~written]).all()
    with pytest.raises(AssertionError):
        pa.reshape_and_cache(kc, vc, key, val, [9, 9, 2])
