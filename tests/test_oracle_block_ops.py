"""Pins of the whole-block copy / swap oracle (``oracle/block_ops.py``).

* The walkthrough of "03 -- PagedAttention & the vLLM V1 Architecture"
  (section "The block table walkthrough"), replayed with real K/V values:
  with copy-on-write done by ``copy_blocks_in_pool`` (whole block), every
  position of both sequences reads back the value that was written for it.
* A swap round trip (blocks out to a host pool, back into other device
  blocks, table rewritten) leaves every sequence's gathered K/V unchanged.
* Brute force over every element: destination blocks equal their sources,
  all other blocks are untouched.
Planted mistakes (destination off by one, source and destination swapped,
only the first half of a block copied) must fail.
"""
import pytest
import torch

import oracle.block_ops as bo
from oracle import paged_attention as pa
from oracle.block_manager import BlockManager


def _walkthrough_values(copy_fn):
    B, H, D = 4, 2, 3
    g = torch.Generator().manual_seed(2)
    k_pool = torch.full((16, H, B, D), float("nan"))
    v_pool = torch.full((16, H, D, B), float("nan"))
    pools = {"k": k_pool, "v": v_pool}

    def hook(src, dst, n_valid):
        m = torch.tensor([[src, dst]])
        pools["k"] = copy_fn(pools["k"], m)
        pools["v"] = copy_fn(pools["v"], m)

    bm = BlockManager(range(16), B, copy_hook=hook)
    written = {0: [], 1: []}

    def write(seq, n):
        for _ in range(n):
            slot = bm.append_token(seq)
            kv = torch.randn(2, 1, H, D, generator=g)
            pools["k"], pools["v"] = pa.reshape_and_cache(pools["k"], pools["v"], kv[0], kv[1],
                                                          torch.tensor([slot]))
            written[seq].append(kv)

    bm.add_sequence(0)
    write(0, 6)
    bm.fork(0, 1)
    written[1] = list(written[0])
    write(1, 1)
    write(0, 3)
    write(1, 2)
    write(0, 3)
    write(1, 1)
    assert bm.table(0) == [0, 1, 3] and bm.table(1) == [0, 2, 4]   # the page's tables
    ok = True
    for seq in (0, 1):
        K, V = pa.gather_kv(pools["k"], pools["v"], bm.table(seq), len(written[seq]))
        for p, kv in enumerate(written[seq]):
            ok &= torch.equal(K[p], kv[0, 0]) and torch.equal(V[p], kv[1, 0])
    return ok


def test_walkthrough_copy_on_write_keeps_every_token():
    assert _walkthrough_values(bo.copy_blocks_in_pool)


def test_swap_round_trip_preserves_sequences():
    g = torch.Generator().manual_seed(4)
    NB, H, B, D = 10, 2, 4, 8
    kc = torch.randn(NB, H, B, D, generator=g).to(torch.bfloat16)
    vc = torch.randn(NB, H, D, B, generator=g).to(torch.bfloat16)
    table, L = [7, 2, 5], 11
    host_k = torch.zeros(6, H, B, D, dtype=torch.bfloat16)
    host_v = torch.zeros(6, H, D, B, dtype=torch.bfloat16)
    out_map = torch.tensor([[7, 3], [2, 0], [5, 4]])
    host_k = bo.copy_blocks(host_k, kc, out_map)
    host_v = bo.copy_blocks(host_v, vc, out_map)
    kc2 = torch.full_like(kc, float("nan"))
    vc2 = torch.full_like(vc, float("nan"))
    in_map = torch.tensor([[3, 1], [0, 8], [4, 6]])
    kc2 = bo.copy_blocks(kc2, host_k, in_map)
    vc2 = bo.copy_blocks(vc2, host_v, in_map)
    K0, V0 = pa.gather_kv(kc, vc, table, L)
    K1, V1 = pa.gather_kv(kc2, vc2, [1, 8, 6], L)
    assert torch.equal(K0, K1) and torch.equal(V0, V1)


def _brute_ok(fn):
    g = torch.Generator().manual_seed(6)
    src = torch.randn(9, 2, 3, generator=g)
    dst = torch.randn(7, 2, 3, generator=g)
    m = torch.tensor([[8, 0], [1, 6], [4, 3]])
    got = fn(dst, src, m)
    want = dst.clone()
    pairs = {0: 8, 6: 1, 3: 4}
    for b in range(7):
        for i in range(2):
            for j in range(3):
                want[b, i, j] = src[pairs[b], i, j] if b in pairs else dst[b, i, j]
    return torch.equal(got, want)


def test_copy_matches_brute_force():
    assert _brute_ok(bo.copy_blocks)


def test_rejects_overlapping_mappings():
    pool = torch.zeros(4, 2)
    with pytest.raises(AssertionError):
        bo.copy_blocks(pool, pool, torch.tensor([[0, 1], [2, 1]]))
    with pytest.raises(AssertionError):
        bo.copy_blocks_in_pool(pool, torch.tensor([[0, 1], [1, 2]]))


def _dst_off_by_one(dst_pool, src_pool, m, same_pool=False):
    m = torch.as_tensor(m).reshape(-1, 2).clone()
    m[:, 1] = (m[:, 1] + 1) % dst_pool.shape[0]
    return _orig(dst_pool, src_pool, m)


def _swapped_roles(dst_pool, src_pool, m, same_pool=False):
    # reads the first column of each pair as the destination
    out = dst_pool.clone()
    for s, d in torch.as_tensor(m).reshape(-1, 2).tolist():
        if s < dst_pool.shape[0] and d < src_pool.shape[0]:
            out[s] = src_pool[d]
    return out


def _half_block(dst_pool, src_pool, m, same_pool=False):
    out = dst_pool.clone()
    for s, d in torch.as_tensor(m).reshape(-1, 2).tolist():
        n = out[d].numel() // 2
        out[d].view(-1)[:n] = src_pool[s].reshape(-1)[:n]
    return out


_orig = bo.copy_blocks


@pytest.mark.parametrize("bad", [_dst_off_by_one, _swapped_roles, _half_block])
def test_planted_copy_mistake_fails(monkeypatch, bad):
    monkeypatch.setattr(bo, "copy_blocks", bad)
    ok = _brute_ok(bo.copy_blocks)
    try:
        ok = ok and _walkthrough_values(lambda p, m: bo.copy_blocks(p, p, m))
    except (AssertionError, IndexError):
        ok = False
    assert not ok
