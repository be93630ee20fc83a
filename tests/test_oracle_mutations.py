"""Planted mistakes in the oracle must fail its pins.

Each case swaps one oracle function for a plausibly wrong version (on the
CPU, through monkeypatch) and checks that at least one pin -- brute force or
the float64 library reduction -- now disagrees.  This shows the pins are
strong enough to catch a dropped term, a wrong index or a transposed operand.
"""
import math

import pytest
import torch

from oracle import paged_attention as pa
from tests.test_oracle_attention import _brute_force, _dense_case, _sdpa


def _pins_pass():
    ok = True
    lens, q_lens = [12, 10, 33, 9], [1, 2, 1, 3]
    dk, dv, kc, vc, bt, q, qsl = _dense_case(lens, q_lens, 4, 2, 8, 4, 11, shared_prefix=4)
    got = pa.chunked_prefill(q, kc, vc, bt, lens, qsl, 0.35)
    ok &= bool(torch.allclose(got, _brute_force(dk, dv, q, qsl, lens, 0.35), atol=1e-12))
    lens, q_lens = [130, 47], [1, 20]
    dk, dv, kc, vc, bt, q, qsl = _dense_case(lens, q_lens, 8, 2, 16, 16, 2)
    got = pa.chunked_prefill(q, kc, vc, bt, lens, qsl, 0.2)
    ok &= bool(torch.allclose(got, _sdpa(q, dk, dv, qsl, lens, 0.2), atol=1e-12))
    return ok


def _gather_swapped_offset(k_cache, v_cache, table_row, length):
    B = k_cache.shape[2]
    pos = torch.arange(length)
    row = torch.as_tensor(table_row).long()
    blocks = row[pos // B]
    offs = (B - 1) - pos % B                  # reversed offset inside a block
    return k_cache[blocks, :, offs, :], v_cache[blocks, :, :, offs]


def _gather_v_from_k_layout(k_cache, v_cache, table_row, length):
    B = k_cache.shape[2]
    pos = torch.arange(length)
    row = torch.as_tensor(table_row).long()
    blocks = row[pos // B]
    offs = pos % B
    Vt = v_cache.transpose(2, 3)              # reads V as if it were token-major
    return k_cache[blocks, :, offs, :], Vt.reshape(v_cache.shape)[blocks, :, :, offs]


def _attention_factory(kind):
    orig = pa.attention

    def f(q, K, V, positions, scale):
        if kind == "no_scale":
            return orig(q, K, V, positions, 1.0)
        if kind == "off_by_one":
            return orig(q, K, V, [p - 1 if p > 0 else p for p in positions], scale)
        if kind == "interleaved_gqa":
            idx = torch.arange(q.shape[1]) % K.shape[1]   # h -> KV head h mod H_kv
            return orig(q, K[:, idx], V[:, idx], positions, scale)
        raise ValueError(kind)
    return f


def test_unmodified_oracle_passes():
    assert _pins_pass()


@pytest.mark.parametrize("mutation", [
    ("gather_kv", _gather_swapped_offset),
    ("gather_kv", _gather_v_from_k_layout),
    ("attention", _attention_factory("no_scale")),
    ("attention", _attention_factory("off_by_one")),
    ("attention", _attention_factory("interleaved_gqa")),
])
def test_planted_mistake_fails_a_pin(monkeypatch, mutation):
    name, fn = mutation
    monkeypatch.setattr(pa, name, fn)
    assert not _pins_pass()


def test_planted_cache_write_mistake_fails_brute_force(monkeypatch):
    orig = pa.reshape_and_cache

    def bad(k_cache, v_cache, key, value, slot_mapping):
        k, v = orig(k_cache, v_cache, key, value, slot_mapping)
        return k, v.flip(-1)                  # tokens of each V row reversed
    monkeypatch.setattr(pa, "reshape_and_cache", bad)
    assert not _pins_pass()
