"""Pins of the closed forms in oracle/sizes.py to the numbers the pages print."""
import json
import math
import os
from fractions import Fraction

import pytest

from oracle import sizes
from tests.conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_blocks_for_a_2048_token_prompt():
    g = _load("sizing.json")["blocks_for_prompt"]
    assert sizes.num_blocks(g["prompt_tokens"], g["block_size"]) == g["printed_blocks"]


def test_kv_bytes_per_sequence_70b_fp8():
    g = _load("sizing.json")["kv_per_sequence"]
    b = sizes.kv_bytes(g["ctx"], g["layers"], g["kv_heads"], g["head_dim"], g["elem_bytes"])
    assert b == 2 * 80 * 8 * 128 * 8192
    assert round(b / 1e9, 2) == g["printed_gb"]


def test_concurrency_bound_and_weights():
    g = _load("sizing.json")
    c = g["concurrency"]
    assert sizes.max_concurrency(c["total_vram_gb"], c["weights_gb"], c["kv_per_seq_gb"]) == c["printed_max_seqs"]
    w = g["weights"]
    assert math.isclose(w["params_billion"] * w["bytes_per_param"] * w["overhead"], w["printed_gb"])


def test_tail_block_example():
    g = _load("tail_block_example.json")
    B, S = g["block_size"], g["seq_len"]
    nb = sizes.num_blocks(S, B)
    assert nb == len(g["physical_blocks"])
    assert S - (nb - 1) * B == g["last_block_valid_tokens"]
    assert nb * B - S == g["last_block_free_slots"]
    frac = sizes.internal_fragmentation(S, B)
    assert frac == Fraction(28, 96)
    assert math.floor(float(frac) * 1000) / 10 == g["printed_waste_percent"]
    be = g["bound_example"]
    assert math.floor(be["block_size"] / be["seq_len"] * 1e4) / 100 == be["printed_bound_percent"]


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64])
def test_fragmentation_bound_holds_for_every_length(B):
    for S in range(1, 700):
        f = sizes.internal_fragmentation(S, B)
        assert 0 <= f < Fraction(B, S)
        if S % B == 0:
            assert f == 0


def test_paged_bytes_equal_token_bytes_when_aligned_and_exceed_otherwise():
    for S in range(1, 300):
        tok = sizes.kv_bytes(S, 2, 8, 128, 2)
        paged = sizes.paged_bytes(S, 2, 8, 128, 16, 2)
        assert paged >= tok
        assert (paged == tok) == (S % 16 == 0)
        assert paged - tok == (sizes.num_blocks(S, 16) * 16 - S) * 2 * 2 * 8 * 128 * 2


def test_block_bytes_is_two_k_and_v_times_elements():
    assert sizes.block_bytes(1, 8, 128, 16, 2) == 2 * 8 * 128 * 16 * 2 == 65536
