"""The random shapes of the GPU fuzz cases (tests/test_gpu_fuzz.py) reach
what they are meant to: both head_dims on every path, both kinds of batch,
odd group sizes, and an oracle cost within the cap.  CPU only."""
from tests.test_gpu_fuzz import MAX_ORACLE_MACS, N_CASES, draw, draw_shared

KINDS = ("bf16", "f32", "fp8", "fp8chunk", "append", "append8")


def test_fuzz_draws_are_reproducible():
    for kind in KINDS:
        for i in range(N_CASES):
            assert draw(kind, i) == draw(kind, i)


def test_fuzz_draws_cover_the_shapes():
    seen = set()
    for kind in KINDS:
        for i in range(N_CASES):
            Hq, Hkv, D, B, lens, qls = draw(kind, i)
            G = Hq // Hkv
            assert Hq % Hkv == 0 and 1 <= G <= 16 and len(lens) == len(qls)
            assert all(1 <= q <= L for q, L in zip(qls, lens))
            assert sum(q * L for q, L in zip(qls, lens)) * Hq * D <= MAX_ORACLE_MACS
            seen.add((kind, "D", D))
            seen.add((kind, "chunked", max(qls) > 1))
            seen.add(("G odd", G % 2 == 1 and G > 1))
            seen.add((kind, "B", B))
    for kind in KINDS:
        assert (kind, "D", 64) in seen and (kind, "D", 128) in seen, kind
    assert ("bf16", "chunked", True) in seen and ("bf16", "chunked", False) in seen
    assert ("f32", "chunked", True) in seen and ("f32", "chunked", False) in seen
    assert ("fp8", "chunked", True) not in seen            # e4m3 decode: single-token rows
    assert ("append", "chunked", True) not in seen         # appending decode: one new token
    assert ("append8", "chunked", True) not in seen
    assert ("fp8chunk", "chunked", False) not in seen      # every e4m3 chunked case has a chunk
    assert ("G odd", True) in seen
    for B in (8, 16, 32, 64):
        assert ("bf16", "B", B) in seen, B
    for B in (1, 4):
        assert ("f32", "B", B) in seen, B


def test_shared_prefix_draws():
    seen = set()
    for fp8 in (False, True):
        for i in range(N_CASES):
            Hq, Hkv, D, B, prefix, lens = draw_shared(fp8, i)
            assert draw_shared(fp8, i) == (Hq, Hkv, D, B, prefix, lens)
            assert prefix % B == 0 and prefix >= B and min(lens) > prefix
            assert sum(lens) * Hq * D <= MAX_ORACLE_MACS
            step = 64 if fp8 else 32
            seen.add((fp8, "D", D))
            seen.add((fp8, "prefix under a step", prefix < step))
            seen.add((fp8, "one sequence", len(lens) == 1))
            seen.add((fp8, "many", len(lens) >= 16))
    for fp8 in (False, True):
        assert (fp8, "D", 64) in seen and (fp8, "D", 128) in seen
        assert (fp8, "many", True) in seen
