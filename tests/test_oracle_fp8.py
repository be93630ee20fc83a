"""Pins for the FP8 (e4m3) KV-cache oracle (``oracle/fp8.py``).

The oracle's format, rounding and scale handling are pinned to things other
than itself:

* code values worked out by hand from the OCP e4m3 definition (bias 7,
  subnormals m * 2^-9, 0x7F/0xFF NaN, largest finite 448);
* the library routine ``torch.float8_e4m3fn`` (decode of every code, and
  round-to-nearest-even encode of a million values);
* hand-computed ties (to the even code), saturation and division by the
  scale;
* a brute-force cache write that picks, for every element, the nearest of
  all 256 codes by scanning them, and a brute-force attention over the
  dequantised values.

Planted mistakes (ties away from zero, a missing clamp, multiplying by the
scale, the K scale used for V, scales indexed by the wrong block) must each
fail one of these pins.
"""
import math

import pytest
import torch

import oracle.fp8 as f8
from tests.test_oracle_attention import _brute_force

# (code, value) from the definition: sign | exponent (bias 7) | mantissa.
HAND = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0),
    (0x4C, 6.0), (0x77, 240.0), (0x78, 256.0), (0x7D, 416.0), (0x7E, 448.0),
    (0x80, -0.0), (0xB8, -1.0), (0xFE, -448.0),
]


def test_code_values_from_the_format_definition():
    for code, val in HAND:
        got = f8.e4m3_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)
    assert math.isnan(f8.e4m3_value(0x7F)) and math.isnan(f8.e4m3_value(0xFF))


def test_decode_table_matches_the_library_type():
    t = f8.decode_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double()
    nan = torch.isnan(ref)
    assert torch.equal(torch.isnan(t), nan)
    assert torch.equal(t[~nan], ref[~nan])
    assert torch.equal(torch.signbit(t[~nan]), torch.signbit(ref[~nan]))
    pos = t[:127]
    assert bool((pos[1:] > pos[:-1]).all()) and pos[-1] == f8.E4M3_MAX


@pytest.mark.parametrize("y,code", [
    (1.0625, 0x38),        # halfway 1.0 / 1.125 -> even mantissa (1.0)
    (1.1875, 0x3A),        # halfway 1.125 / 1.25 -> 1.25
    (2.0 ** -10, 0x00),    # halfway 0 / 2^-9 -> 0
    (3 * 2.0 ** -10, 0x02),  # halfway 2^-9 / 2^-8 -> 2^-8
    (5 * 2.0 ** -10, 0x02),  # halfway 2*2^-9 / 3*2^-9 -> even (2)
    (432.0, 0x7E),         # halfway 416 / 448 -> 448
    (4.8, 0x4A),           # nearest: 5.0 (not 4.5)
    (-2.0 ** -11, 0x80),   # rounds to zero, keeps the sign
    (-0.0, 0x80),
    (448.0, 0x7E),
])
def test_encode_rounds_to_nearest_even(y, code):
    assert int(f8.encode(torch.tensor([y], dtype=torch.float64))[0]) == code


def test_encode_matches_the_library_cast():
    g = torch.Generator().manual_seed(5)
    x = torch.cat([torch.randn(1 << 20, generator=g) * 40,
                   torch.exp2(torch.linspace(-13, 8.8, 4001))]).clamp(-448, 448)
    assert torch.equal(f8.encode(x), x.to(torch.float8_e4m3fn).view(torch.uint8))
    vals = f8.decode_table()[:127]
    assert torch.equal(f8.encode(vals), torch.arange(127, dtype=torch.uint8))  # exact values


@pytest.mark.parametrize("x,s,code", [
    (3.0, 0.5, 0x4C),          # 6.0
    (0.3, 2.0 ** -4, 0x4A),    # 4.8 -> 5.0
    (1000.0, 1.0, 0x7E),       # saturates at 448
    (-1000.0, 1.0, 0xFE),
    (1.0, 1.0 / 448, 0x7E),
    (-0.0, 0.25, 0x80),
])
def test_quantize_divides_by_the_scale_and_saturates(x, s, code):
    assert int(f8.quantize(torch.tensor([x]), s)[0]) == code


def _nearest_code_brute(y: float) -> int:
    """Scan all finite codes of y's sign; nearest value, ties to even code."""
    best, best_d = None, None
    for c in range(256):
        v = f8.e4m3_value(c)
        if math.isnan(v) or math.copysign(1, v) != math.copysign(1, y):
            continue
        d = abs(v - y)
        if best is None or d < best_d or (d == best_d and c % 2 == 0 and best % 2 == 1):
            best, best_d = c, d
    return best


def _tiny_fp8_case(seed=3, NB=6, H=2, B=4, D=8, T=5):
    g = torch.Generator().manual_seed(seed)
    k_cache = torch.full((NB, H, B, D), 0x7F, dtype=torch.uint8)  # NaN poison
    v_cache = torch.full((NB, H, D, B), 0x7F, dtype=torch.uint8)
    ks = (torch.rand(NB, H, generator=g) * 0.05 + 0.005).float()
    vs = (torch.rand(NB, H, generator=g) * 0.05 + 0.005).float()
    key = (torch.randn(T, H, D, generator=g) * 3).to(torch.bfloat16)
    value = (torch.randn(T, H, D, generator=g) * 3).to(torch.bfloat16)
    slots = torch.tensor([5, 0, -1, 22, 13])
    return k_cache, v_cache, ks, vs, key, value, slots


def _fp8_pins_pass():
    k_cache, v_cache, ks, vs, key, value, slots = _tiny_fp8_case()
    B = k_cache.shape[2]
    kq, vq = f8.reshape_and_cache_fp8(k_cache, v_cache, ks, vs, key, value, slots)
    ek, ev = k_cache.clone(), v_cache.clone()
    for t, slot in enumerate(slots.tolist()):
        if slot < 0:
            continue
        blk, off = divmod(slot, B)
        for h in range(k_cache.shape[1]):
            for d in range(k_cache.shape[3]):
                yk = float(torch.tensor(float(key[t, h, d]), dtype=torch.float32)
                           / torch.tensor(float(ks[blk, h]), dtype=torch.float32))
                yv = float(torch.tensor(float(value[t, h, d]), dtype=torch.float32)
                           / torch.tensor(float(vs[blk, h]), dtype=torch.float32))
                ek[blk, h, off, d] = _nearest_code_brute(max(-448.0, min(448.0, yk)))
                ev[blk, h, d, off] = _nearest_code_brute(max(-448.0, min(448.0, yv)))
    ok = torch.equal(kq, ek) and torch.equal(vq, ev)
    # attention over the dequantised pools == brute force on hand-dequantised K/V
    lens, bt = [6, 3], torch.tensor([[1, 3], [5, 0]])
    q = torch.randn(2, 4, 8, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    kq2 = kq.clone()
    vq2 = vq.clone()
    kq2[kq2 == 0x7F] = 0x3A   # give the unwritten slots finite codes
    vq2[vq2 == 0x7F] = 0x31
    dk, dv = [], []
    for s, L in enumerate(lens):
        k_s = torch.zeros(L, 2, 8, dtype=torch.float64)
        v_s = torch.zeros_like(k_s)
        for p in range(L):
            blk, off = int(bt[s, p // B]), p % B
            for h in range(2):
                for d in range(8):
                    k_s[p, h, d] = f8.e4m3_value(int(kq2[blk, h, off, d])) * float(ks[blk, h])
                    v_s[p, h, d] = f8.e4m3_value(int(vq2[blk, h, d, off])) * float(vs[blk, h])
        dk.append(k_s)
        dv.append(v_s)
    qsl = [0, 1, 2]
    got = f8.paged_attention_fp8(q, kq2, vq2, ks, vs, bt, lens, qsl, 0.3)
    ok = ok and bool(torch.allclose(got, _brute_force(dk, dv, q, qsl, lens, 0.3), atol=1e-12))
    return ok


def test_cache_write_and_attention_match_brute_force():
    assert _fp8_pins_pass()


def _encode_ties_away(y):
    y = y.to(torch.float64).reshape(-1)
    pos = f8.decode_table()[:127]
    mag = y.abs()
    hi = torch.searchsorted(pos, mag).clamp(max=126)
    lo = (hi - 1).clamp(min=0)
    code = torch.where((pos[hi] - mag) <= (mag - pos[lo]), hi, lo)
    return (code | (torch.signbit(y).long() << 7)).to(torch.uint8)


def _quantize_no_clamp(x, scale):
    y = x.to(torch.float32) / torch.as_tensor(scale, dtype=torch.float32)
    return _encode_ties_away(y.clamp(-1e9, 1e9).where(y.abs() <= 448, torch.sign(y) * 416.0)
                             ).reshape(x.shape)


def _quantize_multiply(x, scale):
    y = torch.clamp(x.to(torch.float32) * torch.as_tensor(scale, dtype=torch.float32), -448, 448)
    return f8.encode(y).reshape(x.shape)


_orig_gather = f8.gather_dequantized


def _gather_wrong_block_scale(k_cache, v_cache, k_scales, v_scales, table_row, length):
    return _orig_gather(k_cache, v_cache, k_scales.roll(1, 0), v_scales.roll(1, 0),
                        table_row, length)


@pytest.mark.parametrize("name,fn", [
    ("encode", _encode_ties_away),
    ("quantize", _quantize_no_clamp),
    ("quantize", _quantize_multiply),
    ("gather_dequantized", _gather_wrong_block_scale),
])
def test_planted_fp8_mistake_fails_a_pin(monkeypatch, name, fn):
    monkeypatch.setattr(f8, name, fn)
    try:
        ok = _fp8_pins_pass()
        ok = ok and all(int(f8.encode(torch.tensor([y], dtype=torch.float64))[0]) == c
                        for y, c in [(1.0625, 0x38), (2.0 ** -10, 0x00)])
        ok = ok and int(f8.quantize(torch.tensor([1000.0]), 1.0)[0]) == 0x7E
    except AssertionError:
        ok = False
    assert not ok


def test_planted_v_scale_mistake_fails_brute_force(monkeypatch):
    orig = f8.reshape_and_cache_fp8

    def bad(k_cache, v_cache, k_scales, v_scales, key, value, slot_mapping):
        return orig(k_cache, v_cache, k_scales, k_scales, key, value, slot_mapping)
    monkeypatch.setattr(f8, "reshape_and_cache_fp8", bad)
    assert not _fp8_pins_pass()


def test_per_sequence_dequantisation_equals_whole_pool_dequantisation():
    """The oracle dequantises each gathered sequence; the plain reading
    dequantises the whole pools and runs ``paged_attention`` on them."""
    from oracle import paged_attention as pa
    g = torch.Generator().manual_seed(12)
    NB, H, B, D = 9, 2, 4, 8
    kc = torch.randint(0, 126, (NB, H, B, D), generator=g).to(torch.uint8)
    vc = torch.randint(128, 254, (NB, H, D, B), generator=g).to(torch.uint8)
    ks = torch.rand(NB, H, generator=g) * 0.1 + 0.01
    vs = torch.rand(NB, H, generator=g) * 0.1 + 0.01
    bt = torch.tensor([[4, 1, 7], [2, 8, 0]])
    lens, qsl = [11, 6], [0, 3, 4]
    q = torch.randn(4, 4, D, generator=g, dtype=torch.float64)
    got = f8.paged_attention_fp8(q, kc, vc, ks, vs, bt, lens, qsl, 0.4)
    want = pa.paged_attention(q, f8.dequantize_pool(kc, ks), f8.dequantize_pool(vc, vs), bt,
                              lens, qsl, 0.4)
    assert torch.allclose(got, want, rtol=0, atol=1e-13)
