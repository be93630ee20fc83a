"""CPU checks of the C ABI: the library loads, exports every symbol that
include/pa.h declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest
import torch

from paged_kv_cache_19_amd import binding
from tests.conftest import ROOT

HEADERS = [os.path.join(ROOT, "include", "pa.h"), os.path.join(ROOT, "include", "pa_sched.h")]
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation first


def _declared():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from paged_kv_cache_19_amd import build
        build.build()
    os.environ.pop("PA_CHECK", None)
    return binding.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) == 31, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.SIGNATURES)


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("g++", "-std=c++11")])
def test_headers_build_a_c_and_cxx_caller(lib, tmp_path, compiler, std):
    """Both headers compile as strict C99 and C++11, every declared function
    links against libpa.so by its declared name, and host-only calls run."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    names = _declared()
    src = tmp_path / ("caller.c" if compiler == "gcc" else "caller.cpp")
    src.write_text(
        '#include <stdio.h>\n#include "pa.h"\n#include "pa_sched.h"\n'
        "typedef void (*fn)(void);\n"
        "static fn table[] = {\n"
        + "".join(f"  (fn)&{n},\n" for n in names)
        + "};\n"
        "int main(void) {\n"
        "  unsigned n = 0, i;\n"
        "  for (i = 0; i < sizeof table / sizeof table[0]; ++i) n += table[i] != 0;\n"
        '  printf("%u %d %s\\n", n, pa_version(), pa_status_string(0));\n'
        "  return 0;\n}\n")
    exe = tmp_path / "caller"
    libdir = os.path.dirname(binding.LIB_PATH)
    subprocess.run([compiler, std, "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-Wno-cast-function-type", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe), "-L", libdir, "-lpa", f"-Wl,-rpath,{libdir}"],
                   check=True, capture_output=True, text=True)
    got = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert got[:2] == [str(len(names)), "100"], got
    assert got[2].startswith(binding.STATUS[0]), got


def test_status_strings_and_version(lib):
    for code, name in binding.STATUS.items():
        assert binding.status_string(code).startswith(name)
    assert binding.status_string(12345) == "unknown pa_status"
    assert binding.version() == 100


def test_workspace_queries(lib):
    n = lib.pa_decode_workspace_bytes(128, 64, 128, 8192, 16, 512)
    splits = 16
    # partials (o then (m, l), fp32) plus a header of 16 + 4 * (128 + 1) bytes rounded to 256
    assert n == 128 * 64 * splits * 128 * 4 + 128 * 64 * splits * 2 * 4 + 768
    # balanced decode (split 0): a row's 256 steps plus the 3-step start-up cost of a
    # piece, cut into shares of at least 8: up to ceil(259 / 8) + 1 = 34 pieces per row,
    # plus a header of 16 + 4 * (128 + 1) bytes rounded to 256
    assert lib.pa_decode_workspace_bytes(128, 64, 128, 8192, 16, 0) == \
        128 * 64 * 34 * 128 * 4 + 128 * 64 * 34 * 2 * 4 + 768
    assert lib.pa_decode_workspace_bytes(4, 8, 64, 64, 4, 0) > 0
    assert lib.pa_decode_workspace_bytes(4, 8, 64, 64, 3, 0) == 0       # B not a power of 2
    assert lib.pa_decode_workspace_bytes(4, 8, 64, 64, 16, 100) == 0    # split not % 64
    assert lib.pa_decode_workspace_bytes(4, 8, 64, 64, 16, 2048) > 0    # any multiple of 64
    assert lib.pa_decode_workspace_bytes(4, 8, 64, 0, 16, 0) == 0
    # chunked prefill: chunk rows get max(ceil(8704 / 2048) = 5 fixed splits (vector-ALU
    # path), ceil(272 steps / 91) + 1 = 4 stream-K pieces (MFMA path, ranges of at least
    # ceil(272 / 3) = 91 steps)) = 5 slots each, plus an int32 piece count per row; the
    # balanced decode of single-token rows gets ceil((272 + 3) / 8) + 1 = 36 pieces
    # per (sequence, head) row; header 16 + 4 * 65 bytes rounded to 256.
    def al(x):
        return -(-x // 256) * 256
    assert lib.pa_chunked_prefill_workspace_bytes(64, 2108, 32, 128, 8704, 16, 0) == \
        al(2108 * 32 * 5 * 128 * 4) + al(2108 * 32 * 5 * 8) + al(2108 * 32 * 4) + \
        al(64 * 32 * 36 * 128 * 4) + al(64 * 32 * 36 * 8) + 512
    # fixed ranges of 1024 keys (32 steps): ceil(272 / 32) + 1 = 10 slots per chunk row
    assert lib.pa_chunked_prefill_workspace_bytes(64, 2108, 32, 128, 8704, 16, 1024) == \
        al(2108 * 32 * 10 * 128 * 4) + al(2108 * 32 * 10 * 8) + al(2108 * 32 * 4) + \
        al(64 * 32 * 36 * 128 * 4) + al(64 * 32 * 36 * 8) + 512
    assert lib.pa_chunked_prefill_workspace_bytes(64, 2108, 32, 128, 8704, 16, 96) == 0
    # shared prefix of 32 blocks (512 keys, 16 steps): a row also keeps up to
    # ceil((16 + 3) / 8) + 1 = 4 prefix pieces (34 + 4 = 38 slots), and the header
    # room for one prefix entry per sequence: 16 + 4 * (256 + 1) bytes rounded to 256
    sp = lib.pa_decode_shared_prefix_workspace_bytes
    assert sp(128, 64, 128, 8192, 16, 32) == \
        128 * 64 * 38 * 128 * 4 + 128 * 64 * 38 * 2 * 4 + 1280
    assert sp(4, 8, 64, 64, 16, 4) > 0
    assert sp(4, 8, 64, 64, 16, 5) == 0      # prefix longer than max_seq_len
    assert sp(4, 8, 64, 64, 4, 1) == 0       # block_size below 8
    assert sp(4, 8, 64, 64, 16, -1) == 0


def _decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, maxb=4, lens=FAKE, S=2, maxlen=64,
             Hq=8, Hkv=2, D=128, B=16, NB=8, scale=0.1, dtype=1, split=0, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["maxb"], None, a["lens"],
                         a["S"], a["maxlen"], a["Hq"], a["Hkv"], a["D"], a["B"], a["NB"],
                         a["scale"], a["dtype"], a["split"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), -1), (dict(q=None), -1), (dict(kc=None), -1), (dict(bt=None), -1),
    (dict(lens=None), -1), (dict(dtype=7), -3), (dict(Hq=6, Hkv=4), -2),
    (dict(Hq=34, Hkv=2), -4), (dict(D=96), -4), (dict(B=12), -4), (dict(B=128), -4),
    (dict(maxb=0), -2), (dict(NB=0), -2), (dict(maxlen=0), -2), (dict(scale=float("nan")), -2),
    (dict(scale=0.0), -2), (dict(scale=-0.1), -2),
    (dict(split=96), -2), (dict(ws=None), -5), (dict(wsb=16), -5), (dict(S=70000), -4),
])
def test_decode_rejects_bad_arguments(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_empty_batch_is_a_no_op(lib):
    assert _decode(lib, S=0, out=None) == 0


def test_other_entry_points_reject_bad_arguments(lib):
    # slot mapping
    assert lib.pa_compute_slot_mapping(None, FAKE, 4, FAKE, None, 2, 2, 16, None) == -1
    assert lib.pa_compute_slot_mapping(FAKE, FAKE, 4, FAKE, None, 2, 3, 16, None) == -2
    assert lib.pa_compute_slot_mapping(FAKE, FAKE, 4, FAKE, None, 2, 2, 24, None) == -4
    assert lib.pa_compute_slot_mapping(FAKE, FAKE, 0, FAKE, None, 2, 2, 16, None) == -2
    assert lib.pa_compute_slot_mapping(None, None, 4, None, None, 0, 0, 16, None) == 0
    # cache write
    rc = lib.pa_reshape_and_cache
    assert rc(FAKE, FAKE, FAKE, FAKE, None, 4, 2, 128, 16, 8, 1, None) == -1
    assert rc(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 128, 16, 8, 5, None) == -3
    assert rc(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 80, 16, 8, 1, None) == -4
    assert rc(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0, 128, 16, 8, 1, None) == -2
    assert rc(None, None, None, None, None, 0, 2, 128, 16, 8, 1, None) == 0
    # chunked prefill: query_start_loc is required
    cp = lib.pa_chunked_prefill
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, FAKE, None, 2, 10, 64, 8, 8, 2, 128, 16, 8, 0.1,
            1, 0, FAKE, 1 << 30, None]
    assert cp(*args) == -1
    args[8] = FAKE
    args[21] = None
    assert cp(*args) == -5
    # the chunk kernel takes K / V pools under 2^40 bytes: 2^27 blocks of
    # 2 x 16 x 128 bf16 make 2^40 bytes (refused before any device access)
    args[21] = FAKE
    args[17] = 1 << 27
    assert cp(*args) == -4
    # pa_chunked_prefill_fp8: the same limit on each bf16 staging pool
    f8 = lib.pa_chunked_prefill_fp8
    f8args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, FAKE, FAKE, 2, 10, 64, 8, 8, 2,
              128, 16, 8, 1 << 27, 0.1, FAKE, 1 << 30, None]
    assert f8(*f8args) == -4
    f8args[20] = (1 << 27) - 1
    f8args[23] = 16
    assert f8(*f8args) == -5


def _append(lib, fp8=False, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, bt=FAKE,
             maxb=4, lens=FAKE, S=2, maxlen=64, Hq=8, Hkv=2, D=128, B=16, NB=8, scale=0.1,
             dtype=1, split=0, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    if fp8:
        return lib.pa_decode_fp8_append(a["out"], a["q"], a["k"], a["v"], a["kc"], a["vc"],
                                        a["ks"], a["vs"], a["bt"], a["maxb"], None, a["lens"],
                                        a["S"], a["maxlen"], a["Hq"], a["Hkv"], a["D"], a["B"],
                                        a["NB"], a["scale"], a["ws"], a["wsb"], None)
    return lib.pa_decode_append(a["out"], a["q"], a["k"], a["v"], a["kc"], a["vc"], a["bt"],
                                a["maxb"], None, a["lens"], a["S"], a["maxlen"], a["Hq"],
                                a["Hkv"], a["D"], a["B"], a["NB"], a["scale"], a["dtype"],
                                a["split"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("kw,code", [
    (dict(k=None), -1), (dict(v=None), -1), (dict(out=None), -1), (dict(kc=None), -1),
    (dict(bt=None), -1), (dict(Hq=6, Hkv=4), -2), (dict(D=96), -4), (dict(B=128), -4),
    (dict(scale=0.0), -2), (dict(ws=None), -5), (dict(wsb=16), -5),
])
def test_appending_decode_rejects_bad_arguments(lib, fp8, kw, code):
    """pa_decode_append / pa_decode_fp8_append check their arguments like
    pa_decode / pa_decode_fp8, and need both new-token arrays."""
    assert _append(lib, fp8=fp8, **kw) == code


def _shared_append(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, ks=None, vs=None, bt=FAKE,
             maxb=4, lens=FAKE, S=2, maxlen=64, Hq=8, Hkv=2, D=128, B=16, NB=8, pb=2, scale=0.1,
             ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.pa_decode_shared_prefix_append(a["out"], a["q"], a["k"], a["v"], a["kc"], a["vc"],
                                              a["ks"], a["vs"], a["bt"], a["maxb"], None,
                                              a["lens"], a["S"], a["maxlen"], a["Hq"], a["Hkv"],
                                              a["D"], a["B"], a["NB"], a["pb"], a["scale"],
                                              a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), -1), (dict(v=None), -1), (dict(out=None), -1), (dict(pb=-1), -2),
    (dict(ks=FAKE), -2), (dict(ks=FAKE, vs=FAKE, B=8), -4), (dict(pb=5), -2), (dict(D=96), -4),
    (dict(ws=None), -5), (dict(wsb=16), -5), (dict(S=4000), -4),
])
def test_shared_prefix_append_rejects_bad_arguments(lib, kw, code):
    assert _shared_append(lib, **kw) == code


def test_appending_decode_limits_and_empty_batch(lib):
    assert _append(lib, S=0, k=None, v=None, out=None) == 0
    assert _append(lib, fp8=True, S=0, k=None, v=None, out=None) == 0
    assert _append(lib, fp8=True, ks=None) == -1
    assert _append(lib, fp8=True, B=8) == -4       # e4m3 pools need block_size >= 16
    assert _append(lib, fp8=True, S=5000) == -4    # the e4m3 decode stops at 4,096
    assert _append(lib, dtype=7) == -3
    assert _append(lib, split=96) == -2
    assert _shared_append(lib, S=0, k=None, v=None, out=None) == 0


def _shared(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, ks=None, vs=None, bt=FAKE, maxb=4, lens=FAKE,
             S=2, maxlen=64, Hq=8, Hkv=2, D=128, B=16, NB=8, pb=2, scale=0.1, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return lib.pa_decode_shared_prefix(a["out"], a["q"], a["kc"], a["vc"], a["ks"], a["vs"],
                                       a["bt"], a["maxb"], None, a["lens"], a["S"], a["maxlen"],
                                       a["Hq"], a["Hkv"], a["D"], a["B"], a["NB"], a["pb"],
                                       a["scale"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), -1), (dict(bt=None), -1), (dict(pb=-1), -2),
    (dict(ks=FAKE), -2),                     # one scale array without the other
    (dict(ks=FAKE, vs=FAKE, B=8), -4),       # e4m3 pools need block_size >= 16
    (dict(B=4), -4), (dict(pb=5), -2),       # prefix past max_seq_len
    (dict(pb=5, maxlen=256), -2),            # prefix past the table width
    (dict(S=4000), -4),                      # 4000 + 1000 prefix entries > 4096
    (dict(Hq=6, Hkv=4), -2), (dict(D=96), -4), (dict(ws=None), -5), (dict(wsb=16), -5),
])
def test_shared_prefix_decode_rejects_bad_arguments(lib, kw, code):
    assert _shared(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(S=4000, pb=0), -5),                 # no prefix: pa_decode's limits (fails on ws only)
    (dict(S=4000, pb=1), -5),                 # 16 keys < one 32-key step: no prefix entry
    (dict(S=5000, pb=0), -5),                 # bf16 beyond 4,096: the fixed-split path
    (dict(S=4000, pb=3, ks=FAKE, vs=FAKE), -5),            # 48 keys < 64: fp8 pa_decode path,
    (dict(S=5000, pb=0, ks=FAKE, vs=FAKE, ws=FAKE), -4),   # which stops at 4,096 sequences
])
def test_shared_prefix_without_a_whole_step_takes_decode_limits(lib, kw, code):
    """A prefix shorter than one key step adds no prefix entries, so the
    entry limit is pa_decode's (bf16) or pa_decode_fp8's (e4m3)."""
    kw.setdefault("ws", None)
    assert _shared(lib, **kw) == code


def test_shared_prefix_decode_empty_batch_is_a_no_op(lib):
    assert _shared(lib, S=0, out=None) == 0


def test_binding_refuses_host_tensors(lib):
    import torch
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        binding.compute_slot_mapping(t.view(2, 2), t[:2], None, 16)


def test_block_copy_entry_points_reject_bad_arguments(lib):
    m = FAKE
    assert lib.pa_copy_blocks(FAKE, m, 0, 64, 8, None) == 0           # nothing to do
    assert lib.pa_copy_blocks(FAKE, m, 2, 0, 8, None) == -2           # block_bytes 0
    assert lib.pa_copy_blocks(FAKE, m, 2, 6, 8, None) == -2           # not a multiple of 4
    assert lib.pa_copy_blocks(FAKE, m, -1, 64, 8, None) == -2
    assert lib.pa_copy_blocks(FAKE, m, 2, 64, 0, None) == -2
    assert lib.pa_copy_blocks(None, m, 2, 64, 8, None) == -1
    assert lib.pa_copy_blocks(FAKE, None, 2, 64, 8, None) == -1
    assert lib.pa_swap_blocks(FAKE, FAKE, m, 2, 64, 8, 8, None) == -2   # same pool: use copy
    assert lib.pa_swap_blocks(None, FAKE, m, 2, 64, 8, 8, None) == -1
    assert lib.pa_swap_blocks(FAKE, ctypes.c_void_p(32), m, 2, 64, 8, 0, None) == -2


def _cpu_case(dtype=None, D=64, B=16, Hkv=2, Hq=8, NB=10, S=3):
    dtype = dtype or torch.bfloat16
    return dict(
        q=torch.zeros(S, Hq, D, dtype=dtype), kc=torch.zeros(NB, Hkv, B, D, dtype=dtype),
        vc=torch.zeros(NB, Hkv, D, B, dtype=dtype), bt=torch.zeros(S, 4, dtype=torch.int32),
        lens=torch.ones(S, dtype=torch.int32), key=torch.zeros(S, Hkv, D, dtype=dtype),
        slots=torch.zeros(S, dtype=torch.int64))


@pytest.mark.parametrize("mutate,match", [
    (lambda c: c.update(vc=c["vc"].transpose(2, 3).contiguous()), "v_cache must be"),
    (lambda c: c.update(kc=c["kc"].float(), vc=c["vc"].float()), "share one dtype"),
    (lambda c: c.update(q=c["q"][:, :, :32].contiguous()), "query must be"),
    (lambda c: c.update(bt=c["bt"].long()), "block_tables must be int32"),
    (lambda c: c.update(lens=c["lens"][:2].contiguous()), "seq_lens must be int32"),
])
def test_binding_decode_checks_shapes_and_dtypes(lib, mutate, match):
    """Mismatches between query, pools and metadata are refused before any
    pointer reaches the library: a token-major V pool, a query of another
    dtype, a wrong head_dim, int64 tables, short seq_lens."""
    c = _cpu_case()
    mutate(c)
    with pytest.raises(ValueError, match=match):
        binding.decode(c["q"], c["kc"], c["vc"], c["bt"], c["lens"], 64, 0.125,
                       out=torch.empty_like(c["q"]))


@pytest.mark.parametrize("mutate,match", [
    (lambda c: c.update(key=c["key"].float()), "share one dtype"),
    (lambda c: c.update(key=c["key"][:, :1].contiguous()), "key must be"),
    (lambda c: c.update(slots=c["slots"].int()), "slot_mapping must be int64"),
    (lambda c: c.update(vc=c["vc"][:, :, :32].contiguous()), "v_cache must be"),
])
def test_binding_cache_write_checks_shapes_and_dtypes(lib, mutate, match):
    """An fp32 key into a bf16 pool (which would write past the pool's end),
    a key with the wrong head count, int32 slots and a wrong V pool are
    refused."""
    c = _cpu_case()
    mutate(c)
    with pytest.raises(ValueError, match=match):
        binding.reshape_and_cache(c["key"], c["key"].clone(), c["kc"], c["vc"], c["slots"])


def test_binding_chunked_prefill_checks_query_start_loc(lib):
    c = _cpu_case()
    qsl = torch.tensor([0, 1, 2], dtype=torch.int32)          # needs S + 1 = 4 entries
    with pytest.raises(ValueError, match="query_start_loc must be"):
        binding.chunked_prefill(c["q"], c["kc"], c["vc"], c["bt"], c["lens"], qsl, 64, 1, 0.125)


def test_binding_fp8_checks_scales(lib):
    c = _cpu_case()
    k8 = torch.zeros(10, 2, 16, 64, dtype=torch.uint8)
    v8 = torch.zeros(10, 2, 64, 16, dtype=torch.uint8)
    ks = torch.ones(10, 2)
    with pytest.raises(ValueError, match="k_scales and v_scales must be"):
        binding.decode_fp8(c["q"], k8, v8, ks, ks[:5].contiguous(), c["bt"], c["lens"], 64, 0.125)
    with pytest.raises(ValueError, match="v_cache must be"):
        binding.decode_fp8(c["q"], k8, v8.transpose(2, 3).contiguous(), ks, ks, c["bt"],
                           c["lens"], 64, 0.125)


def test_noalloc_refuses_a_batch_beyond_its_scratch(lib):
    """pa_decode_noalloc checks the batch's workspace against its static
    scratch before anything else touches the GPU."""
    S, Hq, D, L, B = 1024, 64, 128, 8192, 16
    assert lib.pa_decode_workspace_bytes(S, Hq, D, L, B, 0) > binding.NOALLOC_SCRATCH_BYTES
    rc = lib.pa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 512, None, FAKE, S, L, Hq, 8, D, B,
                               100000, 0.088, binding.PA_BF16, 0, None)
    assert rc == binding.PA_ERR_SCRATCH
    assert binding.status_string(rc).startswith("PA_ERR_SCRATCH")
    # invalid sizes are pa_decode's errors, reported before the scratch is looked up
    assert lib.pa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 512, None, FAKE, 4, 64, 8, 2, 96,
                                 16, 64, 0.1, binding.PA_BF16, 0, None) == -4
    assert lib.pa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 512, None, FAKE, 4, 64, 8, 2, 128,
                                 16, 64, 0.1, binding.PA_BF16, 100, None) == -2
