"""Hardware probes of one MI355X, run from the repository root:

    python -m paged_kv_cache_19_amd.probes

They measure what the kernels' rooflines are compared against, with the
builder-written kernels of ``libpa_probe.so`` (``csrc/probe/pa_probe.hip``):

- the read rate of random tiles from a 4 GiB pool, over tile sizes and wave
  counts (four tiles in flight per wave): how the rate depends on the bytes in
  flight across the chip;
- the same for 4 KiB tiles read in two load layouts, 1 KiB contiguous per
  load and 64 bytes of each of 16 rows per load (an MFMA A operand);
- the rate of back-to-back ``v_mfma_f32_32x32x16_bf16``;
- how matrix and vector work overlap on a SIMD: bursts of 8 MFMAs and of a
  softmax-like vector mix, alone, one after the other in each wave,
  interleaved in each wave, or in separate waves.

Prints a markdown report.  Measurement only: nothing here is on the
attention path.
"""
from __future__ import annotations

import ctypes
import os
import statistics

import torch

from paged_kv_cache_19_amd.build import PROBE_LIB


def _lib():
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError("libpa_probe.so is not built (python -m paged_kv_cache_19_amd.build)")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.pa_probe_read_tiles.restype = ctypes.c_int
    lib.pa_probe_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_void_p]
    lib.pa_probe_read_rows.restype = ctypes.c_int
    lib.pa_probe_read_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p]
    lib.pa_probe_mfma.restype = ctypes.c_int
    lib.pa_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p]
    lib.pa_probe_overlap.restype = ctypes.c_int
    lib.pa_probe_overlap.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p]
    return lib


def _time_ms(launch, reps: int, warm: int) -> float:
    """Median milliseconds of ``launch()`` over ``reps`` timed runs after
    ``warm`` untimed ones (HIP events on the current stream)."""
    st = torch.cuda.current_stream()
    times = []
    for k in range(warm + reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(st)
        rc = launch(ctypes.c_void_p(st.cuda_stream))
        b.record(st)
        if rc != 0:
            raise RuntimeError(f"probe returned {rc}")
        torch.cuda.synchronize()
        if k >= warm:
            times.append(a.elapsed_time(b))
    return statistics.median(times)


def read_rates(lib, pool_bytes: int = 4 << 30):
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4096 * 64, dtype=torch.int32, device="cuda")
    rows = []
    for tile in (1024, 2048, 4096, 8192):
        n = pool_bytes // tile
        ids = torch.randperm(n, dtype=torch.int32, device="cuda",
                             generator=torch.Generator(device="cuda").manual_seed(7))
        row = [tile]
        for waves in (1024, 2048, 4096):
            ms = _time_ms(lambda s: lib.pa_probe_read_tiles(pool.data_ptr(), pool_bytes,
                                                            ids.data_ptr(), n, tile,
                                                            sink.data_ptr(), waves, s), 4, 1)
            row.append(pool_bytes / (ms * 1e-3) / 1e9)
        rows.append(row)
        del ids
    del pool, sink
    torch.cuda.empty_cache()
    return rows


def read_layouts(lib, pool_bytes: int = 4 << 30):
    """GB/s of random 4 KiB tiles read 1 KiB contiguous per load, and read
    64 bytes of each of 16 rows per load (the MFMA A-operand layout)."""
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4096 * 64, dtype=torch.int32, device="cuda")
    n = pool_bytes // 4096
    ids = torch.randperm(n, dtype=torch.int32, device="cuda",
                         generator=torch.Generator(device="cuda").manual_seed(7))
    rows = []
    for name, call in (("1 KiB contiguous per load", lambda w, s: lib.pa_probe_read_tiles(
                            pool.data_ptr(), pool_bytes, ids.data_ptr(), n, 4096, sink.data_ptr(),
                            w, s)),
                       ("64 B of each of 16 rows per load", lambda w, s: lib.pa_probe_read_rows(
                            pool.data_ptr(), pool_bytes, ids.data_ptr(), n, sink.data_ptr(), w,
                            s))):
        row = [name]
        for waves in (1024, 2048, 4096):
            ms = _time_ms(lambda s: call(waves, s), 4, 1)
            row.append(pool_bytes / (ms * 1e-3) / 1e9)
        rows.append(row)
    del pool, sink, ids
    torch.cuda.empty_cache()
    return rows


def mfma_rate(lib, iters: int = 8192):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 2 * cus
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    cold = _time_ms(lambda s: lib.pa_probe_mfma(sink.data_ptr(), wgs, iters, s), 3, 0)
    warm = _time_ms(lambda s: lib.pa_probe_mfma(sink.data_ptr(), wgs, iters, s), 7, 20)
    flops = wgs * 4 * iters * 4 * 2 * 32 * 32 * 16
    return flops / (cold * 1e-3) / 1e12, flops / (warm * 1e-3) / 1e12


def overlap_times(lib, exp_mix: bool, iters: int = 2000):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")

    def t(mode, wps):
        return _time_ms(lambda s: lib.pa_probe_overlap(sink.data_ptr(), mode, int(exp_mix), cus,
                                                       wps, iters, s), 5, 3)
    return {(mode, wps): t(mode, wps) for wps in (1, 2) for mode in range(6)
            if not (mode >= 4 and wps == 1)}


def main() -> None:
    assert torch.cuda.is_available(), "the probes need a GPU"
    lib = _lib()
    props = torch.cuda.get_device_properties(0)
    print(f"# Hardware probes: {props.name}, {props.multi_processor_count} CUs\n")
    print("Command (from the repository root): `python -m paged_kv_cache_19_amd.probes`\n")
    print("## Random-tile reads from a 4 GiB pool (GB/s; four tiles in flight per wave)\n")
    print("| tile | 1,024 waves | 2,048 waves | 4,096 waves |")
    print("|---|---|---|---|")
    for tile, *r in read_rates(lib):
        print(f"| {tile // 1024} KiB | " + " | ".join(f"{x:.0f}" for x in r) + " |")
    print("\n## Random 4 KiB tiles (16 rows of 256 B) by load layout (GB/s; four tiles in flight "
          "per wave)\n")
    print("| layout | 1,024 waves | 2,048 waves | 4,096 waves |")
    print("|---|---|---|---|")
    for name, *r in read_layouts(lib):
        print(f"| {name} | " + " | ".join(f"{x:.0f}" for x in r) + " |")
    cold, warm = mfma_rate(lib)
    print("\n## Back-to-back v_mfma_f32_32x32x16_bf16 (two workgroups of four waves per CU, "
          "four accumulators per wave)\n")
    print(f"- first runs of the process: {cold:.0f} TFLOP/s")
    print(f"- after 20 untimed runs: {warm:.0f} TFLOP/s ({warm / 2500 * 100:.1f}% of 2.5 PFLOP/s)")
    print("\n## Matrix and vector work on one SIMD (ms; one workgroup per CU, 2,000 bursts "
          "per wave; a matrix burst is 8 MFMAs)\n")
    for exp_mix, label in ((True, "16 exponentials and 32 fmas"), (False, "48 fmas")):
        o = overlap_times(lib, exp_mix)
        print(f"Vector burst: {label} per lane.\n")
        print("| waves per SIMD | matrix only | vector only | both, one after the other | "
              "both, interleaved 1 MFMA : 10 vector | waves 0-3 matrix, 4-7 vector | "
              "even waves matrix, odd vector |")
        print("|---|---|---|---|---|---|---|")
        for wps in (1, 2):
            split = (f"{o[(4, 2)]:.3f} | {o[(5, 2)]:.3f}" if wps == 2 else "— | —")
            print(f"| {wps} | {o[(0, wps)]:.3f} | {o[(1, wps)]:.3f} | {o[(2, wps)]:.3f} | "
                  f"{o[(3, wps)]:.3f} | {split} |")
        s1 = o[(0, 1)] + o[(1, 1)]
        print(f"\nOne wave per SIMD, both kinds in the wave: {o[(2, 1)] / s1:.2f} of the sum "
              f"of the parts in sequence, {o[(3, 1)] / s1:.2f} interleaved. Split between the "
              f"two waves of a SIMD: {min(o[(4, 2)], o[(5, 2)]) / s1:.2f} of that sum "
              f"(1.00 = no overlap; {max(o[(0, 1)], o[(1, 1)]) / s1:.2f} = full overlap).\n")


if __name__ == "__main__":
    main()
