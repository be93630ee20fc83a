"""Thin ctypes binding of libpa (include/pa.h), same names as the C ABI.

Argument marshalling only: every step of the path runs in libpa's HIP
kernels.  torch supplies device memory (tensors are passed by data pointer)
and the current HIP stream.  There is no fallback: if ``libpa.so`` is
missing, or a call returns an error, a ``PAError`` is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_F32 = 0
PA_BF16 = 1

STATUS = {
    0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_DTYPE",
    -4: "PA_ERR_UNSUPPORTED", -5: "PA_ERR_WORKSPACE", -6: "PA_ERR_INDEX", -7: "PA_ERR_HIP",
    -8: "PA_ERR_SCRATCH",
}
PA_ERR_SCRATCH = -8
NOALLOC_SCRATCH_BYTES = 160 * 1024 * 1024   # PA_NOALLOC_SCRATCH_BYTES of include/pa.h

# (name, restype, argtypes) of every symbol include/pa.h declares.
_i32, _f32, _sz, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_version": (ctypes.c_int, []),
    "pa_compute_slot_mapping": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp]),
    "pa_reshape_and_cache": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _vp]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32,
                                 _i32, _i32, _i32, _i32, _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_chunked_prefill_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_chunked_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32,
                                          _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                          _i32, _i32, _vp, _sz, _vp]),
    "pa_copy_blocks": (ctypes.c_int, [_vp, _vp, _i32, ctypes.c_int64, _i32, _vp]),
    "pa_swap_blocks": (ctypes.c_int, [_vp, _vp, _vp, _i32, ctypes.c_int64, _i32, _i32, _vp]),
    "pa_sched_create": (_vp, [_i32, _i32, _i32, _i32, _vp]),
    "pa_sched_destroy": (None, [_vp]),
    "pa_sched_add_request": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _i32, _i32]),
    "pa_sched_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp]),
    "pa_sched_get_batch": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp]),
    "pa_sched_update": (ctypes.c_int, [_vp, _vp, _vp, _i32]),
    "pa_sched_block_refcounts": (ctypes.c_int, [_vp, _vp, _i32]),
    "pa_sched_counts": (ctypes.c_int, [_vp, _vp, _vp, _vp]),
    "pa_sched_enable_swap": (ctypes.c_int, [_vp, _i32]),
    "pa_sched_get_swaps": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pa_reshape_and_cache_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                                _i32, _i32, _i32, _vp]),
    "pa_decode_fp8_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32,
                                     _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp]),
    "pa_decode_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                         _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _vp]),
    "pa_chunked_prefill_fp8_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                     _i32, ctypes.c_int64]),
    "pa_chunked_prefill_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                                              _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                              _i32, ctypes.c_int64, _f32, _vp, _sz, _vp]),
    "pa_decode_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32,
                                        _vp, _sz, _vp]),
    "pa_decode_fp8_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                            _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                            _f32, _vp, _sz, _vp]),
    "pa_decode_shared_prefix_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                      _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                                      _i32, _i32, _i32, _i32, _f32, _vp, _sz,
                                                      _vp]),
    "pa_decode_shared_prefix_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_shared_prefix": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                                               _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                               _f32, _vp, _sz, _vp]),
}


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libpa.so (built in-tree); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PAError("load", -7) from FileNotFoundError(
                f"{LIB_PATH} is missing: run `python -m paged_kv_cache_19_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PAError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libpa takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libpa takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _same_device(*ts) -> None:
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(map(str, devs))}")


def _want(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _pools(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """Shapes of a K/V pool pair: K [NB, H_kv, B, D] and V [NB, H_kv, D, B]
    (the V pool keeps each head_dim row's B tokens contiguous).  Returns
    (NB, H_kv, B, D).  A V pool laid out like K is refused whenever B != D;
    with B == D the two layouts have one shape and only the caller can tell."""
    _want(k_cache.dim() == 4 and v_cache.dim() == 4,
          "k_cache and v_cache are 4-d pools [NB, H_kv, B, D] / [NB, H_kv, D, B]")
    NB, Hkv, B, D = k_cache.shape
    _want(tuple(v_cache.shape) == (NB, Hkv, D, B),
          f"v_cache must be [NB, H_kv, D, B] = {(NB, Hkv, D, B)} for k_cache {tuple(k_cache.shape)}"
          f", got {tuple(v_cache.shape)}")
    _want(k_cache.dtype == v_cache.dtype, "k_cache and v_cache have different dtypes")
    return NB, Hkv, B, D


def _metadata(block_tables: torch.Tensor, seq_lens: torch.Tensor, num_seqs: int,
              block_refcounts: Optional[torch.Tensor], num_blocks: int,
              query_start_loc: Optional[torch.Tensor] = None) -> None:
    _want(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == num_seqs,
          f"block_tables must be int32 [{num_seqs}, max_blocks_per_seq]")
    _want(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (num_seqs,),
          f"seq_lens must be int32 [{num_seqs}]")
    if query_start_loc is not None:
        _want(query_start_loc.dtype == torch.int32
              and tuple(query_start_loc.shape) == (num_seqs + 1,),
              f"query_start_loc must be int32 [{num_seqs + 1}]")
    if block_refcounts is not None:
        _want(block_refcounts.dtype == torch.int32
              and tuple(block_refcounts.shape) == (num_blocks,),
              f"block_refcounts must be int32 [{num_blocks}]")


def _rows(query: torch.Tensor, out: Optional[torch.Tensor], Hkv: int, D: int) -> None:
    _want(query.dim() == 3 and query.shape[2] == D, f"query must be [T, H_q, {D}]")
    _want(query.shape[1] % Hkv == 0, f"num_q_heads {query.shape[1]} is not a multiple of {Hkv}")
    if out is not None:
        _want(out.shape == query.shape and out.dtype == query.dtype,
              "out must have the shape and dtype of query")


def _workspace(ws: Optional[torch.Tensor]) -> None:
    if ws is not None:
        _want(ws.dtype == torch.uint8 and ws.dim() == 1, "workspace is a 1-d uint8 tensor")


def status_string(status: int) -> str:
    return lib().pa_status_string(status).decode()


def version() -> int:
    return lib().pa_version()


def compute_slot_mapping(block_tables: torch.Tensor, seq_lens: torch.Tensor,
                         query_start_loc: Optional[torch.Tensor], block_size: int,
                         num_tokens: Optional[int] = None, out: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    S = seq_lens.numel()
    _metadata(block_tables, seq_lens, S, None, 0, query_start_loc)
    _same_device(block_tables, seq_lens, query_start_loc, out)
    if num_tokens is None:
        num_tokens = S if query_start_loc is None else int(query_start_loc[-1].item())
    if out is not None:
        _want(out.dtype == torch.int64 and tuple(out.shape) == (num_tokens,),
              f"slot_mapping out must be int64 [{num_tokens}]")
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int64, device=seq_lens.device)
    _check("pa_compute_slot_mapping", lib().pa_compute_slot_mapping(
        _ptr(out), _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
        _ptr(query_start_loc), S, num_tokens, block_size, _stream(stream)))
    return out


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    NB, Hkv, B, D = _pools(k_cache, v_cache)
    _want(key.dim() == 3 and tuple(key.shape[1:]) == (Hkv, D),
          f"key must be [T, {Hkv}, {D}] for these pools")
    _want(value.shape == key.shape, "value must have the shape of key")
    _want(key.dtype == value.dtype == k_cache.dtype,
          f"key, value and the pools must share one dtype ({key.dtype}, {value.dtype}, "
          f"{k_cache.dtype})")
    T, H = key.shape[0], Hkv
    _want(slot_mapping.dtype == torch.int64 and tuple(slot_mapping.shape) == (T,),
          f"slot_mapping must be int64 [{T}]")
    _same_device(key, value, k_cache, v_cache, slot_mapping)
    _check("pa_reshape_and_cache", lib().pa_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, H, D, B,
        NB, _dtype(key), _stream(stream)))


def decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len, block_size,
                           kv_split_tokens=0) -> int:
    n = lib().pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len,
                                        block_size, kv_split_tokens)
    if n == 0:
        raise PAError("pa_decode_workspace_bytes", -2)
    return n


def chunked_prefill_workspace_bytes(num_seqs, num_tokens, num_q_heads, head_dim, max_seq_len,
                                    block_size, kv_split_tokens=0) -> int:
    n = lib().pa_chunked_prefill_workspace_bytes(num_seqs, num_tokens, num_q_heads, head_dim,
                                                 max_seq_len, block_size, kv_split_tokens)
    if n == 0:
        raise PAError("pa_chunked_prefill_workspace_bytes", -2)
    return n


def decode(query: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, scale: float,
           kv_split_tokens: int = 0, block_refcounts: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    NB, Hkv, B, D = _pools(k_cache, v_cache)
    _rows(query, out, Hkv, D)
    _want(query.dtype == k_cache.dtype,
          f"query and the pools must share one dtype ({query.dtype}, {k_cache.dtype})")
    S, Hq = query.shape[0], query.shape[1]
    _metadata(block_tables, seq_lens, S, block_refcounts, NB)
    _workspace(workspace)
    _same_device(query, k_cache, v_cache, block_tables, seq_lens, block_refcounts, out, workspace)
    if out is None:
        out = torch.empty_like(query)
    if workspace is None:  # needs no initialisation
        workspace = torch.empty(decode_workspace_bytes(S, Hq, D, max_seq_len, B, kv_split_tokens),
                                dtype=torch.uint8, device=query.device)
    _check("pa_decode", lib().pa_decode(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(block_refcounts), _ptr(seq_lens), S, max_seq_len, Hq, Hkv,
        D, B, NB, scale,
        _dtype(query), kv_split_tokens, _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def _new_tokens(key: torch.Tensor, value: torch.Tensor, S: int, Hkv: int, D: int,
                dtype: torch.dtype) -> None:
    _want(key.dim() == 3 and tuple(key.shape) == (S, Hkv, D),
          f"key must be [{S}, {Hkv}, {D}]: one new token per sequence")
    _want(value.shape == key.shape, "value must have the shape of key")
    _want(key.dtype == value.dtype == dtype,
          f"key and value must be {dtype} ({key.dtype}, {value.dtype})")


def decode_append(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                  k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                  seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                  kv_split_tokens: int = 0, block_refcounts: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """pa_decode_append: each sequence's new token (key/value [S, H_kv, D])
    written at position seq_len - 1 of its table, then the decode; the pools
    are modified in place."""
    NB, Hkv, B, D = _pools(k_cache, v_cache)
    _rows(query, out, Hkv, D)
    _want(query.dtype == k_cache.dtype,
          f"query and the pools must share one dtype ({query.dtype}, {k_cache.dtype})")
    S, Hq = query.shape[0], query.shape[1]
    _new_tokens(key, value, S, Hkv, D, k_cache.dtype)
    _metadata(block_tables, seq_lens, S, block_refcounts, NB)
    _workspace(workspace)
    _same_device(query, key, value, k_cache, v_cache, block_tables, seq_lens, block_refcounts,
                 out, workspace)
    if out is None:
        out = torch.empty_like(query)
    if workspace is None:  # needs no initialisation
        workspace = torch.empty(decode_workspace_bytes(S, Hq, D, max_seq_len, B, kv_split_tokens),
                                dtype=torch.uint8, device=query.device)
    _check("pa_decode_append", lib().pa_decode_append(
        _ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), block_tables.shape[1], _ptr(block_refcounts), _ptr(seq_lens), S,
        max_seq_len, Hq, Hkv, D, B, NB, scale, _dtype(query), kv_split_tokens, _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return out


def decode_noalloc(query: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                   scale: float, out: torch.Tensor, kv_split_tokens: int = 0,
                   block_refcounts: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_decode with the library's static scratch as workspace: nothing is
    allocated (the caller passes ``out``)."""
    NB, Hkv, B, D = _pools(k_cache, v_cache)
    _rows(query, out, Hkv, D)
    _want(query.dtype == k_cache.dtype,
          f"query and the pools must share one dtype ({query.dtype}, {k_cache.dtype})")
    S, Hq = query.shape[0], query.shape[1]
    _metadata(block_tables, seq_lens, S, block_refcounts, NB)
    _same_device(query, k_cache, v_cache, block_tables, seq_lens, block_refcounts, out)
    _check("pa_decode_noalloc", lib().pa_decode_noalloc(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(block_refcounts), _ptr(seq_lens), S, max_seq_len, Hq, Hkv,
        D, B, NB, scale, _dtype(query), kv_split_tokens, _stream(stream)))
    return out


def chunked_prefill(query: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    block_tables: torch.Tensor, seq_lens: torch.Tensor,
                    query_start_loc: torch.Tensor, max_seq_len: int, max_query_len: int,
                    scale: float, kv_split_tokens: int = 0,
                    block_refcounts: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    NB, Hkv, B, D = _pools(k_cache, v_cache)
    _rows(query, out, Hkv, D)
    _want(query.dtype == k_cache.dtype,
          f"query and the pools must share one dtype ({query.dtype}, {k_cache.dtype})")
    T, Hq = query.shape[0], query.shape[1]
    S = seq_lens.numel()
    _metadata(block_tables, seq_lens, S, block_refcounts, NB, query_start_loc)
    _workspace(workspace)
    _same_device(query, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                 block_refcounts, out, workspace)
    if out is None:
        out = torch.empty_like(query)
    if workspace is None:  # needs no initialisation
        workspace = torch.empty(chunked_prefill_workspace_bytes(S, T, Hq, D, max_seq_len, B,
                                                                kv_split_tokens),
                                dtype=torch.uint8, device=query.device)
    _check("pa_chunked_prefill", lib().pa_chunked_prefill(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(block_refcounts), _ptr(seq_lens), _ptr(query_start_loc), S,
        T, max_seq_len,
        max_query_len, Hq, Hkv, D, B, NB, scale, _dtype(query), kv_split_tokens,
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


# -- whole-block copies ---------------------------------------------------------

def _pool_ptr(t: torch.Tensor):
    """Data pointer of a pool: a device tensor or a pinned host tensor."""
    if not t.is_contiguous():
        raise ValueError("libpa takes contiguous tensors")
    if not t.is_cuda and not t.is_pinned():
        raise ValueError("a host pool must be pinned memory")
    return ctypes.c_void_p(t.data_ptr())


def _block_bytes(pool: torch.Tensor) -> int:
    return pool[0].numel() * pool.element_size()


def copy_blocks(pool: torch.Tensor, block_mapping: torch.Tensor, stream=None) -> None:
    """Copy-on-write inside one pool: block d = block s for every (s, d) row
    of the device int64 ``block_mapping`` [n, 2]."""
    _want(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2
          and block_mapping.shape[1] == 2, "block_mapping must be int64 [n, 2]")
    _same_device(pool, block_mapping)
    _check("pa_copy_blocks", lib().pa_copy_blocks(
        _ptr(pool), _ptr(block_mapping), block_mapping.shape[0], _block_bytes(pool),
        pool.shape[0], _stream(stream)))


def swap_blocks(dst_pool: torch.Tensor, src_pool: torch.Tensor, block_mapping: torch.Tensor,
                stream=None) -> None:
    """Copy blocks between pools (device or pinned host): block d of
    ``dst_pool`` = block s of ``src_pool`` for every (s, d) row."""
    if _block_bytes(dst_pool) != _block_bytes(src_pool):
        raise ValueError("pools with different block sizes")
    _want(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2
          and block_mapping.shape[1] == 2, "block_mapping must be int64 [n, 2]")
    _want(block_mapping.is_cuda, "block_mapping is a device tensor")
    _check("pa_swap_blocks", lib().pa_swap_blocks(
        _pool_ptr(dst_pool), _pool_ptr(src_pool), _ptr(block_mapping), block_mapping.shape[0],
        _block_bytes(dst_pool), dst_pool.shape[0], src_pool.shape[0], _stream(stream)))


# -- FP8 (e4m3) KV cache -------------------------------------------------------

def _fp8_pool(t: torch.Tensor) -> None:
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError(f"an fp8 pool is uint8 or float8_e4m3fn, not {t.dtype}")


def _f32(t: torch.Tensor) -> None:
    if t.dtype != torch.float32:
        raise ValueError("scales are float32 [num_blocks, num_kv_heads]")


def _fp8_pools(k_cache, v_cache, k_scales, v_scales):
    """Shapes of an e4m3 pool pair and its scales; returns (NB, H_kv, B, D)."""
    NB, Hkv, B, D = _pools(k_cache, v_cache)
    _fp8_pool(k_cache)
    _f32(k_scales)
    _f32(v_scales)
    _want(tuple(k_scales.shape) == (NB, Hkv) and tuple(v_scales.shape) == (NB, Hkv),
          f"k_scales and v_scales must be float32 [{NB}, {Hkv}]")
    return NB, Hkv, B, D


def reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, k_scales: torch.Tensor, v_scales: torch.Tensor,
                          slot_mapping: torch.Tensor, stream=None) -> None:
    NB, H, B, D = _fp8_pools(k_cache, v_cache, k_scales, v_scales)
    if key.dtype != torch.bfloat16 or value.dtype != torch.bfloat16:
        raise ValueError("key/value are bf16")
    _want(key.dim() == 3 and tuple(key.shape[1:]) == (H, D) and value.shape == key.shape,
          f"key and value must be [T, {H}, {D}] for these pools")
    T = key.shape[0]
    _want(slot_mapping.dtype == torch.int64 and tuple(slot_mapping.shape) == (T,),
          f"slot_mapping must be int64 [{T}]")
    _same_device(key, value, k_cache, v_cache, k_scales, v_scales, slot_mapping)
    _check("pa_reshape_and_cache_fp8", lib().pa_reshape_and_cache_fp8(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _ptr(slot_mapping), T, H, D, B, NB, _stream(stream)))


def decode_fp8_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len, block_size) -> int:
    n = lib().pa_decode_fp8_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len,
                                            block_size)
    if n == 0:
        raise PAError("pa_decode_fp8_workspace_bytes", -2)
    return n


def decode_fp8(query: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               k_scales: torch.Tensor, v_scales: torch.Tensor, block_tables: torch.Tensor,
               seq_lens: torch.Tensor, max_seq_len: int, scale: float,
               block_refcounts: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    NB, Hkv, B, D = _fp8_pools(k_cache, v_cache, k_scales, v_scales)
    if query.dtype != torch.bfloat16:
        raise ValueError("the fp8 decode takes a bf16 query")
    _rows(query, out, Hkv, D)
    S, Hq = query.shape[0], query.shape[1]
    _metadata(block_tables, seq_lens, S, block_refcounts, NB)
    _workspace(workspace)
    _same_device(query, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                 block_refcounts, out, workspace)
    if out is None:
        out = torch.empty_like(query)
    if workspace is None:  # needs no initialisation
        workspace = torch.empty(decode_fp8_workspace_bytes(S, Hq, D, max_seq_len, B),
                                dtype=torch.uint8, device=query.device)
    _check("pa_decode_fp8", lib().pa_decode_fp8(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), block_tables.shape[1], _ptr(block_refcounts), _ptr(seq_lens), S,
        max_seq_len, Hq, Hkv, D, B, NB, scale, _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out


def decode_fp8_append(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                      k_cache: torch.Tensor, v_cache: torch.Tensor, k_scales: torch.Tensor,
                      v_scales: torch.Tensor, block_tables: torch.Tensor,
                      seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                      block_refcounts: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_decode_fp8_append: bf16 key/value [S, H_kv, D] quantised into the
    e4m3 pools at position seq_len - 1, then the e4m3 decode."""
    NB, Hkv, B, D = _fp8_pools(k_cache, v_cache, k_scales, v_scales)
    if query.dtype != torch.bfloat16:
        raise ValueError("the fp8 decode takes a bf16 query")
    _rows(query, out, Hkv, D)
    S, Hq = query.shape[0], query.shape[1]
    _new_tokens(key, value, S, Hkv, D, torch.bfloat16)
    _metadata(block_tables, seq_lens, S, block_refcounts, NB)
    _workspace(workspace)
    _same_device(query, key, value, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                 block_refcounts, out, workspace)
    if out is None:
        out = torch.empty_like(query)
    if workspace is None:  # needs no initialisation
        workspace = torch.empty(decode_fp8_workspace_bytes(S, Hq, D, max_seq_len, B),
                                dtype=torch.uint8, device=query.device)
    _check("pa_decode_fp8_append", lib().pa_decode_fp8_append(
        _ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), block_tables.shape[1],
        _ptr(block_refcounts), _ptr(seq_lens), S, max_seq_len, Hq, Hkv, D, B, NB, scale,
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def chunked_prefill_fp8_workspace_bytes(num_seqs, num_tokens, num_q_heads, num_kv_heads,
                                        head_dim, max_seq_len, max_blocks_per_seq, block_size,
                                        chunk_context_blocks) -> int:
    n = lib().pa_chunked_prefill_fp8_workspace_bytes(num_seqs, num_tokens, num_q_heads,
                                                     num_kv_heads, head_dim, max_seq_len,
                                                     max_blocks_per_seq, block_size,
                                                     chunk_context_blocks)
    if n == 0:
        raise PAError("pa_chunked_prefill_fp8_workspace_bytes", -2)
    return n


def chunk_context_blocks(seq_lens, query_start_loc, block_size: int) -> int:
    """Staging blocks pa_chunked_prefill_fp8 needs: the sum of ceil(L / B)
    over sequences with more than one query row (host lists or tensors)."""
    lens = [int(x) for x in (seq_lens.tolist() if hasattr(seq_lens, "tolist") else seq_lens)]
    qsl = [int(x) for x in (query_start_loc.tolist() if hasattr(query_start_loc, "tolist")
                            else query_start_loc)]
    return sum(-(-L // block_size) for s, L in enumerate(lens) if qsl[s + 1] - qsl[s] > 1)


def chunked_prefill_fp8(query: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        k_scales: torch.Tensor, v_scales: torch.Tensor,
                        block_tables: torch.Tensor, seq_lens: torch.Tensor,
                        query_start_loc: torch.Tensor, max_seq_len: int, max_query_len: int,
                        scale: float, chunk_context_blocks: int,
                        block_refcounts: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_chunked_prefill over e4m3 pools (query chunks staged as bf16)."""
    NB, Hkv, B, D = _fp8_pools(k_cache, v_cache, k_scales, v_scales)
    if query.dtype != torch.bfloat16:
        raise ValueError("the fp8 chunked prefill takes a bf16 query")
    _rows(query, out, Hkv, D)
    T, Hq = query.shape[0], query.shape[1]
    S = seq_lens.numel()
    _metadata(block_tables, seq_lens, S, block_refcounts, NB, query_start_loc)
    _workspace(workspace)
    _same_device(query, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                 query_start_loc, block_refcounts, out, workspace)
    if out is None:
        out = torch.empty_like(query)
    if workspace is None:  # needs no initialisation
        workspace = torch.empty(chunked_prefill_fp8_workspace_bytes(
            S, T, Hq, Hkv, D, max_seq_len, block_tables.shape[1], B, chunk_context_blocks),
            dtype=torch.uint8, device=query.device)
    _check("pa_chunked_prefill_fp8", lib().pa_chunked_prefill_fp8(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), block_tables.shape[1], _ptr(block_refcounts), _ptr(seq_lens),
        _ptr(query_start_loc), S, T, max_seq_len, max_query_len, Hq, Hkv, D, B, NB,
        chunk_context_blocks, scale, _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len,
                                         block_size, prefix_blocks) -> int:
    n = lib().pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                      max_seq_len, block_size, prefix_blocks)
    if n == 0:
        raise PAError("pa_decode_shared_prefix_workspace_bytes", -2)
    return n


def decode_shared_prefix(query: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                         scale: float, prefix_blocks: int,
                         k_scales: Optional[torch.Tensor] = None,
                         v_scales: Optional[torch.Tensor] = None,
                         block_refcounts: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_decode (bf16 pools) or pa_decode_fp8 (e4m3 pools, with k_scales and
    v_scales) for a batch whose tables all start with the same prefix_blocks
    blocks."""
    if query.dtype != torch.bfloat16:
        raise ValueError("the shared-prefix decode takes a bf16 query")
    if (k_scales is None) != (v_scales is None):
        raise ValueError("pass both k_scales and v_scales (e4m3 pools) or neither")
    if k_scales is not None:
        NB, Hkv, B, D = _fp8_pools(k_cache, v_cache, k_scales, v_scales)
    else:
        NB, Hkv, B, D = _pools(k_cache, v_cache)
        _want(k_cache.dtype == torch.bfloat16, "without scales the pools are bf16")
    _rows(query, out, Hkv, D)
    S, Hq = query.shape[0], query.shape[1]
    _metadata(block_tables, seq_lens, S, block_refcounts, NB)
    _workspace(workspace)
    _same_device(query, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                 block_refcounts, out, workspace)
    if out is None:
        out = torch.empty_like(query)
    if workspace is None:  # needs no initialisation
        workspace = torch.empty(decode_shared_prefix_workspace_bytes(S, Hq, D, max_seq_len, B,
                                                                     prefix_blocks),
                                dtype=torch.uint8, device=query.device)
    _check("pa_decode_shared_prefix", lib().pa_decode_shared_prefix(
        _ptr(out), _ptr(query), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), block_tables.shape[1], _ptr(block_refcounts), _ptr(seq_lens), S,
        max_seq_len, Hq, Hkv, D, B, NB, prefix_blocks, scale, _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return out


def decode_shared_prefix_append(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                                k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_tables: torch.Tensor, seq_lens: torch.Tensor,
                                max_seq_len: int, scale: float, prefix_blocks: int,
                                k_scales: Optional[torch.Tensor] = None,
                                v_scales: Optional[torch.Tensor] = None,
                                block_refcounts: Optional[torch.Tensor] = None,
                                out: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None,
                                stream=None) -> torch.Tensor:
    """pa_decode_shared_prefix_append: each sequence's new token (bf16
    key/value [S, H_kv, D]) written at position seq_len - 1 (quantised for
    e4m3 pools) and the shared-prefix decode, in one call."""
    if query.dtype != torch.bfloat16:
        raise ValueError("the shared-prefix decode takes a bf16 query")
    if (k_scales is None) != (v_scales is None):
        raise ValueError("pass both k_scales and v_scales (e4m3 pools) or neither")
    if k_scales is not None:
        NB, Hkv, B, D = _fp8_pools(k_cache, v_cache, k_scales, v_scales)
    else:
        NB, Hkv, B, D = _pools(k_cache, v_cache)
        _want(k_cache.dtype == torch.bfloat16, "without scales the pools are bf16")
    _rows(query, out, Hkv, D)
    S, Hq = query.shape[0], query.shape[1]
    _new_tokens(key, value, S, Hkv, D, torch.bfloat16)
    _metadata(block_tables, seq_lens, S, block_refcounts, NB)
    _workspace(workspace)
    _same_device(query, key, value, k_cache, v_cache, k_scales, v_scales, block_tables,
                 seq_lens, block_refcounts, out, workspace)
    if out is None:
        out = torch.empty_like(query)
    if workspace is None:  # needs no initialisation
        workspace = torch.empty(decode_shared_prefix_workspace_bytes(S, Hq, D, max_seq_len, B,
                                                                     prefix_blocks),
                                dtype=torch.uint8, device=query.device)
    _check("pa_decode_shared_prefix_append", lib().pa_decode_shared_prefix_append(
        _ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), block_tables.shape[1],
        _ptr(block_refcounts), _ptr(seq_lens), S, max_seq_len, Hq, Hkv, D, B, NB, prefix_blocks,
        scale, _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


# -- host batch builder (include/pa_sched.h) ------------------------------------

class BatchBuilder:
    """The native batch builder: queue requests, schedule steps, feed back
    sampled tokens.  Host memory only; arrays are numpy."""

    def __init__(self, num_blocks: int, block_size: int, token_budget: int, chunk_tokens: int,
                 free_order=None, num_host_blocks: int = 0):
        import numpy as np
        self._np = np
        fo = None
        if free_order is not None:
            fo = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
        self.num_blocks = num_blocks
        self._h = lib().pa_sched_create(num_blocks, block_size, token_budget, chunk_tokens,
                                        None if fo is None else fo.ctypes.data_as(ctypes.c_void_p))
        if not self._h:
            raise PAError("pa_sched_create", -2)
        if num_host_blocks:
            _check("pa_sched_enable_swap", lib().pa_sched_enable_swap(self._h, num_host_blocks))

    def close(self) -> None:
        if self._h:
            lib().pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_request(self, req_id: int, prompt, max_new_tokens: int) -> None:
        p = self._np.ascontiguousarray(self._np.asarray(prompt, dtype=self._np.int32))
        _check("pa_sched_add_request", lib().pa_sched_add_request(
            self._h, req_id, p.ctypes.data_as(ctypes.c_void_p), p.size, max_new_tokens))

    def step(self, pad_block: int = 0) -> dict:
        np = self._np
        n = [ctypes.c_int32() for _ in range(4)]
        _check("pa_sched_step", lib().pa_sched_step(self._h, *[ctypes.byref(x) for x in n]))
        S, T, MB, P = (x.value for x in n)
        mb = max(MB, 1)
        out = {
            "req_ids": np.zeros(S, np.int64), "seq_lens": np.zeros(S, np.int32),
            "query_start_loc": np.zeros(S + 1, np.int32),
            "block_tables": np.zeros((S, mb), np.int32), "slot_mapping": np.zeros(T, np.int64),
            "preempted": np.zeros(P, np.int64),
        }

        def ptr(a):
            return a.ctypes.data_as(ctypes.c_void_p)
        _check("pa_sched_get_batch", lib().pa_sched_get_batch(
            self._h, ptr(out["req_ids"]), ptr(out["seq_lens"]), ptr(out["query_start_loc"]),
            ptr(out["block_tables"]), mb, pad_block, ptr(out["slot_mapping"]),
            ptr(out["preempted"]) if P else None))
        no, ni, ns = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check("pa_sched_get_swaps", lib().pa_sched_get_swaps(
            self._h, ctypes.byref(no), ctypes.byref(ni), None, None, None, ctypes.byref(ns)))
        out["swap_out"] = np.zeros((no.value, 2), np.int64)
        out["swap_in"] = np.zeros((ni.value, 2), np.int64)
        out["swapped_out"] = np.zeros(ns.value, np.int64)
        _check("pa_sched_get_swaps", lib().pa_sched_get_swaps(
            self._h, ctypes.byref(no), ctypes.byref(ni), ptr(out["swap_out"]),
            ptr(out["swap_in"]), ptr(out["swapped_out"]), ctypes.byref(ns)))
        return out

    def update(self, sampled: dict) -> None:
        np = self._np
        ids = np.ascontiguousarray(np.fromiter(sampled.keys(), np.int64, len(sampled)))
        toks = np.ascontiguousarray(np.fromiter(sampled.values(), np.int32, len(sampled)))
        _check("pa_sched_update", lib().pa_sched_update(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), toks.ctypes.data_as(ctypes.c_void_p),
            len(sampled)))

    def block_refcounts(self):
        out = self._np.zeros(self.num_blocks, self._np.int32)
        _check("pa_sched_block_refcounts", lib().pa_sched_block_refcounts(
            self._h, out.ctypes.data_as(ctypes.c_void_p), self.num_blocks))
        return out

    def counts(self):
        w, r, f = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check("pa_sched_counts", lib().pa_sched_counts(self._h, ctypes.byref(w),
                                                        ctypes.byref(r), ctypes.byref(f)))
        return w.value, r.value, f.value
