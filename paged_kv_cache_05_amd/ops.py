"""Thin ctypes binding over libpa.so (argument marshalling only).

Every function takes torch tensors that already live on the GPU, checks their shapes and
dtypes, and calls the C entry point of the same name on the current HIP stream.  All work runs
in the library's kernels; nothing here computes.  If ``libpa.so`` has not been built, or a
tensor is not on the GPU, the call raises -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import pathlib
import re

LIB_PATH = pathlib.Path(__file__).resolve().with_name("libpa.so")
HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "pa.h"

PA_OK = 0
KERNELS = {"auto": 0, "valu": 1, "mfma": 2}
PA_DECODE_SHARED_BLOCKS = 0x1


class PaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None

_c_int, _c_size, _c_float, _p = ctypes.c_int32, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p

_SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [_c_int]),
    "pa_version": (_c_int, []),
    "pa_decode_auto_partition": (_c_int, [_c_int] * 6),
    "pa_decode_workspace_bytes": (_c_size, [_c_int] * 7),
    "pa_decode": (_c_int, [_p] * 6 + [_c_int] * 7 + [_c_float, _c_int, _c_int, _p, _c_size, _p]),
    "pa_decode_ex": (_c_int, [_p] * 6 + [_c_int] * 7 + [_c_float, _c_int, _c_int, _p, _c_size,
                                                          _c_int, ctypes.c_uint32, _p]),
    "pa_decode_partitions": (_c_int, [_p] * 6 + [_c_int] * 7 + [_c_float, _c_int, _c_int, _p,
                                                                  _c_size, _c_int, ctypes.c_uint32,
                                                                  _p]),
    "pa_decode_merge": (_c_int, [_p, _p] + [_c_int] * 8 + [_p, _c_size, _p]),
    "pa_reshape_and_cache": (_c_int, [_p] * 5 + [_c_int] * 6 + [_p]),
    "pa_copy_blocks": (_c_int, [_p] * 3 + [_c_int] * 6 + [_p]),
    "pa_swap_blocks": (_c_int, [_p, _p, _c_int, _p, _p, _c_int, _p] + [_c_int] * 5 + [_p]),
    "pa_prefill": (_c_int, [_p] * 7 + [_c_int] * 8 + [_c_float, _c_int, ctypes.c_uint32, _p]),
    "pa_prefill_workspace_bytes": (_c_size, [_c_int] * 9),
    "pa_prefill_ex": (_c_int, [_p] * 7 + [_c_int] * 9 + [_c_float, _c_int, _c_int, _p, _c_size,
                                                       ctypes.c_uint32, _p]),
    "pa_append_slots": (_c_int, [_p] * 5 + [_c_int] * 4 + [_p, _c_int] + [_p] * 4 + [_p]),
    "pa_fork_seqs": (_c_int, [_p] * 3 + [_c_int] * 4 + [_p, _c_int, _p]),
    "pa_free_seqs": (_c_int, [_p] * 5 + [_c_int] * 4 + [_p, _c_int, _p]),
    "pa_copy_blocks_counted": (_c_int, [_p] * 4 + [_c_int] * 6 + [_p]),
    "pa_block_hashes": (_c_int, [_p, _p] + [_c_int] * 3 + [_p, _p]),
    "pa_reshape_and_cache_fp8": (_c_int, [_p] * 5 + [_c_int] * 6 + [_c_float, _c_float, _p]),
    "pa_decode_fp8": (_c_int, [_p] * 6 + [_c_int] * 7 + [_c_float, _c_int, _c_float, _c_float,
                                                      _c_int, _p, _c_size, ctypes.c_uint32, _p]),
    "pa_decode_fp8_partitions": (_c_int, [_p] * 6 + [_c_int] * 7 + [_c_float, _c_int, _c_float,
                                                                 _c_float, _c_int, _p, _c_size,
                                                                 ctypes.c_uint32, _p]),
    "pa_read_tiles": (_c_int, [_p, ctypes.c_int64, _c_int, _p, _c_int, _p, _p]),
    "pa_prefill_fp8": (_c_int, [_p] * 7 + [_c_int] * 9 + [_c_float, _c_int, _c_float, _c_float,
                                                       _c_int, _p, _c_size, ctypes.c_uint32, _p]),
}


def header_symbols() -> list[str]:
    """Every function include/pa.h declares."""
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(pa_\w+)\s*\(", text, re.M)))


def load():
    """Load libpa.so (once); raises if it has not been built.

    torch is imported first: it loads its own copy of the HIP runtime, whose soname
    (libamdhip64.so.7) is the one libpa.so links against, so the library binds to that copy.
    Loaded before torch, libpa.so would pull in the system copy as well, and its calls would go
    to a second runtime that does not see torch's device state (its hipGetDevice reports no
    device)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "paged_kv_cache_05_amd.build.build() (hipcc, gfx950)")
        lib = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().pa_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != PA_OK:
        raise PaError(status, f"{what}: {status_string(status)}")


# ---------------------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.uint8: 3,
             torch.float8_e4m3fn: 3}
    if t.dtype not in codes:
        raise TypeError(f"unsupported element type {t.dtype}")
    return codes[t.dtype]


def _dev(*tensors):
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("every tensor must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors are on different devices")
    return dev


def _stream(dev, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                    partition_size=0) -> int:
    return int(load().pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                block_size, max_blocks_per_seq, partition_size))


def auto_partition(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq) -> int:
    return int(load().pa_decode_auto_partition(num_seqs, num_heads, num_kv_heads, head_dim,
                                               block_size, max_blocks_per_seq))


def _decode_shapes(out, query, key_cache, value_cache, block_tables, context_lens):
    import torch
    S, Hq, D = query.shape
    NB, Hkv, BS, D2 = key_cache.shape
    if tuple(value_cache.shape) != tuple(key_cache.shape) or D2 != D:
        raise ValueError("key_cache/value_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    if tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must have the query's shape")
    if not (out.dtype == query.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("out, query and both pools must share one element type")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs, max_blocks] and context_lens [num_seqs]")
    return S, Hq, Hkv, D, BS, NB, block_tables.shape[1]


def decode(out, query, key_cache, value_cache, block_tables, context_lens, scale, *,
           partition_size=0, kernel="auto", shared_blocks=False, workspace=None, stream=None):
    """pa_decode_ex: paged decode attention into ``out`` ([S, Hq, d]).  ``shared_blocks``
    sets PA_DECODE_SHARED_BLOCKS (blocks read by several sequences: cache-allocating loads)."""
    import torch
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens, workspace)
    S, Hq, Hkv, D, BS, NB, maxb = _decode_shapes(out, query, key_cache, value_cache, block_tables,
                                                 context_lens)
    need = workspace_bytes(S, Hq, Hkv, D, BS, maxb, partition_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pa_decode_ex(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                               _ptr(block_tables), _ptr(context_lens), S, Hq, Hkv, D, BS, NB, maxb,
                               float(scale), _dtype_code(query), int(partition_size),
                               _ptr(workspace), wsb, KERNELS[kernel],
                               PA_DECODE_SHARED_BLOCKS if shared_blocks else 0, _stream(dev, stream)),
           "pa_decode_ex")
    return out


def decode_partitions(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                      workspace, *, partition_size=0, kernel="auto", shared_blocks=False,
                      stream=None):
    """pa_decode_partitions: the first of pa_decode's two launches."""
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens, workspace)
    S, Hq, Hkv, D, BS, NB, maxb = _decode_shapes(out, query, key_cache, value_cache, block_tables,
                                                 context_lens)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pa_decode_partitions(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                       _ptr(block_tables), _ptr(context_lens), S, Hq, Hkv, D, BS,
                                       NB, maxb, float(scale), _dtype_code(query),
                                       int(partition_size), _ptr(workspace), wsb, KERNELS[kernel],
                                       PA_DECODE_SHARED_BLOCKS if shared_blocks else 0,
                                       _stream(dev, stream)), "pa_decode_partitions")


def decode_merge(out, context_lens, num_kv_heads, block_size, max_blocks_per_seq, workspace, *,
                 partition_size=0, stream=None):
    """pa_decode_merge: the second of pa_decode's two launches."""
    dev = _dev(out, context_lens, workspace)
    S, Hq, D = out.shape
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pa_decode_merge(_ptr(out), _ptr(context_lens), S, Hq, num_kv_heads, D,
                                  block_size, max_blocks_per_seq, _dtype_code(out),
                                  int(partition_size), _ptr(workspace), wsb, _stream(dev, stream)),
           "pa_decode_merge")


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, *, stream=None):
    """pa_reshape_and_cache: store key/value [N, Hkv, d] at slot_mapping [N] (int64)."""
    import torch
    dev = _dev(key, value, key_cache, value_cache, slot_mapping)
    N, Hkv, D = key.shape
    NB, Hkv2, BS, D2 = key_cache.shape
    if (Hkv2, D2) != (Hkv, D) or tuple(value.shape) != tuple(key.shape) \
            or tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("shape mismatch between new tokens and the pools")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (N,):
        raise TypeError("slot_mapping must be int64 [num_tokens]")
    if not (key.dtype == value.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("key, value and both pools must share one element type")
    _check(load().pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                       _ptr(slot_mapping), N, Hkv, D, BS, NB, _dtype_code(key),
                                       _stream(dev, stream)), "pa_reshape_and_cache")


def copy_blocks(key_cache, value_cache, block_mapping, *, stream=None):
    """pa_copy_blocks: copy whole blocks src -> dst for each row of block_mapping [P, 2] (int64)."""
    import torch
    dev = _dev(key_cache, value_cache, block_mapping)
    NB, Hkv, BS, D = key_cache.shape
    if tuple(value_cache.shape) != tuple(key_cache.shape) or key_cache.dtype != value_cache.dtype:
        raise ValueError("key_cache and value_cache must match")
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise TypeError("block_mapping must be int64 [num_pairs, 2]")
    _check(load().pa_copy_blocks(_ptr(key_cache), _ptr(value_cache), _ptr(block_mapping),
                                 block_mapping.shape[0], Hkv, D, BS, NB, _dtype_code(key_cache),
                                 _stream(dev, stream)), "pa_copy_blocks")


def swap_blocks(src_key, src_value, dst_key, dst_value, block_mapping, *, stream=None):
    """pa_swap_blocks: copy whole blocks between two pools (GPU <-> pinned host), per row
    (src, dst) of block_mapping [P, 2] (int64, on the GPU or pinned).  Host pools must be
    pinned; the copy is asynchronous on the GPU stream."""
    import torch
    gpu = [t for t in (src_key, src_value, dst_key, dst_value, block_mapping) if t.is_cuda]
    if not gpu:
        raise ValueError("at least one pool must be on the GPU")
    dev = gpu[0].device
    for t in (src_key, src_value, dst_key, dst_value, block_mapping):
        if not t.is_contiguous():
            raise ValueError("every tensor must be contiguous")
        if t.is_cuda and t.device != dev:
            raise ValueError("GPU tensors are on different devices")
        if not t.is_cuda and not t.is_pinned():
            raise ValueError("host tensors must be pinned (pin_memory=True)")
    NS, Hkv, BS, D = src_key.shape
    ND = dst_key.shape[0]
    if tuple(src_value.shape) != tuple(src_key.shape) or tuple(dst_value.shape) != tuple(dst_key.shape) \
            or tuple(dst_key.shape[1:]) != (Hkv, BS, D):
        raise ValueError("pools must be [blocks, num_kv_heads, block_size, head_dim] with equal block shape")
    if not (src_key.dtype == src_value.dtype == dst_key.dtype == dst_value.dtype):
        raise TypeError("all pools must share one element type")
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise TypeError("block_mapping must be int64 [num_pairs, 2]")
    _check(load().pa_swap_blocks(_ptr(src_key), _ptr(src_value), NS, _ptr(dst_key), _ptr(dst_value),
                                 ND, _ptr(block_mapping), block_mapping.shape[0], Hkv, D, BS,
                                 _dtype_code(src_key), _stream(dev, stream)), "pa_swap_blocks")


PA_PREFILL_BF16_P = 0x1


def prefill_workspace_bytes(num_seqs, num_tokens, num_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, max_query_len, kv_split=0) -> int:
    return int(load().pa_prefill_workspace_bytes(num_seqs, num_tokens, num_heads, num_kv_heads,
                                                 head_dim, block_size, max_blocks_per_seq,
                                                 max_query_len, kv_split))


def prefill(out, query, key_cache, value_cache, block_tables, query_start_loc, context_lens, scale,
            max_query_len, *, bf16_p=False, kv_split=0, workspace=None, stream=None):
    """pa_prefill_ex: causal attention of each sequence's chunk of new tokens over the paged
    cache.

    ``query``/``out`` [T, Hq, d] hold the chunks back to back; sequence s owns rows
    ``query_start_loc[s] .. query_start_loc[s+1]-1`` (int32 [S+1]); ``context_lens`` (int32 [S])
    counts the cached tokens including the chunk.  ``max_query_len`` is a host integer no
    smaller than any chunk.  ``bf16_p`` sets PA_PREFILL_BF16_P.  ``kv_split``: tokens per key
    split (0: the library's choice); the workspace is allocated here when not given."""
    import torch
    dev = _dev(out, query, key_cache, value_cache, block_tables, query_start_loc, context_lens)
    T, Hq, D = query.shape
    NB, Hkv, BS, D2 = key_cache.shape
    S = context_lens.shape[0]
    if tuple(value_cache.shape) != tuple(key_cache.shape) or D2 != D:
        raise ValueError("key_cache/value_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    if tuple(out.shape) != (T, Hq, D):
        raise ValueError("out must have the query's shape")
    if not (out.dtype == query.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("out, query and both pools must share one element type")
    if (block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32
            or query_start_loc.dtype != torch.int32):
        raise TypeError("block_tables, query_start_loc and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(query_start_loc.shape) != (S + 1,):
        raise ValueError("block_tables must be [S, max_blocks] and query_start_loc [S + 1]")
    maxb = block_tables.shape[1]
    need = prefill_workspace_bytes(S, T, Hq, Hkv, D, BS, maxb, int(max_query_len), int(kv_split))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(load().pa_prefill_ex(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                _ptr(block_tables), _ptr(query_start_loc), _ptr(context_lens), S,
                                T, Hq, Hkv, D, BS, NB, maxb, int(max_query_len), float(scale),
                                _dtype_code(query), int(kv_split), _ptr(workspace),
                                workspace.numel() if workspace is not None else 0,
                                PA_PREFILL_BF16_P if bf16_p else 0, _stream(dev, stream)),
           "pa_prefill_ex")
    return out


PA_FP8_E4M3 = 3


def _fp8_pools(key_cache, value_cache):
    import torch
    for t in (key_cache, value_cache):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError("8-bit pools must be uint8 or float8_e4m3fn tensors")
    if tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("key_cache and value_cache must match")
    return key_cache.shape


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale, *,
                          stream=None):
    """pa_reshape_and_cache_fp8: quantize key/value [N, Hkv, d] (f16/bf16) into E4M3 pools."""
    import torch
    dev = _dev(key, value, key_cache, value_cache, slot_mapping)
    NB, Hkv, BS, D = _fp8_pools(key_cache, value_cache)
    N = key.shape[0]
    if tuple(key.shape) != (N, Hkv, D) or tuple(value.shape) != (N, Hkv, D) or key.dtype != value.dtype:
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_dim] of one type")
    if slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != (N,):
        raise TypeError("slot_mapping must be int64 [num_tokens]")
    _check(load().pa_reshape_and_cache_fp8(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                           _ptr(slot_mapping), N, Hkv, D, BS, NB, _dtype_code(key),
                                           float(k_scale), float(v_scale), _stream(dev, stream)),
           "pa_reshape_and_cache_fp8")


def _decode_fp8_args(out, query, key_cache, value_cache, block_tables, context_lens):
    import torch
    S, Hq, D = query.shape
    NB, Hkv, BS, D2 = _fp8_pools(key_cache, value_cache)
    if D2 != D or tuple(out.shape) != (S, Hq, D) or out.dtype != query.dtype:
        raise ValueError("out must match the query; pools [num_blocks, num_kv_heads, block_size, head_dim]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [num_seqs, max_blocks] and context_lens [num_seqs]")
    return S, Hq, Hkv, D, BS, NB, block_tables.shape[1]


def decode_fp8(out, query, key_cache, value_cache, block_tables, context_lens, scale, k_scale,
               v_scale, *, partition_size=0, shared_blocks=False, workspace=None, stream=None):
    """pa_decode_fp8: paged decode attention over E4M3 pools (codes times k_scale / v_scale)."""
    import torch
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens, workspace)
    S, Hq, Hkv, D, BS, NB, maxb = _decode_fp8_args(out, query, key_cache, value_cache,
                                                   block_tables, context_lens)
    need = workspace_bytes(S, Hq, Hkv, D, BS, maxb, partition_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pa_decode_fp8(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                _ptr(block_tables), _ptr(context_lens), S, Hq, Hkv, D, BS, NB, maxb,
                                float(scale), _dtype_code(query), float(k_scale), float(v_scale),
                                int(partition_size), _ptr(workspace), wsb,
                                PA_DECODE_SHARED_BLOCKS if shared_blocks else 0,
                                _stream(dev, stream)), "pa_decode_fp8")
    return out


def decode_fp8_partitions(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                          k_scale, v_scale, workspace, *, partition_size=0, shared_blocks=False,
                          stream=None):
    """pa_decode_fp8_partitions: the first of pa_decode_fp8's two launches."""
    dev = _dev(out, query, key_cache, value_cache, block_tables, context_lens, workspace)
    S, Hq, Hkv, D, BS, NB, maxb = _decode_fp8_args(out, query, key_cache, value_cache,
                                                   block_tables, context_lens)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pa_decode_fp8_partitions(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                           _ptr(block_tables), _ptr(context_lens), S, Hq, Hkv, D,
                                           BS, NB, maxb, float(scale), _dtype_code(query),
                                           float(k_scale), float(v_scale), int(partition_size),
                                           _ptr(workspace), wsb,
                                           PA_DECODE_SHARED_BLOCKS if shared_blocks else 0,
                                           _stream(dev, stream)), "pa_decode_fp8_partitions")


def prefill_fp8(out, query, key_cache, value_cache, block_tables, query_start_loc, context_lens,
                scale, max_query_len, k_scale, v_scale, *, bf16_p=False, kv_split=0,
                workspace=None, stream=None):
    """pa_prefill_fp8: ``prefill`` over E4M3 pools (codes times k_scale / v_scale)."""
    import torch
    dev = _dev(out, query, key_cache, value_cache, block_tables, query_start_loc, context_lens)
    T, Hq, D = query.shape
    NB, Hkv, BS, D2 = _fp8_pools(key_cache, value_cache)
    S = context_lens.shape[0]
    if D2 != D or tuple(out.shape) != (T, Hq, D) or out.dtype != query.dtype:
        raise ValueError("out must match the query; pools [num_blocks, num_kv_heads, block_size, head_dim]")
    if (block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32
            or query_start_loc.dtype != torch.int32):
        raise TypeError("block_tables, query_start_loc and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(query_start_loc.shape) != (S + 1,):
        raise ValueError("block_tables must be [S, max_blocks] and query_start_loc [S + 1]")
    maxb = block_tables.shape[1]
    need = prefill_workspace_bytes(S, T, Hq, Hkv, D, BS, maxb, int(max_query_len), int(kv_split))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(load().pa_prefill_fp8(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                 _ptr(block_tables), _ptr(query_start_loc), _ptr(context_lens), S,
                                 T, Hq, Hkv, D, BS, NB, maxb, int(max_query_len), float(scale),
                                 _dtype_code(query), float(k_scale), float(v_scale), int(kv_split),
                                 _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                 PA_PREFILL_BF16_P if bf16_p else 0, _stream(dev, stream)),
           "pa_prefill_fp8")
    return out


# ---------------------------------------------------------------------------------------
# block engine on the device
# ---------------------------------------------------------------------------------------
def _engine(block_tables, context_lens, ref_counts, free_stack=None, free_top=None):
    import torch
    for t in (block_tables, context_lens, ref_counts, free_stack, free_top):
        if t is not None and t.dtype != torch.int32:
            raise TypeError("block-engine arrays are int32")
    if block_tables.dim() != 2 or context_lens.shape != (block_tables.shape[0],):
        raise ValueError("block_tables [num_seqs, max_blocks] and context_lens [num_seqs]")
    if free_stack is not None and free_stack.shape != ref_counts.shape:
        raise ValueError("free_stack must have one entry per block")
    return block_tables.shape[0], block_tables.shape[1], ref_counts.numel()


def append_slots(block_tables, context_lens, ref_counts, free_stack, free_top, seq_ids, block_size,
                 slot_mapping, block_mapping, num_pairs, status, *, stream=None):
    """pa_append_slots: one token per sequence in seq_ids (int32), with copy-on-write; writes
    slot_mapping (int64 [n]), block_mapping (int64 [n, 2]), num_pairs and status (int32 [1])."""
    import torch
    dev = _dev(block_tables, context_lens, ref_counts, free_stack, free_top, seq_ids, slot_mapping,
               block_mapping, num_pairs, status)
    S, maxb, NB = _engine(block_tables, context_lens, ref_counts, free_stack, free_top)
    n = seq_ids.numel()
    if slot_mapping.dtype != torch.int64 or block_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping and block_mapping are int64")
    if slot_mapping.numel() < n or block_mapping.numel() < 2 * n:
        raise ValueError("slot_mapping [n] and block_mapping [n, 2] needed")
    _check(load().pa_append_slots(_ptr(block_tables), _ptr(context_lens), _ptr(ref_counts),
                                  _ptr(free_stack), _ptr(free_top), S, maxb, int(block_size), NB,
                                  _ptr(seq_ids), n, _ptr(slot_mapping), _ptr(block_mapping),
                                  _ptr(num_pairs), _ptr(status), _stream(dev, stream)),
           "pa_append_slots")


def fork_seqs(block_tables, context_lens, ref_counts, parent_child, block_size, *, stream=None):
    """pa_fork_seqs: parent_child int32 [n, 2]."""
    dev = _dev(block_tables, context_lens, ref_counts, parent_child)
    S, maxb, NB = _engine(block_tables, context_lens, ref_counts)
    _check(load().pa_fork_seqs(_ptr(block_tables), _ptr(context_lens), _ptr(ref_counts), S, maxb,
                               int(block_size), NB, _ptr(parent_child), parent_child.shape[0],
                               _stream(dev, stream)), "pa_fork_seqs")


def free_seqs(block_tables, context_lens, ref_counts, free_stack, free_top, seq_ids, block_size, *,
              stream=None):
    """pa_free_seqs: seq_ids int32 [n]."""
    dev = _dev(block_tables, context_lens, ref_counts, free_stack, free_top, seq_ids)
    S, maxb, NB = _engine(block_tables, context_lens, ref_counts, free_stack, free_top)
    _check(load().pa_free_seqs(_ptr(block_tables), _ptr(context_lens), _ptr(ref_counts),
                               _ptr(free_stack), _ptr(free_top), S, maxb, int(block_size), NB,
                               _ptr(seq_ids), seq_ids.numel(), _stream(dev, stream)), "pa_free_seqs")


def copy_blocks_counted(key_cache, value_cache, block_mapping, num_pairs, max_pairs, *, stream=None):
    """pa_copy_blocks_counted: the pair count is read from num_pairs (int32 [1], on the GPU);
    block_mapping (int64 [>= max_pairs, 2]) holds max_pairs readable rows."""
    dev = _dev(key_cache, value_cache, block_mapping, num_pairs)
    NB, Hkv, BS, D = key_cache.shape
    if block_mapping.numel() < 2 * int(max_pairs):
        raise ValueError("block_mapping must hold max_pairs rows")
    _check(load().pa_copy_blocks_counted(_ptr(key_cache), _ptr(value_cache), _ptr(block_mapping),
                                         _ptr(num_pairs), int(max_pairs), Hkv, D, BS, NB,
                                         _dtype_code(key_cache), _stream(dev, stream)),
           "pa_copy_blocks_counted")


def block_hashes(token_ids, num_tokens, block_size, hashes, *, stream=None):
    """pa_block_hashes: token_ids int32 [S, T], num_tokens int32 [S] -> hashes [S, T // bs]
    (a 64-bit tensor; the bits are the unsigned FNV-1a values)."""
    import torch
    dev = _dev(token_ids, num_tokens, hashes)
    S, T = token_ids.shape
    if token_ids.dtype != torch.int32 or num_tokens.dtype != torch.int32:
        raise TypeError("token_ids and num_tokens are int32")
    if hashes.element_size() != 8 or tuple(hashes.shape) != (S, T // int(block_size)):
        raise ValueError("hashes must be 64-bit [num_seqs, max_tokens // block_size]")
    _check(load().pa_block_hashes(_ptr(token_ids), _ptr(num_tokens), S, T, int(block_size),
                                  _ptr(hashes), _stream(dev, stream)), "pa_block_hashes")


# ---------------------------------------------------------------------------------------
# read-only bandwidth probe
# ---------------------------------------------------------------------------------------
def read_tiles(buffer, tile_bytes, xor_out, tile_ids=None, *, stream=None):
    """pa_read_tiles: read tiles of ``tile_bytes`` bytes of ``buffer`` (any contiguous GPU
    tensor) -- tile t is tile ``tile_ids[t]`` (int32), or tile t itself when ``tile_ids`` is
    None -- and write the XOR of each tile's 32-bit words to ``xor_out`` (32-bit, one entry per
    tile read)."""
    import torch
    dev = _dev(buffer, xor_out, tile_ids)
    nbytes = buffer.numel() * buffer.element_size()
    if xor_out.element_size() != 4:
        raise TypeError("xor_out must hold 32-bit words")
    n = tile_ids.numel() if tile_ids is not None else xor_out.numel()
    if tile_ids is not None and tile_ids.dtype != torch.int32:
        raise TypeError("tile_ids must be int32")
    if xor_out.numel() < n:
        raise ValueError("xor_out needs one entry per tile read")
    _check(load().pa_read_tiles(_ptr(buffer), nbytes // int(tile_bytes), int(tile_bytes),
                                _ptr(tile_ids), n, _ptr(xor_out), _stream(dev, stream)),
           "pa_read_tiles")
