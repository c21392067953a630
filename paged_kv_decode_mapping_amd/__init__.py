"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over libpa.so, the C ABI declared in include/pa.h.
The functions keep the C names (`pa_cache_write`, `pa_decode`, ...) and only
marshal arguments: they check shapes and dtypes, pass `data_ptr()`s, sizes
and torch's current HIP stream, and turn a negative status into an
exception. Every step of the computation runs in the HIP kernels; there is
no fallback: if libpa.so is missing or fails to load, the calls raise.

Build the library first:  python -m paged_kv_decode_mapping_amd.build
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libpa.so")

PA_OK = 0
PA_ERR_NULL = -1
PA_ERR_SHAPE = -2
PA_ERR_UNSUPPORTED = -3
PA_ERR_ALIGN = -4
PA_ERR_DTYPE = -5
PA_ERR_WORKSPACE = -6
PA_ERR_LAUNCH = -7
PA_ERR_DEVICE = -8
PA_ERR_PRECONDITION = -9
PA_KV_BF16 = 1
PA_KV_FP8_E4M3FN = 2
PA_VARIANT_AUTO = 0
PA_VARIANT_VALU = 1
PA_VARIANT_MFMA = 2
_VARIANTS = {"auto": PA_VARIANT_AUTO, "valu": PA_VARIANT_VALU, "mfma": PA_VARIANT_MFMA}

_lib = None


class PAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} (status {status})")


class pa_decode_opts(ctypes.Structure):
    _fields_ = [("partition_tokens", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("waves_per_group", ctypes.c_int32), ("prefetch_tiles", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("heads_per_tile", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class pa_decode_plan(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("waves_per_group", ctypes.c_int32),
                ("partition_tokens", ctypes.c_int32), ("num_partitions", ctypes.c_int32),
                ("prefetch_tiles", ctypes.c_int32), ("scheduled", ctypes.c_int32),
                ("num_workgroups", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
                ("heads_per_tile", ctypes.c_int32)]


def load_library(path: Optional[str] = None):
    """Load libpa.so (after torch, so that both share torch's HIP runtime)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    import torch  # noqa: F401  (brings in the HIP runtime libpa links against)
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run: python -m paged_kv_decode_mapping_amd.build")
    lib = ctypes.CDLL(p)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.pa_cache_write.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i64, i32, f32, f32, P]
    lib.pa_cache_write.restype = ctypes.c_int
    lib.pa_decode.argtypes = [P, P, P, P, P, f32, P, i32, i32, i32, i32, i32, i32, i64, i32, f32, f32,
                              P, sz, ctypes.POINTER(pa_decode_opts), P]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_get_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(pa_decode_opts),
                                       ctypes.POINTER(pa_decode_plan)]
    lib.pa_decode_get_plan.restype = ctypes.c_int
    lib.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(pa_decode_opts)]
    lib.pa_decode_workspace_size.restype = sz
    lib.pa_fp8_e4m3fn_encode_host.argtypes = [P, P, i64]
    lib.pa_fp8_e4m3fn_encode_host.restype = None
    lib.pa_decode_multi.argtypes = [P, P, P, P, P, P, f32, P, i32, i32, i32, i32, i32, i32, i32, i32, i64,
                                    i32, f32, f32, P, sz, i32, P]
    lib.pa_decode_multi.restype = ctypes.c_int
    lib.pa_decode_multi_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32]
    lib.pa_decode_multi_workspace_size.restype = sz
    lib.pa_decode_cascade.argtypes = [P, P, P, P, P, P, P, P, f32, P, i32, i32, i32, i32, i32, i32, i64,
                                      i32, i32, i32, i32, f32, f32, P, sz, ctypes.POINTER(pa_decode_opts), P]
    lib.pa_decode_cascade.restype = ctypes.c_int
    lib.pa_decode_cascade_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                                     ctypes.POINTER(pa_decode_opts)]
    lib.pa_decode_cascade_workspace_size.restype = sz
    lib.pa_check_cascade_inputs.argtypes = [P, P, P, i32, i32, i32, i32, i32, i64, P]
    lib.pa_check_cascade_inputs.restype = ctypes.c_int
    lib.pa_probe_stream_read.argtypes = [P, i64, i32, P, P]
    lib.pa_probe_stream_read.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [P, P, P, i64, i32, i32, i32, i64, i32, P]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_check_cache_write_inputs.argtypes = [P, i64, i32, i64, P]
    lib.pa_check_cache_write_inputs.restype = ctypes.c_int
    lib.pa_check_decode_inputs.argtypes = [P, P, i32, i32, i32, i64, P]
    lib.pa_check_decode_inputs.restype = ctypes.c_int
    lib.pa_strerror.argtypes = [ctypes.c_int]
    lib.pa_strerror.restype = ctypes.c_char_p
    lib.pa_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().pa_strerror(int(status)).decode()


def _opts(partition_tokens: int = 0, variant="auto", waves: int = 0, prefetch: int = 0,
          schedule: int = 0, heads_per_tile: int = 0) -> pa_decode_opts:
    v = _VARIANTS[variant] if isinstance(variant, str) else int(variant)
    return pa_decode_opts(int(partition_tokens), v, int(waves), int(prefetch), int(schedule), int(heads_per_tile), 0)


def _kv_dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return PA_KV_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_KV_FP8_E4M3FN
    raise TypeError(f"KV cache dtype {t.dtype} is not bfloat16 or float8_e4m3fn/uint8")


def _stream_ptr(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _check(t, name, dtype=None, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def pa_cache_write(k, v, slot_mapping, k_cache, v_cache, k_scale: float = 1.0, v_scale: float = 1.0,
                   stream=None) -> None:
    """Write new tokens' K/V rows [T, Hkv, D] into the caches [N, bs, Hkv, D] at slot_mapping [T]."""
    import torch
    lib = load_library()
    _check(k, "k", torch.bfloat16, 3)
    _check(v, "v", torch.bfloat16, 3)
    _check(slot_mapping, "slot_mapping", torch.int64, 1)
    _check(k_cache, "k_cache", None, 4)
    _check(v_cache, "v_cache", None, 4)
    kvd = _kv_dtype(k_cache)
    if _kv_dtype(v_cache) != kvd:
        raise TypeError("k_cache and v_cache dtypes differ")
    N, bs, Hkv, D = k_cache.shape
    T = k.shape[0]
    if k.shape != (T, Hkv, D) or v.shape != (T, Hkv, D) or slot_mapping.shape != (T,) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    st = lib.pa_cache_write(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
                            v_cache.data_ptr(), T, Hkv, D, bs, N, kvd, float(k_scale), float(v_scale),
                            _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_cache_write")


def pa_decode_multi(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
                    max_query_len: int, out=None, *, k_scale: float = 1.0, v_scale: float = 1.0,
                    workspace=None, partition_tokens: int = 0, stream=None):
    """Multi-token paged attention: q [T_q, Hq, D] bf16, query_start [S + 1]
    int32; the last query_start[i+1] - query_start[i] of sequence i's
    context_lens[i] cached tokens attend causally. Returns out [T_q, Hq, D]."""
    import torch
    lib = load_library()
    _check(q, "q", torch.bfloat16, 3)
    _check(k_cache, "k_cache", None, 4)
    _check(v_cache, "v_cache", None, 4)
    _check(block_tables, "block_tables", torch.int32, 2)
    _check(context_lens, "context_lens", torch.int32, 1)
    _check(query_start, "query_start", torch.int32, 1)
    kvd = _kv_dtype(k_cache)
    if _kv_dtype(v_cache) != kvd or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache differ")
    Tq, Hq, D = q.shape
    N, bs, Hkv, D2 = k_cache.shape
    S = context_lens.shape[0]
    if D2 != D or block_tables.shape[0] != S or query_start.shape != (S + 1,):
        raise ValueError("shape mismatch")
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, 3)
        if out.shape != q.shape:
            raise ValueError("out shape")
    need = lib.pa_decode_multi_workspace_size(S, Tq, int(max_query_len), Hq, Hkv, D, bs, MB, kvd,
                                              int(partition_tokens))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.pa_decode_multi(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                             context_lens.data_ptr(), query_start.data_ptr(), float(scale), out.data_ptr(), S, Tq,
                             int(max_query_len), Hq, Hkv, D, bs, MB, N, kvd, float(k_scale), float(v_scale),
                             ws_ptr, ws_bytes, int(partition_tokens), _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_decode_multi")
    return out


def pa_decode_multi_workspace_size(num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads,
                                   head_dim, block_size, max_blocks_per_seq, kv_dtype=PA_KV_BF16,
                                   partition_tokens=0) -> int:
    return int(load_library().pa_decode_multi_workspace_size(num_seqs, num_query_tokens, max_query_len,
                                                             num_q_heads, num_kv_heads, head_dim, block_size,
                                                             max_blocks_per_seq, kv_dtype, partition_tokens))


def pa_copy_blocks(k_cache, v_cache, block_mapping, stream=None) -> None:
    """Copy whole physical blocks of both caches [N, bs, Hkv, D] for (src, dst)
    pairs block_mapping [n, 2] int64 (copy-on-write's copy)."""
    import torch
    lib = load_library()
    _check(k_cache, "k_cache", None, 4)
    _check(v_cache, "v_cache", None, 4)
    _check(block_mapping, "block_mapping", torch.int64, 2)
    kvd = _kv_dtype(k_cache)
    if _kv_dtype(v_cache) != kvd or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache differ")
    if block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [n, 2]")
    N, bs, Hkv, D = k_cache.shape
    st = lib.pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), block_mapping.data_ptr(),
                            block_mapping.shape[0], Hkv, D, bs, N, kvd, _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_copy_blocks")


def pa_decode_get_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                       kv_dtype=PA_KV_BF16, partition_tokens=0, variant="auto", waves=0, prefetch=0,
                       schedule=0, heads_per_tile=0) -> dict:
    lib = load_library()
    o = _opts(partition_tokens, variant, waves, prefetch, schedule, heads_per_tile)
    p = pa_decode_plan()
    st = lib.pa_decode_get_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, kv_dtype, ctypes.byref(o), ctypes.byref(p))
    if st != PA_OK:
        raise PAError(st, "pa_decode_get_plan")
    return {"variant": {1: "valu", 2: "mfma"}[p.variant], "waves_per_group": p.waves_per_group,
            "partition_tokens": p.partition_tokens, "num_partitions": p.num_partitions,
            "prefetch_tiles": p.prefetch_tiles, "scheduled": bool(p.scheduled),
            "num_workgroups": p.num_workgroups,
            "workspace_bytes": p.workspace_bytes, "heads_per_tile": p.heads_per_tile}


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, out=None, *,
              k_scale: float = 1.0, v_scale: float = 1.0, workspace=None, partition_tokens: int = 0,
              variant="auto", waves: int = 0, prefetch: int = 0, schedule: int = 0, heads_per_tile: int = 0,
              stream=None):
    """Decode step: q [S, Hq, D] bf16 attends through block_tables [S, MB] int32 and
    context_lens [S] int32 over the paged caches [N, bs, Hkv, D]. Returns out [S, Hq, D] bf16.

    `workspace` (a uint8 device tensor, 256-byte aligned) is allocated here when
    the plan needs one and none is passed."""
    import torch
    lib = load_library()
    _check(q, "q", torch.bfloat16, 3)
    _check(k_cache, "k_cache", None, 4)
    _check(v_cache, "v_cache", None, 4)
    _check(block_tables, "block_tables", torch.int32, 2)
    _check(context_lens, "context_lens", torch.int32, 1)
    kvd = _kv_dtype(k_cache)
    if _kv_dtype(v_cache) != kvd or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache differ")
    S, Hq, D = q.shape
    N, bs, Hkv, D2 = k_cache.shape
    if D2 != D or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("shape mismatch")
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, 3)
        if out.shape != q.shape:
            raise ValueError("out shape")
    o = _opts(partition_tokens, variant, waves, prefetch, schedule, heads_per_tile)
    need = lib.pa_decode_workspace_size(S, Hq, Hkv, D, bs, MB, kvd, ctypes.byref(o))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.pa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                       context_lens.data_ptr(), float(scale), out.data_ptr(), S, Hq, Hkv, D, bs, MB, N,
                       kvd, float(k_scale), float(v_scale), ws_ptr, ws_bytes, ctypes.byref(o),
                       _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_decode")
    return out


def pa_decode_cascade(q, k_cache, v_cache, block_tables, context_lens, prefix_tables, prefix_lens, group_start,
                      scale: float, out=None, *, max_group_size: int, k_scale: float = 1.0, v_scale: float = 1.0,
                      workspace=None, partition_tokens: int = 0, variant="auto", waves: int = 0, prefetch: int = 0,
                      heads_per_tile: int = 0, stream=None):
    """Decode step for a batch whose prefix groups (sequences group_start[k] ..
    group_start[k+1] - 1) share a cached prefix: prefix_tables [G, PMB] int32
    and prefix_lens [G] int32 name each prefix's blocks and length; each
    prefix is read once per group. max_group_size (host) bounds the group
    sizes. Otherwise as pa_decode; returns out [S, Hq, D] bf16."""
    import torch
    lib = load_library()
    _check(q, "q", torch.bfloat16, 3)
    _check(k_cache, "k_cache", None, 4)
    _check(v_cache, "v_cache", None, 4)
    _check(block_tables, "block_tables", torch.int32, 2)
    _check(context_lens, "context_lens", torch.int32, 1)
    _check(prefix_tables, "prefix_tables", torch.int32, 2)
    _check(prefix_lens, "prefix_lens", torch.int32, 1)
    _check(group_start, "group_start", torch.int32, 1)
    kvd = _kv_dtype(k_cache)
    if _kv_dtype(v_cache) != kvd or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache differ")
    S, Hq, D = q.shape
    N, bs, Hkv, D2 = k_cache.shape
    G, PMB = prefix_tables.shape
    if D2 != D or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("shape mismatch")
    if prefix_lens.shape != (G,) or group_start.shape != (G + 1,):
        raise ValueError("group arrays: prefix_lens [G], group_start [G + 1]")
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, 3)
        if out.shape != q.shape:
            raise ValueError("out shape")
    o = _opts(partition_tokens, variant, waves, prefetch, 0, heads_per_tile)
    need = lib.pa_decode_cascade_workspace_size(S, Hq, Hkv, D, bs, MB, G, int(max_group_size), PMB, kvd,
                                                ctypes.byref(o))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ptr = lambda t: t.data_ptr() if t.numel() else None
    st = lib.pa_decode_cascade(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                               context_lens.data_ptr(), ptr(prefix_tables), ptr(prefix_lens), ptr(group_start),
                               float(scale), out.data_ptr(), S, Hq, Hkv, D, bs, MB, N, G, int(max_group_size),
                               PMB, kvd, float(k_scale), float(v_scale), ws_ptr, ws_bytes, ctypes.byref(o),
                               _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_decode_cascade")
    return out


def pa_decode_cascade_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                     max_blocks_per_seq, num_groups, max_group_size, max_prefix_blocks,
                                     kv_dtype=PA_KV_BF16, partition_tokens=0, variant="auto", waves=0,
                                     prefetch=0, heads_per_tile=0) -> int:
    o = _opts(partition_tokens, variant, waves, prefetch, 0, heads_per_tile)
    return int(load_library().pa_decode_cascade_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_groups,
        max_group_size, max_prefix_blocks, kv_dtype, ctypes.byref(o)))


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                             kv_dtype=PA_KV_BF16, partition_tokens=0, variant="auto", waves=0, prefetch=0,
                             schedule=0, heads_per_tile=0) -> int:
    o = _opts(partition_tokens, variant, waves, prefetch, schedule, heads_per_tile)
    return int(load_library().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                       block_size, max_blocks_per_seq, kv_dtype,
                                                       ctypes.byref(o)))


def pa_check_cache_write_inputs(slot_mapping, num_blocks: int, block_size: int, stream=None) -> int:
    """Check pa_cache_write's device-side preconditions (slots distinct, each
    negative or inside the pool). Synchronises. Returns PA_OK or
    PA_ERR_PRECONDITION; raises on argument errors."""
    import torch
    lib = load_library()
    _check(slot_mapping, "slot_mapping", torch.int64, 1)
    st = lib.pa_check_cache_write_inputs(slot_mapping.data_ptr(), slot_mapping.numel(), int(block_size),
                                         int(num_blocks), _stream_ptr(stream))
    if st not in (PA_OK, PA_ERR_PRECONDITION):
        raise PAError(st, "pa_check_cache_write_inputs")
    return st


def pa_check_decode_inputs(block_tables, context_lens, num_blocks: int, block_size: int, stream=None) -> int:
    """Check pa_decode's device-side preconditions (lengths within the table
    row, covering table entries inside the pool). Synchronises. Returns PA_OK
    or PA_ERR_PRECONDITION; raises on argument errors."""
    import torch
    lib = load_library()
    _check(block_tables, "block_tables", torch.int32, 2)
    _check(context_lens, "context_lens", torch.int32, 1)
    S, MB = block_tables.shape
    if context_lens.shape != (S,):
        raise ValueError("shape mismatch")
    st = lib.pa_check_decode_inputs(block_tables.data_ptr(), context_lens.data_ptr(), S, int(block_size), MB,
                                    int(num_blocks), _stream_ptr(stream))
    if st not in (PA_OK, PA_ERR_PRECONDITION):
        raise PAError(st, "pa_check_decode_inputs")
    return st


def pa_check_cascade_inputs(prefix_tables, prefix_lens, group_start, num_seqs: int, max_group_size: int,
                            num_blocks: int, block_size: int, stream=None) -> int:
    """Check pa_decode_cascade's group arrays (offsets rising within the batch,
    group sizes, whole-block prefix lengths within the table row, covering
    prefix table entries inside the pool). Synchronises. Returns PA_OK or
    PA_ERR_PRECONDITION; raises on argument errors."""
    import torch
    lib = load_library()
    _check(prefix_tables, "prefix_tables", torch.int32, 2)
    _check(prefix_lens, "prefix_lens", torch.int32, 1)
    _check(group_start, "group_start", torch.int32, 1)
    G, PMB = prefix_tables.shape
    if prefix_lens.shape != (G,) or group_start.shape != (G + 1,):
        raise ValueError("group arrays: prefix_lens [G], group_start [G + 1]")
    ptr = lambda t: t.data_ptr() if t.numel() else None
    st = lib.pa_check_cascade_inputs(ptr(prefix_tables), ptr(prefix_lens), ptr(group_start), G,
                                     int(max_group_size), PMB, int(num_seqs), int(block_size), int(num_blocks),
                                     _stream_ptr(stream))
    if st not in (PA_OK, PA_ERR_PRECONDITION):
        raise PAError(st, "pa_check_cascade_inputs")
    return st


def pa_probe_stream_read(buf, sink, nontemporal: bool = True, stream=None) -> None:
    """Read every byte of the device tensor `buf` once (a streaming-read
    reference kernel); `sink` is a device int32/uint32 tensor of >= 256 entries."""
    lib = load_library()
    _check(buf, "buf")
    _check(sink, "sink")
    if sink.numel() < 256 or sink.element_size() != 4:
        raise ValueError("sink must hold at least 256 32-bit words")
    st = lib.pa_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), 1 if nontemporal else 0,
                                  sink.data_ptr(), _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_probe_stream_read")


def fp8_encode_host(x) -> "numpy.ndarray":
    """The kernels' fp8 encoder run on the host (float32 inputs already divided by the scale)."""
    import numpy as np
    lib = load_library()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib.pa_fp8_e4m3fn_encode_host(x.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p), x.size)
    return out
