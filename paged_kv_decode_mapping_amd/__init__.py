"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over libpa.so, the C ABI declared in include/pa.h.
The functions keep the C names (`pa_cache_write`, `pa_decode`, ...) and only
marshal arguments: each torch tensor becomes a pa_tensor (data pointer,
element type, shape, strides), the stream is the caller's or torch's current
one, and a negative status becomes an exception. Shapes, types and strides
are checked by the library. Every step of the computation runs in the HIP kernels; there is
no fallback: if libpa.so is missing or fails to load, the calls raise.

Build the library first:  python -m paged_kv_decode_mapping_amd.build
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY names another build of libpa.so to load instead (the sanitizer
# test's instrumented host code)
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(PKG_DIR, "libpa.so")

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
PA_ERR_LAYOUT = -10
PA_ERR_SCRATCH = -11
PA_NO_ALLOC_SCRATCH = 32 << 20
PA_DTYPE_BF16 = 1
PA_DTYPE_FP8_E4M3FN = 2
PA_DTYPE_I32 = 4
PA_DTYPE_I64 = 5
# KV-cache element types (the cache tensors' dtype codes)
PA_KV_BF16 = PA_DTYPE_BF16
PA_KV_FP8_E4M3FN = PA_DTYPE_FP8_E4M3FN
PA_VARIANT_AUTO = 0
PA_VARIANT_VALU = 1
PA_VARIANT_MFMA = 2
_VARIANTS = {"auto": PA_VARIANT_AUTO, "valu": PA_VARIANT_VALU, "mfma": PA_VARIANT_MFMA}

_lib = None


class PAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} (status {status})")


class pa_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class pa_decode_opts(ctypes.Structure):
    _fields_ = [("partition_tokens", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("waves_per_group", ctypes.c_int32), ("prefetch_tiles", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("heads_per_tile", ctypes.c_int32),
                ("wave_partitions", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class pa_decode_plan(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("waves_per_group", ctypes.c_int32),
                ("partition_tokens", ctypes.c_int32), ("num_partitions", ctypes.c_int32),
                ("prefetch_tiles", ctypes.c_int32), ("scheduled", ctypes.c_int32),
                ("num_workgroups", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
                ("heads_per_tile", ctypes.c_int32), ("wave_partitions", ctypes.c_int32)]


class TensorSpec(NamedTuple):
    """Shape, element type (PA_DTYPE_*) and element strides of a tensor
    without data: what the plan and workspace-size calls read. stride None =
    contiguous."""
    shape: Tuple[int, ...]
    dtype: int
    stride: Optional[Tuple[int, ...]] = None


def contiguous_strides(shape) -> Tuple[int, ...]:
    st, acc = [], 1
    for n in reversed(shape):
        st.append(acc)
        acc *= int(n)
    return tuple(reversed(st))


def head_major_strides(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int) -> Tuple[int, ...]:
    """Strides of a pool stored as [N, Hkv, bs, D] and described as [N, bs, Hkv, D]."""
    return (num_kv_heads * block_size * head_dim, head_dim, block_size * head_dim, 1)


def decode_specs(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                 kv_dtype=PA_DTYPE_BF16, num_blocks=1, head_major=False):
    """(q, k_cache, block_tables) specs of a decode call with these sizes (for
    pa_decode_get_plan and the workspace-size calls)."""
    cshape = (num_blocks, block_size, num_kv_heads, head_dim)
    cst = head_major_strides(*cshape) if head_major else None
    return (TensorSpec((num_seqs, num_q_heads, head_dim), PA_DTYPE_BF16),
            TensorSpec(cshape, kv_dtype, cst),
            TensorSpec((num_seqs, max_blocks_per_seq), PA_DTYPE_I32))


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
    T = ctypes.POINTER(pa_tensor)
    O = ctypes.POINTER(pa_decode_opts)
    sigs = {
        "pa_cache_write": ([T, T, T, T, T, f32, f32, P], ctypes.c_int),
        "pa_copy_blocks": ([T, T, T, P], ctypes.c_int),
        "pa_decode": ([T, T, T, T, T, f32, T, f32, f32, P, sz, O, P], ctypes.c_int),
        "pa_decode_no_alloc": ([T, T, T, T, T, f32, T, f32, f32, O, P], ctypes.c_int),
        "pa_decode_get_plan": ([T, T, T, O, ctypes.POINTER(pa_decode_plan)], ctypes.c_int),
        "pa_decode_workspace_size": ([T, T, T, O], sz),
        "pa_decode_multi": ([T, T, T, T, T, T, f32, T, i32, f32, f32, P, sz, i32, P], ctypes.c_int),
        "pa_decode_multi_workspace_size": ([T, T, T, i32, i32], sz),
        "pa_decode_cascade": ([T, T, T, T, T, T, T, T, f32, T, i32, f32, f32, P, sz, O, P], ctypes.c_int),
        "pa_decode_cascade_workspace_size": ([T, T, T, T, i32, O], sz),
        "pa_check_cache_write_inputs": ([T, T, P], ctypes.c_int),
        "pa_check_decode_inputs": ([T, T, T, P], ctypes.c_int),
        "pa_check_multi_inputs": ([T, T, T, i32, T, P], ctypes.c_int),
        "pa_check_cascade_inputs": ([T, T, T, i32, i32, T, P], ctypes.c_int),
        "pa_probe_stream_read": ([P, i64, i32, P, P], ctypes.c_int),
        "pa_fp8_e4m3fn_encode_host": ([P, P, i64], None),
        "pa_strerror": ([ctypes.c_int], ctypes.c_char_p),
        "pa_version": ([], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().pa_strerror(int(status)).decode()


def _opts(partition_tokens: int = 0, variant="auto", waves: int = 0, prefetch: int = 0,
          schedule: int = 0, heads_per_tile: int = 0, wave_partitions: int = 0) -> pa_decode_opts:
    v = _VARIANTS[variant] if isinstance(variant, str) else int(variant)
    return pa_decode_opts(int(partition_tokens), v, int(waves), int(prefetch), int(schedule), int(heads_per_tile),
                          int(wave_partitions), 0)


def _dtype_code(t) -> int:
    import torch
    return {torch.bfloat16: PA_DTYPE_BF16, torch.float8_e4m3fn: PA_DTYPE_FP8_E4M3FN, torch.uint8: PA_DTYPE_FP8_E4M3FN,
            torch.int32: PA_DTYPE_I32, torch.int64: PA_DTYPE_I64}.get(t.dtype, 0)


def desc(t) -> Optional[pa_tensor]:
    """The pa_tensor of a device tensor or a TensorSpec (None stays None):
    data pointer, element type, shape and strides, passed as they are (the
    library checks them)."""
    if t is None:
        return None
    d = pa_tensor()
    if isinstance(t, TensorSpec):
        shape, stride = tuple(t.shape), tuple(t.stride) if t.stride is not None else contiguous_strides(t.shape)
        d.data, d.dtype = None, int(t.dtype)
    else:
        import torch
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"expected a torch.Tensor or TensorSpec, got {type(t).__name__}")
        if not t.is_cuda:
            raise ValueError("tensors passed to the library must be device tensors")
        shape, stride = tuple(t.shape), tuple(t.stride())
        d.data, d.dtype = (t.data_ptr() or None), _dtype_code(t)
    if not 1 <= len(shape) <= 4:
        raise ValueError(f"tensors of rank 1..4 only (got {len(shape)})")
    d.ndim = len(shape)
    for i, (n, st) in enumerate(zip(shape, stride)):
        d.shape[i] = int(n)
        d.stride[i] = int(st)
    return d


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _stream_ptr(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _new(stream, fn):
    """Allocate a tensor the call will use on `stream`: with torch's caching
    allocator on that stream, so the block cannot be handed to other work on
    another stream while the call's kernels still use it."""
    import torch
    if stream is None:
        return fn()
    with torch.cuda.stream(stream):
        return fn()


def _workspace(need: int, workspace, device, stream):
    import torch
    if need and workspace is None:
        workspace = _new(stream, lambda: torch.empty(need, dtype=torch.uint8, device=device))
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def pa_cache_write(k, v, slot_mapping, k_cache, v_cache, k_scale: float = 1.0, v_scale: float = 1.0,
                   stream=None) -> None:
    """Write new tokens' K/V rows [T, Hkv, D] into the caches [N, bs, Hkv, D] at slot_mapping [T]."""
    lib = load_library()
    d = [desc(t) for t in (k, v, slot_mapping, k_cache, v_cache)]
    st = lib.pa_cache_write(*map(_ref, d), float(k_scale), float(v_scale), _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_cache_write")


def pa_copy_blocks(k_cache, v_cache, block_mapping, stream=None) -> None:
    """Copy whole physical blocks of both caches [N, bs, Hkv, D] for (src, dst)
    pairs block_mapping [n, 2] int64 (copy-on-write's copy)."""
    lib = load_library()
    d = [desc(t) for t in (k_cache, v_cache, block_mapping)]
    st = lib.pa_copy_blocks(*map(_ref, d), _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_copy_blocks")


def _plan_dict(p) -> dict:
    return {"variant": {1: "valu", 2: "mfma"}[p.variant], "waves_per_group": p.waves_per_group,
            "partition_tokens": p.partition_tokens, "num_partitions": p.num_partitions,
            "prefetch_tiles": p.prefetch_tiles, "scheduled": bool(p.scheduled),
            "self_scheduled": p.scheduled == 2,
            "num_workgroups": p.num_workgroups,
            "workspace_bytes": p.workspace_bytes, "heads_per_tile": p.heads_per_tile,
            "wave_partitions": bool(p.wave_partitions)}


def pa_decode_get_plan(q, k_cache, block_tables, *, partition_tokens=0, variant="auto", waves=0, prefetch=0,
                       schedule=0, heads_per_tile=0, wave_partitions=0) -> dict:
    """The launch plan pa_decode would use (tensors or TensorSpecs; see decode_specs)."""
    lib = load_library()
    o = _opts(partition_tokens, variant, waves, prefetch, schedule, heads_per_tile, wave_partitions)
    p = pa_decode_plan()
    d = [desc(t) for t in (q, k_cache, block_tables)]
    st = lib.pa_decode_get_plan(*map(_ref, d), ctypes.byref(o), ctypes.byref(p))
    if st != PA_OK:
        raise PAError(st, "pa_decode_get_plan")
    return _plan_dict(p)


def pa_decode_workspace_size(q, k_cache, block_tables, *, partition_tokens=0, variant="auto", waves=0, prefetch=0,
                             schedule=0, heads_per_tile=0, wave_partitions=0) -> int:
    o = _opts(partition_tokens, variant, waves, prefetch, schedule, heads_per_tile, wave_partitions)
    d = [desc(t) for t in (q, k_cache, block_tables)]
    return int(load_library().pa_decode_workspace_size(*map(_ref, d), ctypes.byref(o)))


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, out=None, *,
              k_scale: float = 1.0, v_scale: float = 1.0, workspace=None, partition_tokens: int = 0,
              variant="auto", waves: int = 0, prefetch: int = 0, schedule: int = 0, heads_per_tile: int = 0,
              wave_partitions: int = 0, stream=None):
    """Decode step: q [S, Hq, D] bf16 attends through block_tables [S, MB] int32 and
    context_lens [S] int32 over the paged caches [N, bs, Hkv, D] (any strides the
    library accepts). Returns out [S, Hq, D] bf16.

    `workspace` (a uint8 device tensor, 256-byte aligned) is allocated here, on
    the call's stream, when the plan needs one and none is passed."""
    import torch
    lib = load_library()
    if out is None:
        out = _new(stream, lambda: torch.empty(q.shape, dtype=q.dtype, device=q.device))
    o = _opts(partition_tokens, variant, waves, prefetch, schedule, heads_per_tile, wave_partitions)
    dq, dk, dv, dt, dc, do = (desc(t) for t in (q, k_cache, v_cache, block_tables, context_lens, out))
    need = lib.pa_decode_workspace_size(_ref(dq), _ref(dk), _ref(dt), ctypes.byref(o))
    ws_ptr, ws_bytes = _workspace(need, workspace, q.device, stream)
    st = lib.pa_decode(_ref(dq), _ref(dk), _ref(dv), _ref(dt), _ref(dc), float(scale), _ref(do), float(k_scale),
                       float(v_scale), ws_ptr, ws_bytes, ctypes.byref(o), _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_decode")
    return out


def pa_decode_no_alloc(q, k_cache, v_cache, block_tables, context_lens, scale: float, out, *,
                       k_scale: float = 1.0, v_scale: float = 1.0, partition_tokens: int = 0, variant="auto",
                       waves: int = 0, prefetch: int = 0, schedule: int = 0, heads_per_tile: int = 0,
                       wave_partitions: int = 0, stream=None):
    """pa_decode with the library's static scratch as its workspace: no
    device allocation anywhere, here or in the library (so `out` must be
    given). Raises PAError (PA_ERR_SCRATCH) when the plan needs more than
    PA_NO_ALLOC_SCRATCH bytes. Calls that overlap on one device race on the
    scratch."""
    lib = load_library()
    o = _opts(partition_tokens, variant, waves, prefetch, schedule, heads_per_tile, wave_partitions)
    d = [desc(t) for t in (q, k_cache, v_cache, block_tables, context_lens, out)]
    st = lib.pa_decode_no_alloc(*map(_ref, d[:5]), float(scale), _ref(d[5]), float(k_scale), float(v_scale),
                                ctypes.byref(o), _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_decode_no_alloc")
    return out


def pa_decode_multi(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
                    max_query_len: int, out=None, *, k_scale: float = 1.0, v_scale: float = 1.0,
                    workspace=None, partition_tokens: int = 0, stream=None):
    """Multi-token paged attention: q [T_q, Hq, D] bf16, query_start [S + 1]
    int32; the last query_start[i+1] - query_start[i] of sequence i's
    context_lens[i] cached tokens attend causally. Returns out [T_q, Hq, D]."""
    import torch
    lib = load_library()
    if out is None:
        out = _new(stream, lambda: torch.empty(q.shape, dtype=q.dtype, device=q.device))
    dq, dk, dv, dt, dc, dqs, do = (desc(t) for t in (q, k_cache, v_cache, block_tables, context_lens, query_start,
                                                       out))
    need = lib.pa_decode_multi_workspace_size(_ref(dq), _ref(dk), _ref(dt), int(max_query_len),
                                              int(partition_tokens))
    ws_ptr, ws_bytes = _workspace(need, workspace, q.device, stream)
    st = lib.pa_decode_multi(_ref(dq), _ref(dk), _ref(dv), _ref(dt), _ref(dc), _ref(dqs), float(scale), _ref(do),
                             int(max_query_len), float(k_scale), float(v_scale), ws_ptr, ws_bytes,
                             int(partition_tokens), _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_decode_multi")
    return out


def pa_decode_multi_workspace_size(q, k_cache, block_tables, max_query_len: int, partition_tokens: int = 0) -> int:
    d = [desc(t) for t in (q, k_cache, block_tables)]
    return int(load_library().pa_decode_multi_workspace_size(*map(_ref, d), int(max_query_len),
                                                             int(partition_tokens)))


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
    if out is None:
        out = _new(stream, lambda: torch.empty(q.shape, dtype=q.dtype, device=q.device))
    o = _opts(partition_tokens, variant, waves, prefetch, 0, heads_per_tile)
    d = [desc(t) for t in (q, k_cache, v_cache, block_tables, context_lens, prefix_tables, prefix_lens,
                           group_start, out)]
    need = lib.pa_decode_cascade_workspace_size(_ref(d[0]), _ref(d[1]), _ref(d[3]), _ref(d[5]), int(max_group_size),
                                                ctypes.byref(o))
    ws_ptr, ws_bytes = _workspace(need, workspace, q.device, stream)
    st = lib.pa_decode_cascade(*map(_ref, d[:8]), float(scale), _ref(d[8]), int(max_group_size), float(k_scale),
                               float(v_scale), ws_ptr, ws_bytes, ctypes.byref(o), _stream_ptr(stream))
    if st != PA_OK:
        raise PAError(st, "pa_decode_cascade")
    return out


def pa_decode_cascade_workspace_size(q, k_cache, block_tables, prefix_tables, max_group_size: int, *,
                                     partition_tokens=0, variant="auto", waves=0, prefetch=0,
                                     heads_per_tile=0) -> int:
    o = _opts(partition_tokens, variant, waves, prefetch, 0, heads_per_tile)
    d = [desc(t) for t in (q, k_cache, block_tables, prefix_tables)]
    return int(load_library().pa_decode_cascade_workspace_size(*map(_ref, d), int(max_group_size), ctypes.byref(o)))


def _checked(st, what):
    if st not in (PA_OK, PA_ERR_PRECONDITION):
        raise PAError(st, what)
    return st


def pa_check_cache_write_inputs(slot_mapping, k_cache, stream=None) -> int:
    """Check pa_cache_write's device-side preconditions (slots distinct, each
    negative or inside the pool). Synchronises. Returns PA_OK or
    PA_ERR_PRECONDITION; raises on argument errors."""
    d = [desc(t) for t in (slot_mapping, k_cache)]
    return _checked(load_library().pa_check_cache_write_inputs(*map(_ref, d), _stream_ptr(stream)),
                    "pa_check_cache_write_inputs")


def pa_check_decode_inputs(block_tables, context_lens, k_cache, stream=None) -> int:
    """Check pa_decode's device-side preconditions (lengths within the table
    row, covering table entries inside the pool). Synchronises. Returns PA_OK
    or PA_ERR_PRECONDITION; raises on argument errors."""
    d = [desc(t) for t in (block_tables, context_lens, k_cache)]
    return _checked(load_library().pa_check_decode_inputs(*map(_ref, d), _stream_ptr(stream)),
                    "pa_check_decode_inputs")


def pa_check_multi_inputs(block_tables, context_lens, query_start, max_query_len: int, k_cache, stream=None) -> int:
    """Check pa_decode_multi's device-side preconditions (pa_check_decode_inputs',
    and every sequence's query count within max_query_len and its context)."""
    d = [desc(t) for t in (block_tables, context_lens, query_start)]
    return _checked(load_library().pa_check_multi_inputs(*map(_ref, d), int(max_query_len), _ref(desc(k_cache)),
                                                         _stream_ptr(stream)), "pa_check_multi_inputs")


def pa_check_cascade_inputs(prefix_tables, prefix_lens, group_start, max_group_size: int, num_seqs: int, k_cache,
                            stream=None) -> int:
    """Check pa_decode_cascade's group arrays (offsets rising within the batch,
    group sizes, whole-block prefix lengths within the table row, covering
    prefix table entries inside the pool). Synchronises. Returns PA_OK or
    PA_ERR_PRECONDITION; raises on argument errors."""
    d = [desc(t) for t in (prefix_tables, prefix_lens, group_start)]
    return _checked(load_library().pa_check_cascade_inputs(*map(_ref, d), int(max_group_size), int(num_seqs),
                                                           _ref(desc(k_cache)), _stream_ptr(stream)),
                    "pa_check_cascade_inputs")


def pa_probe_stream_read(buf, sink, nontemporal: bool = True, stream=None) -> None:
    """Read every byte of the device tensor `buf` once (a streaming-read
    reference kernel); `sink` is a device int32/uint32 tensor of >= 256 entries."""
    lib = load_library()
    for t in (buf, sink):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("buf and sink must be contiguous device tensors")
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
