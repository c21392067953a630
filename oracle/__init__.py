"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package. The product library (the HIP kernels behind the C ABI) never
imports, links or calls it, and the two share no code.

The arithmetic lives in `pa_oracle.c` (plain C, float64, OpenMP over
(sequence, KV head)); this module builds it with gcc and marshals numpy
arrays into it. Each C function states the passage of the pages it follows.
Every oracle function here is pinned by a CPU test against something other
than itself (a library routine, a closed form, an invariant or brute force);
none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

KV_BF16 = 1
KV_FP8_E4M3FN = 2


def build(force: bool = False) -> str:
    """Compile pa_oracle.c with gcc (no fast-math) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        # PA_ORACLE_LIB names another build of pa_oracle.c to load instead
        # (the sanitizer test's instrumented one)
        path = os.environ.get("PA_ORACLE_LIB")
        if not path:
            build()
            path = _LIB_PATH
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3fn_to_f64.restype = ctypes.c_double
        lib.oracle_f32_to_e4m3fn.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_e4m3fn.restype = ctypes.c_uint8
        lib.oracle_quantize_bf16.argtypes = [ctypes.c_uint16, ctypes.c_float]
        lib.oracle_quantize_bf16.restype = ctypes.c_uint8
        lib.oracle_cache_write.argtypes = [P, P, P, i64, i64, i64, i64, i64, ctypes.c_int,
                                           ctypes.c_float, ctypes.c_float, P, P]
        lib.oracle_cache_write.restype = i64
        lib.oracle_decode_units.argtypes = [P, P, P, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                            P, P, i64, i64, i64, i64, i64, i64, i64, ctypes.c_double,
                                            P, i64, P, ctypes.c_int]
        lib.oracle_decode_units.restype = ctypes.c_int
        lib.oracle_multi_units.argtypes = [P, P, P, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                           P, P, P, i64, i64, i64, i64, i64, i64, i64, ctypes.c_double,
                                           P, i64, P, ctypes.c_int]
        lib.oracle_multi_units.restype = ctypes.c_int
        lib.oracle_copy_blocks.argtypes = [P, P, P, i64, i64, i64, i64, i64, i64]
        lib.oracle_copy_blocks.restype = i64
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([lib.oracle_bf16_to_f64(int(b)) for b in flat], dtype=np.float64).reshape(np.shape(bits))


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.asarray(codes, dtype=np.uint8).reshape(-1)
    return np.array([lib.oracle_e4m3fn_to_f64(int(c)) for c in flat], dtype=np.float64).reshape(np.shape(codes))


def f32_to_e4m3fn(x: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.asarray(x, dtype=np.float32).reshape(-1)
    return np.array([lib.oracle_f32_to_e4m3fn(float(v)) for v in flat], dtype=np.uint8).reshape(np.shape(x))


def quantize_bf16(bits: np.ndarray, scale: float) -> np.ndarray:
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([lib.oracle_quantize_bf16(int(b), scale) for b in flat], dtype=np.uint8).reshape(np.shape(bits))


def cache_write(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                k_cache: np.ndarray, v_cache: np.ndarray, *, kv_dtype: int = KV_BF16,
                k_scale: float = 1.0, v_scale: float = 1.0) -> int:
    """In-place paged cache write. Caches: uint16 bf16 bits or uint8 e4m3fn codes, [N, bs, Hkv, D]."""
    lib = _load()
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    N, bs, Hkv, D = k_cache.shape
    T = int(slots.shape[0])
    assert k.shape == (T, Hkv, D) and v.shape == (T, Hkv, D)
    want = np.uint16 if kv_dtype == KV_BF16 else np.uint8
    assert k_cache.dtype == want and v_cache.dtype == want
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    n = lib.oracle_cache_write(_ptr(k), _ptr(v), _ptr(slots), T, Hkv, D, bs, N, kv_dtype,
                               k_scale, v_scale, _ptr(k_cache), _ptr(v_cache))
    if n < 0:
        raise ValueError("slot outside the pool")
    return int(n)


def decode_units(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                 units: Sequence[int], num_q_heads: int, *, kv_dtype: int = KV_BF16,
                 k_scale: float = 1.0, v_scale: float = 1.0, threads: int = 0) -> np.ndarray:
    """Decode for (seq * Hkv + kv_head) units -> float64 [n_units, g, D]."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    S, Hq, D = q.shape
    assert Hq == num_q_heads
    N, bs, Hkv, D2 = k_cache.shape
    assert D2 == D and Hq % Hkv == 0
    g = Hq // Hkv
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    MB = tables.shape[1]
    units = np.ascontiguousarray(np.asarray(units, dtype=np.int64))
    if len(units) and (units.min() < 0 or units.max() >= S * Hkv):
        raise ValueError("unit outside [0, num_seqs * num_kv_heads)")
    out = np.zeros((len(units), g, D), dtype=np.float64)
    kc = np.ascontiguousarray(k_cache)
    vc = np.ascontiguousarray(v_cache)
    rc = lib.oracle_decode_units(_ptr(q), _ptr(kc), _ptr(vc), kv_dtype, k_scale, v_scale,
                                 _ptr(tables), _ptr(ctx), S, Hq, Hkv, D, bs, N, MB, float(scale),
                                 _ptr(units), len(units), _ptr(out), int(threads))
    if rc != 0:
        raise ValueError("block id outside the pool or context longer than its table row")
    return out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, *, kv_dtype: int = KV_BF16,
           k_scale: float = 1.0, v_scale: float = 1.0, threads: int = 0) -> np.ndarray:
    """Full decode -> float64 [S, Hq, D]."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    out = decode_units(q, k_cache, v_cache, block_tables, context_lens, scale,
                       np.arange(S * Hkv), Hq, kv_dtype=kv_dtype, k_scale=k_scale,
                       v_scale=v_scale, threads=threads)
    return out.reshape(S, Hq, D)


def decode_workload(w, *, units: Optional[Sequence[int]] = None, kv_dtype: int = KV_BF16,
                    k_cache=None, v_cache=None, k_scale: float = 1.0, v_scale: float = 1.0,
                    threads: int = 0) -> np.ndarray:
    """Decode a generated workload (all units -> [S, Hq, D], else [n_units, g, D])."""
    kc = w.k_cache if k_cache is None else k_cache
    vc = w.v_cache if v_cache is None else v_cache
    if units is None:
        return decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, kv_dtype=kv_dtype,
                      k_scale=k_scale, v_scale=v_scale, threads=threads)
    return decode_units(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, units,
                        w.spec.num_q_heads, kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale,
                        threads=threads)


def multi_decode(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, *,
                 units: Optional[Sequence[int]] = None, kv_dtype: int = KV_BF16, k_scale: float = 1.0,
                 v_scale: float = 1.0, threads: int = 0) -> np.ndarray:
    """Multi-token paged attention -> float64 [T_q, Hq, D]: the last
    query_start[i+1] - query_start[i] of sequence i's context_lens[i] tokens
    attend causally. Rows of units not requested stay NaN."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    Tq, Hq, D = q.shape
    N, bs, Hkv, D2 = k_cache.shape
    assert D2 == D and Hq % Hkv == 0
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    S = ctx.shape[0]
    assert qs.shape == (S + 1,) and qs[0] == 0 and qs[-1] == Tq and np.all(np.diff(qs) >= 0)
    MB = tables.shape[1]
    if units is None:
        units = np.arange(S * Hkv)
    units = np.ascontiguousarray(np.asarray(units, dtype=np.int64))
    out = np.full((Tq, Hq, D), np.nan, dtype=np.float64)
    kc = np.ascontiguousarray(k_cache)
    vc = np.ascontiguousarray(v_cache)
    rc = lib.oracle_multi_units(_ptr(q), _ptr(kc), _ptr(vc), kv_dtype, k_scale, v_scale, _ptr(tables),
                                _ptr(ctx), _ptr(qs), S, Hq, Hkv, D, bs, N, MB, float(scale), _ptr(units),
                                len(units), _ptr(out), int(threads))
    if rc != 0:
        raise ValueError("block id outside the pool, context longer than its table row, "
                         "or more query tokens than context")
    return out


def cascade_tables(block_tables, context_lens, prefix_tables, prefix_lens, group_start, block_size: int,
                   max_group_size: Optional[int] = None) -> np.ndarray:
    """The block table a cascade decode reads through (Tutorial §4.3, prefix
    caching: a cached prefix is a list of physical blocks plus a length,
    reused by every request that starts with it). Group k is the run of
    sequences group_start[k] .. group_start[k+1] - 1 (its first
    max_group_size members, when given); member i holds shared_i =
    min(context_lens[i], prefix_lens[k]) prefix tokens, so its logical
    blocks b with b * block_size < shared_i are the prefix's blocks
    prefix_tables[k][b], and the rest come from its own row. Returns the
    composed int32 [S, MB] table (rows of sequences in no group unchanged).
    Prefix lengths must be whole blocks, so no block mixes the two sources."""
    tables = np.array(block_tables, dtype=np.int32, copy=True)
    ctx = np.asarray(context_lens, dtype=np.int64)
    pt = np.asarray(prefix_tables, dtype=np.int64)
    pl = np.asarray(prefix_lens, dtype=np.int64)
    gs = np.asarray(group_start, dtype=np.int64)
    S, MB = tables.shape
    G = pl.shape[0]
    assert gs.shape == (G + 1,) and pt.shape[0] == G
    assert np.all(np.diff(gs) >= 0) and (G == 0 or (gs[0] >= 0 and gs[-1] <= S))
    assert np.all(pl % block_size == 0) and np.all(pl >= 0) and np.all(pl <= pt.shape[1] * block_size)
    for k in range(G):
        last = gs[k + 1] if max_group_size is None else min(gs[k + 1], gs[k] + max_group_size)
        for i in range(int(gs[k]), int(last)):
            shared = min(int(ctx[i]), int(pl[k]))
            nb = (shared + block_size - 1) // block_size
            tables[i, :nb] = pt[k, :nb]
    return tables


def cascade_decode(q, k_cache, v_cache, block_tables, context_lens, prefix_tables, prefix_lens, group_start,
                   scale, *, max_group_size: Optional[int] = None, units: Optional[Sequence[int]] = None,
                   kv_dtype: int = KV_BF16, k_scale: float = 1.0, v_scale: float = 1.0,
                   threads: int = 0) -> np.ndarray:
    """Decode of a cascade call -> float64 [S, Hq, D] (or [n_units, g, D] for
    `units`): the plain decode definition over each sequence's context,
    gathered through the table cascade_tables() composes."""
    bs = k_cache.shape[1]
    tables = cascade_tables(block_tables, context_lens, prefix_tables, prefix_lens, group_start, bs,
                            max_group_size)
    if units is None:
        return decode(q, k_cache, v_cache, tables, context_lens, scale, kv_dtype=kv_dtype, k_scale=k_scale,
                      v_scale=v_scale, threads=threads)
    return decode_units(q, k_cache, v_cache, tables, context_lens, scale, units, q.shape[1], kv_dtype=kv_dtype,
                        k_scale=k_scale, v_scale=v_scale, threads=threads)


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs) -> int:
    """In-place block copy of both caches ([N, bs, Hkv, D], uint16 bf16 bits or
    uint8 fp8 codes) for (src, dst) pairs; negative ids are skipped."""
    lib = _load()
    pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
    assert k_cache.shape == v_cache.shape and k_cache.dtype == v_cache.dtype
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    N, bs, Hkv, D = k_cache.shape
    n = lib.oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pr), pr.shape[0], N, bs, Hkv, D,
                               k_cache.dtype.itemsize)
    if n < 0:
        raise ValueError("block id outside the pool or a repeated destination")
    return int(n)


def quantize_pool(bits: np.ndarray, scale: float) -> np.ndarray:
    """fp8 codes of a whole bf16 pool, through the oracle's cache write (every row written)."""
    N, bs, Hkv, D = bits.shape
    rows = np.ascontiguousarray(bits.reshape(N * bs, Hkv, D))
    out_k = np.zeros((N, bs, Hkv, D), dtype=np.uint8)
    out_v = np.zeros((N, bs, Hkv, D), dtype=np.uint8)
    cache_write(rows, rows, np.arange(N * bs, dtype=np.int64), out_k, out_v,
                kv_dtype=KV_FP8_E4M3FN, k_scale=scale, v_scale=scale)
    return out_k
