"""CPU oracle for paged decode attention: ctypes wrapper over pkv_oracle.c.

TEST INFRASTRUCTURE ONLY.  The tests, the package smoke check and the CPU
baseline of the benchmark may import this module; the product package must
not, and nothing here imports the product package.  See pkv_oracle.c for
what is computed and the passages of the pages it follows:

  "vLLM 推理引擎源码级拆解" (chenxutan.com/d/5333) §2.1-2.3 - block pool,
  block table, address translation and single-query attention with
  softmax; §2.2 - the append rule the cache writer implements.

Arrays are numpy.  Storage conventions: 'f32' float32, 'f16' float16,
'bf16' uint16 bit patterns, 'fp8' uint8 OCP E4M3 codes.  Outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_DT = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}
_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    P, I, D, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_float
    SZ = ctypes.c_size_t
    lib.orc_e4m3_encode.argtypes = [F]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = D
    lib.orc_e4m3_encode_array.argtypes = [P, P, SZ]
    lib.orc_e4m3_decode_array.argtypes = [P, P, SZ]
    lib.orc_widen_array.argtypes = [P, I, P, SZ]
    lib.orc_reshape_and_cache.argtypes = [P, P, I, P, P, I, P, I, I, I, I, I, F, F]
    lib.orc_reshape_and_cache.restype = I
    lib.orc_paged_decode.argtypes = [P, P, I, P, P, I, P, I, P, I, I, I, I, I, I,
                                     D, D, D, P, I, I]
    lib.orc_paged_decode.restype = I
    lib.orc_paged_decode_mixed.argtypes = [P, P, I, P, P, I, P, I, P, P, I, I, I, I, I, I,
                                           D, D, D, P, I, I]
    lib.orc_paged_decode_mixed.restype = I
    lib.orc_paged_multi.argtypes = [P, P, I, P, P, I, P, I, P, P, I, I, I, I, I, I,
                                    D, D, D, P, I, I]
    lib.orc_paged_multi.restype = I
    lib.orc_paged_partials.argtypes = [P, P, P, P, I, P, P, I, P, I, P, I, I, I, I,
                                       I, I, D, D, D, I, I, I]
    lib.orc_paged_partials.restype = I
    lib.orc_partition_reduce.argtypes = [P, P, P, P, P, I, I, I, I, I]
    lib.orc_partition_reduce.restype = I
    lib.orc_gather_sequence.argtypes = [P, P, P, P, I, P, I, P, I, I, I, I, I, D, D, I, I]
    lib.orc_gather_sequence.restype = I
    lib.orc_openmp_max_threads.restype = I
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def max_threads() -> int:
    return int(_load().orc_openmp_max_threads())


# --- scalar formats ------------------------------------------------------

def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E4M3 codes: round to nearest even, saturate to +-448."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_encode_array(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e4m3_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact value of stored elements as float64 (fp8: the code's value)."""
    x = _c(x, _NP[dtype])
    out = np.empty(x.shape, np.float64)
    _load().orc_widen_array(_ptr(x), _DT[dtype], _ptr(out), x.size)
    return out


# --- the three operations ------------------------------------------------

def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, *,
                      src_dtype: str, cache_dtype: str,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Writes key/value [T, Hkv, D] into the caches [NB, bs, Hkv, D] in place."""
    key = _c(key, _NP[src_dtype])
    value = _c(value, _NP[src_dtype])
    slot_mapping = _c(slot_mapping, np.int64)
    for c in (k_cache, v_cache):
        if not c.flags.c_contiguous or c.dtype != np.dtype(_NP[cache_dtype]):
            raise TypeError("cache must be a C-contiguous %s array" % cache_dtype)
    T, Hkv, D = key.shape
    NB, bs = k_cache.shape[0], k_cache.shape[1]
    rc = _load().orc_reshape_and_cache(
        _ptr(key), _ptr(value), _DT[src_dtype], _ptr(k_cache), _ptr(v_cache),
        _DT[cache_dtype], _ptr(slot_mapping), T, Hkv, D, bs, NB,
        float(k_scale), float(v_scale))
    _check(rc, "reshape_and_cache")


def paged_decode(query, k_cache, v_cache, block_tables, seq_lens, *,
                 q_dtype: str, cache_dtype: str, scale: float,
                 k_scale: float = 1.0, v_scale: float = 1.0,
                 rows: Optional[Sequence[int]] = None,
                 threads: int = 0) -> np.ndarray:
    """Single-query attention per sequence over the paged caches.

    Returns float64 [S, Hq, D].  ``rows`` (flat s*Hq + hq) restricts the work
    to those output rows; the others are NaN."""
    query = _c(query, _NP[q_dtype])
    k_cache = _c(k_cache, _NP[cache_dtype])
    v_cache = _c(v_cache, _NP[cache_dtype])
    block_tables = _c(block_tables, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    S, Hq, D = query.shape
    NB, bs, Hkv, D2 = k_cache.shape
    assert D2 == D and block_tables.shape[0] == S and seq_lens.shape == (S,)
    out = np.full((S, Hq, D), np.nan, np.float64)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    rc = _load().orc_paged_decode(
        _ptr(out), _ptr(query), _DT[q_dtype], _ptr(k_cache), _ptr(v_cache),
        _DT[cache_dtype], _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), S, Hq, Hkv, D, bs, NB, float(scale), float(k_scale),
        float(v_scale), _ptr(r), 0 if r is None else r.size, int(threads))
    _check(rc, "paged_decode")
    return out


def paged_decode_mixed(query, k_cache, v_cache, block_tables, seq_lens, seq_block_sizes, *,
                       q_dtype: str, cache_dtype: str, scale: float,
                       k_scale: float = 1.0, v_scale: float = 1.0,
                       rows: Optional[Sequence[int]] = None,
                       threads: int = 0) -> np.ndarray:
    """paged_decode over a pool of pages (k_cache [num_pages, page, Hkv, D])
    whose sequences have blocks of seq_block_sizes[s] tokens, each that many
    / page consecutive pages from the page the table names ("vLLM 0.5 深度拆解"
    §1.3 block sizes per request; the page layout is this library's reading)."""
    query = _c(query, _NP[q_dtype])
    k_cache = _c(k_cache, _NP[cache_dtype])
    v_cache = _c(v_cache, _NP[cache_dtype])
    block_tables = _c(block_tables, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    seq_bs = _c(seq_block_sizes, np.int32)
    S, Hq, D = query.shape
    NP, page, Hkv, D2 = k_cache.shape
    assert D2 == D and block_tables.shape[0] == S and seq_lens.shape == (S,)
    assert seq_bs.shape == (S,)
    out = np.full((S, Hq, D), np.nan, np.float64)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    rc = _load().orc_paged_decode_mixed(
        _ptr(out), _ptr(query), _DT[q_dtype], _ptr(k_cache), _ptr(v_cache),
        _DT[cache_dtype], _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), _ptr(seq_bs), S, Hq, Hkv, D, page, NP, float(scale),
        float(k_scale), float(v_scale), _ptr(r), 0 if r is None else r.size, int(threads))
    _check(rc, "paged_decode_mixed")
    return out


def paged_multi(query, k_cache, v_cache, block_tables, seq_lens, query_start, *,
                q_dtype: str, cache_dtype: str, scale: float,
                k_scale: float = 1.0, v_scale: float = 1.0,
                rows: Optional[Sequence[int]] = None,
                threads: int = 0) -> np.ndarray:
    """Several new query tokens per sequence (chunked prefill, speculative
    verification).  query [total_q, Hq, D]; query_start [S + 1] (exclusive
    prefix of the per-sequence query counts Qn).  Query token i of sequence
    s sits at position seq_lens[s] - Qn + i and sees tokens up to it.
    Returns float64 [total_q, Hq, D]; ``rows`` (flat qtok*Hq + hq) restricts
    the work, the others are NaN."""
    query = _c(query, _NP[q_dtype])
    k_cache = _c(k_cache, _NP[cache_dtype])
    v_cache = _c(v_cache, _NP[cache_dtype])
    block_tables = _c(block_tables, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    query_start = _c(query_start, np.int32)
    TQ, Hq, D = query.shape
    NB, bs, Hkv, D2 = k_cache.shape
    S = seq_lens.shape[0]
    assert D2 == D and block_tables.shape[0] == S and query_start.shape == (S + 1,)
    assert int(query_start[-1]) == TQ
    out = np.full((TQ, Hq, D), np.nan, np.float64)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    rc = _load().orc_paged_multi(
        _ptr(out), _ptr(query), _DT[q_dtype], _ptr(k_cache), _ptr(v_cache),
        _DT[cache_dtype], _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), _ptr(query_start), S, Hq, Hkv, D, bs, NB, float(scale),
        float(k_scale), float(v_scale), _ptr(r), 0 if r is None else r.size,
        int(threads))
    _check(rc, "paged_multi")
    return out


def paged_partials(query, k_cache, v_cache, block_tables, seq_lens, *,
                   q_dtype: str, cache_dtype: str, scale: float,
                   partition_size: int, P_max: int, k_scale: float = 1.0,
                   v_scale: float = 1.0, threads: int = 0):
    """Split-K partials (m, l, o) per (s, hq, partition), float64.

    m, l: [S, Hq, P_max]; o: [S, Hq, P_max, D].  Unused partitions are NaN."""
    query = _c(query, _NP[q_dtype])
    k_cache = _c(k_cache, _NP[cache_dtype])
    v_cache = _c(v_cache, _NP[cache_dtype])
    block_tables = _c(block_tables, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    S, Hq, D = query.shape
    NB, bs, Hkv, _ = k_cache.shape
    m = np.full((S, Hq, P_max), np.nan)
    l = np.full((S, Hq, P_max), np.nan)
    o = np.full((S, Hq, P_max, D), np.nan)
    rc = _load().orc_paged_partials(
        _ptr(m), _ptr(l), _ptr(o), _ptr(query), _DT[q_dtype], _ptr(k_cache),
        _ptr(v_cache), _DT[cache_dtype], _ptr(block_tables),
        block_tables.shape[1], _ptr(seq_lens), S, Hq, Hkv, D, bs, NB,
        float(scale), float(k_scale), float(v_scale), int(partition_size),
        int(P_max), int(threads))
    _check(rc, "paged_partials")
    return m, l, o


def partition_reduce(m, l, o, seq_lens, *, partition_size: int) -> np.ndarray:
    """Merges split-K partials into the float64 output [S, Hq, D]."""
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    o = _c(o, np.float64)
    seq_lens = _c(seq_lens, np.int32)
    S, Hq, P_max, D = o.shape
    out = np.full((S, Hq, D), np.nan)
    rc = _load().orc_partition_reduce(
        _ptr(out), _ptr(m), _ptr(l), _ptr(o), _ptr(seq_lens), S, Hq, D,
        int(partition_size), P_max)
    _check(rc, "partition_reduce")
    return out


def gather_sequence(k_cache, v_cache, block_tables, seq_lens, s: int, h: int, *,
                    cache_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0):
    """The gather step alone: logical K, V [L, D] of (sequence s, KV head h)."""
    k_cache = _c(k_cache, _NP[cache_dtype])
    v_cache = _c(v_cache, _NP[cache_dtype])
    block_tables = _c(block_tables, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    NB, bs, Hkv, D = k_cache.shape
    L = max(int(seq_lens[s]), 0)
    K = np.zeros((L, D))
    V = np.zeros((L, D))
    rc = _load().orc_gather_sequence(
        _ptr(K), _ptr(V), _ptr(k_cache), _ptr(v_cache), _DT[cache_dtype],
        _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
        seq_lens.size, Hkv, D, bs, NB, float(k_scale), float(v_scale), s, h)
    _check(rc, "gather_sequence")
    return K, V
