"""fp64 CPU oracle for paged decode attention, attention for several new tokens per
sequence, and the KV-cache write.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never imports, links or calls it, and it shares no code with the GPU library.

The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only compiles it
with gcc and marshals numpy arrays into it.  Element arrays are passed as raw
storage: ``float32`` for fp32, ``float16`` for fp16 and ``uint16`` bit patterns for
bf16 (numpy has no bfloat16), with the dtype named explicitly.

Pages cited (title, site): [AB] "什么是分页注意力（PagedAttention）？" aiboss88.com;
[CY] "深入解析 PagedAttention：vLLM 显存优化的核心魔法" cygnushan.xyz;
[ASP] "PagedAttention" awesome-system-papers; [RK] "什么是 LLM 中的分页注意力
(Paged Attention)?它是如何工作的?" news.rkmt.cn.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

OK, BAD_ARG, BAD_LEN, BAD_BLOCK, BAD_SLOT, DUP_SLOT, NOMEM = range(7)
_NAMES = ["OK", "BAD_ARG", "BAD_LEN", "BAD_BLOCK", "BAD_SLOT", "DUP_SLOT", "NOMEM"]


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what}: {_NAMES[code] if 0 <= code < len(_NAMES) else code}")
        self.code = code


def build() -> str:
    """Compile liboracle.so with gcc (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
         _SRC, "-o", tmp, "-lm"],
        check=True,
    )
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        p, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_decode.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64, i32,
                                      dbl, p]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_multi_token.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                                           i64, i32, dbl, p]
        lib.oracle_multi_token.restype = ctypes.c_int
        lib.oracle_cache_write.argtypes = [p, p, p, i32, i32, i32, i32, i64, i32, p, p]
        lib.oracle_cache_write.restype = ctypes.c_int
        lib.oracle_decode_elements.argtypes = [p, i64, i32, p]
        lib.oracle_decode_elements.restype = None
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _storage(a: np.ndarray, dtype: str) -> np.ndarray:
    want = _STORAGE[dtype]
    if a.dtype != want:
        raise TypeError(f"{dtype} data must be stored as {np.dtype(want).name}, got {a.dtype}")
    return np.ascontiguousarray(a)


def set_threads(n: int) -> int:
    """Set the OpenMP thread count (n <= 0 keeps it); returns the count in force."""
    return _load().oracle_set_threads(int(n))


def decode_elements(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Widen raw fp32/fp16/bf16 storage to float64 exactly (exposed for pinning)."""
    raw = _storage(raw, dtype)
    out = np.empty(raw.shape, dtype=np.float64)
    _load().oracle_decode_elements(_ptr(raw), raw.size, DTYPES[dtype], _ptr(out))
    return out


def decode(q, k_cache, v_cache, block_tables, seq_lens, block_size: int, num_kv_heads: int,
           scale: float, dtype: str) -> np.ndarray:
    """Reference decode attention; returns float64 [S, Hq, D].

    q [S, Hq, D]; k_cache [N, Hkv, bs, D]; v_cache [N, Hkv, D, bs];
    block_tables int32 [S, max_blocks]; seq_lens int32 [S].  ``scale`` is used as
    given (pass the fp32 value the GPU receives).
    """
    q = _storage(q, dtype)
    k_cache = _storage(k_cache, dtype)
    v_cache = _storage(v_cache, dtype)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    S, Hq, D = q.shape
    N = k_cache.shape[0]
    if k_cache.shape != (N, num_kv_heads, block_size, D):
        raise ValueError(f"k_cache shape {k_cache.shape}")
    if v_cache.shape != (N, num_kv_heads, D, block_size):
        raise ValueError(f"v_cache shape {v_cache.shape}")
    if bt.ndim != 2 or bt.shape[0] != S or sl.shape != (S,):
        raise ValueError("block_tables / seq_lens shape")
    out = np.zeros((S, Hq, D), dtype=np.float64)
    rc = _load().oracle_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(sl), S, Hq,
                               num_kv_heads, D, block_size, bt.shape[1], N, DTYPES[dtype],
                               float(scale), _ptr(out))
    if rc != OK:
        raise OracleError(rc, "decode")
    return out


def multi_token(q, k_cache, v_cache, block_tables, seq_lens, query_start, block_size: int,
                num_kv_heads: int, scale: float, dtype: str) -> np.ndarray:
    """Reference attention for several new tokens per sequence; returns float64
    [T, Hq, D].  q [T, Hq, D] holds sequence s's new tokens in rows
    query_start[s] .. query_start[s+1]-1 (int32 [S+1], query_start[0] = 0); they are
    the last n_s of its seq_lens[s] cached tokens, and token j sees positions
    0 .. seq_lens[s] - n_s + j."""
    q = _storage(q, dtype)
    k_cache = _storage(k_cache, dtype)
    v_cache = _storage(v_cache, dtype)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    T, Hq, D = q.shape
    S = sl.shape[0]
    N = k_cache.shape[0]
    if k_cache.shape != (N, num_kv_heads, block_size, D):
        raise ValueError(f"k_cache shape {k_cache.shape}")
    if v_cache.shape != (N, num_kv_heads, D, block_size):
        raise ValueError(f"v_cache shape {v_cache.shape}")
    if bt.ndim != 2 or bt.shape[0] != S or qs.shape != (S + 1,):
        raise ValueError("block_tables / query_start shape")
    out = np.zeros((T, Hq, D), dtype=np.float64)
    rc = _load().oracle_multi_token(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(sl),
                                    _ptr(qs), S, T, Hq, num_kv_heads, D, block_size, bt.shape[1],
                                    N, DTYPES[dtype], float(scale), _ptr(out))
    if rc != OK:
        raise OracleError(rc, "multi_token")
    return out


def cache_write(k, v, slot_mapping, k_cache: np.ndarray, v_cache: np.ndarray, block_size: int,
                dtype: str) -> None:
    """Reference cache write, in place on host arrays (k, v: [T, Hkv, D])."""
    k = _storage(k, dtype)
    v = _storage(v, dtype)
    for c in (k_cache, v_cache):
        if c.dtype != _STORAGE[dtype] or not c.flags.c_contiguous:
            raise TypeError("cache arrays must be contiguous storage of the given dtype")
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T, Hkv, D = k.shape
    N = k_cache.shape[0]
    if k_cache.shape != (N, Hkv, block_size, D) or v_cache.shape != (N, Hkv, D, block_size):
        raise ValueError("cache shapes")
    if sm.shape != (T,) or v.shape != k.shape:
        raise ValueError("k / v / slot_mapping shapes")
    rc = _load().oracle_cache_write(_ptr(k), _ptr(v), _ptr(sm), T, Hkv, D, block_size, N,
                                    ELEM_BYTES[dtype], _ptr(k_cache), _ptr(v_cache))
    if rc != OK:
        raise OracleError(rc, "cache_write")
