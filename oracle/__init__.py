"""CPU oracle for KV-cache attention -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never does, and this package imports nothing from it.

The arithmetic lives in ``kvc_oracle.c`` (plain C, double precision); this
module only builds it with gcc and marshals numpy arrays through ctypes.

Array conventions (numpy, C-contiguous):
  * fp32 tensors are ``np.float32``; bf16 tensors are their raw bits as
    ``np.uint16`` (the high half of an fp32).
  * caches are ``[L, B, Hkv, Tmax, D]``; new rows and queries are
    ``[n_layers, B, H, N, D]``; ``hist_len`` is ``int32[B]``.
  * paged caches are pools ``[L, num_blocks, Hkv, block_size, D]`` with an
    ``int32[B, max_blocks]`` block table.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
OK, E_ARG, E_CAPACITY = 0, -1, -4


class OracleError(RuntimeError):
    pass


def compile_library(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc.  No fast-math and no FMA contraction, so
    every double operation happens as written."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-o", out + ".tmp", src, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build() -> str:
    return compile_library()


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load liboracle.so, compiling it first if it has not been built."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            compile_library()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_cache_bytes.argtypes = [i64] * 6
    lib.oracle_cache_bytes.restype = ctypes.c_uint64
    lib.oracle_append.argtypes = [vp, vp] + [i32] * 8 + [vp, vp, i32, vp]
    lib.oracle_append.restype = i32
    lib.oracle_attention.argtypes = [vp, vp, vp] + [i32] * 10 + [vp, dbl, vp]
    lib.oracle_attention.restype = i32
    lib.oracle_prefill.argtypes = [vp, vp] + [i32] * 8 + [vp, vp, vp, i32, i32, dbl, vp]
    lib.oracle_prefill.restype = i32
    lib.oracle_prefill_varlen.argtypes = [vp, vp] + [i32] * 8 + [vp, vp, vp, i32, vp, vp, dbl, vp]
    lib.oracle_prefill_varlen.restype = i32
    lib.oracle_paged_append.argtypes = [vp, vp] + [i32] * 8 + [vp, vp, i32, i32, vp, vp, i32]
    lib.oracle_paged_append.restype = i32
    lib.oracle_paged_attention.argtypes = [vp, vp, vp] + [i32] * 11 + [vp, vp, i32, dbl, vp]
    lib.oracle_paged_attention.restype = i32
    lib.oracle_paged_prefill_varlen.argtypes = [vp, vp] + [i32] * 8 + [vp, vp, vp, i32, i32, vp,
                                                                       vp, vp, i32, dbl, vp]
    lib.oracle_paged_prefill_varlen.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_set_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a: np.ndarray) -> int:
    if not a.flags.c_contiguous:
        raise ValueError("oracle arrays must be C-contiguous")
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise OracleError(f"{what} returned {rc}")


def cache_bytes(layers, batch, kv_heads, tokens, head_dim, elem_bytes, lib=None) -> int:
    lib = lib or load()
    return int(lib.oracle_cache_bytes(layers, batch, kv_heads, tokens, head_dim, elem_bytes))


def append(k_cache, v_cache, k_new, v_new, hist_len, layer0=0, lib=None) -> None:
    """In-place append of ``k_new``/``v_new`` ([n_layers,B,Hkv,N,D]) at
    positions ``hist_len[b] ..`` of layers ``layer0 ..``."""
    lib = lib or load()
    L, B, Hkv, Tmax, D = k_cache.shape
    n_layers, B2, H2, N, D2 = k_new.shape
    if (B2, H2, D2) != (B, Hkv, D) or v_new.shape != k_new.shape or v_cache.shape != k_cache.shape:
        raise ValueError("append: shape mismatch")
    dt = _dtype_code(k_cache)
    if _dtype_code(k_new) != dt or _dtype_code(v_new) != dt or _dtype_code(v_cache) != dt:
        raise TypeError("append: dtype mismatch")
    hist = np.ascontiguousarray(hist_len, dtype=np.int32)
    rc = lib.oracle_append(_ptr(k_cache), _ptr(v_cache), L, B, Hkv, Tmax, D, dt,
                           layer0, n_layers, _ptr(k_new), _ptr(v_new), N, _ptr(hist))
    _check(rc, "oracle_append")


def attention(q, k_cache, v_cache, hist_len, scale, layer0=0, lib=None) -> np.ndarray:
    """Attention of q ([n_layers,B,Hq,N,D]) against the cache, new row i of
    batch b seeing keys 0..hist_len[b]+i.  Returns float64, q's shape."""
    lib = lib or load()
    L, B, Hkv, Tmax, D = k_cache.shape
    n_layers, B2, Hq, N, D2 = q.shape
    if (B2, D2) != (B, D) or v_cache.shape != k_cache.shape:
        raise ValueError("attention: shape mismatch")
    dt = _dtype_code(k_cache)
    if _dtype_code(q) != dt or _dtype_code(v_cache) != dt:
        raise TypeError("attention: dtype mismatch")
    hist = np.ascontiguousarray(hist_len, dtype=np.int32)
    out = np.zeros(q.shape, dtype=np.float64)
    rc = lib.oracle_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), L, B, Hkv, Tmax, D, dt,
                              layer0, n_layers, Hq, N, _ptr(hist), float(scale), _ptr(out))
    _check(rc, "oracle_attention")
    return out


def prefill(k_cache, v_cache, q, k, v, scale, layer0=0, lib=None) -> np.ndarray:
    """Causal prefill of an S-token prompt into an empty cache (positions
    [0,S)); q is [n_layers,B,Hq,S,D], k/v are [n_layers,B,Hkv,S,D]."""
    lib = lib or load()
    L, B, Hkv, Tmax, D = k_cache.shape
    n_layers, B2, Hq, S, D2 = q.shape
    if (B2, D2) != (B, D) or k.shape != (n_layers, B, Hkv, S, D) or v.shape != k.shape:
        raise ValueError("prefill: shape mismatch")
    dt = _dtype_code(k_cache)
    for a in (v_cache, q, k, v):
        if _dtype_code(a) != dt:
            raise TypeError("prefill: dtype mismatch")
    out = np.zeros(q.shape, dtype=np.float64)
    rc = lib.oracle_prefill(_ptr(k_cache), _ptr(v_cache), L, B, Hkv, Tmax, D, dt, layer0,
                            n_layers, _ptr(q), _ptr(k), _ptr(v), Hq, S, float(scale), _ptr(out))
    _check(rc, "oracle_prefill")
    return out


def prefill_varlen(k_cache, v_cache, q, k, v, cu_seqlens, hist_len, scale, layer0=0,
                   lib=None) -> np.ndarray:
    """Packed variable-length prefill with history: q [n_layers, T, Hq, D],
    k/v [n_layers, T, Hkv, D] token-major, sequence b's new tokens at
    cu_seqlens[b] .. cu_seqlens[b+1]-1 going to cache positions hist_len[b]
    ..  Returns float64 [n_layers, T, Hq, D]."""
    lib = lib or load()
    L, B, Hkv, Tmax, D = k_cache.shape
    n_layers, T, Hq, D2 = q.shape
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    if D2 != D or k.shape != (n_layers, T, Hkv, D) or v.shape != k.shape or cu.shape != (B + 1,):
        raise ValueError("prefill_varlen: shape mismatch")
    if int(cu[-1]) != T:
        raise ValueError("prefill_varlen: cu_seqlens[B] must equal the packed token count")
    dt = _dtype_code(k_cache)
    for a in (v_cache, q, k, v):
        if _dtype_code(a) != dt:
            raise TypeError("prefill_varlen: dtype mismatch")
    hist = np.ascontiguousarray(hist_len, dtype=np.int32)
    out = np.zeros(q.shape, dtype=np.float64)
    rc = lib.oracle_prefill_varlen(_ptr(k_cache), _ptr(v_cache), L, B, Hkv, Tmax, D, dt, layer0,
                                   n_layers, _ptr(q), _ptr(k), _ptr(v), Hq, _ptr(cu), _ptr(hist),
                                   float(scale), _ptr(out))
    _check(rc, "oracle_prefill_varlen")
    return out


def _paged_shapes(k_pool, v_pool, block_table, what):
    L, num_blocks, Hkv, bs, D = k_pool.shape
    if v_pool.shape != k_pool.shape:
        raise ValueError(f"{what}: shape mismatch")
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    if bt.ndim != 2:
        raise ValueError(f"{what}: block_table must be [B, max_blocks]")
    return L, num_blocks, Hkv, bs, D, bt


def paged_append(k_pool, v_pool, k_new, v_new, hist_len, block_table, layer0=0, lib=None) -> None:
    """In-place append into a paged cache: pools [L, num_blocks, Hkv,
    block_size, D], new rows [n_layers, B, Hkv, N, D], block_table int32
    [B, max_blocks]."""
    lib = lib or load()
    L, nblk, Hkv, bs, D, bt = _paged_shapes(k_pool, v_pool, block_table, "paged_append")
    n_layers, B, H2, N, D2 = k_new.shape
    if (H2, D2) != (Hkv, D) or v_new.shape != k_new.shape or bt.shape[0] != B:
        raise ValueError("paged_append: shape mismatch")
    dt = _dtype_code(k_pool)
    for a in (v_pool, k_new, v_new):
        if _dtype_code(a) != dt:
            raise TypeError("paged_append: dtype mismatch")
    hist = np.ascontiguousarray(hist_len, dtype=np.int32)
    rc = lib.oracle_paged_append(_ptr(k_pool), _ptr(v_pool), L, nblk, Hkv, bs, D, dt, layer0,
                                 n_layers, _ptr(k_new), _ptr(v_new), B, N, _ptr(hist), _ptr(bt),
                                 bt.shape[1])
    _check(rc, "oracle_paged_append")


def paged_attention(q, k_pool, v_pool, hist_len, block_table, scale, layer0=0, lib=None) -> np.ndarray:
    """Attention of q ([n_layers,B,Hq,N,D]) against a paged cache, new row i
    of sequence b seeing positions 0..hist_len[b]+i.  Returns float64."""
    lib = lib or load()
    L, nblk, Hkv, bs, D, bt = _paged_shapes(k_pool, v_pool, block_table, "paged_attention")
    n_layers, B, Hq, N, D2 = q.shape
    if D2 != D or bt.shape[0] != B:
        raise ValueError("paged_attention: shape mismatch")
    dt = _dtype_code(k_pool)
    if _dtype_code(q) != dt or _dtype_code(v_pool) != dt:
        raise TypeError("paged_attention: dtype mismatch")
    hist = np.ascontiguousarray(hist_len, dtype=np.int32)
    out = np.zeros(q.shape, dtype=np.float64)
    rc = lib.oracle_paged_attention(_ptr(q), _ptr(k_pool), _ptr(v_pool), L, nblk, Hkv, bs, D, dt,
                                    layer0, n_layers, Hq, B, N, _ptr(hist), _ptr(bt), bt.shape[1],
                                    float(scale), _ptr(out))
    _check(rc, "oracle_paged_attention")
    return out


def paged_prefill_varlen(k_pool, v_pool, q, k, v, cu_seqlens, hist_len, block_table, scale,
                         layer0=0, lib=None) -> np.ndarray:
    """prefill_varlen into a paged cache (pools [L, num_blocks, Hkv,
    block_size, D], block_table int32 [B, max_blocks])."""
    lib = lib or load()
    L, nblk, Hkv, bs, D, bt = _paged_shapes(k_pool, v_pool, block_table, "paged_prefill_varlen")
    n_layers, T, Hq, D2 = q.shape
    B = bt.shape[0]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    if D2 != D or k.shape != (n_layers, T, Hkv, D) or v.shape != k.shape or cu.shape != (B + 1,):
        raise ValueError("paged_prefill_varlen: shape mismatch")
    if int(cu[-1]) != T:
        raise ValueError("paged_prefill_varlen: cu_seqlens[B] must equal the packed token count")
    dt = _dtype_code(k_pool)
    for a in (v_pool, q, k, v):
        if _dtype_code(a) != dt:
            raise TypeError("paged_prefill_varlen: dtype mismatch")
    hist = np.ascontiguousarray(hist_len, dtype=np.int32)
    out = np.zeros(q.shape, dtype=np.float64)
    rc = lib.oracle_paged_prefill_varlen(_ptr(k_pool), _ptr(v_pool), L, nblk, Hkv, bs, D, dt,
                                         layer0, n_layers, _ptr(q), _ptr(k), _ptr(v), Hq, B,
                                         _ptr(cu), _ptr(hist), _ptr(bt), bt.shape[1], float(scale),
                                         _ptr(out))
    _check(rc, "oracle_paged_prefill_varlen")
    return out


def set_threads(n: int, lib=None) -> None:
    (lib or load()).oracle_set_threads(int(n))


def max_threads(lib=None) -> int:
    return int((lib or load()).oracle_max_threads())
