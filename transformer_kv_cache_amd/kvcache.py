"""Thin Python binding of libkvcache.so (C ABI in include/kvcache.h).

Argument marshalling only: torch tensors are checked for device, dtype, shape
and contiguity, and their device pointers, sizes and the current HIP stream
are handed to the library.  Every step of the computation runs in the HIP
kernels; there is no fallback.  If the library has not been built the first
call raises ``KVCacheLibraryMissing``.

Layouts (row-major, contiguous):
  cache K, V        [L, B, Hkv, Tmax, D]
  q, o              [n_layers, B, Hq, N, D]
  k_new, v_new      [n_layers, B, Hkv, N, D]
  hist_len          host int32[B] (list, numpy array or CPU tensor)
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvcache.so")

KVC_F32, KVC_BF16 = 0, 1
ABI_VERSION = 13  # KVC_ABI_VERSION of the header these signatures follow
MAX_LINEAR_ROWS = 8  # rows kvc_linear_f32 takes (kMaxLinearRows)
_DTYPE_CODE = {torch.float32: KVC_F32, torch.bfloat16: KVC_BF16}
_STATUS = {0: "OK", -1: "E_NULL", -2: "E_SHAPE", -3: "E_DTYPE", -4: "E_CAPACITY",
           -5: "E_WORKSPACE", -6: "E_UNSUPPORTED", -7: "E_HIP"}


class KVCacheLibraryMissing(ImportError):
    pass


class KVCacheError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class CacheDesc(ctypes.Structure):
    """Mirror of ``kvc_cache``."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("L", ctypes.c_int32), ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("Tmax", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class PagedCacheDesc(ctypes.Structure):
    """Mirror of ``kvc_paged_cache``."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("L", ctypes.c_int32), ("num_blocks", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None
_lib_lock = threading.Lock()


def library(path: str | None = None) -> ctypes.CDLL:
    """Load libkvcache.so (once) and declare its signatures."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise KVCacheLibraryMissing(
            f"{p} is not built; run `python -m transformer_kv_cache_amd.build`")
    with _lib_lock:
        lib = ctypes.CDLL(p)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cp = ctypes.POINTER(CacheDesc)
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.kvc_abi_version.argtypes, lib.kvc_abi_version.restype = [], i32
        if lib.kvc_abi_version() != ABI_VERSION:
            raise KVCacheLibraryMissing(
                f"{p} has ABI version {lib.kvc_abi_version()}, this binding needs {ABI_VERSION}; "
                "rebuild with `python -m transformer_kv_cache_amd.build`")
        lib.kvc_last_error.argtypes, lib.kvc_last_error.restype = [], ctypes.c_char_p
        lib.kvc_cache_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
        lib.kvc_cache_bytes.restype = ctypes.c_uint64
        lib.kvc_append.argtypes = [cp, i32, i32, vp, vp, i32, ip, vp]
        lib.kvc_append.restype = i32
        lib.kvc_decode_workspace_bytes.argtypes = [cp, i32, i32, i32]
        lib.kvc_decode_workspace_bytes.restype = sz
        lib.kvc_attn_decode.argtypes = [cp, i32, i32, vp, i32, i32, ip, ctypes.c_float, vp, vp, sz, vp]
        lib.kvc_attn_decode.restype = i32
        lib.kvc_decode_step.argtypes = [cp, i32, i32, vp, vp, vp, i32, i32, ip, ctypes.c_float, vp,
                                        vp, sz, vp]
        lib.kvc_decode_step.restype = i32
        lib.kvc_decode_split.argtypes = [cp, i32, i32, vp, vp, vp, i32, i32, ip, ctypes.c_float, vp,
                                         vp, sz, vp]
        lib.kvc_decode_split.restype = i32
        lib.kvc_decode_combine.argtypes = [cp, i32, i32, vp, vp, vp, i32, i32, ip, ctypes.c_float, vp,
                                           vp, sz, vp]
        lib.kvc_decode_combine.restype = i32
        lib.kvc_attn_prefill.argtypes = [cp, i32, i32, vp, vp, vp, i32, i32, ctypes.c_float, vp, vp]
        lib.kvc_attn_prefill.restype = i32
        lib.kvc_attn_prefill_varlen.argtypes = [cp, i32, i32, vp, vp, vp, i32, ip, ip,
                                                ctypes.c_float, vp, vp]
        lib.kvc_attn_prefill_varlen.restype = i32
        pp = ctypes.POINTER(PagedCacheDesc)
        f32 = ctypes.c_float
        lib.kvc_paged_cache_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
        lib.kvc_paged_cache_bytes.restype = ctypes.c_uint64
        lib.kvc_paged_append.argtypes = [pp, i32, i32, vp, vp, i32, i32, ip, vp, i32, vp]
        lib.kvc_paged_append.restype = i32
        lib.kvc_paged_decode_workspace_bytes.argtypes = [pp, i32, i32, i32, i32, i32]
        lib.kvc_paged_decode_workspace_bytes.restype = sz
        lib.kvc_paged_attn_decode.argtypes = [pp, i32, i32, vp, i32, i32, i32, ip, vp, i32, f32, vp,
                                              vp, sz, vp]
        lib.kvc_paged_attn_decode.restype = i32
        lib.kvc_paged_decode_step.argtypes = [pp, i32, i32, vp, vp, vp, i32, i32, i32, ip, vp, i32,
                                              f32, vp, vp, sz, vp]
        lib.kvc_paged_decode_step.restype = i32
        lib.kvc_paged_attn_prefill_varlen.argtypes = [pp, i32, i32, vp, vp, vp, i32, i32, ip, ip,
                                                      vp, i32, f32, vp, vp]
        lib.kvc_paged_attn_prefill_varlen.restype = i32
        lib.kvc_decode_step_dl.argtypes = [cp, i32, i32, vp, vp, vp, i32, i32, vp, i32,
                                           ctypes.c_float, vp, vp, sz, vp]
        lib.kvc_decode_step_dl.restype = i32
        lib.kvc_decode_step_noalloc.argtypes = [cp, i32, i32, vp, vp, vp, i32, i32, ip,
                                                ctypes.c_float, vp, vp]
        lib.kvc_decode_step_noalloc.restype = i32
        lib.kvc_paged_decode_step_dl.argtypes = [pp, i32, i32, vp, vp, vp, i32, i32, i32, vp, i32,
                                                 vp, i32, f32, vp, vp, sz, vp]
        lib.kvc_paged_decode_step_dl.restype = i32
        lib.kvc_lengths_add.argtypes = [vp, i32, i32, vp]
        lib.kvc_lengths_add.restype = i32
        lib.kvc_linear_f32.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp, vp, f32, i32, vp, vp, i32, vp]
        lib.kvc_linear_f32.restype = i32
        lib.kvc_gemm_f32.argtypes = [vp, i32, i32, i32, vp, i32, vp, i32, vp, vp, i32, vp, ctypes.c_size_t, vp]
        lib.kvc_gemm_f32.restype = i32
        lib.kvc_gemm_workspace_bytes.argtypes = [i32, i32, i32]
        lib.kvc_gemm_workspace_bytes.restype = ctypes.c_size_t
        lib.kvc_layernorm_f32.argtypes = [vp, i32, i32, vp, vp, f32, vp, vp]
        lib.kvc_layernorm_f32.restype = i32
        lib.kvc_embed_f32.argtypes = [vp, i32, vp, i32, i32, vp, i32, i32, vp, vp, vp]
        lib.kvc_embed_f32.restype = i32
        lib.kvc_argmax_f32.argtypes = [vp, i64, vp, vp, vp, i64, vp]
        lib.kvc_argmax_f32.restype = i32
        if path is None:
            _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise KVCacheError(status, library().kvc_last_error().decode())


def cache_bytes(L, B, Hkv, Tmax, D, dtype=torch.float32) -> int:
    """2 x L x Hkv x D x Tmax x B x element size (the cache-size formula)."""
    return int(library().kvc_cache_bytes(L, B, Hkv, Tmax, D, _DTYPE_CODE[dtype]))


class KVCache:
    """A preallocated per-model cache: ``k`` and ``v`` are [L,B,Hkv,Tmax,D]
    torch tensors on one GPU.  Pass existing tensors or let it allocate."""

    def __init__(self, L, B, Hkv, Tmax, D, dtype=torch.float32, device="cuda", k=None, v=None):
        if dtype not in _DTYPE_CODE:
            raise TypeError(f"unsupported cache dtype {dtype}")
        shape = (L, B, Hkv, Tmax, D)
        self.k = k if k is not None else torch.empty(shape, dtype=dtype, device=device)
        self.v = v if v is not None else torch.empty(shape, dtype=dtype, device=device)
        for t in (self.k, self.v):
            if tuple(t.shape) != shape or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError("cache tensors must be contiguous CUDA tensors of shape "
                                 f"{shape} and dtype {dtype}")
        self.L, self.B, self.Hkv, self.Tmax, self.D, self.dtype = L, B, Hkv, Tmax, D, dtype

    @property
    def device(self):
        return self.k.device

    def desc(self) -> CacheDesc:
        return CacheDesc(self.k.data_ptr(), self.v.data_ptr(), self.L, self.B, self.Hkv,
                         self.Tmax, self.D, _DTYPE_CODE[self.dtype])

    @property
    def nbytes(self) -> int:
        return cache_bytes(self.L, self.B, self.Hkv, self.Tmax, self.D, self.dtype)

    def geometry(self) -> tuple:
        return (self.L, self.B, self.Hkv, self.Tmax, self.D, self.dtype)


def _hist(hist_len, B):
    h = np.ascontiguousarray(
        hist_len.cpu().numpy() if isinstance(hist_len, torch.Tensor) else hist_len, dtype=np.int32)
    if h.shape != (B,):
        raise ValueError(f"hist_len must have shape ({B},), got {h.shape}")
    return h, h.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensor(name, t, cache, shape):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != cache.device:
        raise ValueError(f"{name} must be a CUDA tensor on {cache.device}")
    if t.dtype != cache.dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, cache has {cache.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def append(cache: KVCache, k_new, v_new, hist_len, layer0: int = 0, stream=None) -> None:
    """Write k_new/v_new ([n_layers,B,Hkv,N,D]) into cache rows
    [hist_len[b], hist_len[b]+N) of layers layer0 .. layer0+n_layers-1."""
    n_layers, _, _, N, _ = k_new.shape
    shape = (n_layers, cache.B, cache.Hkv, N, cache.D)
    _check_tensor("k_new", k_new, cache, shape)
    _check_tensor("v_new", v_new, cache, shape)
    _, hp = _hist(hist_len, cache.B)
    d = cache.desc()
    _check(library().kvc_append(ctypes.byref(d), layer0, n_layers, k_new.data_ptr(),
                                v_new.data_ptr(), N, hp, _stream(cache.device, stream)))


def decode_workspace_bytes(cache: KVCache, n_layers: int, Hq: int, N: int) -> int:
    d = cache.desc()
    return int(library().kvc_decode_workspace_bytes(ctypes.byref(d), n_layers, Hq, N))


def new_decode_workspace(cache: KVCache, n_layers: int, Hq: int, N: int) -> torch.Tensor:
    """A 256-byte aligned workspace for kvc_attn_decode with this geometry,
    zero-filled: its arrival counters must start at zero, and every call
    leaves them at zero again."""
    return _aligned_workspace(decode_workspace_bytes(cache, n_layers, Hq, N), cache.device)


_ws_cache: dict = {}


def _aligned_workspace(nbytes, device):
    n = max(int(nbytes), 256)
    ws = torch.zeros(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def _default_workspace(cache, n_layers, Hq, N, stream, need=None, B=None):
    """One zero-filled workspace per (device, stream, call geometry): calls
    on one stream run one after another, so calls of one geometry share it
    (each leaves its arrival counters zero; another geometry could use those
    bytes as scratch, hence one per geometry).  It is allocated on that
    stream, and never during graph capture: a captured call must be given
    its own workspace."""
    if need is None:
        need = decode_workspace_bytes(cache, n_layers, Hq, N)
    s = stream if stream is not None else torch.cuda.current_stream(cache.device)
    key = (cache.device, int(s.cuda_stream), type(cache).__name__, cache.geometry(),
           n_layers, Hq, N, B, need)
    ws = _ws_cache.get(key)
    if ws is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("pass an explicit workspace to decode calls captured in a graph")
        with torch.cuda.stream(s):
            ws = _aligned_workspace(need, cache.device)
        _ws_cache[key] = ws
    return ws


def attn_decode(cache: KVCache, q, hist_len, scale: float | None = None, out=None,
                layer0: int = 0, workspace=None, stream=None):
    """Attention of q ([n_layers,B,Hq,N,D]) against the cache; new row i of
    sequence b sees keys 0 .. hist_len[b]+i.  The N new K/V rows must already
    be appended.  Returns ``out`` (allocated if None)."""
    n_layers, _, Hq, N, _ = q.shape
    shape = (n_layers, cache.B, Hq, N, cache.D)
    _check_tensor("q", q, cache, shape)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, cache, shape)
    if scale is None:
        scale = 1.0 / math.sqrt(cache.D)
    _, hp = _hist(hist_len, cache.B)
    if workspace is None:
        workspace = _default_workspace(cache, n_layers, Hq, N, stream)
    if workspace.device != cache.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the cache's device")
    d = cache.desc()
    _check(library().kvc_attn_decode(
        ctypes.byref(d), layer0, n_layers, q.data_ptr(), Hq, N, hp, float(scale), out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(cache.device, stream)))
    return out


def decode_step(cache: KVCache, q, k_new, v_new, hist_len, scale: float | None = None,
                out=None, layer0: int = 0, workspace=None, stream=None):
    """append + attn_decode in one launch: writes k_new/v_new into rows
    [hist_len[b], hist_len[b]+N) and returns the attention of q over keys
    0 .. hist_len[b]+i.  Same results as the two separate calls."""
    n_layers, _, Hq, N, _ = q.shape
    shape = (n_layers, cache.B, Hq, N, cache.D)
    _check_tensor("q", q, cache, shape)
    kshape = (n_layers, cache.B, cache.Hkv, N, cache.D)
    _check_tensor("k_new", k_new, cache, kshape)
    _check_tensor("v_new", v_new, cache, kshape)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, cache, shape)
    if scale is None:
        scale = 1.0 / math.sqrt(cache.D)
    _, hp = _hist(hist_len, cache.B)
    if workspace is None:
        workspace = _default_workspace(cache, n_layers, Hq, N, stream)
    if workspace.device != cache.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the cache's device")
    d = cache.desc()
    _check(library().kvc_decode_step(
        ctypes.byref(d), layer0, n_layers, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), Hq, N,
        hp, float(scale), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(cache.device, stream)))
    return out


def decode_step_noalloc(cache: KVCache, q, k_new, v_new, hist_len, out,
                        scale: float | None = None, layer0: int = 0, stream=None):
    """decode_step with no workspace: the library's per-GPU scratch holds
    the split states, so the call allocates nothing (``out`` must be given).
    Calls that may overlap on one GPU must not use it."""
    n_layers, _, Hq, N, _ = q.shape
    shape = (n_layers, cache.B, Hq, N, cache.D)
    _check_tensor("q", q, cache, shape)
    kshape = (n_layers, cache.B, cache.Hkv, N, cache.D)
    _check_tensor("k_new", k_new, cache, kshape)
    _check_tensor("v_new", v_new, cache, kshape)
    _check_tensor("out", out, cache, shape)
    if scale is None:
        scale = 1.0 / math.sqrt(cache.D)
    _, hp = _hist(hist_len, cache.B)
    d = cache.desc()
    _check(library().kvc_decode_step_noalloc(
        ctypes.byref(d), layer0, n_layers, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), Hq, N,
        hp, float(scale), out.data_ptr(), _stream(cache.device, stream)))
    return out


def decode_step_dl(cache: KVCache, q, k_new, v_new, hist_len_dev, hist_max: int,
                   scale: float | None = None, out=None, layer0: int = 0, workspace=None,
                   stream=None):
    """decode_step with the lengths in ``hist_len_dev`` (an int32 CUDA tensor
    [B], read on the device), so that a captured HIP graph of the step stays
    valid as the lengths grow.  ``hist_max`` bounds every length; the kernels
    clamp to it."""
    n_layers, _, Hq, N, _ = q.shape
    shape = (n_layers, cache.B, Hq, N, cache.D)
    _check_tensor("q", q, cache, shape)
    kshape = (n_layers, cache.B, cache.Hkv, N, cache.D)
    _check_tensor("k_new", k_new, cache, kshape)
    _check_tensor("v_new", v_new, cache, kshape)
    if (not isinstance(hist_len_dev, torch.Tensor) or hist_len_dev.dtype != torch.int32
            or not hist_len_dev.is_cuda or hist_len_dev.device != cache.device
            or not hist_len_dev.is_contiguous() or hist_len_dev.numel() != cache.B):
        raise ValueError(f"hist_len_dev must be a contiguous int32 CUDA tensor of {cache.B} "
                         "elements on the cache's device")
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, cache, shape)
    if scale is None:
        scale = 1.0 / math.sqrt(cache.D)
    if workspace is None:
        workspace = _default_workspace(cache, n_layers, Hq, N, stream)
    if workspace.device != cache.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the cache's device")
    d = cache.desc()
    _check(library().kvc_decode_step_dl(
        ctypes.byref(d), layer0, n_layers, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), Hq, N,
        hist_len_dev.data_ptr(), int(hist_max), float(scale), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(cache.device, stream)))
    return out


def lengths_add(hist_len_dev, n: int, stream=None) -> None:
    """hist_len_dev += n on the device (after a captured decode_step_dl)."""
    if (not isinstance(hist_len_dev, torch.Tensor) or hist_len_dev.dtype != torch.int32
            or not hist_len_dev.is_cuda or not hist_len_dev.is_contiguous()):
        raise ValueError("hist_len_dev must be a contiguous int32 CUDA tensor")
    _check(library().kvc_lengths_add(hist_len_dev.data_ptr(), hist_len_dev.numel(), int(n),
                                     _stream(hist_len_dev.device, stream)))


def _decode_phase(fn_name, cache, q, hist_len, k_new, v_new, scale, out, layer0, workspace,
                  stream):
    n_layers, _, Hq, N, _ = q.shape
    shape = (n_layers, cache.B, Hq, N, cache.D)
    _check_tensor("q", q, cache, shape)
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new or neither")
    if k_new is not None:
        kshape = (n_layers, cache.B, cache.Hkv, N, cache.D)
        _check_tensor("k_new", k_new, cache, kshape)
        _check_tensor("v_new", v_new, cache, kshape)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, cache, shape)
    if scale is None:
        scale = 1.0 / math.sqrt(cache.D)
    _, hp = _hist(hist_len, cache.B)
    if workspace is None:
        workspace = _default_workspace(cache, n_layers, Hq, N, stream)
    d = cache.desc()
    _check(getattr(library(), fn_name)(
        ctypes.byref(d), layer0, n_layers, q.data_ptr(),
        None if k_new is None else k_new.data_ptr(), None if v_new is None else v_new.data_ptr(),
        Hq, N, hp, float(scale), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(cache.device, stream)))
    return out


def decode_split(cache: KVCache, q, hist_len, k_new=None, v_new=None, scale: float | None = None,
                 out=None, layer0: int = 0, workspace=None, stream=None):
    """First phase of attn_decode (k_new/v_new None) or decode_step (both
    given): per-split softmax states, or outputs where nothing is left to
    merge."""
    return _decode_phase("kvc_decode_split", cache, q, hist_len, k_new, v_new, scale, out,
                         layer0, workspace, stream)


def decode_combine(cache: KVCache, q, hist_len, k_new=None, v_new=None,
                   scale: float | None = None, out=None, layer0: int = 0, workspace=None,
                   stream=None):
    """Second phase: takes the same arguments as the decode_split call it
    completes and merges its split states into `out`."""
    return _decode_phase("kvc_decode_combine", cache, q, hist_len, k_new, v_new, scale, out,
                         layer0, workspace, stream)


def attn_prefill(cache: KVCache, q, k, v, scale: float | None = None, out=None,
                 layer0: int = 0, stream=None):
    """Causal attention over an S-token prompt (q [n_layers,B,Hq,S,D], k/v
    [n_layers,B,Hkv,S,D]); also writes k/v into cache rows [0, S)."""
    n_layers, _, Hq, S, _ = q.shape
    _check_tensor("q", q, cache, (n_layers, cache.B, Hq, S, cache.D))
    _check_tensor("k", k, cache, (n_layers, cache.B, cache.Hkv, S, cache.D))
    _check_tensor("v", v, cache, (n_layers, cache.B, cache.Hkv, S, cache.D))
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, cache, q.shape)
    if scale is None:
        scale = 1.0 / math.sqrt(cache.D)
    d = cache.desc()
    _check(library().kvc_attn_prefill(
        ctypes.byref(d), layer0, n_layers, q.data_ptr(), k.data_ptr(), v.data_ptr(), Hq, S,
        float(scale), out.data_ptr(), _stream(cache.device, stream)))
    return out


def attn_prefill_varlen(cache: KVCache, q, k, v, cu_seqlens, hist_len, scale: float | None = None,
                        out=None, layer0: int = 0, stream=None):
    """Packed variable-length prefill with history: q [n_layers,T,Hq,D], k/v
    [n_layers,T,Hkv,D] token-major; sequence b's new tokens are rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1 and go to cache positions hist_len[b]
    ..; new token i of sequence b attends to positions 0 .. hist_len[b]+i."""
    n_layers, T, Hq, _ = q.shape
    _check_tensor("q", q, cache, (n_layers, T, Hq, cache.D))
    _check_tensor("k", k, cache, (n_layers, T, cache.Hkv, cache.D))
    _check_tensor("v", v, cache, (n_layers, T, cache.Hkv, cache.D))
    cu = np.ascontiguousarray(
        cu_seqlens.cpu().numpy() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens,
        dtype=np.int32)
    if cu.shape != (cache.B + 1,) or int(cu[-1]) != T:
        raise ValueError(f"cu_seqlens must have shape ({cache.B + 1},) and end at T = {T}")
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, cache, tuple(q.shape))
    if scale is None:
        scale = 1.0 / math.sqrt(cache.D)
    _, hp = _hist(hist_len, cache.B)
    d = cache.desc()
    _check(library().kvc_attn_prefill_varlen(
        ctypes.byref(d), layer0, n_layers, q.data_ptr(), k.data_ptr(), v.data_ptr(), Hq,
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), hp, float(scale), out.data_ptr(),
        _stream(cache.device, stream)))
    return out


# ---- paged cache ------------------------------------------------------------

def paged_cache_bytes(L, num_blocks, Hkv, block_size, D, dtype=torch.float32) -> int:
    """2 x L x num_blocks x Hkv x block_size x D x element size."""
    return int(library().kvc_paged_cache_bytes(L, num_blocks, Hkv, block_size, D,
                                               _DTYPE_CODE[dtype]))


class PagedKVCache:
    """Block pools ``k``, ``v`` of shape [L, num_blocks, Hkv, block_size, D]
    on one GPU, shared by all sequences; each call takes the sequences'
    block table (int32 [B, max_blocks] on the same device): position t of
    sequence b is row t % block_size of block block_table[b, t // block_size]."""

    def __init__(self, L, num_blocks, Hkv, block_size, D, dtype=torch.float32, device="cuda",
                 k=None, v=None):
        if dtype not in _DTYPE_CODE:
            raise TypeError(f"unsupported cache dtype {dtype}")
        shape = (L, num_blocks, Hkv, block_size, D)
        self.k = k if k is not None else torch.empty(shape, dtype=dtype, device=device)
        self.v = v if v is not None else torch.empty(shape, dtype=dtype, device=device)
        for t in (self.k, self.v):
            if tuple(t.shape) != shape or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError("pool tensors must be contiguous CUDA tensors of shape "
                                 f"{shape} and dtype {dtype}")
        self.L, self.num_blocks, self.Hkv, self.block_size, self.D = L, num_blocks, Hkv, block_size, D
        self.dtype = dtype

    @property
    def device(self):
        return self.k.device

    def desc(self) -> PagedCacheDesc:
        return PagedCacheDesc(self.k.data_ptr(), self.v.data_ptr(), self.L, self.num_blocks,
                              self.Hkv, self.block_size, self.D, _DTYPE_CODE[self.dtype])

    def geometry(self) -> tuple:
        return (self.L, self.num_blocks, self.Hkv, self.block_size, self.D, self.dtype)


def _check_table(cache, block_table):
    if (not isinstance(block_table, torch.Tensor) or block_table.dtype != torch.int32
            or block_table.device != cache.device or block_table.dim() != 2
            or not block_table.is_contiguous()):
        raise ValueError("block_table must be a contiguous int32 [B, max_blocks] tensor on "
                         f"{cache.device}")
    return block_table.shape[0], block_table.shape[1]


def paged_append(cache: PagedKVCache, k_new, v_new, hist_len, block_table, layer0: int = 0,
                 stream=None) -> None:
    """Write k_new/v_new ([n_layers,B,Hkv,N,D]) at positions hist_len[b] ..
    of each sequence, into the slots its block table names."""
    B, mb = _check_table(cache, block_table)
    n_layers, _, _, N, _ = k_new.shape
    shape = (n_layers, B, cache.Hkv, N, cache.D)
    _check_tensor("k_new", k_new, cache, shape)
    _check_tensor("v_new", v_new, cache, shape)
    _, hp = _hist(hist_len, B)
    d = cache.desc()
    _check(library().kvc_paged_append(ctypes.byref(d), layer0, n_layers, k_new.data_ptr(),
                                      v_new.data_ptr(), B, N, hp, block_table.data_ptr(), mb,
                                      _stream(cache.device, stream)))


def paged_decode_workspace_bytes(cache: PagedKVCache, n_layers, B, Hq, N, max_blocks) -> int:
    d = cache.desc()
    return int(library().kvc_paged_decode_workspace_bytes(ctypes.byref(d), n_layers, B, Hq, N,
                                                          max_blocks))


def new_paged_decode_workspace(cache: PagedKVCache, n_layers, B, Hq, N, max_blocks):
    return _aligned_workspace(paged_decode_workspace_bytes(cache, n_layers, B, Hq, N, max_blocks),
                              cache.device)


def _paged_decode(fn_name, cache, q, k_new, v_new, hist_len, block_table, scale, out, layer0,
                  workspace, stream):
    B, mb = _check_table(cache, block_table)
    n_layers, _, Hq, N, _ = q.shape
    shape = (n_layers, B, Hq, N, cache.D)
    _check_tensor("q", q, cache, shape)
    if k_new is not None:
        kshape = (n_layers, B, cache.Hkv, N, cache.D)
        _check_tensor("k_new", k_new, cache, kshape)
        _check_tensor("v_new", v_new, cache, kshape)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, cache, shape)
    if scale is None:
        scale = 1.0 / math.sqrt(cache.D)
    _, hp = _hist(hist_len, B)
    if workspace is None:
        need = paged_decode_workspace_bytes(cache, n_layers, B, Hq, N, mb)
        workspace = _default_workspace(cache, n_layers, Hq, N, stream, need=need, B=(B, mb))
    if workspace.device != cache.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the cache's device")
    d = cache.desc()
    lib = library()
    wsb = workspace.numel() * workspace.element_size()
    st = _stream(cache.device, stream)
    if k_new is None:
        status = lib.kvc_paged_attn_decode(ctypes.byref(d), layer0, n_layers, q.data_ptr(), Hq, B,
                                           N, hp, block_table.data_ptr(), mb, float(scale),
                                           out.data_ptr(), workspace.data_ptr(), wsb, st)
    else:
        status = lib.kvc_paged_decode_step(ctypes.byref(d), layer0, n_layers, q.data_ptr(),
                                           k_new.data_ptr(), v_new.data_ptr(), Hq, B, N, hp,
                                           block_table.data_ptr(), mb, float(scale),
                                           out.data_ptr(), workspace.data_ptr(), wsb, st)
    _check(status)
    return out


def paged_decode_step_dl(cache: PagedKVCache, q, k_new, v_new, hist_len_dev, hist_max: int,
                         block_table, scale: float | None = None, out=None, layer0: int = 0,
                         workspace=None, stream=None):
    """paged_decode_step with the lengths in ``hist_len_dev`` (int32 CUDA
    tensor [B], read on the device; ``hist_max`` bounds them), for steps
    captured once in a HIP graph."""
    B, mb = _check_table(cache, block_table)
    n_layers, _, Hq, N, _ = q.shape
    shape = (n_layers, B, Hq, N, cache.D)
    _check_tensor("q", q, cache, shape)
    kshape = (n_layers, B, cache.Hkv, N, cache.D)
    _check_tensor("k_new", k_new, cache, kshape)
    _check_tensor("v_new", v_new, cache, kshape)
    if (not isinstance(hist_len_dev, torch.Tensor) or hist_len_dev.dtype != torch.int32
            or not hist_len_dev.is_cuda or hist_len_dev.device != cache.device
            or not hist_len_dev.is_contiguous() or hist_len_dev.numel() != B):
        raise ValueError(f"hist_len_dev must be a contiguous int32 CUDA tensor of {B} elements "
                         "on the cache's device")
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, cache, shape)
    if scale is None:
        scale = 1.0 / math.sqrt(cache.D)
    if workspace is None:
        need = paged_decode_workspace_bytes(cache, n_layers, B, Hq, N, mb)
        workspace = _default_workspace(cache, n_layers, Hq, N, stream, need=need, B=(B, mb))
    if workspace.device != cache.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the cache's device")
    d = cache.desc()
    _check(library().kvc_paged_decode_step_dl(
        ctypes.byref(d), layer0, n_layers, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), Hq, B,
        N, hist_len_dev.data_ptr(), int(hist_max), block_table.data_ptr(), mb, float(scale),
        out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(cache.device, stream)))
    return out


def paged_attn_decode(cache: PagedKVCache, q, hist_len, block_table, scale: float | None = None,
                      out=None, layer0: int = 0, workspace=None, stream=None):
    """attn_decode over a paged cache (the N new rows already appended)."""
    return _paged_decode("attn", cache, q, None, None, hist_len, block_table, scale, out, layer0,
                         workspace, stream)


def paged_decode_step(cache: PagedKVCache, q, k_new, v_new, hist_len, block_table,
                      scale: float | None = None, out=None, layer0: int = 0, workspace=None,
                      stream=None):
    """paged_append + paged_attn_decode in the decode step's launches."""
    if k_new is None or v_new is None:
        raise ValueError("paged_decode_step needs k_new and v_new")
    return _paged_decode("step", cache, q, k_new, v_new, hist_len, block_table, scale, out, layer0,
                         workspace, stream)


def paged_attn_prefill_varlen(cache: PagedKVCache, q, k, v, cu_seqlens, hist_len, block_table,
                              scale: float | None = None, out=None, layer0: int = 0, stream=None):
    """attn_prefill_varlen into a paged cache: history read and new rows
    written through block_table (int32 [B, max_blocks] on the device)."""
    B, mb = _check_table(cache, block_table)
    n_layers, T, Hq, _ = q.shape
    _check_tensor("q", q, cache, (n_layers, T, Hq, cache.D))
    _check_tensor("k", k, cache, (n_layers, T, cache.Hkv, cache.D))
    _check_tensor("v", v, cache, (n_layers, T, cache.Hkv, cache.D))
    cu = np.ascontiguousarray(
        cu_seqlens.cpu().numpy() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens,
        dtype=np.int32)
    if cu.shape != (B + 1,) or int(cu[-1]) != T:
        raise ValueError(f"cu_seqlens must have shape ({B + 1},) and end at T = {T}")
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, cache, tuple(q.shape))
    if scale is None:
        scale = 1.0 / math.sqrt(cache.D)
    _, hp = _hist(hist_len, B)
    d = cache.desc()
    _check(library().kvc_paged_attn_prefill_varlen(
        ctypes.byref(d), layer0, n_layers, q.data_ptr(), k.data_ptr(), v.data_ptr(), Hq, B,
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), hp, block_table.data_ptr(), mb,
        float(scale), out.data_ptr(), _stream(cache.device, stream)))
    return out


def linear(x, wt, bias=None, ln=None, act=None, residual=None, out=None, ln_eps=1e-5,
           a_heads: int = 0, qkv_heads: int = 0, stream=None):
    """y = act(LN(x) wt^T + bias) + residual for the few rows of a decode step
    (fp32; x [M, K] with M <= 8, or [H, M, K/H] head-major with ``a_heads`` =
    H; wt [N, K]: the weight transposed).  ``ln`` is (gain, shift) or None;
    ``act`` is None or "gelu" (tanh form); with ``qkv_heads`` = H the result
    is laid out [3, H, M, N/(3H)] (q, k, v of the decode call); ``out`` may
    be ``residual``."""
    for name, t in (("x", x), ("wt", wt)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 \
                or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 CUDA tensor")
    if wt.dim() != 2:
        raise ValueError("wt must be [N, K]")
    N, K = wt.shape
    if a_heads:
        if x.dim() != 3 or x.shape[0] != a_heads or x.shape[0] * x.shape[2] != K:
            raise ValueError(f"x must be [{a_heads}, M, {K // max(a_heads, 1)}]")
        M = x.shape[1]
    else:
        if x.dim() != 2 or x.shape[1] != K:
            raise ValueError(f"x must be [M, {K}]")
        M = x.shape[0]

    def vec(name, t, n):
        if t is None:
            return None
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"{name} must be a contiguous fp32 CUDA tensor of {n} elements")
        return t

    bias = vec("bias", bias, N)
    g, b = (None, None) if ln is None else (vec("ln gain", ln[0], K), vec("ln shift", ln[1], K))
    residual = vec("residual", residual, M * N)
    shape = (3, qkv_heads, M, N // (3 * qkv_heads)) if qkv_heads else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    vec("out", out, M * N)
    codes = {None: 0, "gelu": 1}
    if act not in codes:
        raise ValueError(f"act must be None or 'gelu', got {act!r}")
    ptr = lambda t: None if t is None else t.data_ptr()
    _check(library().kvc_linear_f32(x.data_ptr(), a_heads, M, K, wt.data_ptr(), N, ptr(bias), ptr(g),
                                    ptr(b), float(ln_eps), codes[act], ptr(residual), out.data_ptr(),
                                    qkv_heads, _stream(x.device, stream)))
    return out


def _f32_matrix(name, t):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp32 CUDA tensor")
    return t


_gemm_ws = {}
_gemm_ws_retired = []


def gemm_workspace(M: int, K: int, N: int, device, stream=None):
    """The zero-filled split-K workspace kvc_gemm_f32 uses for this product:
    one per device, grown as needed (a retired buffer is kept alive, since
    queued work or a captured graph may still use it) and shared by every
    product that does not bring its own -- each call leaves its counters
    zero, so calls that follow one another may share it; products on
    different streams that can overlap must each pass their own.  None when
    the product does not split.  Not grown during graph capture: run the
    largest product once before capturing, or pass a workspace."""
    need = int(library().kvc_gemm_workspace_bytes(M, K, N))
    if need == 0:
        return None
    device = torch.device(device)
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    ws = _gemm_ws.get(device)
    if ws is None or ws.numel() < need:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("gemm: run the product once before capture, or pass a workspace")
        s = stream if stream is not None else torch.cuda.current_stream(device)
        with torch.cuda.stream(s):
            ws = _aligned_workspace(max(need, 0 if ws is None else ws.numel()), device)
        if device in _gemm_ws:
            _gemm_ws_retired.append(_gemm_ws[device])
        _gemm_ws[device] = ws
    return ws


def gemm(a, wt, bias=None, act=None, residual=None, out=None, a_heads: int = 0,
         qkv_heads: int = 0, workspace="auto", stream=None):
    """y = act(a wt^T + bias) + residual on the matrix cores (fp32), for
    prompt-sized inputs.  a is [M, K], or [H, M, K/H] head-major with
    ``a_heads`` = H; wt is the weight transposed, [N, K].  With ``qkv_heads``
    = H the result is laid out [3, H, M, N/(3H)] (q, k, v for the attention
    calls).  ``out`` may be ``residual``.  ``workspace``: "auto" (the
    device's shared split-K workspace, see gemm_workspace), None (no split)
    or a zero-filled uint8 tensor of at least kvc_gemm_workspace_bytes(M, K,
    N) bytes."""
    _f32_matrix("a", a)
    _f32_matrix("wt", wt)
    if wt.dim() != 2:
        raise ValueError("wt must be [N, K]")
    N, K = wt.shape
    if a_heads:
        if a.dim() != 3 or a.shape[0] != a_heads or a.shape[0] * a.shape[2] != K:
            raise ValueError(f"a must be [{a_heads}, M, {K // max(a_heads, 1)}]")
        M = a.shape[1]
    else:
        if a.dim() != 2 or a.shape[1] != K:
            raise ValueError(f"a must be [M, {K}]")
        M = a.shape[0]
    shape = (3, qkv_heads, M, N // (3 * qkv_heads)) if qkv_heads else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=a.device)
    _f32_matrix("out", out)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must have shape {shape}")
    for name, t, n in (("bias", bias, N), ("residual", residual, M * N)):
        if t is not None and (_f32_matrix(name, t).numel() != n):
            raise ValueError(f"{name} must have {n} elements")
    codes = {None: 0, "gelu": 1}
    if act not in codes:
        raise ValueError(f"act must be None or 'gelu', got {act!r}")
    ptr = lambda t: None if t is None else t.data_ptr()
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a tensor")
        workspace = gemm_workspace(M, K, N, a.device, stream) if M > 0 else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().kvc_gemm_f32(a.data_ptr(), a_heads, M, K, wt.data_ptr(), N, ptr(bias),
                                  codes[act], ptr(residual), out.data_ptr(), qkv_heads,
                                  ptr(workspace), ws_bytes, _stream(a.device, stream)))
    return out


def layer_norm(x, g, b, eps: float = 1e-5, out=None, stream=None):
    """Row-wise layer norm of x [M, K] (fp32) with gain g and shift b [K];
    ``out`` may be ``x``."""
    _f32_matrix("x", x)
    M, K = x.shape
    for name, t in (("g", g), ("b", b)):
        if _f32_matrix(name, t).numel() != K:
            raise ValueError(f"{name} must have {K} elements")
    if out is None:
        out = torch.empty_like(x)
    _f32_matrix("out", out)
    if tuple(out.shape) != (M, K):
        raise ValueError(f"out must have shape {(M, K)}")
    _check(library().kvc_layernorm_f32(x.data_ptr(), M, K, g.data_ptr(), b.data_ptr(), float(eps),
                                       out.data_ptr(), _stream(x.device, stream)))
    return out


def embed(wte, wpe, ids, pos0: int = 0, pos=None, out=None, stream=None):
    """Token + position embedding: row i is wte[ids[i]] + wpe[p0 + i], p0 =
    ``pos[0]`` (a device int32 tensor) if given, else ``pos0``.  wte [V, d],
    wpe [T, d] fp32; ids int64 [N] on the device.  Rows with an id or a
    position out of range come back NaN."""
    _f32_matrix("wte", wte)
    _f32_matrix("wpe", wpe)
    if wte.dim() != 2 or wpe.dim() != 2 or wte.shape[1] != wpe.shape[1]:
        raise ValueError("wte must be [V, d] and wpe [T, d]")
    if (not isinstance(ids, torch.Tensor) or ids.dtype != torch.int64 or ids.device != wte.device
            or ids.dim() != 1 or not ids.is_contiguous()):
        raise ValueError(f"ids must be a contiguous int64 vector on {wte.device}")
    if pos is not None and (not isinstance(pos, torch.Tensor) or pos.dtype != torch.int32
                            or pos.device != wte.device or pos.numel() < 1):
        raise ValueError(f"pos must be an int32 tensor on {wte.device}")
    (V, d), T, N = wte.shape, wpe.shape[0], ids.shape[0]
    if out is None:
        out = torch.empty((N, d), dtype=torch.float32, device=wte.device)
    _f32_matrix("out", out)
    if tuple(out.shape) != (N, d):
        raise ValueError(f"out must have shape {(N, d)}")
    _check(library().kvc_embed_f32(wte.data_ptr(), V, wpe.data_ptr(), T, d, ids.data_ptr(), N, int(pos0),
                                   None if pos is None else pos.data_ptr(), out.data_ptr(),
                                   _stream(wte.device, stream)))
    return out


def argmax(x, out=None, seq=None, seq_pos=None, stream=None):
    """Index of the first maximum of the fp32 vector ``x`` (a NaN counts as
    the largest value) into ``out`` (int64 [1] on the device).  With ``seq``
    (int64 [capacity]) and ``seq_pos`` (int64 [1]) the same launch also does
    ``seq_pos += 1; seq[seq_pos] = index`` (skipped past the capacity)."""
    if (not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.dim() != 1
            or not x.is_contiguous() or x.device.type != "cuda"):
        raise ValueError("x must be a contiguous fp32 vector on the GPU")
    if out is None:
        out = torch.empty(1, dtype=torch.int64, device=x.device)
    for name, t in (("out", out), ("seq", seq), ("seq_pos", seq_pos)):
        if t is not None and (not isinstance(t, torch.Tensor) or t.dtype != torch.int64
                              or t.device != x.device or t.numel() < 1 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int64 tensor on {x.device}")
    if (seq is None) != (seq_pos is None):
        raise ValueError("seq and seq_pos go together")
    _check(library().kvc_argmax_f32(x.data_ptr(), x.numel(), out.data_ptr(),
                                    None if seq is None else seq.data_ptr(),
                                    None if seq_pos is None else seq_pos.data_ptr(),
                                    0 if seq is None else seq.numel(), _stream(x.device, stream)))
    return out
