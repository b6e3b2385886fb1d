"""Seeded synthetic inputs for the KV-cache attention workloads.

This module is shared by the tests, the smoke check and the benchmark, and
feeds both the HIP path and the CPU oracle with the same bytes.  It holds no
attention arithmetic: only random draws, bf16 rounding of the draws, canary
fills and the layout of the draws into cache-shaped arrays.

Recipe:
  * ``numpy.random.default_rng(seed)`` (PCG64), ``standard_normal(shape,
    dtype=float32)``: N(0,1) fp32 samples, as GPT-2-Small-shaped activations
    would be after their projections (the pages use trained weights, which are
    not available; N(0,1) stands in for them).
  * Draw order inside one call: lengths first (if any), then history K, history
    V, then for each phase (prefill, then each decode step) q, k, v as whole
    ``[n_layers, B, H, N, D]`` tensors.
  * bf16 tensors are the fp32 draws rounded once to nearest-even.
  * Cache slots that hold no token carry a NaN canary bit pattern, so a kernel
    that reads past a sequence's length, or writes where it should not, shows
    up bit-exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32_CANARY = np.uint32(0x7FC0CA7A)  # quiet NaN with a payload
BF16_CANARY = np.uint16(0x7FCA)  # quiet NaN


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 by round-to-nearest-even; returns uint16 bits.
    NaN inputs map to the quiet NaN 0x7FC0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_dtype(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 draws stored as 'f32' (float32) or 'bf16' (uint16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x_f32)
    raise ValueError(dtype)


def to_float(x: np.ndarray) -> np.ndarray:
    """Stored array (float32 or bf16 bits) to float64 values."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def canary_cache(shape, dtype: str) -> np.ndarray:
    """A cache-shaped array filled entirely with the canary pattern."""
    if dtype == "f32":
        return np.full(shape, F32_CANARY, dtype=np.uint32).view(np.float32)
    if dtype == "bf16":
        return np.full(shape, BF16_CANARY, dtype=np.uint16)
    raise ValueError(dtype)


def is_canary(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.float32:
        return x.view(np.uint32) == F32_CANARY
    return x == BF16_CANARY


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


@dataclass
class Workload:
    """One seeded workload: cache geometry, history, and phases.

    ``k_cache``/``v_cache`` are ``[L,B,Hkv,Tmax,D]`` with history rows
    [0, hist[b]) filled and the rest canary.  ``prefill`` is None or
    ``(q, k, v)`` of ``[L,B,H,S,D]``; ``steps`` is a list of ``(q, k, v)`` of
    ``[L,B,H,N,D]`` decode inputs applied in order after the prefill.
    """
    name: str
    dtype: str
    L: int
    B: int
    Hq: int
    Hkv: int
    D: int
    Tmax: int
    hist: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    prefill: tuple | None = None
    steps: list = field(default_factory=list)
    # score scale of every call; None means the usual 1/sqrt(D)
    scale_value: float | None = None

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D) if self.scale_value is None else self.scale_value


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def make_workload(name, *, seed, dtype, L, B, Hq, Hkv, D, Tmax, hist=None,
                  prefill_len=0, step_lens=(), draw_lengths=None) -> Workload:
    """General generator.  ``hist`` gives each sequence's history length (rows
    drawn N(0,1) into the cache); ``draw_lengths=(lo, hi)`` instead draws the
    number of keys each sequence sees after one appended row,
    L_b ~ U[lo, hi], so that hist = L_b - 1."""
    rng = np.random.default_rng(seed)
    if draw_lengths is not None:
        lo, hi = draw_lengths
        seen = rng.integers(lo, hi + 1, size=B)
        hist = (seen - 1).astype(np.int32)
    elif hist is None:
        hist = np.zeros(B, dtype=np.int32)
    hist = np.asarray(hist, dtype=np.int32).copy()
    if hist.shape != (B,):
        hist = np.full(B, int(hist.reshape(-1)[0]), dtype=np.int32)
    shape = (L, B, Hkv, Tmax, D)
    kc = canary_cache(shape, dtype)
    vc = canary_cache(shape, dtype)
    pmax = int(hist.max()) if B else 0
    if pmax > 0:
        kh = as_dtype(_normal(rng, (L, B, Hkv, pmax, D)), dtype)
        vh = as_dtype(_normal(rng, (L, B, Hkv, pmax, D)), dtype)
        for b in range(B):
            p = int(hist[b])
            kc[:, b, :, :p, :] = kh[:, b, :, :p, :]
            vc[:, b, :, :p, :] = vh[:, b, :, :p, :]
    pre = None
    if prefill_len:
        pre = tuple(as_dtype(_normal(rng, (L, B, H, prefill_len, D)), dtype)
                    for H in (Hq, Hkv, Hkv))
    steps = []
    for n in step_lens:
        steps.append(tuple(as_dtype(_normal(rng, (L, B, H, n, D)), dtype)
                           for H in (Hq, Hkv, Hkv)))
    return Workload(name, dtype, L, B, Hq, Hkv, D, Tmax, hist, kc, vc, pre, steps)


# ---- the five workloads, GPT-2 Small shaped (12 layers, 12 heads, D = 64) ----

def single_layer_generation(seed=0) -> Workload:
    """One attention layer, fp32, B=1, H=12, D=64, Tmax=32: a 16-token prompt
    prefill, then four single-token decode steps."""
    return make_workload("single_layer_generation", seed=seed, dtype="f32", L=1, B=1,
                         Hq=12, Hkv=12, D=64, Tmax=32, prefill_len=16,
                         step_lens=(1, 1, 1, 1))


def decode_12layer(P, seed=0, dtype="f32") -> Workload:
    """All 12 layers, B=1, H=12, D=64, Tmax=1024: history P, one new token."""
    return make_workload(f"decode_12layer_P{P}", seed=seed, dtype=dtype, L=12, B=1,
                         Hq=12, Hkv=12, D=64, Tmax=1024, hist=[P], step_lens=(1,))


def chunked_decode(P=1000, N=8, seed=0) -> Workload:
    """12 layers, fp32, B=1, H=12, D=64: history P plus N rows in one call."""
    return make_workload(f"chunked_decode_P{P}_N{N}", seed=seed, dtype="f32", L=12, B=1,
                         Hq=12, Hkv=12, D=64, Tmax=1024, hist=[P], step_lens=(N,))


def causal_prefill(S, dtype, seed=0, L=12) -> Workload:
    """Causal prefill, B=1, H=12, D=64, prompt S, into an empty Tmax=1024 cache."""
    return make_workload(f"prefill_S{S}_{dtype}", seed=seed, dtype=dtype, L=L, B=1,
                         Hq=12, Hkv=12, D=64, Tmax=1024, prefill_len=S)


def batched_decode(seed=0, gqa=False, B=8, L=12, tp=1) -> Workload:
    """bf16 cache, B sequences whose visible-key counts are U[1, 1024],
    Tmax=1024; MHA (H=12, D=64) or GQA (32 query heads, 8 KV heads, D=128).
    ``tp`` > 1 (GQA only) gives one GPU's share under tp-way tensor
    parallelism over the KV heads: 32/tp query and 8/tp KV heads, the same
    lengths (they are drawn first)."""
    if gqa:
        if tp < 1 or 8 % tp:
            raise ValueError("tp must divide the 8 KV heads")
        return make_workload("batched_decode_gqa" + (f"_tp{tp}" if tp > 1 else ""), seed=seed,
                             dtype="bf16", L=L, B=B, Hq=32 // tp, Hkv=8 // tp, D=128, Tmax=1024,
                             draw_lengths=(1, 1024), step_lens=(1,))
    if tp != 1:
        raise ValueError("tp applies to the GQA workload")
    return make_workload("batched_decode_mha", seed=seed, dtype="bf16", L=L, B=B,
                         Hq=12, Hkv=12, D=64, Tmax=1024, draw_lengths=(1, 1024),
                         step_lens=(1,))


# ---- paged cache inputs -----------------------------------------------------

@dataclass
class PagedWorkload:
    """Seeded inputs for a paged cache: pools ``k_pool``/``v_pool`` of shape
    ``[L, num_blocks, Hkv, block_size, D]`` and a block table ``int32[B,
    max_blocks]``.  Every block a table names holds N(0,1) rows; the blocks no
    table names hold the canary.  Which rows make up a sequence's history is
    up to the code under test -- this module only draws bytes and block ids.
    ``steps`` as in ``Workload``."""
    name: str
    dtype: str
    L: int
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    num_blocks: int
    max_blocks: int
    hist: np.ndarray
    block_table: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    steps: list = field(default_factory=list)
    # score scale of every call; None means the usual 1/sqrt(D)
    scale_value: float | None = None

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D) if self.scale_value is None else self.scale_value


def make_paged_workload(name, *, seed, dtype, L, B, Hq, Hkv, D, block_size, max_blocks,
                        hist=None, step_lens=(1,), draw_lengths=None, spare_blocks=7,
                        shared_prefix_blocks=0) -> PagedWorkload:
    """Each sequence gets ``max_blocks`` distinct blocks drawn from a shuffled
    pool of ``B * max_blocks + spare_blocks`` (the first
    ``shared_prefix_blocks`` entries of every row are the same blocks, as for
    a common prompt).  ``hist``/``draw_lengths`` as in ``make_workload``."""
    rng = np.random.default_rng(seed)
    if draw_lengths is not None:
        lo, hi = draw_lengths
        hist = (rng.integers(lo, hi + 1, size=B) - 1).astype(np.int32)
    elif hist is None:
        hist = np.zeros(B, dtype=np.int32)
    hist = np.asarray(hist, dtype=np.int32).copy()
    if hist.shape != (B,):
        hist = np.full(B, int(hist.reshape(-1)[0]), dtype=np.int32)
    sp = shared_prefix_blocks
    num_blocks = sp + B * (max_blocks - sp) + spare_blocks
    ids = rng.permutation(num_blocks).astype(np.int32)
    table = np.empty((B, max_blocks), np.int32)
    table[:, :sp] = ids[:sp]
    table[:, sp:] = ids[sp:sp + B * (max_blocks - sp)].reshape(B, max_blocks - sp)
    shape = (L, num_blocks, Hkv, block_size, D)
    kp = canary_cache(shape, dtype)
    vp = canary_cache(shape, dtype)
    used = np.unique(table)
    kp[:, used] = as_dtype(_normal(rng, (L, used.size, Hkv, block_size, D)), dtype)
    vp[:, used] = as_dtype(_normal(rng, (L, used.size, Hkv, block_size, D)), dtype)
    steps = [tuple(as_dtype(_normal(rng, (L, B, H, n, D)), dtype) for H in (Hq, Hkv, Hkv))
             for n in step_lens]
    return PagedWorkload(name, dtype, L, B, Hq, Hkv, D, block_size, num_blocks, max_blocks,
                         hist, table, kp, vp, steps)


def paged_decode_12layer(P, block_size=16, seed=0, dtype="f32", N=1) -> PagedWorkload:
    """The 12-layer decode workload (B=1, H=12, D=64, 1024 positions) on a
    paged cache of ``block_size``-position blocks."""
    return make_paged_workload(f"paged_decode_12layer_P{P}_bs{block_size}_N{N}", seed=seed,
                               dtype=dtype, L=12, B=1, Hq=12, Hkv=12, D=64,
                               block_size=block_size, max_blocks=1024 // block_size, hist=[P],
                               step_lens=(N,))


def paged_batched_decode(seed=0, gqa=False, block_size=16, B=8, L=12) -> PagedWorkload:
    """The batched bf16 decode workload (visible keys U[1, 1024]) on a paged
    cache; MHA (H=12, D=64) or GQA (32 query heads, 8 KV heads, D=128)."""
    Hq, Hkv, D = (32, 8, 128) if gqa else (12, 12, 64)
    return make_paged_workload(f"paged_batched_{'gqa' if gqa else 'mha'}_bs{block_size}",
                               seed=seed, dtype="bf16", L=L, B=B, Hq=Hq, Hkv=Hkv, D=D,
                               block_size=block_size, max_blocks=1024 // block_size,
                               draw_lengths=(1, 1024))


# ---- packed variable-length prefill inputs ---------------------------------

@dataclass
class VarlenWorkload:
    """A cache with per-sequence history (as ``Workload``) plus one packed
    prefill: ``q`` ``[L, T, Hq, D]``, ``k``/``v`` ``[L, T, Hkv, D]``
    token-major, sequence b's new tokens at rows ``cu_seqlens[b] ..
    cu_seqlens[b+1]-1``."""
    name: str
    dtype: str
    L: int
    B: int
    Hq: int
    Hkv: int
    D: int
    Tmax: int
    hist: np.ndarray
    cu_seqlens: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


def make_varlen_workload(name, *, seed, dtype, L, B, Hq, Hkv, D, Tmax, hist, lens) -> VarlenWorkload:
    base = make_workload(name, seed=seed, dtype=dtype, L=L, B=B, Hq=Hq, Hkv=Hkv, D=D, Tmax=Tmax,
                         hist=hist)
    rng = np.random.default_rng(seed + 7919)
    lens = np.asarray(lens, dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = (as_dtype(_normal(rng, (L, T, H, D)), dtype) for H in (Hq, Hkv, Hkv))
    return VarlenWorkload(name, dtype, L, B, Hq, Hkv, D, Tmax, base.hist, cu, base.k_cache,
                          base.v_cache, q, k, v)


def varlen_prefill_batch(seed=0, dtype="bf16", gqa=False, B=8, L=12) -> VarlenWorkload:
    """A packed batch of B prompts: prompt lengths U[1, 512] on cached
    prefixes U[0, 512] (a prefix-cache hit, or an earlier chunk), Tmax=1024;
    MHA (H=12, D=64) or GQA (32 query heads, 8 KV heads, D=128)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 513, size=B)
    hist = rng.integers(0, 513, size=B)
    Hq, Hkv, D = (32, 8, 128) if gqa else (12, 12, 64)
    return make_varlen_workload(f"varlen_prefill_{'gqa' if gqa else 'mha'}_{dtype}", seed=seed,
                                dtype=dtype, L=L, B=B, Hq=Hq, Hkv=Hkv, D=D, Tmax=1024, hist=hist,
                                lens=lens)


@dataclass
class PagedVarlenWorkload:
    """A paged cache with per-sequence history (as ``PagedWorkload``) plus one
    packed prefill laid out as in ``VarlenWorkload``."""
    pool: PagedWorkload
    cu_seqlens: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    def __getattr__(self, name):
        return getattr(self.pool, name)


def make_paged_varlen_workload(name, *, seed, dtype, L, B, Hq, Hkv, D, block_size, max_blocks,
                               hist, lens, shared_prefix_blocks=0) -> PagedVarlenWorkload:
    pool = make_paged_workload(name, seed=seed, dtype=dtype, L=L, B=B, Hq=Hq, Hkv=Hkv, D=D,
                               block_size=block_size, max_blocks=max_blocks, hist=hist,
                               step_lens=(), shared_prefix_blocks=shared_prefix_blocks)
    rng = np.random.default_rng(seed + 104729)
    lens = np.asarray(lens, dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = (as_dtype(_normal(rng, (L, T, H, D)), dtype) for H in (Hq, Hkv, Hkv))
    return PagedVarlenWorkload(pool, cu, q, k, v)


def paged_from_contiguous(k_cache, v_cache, block_size, seed=0, spare_blocks=3):
    """The rows of a contiguous cache ``[L, B, Hkv, Tmax, D]`` laid out in
    block pools through a shuffled table: returns (k_pool, v_pool,
    block_table), block ``table[b][j]`` holding positions ``j*block_size ..
    (j+1)*block_size - 1`` of sequence ``b``; spare blocks hold canaries."""
    L, B, Hkv, Tmax, D = k_cache.shape
    if Tmax % block_size:
        raise ValueError("Tmax must be a multiple of block_size")
    mb = Tmax // block_size
    nblk = B * mb + spare_blocks
    rng = np.random.default_rng(seed)
    table = rng.permutation(nblk)[:B * mb].astype(np.int32).reshape(B, mb)
    shape = (L, nblk, Hkv, block_size, D)
    dtype = "bf16" if k_cache.dtype == np.uint16 else "f32"
    kp, vp = canary_cache(shape, dtype), canary_cache(shape, dtype)
    blocks = lambda c: np.transpose(c.reshape(L, B, Hkv, mb, block_size, D), (0, 1, 3, 2, 4, 5))
    kp[:, table.reshape(-1)] = blocks(k_cache).reshape(L, B * mb, Hkv, block_size, D)
    vp[:, table.reshape(-1)] = blocks(v_cache).reshape(L, B * mb, Hkv, block_size, D)
    return kp, vp, table


# ---- synthetic GPT-2-shaped weights ------------------------------------------

@dataclass
class GPT2Weights:
    """Random weights of a GPT-2-style decoder (the pages run GPT-2 Small:
    12 layers, width 768, 12 heads, 1024 positions; trained weights are not
    available, so N(0, 0.02) draws stand in for them).  Per-layer tensors are
    stacked on a leading layer axis; linear weights are ``[in, out]``."""
    L: int
    d: int
    H: int
    V: int
    T: int
    wte: np.ndarray      # [V, d] token embedding, also the output projection
    wpe: np.ndarray      # [T, d] position embedding
    ln1_g: np.ndarray    # [L, d]
    ln1_b: np.ndarray
    w_qkv: np.ndarray    # [L, d, 3d]
    b_qkv: np.ndarray    # [L, 3d]
    w_o: np.ndarray      # [L, d, d]
    b_o: np.ndarray      # [L, d]
    ln2_g: np.ndarray
    ln2_b: np.ndarray
    w_fc: np.ndarray     # [L, d, 4d]
    b_fc: np.ndarray     # [L, 4d]
    w_pr: np.ndarray     # [L, 4d, d]
    b_pr: np.ndarray     # [L, d]
    lnf_g: np.ndarray    # [d]
    lnf_b: np.ndarray

    @property
    def D(self) -> int:
        return self.d // self.H


def gpt2_weights(seed=0, L=12, d=768, H=12, V=50257, T=1024) -> GPT2Weights:
    """fp32 draws in field order: weights N(0, 0.02), biases N(0, 0.02),
    layer-norm gains 1 + N(0, 0.1) and shifts N(0, 0.02)."""
    rng = np.random.default_rng(seed)
    n = lambda *shape, s=0.02: (s * rng.standard_normal(shape, dtype=np.float32)).astype(np.float32)
    g = lambda *shape: (1.0 + n(*shape, s=0.1)).astype(np.float32)
    return GPT2Weights(L, d, H, V, T,
                       wte=n(V, d), wpe=n(T, d),
                       ln1_g=g(L, d), ln1_b=n(L, d),
                       w_qkv=n(L, d, 3 * d), b_qkv=n(L, 3 * d),
                       w_o=n(L, d, d), b_o=n(L, d),
                       ln2_g=g(L, d), ln2_b=n(L, d),
                       w_fc=n(L, d, 4 * d), b_fc=n(L, 4 * d),
                       w_pr=n(L, 4 * d, d), b_pr=n(L, d),
                       lnf_g=g(d), lnf_b=n(d))


def token_ids(seed, n, V) -> np.ndarray:
    """n token ids uniform in [0, V)."""
    return np.random.default_rng(seed).integers(0, V, size=n).astype(np.int64)
