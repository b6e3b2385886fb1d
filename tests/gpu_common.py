"""Helpers shared by the GPU parity tests: moving seeded numpy inputs to the
device and back, and running one workload through the HIP path and through
the oracle on the same bytes."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from transformer_kv_cache_amd import synth
from transformer_kv_cache_amd.hostio import to_dev, to_host, torch_dtype  # noqa: F401 (re-exported)

TOL = {"f32": 1e-4, "bf16": 2e-2}  # max abs error against the oracle


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a


def run_gpu(w: synth.Workload, fused: bool = False):
    """Prefill (if any) then every decode step through libkvcache.so, as
    kvc_append + kvc_attn_decode, or as one kvc_decode_step if `fused`.
    Returns (outputs as numpy in the workload dtype, final K, final V)."""
    from transformer_kv_cache_amd import kvcache as K
    kc, vc = to_dev(w.k_cache), to_dev(w.v_cache)
    cache = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, torch_dtype(w.dtype), k=kc, v=vc)
    hist = w.hist.copy()
    outs = []
    if w.prefill is not None:
        q, k, v = (to_dev(a) for a in w.prefill)
        outs.append(K.attn_prefill(cache, q, k, v, scale=w.scale))
        hist[:] = w.prefill[0].shape[3]
    for (q, k, v) in w.steps:
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        if fused:
            outs.append(K.decode_step(cache, qd, kd, vd, hist, scale=w.scale))
        else:
            K.append(cache, kd, vd, hist)
            outs.append(K.attn_decode(cache, qd, hist, scale=w.scale))
        hist += q.shape[3]
    torch.cuda.synchronize()
    return [to_host(o) for o in outs], to_host(cache.k), to_host(cache.v)


def run_oracle(w: synth.Workload):
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    hist = w.hist.copy()
    outs = []
    if w.prefill is not None:
        outs.append(oracle.prefill(kc, vc, *w.prefill, w.scale))
        hist[:] = w.prefill[0].shape[3]
    for (q, k, v) in w.steps:
        oracle.append(kc, vc, k, v, hist)
        outs.append(oracle.attention(q, kc, vc, hist, w.scale))
        hist += q.shape[3]
    return outs, kc, vc


def assert_matches(w: synth.Workload, gpu, ref, tol=None):
    """Outputs within the dtype tolerance, cache bytes identical (canary
    slots included)."""
    tol = TOL[w.dtype] if tol is None else tol
    g_outs, g_k, g_v = gpu
    r_outs, r_k, r_v = ref
    assert len(g_outs) == len(r_outs)
    for n, (g, r) in enumerate(zip(g_outs, r_outs)):
        gf = synth.to_float(g)
        assert np.isfinite(gf).all(), f"{w.name} phase {n}: non-finite output"
        err = float(np.max(np.abs(gf - r))) if r.size else 0.0
        assert err <= tol, f"{w.name} phase {n}: max abs error {err:.3e} > {tol:.1e}"
    assert np.array_equal(bits(g_k), bits(r_k)), f"{w.name}: K cache bytes differ"
    assert np.array_equal(bits(g_v), bits(r_v)), f"{w.name}: V cache bytes differ"


def run_paged(w, fused, layer0=0, n_layers=None):
    """Every step of `w` through the paged entry points.  Returns (outputs,
    final K pool, final V pool) as numpy."""
    from transformer_kv_cache_amd import kvcache as K
    cache = K.PagedKVCache(w.L, w.num_blocks, w.Hkv, w.block_size, w.D, torch_dtype(w.dtype),
                           k=to_dev(w.k_pool), v=to_dev(w.v_pool))
    bt = torch.from_numpy(w.block_table).cuda()
    hist = w.hist.copy()
    outs = []
    for (q, k, v) in w.steps:
        nl = n_layers or q.shape[0]
        qd, kd, vd = (to_dev(np.ascontiguousarray(a[:nl])) for a in (q, k, v))
        if fused:
            outs.append(K.paged_decode_step(cache, qd, kd, vd, hist, bt, scale=w.scale,
                                            layer0=layer0))
        else:
            K.paged_append(cache, kd, vd, hist, bt, layer0=layer0)
            outs.append(K.paged_attn_decode(cache, qd, hist, bt, scale=w.scale, layer0=layer0))
        hist += q.shape[3]
    torch.cuda.synchronize()
    return [to_host(o) for o in outs], to_host(cache.k), to_host(cache.v)


def run_paged_oracle(w, layer0=0, n_layers=None):
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    hist = w.hist.copy()
    outs = []
    for (q, k, v) in w.steps:
        nl = n_layers or q.shape[0]
        q, k, v = (np.ascontiguousarray(a[:nl]) for a in (q, k, v))
        oracle.paged_append(kp, vp, k, v, hist, w.block_table, layer0=layer0)
        outs.append(oracle.paged_attention(q, kp, vp, hist, w.block_table, w.scale,
                                           layer0=layer0))
        hist += q.shape[3]
    return outs, kp, vp
