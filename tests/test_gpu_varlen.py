"""Parity of kvc_attn_prefill_varlen (through the C ABI) with the oracle's
packed variable-length prefill, on the same seeded bytes: cache bytes
bit-exact (canaries included), outputs within 1e-4 (fp32) or 2e-2 (bf16).
Covers ragged lengths (0, 1, tile edges), cached prefixes on and off tile
edges, GQA, batches over one launch's slice, layer0 > 0, and the identities
that tie it to the padded prefill and to chunking."""
import numpy as np
import pytest
import torch

import oracle
from transformer_kv_cache_amd import synth
from gpu_common import TOL, bits, to_dev, to_host, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_kv_cache_amd import kvcache as K
    K.library()  # fail loudly if the HIP library is missing
    return K


def run_varlen(w, layer0=0, n_layers=None):
    from transformer_kv_cache_amd import kvcache as K
    nl = n_layers or w.q.shape[0]
    cache = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, torch_dtype(w.dtype), k=to_dev(w.k_cache),
                      v=to_dev(w.v_cache))
    q, k, v = (to_dev(np.ascontiguousarray(a[:nl])) for a in (w.q, w.k, w.v))
    o = K.attn_prefill_varlen(cache, q, k, v, w.cu_seqlens, w.hist, scale=w.scale, layer0=layer0)
    torch.cuda.synchronize()
    return to_host(o), to_host(cache.k), to_host(cache.v)


def check(w, layer0=0, n_layers=None):
    lens = np.diff(w.cu_seqlens)
    print(f"[varlen] {w.name} dtype={w.dtype} L={w.L} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
          f"lens={lens.tolist()[:8]} hist={w.hist.tolist()[:8]} layer0={layer0}", flush=True)
    o, gk, gv = run_varlen(w, layer0, n_layers)
    nl = n_layers or w.q.shape[0]
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    ref = oracle.prefill_varlen(kc, vc, *(np.ascontiguousarray(a[:nl]) for a in (w.q, w.k, w.v)),
                                w.cu_seqlens, w.hist, w.scale, layer0=layer0)
    assert np.array_equal(bits(gk), bits(kc)), "K cache bytes differ"
    assert np.array_equal(bits(gv), bits(vc)), "V cache bytes differ"
    of = synth.to_float(o)
    assert np.isfinite(of).all()
    err = float(np.max(np.abs(of.astype(np.float64) - ref))) if o.size else 0.0
    assert err <= TOL[w.dtype], f"max abs err {err}"
    return o


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_ragged_with_history(dtype):
    w = synth.make_varlen_workload(f"ragged_{dtype}", seed=51, dtype=dtype, L=3, B=7, Hq=12,
                                   Hkv=12, D=64, Tmax=1024,
                                   hist=[0, 1, 63, 64, 65, 300, 900],
                                   lens=[130, 1, 0, 127, 128, 129, 124])
    check(w)


@pytest.mark.parametrize("gqa", [False, True])
def test_varlen_prefill_batch(gqa):
    check(synth.varlen_prefill_batch(seed=52, gqa=gqa))


def test_varlen_fp32_gqa_d128_layer0():
    w = synth.make_varlen_workload("gqa_f32_d128", seed=53, dtype="f32", L=3, B=3, Hq=8, Hkv=2,
                                   D=128, Tmax=512, hist=[10, 0, 200], lens=[70, 257, 31])
    check(w, layer0=1, n_layers=2)


def test_varlen_many_sequences():
    """70 sequences: two launches over batch slices."""
    rng = np.random.default_rng(54)
    w = synth.make_varlen_workload("many", seed=54, dtype="bf16", L=1, B=70, Hq=4, Hkv=4, D=64,
                                   Tmax=256, hist=rng.integers(0, 100, size=70),
                                   lens=rng.integers(0, 60, size=70))
    check(w)


def test_varlen_no_history_equals_padded_prefill():
    """Equal lengths, no history: the packed call and kvc_attn_prefill on
    the padded layout give the same bytes (one kernel, two layouts)."""
    from transformer_kv_cache_amd import kvcache as K
    w = synth.causal_prefill(300, "bf16", seed=55, L=4)
    q, k, v = w.prefill
    L, B, Hq, S, D = q.shape
    cache = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, torch.bfloat16, k=to_dev(w.k_cache),
                      v=to_dev(w.v_cache))
    o_pad = to_host(K.attn_prefill(cache, to_dev(q), to_dev(k), to_dev(v), scale=w.scale))
    pk = lambda x: np.ascontiguousarray(np.transpose(x, (0, 1, 3, 2, 4)).reshape(L, B * S, -1, D))
    cache2 = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, torch.bfloat16, k=to_dev(w.k_cache),
                       v=to_dev(w.v_cache))
    o_pack = to_host(K.attn_prefill_varlen(cache2, to_dev(pk(q)), to_dev(pk(k)), to_dev(pk(v)),
                                           [0, S], [0], scale=w.scale))
    assert np.array_equal(o_pack, pk(o_pad))
    assert np.array_equal(to_host(cache.k), to_host(cache2.k))


def test_varlen_chunked_prefill_matches_whole_prompt():
    """A 700-token prompt prefilled whole, and in chunks of 300 + 400 (the
    second with history 300), leave the same cache and the same outputs for
    the last 400 tokens, within tolerance ([KV-4] "Prefill 阶段": chunked
    prefill)."""
    from transformer_kv_cache_amd import kvcache as K
    w = synth.causal_prefill(700, "f32", seed=56, L=2)
    q, k, v = w.prefill
    pk = lambda x: np.ascontiguousarray(np.transpose(x, (0, 1, 3, 2, 4)).reshape(x.shape[0], -1, x.shape[2], x.shape[4]))
    cache = K.KVCache(w.L, 1, w.Hkv, w.Tmax, w.D, torch.float32, k=to_dev(w.k_cache),
                      v=to_dev(w.v_cache))
    whole = to_host(K.attn_prefill(cache, to_dev(q), to_dev(k), to_dev(v), scale=w.scale))
    cache2 = K.KVCache(w.L, 1, w.Hkv, w.Tmax, w.D, torch.float32, k=to_dev(w.k_cache),
                       v=to_dev(w.v_cache))
    chunk = lambda x, a, b: pk(np.ascontiguousarray(x[:, :, :, a:b]))
    K.attn_prefill_varlen(cache2, to_dev(chunk(q, 0, 300)), to_dev(chunk(k, 0, 300)),
                          to_dev(chunk(v, 0, 300)), [0, 300], [0], scale=w.scale)
    o2 = to_host(K.attn_prefill_varlen(cache2, to_dev(chunk(q, 300, 700)),
                                       to_dev(chunk(k, 300, 700)), to_dev(chunk(v, 300, 700)),
                                       [0, 400], [300], scale=w.scale))
    assert np.array_equal(bits(to_host(cache.k)), bits(to_host(cache2.k)))
    assert np.array_equal(bits(to_host(cache.v)), bits(to_host(cache2.v)))
    ref = pk(np.ascontiguousarray(whole[:, :, :, 300:]))
    assert float(np.max(np.abs(o2.astype(np.float64) - ref))) <= TOL["f32"]
