"""The GPT-2-style decoder around the cache entry points
(transformer_kv_cache_amd/gpt2.py) against the float64 oracle
(oracle/gpt2.py), on the same synthetic weights and token ids.  Following
[KV-2] "正确性先于性能": last-position logits at every greedy step, cached
and recomputed, a multi-token decode chunk, an empty cache, the position
limit, and the greedy tokens themselves.

Tolerance: logits within 1e-4 absolute (and the same greedy tokens).  The
GPU path is fp32 end to end (the library's fp32 matrix-core products, fp32
cache); rounding of some hundred chained fp32 operations on unit-scale
activations moves the logits by ~1e-6 to 1e-5, while a wiring mistake (a
position offset, a mask, a head split, a weight used untransposed) moves
them by ~1e-1."""
import numpy as np
import pytest
import torch

import oracle.gpt2 as G
from transformer_kv_cache_amd import synth

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_kv_cache_amd import kvcache as K
    K.library()  # fail loudly if the HIP library is missing


def model(w):
    from transformer_kv_cache_amd.gpt2 import GPT2
    return GPT2(w)


SMALL = dict(seed=21, L=2, d=128, H=2, V=300, T=64)


@pytest.mark.parametrize("cached", [True, False])
def test_small_greedy_generation_matches_oracle(cached):
    w = synth.gpt2_weights(**SMALL)
    prompt = synth.token_ids(22, 9, w.V).tolist()
    print(f"[gpt2] small greedy cached={cached}", flush=True)
    toks, z = model(w).generate(prompt, 16, cached=cached)
    rt, rz = G.generate(w, prompt, 16, cached=True)
    assert toks == rt
    assert np.max(np.abs(z - rz)) <= TOL


def test_small_chunked_decode_and_limits():
    """Prefill of one token (empty cache), a 5-token decode chunk, single
    tokens up to the last position: every position's logits vs the oracle's
    full forward."""
    from transformer_kv_cache_amd.gpt2 import GPT2
    w = synth.gpt2_weights(**SMALL)
    m = GPT2(w)
    ids = synth.token_ids(23, w.T, w.V)
    full = G.forward(w, ids)
    cache = m.new_cache()
    P = 0
    for n in [1, 5, 40, 1, 1, 16]:
        print(f"[gpt2] chunk P={P} n={n}", flush=True)
        z = m.forward(torch.from_numpy(ids[P:P + n]).cuda(), cache, P).double().cpu().numpy()
        assert np.max(np.abs(z - full[P:P + n])) <= TOL, (P, n)
        P += n
    assert P == w.T
    with pytest.raises(ValueError):
        m.forward(torch.from_numpy(ids[:1]).cuda(), cache, P)


def test_gpt2_small_shape_matches_oracle():
    """The pages' model size (12 layers, width 768, 12 heads, 50257-token
    vocabulary, 1024 positions): a 200-token prompt and three cached decode
    steps, last-position logits vs the oracle."""
    from transformer_kv_cache_amd.gpt2 import GPT2
    w = synth.gpt2_weights(seed=24)
    m = GPT2(w)
    ids = synth.token_ids(25, 203, w.V)
    cache = m.new_cache()
    oc = G.Cache(w)
    print("[gpt2] full-size prefill 200", flush=True)
    z = m.forward(torch.from_numpy(ids[:200]).cuda(), cache, 0, last_only=True)
    rz = G.forward(w, ids[:200], oc)[-1]
    assert np.max(np.abs(z[0].double().cpu().numpy() - rz)) <= TOL
    for P in (200, 201, 202):
        print(f"[gpt2] full-size decode P={P}", flush=True)
        z = m.forward(torch.from_numpy(ids[P:P + 1]).cuda(), cache, P, last_only=True)
        rz = G.forward(w, ids[P:P + 1], oc)[-1]
        assert np.max(np.abs(z[0].double().cpu().numpy() - rz)) <= TOL


def test_graph_generation_loop_matches_oracle():
    """The whole token step captured once (device lengths) and replayed:
    the greedy tokens equal the oracle's cached generation."""
    from transformer_kv_cache_amd.gpt2 import GPT2
    w = synth.gpt2_weights(**SMALL)
    prompt = synth.token_ids(26, 7, w.V).tolist()
    print("[gpt2] graph generation loop", flush=True)
    toks, ms = GPT2(w).generate_graph(prompt, 20)
    rt, _ = G.generate(w, prompt, 20, cached=True)
    assert toks == rt
    assert ms > 0
