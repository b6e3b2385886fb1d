"""Parity of the paged-cache entry points (through the C ABI) with the CPU
oracle's paged functions, on the same seeded pools and block tables: pool
bytes bit-exact after every call (canaries in blocks no table names, and in
unwritten rows, included), outputs within 1e-4 (fp32) or 2e-2 (bf16) max abs
error.  Covers the one-row-per-KV-head kernel and the matrix-core kernel,
block sizes 1 to 256, histories on and off block boundaries, shared prefix
blocks, layer0 > 0, and the fused step against append + attention."""
import numpy as np
import pytest
import torch

import oracle
from transformer_kv_cache_amd import synth
from gpu_common import TOL, bits, run_paged, run_paged_oracle, to_dev, to_host, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_kv_cache_amd import kvcache as K
    K.library()  # fail loudly if the HIP library is missing
    return K


def check(w, fused, layer0=0, n_layers=None):
    print(f"[paged] {w.name} dtype={w.dtype} L={w.L} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
          f"bs={w.block_size} blocks={w.num_blocks} hist={w.hist.tolist()[:8]} fused={fused} "
          f"layer0={layer0}", flush=True)
    g_outs, gk, gv = run_paged(w, fused, layer0, n_layers)
    r_outs, rk, rv = run_paged_oracle(w, layer0, n_layers)
    assert np.array_equal(bits(gk), bits(rk)), "K pool bytes differ"
    assert np.array_equal(bits(gv), bits(rv)), "V pool bytes differ"
    for n, (g, r) in enumerate(zip(g_outs, r_outs)):
        gf = synth.to_float(g)
        assert np.isfinite(gf).all(), f"{w.name} step {n}: non-finite output"
        err = float(np.max(np.abs(gf.astype(np.float64) - r)))
        assert err <= TOL[w.dtype], f"{w.name} step {n}: max abs err {err}"
    return g_outs


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("bs", [16, 64])
def test_paged_decode_12layer(fused, bs):
    """The headline workload (12 layers, fp32, T=1024) on a paged cache."""
    check(synth.paged_decode_12layer(1023, block_size=bs, seed=41), fused)


@pytest.mark.parametrize("P", [0, 1, 15, 16, 17, 511, 1008])
def test_paged_histories_around_block_edges(P):
    check(synth.paged_decode_12layer(P, block_size=16, seed=42 + P), True)


@pytest.mark.parametrize("bs", [1, 2, 8, 32, 128, 256])
def test_paged_block_sizes(bs):
    w = synth.make_paged_workload(f"paged_bs{bs}", seed=43, dtype="f32", L=2, B=3, Hq=4, Hkv=4,
                                  D=64, block_size=bs, max_blocks=512 // bs,
                                  hist=[0, 200, 509], step_lens=(1, 1))
    check(w, True)


@pytest.mark.parametrize("block_size", [1, 16, 256])
@pytest.mark.parametrize("fused", [False, True])
def test_paged_chunked(fused, block_size):
    """N = 8 new rows per call, 12 layers (144 KV heads: one workgroup per
    head over the whole key range, block ids staged in LDS) through the
    table, at block sizes from one position to more than a chunk."""
    check(synth.paged_decode_12layer(1000, block_size=block_size, seed=44, N=8), fused)


@pytest.mark.parametrize("gqa", [False, True])
def test_paged_batched_bf16(gqa):
    check(synth.paged_batched_decode(seed=45, gqa=gqa, block_size=16), True)


def test_paged_shared_prefix_and_layer0():
    """Sequences share their first 4 blocks (a common prompt); layers 1..2 of
    a 3-layer pool; two steps."""
    w = synth.make_paged_workload("paged_shared_prefix", seed=46, dtype="bf16", L=3, B=4,
                                  Hq=8, Hkv=2, D=128, block_size=16, max_blocks=16,
                                  hist=[64, 70, 100, 250], step_lens=(1, 3),
                                  shared_prefix_blocks=4)
    check(w, True, layer0=1, n_layers=2)


def test_paged_fused_equals_two_calls_bitwise():
    """paged_decode_step and paged_append + paged_attn_decode: same bytes."""
    for w in (synth.paged_decode_12layer(700, block_size=32, seed=47),
              synth.paged_batched_decode(seed=48, gqa=True, block_size=32)):
        a, ak, av = run_paged(w, True)
        b, bk, bv = run_paged(w, False)
        assert np.array_equal(bits(ak), bits(bk)) and np.array_equal(bits(av), bits(bv))
        for x, y in zip(a, b):
            assert np.array_equal(bits(x), bits(y)), w.name


def test_paged_matches_contiguous_outputs():
    """The same history laid out contiguously and in shuffled blocks gives
    bit-identical outputs (the kernels visit the same keys in the same
    order)."""
    from transformer_kv_cache_amd import kvcache as K
    w = synth.decode_12layer(900, seed=49)
    bs, mb = 16, 64
    rng = np.random.default_rng(50)
    table = rng.permutation(mb + 5)[:mb].astype(np.int32).reshape(1, mb)
    # pools holding the contiguous rows, written by the paged append itself
    kp = synth.canary_cache((w.L, mb + 5, w.Hkv, bs, w.D), w.dtype)
    vp = synth.canary_cache((w.L, mb + 5, w.Hkv, bs, w.D), w.dtype)
    pc = K.PagedKVCache(w.L, mb + 5, w.Hkv, bs, w.D, torch.float32, k=to_dev(kp), v=to_dev(vp))
    bt = torch.from_numpy(table).cuda()
    hist_rows = to_dev(np.ascontiguousarray(w.k_cache[:, :, :, :900]))
    hist_vrows = to_dev(np.ascontiguousarray(w.v_cache[:, :, :, :900]))
    K.paged_append(pc, hist_rows, hist_vrows, [0], bt)
    cc = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, torch.float32, k=to_dev(w.k_cache),
                   v=to_dev(w.v_cache))
    q, k, v = (to_dev(a) for a in w.steps[0])
    o_c = to_host(K.decode_step(cc, q, k, v, w.hist, scale=w.scale))
    o_p = to_host(K.paged_decode_step(pc, q, k, v, w.hist, bt, scale=w.scale))
    assert np.array_equal(bits(o_c), bits(o_p))
