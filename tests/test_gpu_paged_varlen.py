"""Parity of kvc_paged_attn_prefill_varlen (through the C ABI) with the
oracle's paged packed prefill, on the same seeded pools, block tables and
packed rows: pool bytes bit-exact (canaries in blocks no table names, and in
rows past each sequence's end, included), outputs within 1e-4 (fp32) or
2e-2 (bf16) max abs error.  Covers ragged lengths (0, 1, tile edges),
histories on and off block edges, block sizes 1 to 256, GQA, layer0 > 0,
batches over one launch's slice, shared prefix blocks, and bit-identity with
the contiguous-cache prefill on the same rows."""
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


def run_gpu(w, layer0=0, n_layers=None):
    from transformer_kv_cache_amd import kvcache as K
    nl = n_layers or w.q.shape[0]
    cache = K.PagedKVCache(w.L, w.num_blocks, w.Hkv, w.block_size, w.D, torch_dtype(w.dtype),
                           k=to_dev(w.k_pool), v=to_dev(w.v_pool))
    bt = torch.from_numpy(w.block_table).cuda()
    q, k, v = (to_dev(np.ascontiguousarray(a[:nl])) for a in (w.q, w.k, w.v))
    o = K.paged_attn_prefill_varlen(cache, q, k, v, w.cu_seqlens, w.hist, bt, scale=w.scale,
                                    layer0=layer0)
    torch.cuda.synchronize()
    return to_host(o), to_host(cache.k), to_host(cache.v)


def check(w, layer0=0, n_layers=None):
    lens = np.diff(w.cu_seqlens)
    print(f"[paged varlen] {w.name} dtype={w.dtype} L={w.L} B={w.B} Hq={w.Hq} Hkv={w.Hkv} "
          f"D={w.D} bs={w.block_size} lens={lens.tolist()[:8]} hist={w.hist.tolist()[:8]} "
          f"layer0={layer0}", flush=True)
    o, gk, gv = run_gpu(w, layer0, n_layers)
    nl = n_layers or w.q.shape[0]
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    ref = oracle.paged_prefill_varlen(kp, vp, *(np.ascontiguousarray(a[:nl])
                                                for a in (w.q, w.k, w.v)),
                                      w.cu_seqlens, w.hist, w.block_table, w.scale,
                                      layer0=layer0)
    assert np.array_equal(bits(gk), bits(kp)), "K pool bytes differ"
    assert np.array_equal(bits(gv), bits(vp)), "V pool bytes differ"
    of = synth.to_float(o)
    assert np.isfinite(of).all()
    err = float(np.max(np.abs(of.astype(np.float64) - ref))) if o.size else 0.0
    assert err <= TOL[w.dtype], f"max abs err {err}"
    return o


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_varlen_ragged_with_history(dtype):
    w = synth.make_paged_varlen_workload(f"paged_ragged_{dtype}", seed=61, dtype=dtype, L=3, B=7,
                                         Hq=12, Hkv=12, D=64, block_size=16, max_blocks=64,
                                         hist=[0, 1, 63, 64, 65, 300, 880],
                                         lens=[130, 1, 0, 127, 128, 129, 124])
    check(w)


@pytest.mark.parametrize("bs", [1, 8, 64, 256])
def test_paged_varlen_block_sizes(bs):
    w = synth.make_paged_varlen_workload(f"paged_varlen_bs{bs}", seed=62, dtype="f32", L=2, B=3,
                                         Hq=4, Hkv=4, D=64, block_size=bs, max_blocks=512 // bs,
                                         hist=[0, 200, 381], lens=[300, 77, 131])
    check(w)


def test_paged_varlen_gqa_d128_layer0():
    w = synth.make_paged_varlen_workload("paged_varlen_gqa_d128", seed=63, dtype="bf16", L=3,
                                         B=4, Hq=32, Hkv=8, D=128, block_size=32, max_blocks=24,
                                         hist=[10, 0, 200, 511], lens=[70, 257, 31, 250])
    check(w, layer0=1, n_layers=2)


def test_paged_varlen_many_sequences():
    """70 sequences: two launches over batch slices."""
    rng = np.random.default_rng(64)
    w = synth.make_paged_varlen_workload("paged_varlen_many", seed=64, dtype="bf16", L=1, B=70,
                                         Hq=4, Hkv=4, D=64, block_size=16, max_blocks=10,
                                         hist=rng.integers(0, 100, size=70),
                                         lens=rng.integers(0, 60, size=70))
    check(w)


def test_paged_varlen_shared_prefix():
    """Sequences share their first 4 blocks, all of it history (a common
    prompt): reads through shared blocks, writes only into private ones."""
    w = synth.make_paged_varlen_workload("paged_varlen_shared", seed=65, dtype="f32", L=2, B=4,
                                         Hq=8, Hkv=2, D=64, block_size=16, max_blocks=20,
                                         hist=[64, 70, 100, 250], lens=[200, 1, 150, 70],
                                         shared_prefix_blocks=4)
    check(w)


def test_paged_varlen_equals_contiguous_bitwise():
    """The same history laid out contiguously and in shuffled blocks, and the
    same packed rows: bit-identical outputs, and every cache row equal to
    its slot in the pools (the kernel visits the same keys in the same
    order)."""
    from transformer_kv_cache_amd import kvcache as K
    w = synth.make_varlen_workload("contig", seed=66, dtype="bf16", L=2, B=3, Hq=12, Hkv=12,
                                   D=64, Tmax=512, hist=[0, 77, 320], lens=[256, 200, 190])
    cc = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, torch.bfloat16, k=to_dev(w.k_cache),
                   v=to_dev(w.v_cache))
    o_c = to_host(K.attn_prefill_varlen(cc, to_dev(w.q), to_dev(w.k), to_dev(w.v),
                                        w.cu_seqlens, w.hist, scale=w.scale))
    bs, mb = 32, w.Tmax // 32
    kp, vp, table = synth.paged_from_contiguous(w.k_cache, w.v_cache, bs, seed=67)
    nblk = kp.shape[1]
    pc = K.PagedKVCache(w.L, nblk, w.Hkv, bs, w.D, torch.bfloat16, k=to_dev(kp), v=to_dev(vp))
    o_p = to_host(K.paged_attn_prefill_varlen(pc, to_dev(w.q), to_dev(w.k), to_dev(w.v),
                                              w.cu_seqlens, w.hist,
                                              torch.from_numpy(table).cuda(), scale=w.scale))
    assert np.array_equal(bits(o_c), bits(o_p))
    gk, gv, ck, cv = to_host(pc.k), to_host(pc.v), to_host(cc.k), to_host(cc.v)
    for b in range(w.B):
        for j in range(mb):
            assert np.array_equal(bits(gk[:, table[b, j]]), bits(ck[:, b, :, j * bs:(j + 1) * bs]))
            assert np.array_equal(bits(gv[:, table[b, j]]), bits(cv[:, b, :, j * bs:(j + 1) * bs]))
