"""Parity of the HIP path (through the C ABI) with the CPU oracle, element by
element on the same seeded inputs: cache bytes bit-exact (NaN canaries in
unused slots included), outputs within 1e-4 (fp32) or 2e-2 (bf16) max abs
error.  Covers the five GPT-2-Small workloads at full size plus ragged and
degenerate shapes."""
import math

import numpy as np
import pytest
import torch

import oracle
from transformer_kv_cache_amd import synth
from gpu_common import TOL, assert_matches, bits, run_gpu, run_oracle, to_dev, to_host, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_kv_cache_amd import kvcache as K
    K.library()  # fail loudly if the HIP library is missing
    return K


def check(w, fused=False):
    print(f"[parity] {w.name} dtype={w.dtype} L={w.L} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
          f"Tmax={w.Tmax} hist={w.hist.tolist()[:8]} fused={fused}", flush=True)
    assert_matches(w, run_gpu(w, fused), run_oracle(w))


# ---------------------------------------------------------------- workloads

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_single_layer_generation(seed):
    """Prompt of 16 then four single-token steps, one layer, Tmax=32."""
    w = synth.single_layer_generation(seed)
    gpu = run_gpu(w)
    assert_matches(w, gpu, run_oracle(w))
    k = gpu[1]
    assert not synth.is_canary(k[:, :, :, :20]).any() and synth.is_canary(k[:, :, :, 20:]).all()


SEEDS = [0, 1, 2]


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("P", [128, 512, 1000, 1023])
def test_decode_12layer(P, seed):
    check(synth.decode_12layer(P, seed=seed))


# One query row per KV head with 128 to 512 rows per call (half a workgroup
# to two per CU on a 256-CU GPU) runs one workgroup per row, streaming
# chunks of 8 keys per lane group (64 keys for fp32 D=64, 32 for fp32 D=128,
# 128 for bf16 D=64, 64 for bf16 D=128) two at a time: every chunk boundary,
# odd and even chunk counts, an empty history, ragged batches and each dtype
# and head size.
ROW_KERNEL_CASES = [
    # (dtype, D, L, H, hist)
    ("f32", 64, 12, 12, [0]),
    ("f32", 64, 12, 12, [1]),
    ("f32", 64, 12, 12, [2]),
    ("f32", 64, 12, 12, [63]),
    ("f32", 64, 12, 12, [64]),
    ("f32", 64, 12, 12, [65]),
    ("f32", 64, 12, 12, [127]),
    ("f32", 64, 12, 12, [128]),
    ("f32", 64, 12, 12, [129]),
    ("f32", 64, 12, 12, [255]),
    ("f32", 64, 12, 12, [383]),
    ("f32", 64, 12, 12, [1022]),
    ("f32", 64, 12, 12, [5, 1000]),
    ("f32", 64, 12, 12, [0, 17, 700]),
    ("bf16", 64, 12, 12, [127]),
    ("bf16", 64, 12, 12, [128]),
    ("bf16", 64, 12, 12, [255]),
    ("bf16", 64, 12, 12, [1023]),
    ("bf16", 64, 12, 12, [3, 513]),
    ("f32", 128, 12, 16, [31]),
    ("f32", 128, 12, 16, [32]),
    ("f32", 128, 12, 16, [33]),
    ("f32", 128, 12, 16, [1000]),
    ("bf16", 128, 8, 16, [63]),
    ("bf16", 128, 8, 16, [64]),
    ("bf16", 128, 8, 16, [129]),
    ("bf16", 128, 8, 16, [1023]),
]


# Two to eight query rows per KV head with 128 to 512 KV heads per call run
# one workgroup per KV head over the whole key range in chunks of 4 keys per
# lane group (64 keys for fp32 D=64 and bf16 D=128, 128 for bf16 D=64): keys
# P + N around the chunk boundaries, an empty history, GQA groups and a
# chunk that is also a GQA group.
ROWS_LOOP_CASES = [
    # (dtype, D, L, Hq, Hkv, N, hist)
    ("f32", 64, 12, 12, 12, 8, [0]),
    ("f32", 64, 12, 12, 12, 8, [55]),
    ("f32", 64, 12, 12, 12, 8, [56]),
    ("f32", 64, 12, 12, 12, 8, [57]),
    ("f32", 64, 12, 12, 12, 8, [120]),
    ("f32", 64, 12, 12, 12, 3, [61, 200]),
    ("bf16", 128, 12, 48, 12, 1, [63]),
    ("bf16", 128, 12, 48, 12, 1, [64]),
    ("bf16", 128, 12, 48, 12, 1, [1000]),
    ("bf16", 128, 12, 24, 12, 3, [5, 300]),
    ("bf16", 64, 12, 48, 12, 1, [127]),
    ("bf16", 64, 12, 48, 12, 1, [128]),
]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("case", range(len(ROWS_LOOP_CASES)))
def test_rows_loop_kernel_shapes(case, fused):
    dtype, D, L, Hq, Hkv, N, hist = ROWS_LOOP_CASES[case]
    w = synth.make_workload(f"rows_loop_{case}", seed=150 + case, dtype=dtype, L=L, B=len(hist),
                            Hq=Hq, Hkv=Hkv, D=D, Tmax=1024, hist=hist, step_lens=(N,))
    check(w, fused=fused)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("case", range(len(ROW_KERNEL_CASES)))
def test_row_kernel_shapes(case, fused):
    dtype, D, L, H, hist = ROW_KERNEL_CASES[case]
    w = synth.make_workload(f"row_kernel_{case}", seed=100 + case, dtype=dtype, L=L, B=len(hist),
                            Hq=H, Hkv=H, D=D, Tmax=1024, hist=hist, step_lens=(1,))
    check(w, fused=fused)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("seed", SEEDS)
def test_chunked_decode(seed, fused):
    check(synth.chunked_decode(1000, 8, seed=seed), fused=fused)


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("S", [256, 1024])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_causal_prefill(S, dtype, seed):
    check(synth.causal_prefill(S, dtype, seed=seed))


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("gqa", [False, True])
def test_batched_decode(gqa, seed):
    check(synth.batched_decode(seed=seed, gqa=gqa))


@pytest.mark.parametrize("seed", SEEDS)
def test_decode_12layer_fused_step(seed):
    """The headline step as the benchmark runs it (kvc_decode_step: one
    launch, in-launch merge) at T = 1024."""
    check(synth.decode_12layer(1023, seed=seed), fused=True)


# ------------------------------------------------------------- edge cases

@pytest.mark.parametrize("S", [1, 2, 31, 63, 64, 65, 127, 128, 129, 200])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_ragged(S, dtype):
    check(synth.make_workload(f"prefill_ragged_S{S}", seed=S, dtype=dtype, L=2, B=2, Hq=3,
                              Hkv=3, D=64, Tmax=256, prefill_len=S))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_long_prompt(dtype, D):
    """A 3000-token prompt (47 key tiles for the last query tile, a ragged
    last tile) with GQA, then two decode steps on top of it."""
    check(synth.make_workload(f"prefill_long_D{D}", seed=400 + D, dtype=dtype, L=1, B=1, Hq=4,
                              Hkv=2, D=D, Tmax=3008, prefill_len=3000, step_lens=(1, 3)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_gqa_and_d128(dtype, D):
    check(synth.make_workload(f"prefill_gqa_D{D}", seed=D, dtype=dtype, L=1, B=2, Hq=8, Hkv=2,
                              D=D, Tmax=200, prefill_len=150, step_lens=(1, 3)))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("scale", [0.0, -0.125, -0.3])
@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_and_negative_scale(dtype, G, scale, fused):
    """Any finite scale: a 200-token prompt (two query tiles, a diagonal
    crossing each) and decode steps of 1 and 3 rows on top, with a zero or a
    negative score scale, through every kernel family (prefill, single-row
    and multi-row decode)."""
    w = synth.make_workload(f"scale_{scale}_G{G}", seed=int(50 + 100 * abs(scale)) + G,
                            dtype=dtype, L=2, B=2, Hq=2 * G, Hkv=2, D=64, Tmax=256,
                            prefill_len=200, step_lens=(1, 3))
    w.scale_value = scale
    check(w, fused=fused)


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 9, 17])
@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_rows_and_groups(N, G, dtype):
    """Every row-tile size (G*N rows per KV head, tiles of up to 8), several
    sequences with different histories including an empty one, and a Tmax
    that is not a multiple of the split size."""
    Tmax = 300
    hist = [0, 37, Tmax - N, 150]
    check(synth.make_workload(f"decode_N{N}_G{G}", seed=N * 10 + G, dtype=dtype, L=2, B=4,
                              Hq=2 * G, Hkv=2, D=64, Tmax=Tmax, hist=hist, step_lens=(N,)))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("G,N", [(2, 1), (4, 1), (1, 2), (1, 3), (2, 2), (4, 2)])
def test_decode_rows_bf16_d128(G, N, fused):
    """A few query rows per KV head with 256-byte bf16 rows (D = 128): GQA
    groups and short chunks, histories on both sides of the 64-key split
    edges, new rows straddling a split edge, an empty history."""
    Tmax = 260
    hist = [0, 63, 64 - N // 2, 127, Tmax - N]
    check(synth.make_workload(f"rows_bf16_G{G}_N{N}", seed=100 + 10 * G + N, dtype="bf16", L=2,
                              B=5, Hq=2 * G, Hkv=2, D=128, Tmax=Tmax, hist=hist, step_lens=(N,)),
          fused=fused)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("N", [2, 4, 6, 7, 8])
def test_decode_rows_f32_split_edges(N, fused):
    """fp32 D = 64 chunks of 2-8 rows around the 64-key split edges."""
    Tmax = 200
    hist = [0, 1, 63 - N, 64, 65, 128 - N // 2, Tmax - N]
    check(synth.make_workload(f"rows_f32_N{N}", seed=200 + N, dtype="f32", L=3, B=7, Hq=3, Hkv=3,
                              D=64, Tmax=Tmax, hist=hist, step_lens=(N,)), fused=fused)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype,D,G,N", [("f32", 64, 1, 1), ("bf16", 64, 1, 1), ("f32", 64, 1, 8),
                                         ("bf16", 128, 4, 1), ("bf16", 128, 2, 3), ("f32", 128, 4, 4)])
def test_long_context_many_splits(dtype, D, G, N, fused):
    """Contexts of several thousand keys: 30-260 split states per query row,
    so the combine merges them over many chunks (every shorter workload fits
    in one), for each split kernel."""
    Tmax = 8192
    hist = [Tmax - N, 4097, 1000]
    check(synth.make_workload(f"long_{dtype}_D{D}_G{G}_N{N}", seed=300 + D + 10 * G + N, dtype=dtype,
                              L=1, B=3, Hq=2 * G, Hkv=2, D=D, Tmax=Tmax, hist=hist,
                              step_lens=(N,)), fused=fused)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_d128(dtype):
    check(synth.make_workload("decode_d128", seed=11, dtype=dtype, L=2, B=3, Hq=8, Hkv=2, D=128,
                              Tmax=520, hist=[519, 0, 260], step_lens=(1,)))


def test_batch_wider_than_one_launch():
    """B = 70 sequences: the host splits the launch over batch slices."""
    rng = np.random.default_rng(3)
    hist = rng.integers(0, 60, size=70)
    check(synth.make_workload("decode_B70", seed=3, dtype="f32", L=1, B=70, Hq=2, Hkv=1, D=64,
                              Tmax=64, hist=hist, step_lens=(2,)))


def test_layer_subset():
    """layer0 > 0: only the named layers' slices are written and read."""
    from transformer_kv_cache_amd import kvcache as K
    w = synth.make_workload("layer_subset", seed=9, dtype="f32", L=4, B=2, Hq=4, Hkv=2, D=64,
                            Tmax=64, hist=[10, 20], step_lens=(3,))
    q, k, v = (np.ascontiguousarray(a[:2]) for a in w.steps[0])
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    oracle.append(kc, vc, k, v, w.hist, layer0=1)
    ref = oracle.attention(q, kc, vc, w.hist, w.scale, layer0=1)
    cache = K.KVCache(4, 2, 2, 64, 64, torch.float32, k=to_dev(w.k_cache), v=to_dev(w.v_cache))
    K.append(cache, to_dev(k), to_dev(v), w.hist, layer0=1)
    out = to_host(K.attn_decode(cache, to_dev(q), w.hist, layer0=1))
    assert np.max(np.abs(out - ref)) <= TOL["f32"]
    assert np.array_equal(bits(to_host(cache.k)), bits(kc))
    assert np.array_equal(bits(to_host(cache.v)), bits(vc))


# ------------------------------------------ fused step (append inside decode)

@pytest.mark.parametrize("seed", [0, 1])
def test_fused_single_layer_generation(seed):
    check(synth.single_layer_generation(seed), fused=True)


@pytest.mark.parametrize("P", [0, 127, 128, 1000, 1023])
def test_fused_decode_12layer(P):
    check(synth.decode_12layer(P, seed=P + 7), fused=True)


def test_fused_chunked_decode():
    check(synth.chunked_decode(1000, 8, seed=3), fused=True)


@pytest.mark.parametrize("gqa", [False, True])
def test_fused_batched_decode(gqa):
    check(synth.batched_decode(seed=6, gqa=gqa), fused=True)


@pytest.mark.parametrize("fused", [False, True])
def test_batched_decode_tp8_shard(fused):
    """One GPU's share of the GQA workload under 8-way tensor parallelism
    (one KV head, four query heads per layer), the shape the benchmark
    times for it."""
    check(synth.batched_decode(seed=3, gqa=True, tp=8), fused=fused)


@pytest.mark.parametrize("N", [1, 3, 8, 9, 17])
@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_rows_and_groups(N, G, dtype):
    """New rows that straddle a split boundary, several row tiles (only tile 0
    writes the new rows), empty and full histories."""
    Tmax = 300
    hist = [0, 128 - N // 2, Tmax - N, 255]
    check(synth.make_workload(f"fused_N{N}_G{G}", seed=N * 10 + G + 1, dtype=dtype, L=2, B=4,
                              Hq=2 * G, Hkv=2, D=64, Tmax=Tmax, hist=hist, step_lens=(N,)),
          fused=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_d128_and_wide_batch(dtype):
    check(synth.make_workload("fused_d128", seed=12, dtype=dtype, L=2, B=3, Hq=8, Hkv=2, D=128,
                              Tmax=520, hist=[518, 0, 260], step_lens=(2,)), fused=True)
    rng = np.random.default_rng(4)
    check(synth.make_workload("fused_B70", seed=4, dtype=dtype, L=1, B=70, Hq=2, Hkv=1, D=64,
                              Tmax=96, hist=rng.integers(0, 90, size=70), step_lens=(3, 1)),
          fused=True)


# ------------------------------------------------------------- invariants

def test_cached_decode_equals_recompute():
    """Prefill of P+N rows, last N outputs, against prefill of P then
    append + decode of N, on the GPU (within tolerance: different kernels)."""
    from transformer_kv_cache_amd import kvcache as K
    P, N, L, H, D, T = 300, 8, 2, 4, 64, 512
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((L, 1, H, P + N, D), dtype=np.float32) for _ in range(3))
    c1 = K.KVCache(L, 1, H, T, D, torch.float32, k=to_dev(synth.canary_cache((L, 1, H, T, D), "f32")),
                   v=to_dev(synth.canary_cache((L, 1, H, T, D), "f32")))
    full = to_host(K.attn_prefill(c1, to_dev(q), to_dev(k), to_dev(v)))
    c2 = K.KVCache(L, 1, H, T, D, torch.float32, k=to_dev(synth.canary_cache((L, 1, H, T, D), "f32")),
                   v=to_dev(synth.canary_cache((L, 1, H, T, D), "f32")))
    head = [to_dev(np.ascontiguousarray(a[:, :, :, :P])) for a in (q, k, v)]
    tail = [to_dev(np.ascontiguousarray(a[:, :, :, P:])) for a in (q, k, v)]
    K.attn_prefill(c2, *head)
    K.append(c2, tail[1], tail[2], [P])
    inc = to_host(K.attn_decode(c2, tail[0], [P]))
    assert np.max(np.abs(full[:, :, :, P:] - inc)) <= TOL["f32"]
    assert np.array_equal(bits(to_host(c1.k)), bits(to_host(c2.k)))


def test_permutation_property_on_gpu():
    """Jointly permuting every cached (K_j, V_j) pair leaves single-row decode
    unchanged and changes chunked decode."""
    from transformer_kv_cache_amd import kvcache as K
    P, L, H, D = 200, 1, 2, 64
    rng = np.random.default_rng(22)
    for N, same in ((1, True), (8, False)):
        T = P + N
        w = synth.make_workload("perm", seed=N, dtype="f32", L=L, B=1, Hq=H, Hkv=H, D=D, Tmax=T,
                                hist=[P], step_lens=(N,))
        q, k, v = w.steps[0]
        cache = K.KVCache(L, 1, H, T, D, torch.float32, k=to_dev(w.k_cache), v=to_dev(w.v_cache))
        K.append(cache, to_dev(k), to_dev(v), [P])
        ref = to_host(K.attn_decode(cache, to_dev(q), [P]))
        perm = torch.from_numpy(rng.permutation(T)).cuda()
        pc = K.KVCache(L, 1, H, T, D, torch.float32, k=cache.k[:, :, :, perm].contiguous(),
                       v=cache.v[:, :, :, perm].contiguous())
        got = to_host(K.attn_decode(pc, to_dev(q), [P]))
        diff = float(np.max(np.abs(got - ref)))
        assert (diff <= TOL["f32"]) if same else (diff > 1e-2), (N, diff)


@pytest.mark.parametrize("case", ["mha_fp32", "mha_fp32_4layers", "gqa_bf16", "chunked"])
def test_split_then_combine_equals_one_call(case):
    """kvc_decode_split + kvc_decode_combine give the same cache bytes as the
    one call (kvc_decode_step / kvc_attn_decode) and match the oracle.  The
    outputs are the same bytes where the one call runs the split kernel too
    (the batched GQA workload: 768 KV heads, and 4 of the 12 layers); where
    its KV heads about fill the chip (the 12-layer single-row and chunked
    steps: 144) it runs one workgroup per KV head over the whole key range
    instead, which sums the same terms in another order, so there the
    outputs agree to fp32 rounding (1e-5, a tenth of the oracle bound)."""
    from transformer_kv_cache_amd import kvcache as K
    w = {"mha_fp32": lambda: synth.decode_12layer(1000, seed=31),
         "mha_fp32_4layers": lambda: synth.decode_12layer(1000, seed=34),
         "gqa_bf16": lambda: synth.batched_decode(seed=32, gqa=True),
         "chunked": lambda: synth.chunked_decode(1000, 8, seed=33)}[case]()
    nl = 4 if case == "mha_fp32_4layers" else w.L
    q, k, v = (np.ascontiguousarray(a[:nl]) for a in w.steps[0])
    ref_out = run_oracle(w)[0][0][:nl]
    dt = torch_dtype(w.dtype)
    outs = {}
    for mode in ("one_call", "two_phases", "two_phases_unfused"):
        cache = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, dt, k=to_dev(w.k_cache), v=to_dev(w.v_cache))
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        if mode == "one_call":
            o = K.decode_step(cache, qd, kd, vd, w.hist)
        elif mode == "two_phases":
            o = K.decode_split(cache, qd, w.hist, kd, vd)
            K.decode_combine(cache, qd, w.hist, kd, vd, out=o)
        else:
            K.append(cache, kd, vd, w.hist)
            o = K.decode_split(cache, qd, w.hist)
            K.decode_combine(cache, qd, w.hist, out=o)
        outs[mode] = (to_host(o), to_host(cache.k), to_host(cache.v))
    for mode in ("two_phases", "two_phases_unfused"):
        assert np.array_equal(bits(outs[mode][1]), bits(outs["one_call"][1])), mode
        assert np.array_equal(bits(outs[mode][2]), bits(outs["one_call"][2])), mode
    assert np.array_equal(bits(outs["two_phases"][0]), bits(outs["two_phases_unfused"][0]))
    if case in ("mha_fp32", "chunked"):
        d = np.max(np.abs(outs["two_phases"][0] - outs["one_call"][0]))
        assert d <= 1e-5, d
    else:
        assert np.array_equal(bits(outs["two_phases"][0]), bits(outs["one_call"][0]))
    for mode in outs:
        assert np.max(np.abs(synth.to_float(outs[mode][0]) - ref_out)) <= TOL[w.dtype], mode


@pytest.mark.parametrize("n_layers", [12, 4, 1])
def test_repeated_calls_reuse_workspace_bitwise(n_layers):
    """Repeated calls on one workspace give bit-identical outputs, whatever
    the scratch part holds (NaN bit patterns), and leave its arrival
    counters (the first 8 bytes per query row, rounded up to 256) zero after
    every call: the one-workgroup-per-row kernel (12 layers), the in-launch
    merge (4 and 1 layers) and the two-launch form alike.  The two-launch
    form gives the one call's bytes where both run the split kernel, and
    agrees to fp32 rounding (1e-5) with the one-workgroup-per-row kernel."""
    from transformer_kv_cache_amd import kvcache as K
    w = synth.decode_12layer(1000, seed=4)
    q, k, v = w.steps[0]
    cache = K.KVCache(12, 1, 12, 1024, 64, torch.float32, k=to_dev(w.k_cache), v=to_dev(w.v_cache))
    K.append(cache, to_dev(k), to_dev(v), w.hist)
    ws = K.new_decode_workspace(cache, n_layers, 12, 1)
    ctr = (8 * n_layers * 12 + 255) // 256 * 256
    qd = to_dev(np.ascontiguousarray(q[:n_layers]))
    one, two = [], []
    for scribble in (False, True):
        if scribble:
            ws[ctr:].fill_(0xFF)  # NaN bit patterns everywhere in the scratch
        for _ in range(3):
            one.append(to_host(K.attn_decode(cache, qd, w.hist, workspace=ws)))
            torch.cuda.synchronize()
            assert not ws[:ctr].any(), "arrival counters not back at zero"
        o = K.decode_split(cache, qd, w.hist, workspace=ws)
        K.decode_combine(cache, qd, w.hist, out=o, workspace=ws)
        two.append(to_host(o))
        torch.cuda.synchronize()
        assert not ws[:ctr].any()
    for o in one[1:]:
        assert np.array_equal(bits(o), bits(one[0]))
    for o in two[1:]:
        assert np.array_equal(bits(o), bits(two[0]))
    if n_layers == 12:
        assert np.max(np.abs(one[0] - two[0])) <= 1e-5
    else:
        assert np.array_equal(bits(one[0]), bits(two[0]))
    assert np.max(np.abs(one[0] - run_oracle(w)[0][0][:n_layers])) <= TOL["f32"]


@pytest.mark.parametrize("n_layers", [4, 12])
def test_in_launch_merge_many_inputs_bitwise(n_layers):
    """Back to back on 48 different query sets: the one-launch merge (4
    layers: 48 rows, so many merging workgroups read split states other
    workgroups of the same launch have just stored) gives bit for bit the
    two-launch form's output every time; the one-workgroup-per-row kernel
    (12 layers) agrees with it to fp32 rounding every time.  The first set is
    also checked against the oracle."""
    from transformer_kv_cache_amd import kvcache as K
    w = synth.decode_12layer(1000, seed=41)
    q0, k, v = w.steps[0]
    cache = K.KVCache(12, 1, 12, 1024, 64, torch.float32, k=to_dev(w.k_cache), v=to_dev(w.v_cache))
    K.append(cache, to_dev(k), to_dev(v), w.hist)
    ws_one = K.new_decode_workspace(cache, n_layers, 12, 1)
    ws_two = K.new_decode_workspace(cache, n_layers, 12, 1)
    rng = np.random.default_rng(41)
    qs = [q0] + [rng.standard_normal(q0.shape).astype(np.float32) for _ in range(47)]
    one, two = [], []
    for q in qs:
        qd = to_dev(np.ascontiguousarray(q[:n_layers]))
        one.append(K.attn_decode(cache, qd, w.hist, workspace=ws_one))
        o = K.decode_split(cache, qd, w.hist, workspace=ws_two)
        K.decode_combine(cache, qd, w.hist, out=o, workspace=ws_two)
        two.append(o)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(one, two)):
        a, b = to_host(a), to_host(b)
        if n_layers == 12:
            assert np.max(np.abs(a - b)) <= 1e-5, f"query set {i}"
        else:
            assert np.array_equal(bits(a), bits(b)), f"query set {i}"
    assert np.max(np.abs(to_host(one[0]) - run_oracle(w)[0][0][:n_layers])) <= TOL["f32"]


def test_capacity_error_leaves_cache_untouched():
    from transformer_kv_cache_amd import kvcache as K
    w = synth.decode_12layer(1023, seed=1)
    cache = K.KVCache(12, 1, 12, 1024, 64, torch.float32, k=to_dev(w.k_cache), v=to_dev(w.v_cache))
    before = to_host(cache.k)
    kn = torch.zeros((12, 1, 12, 2, 64), device="cuda")
    with pytest.raises(K.KVCacheError) as e:
        K.append(cache, kn, kn, [1023])
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(cache.k)), bits(before))


def test_cache_allocation_matches_formula():
    """torch.cuda.memory_allocated grows by exactly the formula's bytes."""
    import gc
    from transformer_kv_cache_amd import kvcache as K
    gc.collect()
    gc.disable()  # no collection of earlier tests' tensors between the readings
    try:
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        cache = K.KVCache(12, 1, 12, 1024, 64, torch.float32)
        grown = torch.cuda.memory_allocated() - before
    finally:
        gc.enable()
    assert cache.nbytes == 75_497_472 == grown
    del cache


@pytest.mark.parametrize("case", ["mha_fp32", "gqa_bf16_chunked"])
def test_graph_replays_match_eager(case):
    """The fused step captured in a HIP graph (as a serving loop or the
    benchmark runs it): every replay, with unrelated eager work and
    synchronisations between replays, gives the eager call's output and
    cache bytes bit for bit."""
    from transformer_kv_cache_amd import kvcache as K
    if case == "mha_fp32":
        w = synth.decode_12layer(1023, seed=8)
    else:
        w = synth.make_workload("graph_gqa", seed=9, dtype="bf16", L=2, B=3, Hq=8, Hkv=2, D=128,
                                Tmax=256, hist=[0, 100, 247], step_lens=(8,))
    q, k, v = (to_dev(a) for a in w.steps[0])
    dt = torch_dtype(w.dtype)
    N = q.shape[3]
    c_eager = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, dt, k=to_dev(w.k_cache), v=to_dev(w.v_cache))
    ref = to_host(K.decode_step(c_eager, q, k, v, w.hist, scale=w.scale))
    ref_k, ref_v = to_host(c_eager.k), to_host(c_eager.v)
    cache = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, dt, k=to_dev(w.k_cache), v=to_dev(w.v_cache))
    ws = K.new_decode_workspace(cache, w.L, w.Hq, N)
    out = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            K.decode_step(cache, q, k, v, w.hist, scale=w.scale, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    other = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, dt, k=to_dev(w.k_cache), v=to_dev(w.v_cache))
    for rep in range(4):
        print(f"[graph] {case} replay {rep}", flush=True)
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(to_host(out)), bits(ref)), f"replay {rep}"
        assert np.array_equal(bits(to_host(cache.k)), bits(ref_k))
        assert np.array_equal(bits(to_host(cache.v)), bits(ref_v))
        # unrelated eager work on the same workspace and another cache, and
        # garbage in its scratch part (its arrival counters, the first 8
        # bytes per query row rounded up to 256, must stay zero)
        K.decode_step(other, q, k, v, w.hist, scale=w.scale, workspace=ws)
        ws[(8 * w.L * w.B * w.Hq * N + 255) // 256 * 256:].fill_(0x7F)
        torch.cuda.synchronize()
