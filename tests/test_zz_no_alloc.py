"""kvc_decode_step_noalloc, the decode step that allocates nothing (its
split states and arrival counters live in the library's per-GPU scratch),
through the C ABI against kvc_decode_step with a caller workspace: outputs
and cache bytes bit for bit, and the oracle within the dtype tolerance, over
calls in a row on one GPU -- each later one smaller than the one before, of
another geometry, and taking another kernel path (in-launch merge, the
multi-row kernel, the two-launch merge), so each finds the scratch as the
previous call left it."""
import numpy as np
import pytest
import torch

from transformer_kv_cache_amd import synth
from gpu_common import TOL, bits, run_oracle, to_dev, to_host, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_kv_cache_amd import kvcache as K
    K.library()  # fail loudly if the HIP library is missing


def _pair(w):
    """One step of `w` through both entry points; returns both results and
    the oracle's output."""
    from transformer_kv_cache_amd import kvcache as K
    q, k, v = (to_dev(a) for a in w.steps[0])
    dt = torch_dtype(w.dtype)
    N = q.shape[3]
    res = []
    for noalloc in (False, True):
        cache = K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, dt, k=to_dev(w.k_cache), v=to_dev(w.v_cache))
        out = torch.full_like(q, float("nan"))
        if noalloc:
            K.decode_step_noalloc(cache, q, k, v, w.hist, out, scale=w.scale)
        else:
            ws = K.new_decode_workspace(cache, w.L, w.Hq, N)
            K.decode_step(cache, q, k, v, w.hist, scale=w.scale, out=out, workspace=ws)
        torch.cuda.synchronize()
        res.append((to_host(out), to_host(cache.k), to_host(cache.v)))
    return res, run_oracle(w)[0][0]


SEQUENCE = [
    # 12-layer fp32 step at T=1024: one launch, in-launch merge (1,152 workgroups)
    ("mha_fp32_12layer_T1024", lambda: synth.decode_12layer(1023, seed=71)),
    # smaller, ragged, an empty history: in-launch merge on another geometry
    ("mha_fp32_small", lambda: synth.make_workload("na_small", seed=72, dtype="f32", L=2, B=3, Hq=4,
                                                   Hkv=4, D=64, Tmax=300, hist=[0, 37, 299],
                                                   step_lens=(1,))),
    # GQA bf16 D=128 (multi-row kernel + combine), smaller still
    ("gqa_bf16_small", lambda: synth.make_workload("na_gqa", seed=73, dtype="bf16", L=1, B=2, Hq=8,
                                                   Hkv=2, D=128, Tmax=200, hist=[150, 3],
                                                   step_lens=(1,))),
    # tiny: a single row with a single split
    ("mha_fp32_tiny", lambda: synth.make_workload("na_tiny", seed=74, dtype="f32", L=1, B=1, Hq=1,
                                                  Hkv=1, D=64, Tmax=64, hist=[40], step_lens=(1,))),
]


@pytest.mark.parametrize("order", ["descending", "again"])
def test_noalloc_matches_workspace_entry_point(order):
    """The sequence of calls, each smaller than the previous; run twice so
    the second pass starts from the scratch the first left behind."""
    for name, make in SEQUENCE:
        w = make()
        print(f"[noalloc] {order} {name} L={w.L} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
              f"Tmax={w.Tmax} hist={w.hist.tolist()}", flush=True)
        (ref, got), oracle_out = _pair(w)
        assert np.array_equal(bits(got[0]), bits(ref[0])), name
        assert np.array_equal(bits(got[1]), bits(ref[1])), name
        assert np.array_equal(bits(got[2]), bits(ref[2])), name
        err = float(np.max(np.abs(synth.to_float(got[0]) - oracle_out)))
        assert err <= TOL[w.dtype], (name, err)


def test_noalloc_large_batch_two_launch_merge_then_small():
    """A batched bf16 step whose grid is too large for the in-launch merge
    (split pass + combine pass in the scratch), then a small in-launch one."""
    for name, make in (("batched_mha_bf16", lambda: synth.batched_decode(seed=75, gqa=False)),
                       ("mha_fp32_small", SEQUENCE[1][1])):
        w = make()
        print(f"[noalloc] {name} B={w.B} hist={w.hist.tolist()}", flush=True)
        (ref, got), oracle_out = _pair(w)
        assert np.array_equal(bits(got[0]), bits(ref[0])), name
        assert np.array_equal(bits(got[1]), bits(ref[1])), name
        err = float(np.max(np.abs(synth.to_float(got[0]) - oracle_out)))
        assert err <= TOL[w.dtype], (name, err)
