"""A seeded sweep of decode shapes through the C ABI against the CPU oracle:
head dims 64 and 128, fp32 and bf16, one to eight KV heads with GQA groups
of 1 to 8, chunks of 1 to 13 new rows, ragged histories up to the cache's
end, contiguous and paged caches (block sizes 1 to 64), the fused step and
append + attention.  The shapes reach every split kernel (one row per KV
head, the multi-row vector kernel, the matrix-core kernel) and the edges of
their splits; each case is small enough for the oracle to finish at once.
Outputs within the dtype tolerance, cache bytes bit-exact."""
import numpy as np
import pytest
import torch

from transformer_kv_cache_amd import synth
from gpu_common import TOL, assert_matches, bits, run_gpu, run_oracle, run_paged, run_paged_oracle

pytestmark = pytest.mark.gpu


def _cases(n=48, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ("f32", "bf16")[i % 2]
        D = (64, 128)[(i // 2) % 2]
        G = int(rng.choice([1, 2, 3, 4, 8]))
        N = int(rng.choice([1, 1, 2, 3, 5, 8, 13]))
        Hkv = int(rng.integers(1, 4))
        B = int(rng.integers(1, 6))
        L = int(rng.integers(1, 3))
        Tmax = int(rng.integers(N + 1, 700))
        hist = rng.integers(0, Tmax - N + 1, size=B)
        hist[rng.integers(0, B)] = Tmax - N  # one sequence fills the cache
        paged = bool(i % 3 == 2)
        bs = int(rng.choice([1, 4, 16, 64]))
        fused = bool(rng.integers(0, 2))
        out.append(dict(i=i, dtype=dtype, D=D, G=G, N=N, Hkv=Hkv, B=B, L=L, Tmax=Tmax,
                        hist=[int(h) for h in hist], paged=paged, bs=bs, fused=fused))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"c{c['i']}")
def test_decode_sweep(case):
    c = case
    print(f"[sweep] {c}", flush=True)
    if not c["paged"]:
        w = synth.make_workload(f"sweep{c['i']}", seed=1000 + c["i"], dtype=c["dtype"], L=c["L"],
                                B=c["B"], Hq=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"],
                                Tmax=c["Tmax"], hist=c["hist"], step_lens=(c["N"],))
        assert_matches(w, run_gpu(w, c["fused"]), run_oracle(w))
        return
    bs = c["bs"]
    max_blocks = (c["Tmax"] + bs - 1) // bs
    w = synth.make_paged_workload(f"sweep{c['i']}", seed=1000 + c["i"], dtype=c["dtype"],
                                  L=c["L"], B=c["B"], Hq=c["G"] * c["Hkv"], Hkv=c["Hkv"],
                                  D=c["D"], block_size=bs, max_blocks=max_blocks,
                                  hist=[min(h, max_blocks * bs - c["N"]) for h in c["hist"]],
                                  step_lens=(c["N"],))
    g_outs, gk, gv = run_paged(w, c["fused"])
    r_outs, rk, rv = run_paged_oracle(w)
    assert np.array_equal(bits(gk), bits(rk)), "K pool bytes differ"
    assert np.array_equal(bits(gv), bits(rv)), "V pool bytes differ"
    for g, r in zip(g_outs, r_outs):
        gf = synth.to_float(g)
        assert np.isfinite(gf).all()
        assert float(np.max(np.abs(gf.astype(np.float64) - r))) <= TOL[w.dtype]
