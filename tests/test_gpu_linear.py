"""kvc_linear_f32 (through the C ABI) against the float64 composition of the
oracle's pinned pieces (oracle/gpt2.py layer_norm and gelu, then a float64
matrix product): y = act(LN?(x) W + b) + res.

Bound per element: recursive fp32 summation of K products errs by at most
K u sum_k |xh_k w_kn| (u = 2^-24), the layer norm adds O(u) relative to xh,
and GELU / the residual add a few ulp of the result; the test allows
4 K u sum_k |xh_k w_kn| + 1e-5 |y| + 1e-6."""
import numpy as np
import pytest
import torch

import oracle.gpt2 as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_kv_cache_amd import kvcache as K
    K.library()  # fail loudly if the HIP library is missing


def run_case(M, K, N, ln, act, res, seed, inplace=False):
    from transformer_kv_cache_amd import kvcache as Kc
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * 2 + 0.5).astype(np.float32)
    w = (0.05 * rng.standard_normal((K, N))).astype(np.float32)
    b = (0.1 * rng.standard_normal(N)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    s = (0.1 * rng.standard_normal(K)).astype(np.float32)
    r = rng.standard_normal((M, N)).astype(np.float32)
    xh = G.layer_norm(x.astype(np.float64), g, s) if ln else x.astype(np.float64)
    ref = xh @ w.astype(np.float64) + b
    if act:
        ref = G.gelu(ref)
    if res:
        ref = ref + r
    bound = 4 * K * 2.0 ** -24 * (np.abs(xh) @ np.abs(w.astype(np.float64))) + 1e-5 * np.abs(ref) + 1e-6
    d = lambda a: torch.from_numpy(a).cuda()
    rt = d(r)
    out = rt if inplace else None
    print(f"[linear] M={M} K={K} N={N} ln={ln} act={act} res={res} inplace={inplace}", flush=True)
    y = Kc.linear(d(x), d(w), bias=d(b), ln=(d(g), d(s)) if ln else None,
                  act="gelu" if act else None, residual=rt if res else None, out=out)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))


@pytest.mark.parametrize("M,K,N", [(1, 768, 2304), (1, 768, 768), (1, 768, 3072), (1, 3072, 768),
                                   (1, 768, 50260), (3, 768, 2304), (8, 768, 3072), (4, 3072, 768),
                                   (1, 4, 4), (2, 12, 20), (8, 1536, 36)])
def test_shapes_plain(M, K, N):
    run_case(M, K, N, ln=False, act=False, res=False, seed=M * 7 + K + N)


@pytest.mark.parametrize("ln,act,res", [(True, False, False), (True, True, False), (False, False, True),
                                        (True, True, True), (False, True, True)])
@pytest.mark.parametrize("M", [1, 5])
def test_fused_epilogues(ln, act, res, M):
    run_case(M, 768, 3072 if act else 768, ln=ln, act=act, res=res, seed=31 + M)


@pytest.mark.parametrize("M", [1, 8])
def test_inplace_residual(M):
    """y written over res (h += x W + b, the residual update of a block)."""
    run_case(M, 768, 768, ln=False, act=False, res=True, seed=41 + M, inplace=True)
