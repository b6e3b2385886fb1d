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
    y = Kc.linear(d(x), d(np.ascontiguousarray(w.T)), bias=d(b), ln=(d(g), d(s)) if ln else None,
                  act="gelu" if act else None, residual=rt if res else None, out=out)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))


@pytest.mark.parametrize("M,K,N", [(1, 768, 2304), (1, 768, 768), (1, 768, 3072), (1, 3072, 768),
                                   (1, 768, 50257), (3, 768, 2304), (8, 768, 3072), (4, 3072, 768),
                                   (1, 4, 4), (2, 12, 20), (8, 1536, 36), (1, 12288, 5),
                                   (2, 1540, 7), (5, 260, 9)])
def test_shapes_plain(M, K, N):
    run_case(M, K, N, ln=False, act=False, res=False, seed=M * 7 + K + N)


@pytest.mark.parametrize("ln,act,res", [(True, False, False), (True, True, False), (False, False, True),
                                        (True, True, True), (False, True, True)])
@pytest.mark.parametrize("M", [1, 5])
def test_fused_epilogues(ln, act, res, M):
    run_case(M, 768, 3072 if act else 768, ln=ln, act=act, res=res, seed=31 + M)


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_attention_layouts(M):
    """kvc_linear_f32 writing q, k, v as [3, H, M, D] (with the layer norm)
    and reading the attention output head-major [H, M, D] (with the
    residual), against the row-major reference converted on the host."""
    from transformer_kv_cache_amd import kvcache as Kc
    H, D = 12, 64
    K = N = H * D
    rng = np.random.default_rng(100 + M)
    x = (rng.standard_normal((M, K)) * 2 + 0.5).astype(np.float32)
    w = (0.05 * rng.standard_normal((K, 3 * N))).astype(np.float32)
    b = (0.1 * rng.standard_normal(3 * N)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    sh = (0.1 * rng.standard_normal(K)).astype(np.float32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    xh = G.layer_norm(x.astype(np.float64), g, sh)
    ref = xh @ w.astype(np.float64) + b
    bound = 4 * K * 2.0 ** -24 * (np.abs(xh) @ np.abs(w.astype(np.float64))) + 1e-5 * np.abs(ref) + 1e-6
    print(f"[linear layouts] M={M}", flush=True)
    y = Kc.linear(d(x), d(w.T), bias=d(b), ln=(d(g), d(sh)), qkv_heads=H)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (3, H, M, D)
    got = y.cpu().numpy().astype(np.float64).transpose(2, 0, 1, 3).reshape(M, 3 * N)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))
    # head-major input with an in-place residual
    a = rng.standard_normal((M, K)).astype(np.float32)
    wo = (0.05 * rng.standard_normal((K, N))).astype(np.float32)
    bo = (0.1 * rng.standard_normal(N)).astype(np.float32)
    r = rng.standard_normal((M, N)).astype(np.float32)
    ref = a.astype(np.float64) @ wo.astype(np.float64) + bo + r
    bound = 4 * K * 2.0 ** -24 * (np.abs(a.astype(np.float64)) @ np.abs(wo.astype(np.float64))) \
        + 1e-5 * np.abs(ref) + 1e-6
    rt = d(r)
    Kc.linear(d(a.reshape(M, H, D).transpose(1, 0, 2)), d(wo.T), bias=d(bo), residual=rt, out=rt, a_heads=H)
    torch.cuda.synchronize()
    got = rt.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))


@pytest.mark.parametrize("M", [1, 8])
def test_inplace_residual(M):
    """y written over res (h += x W + b, the residual update of a block)."""
    run_case(M, 768, 768, ln=False, act=False, res=True, seed=41 + M, inplace=True)


# ---- the prompt-sized product kvc_gemm_f32 and kvc_layernorm_f32 ---------------

def run_gemm(M, K, N, act, res, seed, a_heads=0, qkv_heads=0, inplace=False, bias=True):
    """kvc_gemm_f32 against a float64 product of the same fp32 inputs, with
    the oracle's GELU; a given head-major or the output in the attention
    layout, converted on the host for the reference.  Bound as for the
    decode-time kernel: 4 K u sum_k |a_k w_kn| + 1e-5 |y| + 1e-6."""
    from transformer_kv_cache_amd import kvcache as Kc
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal((M, K)) * 1.5 + 0.2).astype(np.float32)
    w = (0.05 * rng.standard_normal((K, N))).astype(np.float32)
    b = (0.1 * rng.standard_normal(N)).astype(np.float32)
    r = rng.standard_normal((M, N)).astype(np.float32)
    ref = a.astype(np.float64) @ w.astype(np.float64) + (b if bias else 0.0)
    if act:
        ref = G.gelu(ref)
    if res:
        ref = ref + r
    bound = 4 * K * 2.0 ** -24 * (np.abs(a.astype(np.float64)) @ np.abs(w.astype(np.float64))) \
        + 1e-5 * np.abs(ref) + 1e-6
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    a_dev = d(a.reshape(M, a_heads, K // a_heads).transpose(1, 0, 2)) if a_heads else d(a)
    rt = d(r)
    print(f"[gemm] M={M} K={K} N={N} act={act} res={res} a_heads={a_heads} qkv_heads={qkv_heads}",
          flush=True)
    y = Kc.gemm(a_dev, d(w.T), bias=d(b) if bias else None, act="gelu" if act else None,
                residual=rt if res else None, out=rt if inplace else None, a_heads=a_heads,
                qkv_heads=qkv_heads)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    if qkv_heads:
        dh = N // (3 * qkv_heads)
        assert got.shape == (3, qkv_heads, M, dh)
        got = got.transpose(2, 0, 1, 3).reshape(M, N)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))


@pytest.mark.parametrize("M,K,N", [(1000, 768, 2304), (1000, 768, 768), (1000, 768, 3072),
                                   (1000, 3072, 768), (64, 768, 768), (1, 64, 4), (65, 128, 100),
                                   (130, 192, 68), (9, 768, 50257), (3, 64, 6), (200, 320, 36)])
def test_gemm_shapes(M, K, N):
    """GPT-2 Small's prompt products at context 1000, tile edges and ragged
    rows / columns (M and N not multiples of 64), the output projection's
    vocabulary width (an odd N), a K of 5 tiles."""
    run_gemm(M, K, N, act=False, res=False, seed=M + K + N)


@pytest.mark.parametrize("act,res,bias", [(True, False, True), (False, True, True), (True, True, True),
                                          (False, False, False)])
def test_gemm_epilogues(act, res, bias):
    run_gemm(200, 768, 3072 if act else 768, act=act, res=res, seed=11 + act + 2 * res, bias=bias)


@pytest.mark.parametrize("M,K,N,act,res,qkv", [(512, 3072, 768, False, True, 0), (128, 3072, 768, False, False, 0),
                                               (128, 768, 2304, False, False, 12), (1, 768, 4, True, False, 0),
                                               (200, 768, 768, True, True, 0), (65, 640, 100, False, True, 0)])
def test_gemm_split_k(M, K, N, act, res, qkv):
    """Products with few output tiles split K over several workgroups per
    tile (the last sums the partials): against the float64 product, bitwise
    repeatable over calls, with the workspace's counters back at zero, and
    the same within the bound as the unsplit product."""
    from transformer_kv_cache_amd import kvcache as Kc
    need = int(Kc.library().kvc_gemm_workspace_bytes(M, K, N))
    rng = np.random.default_rng(M + K + N)
    a = (rng.standard_normal((M, K)) * 1.5).astype(np.float32)
    w = (0.05 * rng.standard_normal((K, N))).astype(np.float32)
    b = (0.1 * rng.standard_normal(N)).astype(np.float32)
    r = rng.standard_normal((M, N)).astype(np.float32)
    ref = a.astype(np.float64) @ w.astype(np.float64) + b
    if act:
        ref = G.gelu(ref)
    if res:
        ref = ref + r
    bound = 4 * K * 2.0 ** -24 * (np.abs(a.astype(np.float64)) @ np.abs(w.astype(np.float64))) \
        + 1e-5 * np.abs(ref) + 1e-6
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    ws = Kc._aligned_workspace(max(need, 256), "cuda")
    print(f"[gemm split] M={M} K={K} N={N} workspace={need}", flush=True)
    outs = []
    for rep in range(2):
        y = Kc.gemm(d(a), d(w.T), bias=d(b), act="gelu" if act else None, residual=d(r) if res else None,
                    qkv_heads=qkv, workspace=ws)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        if qkv:
            got = got.transpose(2, 0, 1, 3).reshape(M, N)
        outs.append(got)
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.all(np.abs(outs[0].astype(np.float64) - ref) <= bound)
    assert not ws[:2048].any().item(), "arrival counters left nonzero"
    y1 = Kc.gemm(d(a), d(w.T), bias=d(b), act="gelu" if act else None, residual=d(r) if res else None,
                 qkv_heads=qkv, workspace=None).cpu().numpy()
    if qkv:
        y1 = y1.transpose(2, 0, 1, 3).reshape(M, N)
    assert np.all(np.abs(y1.astype(np.float64) - ref) <= bound)
    if M <= 128:
        assert need > 0  # these shapes do split on this GPU


def test_gemm_inplace_residual():
    """y written over res (h += a W + b)."""
    run_gemm(300, 3072, 768, act=False, res=True, seed=13, inplace=True)


@pytest.mark.parametrize("M", [1, 100, 1000])
def test_gemm_attention_layouts(M):
    """QKV product written as [3, H, M, D] (q, k, v for the attention calls)
    and the output projection reading the attention output [H, M, D]."""
    run_gemm(M, 768, 2304, act=False, res=False, seed=17 + M, qkv_heads=12)
    run_gemm(M, 768, 768, act=False, res=True, seed=19 + M, a_heads=12)


@pytest.mark.parametrize("M,K", [(1, 768), (1000, 768), (7, 128), (5, 3072), (3, 4), (2, 4096)])
def test_layernorm(M, K):
    """kvc_layernorm_f32 against the oracle's float64 layer norm of the same
    fp32 rows: within 1e-5 |y| + 1e-5 (the fp32 mean, variance and rsqrt)."""
    from transformer_kv_cache_amd import kvcache as Kc
    rng = np.random.default_rng(M * 31 + K)
    x = (rng.standard_normal((M, K)) * 3 + 1.5).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    b = (0.1 * rng.standard_normal(K)).astype(np.float32)
    ref = G.layer_norm(x.astype(np.float64), g, b)
    d = lambda a: torch.from_numpy(a).cuda()
    print(f"[layernorm] M={M} K={K}", flush=True)
    xd = d(x)
    y = Kc.layer_norm(xd, d(g), d(b))
    Kc.layer_norm(xd, d(g), d(b), out=xd)  # in place
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref) + 1e-5), float(np.max(np.abs(got - ref)))
    assert np.array_equal(xd.cpu().numpy(), y.cpu().numpy())


@pytest.mark.parametrize("d", [768, 12])
def test_embed(d):
    """kvc_embed_f32: row i = wte[ids[i]] + wpe[p0 + i], bit for bit the fp32
    sum numpy forms; p0 from the host or from a device int32; ids or
    positions out of range give NaN rows."""
    from transformer_kv_cache_amd import kvcache as Kc
    rng = np.random.default_rng(d)
    V, T = 50, 20
    wte = rng.standard_normal((V, d)).astype(np.float32)
    wpe = rng.standard_normal((T, d)).astype(np.float32)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tw, tp = dv(wte), dv(wpe)
    print(f"[embed] d={d}", flush=True)
    ids = np.array([3, 0, 49, 7], np.int64)
    y = Kc.embed(tw, tp, dv(ids), pos0=5).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), (wte[ids] + wpe[5:9]).view(np.uint32))
    y = Kc.embed(tw, tp, dv(ids), pos=torch.tensor([9], dtype=torch.int32, device="cuda")).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), (wte[ids] + wpe[9:13]).view(np.uint32))
    bad = np.array([50, -1, 2], np.int64)
    y = Kc.embed(tw, tp, dv(bad), pos0=0).cpu().numpy()
    assert np.isnan(y[:2]).all() and np.array_equal(y[2], wte[2] + wpe[2])
    y = Kc.embed(tw, tp, dv(ids), pos=torch.tensor([18], dtype=torch.int32, device="cuda")).cpu().numpy()
    assert np.array_equal(y[:2], wte[ids[:2]] + wpe[18:20]) and np.isnan(y[2:]).all()


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023, 4096, 8193, 50257, 300001])
def test_argmax(n):
    """kvc_argmax_f32 equals numpy's argmax (the first maximum; a NaN wins,
    the first NaN): random rows, planted ties at both ends, an all -inf row,
    NaN at the start, middle and end; and the token-history bookkeeping,
    which stops writing past the capacity but still counts."""
    from transformer_kv_cache_amd import kvcache as Kc
    rng = np.random.default_rng(n)
    print(f"[argmax] n={n}", flush=True)
    cases = [rng.standard_normal(n).astype(np.float32)]
    t = rng.standard_normal(n).astype(np.float32)
    t[n // 3] = t[-1] = t[n // 2] = 9.0           # ties: the first of them
    cases.append(t)
    cases.append(np.full(n, -np.inf, np.float32))
    for where in (0, n // 2, n - 1):
        t = rng.standard_normal(n).astype(np.float32)
        t[where] = np.nan
        t[(where + n // 4) % n] = np.inf
        cases.append(t)
    t = rng.integers(-3, 3, n).astype(np.float32)  # many equal maxima
    cases.append(t)
    for c in cases:
        x = torch.from_numpy(c).cuda()
        got = int(Kc.argmax(x).item())
        assert got == int(np.argmax(c)), (got, int(np.argmax(c)))
    # history: three calls into a two-slot history starting before slot 0
    x = torch.from_numpy(cases[0]).cuda()
    seq = torch.full((2,), -7, dtype=torch.int64, device="cuda")
    pos = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    out = torch.empty(1, dtype=torch.int64, device="cuda")
    for _ in range(3):
        Kc.argmax(x, out=out, seq=seq, seq_pos=pos)
    want = int(np.argmax(cases[0]))
    assert seq.tolist() == [want, want] and pos.item() == 2 and out.item() == want
