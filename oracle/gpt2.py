"""CPU oracle of a GPT-2-style decoder around the KV cache -- test
infrastructure only (the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it; the product never does).

What it computes.  [KV-2] openai-hub.com/news/2435, "GPT-2缓存实测：千倍计算只
快6倍" and its configuration table: GPT-2 Small (12 layers, width 768, 12
heads, 1024 positions, FP32, batch 1, greedy decoding), generated once with a
KV cache and once recomputing the whole context every step, the two compared
by the last position's logits at every step ("正确性先于性能", tests 2-4).
[KV-4] jennyma11.github.io/infra/ch07-01.html, "Prefill 阶段" / "Decode 阶段":
the prompt fills the cache, each decode step appends its K/V rows and
attends over the history.

The pages fix the sizes but not the block; it follows the published GPT-2
design (a reading): pre-norm residual blocks
    h += W_o . attn(LN1(h) W_qkv + b_qkv) + b_o
    h += W_pr . gelu(LN2(h) W_fc + b_fc) + b_pr
with learned position embeddings, layer norm eps 1e-5, the tanh form of GELU,
a final layer norm and the token embedding reused as the output projection.
q, k, v are the three d-wide thirds of the QKV product, head h owning
columns [h D, (h+1) D) of each; attention is scaled by 1/sqrt(D) and row i of
N new rows on P cached ones sees positions 0 .. P+i ([KV-2] "一个很容易漏掉
的错误").

Everything runs in float64 numpy: matrix products are library calls
(numpy.matmul), the rest is written out.  The attention materialises the full
masked score matrix and subtracts the row maximum.
"""
from __future__ import annotations

import math

import numpy as np

LN_EPS = 1e-5


def layer_norm(x, g, b):
    """(x - mean) / sqrt(var + eps) * g + b over the last axis (biased var)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + LN_EPS) * g + b


def gelu(x):
    """GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def attention(q, k, v, P):
    """q [H, N, D] for positions P .. P+N-1; k, v [H, P+N, D] for positions
    0 .. P+N-1.  Row i sees keys 0 .. P+i."""
    H, N, D = q.shape
    s = (q @ np.swapaxes(k, 1, 2)) / math.sqrt(D)            # [H, N, P+N]
    vis = np.arange(P + N)[None, :] <= (P + np.arange(N))[:, None]
    s = np.where(vis[None], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=-1, keepdims=True)) @ v            # [H, N, D]


class Cache:
    """Per-layer K and V rows of one sequence, float64 [L, H, T, D]."""

    def __init__(self, w):
        self.k = np.zeros((w.L, w.H, w.T, w.D))
        self.v = np.zeros((w.L, w.H, w.T, w.D))
        self.length = 0


def _f(a):
    return np.asarray(a, dtype=np.float64)


def forward(w, ids, cache=None):
    """Logits [N, V] of the N tokens ``ids``.  With ``cache`` they sit at
    positions cache.length .. +N-1 and attend to the cached rows, which the
    call extends; without it they are a whole sequence from position 0."""
    ids = np.asarray(ids, dtype=np.int64)
    N = ids.shape[0]
    P = cache.length if cache is not None else 0
    if P + N > w.T:
        raise ValueError("forward: context longer than the position table")
    H, D, d = w.H, w.D, w.d
    h = _f(w.wte)[ids] + _f(w.wpe)[P:P + N]
    for l in range(w.L):
        a = layer_norm(h, _f(w.ln1_g[l]), _f(w.ln1_b[l]))
        qkv = a @ _f(w.w_qkv[l]) + _f(w.b_qkv[l])                # [N, 3d]
        q, k, v = (qkv[:, j * d:(j + 1) * d].reshape(N, H, D).transpose(1, 0, 2) for j in range(3))
        if cache is not None:
            cache.k[l, :, P:P + N] = k
            cache.v[l, :, P:P + N] = v
            k, v = cache.k[l, :, :P + N], cache.v[l, :, :P + N]
        o = attention(q, k, v, P).transpose(1, 0, 2).reshape(N, d)
        h = h + o @ _f(w.w_o[l]) + _f(w.b_o[l])
        m = layer_norm(h, _f(w.ln2_g[l]), _f(w.ln2_b[l]))
        h = h + gelu(m @ _f(w.w_fc[l]) + _f(w.b_fc[l])) @ _f(w.w_pr[l]) + _f(w.b_pr[l])
    if cache is not None:
        cache.length = P + N
    return layer_norm(h, _f(w.lnf_g), _f(w.lnf_b)) @ _f(w.wte).T


def generate(w, prompt, n_new, cached=True):
    """Greedy decoding of n_new tokens after ``prompt``.  Returns (tokens,
    last-position logits of every step [n_new, V]).  cached=False
    recomputes the whole context at every step."""
    ids = list(np.asarray(prompt, dtype=np.int64))
    cache = Cache(w) if cached else None
    step_logits = []
    nxt = ids
    for _ in range(n_new):
        if cached:
            z = forward(w, nxt, cache)[-1]
        else:
            z = forward(w, ids)[-1]
        step_logits.append(z)
        t = int(np.argmax(z))
        ids.append(t)
        nxt = [t]
    return ids[len(prompt):], np.stack(step_logits)
