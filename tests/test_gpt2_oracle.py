"""Pins of the GPT-2-style oracle (oracle/gpt2.py) against facts that do not
come from the oracle itself: an independent GPT-2 implementation (the
Hugging Face ``transformers`` GPT2LMHeadModel, loaded with the same weights),
which is the pages' first correctness test ([KV-2] "正确性先于性能", test 1:
the no-cache model's full logits against the reference implementation); the
pages' cached-versus-recompute identity (tests 2-4); closed forms of layer
norm and GELU; the pinned C attention oracle; causality; and a closed form of
the whole model when every block is switched off."""
import math

import numpy as np
import pytest

import oracle
import oracle.gpt2 as G
from transformer_kv_cache_amd import synth

W = synth.gpt2_weights(seed=3, L=2, d=128, H=2, V=300, T=48)


def test_cached_decode_equals_recompute_every_step():
    """Greedy generation with the cache and with full recomputation: same
    tokens and the same last-position logits at every step."""
    prompt = synth.token_ids(4, 7, W.V)
    t1, z1 = G.generate(W, prompt, 12, cached=True)
    t2, z2 = G.generate(W, prompt, 12, cached=False)
    assert t1 == t2
    assert np.max(np.abs(z1 - z2)) <= 1e-12 * np.max(np.abs(z2))


@pytest.mark.parametrize("chunks", [(1,), (5, 1, 1), (3, 8, 2), (1, 1, 1, 1, 9)])
def test_chunked_decode_equals_whole_sequence(chunks):
    """Prefill of the first chunk, then decode steps of several tokens at
    once (row i of a chunk sees P+i+1 keys): every position's logits match
    the single full forward, including a one-token prompt on an empty cache."""
    ids = synth.token_ids(5, sum(chunks), W.V)
    full = G.forward(W, ids)
    c, p = G.Cache(W), 0
    for n in chunks:
        z = G.forward(W, ids[p:p + n], c)
        assert np.max(np.abs(z - full[p:p + n])) <= 1e-12 * np.max(np.abs(full))
        p += n
    assert c.length == p


def test_context_limit():
    """Up to the last position of the table, and refused past it."""
    ids = synth.token_ids(6, W.T, W.V)
    c = G.Cache(W)
    G.forward(W, ids[:-1], c)
    G.forward(W, ids[-1:], c)
    assert c.length == W.T
    with pytest.raises(ValueError):
        G.forward(W, ids[:1], c)


def test_layer_norm_closed_form():
    x = np.random.default_rng(0).standard_normal((5, 64)) * 3 + 1.5
    y = G.layer_norm(x, np.ones(64), np.zeros(64))
    assert np.allclose(y.mean(-1), 0, atol=1e-12)
    var = x.var(-1)
    assert np.allclose((y ** 2).mean(-1), var / (var + G.LN_EPS), atol=1e-12)
    g, b = np.linspace(0.5, 2, 64), np.linspace(-1, 1, 64)
    assert np.allclose(G.layer_norm(x, g, b), y * g + b, atol=1e-12)


def test_gelu_closed_forms():
    x = np.linspace(-8, 8, 4001)
    exact = 0.5 * x * (1 + np.vectorize(math.erf)(x / math.sqrt(2)))
    # the tanh form is within 5e-4 of the exact GELU everywhere
    assert np.max(np.abs(G.gelu(x) - exact)) < 5e-4
    # gelu(x) - gelu(-x) = x exactly for the tanh form; gelu(0) = 0
    assert np.allclose(G.gelu(x) - G.gelu(-x), x, atol=1e-12)
    assert G.gelu(np.array([0.0]))[0] == 0.0


def test_attention_matches_pinned_c_oracle():
    """The model's attention against the C oracle (pinned separately) on
    fp32 inputs: 3 cached rows plus 4 new ones, two heads."""
    rng = np.random.default_rng(7)
    H, P, N, D = 2, 3, 4, 64
    q = rng.standard_normal((H, N, D), dtype=np.float32)
    k = rng.standard_normal((H, P + N, D), dtype=np.float32)
    v = rng.standard_normal((H, P + N, D), dtype=np.float32)
    kc = np.zeros((1, 1, H, 16, D), np.float32)
    vc = np.zeros_like(kc)
    kc[0, 0, :, :P + N] = k
    vc[0, 0, :, :P + N] = v
    ref = oracle.attention(q[None, None], kc, vc, np.array([P], np.int32), 1 / math.sqrt(D))[0, 0]
    got = G.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), P)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_attention_large_scores():
    """Scores of several thousand (exp overflows unless the softmax subtracts
    its maximum first): still
    the C oracle's result."""
    rng = np.random.default_rng(11)
    H, P, N, D = 1, 5, 2, 64
    q = (100 * rng.standard_normal((H, N, D))).astype(np.float32)
    k = (100 * rng.standard_normal((H, P + N, D))).astype(np.float32)
    v = rng.standard_normal((H, P + N, D), dtype=np.float32)
    kc = np.zeros((1, 1, H, 8, D), np.float32)
    vc = np.zeros_like(kc)
    kc[0, 0, :, :P + N] = k
    vc[0, 0, :, :P + N] = v
    ref = oracle.attention(q[None, None], kc, vc, np.array([P], np.int32), 1 / math.sqrt(D))[0, 0]
    got = G.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), P)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_causal():
    """Logits of positions 0..t do not depend on the tokens after t."""
    ids = synth.token_ids(8, 20, W.V)
    other = ids.copy()
    other[12:] = (other[12:] + 17) % W.V
    a, b = G.forward(W, ids), G.forward(W, other)
    assert np.array_equal(a[:12], b[:12])
    assert not np.allclose(a[12:], b[12:])


def test_blocks_switched_off_reduce_to_embeddings():
    """With every block's projections and biases zero, attention returns v = 0
    and the MLP returns gelu(0) W = 0, so the logits are
    LN_f(wte[id] + wpe[pos]) . wte^T, whatever the layer count."""
    w = synth.gpt2_weights(seed=9, L=3, d=64, H=2, V=50, T=16)
    for name in ("w_qkv", "b_qkv", "w_o", "b_o", "w_fc", "b_fc", "w_pr", "b_pr"):
        setattr(w, name, np.zeros_like(getattr(w, name)))
    ids = synth.token_ids(10, 9, w.V)
    h = w.wte[ids].astype(np.float64) + w.wpe[:9]
    mu = h.mean(-1, keepdims=True)
    sd = np.sqrt(((h - mu) ** 2).mean(-1, keepdims=True) + 1e-5)
    want = ((h - mu) / sd * w.lnf_g + w.lnf_b) @ w.wte.T.astype(np.float64)
    assert np.max(np.abs(G.forward(w, ids) - want)) <= 1e-12


def _hf_logits(w, ids):
    """Full-sequence logits of ``ids`` from the Hugging Face GPT-2 model
    built in float64 with the weights of ``w`` (dropout off, layer-norm eps
    1e-5, tanh GELU, output projection tied to the token embedding).  Its
    Conv1D layers store [in, out] matrices, the layout of w_qkv, w_o, w_fc
    and w_pr; its attention splits the QKV product into q, k, v thirds and
    each third into heads by its own code, not the oracle's."""
    transformers = pytest.importorskip("transformers")
    import torch
    cfg = transformers.GPT2Config(
        n_layer=w.L, n_embd=w.d, n_head=w.H, vocab_size=w.V, n_positions=w.T,
        layer_norm_epsilon=1e-5, activation_function="gelu_new", resid_pdrop=0.0,
        embd_pdrop=0.0, attn_pdrop=0.0, tie_word_embeddings=True,
        bos_token_id=0, eos_token_id=0)
    model = transformers.GPT2LMHeadModel(cfg).double().eval()
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    sd = {"transformer.wte.weight": t(w.wte), "transformer.wpe.weight": t(w.wpe),
          "transformer.ln_f.weight": t(w.lnf_g), "transformer.ln_f.bias": t(w.lnf_b),
          "lm_head.weight": t(w.wte)}
    for l in range(w.L):
        p = f"transformer.h.{l}."
        sd.update({p + "ln_1.weight": t(w.ln1_g[l]), p + "ln_1.bias": t(w.ln1_b[l]),
                   p + "attn.c_attn.weight": t(w.w_qkv[l]), p + "attn.c_attn.bias": t(w.b_qkv[l]),
                   p + "attn.c_proj.weight": t(w.w_o[l]), p + "attn.c_proj.bias": t(w.b_o[l]),
                   p + "ln_2.weight": t(w.ln2_g[l]), p + "ln_2.bias": t(w.ln2_b[l]),
                   p + "mlp.c_fc.weight": t(w.w_fc[l]), p + "mlp.c_fc.bias": t(w.b_fc[l]),
                   p + "mlp.c_proj.weight": t(w.w_pr[l]), p + "mlp.c_proj.bias": t(w.b_pr[l])})
    missing, unexpected = model.load_state_dict(sd, strict=False)
    assert not unexpected and all("attn.bias" in k or "masked_bias" in k for k in missing), \
        (missing, unexpected)
    with torch.no_grad():
        out = model(torch.from_numpy(np.asarray(ids, dtype=np.int64))[None], use_cache=False)
    return out.logits[0].numpy()


def test_logits_match_reference_implementation():
    """[KV-2] "正确性先于性能", test 1: the no-cache model's full logits
    against an independent GPT-2 implementation on the same weights, every
    position of a 20-token sequence (both float64: agreement to rounding)."""
    ids = synth.token_ids(12, 20, W.V)
    ref = _hf_logits(W, ids)
    assert np.max(np.abs(G.forward(W, ids) - ref)) <= 1e-12


def test_logits_match_reference_implementation_gpt2_small_width():
    """The same at GPT-2 Small's sizes (12 layers, width 768, 12 heads,
    vocabulary 50257, 1024 positions) on a short sequence placed at the
    start of the position table."""
    w = synth.gpt2_weights(seed=4)
    ids = synth.token_ids(13, 5, w.V)
    ref = _hf_logits(w, ids)
    assert np.max(np.abs(G.forward(w, ids) - ref)) <= 1e-12


# ---- plausible mistakes the pins must catch ----------------------------------

MUTANTS = {
    "positions_from_zero_when_cached": ("_f(w.wpe)[P:P + N]", "_f(w.wpe)[0:N]"),
    "mask_without_history": ("(P + np.arange(N))[:, None]", "(np.arange(N))[:, None]"),
    "no_attention_residual": ("h = h + o @ _f(w.w_o[l])", "h = o @ _f(w.w_o[l])"),
    "gelu_wrong_constant": ("(x + 0.044715 * x ** 3)", "(x + 0.44715 * x ** 3)"),
    "scale_by_d": ("/ math.sqrt(D)", "/ D"),
    "eps_outside_sqrt": ("np.sqrt(var + LN_EPS)", "(np.sqrt(var) + LN_EPS)"),
    "no_final_norm": ("return layer_norm(h, _f(w.lnf_g), _f(w.lnf_b)) @", "return h @"),
    "cache_rows_not_written": ("cache.k[l, :, P:P + N] = k", "cache.k[l, :, P:P + N] = 0 * k"),
    "softmax_without_max": ("s = s - s.max(axis=-1, keepdims=True)", "s = s - 0.0"),
    "qkv_thirds_swapped": ("q, k, v = (qkv[:, j * d:", "k, q, v = (qkv[:, j * d:"),
    "heads_interleaved": (".reshape(N, H, D).transpose(1, 0, 2) for j",
                          ".reshape(N, D, H).transpose(2, 0, 1) for j"),
    "layer_norm_gain_and_shift_swapped": ("a = layer_norm(h, _f(w.ln1_g[l]), _f(w.ln1_b[l]))",
                                          "a = layer_norm(h, _f(w.ln1_b[l]), _f(w.ln1_g[l]))"),
    "mlp_without_gelu": ("h = h + gelu(m @ _f(w.w_fc[l])", "h = h + (m @ _f(w.w_fc[l])"),
}

PINS = [test_logits_match_reference_implementation, test_cached_decode_equals_recompute_every_step, test_context_limit, test_layer_norm_closed_form,
        test_gelu_closed_forms, test_attention_matches_pinned_c_oracle, test_attention_large_scores,
        test_causal,
        test_blocks_switched_off_reduce_to_embeddings,
        lambda: test_chunked_decode_equals_whole_sequence((3, 8, 2))]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path, monkeypatch):
    import importlib.util
    src = open(G.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / "gpt2_mutant.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("gpt2_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    monkeypatch.setattr(__import__(__name__), "G", mod)
    caught = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError):
            caught += 1
    assert caught > 0, f"no pin catches {name}"
