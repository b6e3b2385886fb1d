"""A GPT-2-style decoder on the GPU around the KV-cache entry points.

[KV-2] openai-hub.com/news/2435, "GPT-2缓存实测：千倍计算只快6倍": GPT-2 Small
(12 layers, width 768, 12 heads, 1024 positions, FP32, batch 1, greedy
decoding) generated with a KV cache and by recomputing the whole context
every step; the table there gives the per-token latency of both at context
1000.  This module runs both forms on MI355X with synthetic weights
(trained ones are not available):

  * cached: the prompt goes through ``kvc_attn_prefill`` (which also fills
    the cache), each new token through ``kvc_decode_step`` (append + split-K
    attention over the history), one call per layer;
  * recompute: every step runs the whole context through
    ``kvc_attn_prefill`` again on a scratch cache.

The block follows the published GPT-2 design: pre-norm residual blocks,
learned positions, layer-norm eps 1e-5, tanh GELU, final layer norm, token
embedding reused as the output projection; q/k/v are the three d-wide
thirds of the QKV product with head h owning columns [h D, (h+1) D).

Where each step runs:
  * the input embedding (token + position): ``kvc_embed_f32``;
  * attention and every cache access: the library's HIP kernels;
  * the dense layers of a decode step (at most 4 new tokens): the library's
    fused ``kvc_linear_f32`` (layer norm + matrix-vector product + bias +
    GELU / residual in one HBM-bound pass over the weights);
  * the dense layers of a prompt (more tokens): the library's fp32
    matrix-core product ``kvc_gemm_f32`` (bias, GELU and residual fused into
    its store; the QKV product written straight into the attention layout,
    the output projection reading the attention output as the prefill
    writes it) and its row-wise ``kvc_layernorm_f32``.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import kvcache as K


class GPT2:
    """Weights (a ``synth.GPT2Weights``-like object with numpy arrays) on one
    GPU, fp32."""

    def __init__(self, w, device="cuda"):
        torch.backends.cuda.matmul.allow_tf32 = False
        dev = torch.device(device)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        self.L, self.d, self.H, self.V, self.T = w.L, w.d, w.H, w.V, w.T
        self.D = w.d // w.H
        self.scale = 1.0 / math.sqrt(self.D)
        self.device = dev
        self.wte, self.wpe = t(w.wte), t(w.wpe)
        names = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g", "ln2_b",
                 "w_fc", "b_fc", "w_pr", "b_pr")
        self.p = {n: t(getattr(w, n)) for n in names}
        # the dense kernels take each weight transposed ([out, in]), packed
        # once here; the token embedding [V, d] already is the output
        # projection's transposed weight
        self.pt = {n: self.p[n].transpose(1, 2).contiguous() for n in ("w_qkv", "w_o", "w_fc", "w_pr")}
        self.lnf_g, self.lnf_b = t(w.lnf_g), t(w.lnf_b)
        self._ws = {}

    def new_cache(self) -> K.KVCache:
        """An empty [L, 1, H, T, D] cache (batch 1, as in the pages)."""
        return K.KVCache(self.L, 1, self.H, self.T, self.D, torch.float32, device=self.device)

    def _workspace(self, cache, n):
        key = (cache.k.data_ptr(), n)
        if key not in self._ws:
            self._ws[key] = K.new_decode_workspace(cache, 1, self.H, n)
        return self._ws[key]

    def forward(self, ids, cache: K.KVCache, P: int, last_only=False):
        """Logits of the N tokens ``ids`` (int64 tensor on the device) at
        positions P .. P+N-1.  P = 0 prefills ``cache`` with them; P > 0
        appends them to the P cached positions.  ``last_only`` returns the
        last position's logits only ([1, V])."""
        N = int(ids.shape[0])
        if N == 0:
            return torch.empty((0, self.V), dtype=torch.float32, device=self.device)
        if P + N > self.T:
            raise ValueError(f"context {P + N} exceeds {self.T} positions")
        d, H, D, p = self.d, self.H, self.D, self.p
        h = K.embed(self.wte, self.wpe, ids, pos0=P)
        if N <= self.DECODE_ROWS:
            return self._forward_decode(h, cache, P, last_only)
        a = torch.empty_like(h)
        pt = self.pt
        for l in range(self.L):
            K.layer_norm(h, p["ln1_g"][l], p["ln1_b"][l], out=a)
            t = K.gemm(a, pt["w_qkv"][l], p["b_qkv"][l], qkv_heads=H)         # [3, H, N, D]
            q, k, v = (t[j].view(1, 1, H, N, D) for j in range(3))
            if P == 0:
                o = K.attn_prefill(cache, q, k, v, scale=self.scale, layer0=l)
            else:
                o = K.decode_step(cache, q, k, v, [P], scale=self.scale, layer0=l,
                                  workspace=self._workspace(cache, N))
            K.gemm(o.view(H, N, D), pt["w_o"][l], p["b_o"][l], residual=h, out=h, a_heads=H)
            K.layer_norm(h, p["ln2_g"][l], p["ln2_b"][l], out=a)
            f = K.gemm(a, pt["w_fc"][l], p["b_fc"][l], act="gelu")
            K.gemm(f, pt["w_pr"][l], p["b_pr"][l], residual=h, out=h)
        if last_only:
            h = h[-1:]
        if h.shape[0] <= K.MAX_LINEAR_ROWS:
            z = K.linear(h, self.wte, ln=(self.lnf_g, self.lnf_b))
        else:
            # the token embedding [V, d] is already the transposed output weight
            z = K.gemm(K.layer_norm(h, self.lnf_g, self.lnf_b), self.wte)
        return z[:, :self.V]

    DECODE_ROWS = 4  # rows whose dense layers run in kvc_linear_f32 (4 x 3072 inputs fit)

    def _forward_decode(self, h, cache, P, last_only):
        """The layers for N <= DECODE_ROWS tokens, every dense layer fused:
        LN1 + QKV, attention (append + split-K decode, or prefill on an
        empty cache), output projection + residual, LN2 + FC + GELU,
        projection + residual, and LN_f + output projection."""
        N = h.shape[0]
        H, D, p, pt = self.H, self.D, self.p, self.pt
        for l in range(self.L):
            # q, k, v written straight in the attention layout [3, H, N, D]
            t = K.linear(h, pt["w_qkv"][l], p["b_qkv"][l], ln=(p["ln1_g"][l], p["ln1_b"][l]),
                         qkv_heads=H)
            q, k, v = (t[j].view(1, 1, H, N, D) for j in range(3))
            if P == 0:
                o = K.attn_prefill(cache, q, k, v, scale=self.scale, layer0=l)
            else:
                o = K.decode_step(cache, q, k, v, [P], scale=self.scale, layer0=l,
                                  workspace=self._workspace(cache, N))
            # the output projection reads the attention output head-major
            K.linear(o.view(H, N, D), pt["w_o"][l], p["b_o"][l], residual=h, out=h, a_heads=H)
            f = K.linear(h, pt["w_fc"][l], p["b_fc"][l], ln=(p["ln2_g"][l], p["ln2_b"][l]),
                         act="gelu")
            K.linear(f, pt["w_pr"][l], p["b_pr"][l], residual=h, out=h)
        if last_only:
            h = h[-1:]
        z = K.linear(h, self.wte, ln=(self.lnf_g, self.lnf_b))
        return z[:, :self.V]

    def _decode_token_dl(self, tok, hd, cache):
        """One cached decode step for the token ids ``tok`` (int64 [1] on the
        device) at the device position ``hd`` (int32 [1]); every shape and
        argument is fixed, so the step can be captured once and replayed."""
        H, D, p, pt = self.H, self.D, self.p, self.pt
        h = K.embed(self.wte, self.wpe, tok, pos=hd)
        for l in range(self.L):
            t = K.linear(h, pt["w_qkv"][l], p["b_qkv"][l], ln=(p["ln1_g"][l], p["ln1_b"][l]),
                         qkv_heads=H)
            q, k, v = (t[j].view(1, 1, H, 1, D) for j in range(3))
            o = K.decode_step_dl(cache, q, k, v, hd, self.T - 1, scale=self.scale, layer0=l,
                                 workspace=self._workspace(cache, 1))
            K.linear(o.view(H, 1, D), pt["w_o"][l], p["b_o"][l], residual=h, out=h, a_heads=H)
            f = K.linear(h, pt["w_fc"][l], p["b_fc"][l], ln=(p["ln2_g"][l], p["ln2_b"][l]),
                         act="gelu")
            K.linear(f, pt["w_pr"][l], p["b_pr"][l], residual=h, out=h)
        z = K.linear(h, self.wte, ln=(self.lnf_g, self.lnf_b))
        return z[:, :self.V]

    def generate_graph(self, prompt, n_new):
        """Greedy decoding with the whole token step -- every layer, the
        output projection, the argmax and the length update -- captured in
        one HIP graph after the prompt's prefill and replayed n_new - 1 times.
        Returns (tokens, the replay time per token in ms)."""
        if n_new <= 0:
            return [], 0.0
        cache = self.new_cache()
        ids = torch.tensor([int(x) for x in prompt], device=self.device)
        z = self.forward(ids, cache, 0, last_only=True)
        toks = torch.empty(n_new, dtype=torch.int64, device=self.device)
        tok = torch.empty(1, dtype=torch.int64, device=self.device)
        # step counts the tokens chosen so far, minus one: each argmax
        # advances it and files its token at toks[step]
        step = torch.full((1,), -1, dtype=torch.int64, device=self.device)
        K.argmax(z[0], out=tok, seq=toks, seq_pos=step)
        hd = torch.tensor([len(prompt)], dtype=torch.int32, device=self.device)

        def body():
            zz = self._decode_token_dl(tok, hd, cache)
            K.argmax(zz[0], out=tok, seq=toks, seq_pos=step)
            K.lengths_add(hd, 1)

        if n_new == 1:
            return toks.tolist(), 0.0
        # warm up the workspace and the GEMM handles on a scratch copy of the state
        saved = (cache.k.clone(), cache.v.clone(), hd.clone(), tok.clone(), step.clone())
        body()
        cache.k.copy_(saved[0]); cache.v.copy_(saved[1]); hd.copy_(saved[2])
        tok.copy_(saved[3]); step.copy_(saved[4])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                body()
        torch.cuda.current_stream().wait_stream(s)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(n_new - 1):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return toks.tolist(), t0.elapsed_time(t1) / (n_new - 1)

    def generate(self, prompt, n_new, cached=True):
        """Greedy decoding of n_new tokens after ``prompt`` (a list of ids).
        Returns (tokens, last-position logits of every step as a float64
        numpy array [n_new, V])."""
        ids = [int(x) for x in prompt]
        cache = self.new_cache()
        scratch = None if cached else self.new_cache()
        out = []
        P = 0
        nxt = ids
        for _ in range(n_new):
            if cached:
                z = self.forward(torch.tensor(nxt, device=self.device), cache, P, last_only=True)
                P += len(nxt)
            else:
                z = self.forward(torch.tensor(ids, device=self.device), scratch, 0, last_only=True)
            zt = z[0].double().cpu().numpy()
            out.append(zt)
            tok = int(np.argmax(zt))
            ids.append(tok)
            nxt = [tok]
        return ids[len(prompt):], np.stack(out)
