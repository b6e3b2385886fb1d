"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError when the oracle disagrees with what the pages or the
mathematics fix.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with a mistake
planted, and requires every planted mistake to trip at least one pin.

Pages (by address and section):
  [KV-1] gitcode.csdn.net/69e62cef0a2f6a37c5a11c4f.html  "KV Cache 原理", "Decode Shape 示例"
  [KV-2] openai-hub.com/news/2435  "一个很容易漏掉的错误", "GPT-2缓存要占多少显存"
  [KV-4] jennyma11.github.io/infra/ch07-01.html  "Decode 阶段" listing 1-2, "Prefill 阶段"
"""
from __future__ import annotations

import math
import os

import numpy as np

import oracle
from transformer_kv_cache_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _empty_cache(L, B, H, T, D, dtype="f32"):
    return synth.canary_cache((L, B, H, T, D), dtype), synth.canary_cache((L, B, H, T, D), dtype)


def _fill_history(kc, vc, hist, rng):
    L, B, H, T, D = kc.shape
    for b in range(B):
        p = int(hist[b])
        kc[:, b, :, :p] = rng.standard_normal((L, H, p, D), dtype=np.float32)
        vc[:, b, :, :p] = rng.standard_normal((L, H, p, D), dtype=np.float32)


def _decode(lib, kc, vc, q, k, v, hist, scale, layer0=0):
    """append then attention, the decode step's order ([KV-2] "一个很容易漏掉的错误")."""
    oracle.append(kc, vc, k, v, hist, layer0=layer0, lib=lib)
    return oracle.attention(q, kc, vc, hist, scale, layer0=layer0, lib=lib)


# ---------------------------------------------------------------- closed forms

def pin_cache_bytes_golden(lib):
    """Cache size formula against every size the page prints ([KV-2]
    "GPT-2缓存要占多少显存": formula, worked example and size table)."""
    unit = {"B": 1, "KiB": 1024, "MiB": 1024 * 1024}
    with open(os.path.join(GOLDEN, "cache_sizes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            L, B, H, D, T, e, val, u, digits = line.split()
            got = oracle.cache_bytes(int(L), int(B), int(H), int(T), int(D), int(e), lib=lib)
            shown = round(got / unit[u], int(digits))
            assert shown == float(val), (line, got, shown)


def pin_single_key_exact(lib):
    """Softmax over one key is exactly 1, so a row that sees one key returns
    that key's value row exactly (P=0, N=1; and prefill row 0)."""
    rng = _rng(1)
    for dtype in ("f32", "bf16"):
        kc, vc = _empty_cache(2, 2, 3, 5, 8, dtype)
        q, k, v = (synth.as_dtype(rng.standard_normal((2, 2, 3, 1, 8), dtype=np.float32), dtype)
                   for _ in range(3))
        out = _decode(lib, kc, vc, q, k, v, np.zeros(2, np.int32), 0.5)
        assert np.array_equal(out, synth.to_float(v)), dtype
    kc, vc = _empty_cache(1, 1, 2, 6, 4)
    q, k, v = (rng.standard_normal((1, 1, 2, 6, 4), dtype=np.float32) for _ in range(3))
    out = oracle.prefill(kc, vc, q, k, v, 0.5, lib=lib)
    assert np.array_equal(out[:, :, :, 0], v[:, :, :, 0].astype(np.float64))


def pin_zero_query_counts_visible_keys(lib):
    """q = 0 makes every score 0, so row i returns the plain mean of the V rows
    it sees.  With V[j,0] = j that mean is (n-1)/2, which recovers the count
    n = P+i+1 exactly ([KV-2] "一个很容易漏掉的错误": new row i sees P+i+1
    keys).  Different histories per sequence, and a GQA grouping."""
    L, B, Hkv, Hq, T, D, N = 2, 3, 2, 4, 24, 4, 5
    hist = np.array([0, 7, 19], np.int32)
    rng = _rng(2)
    kc, vc = _empty_cache(L, B, Hkv, T, D)
    _fill_history(kc, vc, hist, rng)
    for b in range(B):
        vc[:, b, :, : hist[b], 0] = np.arange(hist[b], dtype=np.float32)
    q = np.zeros((L, B, Hq, N, D), np.float32)
    k = rng.standard_normal((L, B, Hkv, N, D), dtype=np.float32)
    v = rng.standard_normal((L, B, Hkv, N, D), dtype=np.float32)
    for b in range(B):
        v[:, b, :, :, 0] = hist[b] + np.arange(N, dtype=np.float32)
    out = _decode(lib, kc, vc, q, k, v, hist, 1.0)
    for b in range(B):
        for i in range(N):
            n = 2.0 * out[:, b, :, i, 0] + 1.0
            assert np.allclose(n, hist[b] + i + 1, rtol=0, atol=1e-9), (b, i, n)


def pin_uniform_keys_give_mean(lib):
    """All visible keys equal: every score is the same, so the output is the
    mean of the visible V rows, for any q."""
    L, B, H, T, D, N, P = 1, 2, 2, 16, 8, 4, 9
    rng = _rng(3)
    kc, vc = _empty_cache(L, B, H, T, D)
    hist = np.full(B, P, np.int32)
    _fill_history(kc, vc, hist, rng)
    krow = rng.standard_normal(D, dtype=np.float32)
    kc[:, :, :, :P] = krow
    q = rng.standard_normal((L, B, H, N, D), dtype=np.float32)
    k = np.broadcast_to(krow, (L, B, H, N, D)).copy()
    v = rng.standard_normal((L, B, H, N, D), dtype=np.float32)
    out = _decode(lib, kc, vc, q, k, v, hist, 0.3)
    for i in range(N):
        mean = vc[:, :, :, : P + i + 1].astype(np.float64).mean(axis=3)
        assert np.allclose(out[:, :, :, i], mean, rtol=0, atol=1e-12)


def pin_one_hot_selects_value(lib):
    """One key aligned with q and scaled by c dominates: its weight is within
    exp(-margin) of 1, so the output is that key's V row to that bound."""
    D, P = 16, 11
    rng = _rng(4)
    kc, vc = _empty_cache(1, 1, 1, 16, D)
    hist = np.array([P], np.int32)
    _fill_history(kc, vc, hist, rng)
    kc[:] = np.where(np.isnan(kc), kc, kc * np.float32(0.01))
    q = rng.standard_normal((1, 1, 1, 1, D), dtype=np.float32)
    j = 5
    c = np.float32(40.0)
    kc[0, 0, 0, j] = c * q[0, 0, 0, 0] / np.float32(np.dot(q[0, 0, 0, 0], q[0, 0, 0, 0]))
    k = (rng.standard_normal((1, 1, 1, 1, D), dtype=np.float32) * np.float32(0.01))
    v = rng.standard_normal((1, 1, 1, 1, D), dtype=np.float32)
    out = _decode(lib, kc, vc, q, k, v, hist, 1.0)
    bound = (P + 1) * math.exp(-(40.0 - 3.0)) * 10
    assert np.max(np.abs(out[0, 0, 0, 0] - vc[0, 0, 0, j])) < bound


def pin_two_keys_sigmoid(lib):
    """D=1, one head, two keys: softmax of two scores is a logistic function,
    o = v0 + (v1 - v0) * sigmoid(scale*q*(k1 - k0)).  With N=2 new rows and no
    history, row 0 sees only key 0 (o = v0) and row 1 sees both."""
    cases = [(1.0, 0.0, math.log(3.0), 2.0, -6.0, 1.0),
             (0.7, -1.25, 0.5, 0.25, 3.0, 0.125),
             (-2.0, 1.5, -0.75, -1.0, 4.0, 1.0 / math.sqrt(2.0))]
    for qv, k0, k1, v0, v1, scale in cases:
        kc, vc = _empty_cache(1, 1, 1, 3, 1)
        q = np.array([qv, qv], np.float32).reshape(1, 1, 1, 2, 1)
        k = np.array([k0, k1], np.float32).reshape(1, 1, 1, 2, 1)
        v = np.array([v0, v1], np.float32).reshape(1, 1, 1, 2, 1)
        out = _decode(lib, kc, vc, q, k, v, np.zeros(1, np.int32), scale)
        qf, k0f, k1f, v0f, v1f = (float(np.float32(x)) for x in (qv, k0, k1, v0, v1))
        z = scale * qf * (k1f - k0f)
        expect1 = v0f + (v1f - v0f) / (1.0 + math.exp(-z))
        assert out[0, 0, 0, 0, 0] == v0f
        assert abs(out[0, 0, 0, 1, 0] - expect1) < 1e-14, (out[0, 0, 0, 1, 0], expect1)


def pin_zero_and_negative_scale(lib):
    """Any finite scale: with scale 0 every visible key scores 0, so each row
    is the plain mean of its visible V rows (closed form); a negative scale
    is the positive one applied to -q (IEEE negation is exact, so bit for
    bit); and the two-key logistic form holds with a negative scale."""
    L, B, H, T, D, N, P = 1, 2, 2, 16, 8, 3, 6
    rng = _rng(21)
    kc, vc = _empty_cache(L, B, H, T, D)
    hist = np.full(B, P, np.int32)
    _fill_history(kc, vc, hist, rng)
    q, k, v = (rng.standard_normal((L, B, H, N, D), dtype=np.float32) for _ in range(3))
    out0 = _decode(lib, kc.copy(), vc.copy(), q, k, v, hist, 0.0)
    kk, vv = kc.copy(), vc.copy()
    oracle.append(kk, vv, k, v, hist, lib=lib)
    for i in range(N):
        mean = vv[:, :, :, : P + i + 1].astype(np.float64).mean(axis=3)
        assert np.allclose(out0[:, :, :, i], mean, rtol=0, atol=1e-12)
    neg = _decode(lib, kc.copy(), vc.copy(), q, k, v, hist, -0.35)
    pos = _decode(lib, kc.copy(), vc.copy(), -q, k, v, hist, 0.35)
    assert np.array_equal(neg, pos)
    assert not np.allclose(neg, _decode(lib, kc.copy(), vc.copy(), q, k, v, hist, 0.35))
    kc1, vc1 = _empty_cache(1, 1, 1, 3, 1)
    q1 = np.array([0.8, 0.8], np.float32).reshape(1, 1, 1, 2, 1)
    k1 = np.array([-0.5, 1.25], np.float32).reshape(1, 1, 1, 2, 1)
    v1 = np.array([3.0, -1.0], np.float32).reshape(1, 1, 1, 2, 1)
    out1 = _decode(lib, kc1, vc1, q1, k1, v1, np.zeros(1, np.int32), -0.5)
    z = -0.5 * float(np.float32(0.8)) * (1.25 - -0.5)
    assert abs(out1[0, 0, 0, 1, 0] - (3.0 + (-1.0 - 3.0) / (1.0 + math.exp(-z)))) < 1e-14


# ------------------------------------------------------------ library routine

def sdpa_reference(q, kc, vc, hist, scale, N):
    """torch's scaled_dot_product_attention in float64, one sequence at a time,
    with an explicit boolean mask: new row i may see keys j <= P_b + i.  KV
    heads are expanded to query heads with repeat_interleave (contiguous
    groups)."""
    import torch
    L, B, Hkv, T, D = kc.shape
    Hq = q.shape[2]
    out = np.zeros(q.shape, np.float64)
    for b in range(B):
        n = int(hist[b]) + N
        K = torch.from_numpy(synth.to_float(kc[:, b, :, :n])).repeat_interleave(Hq // Hkv, dim=1)
        V = torch.from_numpy(synth.to_float(vc[:, b, :, :n])).repeat_interleave(Hq // Hkv, dim=1)
        Q = torch.from_numpy(synth.to_float(q[:, b]))
        mask = torch.arange(n)[None, :] <= (int(hist[b]) + torch.arange(N))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
        out[:, b] = o.numpy()
    return out


def pin_matches_torch_sdpa(lib, n_cases=12):
    """Random tiny shapes (including GQA, several sequences with different
    histories, bf16 storage) against torch's float64 attention."""
    rng = _rng(5)
    for case in range(n_cases):
        L = int(rng.integers(1, 3))
        B = int(rng.integers(1, 4))
        Hkv = int(rng.integers(1, 4))
        G = int(rng.integers(1, 4))
        D = int(rng.choice([1, 2, 8, 64]))
        N = int(rng.integers(1, 7))
        T = int(rng.integers(N, 40))
        dtype = "bf16" if case % 3 == 2 else "f32"
        hist = rng.integers(0, T - N + 1, size=B).astype(np.int32)
        kc, vc = _empty_cache(L, B, Hkv, T, D, dtype)
        for b in range(B):
            p = int(hist[b])
            kc[:, b, :, :p] = synth.as_dtype(rng.standard_normal((L, Hkv, p, D), dtype=np.float32), dtype)
            vc[:, b, :, :p] = synth.as_dtype(rng.standard_normal((L, Hkv, p, D), dtype=np.float32), dtype)
        q = synth.as_dtype(rng.standard_normal((L, B, Hkv * G, N, D), dtype=np.float32), dtype)
        k = synth.as_dtype(rng.standard_normal((L, B, Hkv, N, D), dtype=np.float32), dtype)
        v = synth.as_dtype(rng.standard_normal((L, B, Hkv, N, D), dtype=np.float32), dtype)
        scale = 1.0 / math.sqrt(D)
        out = _decode(lib, kc, vc, q, k, v, hist, scale)
        ref = sdpa_reference(q, kc, vc, hist, scale, N)
        err = np.max(np.abs(out - ref))
        assert err < 1e-12, (case, L, B, Hkv, G, D, N, T, dtype, err)


# ------------------------------------------------------------------ invariants

def pin_cached_equals_recompute(lib):
    """Prefill of all P+N tokens at once, last N rows, equals prefill of P
    tokens then one decode call of N rows -- bit for bit in the oracle, since
    both visit the same keys in the same order ([KV-1] "KV Cache 原理": the
    history's K/V do not change, so reusing them gives the recomputed
    result)."""
    L, B, H, D, T = 2, 1, 3, 16, 40
    for P, N in ((0, 1), (1, 1), (13, 1), (13, 8), (30, 10)):
        rng = _rng(100 + P + N)
        q, k, v = (rng.standard_normal((L, B, H, P + N, D), dtype=np.float32) for _ in range(3))
        kc, vc = _empty_cache(L, B, H, T, D)
        full = oracle.prefill(kc, vc, q, k, v, 0.25, lib=lib)
        kc2, vc2 = _empty_cache(L, B, H, T, D)
        if P:
            oracle.prefill(kc2, vc2, *(np.ascontiguousarray(a[:, :, :, :P]) for a in (q, k, v)), 0.25, lib=lib)
        tail = [np.ascontiguousarray(a[:, :, :, P:]) for a in (q, k, v)]
        inc = _decode(lib, kc2, vc2, *tail, np.full(B, P, np.int32), 0.25)
        assert np.array_equal(full[:, :, :, P:], inc), (P, N)
        assert np.array_equal(kc.view(np.uint32), kc2.view(np.uint32))


def pin_chunk_invariance(lib):
    """prefill(S) == decode(P=0, N=S) == prefill(S-k) + decode(P=S-k, N=k)."""
    L, B, H, D, T, S = 1, 2, 2, 8, 32, 20
    rng = _rng(6)
    q, k, v = (rng.standard_normal((L, B, H, S, D), dtype=np.float32) for _ in range(3))
    kc, vc = _empty_cache(L, B, H, T, D)
    ref = oracle.prefill(kc, vc, q, k, v, 0.3, lib=lib)
    kc1, vc1 = _empty_cache(L, B, H, T, D)
    dec = _decode(lib, kc1, vc1, q, k, v, np.zeros(B, np.int32), 0.3)
    assert np.array_equal(ref, dec)
    for kk in (1, 8):
        kc2, vc2 = _empty_cache(L, B, H, T, D)
        head = [np.ascontiguousarray(a[:, :, :, : S - kk]) for a in (q, k, v)]
        tail = [np.ascontiguousarray(a[:, :, :, S - kk:]) for a in (q, k, v)]
        o1 = oracle.prefill(kc2, vc2, *head, 0.3, lib=lib)
        o2 = _decode(lib, kc2, vc2, *tail, np.full(B, S - kk, np.int32), 0.3)
        assert np.array_equal(np.concatenate([o1, o2], axis=3), ref), kk


def pin_permutation(lib):
    """[KV-2] "一个很容易漏掉的错误".  With one query row, attention is a
    weighted sum over (key, value) pairs, so jointly permuting all visible
    pairs leaves it unchanged.  With N > 1 new rows the causal mask depends on
    position, so the same permutation changes the result; and building the
    cache in the wrong concatenation order (new rows before the history)
    passes a single-row check but fails a chunked one."""
    L, B, H, D, P = 1, 1, 2, 16, 23
    rng = _rng(7)
    for N, must_match in ((1, True), (8, False)):
        T = P + N
        hist = np.array([P], np.int32)
        kc, vc = _empty_cache(L, B, H, T, D)
        _fill_history(kc, vc, hist, rng)
        q, k, v = (rng.standard_normal((L, B, H, N, D), dtype=np.float32) for _ in range(3))
        ref = _decode(lib, kc, vc, q, k, v, hist, 0.25)
        # joint permutation of every (K_j, V_j) pair the cache now holds
        perm = rng.permutation(T)
        kp, vp = kc[:, :, :, perm].copy(), vc[:, :, :, perm].copy()
        got = oracle.attention(q, kp, vp, hist, 0.25, lib=lib)
        diff = np.max(np.abs(got - ref))
        if must_match:
            assert diff < 1e-13, diff
        else:
            assert diff > 1e-3, diff
        # the concatenation-order bug: cache = concat(new, old)
        kr = np.concatenate([k, kc[:, :, :, :P]], axis=3)
        vr = np.concatenate([v, vc[:, :, :, :P]], axis=3)
        bad = oracle.attention(q, np.ascontiguousarray(kr), np.ascontiguousarray(vr), hist, 0.25, lib=lib)
        diff = np.max(np.abs(bad - ref))
        if must_match:
            assert diff < 1e-13, diff
        else:
            assert diff > 1e-3, diff


def pin_gqa_equals_repeated_mha(lib):
    """GQA with G query heads per KV head equals MHA on KV heads repeated G
    times contiguously (query head hq reads KV head hq // G)."""
    L, B, Hkv, G, D, T, N = 2, 2, 3, 4, 8, 20, 3
    hist = np.array([5, 12], np.int32)
    rng = _rng(8)
    kc, vc = _empty_cache(L, B, Hkv, T, D)
    _fill_history(kc, vc, hist, rng)
    q = rng.standard_normal((L, B, Hkv * G, N, D), dtype=np.float32)
    k = rng.standard_normal((L, B, Hkv, N, D), dtype=np.float32)
    v = rng.standard_normal((L, B, Hkv, N, D), dtype=np.float32)
    gqa = _decode(lib, kc, vc, q, k, v, hist, 0.35)
    kr = np.ascontiguousarray(np.repeat(kc, G, axis=2))
    vr = np.ascontiguousarray(np.repeat(vc, G, axis=2))
    mha = oracle.attention(q, kr, vr, hist, 0.35, lib=lib)
    assert np.array_equal(gqa, mha)


def pin_append_positions_and_canaries(lib):
    """The single-layer generation workload: a 16-token prompt then four
    single-token steps leave rows 0..19 equal to the generated K/V bytes and
    rows 20..31 untouched; an append that would pass Tmax is refused without
    writing ([KV-1] "Decode Shape 示例": the cache grows along the sequence
    axis one row per step)."""
    w = synth.single_layer_generation(seed=0)
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    oracle.prefill(kc, vc, *w.prefill, w.scale, lib=lib)
    hist = np.zeros(1, np.int32) + 16
    for (q, k, v) in w.steps:
        _decode(lib, kc, vc, q, k, v, hist, w.scale)
        hist += 1
    assert int(hist[0]) == 20
    kref = np.concatenate([w.prefill[1]] + [s[1] for s in w.steps], axis=3)
    vref = np.concatenate([w.prefill[2]] + [s[2] for s in w.steps], axis=3)
    assert np.array_equal(kc[:, :, :, :20].view(np.uint32), kref.view(np.uint32))
    assert np.array_equal(vc[:, :, :, :20].view(np.uint32), vref.view(np.uint32))
    assert synth.is_canary(kc[:, :, :, 20:]).all() and synth.is_canary(vc[:, :, :, 20:]).all()
    # writes land in the named layers only
    kc2, vc2 = _empty_cache(3, 1, 2, 4, 4)
    kn = np.ones((1, 1, 2, 2, 4), np.float32)
    oracle.append(kc2, vc2, kn, kn * 2, np.array([1], np.int32), layer0=2, lib=lib)
    assert synth.is_canary(kc2[:2]).all() and synth.is_canary(kc2[2, :, :, [0, 3]]).all()
    assert (kc2[2, :, :, 1:3] == 1).all() and (vc2[2, :, :, 1:3] == 2).all()
    # capacity: P + N > Tmax is refused and nothing is written
    before = kc.copy()
    q, k, v = (np.zeros((1, 1, 12, 13, 64), np.float32) for _ in range(3))
    try:
        oracle.append(kc, vc, k, v, np.array([20], np.int32), lib=lib)
        raise AssertionError("capacity overflow accepted")
    except oracle.OracleError:
        pass
    assert np.array_equal(before.view(np.uint32), kc.view(np.uint32))


def pin_bf16_decode_exact(lib):
    """bf16 storage is the high half of an fp32: a single visible key returns
    exactly the widened value, for every finite bf16 bit pattern."""
    hi = np.arange(0, 65536, dtype=np.uint32)
    finite = ((hi >> 7) & 0xFF) != 0xFF
    vals = hi[finite].astype(np.uint16)
    D = vals.size
    kc, vc = _empty_cache(1, 1, 1, 1, D, "bf16")
    q = np.zeros((1, 1, 1, 1, D), np.uint16)
    k = np.zeros((1, 1, 1, 1, D), np.uint16)
    v = vals.reshape(1, 1, 1, 1, D)
    out = _decode(lib, kc, vc, q, k, v, np.zeros(1, np.int32), 1.0)
    expect = (vals.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(out.reshape(-1), expect)


# ---------------------------------------------------------------- paged cache
# Reading of [KV-2] "显存测量最容易被分配器误导" and [KV-4] "Decode 阶段" (in-place
# writes by slot): pools [L, num_blocks, Hkv, block_size, D], position t of
# sequence b in row t % block_size of block block_table[b][t // block_size].


def _paged_canary(L, nblk, H, bs, D, dtype="f32"):
    return _empty_cache(L, nblk, H, bs, D, dtype)


def pin_paged_identity_is_contiguous(lib):
    """With one KV head and the identity table (sequence b's j-th block is
    block b*max_blocks + j), the pool's bytes are the contiguous cache's bytes
    ([L, B, 1, max_blocks*block_size, D] read as [L, B*max_blocks, 1,
    block_size, D]): a paged decode step must leave the same bytes as the
    contiguous append and give the same outputs as the contiguous attention,
    bit for bit."""
    rng = _rng(61)
    L, B, D, bs, mb = 2, 3, 8, 4, 5
    T = bs * mb
    hist = np.array([0, 7, 13], np.int32)  # empty, inside a block, block boundary +1
    kc, vc = _empty_cache(L, B, 1, T, D)
    _fill_history(kc, vc, hist, rng)
    kp = np.ascontiguousarray(kc.reshape(L, B * mb, 1, bs, D))
    vp = np.ascontiguousarray(vc.reshape(L, B * mb, 1, bs, D))
    bt = np.arange(B * mb, dtype=np.int32).reshape(B, mb)
    for N in (1, 3, 6):
        q = rng.standard_normal((L, B, 2, N, D), dtype=np.float32)
        k = rng.standard_normal((L, B, 1, N, D), dtype=np.float32)
        v = rng.standard_normal((L, B, 1, N, D), dtype=np.float32)
        kc2, vc2, kp2, vp2 = kc.copy(), vc.copy(), kp.copy(), vp.copy()
        ref = _decode(lib, kc2, vc2, q, k, v, hist, 0.4)
        oracle.paged_append(kp2, vp2, k, v, hist, bt, lib=lib)
        got = oracle.paged_attention(q, kp2, vp2, hist, bt, 0.4, lib=lib)
        assert np.array_equal(kp2.reshape(kc2.shape).view(np.uint32), kc2.view(np.uint32)), N
        assert np.array_equal(vp2.reshape(vc2.shape).view(np.uint32), vc2.view(np.uint32)), N
        assert np.array_equal(got, ref), N


def _paged_from_history(lib, kc, vc, hist, bt, nblk, bs, dtype="f32", layer0=0):
    """Pools holding the contiguous history rows of layers [layer0, L), written
    by the paged append itself (P = 0, N = longest history; rows past a
    sequence's own history are written too and never read)."""
    L, B, H, T, D = kc.shape
    kp, vp = _paged_canary(L, nblk, H, bs, D, dtype)
    n = int(hist.max())
    if n:
        kn = np.ascontiguousarray(kc[layer0:, :, :, :n])
        vn = np.ascontiguousarray(vc[layer0:, :, :, :n])
        oracle.paged_append(kp, vp, kn, vn, np.zeros(B, np.int32), bt, layer0=layer0, lib=lib)
    return kp, vp


def pin_paged_block_permutation(lib):
    """Which physical block holds a logical block changes nothing: paged
    decode over a shuffled table (blocks scattered through a larger pool,
    GQA, layers from layer0 = 1 on) equals the contiguous decode, outputs bit
    for bit, and the new rows land where the table says."""
    rng = _rng(62)
    L, B, Hkv, G, D, bs, mb = 3, 3, 2, 2, 8, 4, 6
    nblk = B * mb + 5
    hist = np.array([9, 0, 17], np.int32)
    kc, vc = _empty_cache(L, B, Hkv, bs * mb, D)
    _fill_history(kc, vc, hist, rng)
    bt = rng.permutation(nblk)[: B * mb].astype(np.int32).reshape(B, mb)
    kp, vp = _paged_from_history(lib, kc, vc, hist, bt, nblk, bs, layer0=1)
    N = 4
    q = rng.standard_normal((L - 1, B, Hkv * G, N, D), dtype=np.float32)
    k = rng.standard_normal((L - 1, B, Hkv, N, D), dtype=np.float32)
    v = rng.standard_normal((L - 1, B, Hkv, N, D), dtype=np.float32)
    ref = _decode(lib, kc, vc, q, k, v, hist, 0.3, layer0=1)
    oracle.paged_append(kp, vp, k, v, hist, bt, layer0=1, lib=lib)
    got = oracle.paged_attention(q, kp, vp, hist, bt, 0.3, layer0=1, lib=lib)
    assert np.array_equal(got, ref)
    assert synth.is_canary(kp[0]).all() and synth.is_canary(vp[0]).all()  # layer 0 untouched
    # the table's unused blocks are untouched
    unused = np.setdiff1d(np.arange(nblk), bt)
    assert synth.is_canary(kp[:, unused]).all() and synth.is_canary(vp[:, unused]).all()


def pin_paged_heads_are_independent(lib):
    """A block holds every KV head's rows: appending two KV heads at once
    leaves, for each head, the bytes that appending that head alone into a
    one-head pool leaves; attention per head is unchanged by the other head."""
    rng = _rng(63)
    L, B, Hkv, D, bs, mb = 1, 2, 2, 4, 4, 3
    nblk = 7
    bt = np.array([[5, 0, 3], [6, 2, 1]], np.int32)
    hist = np.array([5, 2], np.int32)
    N = 3
    k = rng.standard_normal((L, B, Hkv, N, D), dtype=np.float32)
    v = rng.standard_normal((L, B, Hkv, N, D), dtype=np.float32)
    q = rng.standard_normal((L, B, Hkv, N, D), dtype=np.float32)
    kp, vp = _paged_canary(L, nblk, Hkv, bs, D)
    oracle.paged_append(kp, vp, k, v, hist, bt, lib=lib)
    for h in range(Hkv):
        kh, vh = _paged_canary(L, nblk, 1, bs, D)
        oracle.paged_append(kh, vh, np.ascontiguousarray(k[:, :, h:h + 1]),
                            np.ascontiguousarray(v[:, :, h:h + 1]), hist, bt, lib=lib)
        assert np.array_equal(kp[:, :, h:h + 1].view(np.uint32), kh.view(np.uint32)), h
        assert np.array_equal(vp[:, :, h:h + 1].view(np.uint32), vh.view(np.uint32)), h
    # attention: the N rows as a prompt (positions 0 .. N-1), all heads at
    # once against each head alone
    h0 = np.zeros(B, np.int32)
    kp2, vp2 = _paged_canary(L, nblk, Hkv, bs, D)
    oracle.paged_append(kp2, vp2, k, v, h0, bt, lib=lib)
    full = oracle.paged_attention(q, kp2, vp2, h0, bt, 0.5, lib=lib)
    for h in range(Hkv):
        kh, vh = _paged_canary(L, nblk, 1, bs, D)
        oracle.paged_append(kh, vh, np.ascontiguousarray(k[:, :, h:h + 1]),
                            np.ascontiguousarray(v[:, :, h:h + 1]), h0, bt, lib=lib)
        one = oracle.paged_attention(np.ascontiguousarray(q[:, :, h:h + 1]), kh, vh, h0, bt, 0.5,
                                     lib=lib)
        assert np.array_equal(full[:, :, h:h + 1], one), h


def pin_paged_shared_prefix(lib):
    """Two sequences whose tables share the blocks of a common prefix give
    the outputs of two sequences holding private copies of it."""
    rng = _rng(64)
    L, Hkv, D, bs = 1, 1, 8, 4
    prefix = rng.standard_normal((L, 1, Hkv, 8, D), dtype=np.float32)  # two full blocks
    tails = rng.standard_normal((L, 2, Hkv, 3, D), dtype=np.float32)
    hist = np.array([11, 11], np.int32)
    N = 1
    q = rng.standard_normal((L, 2, Hkv, N, D), dtype=np.float32)
    k = rng.standard_normal((L, 2, Hkv, N, D), dtype=np.float32)
    v = rng.standard_normal((L, 2, Hkv, N, D), dtype=np.float32)
    outs = []
    for shared in (True, False):
        bt = np.array([[0, 1, 2], [0, 1, 3]], np.int32) if shared else \
            np.array([[0, 1, 2], [4, 5, 3]], np.int32)
        kp, vp = _paged_canary(L, 6, Hkv, bs, D)
        both = np.ascontiguousarray(np.concatenate([prefix, prefix], axis=1))
        oracle.paged_append(kp, vp, both, both * 0.5, np.zeros(2, np.int32), bt, lib=lib)
        oracle.paged_append(kp, vp, tails, tails * 0.5, np.array([8, 8], np.int32), bt, lib=lib)
        oracle.paged_append(kp, vp, k, v, hist, bt, lib=lib)
        outs.append(oracle.paged_attention(q, kp, vp, hist, bt, 0.35, lib=lib))
    assert np.array_equal(outs[0], outs[1])


def pin_paged_refusals(lib):
    """Positions past the table row, or a block id outside the pool, are
    refused and nothing is written."""
    kp, vp = _paged_canary(1, 4, 1, 4, 4)
    kn = np.ones((1, 2, 1, 2, 4), np.float32)
    # sequence 0 overflows its two-block row (7 + 2 > 8); the entry past the
    # row is the next row's first, a valid id, so only the capacity check
    # stands between the call and a write into block 2
    for hist, bt in ((np.array([7, 0], np.int32), np.array([[0, 1], [2, 3]], np.int32)),
                     (np.array([3, 0], np.int32), np.array([[0, 4], [2, 3]], np.int32)),
                     (np.array([3, 0], np.int32), np.array([[0, -1], [2, 3]], np.int32))):
        try:
            oracle.paged_append(kp, vp, kn, kn, hist, bt, lib=lib)
            raise AssertionError(f"accepted hist={hist} table={bt}")
        except oracle.OracleError:
            pass
        assert synth.is_canary(kp).all() and synth.is_canary(vp).all()


# ---------------------------------------------------------------- packed varlen prefill
# [KV-4] "Prefill 阶段": prompts packed along the token axis (token-major
# [n_layers, T, H, D], cu_seqlens boundaries), each with its own cached prefix.


def _pack(x, lens):
    """[n_layers, B, H, Smax, D] padded rows -> token-major packed
    [n_layers, sum(lens), H, D] (sequence b's first lens[b] rows)."""
    parts = [np.transpose(x[:, b, :, :n], (0, 2, 1, 3)) for b, n in enumerate(lens)]
    return np.ascontiguousarray(np.concatenate(parts, axis=1))


def _unpack(y, lens):
    """Inverse of _pack for outputs: list of [n_layers, H, lens[b], D]."""
    out, t = [], 0
    for n in lens:
        out.append(np.transpose(y[:, t:t + n], (0, 2, 1, 3)))
        t += n
    return out


def pin_varlen_equals_padded(lib):
    """Equal lengths and histories: the packed call leaves the cache bytes and
    gives the outputs (bit for bit) of append + attention on the padded
    layout with N = S."""
    rng = _rng(71)
    L, B, Hkv, G, D, T = 2, 3, 2, 2, 8, 24
    S, P = 5, 7
    hist = np.full(B, P, np.int32)
    kc, vc = _empty_cache(L, B, Hkv, T, D)
    _fill_history(kc, vc, hist, rng)
    q = rng.standard_normal((L, B, Hkv * G, S, D), dtype=np.float32)
    k = rng.standard_normal((L, B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((L, B, Hkv, S, D), dtype=np.float32)
    kc2, vc2 = kc.copy(), vc.copy()
    ref = _decode(lib, kc, vc, q, k, v, hist, 0.3)
    lens = [S] * B
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    got = oracle.prefill_varlen(kc2, vc2, _pack(q, lens), _pack(k, lens), _pack(v, lens), cu,
                                hist, 0.3, lib=lib)
    assert np.array_equal(kc2.view(np.uint32), kc.view(np.uint32))
    assert np.array_equal(vc2.view(np.uint32), vc.view(np.uint32))
    for b, ob in enumerate(_unpack(got, lens)):
        assert np.array_equal(ob, ref[:, b]), b


def pin_varlen_ragged_equals_per_sequence(lib):
    """Different lengths (one empty) and histories in one packed call equal
    each sequence's own padded append + attention, bit for bit; layer0 = 1."""
    rng = _rng(72)
    L, B, Hkv, G, D, T = 3, 4, 1, 3, 8, 32
    lens = [3, 0, 9, 1]
    hist = np.array([0, 5, 11, 30], np.int32)
    kc, vc = _empty_cache(L, B, Hkv, T, D)
    _fill_history(kc, vc, hist, rng)
    Smax = max(lens)
    q = rng.standard_normal((L - 1, B, Hkv * G, Smax, D), dtype=np.float32)
    k = rng.standard_normal((L - 1, B, Hkv, Smax, D), dtype=np.float32)
    v = rng.standard_normal((L - 1, B, Hkv, Smax, D), dtype=np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kc2, vc2 = kc.copy(), vc.copy()
    got = _unpack(oracle.prefill_varlen(kc2, vc2, _pack(q, lens), _pack(k, lens), _pack(v, lens),
                                        cu, hist, 0.45, layer0=1, lib=lib), lens)
    for b, n in enumerate(lens):
        kb, vb = np.ascontiguousarray(kc[:, b:b + 1]), np.ascontiguousarray(vc[:, b:b + 1])
        sl = (slice(None), slice(b, b + 1), slice(None), slice(0, n))
        ref = _decode(lib, kb, vb, np.ascontiguousarray(q[sl]), np.ascontiguousarray(k[sl]),
                      np.ascontiguousarray(v[sl]), hist[b:b + 1], 0.45, layer0=1)
        assert np.array_equal(got[b], ref[:, 0]), b
        assert np.array_equal(kc2[:, b:b + 1].view(np.uint32), kb.view(np.uint32)), b
        assert np.array_equal(vc2[:, b:b + 1].view(np.uint32), vb.view(np.uint32)), b


def pin_varlen_refusals(lib):
    """A sequence whose history plus new tokens passes Tmax, or boundaries
    that do not start at 0 or go backwards, are refused; nothing is written."""
    kc, vc = _empty_cache(1, 2, 1, 8, 4)
    q = np.ones((1, 6, 1, 4), np.float32)
    for cu, hist in (([0, 2, 6], [1, 5]),     # 5 + 4 > 8
                     ([1, 2, 6], [0, 0]),     # does not start at 0
                     ([0, 4, 3], [0, 0])):    # goes backwards (T = 3 rows given)
        cu = np.array(cu, np.int32)
        T = int(cu[-1])
        try:
            oracle.prefill_varlen(kc, vc, q[:, :T], q[:, :T], q[:, :T], cu,
                                  np.array(hist, np.int32), 0.5, lib=lib)
            raise AssertionError(f"accepted cu={cu.tolist()} hist={hist}")
        except (oracle.OracleError, ValueError):
            pass
        assert synth.is_canary(kc).all() and synth.is_canary(vc).all()


def pin_paged_varlen_equals_contiguous(lib):
    """The packed prefill into a paged cache (shuffled table) gives the
    contiguous packed prefill's outputs bit for bit, and leaves the new rows
    where a following decode step reads them: that step's outputs match too."""
    rng = _rng(73)
    L, B, Hkv, G, D, bs, mb = 2, 3, 2, 2, 8, 4, 8
    nblk = B * mb + 3
    lens = [6, 0, 9]
    hist = np.array([5, 12, 0], np.int32)
    kc, vc = _empty_cache(L, B, Hkv, bs * mb, D)
    _fill_history(kc, vc, hist, rng)
    bt = rng.permutation(nblk)[: B * mb].astype(np.int32).reshape(B, mb)
    kp, vp = _paged_from_history(lib, kc, vc, hist, bt, nblk, bs)
    T = sum(lens)
    q = rng.standard_normal((L, T, Hkv * G, D), dtype=np.float32)
    k = rng.standard_normal((L, T, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((L, T, Hkv, D), dtype=np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ref = oracle.prefill_varlen(kc, vc, q, k, v, cu, hist, 0.4, lib=lib)
    got = oracle.paged_prefill_varlen(kp, vp, q, k, v, cu, hist, bt, 0.4, lib=lib)
    assert np.array_equal(got, ref)
    h2 = hist + np.array(lens, np.int32)
    q1 = rng.standard_normal((L, B, Hkv * G, 1, D), dtype=np.float32)
    k1 = rng.standard_normal((L, B, Hkv, 1, D), dtype=np.float32)
    v1 = rng.standard_normal((L, B, Hkv, 1, D), dtype=np.float32)
    ref1 = _decode(lib, kc, vc, q1, k1, v1, h2, 0.4)
    oracle.paged_append(kp, vp, k1, v1, h2, bt, lib=lib)
    got1 = oracle.paged_attention(q1, kp, vp, h2, bt, 0.4, lib=lib)
    assert np.array_equal(got1, ref1)


ALL_PINS = [
    pin_cache_bytes_golden,
    pin_single_key_exact,
    pin_zero_query_counts_visible_keys,
    pin_uniform_keys_give_mean,
    pin_one_hot_selects_value,
    pin_two_keys_sigmoid,
    pin_zero_and_negative_scale,
    pin_matches_torch_sdpa,
    pin_cached_equals_recompute,
    pin_chunk_invariance,
    pin_permutation,
    pin_gqa_equals_repeated_mha,
    pin_append_positions_and_canaries,
    pin_bf16_decode_exact,
    pin_paged_identity_is_contiguous,
    pin_paged_block_permutation,
    pin_paged_heads_are_independent,
    pin_paged_shared_prefix,
    pin_paged_refusals,
    pin_varlen_equals_padded,
    pin_varlen_ragged_equals_per_sequence,
    pin_varlen_refusals,
    pin_paged_varlen_equals_contiguous,
]
