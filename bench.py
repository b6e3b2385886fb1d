"""Benchmark of the KV-cache attention hot path on one MI355X.

One step = the whole decode hot path for GPT-2 Small at context 1024: the new
token's K/V rows written into all 12 layers' caches and the attention of the
new query rows against the 1024 cached keys, issued as one kvc_decode_step:
one kernel of one workgroup per query row (144 rows), each streaming its
row's 1023 cached keys, merging them with the new key and appending its row.
Inputs: fp32, B=1, 12 layers x 12 heads, D=64, history P=1023, N(0,1) from a
fixed seed.

Timing: steps are captured in a HIP graph (torch.cuda.CUDAGraph) and replayed;
HIP events on the capture/replay stream bracket exactly --steps steps, five
times after a warm-up, and every figure is the median of the five samples
(min and max reported for the headline).  Eight
cache replicas (604 MB in total, more than twice the 256 MB Infinity Cache)
rotate step by step, so every step streams its K/V from HBM rather than from
a cache level.  The oracle (CPU, double precision) is timed beside it on a
bounded sample of the same steps, and the timed outputs are checked against it.

Prints ONE JSON line.  Extra entries: per-kernel times, the per-layer and
eager launch modes, the decode sweep over history lengths, chunked and batched
decode, and the prefill TFLOP/s with its matrix-core fraction.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                    # MI355X HBM3E
# A plain streaming read of the step's 75.5 MB (2,304 workgroups, each 32 KB
# of 16-byte loads issued at once, cold, back-to-back launches) measured on
# an MI355X at 12.37 us: the most this step's bytes can move at, as a fraction
# of HBM_PEAK_GBS.
PLAIN_READ_FRAC = 0.763
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}   # dense matrix-core peaks
METRIC = "decode attention µs/step + achieved HBM GB/s at T=1024; prefill TFLOP/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_traffic.txt")
DECODE_SOURCES = [os.path.join(ROOT, "transformer_kv_cache_amd", "csrc", f)
                  for f in ("kvc_decode.hip", "kvc_device.h", "kvc_internal.h", "kvc_api.hip")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def elem_bytes(dtype):
    return 4 if dtype == "f32" else 2


def kv_read_bytes(w, N):
    """Every visible K and V row read once."""
    return 2 * w.L * w.Hkv * w.D * elem_bytes(w.dtype) * int(np.sum(w.hist + N))


def q_bytes(w, N):
    """One of q (read) or o (written)."""
    return w.L * w.B * w.Hq * N * w.D * elem_bytes(w.dtype)


def new_rows_bytes(w, N):
    """The N new K and V rows, once."""
    return 2 * w.L * w.B * w.Hkv * N * w.D * elem_bytes(w.dtype)


def decode_bytes(w, N):
    """Algorithmic bytes of one attn_decode call: K/V once, q and o once."""
    return kv_read_bytes(w, N) + 2 * q_bytes(w, N)


def append_bytes(w, N):
    """Algorithmic bytes of one append: new K/V rows read once, written once."""
    return 2 * new_rows_bytes(w, N)


def decode_source_hash():
    h = hashlib.sha256()
    for p in DECODE_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 PMC summary,
    if it was measured on the current decode kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("decode_source_sha256") != decode_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"].split()[0])
    except (KeyError, ValueError, IndexError):
        return None


SAMPLES = 5  # timed samples per figure; the figure is their median


class GraphTimer:
    """Capture `fn(r)` for r in a rotation into HIP graphs and time exactly
    `count` calls with events on the replay stream, SAMPLES times; `time`
    returns the median (microseconds per call) and leaves every sample in
    `samples`."""

    def __init__(self, torch, fn, rotate):
        self.torch = torch
        self.rotate = rotate
        self.fn = fn
        self.graphs = {}
        self.samples = []

    def _graph(self, n):
        if n not in self.graphs:
            torch = self.torch
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for r in range(n):
                        self.fn(r)
            torch.cuda.current_stream().wait_stream(s)
            self.graphs[n] = g
        return self.graphs[n]

    def time(self, count, warm=2):
        torch = self.torch
        full, rem = divmod(count, self.rotate)
        g_full = self._graph(self.rotate)
        g_rem = self._graph(rem) if rem else None
        for _ in range(warm):
            g_full.replay()
        torch.cuda.synchronize()
        self.samples = []
        for _ in range(SAMPLES):
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            start.record()
            for _ in range(full):
                g_full.replay()
            if g_rem is not None:
                g_rem.replay()
            end.record()
            torch.cuda.synchronize()
            self.samples.append(start.elapsed_time(end) * 1e3 / count)  # microseconds per call
        return float(np.median(self.samples))


def replicate(torch, arr_dev, n):
    return [arr_dev] + [arr_dev.clone() for _ in range(n - 1)]


def bench_decode(torch, K, w, steps, warmup, rotate, per_layer=False, eager=False):
    """Time the decode step (append + attention) of workload `w` (one step
    of N rows).  Returns a dict of timings and the device state of replica 0."""
    from transformer_kv_cache_amd.hostio import to_dev, torch_dtype
    q_np, k_np, v_np = w.steps[0]
    N = q_np.shape[3]
    base_k, base_v = to_dev(w.k_cache), to_dev(w.v_cache)
    dt = torch_dtype(w.dtype)
    caches = [K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, dt, k=kk, v=vv)
              for kk, vv in zip(replicate(torch, base_k, rotate), replicate(torch, base_v, rotate))]
    qs = replicate(torch, to_dev(q_np), rotate)
    kns = replicate(torch, to_dev(k_np), rotate)
    vns = replicate(torch, to_dev(v_np), rotate)
    outs = [torch.empty_like(qs[0]) for _ in range(rotate)]
    wss = [K.new_decode_workspace(caches[0], w.L, w.Hq, N) for _ in range(rotate)]
    hist = w.hist.copy()

    def step(r):
        K.decode_step(caches[r], qs[r], kns[r], vns[r], hist, scale=w.scale, out=outs[r],
                      workspace=wss[r])

    def step_two_calls(r):
        K.append(caches[r], kns[r], vns[r], hist)
        K.attn_decode(caches[r], qs[r], hist, scale=w.scale, out=outs[r], workspace=wss[r])

    def decode_only(r):
        K.attn_decode(caches[r], qs[r], hist, scale=w.scale, out=outs[r], workspace=wss[r])

    def split_only(r):
        K.decode_split(caches[r], qs[r], hist, kns[r], vns[r], scale=w.scale, out=outs[r],
                       workspace=wss[r])

    def combine_only(r):
        K.decode_combine(caches[r], qs[r], hist, kns[r], vns[r], scale=w.scale, out=outs[r],
                         workspace=wss[r])

    def append_only(r):
        K.append(caches[r], kns[r], vns[r], hist)

    for i in range(warmup):
        step(i % rotate)
    torch.cuda.synchronize()
    res = {}
    t_step = GraphTimer(torch, step, rotate)
    res["step_us"] = t_step.time(steps)
    res["step_us_min"], res["step_us_max"] = min(t_step.samples), max(t_step.samples)
    res["split_us"] = GraphTimer(torch, split_only, rotate).time(steps)
    res["combine_us"] = GraphTimer(torch, combine_only, rotate).time(steps)
    res["two_call_step_us"] = GraphTimer(torch, step_two_calls, rotate).time(steps)
    res["attn_decode_us"] = GraphTimer(torch, decode_only, rotate).time(steps)
    res["append_us"] = GraphTimer(torch, append_only, rotate).time(steps)
    # the fused step reads the new rows from k_new/v_new and writes them once
    res["step_bytes"] = decode_bytes(w, N) + new_rows_bytes(w, N)
    # split pass alone (kvc_decode_split: the split kernel without a merge; the
    # one-call step of one query row per KV head may run the row kernel instead).
    # One query row per KV head: K/V of the cached keys [0, P) and q read;
    # the merge adds key P from k_new/v_new and appends it.  Several rows per
    # KV head (multi-row kernels): K/V of all keys (new rows from
    # k_new/v_new) and q read, new rows written.
    if (w.Hq // w.Hkv) * N == 1:
        res["split_bytes"] = kv_read_bytes(w, 0) + q_bytes(w, N)
    else:
        res["split_bytes"] = kv_read_bytes(w, N) + q_bytes(w, N) + new_rows_bytes(w, N)
    res["split_gbs"] = res["split_bytes"] / res["split_us"] / 1e3
    res["step_gbs"] = res["step_bytes"] / res["step_us"] / 1e3
    res["attn_decode_bytes"] = decode_bytes(w, N)
    res["attn_decode_gbs"] = res["attn_decode_bytes"] / res["attn_decode_us"] / 1e3
    if eager:
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            step(i % rotate)
        end.record()
        torch.cuda.synchronize()
        res["eager_step_us"] = start.elapsed_time(end) * 1e3 / steps
    if per_layer:
        ws1 = [K.new_decode_workspace(caches[0], 1, w.Hq, N) for _ in range(rotate)]

        def step_per_layer(r):
            for l in range(w.L):
                K.decode_step(caches[r], qs[r][l:l + 1], kns[r][l:l + 1], vns[r][l:l + 1], hist,
                              scale=w.scale, out=outs[r][l:l + 1], layer0=l, workspace=ws1[r])

        for i in range(warmup):
            step_per_layer(i % rotate)
        res["perlayer_step_us"] = GraphTimer(torch, step_per_layer, rotate).time(steps)
    torch.cuda.synchronize()
    res["_out0"] = outs[0]
    return res


def bench_paged_decode(torch, K, w, steps, warmup, rotate):
    """Time the paged decode step of paged workload `w` (one step of N rows),
    pools and inputs rotated over `rotate` replicas like bench_decode."""
    from transformer_kv_cache_amd.hostio import to_dev, torch_dtype
    q_np, k_np, v_np = w.steps[0]
    N = q_np.shape[3]
    dt = torch_dtype(w.dtype)
    base_k, base_v = to_dev(w.k_pool), to_dev(w.v_pool)
    caches = [K.PagedKVCache(w.L, w.num_blocks, w.Hkv, w.block_size, w.D, dt, k=kk, v=vv)
              for kk, vv in zip(replicate(torch, base_k, rotate), replicate(torch, base_v, rotate))]
    qs = replicate(torch, to_dev(q_np), rotate)
    kns = replicate(torch, to_dev(k_np), rotate)
    vns = replicate(torch, to_dev(v_np), rotate)
    bt = torch.from_numpy(w.block_table).cuda()
    outs = [torch.empty_like(qs[0]) for _ in range(rotate)]
    wss = [K.new_paged_decode_workspace(caches[0], w.L, w.B, w.Hq, N, w.max_blocks)
           for _ in range(rotate)]
    hist = w.hist.copy()

    def step(r):
        K.paged_decode_step(caches[r], qs[r], kns[r], vns[r], hist, bt, scale=w.scale,
                            out=outs[r], workspace=wss[r])

    for i in range(warmup):
        step(i % rotate)
    torch.cuda.synchronize()
    res = {"step_us": GraphTimer(torch, step, rotate).time(steps)}
    # algorithmic bytes as for the contiguous step, plus the block-table reads
    e = elem_bytes(w.dtype)
    kv = 2 * w.L * w.Hkv * w.D * e * int(np.sum(w.hist + N))
    qo = 2 * w.L * w.B * w.Hq * N * w.D * e
    new_rows = 2 * w.L * w.B * w.Hkv * N * w.D * e
    res["step_bytes"] = kv + qo + new_rows
    res["step_gbs"] = res["step_bytes"] / res["step_us"] / 1e3
    res["block_size"] = w.block_size
    return res


def bench_prefill(torch, K, S, dtype, reps):
    from transformer_kv_cache_amd.hostio import to_dev, torch_dtype
    from transformer_kv_cache_amd import synth
    w = synth.causal_prefill(S, dtype, seed=7)
    dt = torch_dtype(dtype)
    # replicas so that at least 512 MB of inputs, outputs and cache rows are
    # touched between two uses of one, twice the 256 MB Infinity Cache
    touched = 6 * w.L * w.Hq * S * w.D * elem_bytes(dtype)
    rotate = max(4, -(-512_000_000 // touched))
    q0, k0, v0 = (to_dev(a) for a in w.prefill)
    qs, ks, vs = (replicate(torch, t, rotate) for t in (q0, k0, v0))
    caches = [K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, dt) for _ in range(rotate)]
    outs = [torch.empty_like(q0) for _ in range(rotate)]

    def call(r):
        K.attn_prefill(caches[r], qs[r], ks[r], vs[r], scale=w.scale, out=outs[r])

    for r in range(rotate):
        call(r)
    us = GraphTimer(torch, call, rotate).time(reps)
    flops = 4 * w.D * w.L * w.Hq * S * (S + 1) // 2
    tflops = flops / us / 1e6
    e = elem_bytes(dtype)
    hbm_bytes = 6 * w.L * w.Hq * S * w.D * e  # q, k, v read; o and the K/V cache rows written
    return {"S": S, "dtype": dtype, "us": us, "tflops": tflops,
            "mfma_frac": tflops / MFMA_PEAK_TFLOPS[dtype],
            "hbm_gbs": hbm_bytes / us / 1e3, "algorithmic_flops": flops}


def bench_generation_c1(torch, K, reps=200):
    """The single-layer generation (prompt of 16 prefilled, then four
    single-token fused decode steps, one layer, Tmax=32): the whole sequence
    captured in one graph per replica, timed per sequence."""
    from transformer_kv_cache_amd.hostio import to_dev
    from transformer_kv_cache_amd import synth
    w = synth.single_layer_generation(seed=0)
    rotate = 2
    caches = [K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, torch.float32) for _ in range(rotate)]
    pre = [tuple(to_dev(a) for a in w.prefill) for _ in range(rotate)]
    steps = [[tuple(to_dev(a) for a in st) for st in w.steps] for _ in range(rotate)]
    wss = [K.new_decode_workspace(caches[0], w.L, w.Hq, 1) for _ in range(rotate)]
    outs = [torch.empty_like(pre[0][0]) for _ in range(rotate)]
    step_outs = [torch.empty_like(steps[0][0][0]) for _ in range(rotate)]
    S = w.prefill[0].shape[3]

    def sequence(r):
        q, k, v = pre[r]
        K.attn_prefill(caches[r], q, k, v, scale=w.scale, out=outs[r])
        hist = np.full(w.B, S, dtype=np.int32)
        for (qs, ks, vs) in steps[r]:
            K.decode_step(caches[r], qs, ks, vs, hist, scale=w.scale, out=step_outs[r],
                          workspace=wss[r])
            hist += 1

    for r in range(rotate):
        sequence(r)
    us = GraphTimer(torch, sequence, rotate).time(reps)
    return {"sequence_us": us, "prefill_len": S, "decode_steps": len(w.steps)}


def bench_varlen_prefill(torch, K, w, reps, rotate=4, block_size=0):
    """Time one packed variable-length prefill (synth.VarlenWorkload); with
    block_size > 0 the same rows sit in block pools behind a shuffled table
    and the paged entry point runs."""
    from transformer_kv_cache_amd.hostio import to_dev, torch_dtype
    from transformer_kv_cache_amd import synth
    dt = torch_dtype(w.dtype)
    qs, ks, vs = (replicate(torch, to_dev(a), rotate) for a in (w.q, w.k, w.v))
    outs = [torch.empty_like(qs[0]) for _ in range(rotate)]
    if block_size:
        kp, vp, table = synth.paged_from_contiguous(w.k_cache, w.v_cache, block_size, seed=11)
        bt = torch.from_numpy(table).cuda()
        caches = [K.PagedKVCache(w.L, kp.shape[1], w.Hkv, block_size, w.D, dt, k=kk, v=vv)
                  for kk, vv in zip(replicate(torch, to_dev(kp), rotate),
                                    replicate(torch, to_dev(vp), rotate))]

        def call(r):
            K.paged_attn_prefill_varlen(caches[r], qs[r], ks[r], vs[r], w.cu_seqlens, w.hist, bt,
                                        scale=w.scale, out=outs[r])
    else:
        caches = [K.KVCache(w.L, w.B, w.Hkv, w.Tmax, w.D, dt, k=kk, v=vv) for kk, vv in
                  zip(replicate(torch, to_dev(w.k_cache), rotate),
                      replicate(torch, to_dev(w.v_cache), rotate))]

        def call(r):
            K.attn_prefill_varlen(caches[r], qs[r], ks[r], vs[r], w.cu_seqlens, w.hist,
                                  scale=w.scale, out=outs[r])

    for r in range(rotate):
        call(r)
    us = GraphTimer(torch, call, rotate).time(reps)
    lens = np.diff(w.cu_seqlens).astype(np.int64)
    hist = w.hist.astype(np.int64)
    # new token i of sequence b attends to P_b + i + 1 positions
    flops = int(4 * w.D * w.L * w.Hq * np.sum(lens * hist + lens * (lens + 1) // 2))
    tflops = flops / us / 1e6
    return {"us": us, "tflops": tflops, "mfma_frac": tflops / MFMA_PEAK_TFLOPS[w.dtype],
            "algorithmic_flops": flops, "lengths": lens.tolist(), "history": hist.tolist()}


def bench_gpt2(torch, contexts=(128, 512, 1000), reps=20):
    """Per-token latency of a GPT-2 Small-shaped decoder (synthetic fp32
    weights, batch 1) at each context length T: the cached step (token T-1
    through the decode entry point over T-1 cached positions, every layer,
    then the output projection of the last position) and the recomputing
    step (all T tokens through the prefill entry point), each captured in a
    HIP graph and replayed."""
    from transformer_kv_cache_amd import synth
    from transformer_kv_cache_amd.gpt2 import GPT2
    w = synth.gpt2_weights(seed=0)
    m = GPT2(w)
    ids = torch.from_numpy(synth.token_ids(1, max(contexts), w.V)).cuda()
    cache, scratch = m.new_cache(), m.new_cache()
    res = {}
    for T in contexts:
        m.forward(ids[:T - 1], cache, 0, last_only=True)
        tok = ids[T - 1:T].clone()
        full = ids[:T].clone()

        def cached(r):
            m.forward(tok, cache, T - 1, last_only=True)

        def recompute(r):
            m.forward(full, scratch, 0, last_only=True)

        cached(0)
        recompute(0)
        torch.cuda.synchronize()
        c_us = GraphTimer(torch, cached, 1).time(reps)
        r_us = GraphTimer(torch, recompute, 1).time(reps)
        res[f"T{T}"] = {"cached_ms_per_token": round(c_us / 1e3, 4),
                        "recompute_ms_per_token": round(r_us / 1e3, 4),
                        "speedup": round(r_us / c_us, 2)}
    # the pages' second measurement: a 1016-token greedy generation, here with
    # the whole token step captured once (device lengths) and replayed
    prompt = synth.token_ids(2, 8, w.V).tolist()
    toks, ms = m.generate_graph(prompt, 1016)
    res["generate_1016_tokens_cached_graph"] = {"prompt": len(prompt), "tokens": len(toks),
                                                "ms_per_token": round(ms, 4),
                                                "seconds": round(ms * (len(toks) - 1) / 1e3, 3)}
    res["model"] = "12 layers, width 768, 12 heads, vocabulary 50257, fp32, batch 1, synthetic weights"
    return res


def cpu_baseline(w, target_s, max_steps=100000):
    """The oracle, as it stands, on a bounded sample of the headline step:
    append + attention for all 12 layers, repeated until ~target_s seconds."""
    import oracle
    q, k, v = w.steps[0]
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    threads = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        threads = min(threads, int(omp))
    oracle.set_threads(threads)
    out = None
    n = 0
    t0 = time.perf_counter()
    while n < max_steps:
        oracle.append(kc, vc, k, v, w.hist)
        out = oracle.attention(q, kc, vc, w.hist, w.scale)
        n += 1
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    res = {"seconds": dt, "steps": n, "threads": oracle.max_threads(), "us_per_step": dt / n * 1e6,
           "out": out}
    # the same steps on one thread, over a fifth of the time
    oracle.set_threads(1)
    n1 = 0
    t0 = time.perf_counter()
    while n1 < max_steps:
        oracle.append(kc, vc, k, v, w.hist)
        oracle.attention(q, kc, vc, w.hist, w.scale)
        n1 += 1
        if time.perf_counter() - t0 >= target_s / 5:
            break
    res["one_thread_us_per_step"] = (time.perf_counter() - t0) / n1 * 1e6
    oracle.set_threads(threads)
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=8, help="cache replicas cycled through")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="length of the oracle's timed CPU sample")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the sweep, chunked/batched decode and prefill extras")
    ap.add_argument("--only", choices=["prefill", "multirow", "gpt2"], default=None,
                    help="time only the causal prefill workloads, the multi-row decode "
                         "workloads (chunked, batched MHA / GQA) or the GPT-2 decoder, print them "
                         "and exit (used for rocprofv3 counter runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (used to scale "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path is per-GPU: each GPU would run it on its own shard)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * 1024 * 1024
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 4}), flush=True)
        return
    from transformer_kv_cache_amd import kvcache as K, synth
    from transformer_kv_cache_amd.hostio import to_host

    if not os.path.exists(K.LIB_PATH):
        from transformer_kv_cache_amd import build
        build.build(verbose=False)
    K.library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.only == "prefill":
        pre = []
        for S in (256, 1024):
            for dtype in ("f32", "bf16"):
                log(f"prefill S={S} {dtype}")
                pre.append({"S": S, "dtype": dtype, **bench_prefill(torch, K, S, dtype, 40)})
        print(json.dumps({"prefill_12layer": pre}), flush=True)
        return
    if args.only == "gpt2":
        log("GPT-2 Small-shaped decoder: cached vs recomputed per-token latency")
        print(json.dumps({"gpt2_small_cached_vs_recompute": bench_gpt2(torch)}), flush=True)
        return
    if args.only == "multirow":
        res = {}
        for name, wm in (("chunked_decode_P1000_N8", synth.chunked_decode(1000, 8, seed=1)),
                         ("batched_decode_bf16_mha12_D64", synth.batched_decode(seed=3, gqa=False)),
                         ("batched_decode_bf16_gqa32q8kv_D128", synth.batched_decode(seed=3, gqa=True))):
            log(name)
            r = bench_decode(torch, K, wm, args.steps, args.warmup, 4)
            r.pop("_out0")
            res[name] = r
        print(json.dumps(res), flush=True)
        return

    log("headline: 12-layer fp32 decode at T=1024")
    w = synth.decode_12layer(1023, seed=0)
    head = bench_decode(torch, K, w, args.steps, args.warmup, args.rotate, per_layer=True,
                        eager=True)
    out0 = to_host(head.pop("_out0"))

    log("cpu baseline (oracle)")
    cpu = cpu_baseline(w, args.cpu_seconds)
    max_err = float(np.max(np.abs(out0.astype(np.float64) - cpu["out"])))
    if not max_err <= 1e-4:
        raise SystemExit(f"timed outputs differ from the oracle: max abs error {max_err}")
    step_bytes = head["step_bytes"]

    extras = {}
    if not args.headline_only:
        sweep = {}
        for P in (128, 512, 1000):
            log(f"sweep P={P}")
            r = bench_decode(torch, K, synth.decode_12layer(P, seed=P), args.steps, args.warmup,
                             args.rotate)
            r.pop("_out0")
            sweep[f"P{P}"] = {k: round(v, 3) for k, v in r.items()}
        sweep["P1023"] = {k: round(v, 3) for k, v in head.items()}
        extras["decode_sweep_fp32_12layer"] = sweep
        log("chunked decode P=1000 N=8")
        r = bench_decode(torch, K, synth.chunked_decode(1000, 8, seed=1), args.steps, args.warmup,
                         args.rotate)
        r.pop("_out0")
        extras["chunked_decode_P1000_N8"] = {k: round(v, 3) for k, v in r.items()}
        for gqa in (False, True):
            name = "batched_decode_bf16_" + ("gqa32q8kv_D128" if gqa else "mha12_D64")
            log(name)
            wb = synth.batched_decode(seed=3, gqa=gqa)
            r = bench_decode(torch, K, wb, args.steps, args.warmup, 4)
            r.pop("_out0")
            r = {k: round(v, 3) for k, v in r.items()}
            r["lengths"] = (wb.hist + 1).tolist()
            extras[name] = r
        # One GPU's share of the GQA workload under 8-way tensor parallelism
        # over the KV heads (1 KV head, 4 query heads, same lengths): what
        # each of eight GPUs would run, with no exchange on this path.
        # (an eighth of the bytes: 24 replicas keep the rotation past 512 MB)
        log("batched_decode_bf16_gqa_tp8_shard")
        r = bench_decode(torch, K, synth.batched_decode(seed=3, gqa=True, tp=8), args.steps,
                         args.warmup, 24)
        r.pop("_out0")
        extras["batched_decode_bf16_gqa_tp8_shard"] = {k: round(v, 3) for k, v in r.items()}
        paged = {}
        for bs in (16, 64):
            log(f"paged decode 12-layer fp32 T=1024, block size {bs}")
            r = bench_paged_decode(torch, K, synth.paged_decode_12layer(1023, block_size=bs),
                                   args.steps, args.warmup, args.rotate)
            paged[f"fp32_12layer_T1024_bs{bs}"] = {k: round(v, 3) for k, v in r.items()}
        for gqa in (False, True):
            name = "bf16_" + ("gqa32q8kv_D128" if gqa else "mha12_D64") + "_bs16"
            log(f"paged decode {name}")
            wp = synth.paged_batched_decode(seed=3, gqa=gqa, block_size=16)
            r = {k: round(v, 3) for k, v in
                 bench_paged_decode(torch, K, wp, args.steps, args.warmup, 4).items()}
            r["lengths"] = (wp.hist + 1).tolist()
            paged[name] = r
        extras["paged_decode"] = paged
        pre = []
        for dtype in ("f32", "bf16"):
            for S in (256, 1024):
                log(f"prefill S={S} {dtype}")
                pre.append({k: (round(v, 4) if isinstance(v, float) else v)
                            for k, v in bench_prefill(torch, K, S, dtype, 40).items()})
        extras["prefill_12layer"] = pre
        log("single-layer generation (prompt 16 + 4 decode steps)")
        extras["single_layer_generation"] = {k: (round(v, 3) if isinstance(v, float) else v)
                                             for k, v in bench_generation_c1(torch, K).items()}
        varlen = {}
        for gqa in (False, True):
            name = "bf16_" + ("gqa32q8kv_D128" if gqa else "mha12_D64") + "_B8"
            log(f"varlen prefill {name}")
            wv = synth.varlen_prefill_batch(seed=5, gqa=gqa)
            r = bench_varlen_prefill(torch, K, wv, 20)
            varlen[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
            log(f"varlen prefill {name}, paged cache, block size 16")
            r = bench_varlen_prefill(torch, K, wv, 20, block_size=16)
            varlen[name + "_paged_bs16"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                            for k, v in r.items()}
        extras["prefill_varlen_12layer"] = varlen
        log("GPT-2 Small-shaped decoder: cached vs recomputed per-token latency")
        extras["gpt2_small_cached_vs_recompute"] = bench_gpt2(torch)

    step_us = head["step_us"]
    traffic = read_traffic()
    line = {
        "metric": METRIC,
        "value": round(step_bytes / step_us / 1e3, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic N(0,1), numpy PCG64 seed 0",
        "config": {"workload": "GPT-2 Small KV-cache decode step, 12 layers, fp32, B=1, H=12, "
                               "D=64, Tmax=1024, history 1023 + 1 new token (T=1024)",
                   "layers": 12, "batch": 1, "heads": 12, "head_dim": 64, "context": 1024,
                   "step": "kvc_decode_step: one kernel -- one workgroup per query row streams "
                           "the row's cached keys, merges them with the new key and appends "
                           "its row",
                   "rotating_cache_replicas": args.rotate},
        "decode_us_per_step": round(step_us, 3),
        "decode_us_per_step_min": round(head["step_us_min"], 3),
        "decode_us_per_step_max": round(head["step_us_max"], 3),
        "step_bytes": step_bytes,
        # the step is one kernel launch: its algorithmic bytes over its time
        "roofline": {"bound": "hbm", "achieved": round(step_bytes / step_us / 1e3, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_bytes / step_us / 1e3 / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "decode_row_kernel<f32,D64,KPL8,128 lanes> (the whole step in one "
                               "launch of 144 workgroups: each streams keys [0,1023) of its "
                               "row, adds key 1023 and appends its row)",
                     "launch_us": round(step_us, 3),
                     "algorithmic_bytes": step_bytes,
                     "split_pass_only_us": round(head["split_us"], 3),
                     "split_pass_only_frac": round(head["split_gbs"] / HBM_PEAK_GBS, 4),
                     "plain_read_ceiling_frac": PLAIN_READ_FRAC},
        "cpu_baseline": {"value": round(step_bytes / cpu["us_per_step"] / 1e3, 3), "unit": "GB/s",
                         "cores": cpu["threads"], "kind": "oracle",
                         "sample": f"{cpu['steps']} full decode steps (append + attention, all 12 "
                                   f"layers) of the same workload, {cpu['seconds']:.1f} s",
                         "us_per_step": round(cpu["us_per_step"], 1),
                         "one_thread_us_per_step": round(cpu["one_thread_us_per_step"], 1),
                         "gpu_speedup": round(cpu["us_per_step"] / step_us, 1),
                         "cpu_model": cpu_model()},
        "parity_max_abs_err": max_err,
        "modes": {"graph_fused12_step_us": round(step_us, 3),
                  "graph_two_call_step_us": round(head["two_call_step_us"], 3),
                  "graph_perlayer_step_us": round(head["perlayer_step_us"], 3),
                  "eager_fused12_step_us": round(head["eager_step_us"], 3),
                  "attn_decode_us": round(head["attn_decode_us"], 3),
                  "append_us": round(head["append_us"], 3)},
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
