"""Seeded input generators: bf16 rounding against torch, determinism, and the
shapes and length draws of the five workloads."""
import numpy as np
import torch

from transformer_kv_cache_amd import synth


def test_bf16_rne_matches_torch_all_high_halves():
    """Every high half with low halves covering exact values, ties, near-ties
    and the largest low half; NaN inputs only need to stay NaN."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    x = bits.view(np.float32)
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.isnan(synth.bf16_bits_to_f32(ours[nan])).all()


def test_bf16_widening_is_exact():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = synth.bf16_bits_to_f32(b)
    back = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    fin = ~np.isnan(f)
    assert np.array_equal(f[fin].view(np.uint32), back[fin].view(np.uint32))


def test_generators_are_deterministic_and_shaped():
    a = synth.single_layer_generation(seed=3)
    b = synth.single_layer_generation(seed=3)
    assert np.array_equal(a.prefill[0], b.prefill[0])
    assert a.k_cache.shape == (1, 1, 12, 32, 64) and synth.is_canary(a.k_cache).all()
    assert a.prefill[0].shape == (1, 1, 12, 16, 64) and len(a.steps) == 4
    c = synth.make_workload("x", seed=0, dtype="bf16", L=2, B=3, Hq=4, Hkv=2, D=8,
                            Tmax=16, draw_lengths=(1, 16), step_lens=(1,))
    assert ((c.hist >= 0) & (c.hist <= 15)).all()
    for bb in range(3):
        p = int(c.hist[bb])
        assert not synth.is_canary(c.k_cache[:, bb, :, :p]).any()
        assert synth.is_canary(c.k_cache[:, bb, :, p:]).all()
    assert c.steps[0][0].shape == (2, 3, 4, 1, 8) and c.steps[0][1].shape == (2, 3, 2, 1, 8)


def test_paged_from_contiguous_round_trip():
    w = synth.make_workload("rt", seed=3, dtype="bf16", L=2, B=3, Hq=2, Hkv=2, D=64, Tmax=64,
                            hist=[5, 0, 63])
    kp, vp, table = synth.paged_from_contiguous(w.k_cache, w.v_cache, 16, seed=1)
    assert kp.shape == (2, 3 * 4 + 3, 2, 16, 64) and table.shape == (3, 4)
    assert len(np.unique(table)) == table.size
    for b in range(3):
        for t in range(64):
            assert np.array_equal(kp[:, table[b, t // 16], :, t % 16], w.k_cache[:, b, :, t])
            assert np.array_equal(vp[:, table[b, t // 16], :, t % 16], w.v_cache[:, b, :, t])
    spare = np.setdiff1d(np.arange(kp.shape[1]), table)
    assert synth.is_canary(kp[:, spare]).all() and synth.is_canary(vp[:, spare]).all()


def test_tensor_parallel_shard_keeps_the_lengths():
    """One GPU's share of the GQA workload under tp-way tensor parallelism:
    8/tp KV heads and 32/tp query heads, the same drawn lengths; tp must
    divide the KV heads and only applies to the GQA workload."""
    import pytest
    full = synth.batched_decode(seed=3, gqa=True, L=2)
    for tp in (2, 8):
        s = synth.batched_decode(seed=3, gqa=True, L=2, tp=tp)
        assert (s.Hq, s.Hkv, s.D) == (32 // tp, 8 // tp, 128)
        assert np.array_equal(s.hist, full.hist)
        assert s.k_cache.shape == (2, 8, 8 // tp, 1024, 128)
    for bad in (0, 3, 16):
        with pytest.raises(ValueError):
            synth.batched_decode(seed=3, gqa=True, L=2, tp=bad)
    with pytest.raises(ValueError):
        synth.batched_decode(seed=3, gqa=False, L=2, tp=2)
