"""Checks of the seeded input generator (not of the layer's arithmetic)."""
import numpy as np
import torch

from output_centric_expert_amd import synth


def _deq(q, s):
    v = q.view(torch.float8_e4m3fn).to(torch.float64)
    sc = s.view(torch.float8_e8m0fnu).to(torch.float64).repeat_interleave(32, dim=-1)
    return v * sc


def test_mxfp8_encoder_error_bound():
    torch.manual_seed(0)
    w = torch.randn(64, 256) * 0.02
    q, s = synth.encode_mxfp8(w)
    d = _deq(q, s)
    # shared exponent se = floor(log2 amax) - 8, so every scaled value is <= 2^9 * (1 - tiny)
    se = s.to(torch.int32) - 127
    scale = torch.exp2(se.to(torch.float64)).repeat_interleave(32, dim=-1)
    err = (d - w.double()).abs()
    # E4M3 rounding: half an ulp, ulp = 2^(exp-3) for normals, 2^-9 for subnormals,
    # plus clipping of scaled values in (448, 512) down to 448
    scaled = (w.double() / scale).abs()
    ulp = torch.where(scaled >= 2 ** -6, torch.exp2(torch.floor(torch.log2(scaled)) - 3), torch.full_like(scaled, 2 ** -9))
    clip = (scaled - 448).clamp(min=0)
    assert torch.all(err <= (0.5 * ulp + clip) * scale * (1 + 1e-12))
    assert int(s.min()) >= 100 and int(s.max()) <= 127


def test_mxfp8_encoder_zero_block_and_saturation():
    w = torch.zeros(2, 64)
    w[1, 32:] = torch.linspace(-1, 1, 32)
    w[1, 40] = 1.9   # amax 1.9 -> se = 0 - 8 = -8 -> scaled max 486 -> clipped to 448
    q, s = synth.encode_mxfp8(w)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and torch.all(q[0] == 0)
    assert s[1, 1] == 127 - 8
    assert q[1, 40] == 0x7E


def test_routing_recipe():
    ids, w, p = synth.make_routing(16, 128, 8, seed=5)
    assert ids.dtype == np.int32 and w.dtype == np.float32
    for b in range(16):
        assert len(set(ids[b].tolist())) == 8
        pr = p[b, ids[b]]
        assert np.all(np.diff(pr) <= 0)                      # descending probability
        assert pr[-1] >= np.sort(p[b])[-8]                  # they are the top 8
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)


def test_skewed_routing_concentrates():
    ids, _, _ = synth.make_routing(64, 256, 8, seed=9, zipf_s=1.1)
    counts = np.bincount(ids.ravel(), minlength=256)
    assert np.unique(ids).size < 90                         # far fewer than uniform (~225)
    assert counts.max() >= 32                               # a hot expert serves half the tokens


def test_bf16_activations_round_to_nearest():
    v = np.random.default_rng(1).standard_normal(5000)
    bits = synth.float64_to_bf16_bits(v)
    back = synth.bf16_bits_to_float64(bits)
    ulp = np.exp2(np.floor(np.log2(np.abs(v))) - 7)
    assert np.all(np.abs(back - v) <= 0.5 * ulp)


def test_workload_byte_counts():
    c2 = synth.WORKLOADS["wide_B1_E128_k8_H2048_I768"]
    assert c2.bytes_per_expert == 4_866_048
    L = synth.make_layer("tiny_B1_E8_k2_H256_I128")
    assert L.unique_weight_bytes == 202_752
    assert L.wg_q.shape == (8, 128, 256) and L.wd_s.shape == (8, 256, 4)


def test_seeded_reproducible():
    a = synth.make_layer("tiny_B1_E8_k2_H256_I128")
    b = synth.make_layer("tiny_B1_E8_k2_H256_I128")
    assert np.array_equal(a.x, b.x) and np.array_equal(a.ids, b.ids)
    assert torch.equal(a.wd_q, b.wd_q) and torch.equal(a.wg_s, b.wg_s)
