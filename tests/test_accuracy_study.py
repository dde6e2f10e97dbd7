"""Pins for the accuracy-study references (oracle/accuracy.py), CPU only."""
import numpy as np
import torch

import oracle
from oracle import accuracy as acc
from output_centric_expert_amd import synth


def test_e4m3_round_fixed_points_and_library_rounding():
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    finite = vals[np.isfinite(vals)]
    assert np.array_equal(acc.e4m3_round(finite), finite)
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-12, 9, 20000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(acc.e4m3_round(v.astype(np.float64)), lib)


def test_mx_quantize_matches_independent_encoder():
    torch.manual_seed(1)
    w = torch.randn(16, 256) * 0.05
    w[3, :32] = 0.0                                    # an all-zero block
    q, s = synth.encode_mxfp8(w)
    dec = (q.view(torch.float8_e4m3fn).double() *
           s.view(torch.float8_e8m0fnu).double().repeat_interleave(32, -1)).numpy()
    assert np.array_equal(acc.mx_quantize(w.double().numpy()), dec)


def test_bf16_round_matches_library():
    v = np.random.default_rng(2).standard_normal(10000).astype(np.float32)
    lib = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    assert np.array_equal(acc.bf16_round(v.astype(np.float64)), lib)


def test_dense_reference_equals_oracle_on_decoded_weights():
    L = synth.make_layer(synth.LayerShape("t", 3, 6, 2, 96, 64), seed=4)
    deq = lambda q, s: (q.view(torch.float8_e4m3fn).double() *
                        s.view(torch.float8_e8m0fnu).double().repeat_interleave(32, -1)).numpy()
    x = synth.bf16_bits_to_float64(L.x)
    got = acc.reference_dense(x, L.ids, L.w, deq(L.wg_q, L.wg_s), deq(L.wu_q, L.wu_s), deq(L.wd_q, L.wd_s))
    ref = oracle.moe_decode_layer(L)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_classical_emulation_error_is_quantization_sized():
    """Its error against the float64 MXFP8-weight layer is of the order of E4M3
    rounding of the activations (3 fraction bits), far above float32 rounding."""
    L = synth.make_layer(synth.LayerShape("t", 4, 8, 2, 256, 128), seed=5)
    deq = lambda q, s: (q.view(torch.float8_e4m3fn).double() *
                        s.view(torch.float8_e8m0fnu).double().repeat_interleave(32, -1)).numpy()
    x = synth.bf16_bits_to_float64(L.x)
    cls = acc.classical_emulation(x, L.ids, L.w, deq(L.wg_q, L.wg_s), deq(L.wu_q, L.wu_s), deq(L.wd_q, L.wd_s))
    st = acc.error_stats(cls, oracle.moe_decode_layer(L))
    assert 3e-3 < st["rms_err_over_rms"] < 6e-2
