"""Pins for the accuracy-study references (oracle/accuracy.py), CPU only."""
import numpy as np
import pytest
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


# ---------------------------------------------------------------------------------------
# classical_emulation against a second construction of the same stages from pinned parts
# ---------------------------------------------------------------------------------------

def _classical_second_construction(xbits, ids, w, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s):
    """The classical path built another way: the C oracle's float64 gate/up on the
    MXFP8-rounded activations, mx_quantize of its intermediate, the C oracle's float64 down
    one slot at a time (weight 1), bf16_round of each expert's output, the routing-weighted
    combine in float64, bf16_round of the result. Only the accumulation precision differs
    from classical_emulation (float64 here, float32 there)."""
    E = wg_q.shape[0]
    xq = acc.mx_quantize(synth.bf16_bits_to_float64(xbits))
    xq_bits = synth.float64_to_bf16_bits(xq)
    assert np.array_equal(synth.bf16_bits_to_float64(xq_bits), xq)     # MXFP8 values are bf16 values
    a = oracle.gate_up(xq_bits, ids, wg_q, wg_s, wu_q, wu_s, E)         # [B, k, I] float64
    aq = acc.mx_quantize(a)                                            # blocks of 32 along I
    B, k = ids.shape
    out = np.zeros((B, wd_q.shape[1]))
    for j in range(k):
        y = oracle.down(np.ascontiguousarray(aq[:, j:j + 1, :]), np.ascontiguousarray(ids[:, j:j + 1]),
                        np.ones((B, 1), np.float32), wd_q, wd_s, E)
        out += w[:, j:j + 1].astype(np.float64) * acc.bf16_round(y)
    return acc.bf16_round(out)


def _deq_np(q, s):
    return (q.view(torch.float8_e4m3fn).double() *
            s.view(torch.float8_e8m0fnu).double().repeat_interleave(32, -1)).numpy()


def _classical(L):
    x = synth.bf16_bits_to_float64(L.x)
    return acc.classical_emulation(x, L.ids, L.w, _deq_np(L.wg_q, L.wg_s), _deq_np(L.wu_q, L.wu_s),
                                   _deq_np(L.wd_q, L.wd_s))


def _second(L):
    return _classical_second_construction(L.x, L.ids, L.w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s)


def _bf16_ulp(v):
    """Spacing of bfloat16 numbers at |v| (8 significant bits)."""
    _, e = np.frexp(np.maximum(np.abs(v), 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def _agreement(got, ref):
    """(fraction of outputs bit-identical, largest difference in bf16 ulps of the larger value)."""
    same = float(np.mean(got == ref))
    ulps = float(np.max(np.abs(got - ref) / _bf16_ulp(np.maximum(np.abs(got), np.abs(ref)))))
    return same, ulps


def _exact_layer(seed=11, B=3, E=4, k=2, H=128, I=64):
    """A layer on which every classical stage is exact in float32 and in float64: x = +-1,
    each gate row holds g in {24, 32, 40, 48, 64, 80, 96} matching signs (so SiLU(g) rounds to g
    in float32 and to within 1e-10 of g in float64), each up row one entry u in {1, 2, 4} (with
    a sign), so SiLU(g)*u has at most 3 significant bits and sits on the MXFP8 grid of its block;
    down weights in {-1, 0, 1}; routing weights powers of two. Scales are 2^0."""
    rng = np.random.default_rng(seed)
    code = {0.0: 0x00, 1.0: 0x38, 2.0: 0x40, 4.0: 0x48, -1.0: 0xB8, -2.0: 0xC0, -4.0: 0xC8}
    xs = rng.choice([-1.0, 1.0], size=(B, H))
    x_sign = xs[0]                                     # gate/up rows are built for token 0's signs
    xs[:] = x_sign                                     # every token the same activations
    wg = np.zeros((E, I, H)); wu = np.zeros((E, I, H))
    for e in range(E):
        for i in range(I):
            g = int(rng.choice([24, 32, 40, 48, 64, 80, 96]))
            pos = rng.choice(H, size=g, replace=False)
            wg[e, i, pos] = x_sign[pos]
            h = int(rng.integers(H))
            wu[e, i, h] = float(rng.choice([1.0, 2.0, 4.0])) * float(rng.choice([-1.0, 1.0])) * x_sign[h]
    wd = rng.choice([-1.0, 0.0, 1.0], size=(E, H, I))
    enc = np.vectorize(lambda v: code[float(v)], otypes=[np.uint8])
    ones = lambda n, kk: np.full((E, n, kk // 32), 127, np.uint8)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(B)]).astype(np.int32)
    w = rng.choice([0.125, 0.25, 0.5, 1.0], size=(B, k)).astype(np.float32)
    L = synth.LayerInputs(synth.LayerShape("exact", B, E, k, H, I), seed,
                          synth.float64_to_bf16_bits(xs), ids, w, np.zeros((B, E)),
                          torch.from_numpy(enc(wg)), torch.from_numpy(ones(I, H)),
                          torch.from_numpy(enc(wu)), torch.from_numpy(ones(I, H)),
                          torch.from_numpy(enc(wd)), torch.from_numpy(ones(H, I)))
    return L


def test_classical_emulation_bit_exact_where_every_stage_is_exact():
    L = _exact_layer()
    got, ref = _classical(L), _second(L)
    assert np.array_equal(got, ref)
    assert np.count_nonzero(ref) > 0.9 * ref.size


def _random_layers():
    yield synth.make_layer(synth.LayerShape("t", 6, 8, 2, 256, 128), seed=21)
    yield synth.make_layer(synth.LayerShape("t", 4, 16, 4, 512, 256), seed=22)


def test_classical_emulation_matches_second_construction():
    """float32 against float64 accumulation: nearly every output bit-identical, none more
    than one BF16 ulp apart (a stage boundary crossed by a float32 rounding)."""
    for L in _random_layers():
        same, ulps = _agreement(_classical(L), _second(L))
        assert same >= 0.99, same
        assert ulps <= 1.0, ulps


@pytest.mark.parametrize("stage", ["_cls_quantize_x", "_cls_quantize_a", "_cls_expert_round",
                                   "_cls_final_round"])
def test_classical_emulation_pins_catch_a_dropped_stage(monkeypatch, stage):
    """A copy of the classical path with one rounding stage taken out (planted in the oracle,
    on the CPU) fails the pins above."""
    drop = {"_cls_quantize_x": lambda x: np.asarray(x, np.float32),
            "_cls_quantize_a": lambda act: act,
            "_cls_expert_round": lambda y: y,
            "_cls_final_round": lambda out: np.asarray(out, np.float64)}[stage]
    monkeypatch.setattr(acc, stage, drop)
    caught = []
    L = _exact_layer()
    caught.append(not np.array_equal(_classical(L), _second(L)))
    for L in _random_layers():
        same, ulps = _agreement(_classical(L), _second(L))
        caught.append(same < 0.99 or ulps > 1.0)
    assert any(caught), stage
