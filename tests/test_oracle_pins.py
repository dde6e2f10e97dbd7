"""Pins for the CPU oracle: each checks it against something other than itself.

- the element formats against their definitions (golden anchors) and against
  torch's own float8_e4m3fn / float8_e8m0fnu decoders (a library routine);
- the whole layer at top-k = 1 with weight 1 against a dense SwiGLU MLP built
  from numpy float64 matmuls and torch's SiLU;
- the whole layer on tiny shapes against the brute-force matrix form (every
  expert computed densely, a dense routing matrix);
- the routing combine against its invariants (linearity in the routing weights,
  slot-order invariance, zero-weight slot = absent slot, duplicate ids merge);
- block-scale association, token independence, SiLU extremes, empty batches.

A plausible slip in the oracle -- a dropped term, a sign, a transposed weight,
the scale block indexed along the wrong axis, gate and up swapped -- makes at
least one of these fail.
"""
import math
import os

import numpy as np
import pytest
import torch

from output_centric_expert_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------------------
# independent decode (torch's float8 types) and dense references
# --------------------------------------------------------------------------------------

def lib_e4m3(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def lib_ue8m0(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def lib_dequant(q, s) -> np.ndarray:
    """MXFP8 [.., K] codes + [.., K/32] scales -> float64, via the library decoders."""
    q = q.numpy() if hasattr(q, "numpy") else q
    s = s.numpy() if hasattr(s, "numpy") else s
    return lib_e4m3(q) * np.repeat(lib_ue8m0(s), 32, axis=-1)


def lib_x(x_bits) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def silu(t: np.ndarray) -> np.ndarray:
    return torch.nn.functional.silu(torch.from_numpy(t)).numpy()


def matrix_form(L) -> np.ndarray:
    """Brute force: dense routing matrix R[B, E], every expert evaluated on every token."""
    B, E = L.shape.B, L.shape.E
    R = np.zeros((B, E))
    for b in range(B):
        for j in range(L.shape.k):
            R[b, L.ids[b, j]] += float(L.w[b, j])
    X = lib_x(L.x)
    Wg, Wu, Wd = (lib_dequant(q, s) for q, s in ((L.wg_q, L.wg_s), (L.wu_q, L.wu_s), (L.wd_q, L.wd_s)))
    out = np.zeros((B, L.shape.H))
    for e in range(E):
        act = silu(X @ Wg[e].T) * (X @ Wu[e].T)      # [B, I]
        out += R[:, e:e + 1] * (act @ Wd[e].T)       # [B, H]
    return out


def rel_err(a, b):
    scale = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / scale


def tiny(B=2, E=4, k=2, H=96, I=64, seed=7, zipf=0.0):
    return synth.make_layer(synth.LayerShape(f"t{B}{E}{k}{H}{I}", B, E, k, H, I, zipf), seed=seed)


def run(oracle_lib, L, ids=None, w=None, **kw):
    return oracle_lib.moe_decode(L.x, L.ids if ids is None else ids, L.w if w is None else w,
                                 L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s, **kw)


# --------------------------------------------------------------------------------------
# element formats
# --------------------------------------------------------------------------------------

def _anchors():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_ue8m0_anchors.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                rows.append((line[0], int(line[1], 16), float(line[2])))
    return rows


def same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


def test_format_anchors(oracle_lib):
    rows = _anchors()
    assert len(rows) >= 20
    for fmt, code, val in rows:
        got = oracle_lib.e4m3_value(code) if fmt == "e4m3" else oracle_lib.ue8m0_value(code)
        assert same(got, val), (fmt, hex(code), got, val)


def test_e4m3_all_codes_match_library(oracle_lib):
    ref = lib_e4m3(np.arange(256, dtype=np.uint8))
    for c in range(256):
        assert same(oracle_lib.e4m3_value(c), ref[c]), hex(c)


def test_e4m3_structure(oracle_lib):
    vals = [oracle_lib.e4m3_value(c) for c in range(256)]
    finite = [v for v in vals if not math.isnan(v)]
    assert len(finite) == 254
    pos = vals[:0x7F]
    assert all(b > a for a, b in zip(pos, pos[1:]))        # strictly increasing 0x00..0x7E
    for c in range(0x7F):
        assert same(vals[c | 0x80], -vals[c])                # sign symmetry
    assert max(finite) == 448.0 and min(finite) == -448.0


def test_ue8m0_all_codes_match_library(oracle_lib):
    ref = lib_ue8m0(np.arange(256, dtype=np.uint8))
    for c in range(256):
        got = oracle_lib.ue8m0_value(c)
        assert same(got, ref[c]), hex(c)
        if c < 255:
            assert got == 2.0 ** (c - 127)


def test_bf16_decode_matches_library(oracle_lib):
    rng = np.random.default_rng(3)
    bits = np.concatenate([rng.integers(0, 1 << 16, 4000), [0, 0x8000, 0x3F80, 0x7F80, 0xFF80]])
    ref = lib_x(bits.astype(np.uint16))
    for b_, r in zip(bits, ref):
        assert same(oracle_lib.bf16_value(int(b_)), r)


# --------------------------------------------------------------------------------------
# whole layer against dense references
# --------------------------------------------------------------------------------------

def test_k1_unit_weight_is_dense_swiglu_mlp(oracle_lib):
    L = tiny(B=3, E=5, k=1, H=160, I=96, seed=11)
    w1 = np.ones((3, 1), np.float32)
    out, a = run(oracle_lib, L, w=w1, return_inter=True)
    X = lib_x(L.x)
    for b in range(3):
        e = L.ids[b, 0]
        Wg = lib_dequant(L.wg_q[e], L.wg_s[e])
        Wu = lib_dequant(L.wu_q[e], L.wu_s[e])
        Wd = lib_dequant(L.wd_q[e], L.wd_s[e])
        act = silu(Wg @ X[b]) * (Wu @ X[b])
        assert rel_err(a[b, 0], act) < 1e-12
        assert rel_err(out[b], Wd @ act) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_matrix_form_random_tiny(oracle_lib, seed):
    shape = synth.random_small_shape(np.random.default_rng(100 + seed))
    L = synth.make_layer(shape, seed=200 + seed)
    assert rel_err(run(oracle_lib, L), matrix_form(L)) < 1e-12


def test_matrix_form_tiny_workload(oracle_lib):
    L = synth.make_layer("tiny_B1_E8_k2_H256_I128")
    assert rel_err(run(oracle_lib, L), matrix_form(L)) < 1e-12


def test_matrix_form_skewed_routing(oracle_lib):
    L = tiny(B=4, E=8, k=3, H=64, I=96, seed=5, zipf=1.1)
    assert rel_err(run(oracle_lib, L), matrix_form(L)) < 1e-12


# --------------------------------------------------------------------------------------
# routing-combine invariants
# --------------------------------------------------------------------------------------

def test_linear_in_routing_weights(oracle_lib):
    L = tiny(B=3, E=6, k=3, seed=21)
    rng = np.random.default_rng(0)
    w1 = rng.standard_normal(L.w.shape).astype(np.float32)
    w2 = rng.standard_normal(L.w.shape).astype(np.float32)
    o1, o2 = run(oracle_lib, L, w=w1), run(oracle_lib, L, w=w2)
    o12 = run(oracle_lib, L, w=(w1.astype(np.float64) + w2).astype(np.float32))
    # w1 + w2 is rounded to float32; compare against the sum of the exact parts
    # only where that rounding is exact (it is for these small-magnitude draws
    # except in the last bit), hence a relative bound of a few float32 ulps.
    assert rel_err(o12, o1 + o2) < 1e-6
    o3 = run(oracle_lib, L, w=(w1 * np.float32(0.25)))
    assert rel_err(o3, 0.25 * o1) < 1e-14        # scaling by a power of two is exact
    assert np.all(run(oracle_lib, L, w=np.zeros_like(w1)) == 0.0)


def test_additive_in_routing_weights_exact(oracle_lib):
    """Per-slot decomposition: out(w) = sum_j out(w restricted to slot j)."""
    L = tiny(B=2, E=5, k=3, seed=22)
    full = run(oracle_lib, L)
    parts = np.zeros_like(full)
    for j in range(3):
        wj = np.zeros_like(L.w); wj[:, j] = L.w[:, j]
        parts += run(oracle_lib, L, w=wj)
    assert rel_err(full, parts) < 1e-13


def test_slot_order_invariance(oracle_lib):
    L = tiny(B=3, E=8, k=4, seed=23)
    base = run(oracle_lib, L)
    rng = np.random.default_rng(1)
    for _ in range(4):
        perm = np.stack([rng.permutation(4) for _ in range(3)])
        ids = np.take_along_axis(L.ids, perm, 1)
        w = np.take_along_axis(L.w, perm, 1)
        assert rel_err(run(oracle_lib, L, ids=ids, w=w), base) < 1e-13


def test_zero_weight_slot_is_absent_slot(oracle_lib):
    L = tiny(B=2, E=6, k=3, seed=24)
    w = L.w.copy(); w[:, 2] = 0.0
    with_zero = run(oracle_lib, L, w=w)
    without = oracle_lib.moe_decode(L.x, np.ascontiguousarray(L.ids[:, :2]), np.ascontiguousarray(w[:, :2]),
                                    L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s)
    assert rel_err(with_zero, without) < 1e-14


def test_duplicate_ids_merge(oracle_lib):
    L = tiny(B=2, E=6, k=2, seed=25)
    ids = np.stack([L.ids[:, 0], L.ids[:, 0]], 1).astype(np.int32)
    dup = run(oracle_lib, L, ids=ids, w=L.w)
    merged_w = np.stack([L.w[:, 0] + L.w[:, 1], np.zeros(2, np.float32)], 1).astype(np.float32)
    merged = run(oracle_lib, L, ids=np.ascontiguousarray(ids), w=merged_w)
    assert rel_err(dup, merged) < 1e-6         # w0 + w1 rounded to float32


def test_token_independence(oracle_lib):
    L = tiny(B=4, E=6, k=2, seed=26)
    full = run(oracle_lib, L)
    for b in range(4):
        one = oracle_lib.moe_decode(L.x[b:b + 1], L.ids[b:b + 1], L.w[b:b + 1],
                                    L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s)
        np.testing.assert_array_equal(one[0], full[b])


# --------------------------------------------------------------------------------------
# block-scale association, SiLU extremes, edge cases
# --------------------------------------------------------------------------------------

def test_down_block_scale_association(oracle_lib):
    """Raising one down scale byte by 1 doubles exactly that block's 32 terms."""
    L = tiny(B=1, E=3, k=2, H=64, I=96, seed=27)
    out0, a = run(oracle_lib, L, return_inter=True)
    j, blk, h = 1, 2, 17
    e = int(L.ids[0, j])
    wd_s = L.wd_s.clone(); wd_s[e, h, blk] += 1
    out1 = oracle_lib.moe_decode(L.x, L.ids, L.w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, wd_s)
    Wd = lib_dequant(L.wd_q[e], L.wd_s[e])
    sl = slice(32 * blk, 32 * blk + 32)
    extra = float(L.w[0, j]) * (Wd[h, sl] @ a[0, j, sl])
    delta = out1[0] - out0[0]
    expect = np.zeros_like(delta); expect[h] = extra
    assert np.abs(delta - expect).max() <= 1e-15 * max(1.0, np.abs(out0).max())
    assert abs(extra) > 0


def test_gate_block_scale_association(oracle_lib):
    """Raising one gate scale byte by 1 moves g by exactly that block's partial dot."""
    L = tiny(B=1, E=2, k=1, H=128, I=32, seed=28)
    w1 = np.ones((1, 1), np.float32)
    _, a0 = run(oracle_lib, L, w=w1, return_inter=True)
    e, i, blk = int(L.ids[0, 0]), 5, 3
    wg_s = L.wg_s.clone(); wg_s[e, i, blk] += 1
    _, a1 = oracle_lib.moe_decode(L.x, L.ids, w1, L.wg_q, wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                                  return_inter=True)
    X = lib_x(L.x)[0]
    Wg = lib_dequant(L.wg_q[e], L.wg_s[e]); Wu = lib_dequant(L.wu_q[e], L.wu_s[e])
    g, u = Wg[i] @ X, Wu[i] @ X
    sl = slice(32 * blk, 32 * blk + 32)
    g1 = g + Wg[i, sl] @ X[sl]
    assert abs(a1[0, 0, i] - silu(np.array([g1]))[0] * u) < 1e-13
    others = [r for r in range(32) if r != i]
    np.testing.assert_array_equal(a1[0, 0, others], a0[0, 0, others])


def _const_layer(gate_code, gate_scale, up_code, H=64, I=32, x_val=0x3F80):
    """One expert, all gate codes/scales constant; x constant (bf16 bits)."""
    E = 1
    x = np.full((1, H), x_val, np.uint16)
    ids = np.zeros((1, 1), np.int32)
    w = np.ones((1, 1), np.float32)
    wg_q = torch.full((E, I, H), gate_code, dtype=torch.uint8)
    wg_s = torch.full((E, I, H // 32), gate_scale, dtype=torch.uint8)
    wu_q = torch.full((E, I, H), up_code, dtype=torch.uint8)
    wu_s = torch.full((E, I, H // 32), 127, dtype=torch.uint8)
    wd_q = torch.full((E, H, I), 0x38, dtype=torch.uint8)
    wd_s = torch.full((E, H, I // 32), 127, dtype=torch.uint8)
    return x, ids, w, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s


def test_closed_form_constant_layer(oracle_lib):
    """All-constant weights: a = SiLU(H * 1.0) * (H * 0.5) and out = I * a, closed form."""
    H, I = 64, 32
    args = _const_layer(0x38, 127, 0x30, H=H, I=I)          # gate 1.0, up 0.5, x = 1.0
    out, a = oracle_lib.moe_decode(*args, return_inter=True)
    g, u = float(H), 0.5 * H
    a_exp = g / (1.0 + math.exp(-g)) * u
    assert np.all(a == a_exp)
    assert np.allclose(out, I * a_exp, rtol=1e-15, atol=0)


def test_silu_extremes(oracle_lib):
    # gate -> very negative (x = -1, gate codes 448 * 2^120): SiLU -> -0, never NaN
    out, a = oracle_lib.moe_decode(*_const_layer(0x7E, 247, 0x38, x_val=0xBF80), return_inter=True)
    assert np.all(a == 0.0) and not np.isnan(out).any()
    # x = 0 -> gate = up = 0 -> a = 0 -> out = 0
    out, a = oracle_lib.moe_decode(*_const_layer(0x38, 127, 0x38, x_val=0x0000), return_inter=True)
    assert np.all(a == 0.0) and np.all(out == 0.0)


def test_empty_batch(oracle_lib):
    L = tiny(B=1, E=2, k=1, seed=29)
    out = oracle_lib.moe_decode(L.x[:0], L.ids[:0], L.w[:0], L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s)
    assert out.shape == (0, L.shape.H)


def test_out_of_range_id_gives_nan_for_that_token_only(oracle_lib):
    L = tiny(B=2, E=4, k=2, seed=30)
    ids = L.ids.copy(); ids[1, 1] = 4
    out = run(oracle_lib, L, ids=ids)
    assert np.isnan(out[1]).all() and not np.isnan(out[0]).any()


def test_nan_code_propagates(oracle_lib):
    L = tiny(B=1, E=2, k=1, H=64, I=32, seed=31)
    e = int(L.ids[0, 0])
    wd_q = L.wd_q.clone(); wd_q[e, 3, 0] = 0x7F
    out = oracle_lib.moe_decode(L.x, L.ids, L.w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, wd_q, L.wd_s)
    assert np.isnan(out[0, 3]) and np.isfinite(np.delete(out[0], 3)).all()
