"""Pins for the oracle's MXFP4 weight format (FP4 E2M1 codes two per byte, one
UE8M0 scale per 32 values), each against something other than the oracle:

- all 16 E2M1 codes against the format definition's value table
  (tests/golden/e2m1_values.txt);
- the layer, the gate/up half and the down half on MXFP4 weights against the
  MXFP8 oracle (pinned on its own in test_oracle_pins.py) given the same values
  as E4M3 codes -- the E2M1 -> E4M3 code map comes from torch's float8 encoder
  and the nibbles are unpacked here, low nibble first -- which must agree bit
  for bit (same float64 products, same order);
- the layer at top-1 with weight 1 against a dense SwiGLU MLP on weights decoded
  with numpy from the golden table;
- the input encoder's output decodes to values on the E2M1 grid times the block
  scale, within half a grid step of the draw where the draw is inside the grid
  and within the OCP rule's saturation error above it.

Swapping the nibble order, indexing scales per 16 instead of per 32 values, or a
wrong E2M1 exponent bias each fail several of these.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from output_centric_expert_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")


def golden_e2m1():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, v = line.split()
        vals[int(code, 16)] = float(v)
    assert sorted(vals) == list(range(16))
    return np.array([vals[c] for c in range(16)])


@pytest.fixture(scope="module", autouse=True)
def built():
    oracle.build(force=False)


def unpack_nibbles(q: np.ndarray) -> np.ndarray:
    """[.., K/2] packed bytes -> [.., K] codes, element 2t = low nibble of byte t."""
    lo = q & 0xF
    hi = q >> 4
    return np.stack([lo, hi], axis=-1).reshape(*q.shape[:-1], q.shape[-1] * 2)


def fp4_to_fp8_codes(q4: np.ndarray) -> np.ndarray:
    """Packed E2M1 codes -> E4M3 codes of the same values (torch's float8 encoder)."""
    table = torch.tensor(golden_e2m1(), dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return table[unpack_nibbles(q4)]


def fp4_dequant(q4: np.ndarray, s: np.ndarray) -> np.ndarray:
    g = golden_e2m1()
    scale = np.exp2(s.astype(np.float64) - 127.0)
    return g[unpack_nibbles(q4)] * np.repeat(scale, 32, axis=-1)


def small(B, E, k, H, I, seed, **kw):
    return synth.make_layer(synth.LayerShape(f"fp4_{B}_{E}_{k}_{H}_{I}", B, E, k, H, I, **kw), seed=seed,
                            wformat="mxfp4")


def host(t):
    return t.cpu().numpy()


def test_e2m1_all_codes_match_definition():
    g = golden_e2m1()
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert v == g[c] and np.signbit(v) == np.signbit(g[c]), c


def test_e2m1_structure():
    pos = [oracle.e2m1_value(c) for c in range(8)]
    assert all(b > a for a, b in zip(pos, pos[1:]))          # strictly increasing magnitudes
    for c in range(8):
        assert oracle.e2m1_value(c | 8) == -oracle.e2m1_value(c)
    assert max(pos) == 6.0 and pos[1] == 0.5                  # largest value, smallest subnormal


@pytest.mark.parametrize("shape,seed", [((1, 8, 2, 256, 128), 1), ((3, 6, 3, 96, 160), 2),
                                        ((2, 5, 5, 64, 32), 3), ((4, 4, 1, 32, 64), 4)])
def test_fp4_layer_equals_fp8_layer_on_the_same_values(shape, seed):
    L = small(*shape, seed=seed)
    q = [host(t) for t in (L.wg_q, L.wu_q, L.wd_q)]
    s = [host(t) for t in (L.wg_s, L.wu_s, L.wd_s)]
    out4, a4 = oracle.moe_decode(L.x, L.ids, L.w, q[0], s[0], q[1], s[1], q[2], s[2],
                                 return_inter=True, wformat="mxfp4")
    q8 = [fp4_to_fp8_codes(t) for t in q]
    out8, a8 = oracle.moe_decode(L.x, L.ids, L.w, q8[0], s[0], q8[1], s[1], q8[2], s[2], return_inter=True)
    assert np.array_equal(a4, a8)
    assert np.array_equal(out4, out8)
    # the two halves on their own
    E = shape[1]
    a4h = oracle.gate_up(L.x, L.ids, q[0], s[0], q[1], s[1], E, wformat="mxfp4")
    assert np.array_equal(a4h, a4)
    o4h = oracle.down(a4, L.ids, L.w, q[2], s[2], E, wformat="mxfp4")
    assert np.array_equal(o4h, out4)
    assert np.abs(out4).max() > 0


def test_fp4_nibble_order_matters():
    """Reading the nibbles the other way round changes the layer (the pins above see it)."""
    L = small(2, 4, 2, 64, 64, seed=5)
    q = [host(t) for t in (L.wg_q, L.wu_q, L.wd_q)]
    s = [host(t) for t in (L.wg_s, L.wu_s, L.wd_s)]
    swap = [((t & 0xF) << 4) | (t >> 4) for t in q]
    a = oracle.moe_decode(L.x, L.ids, L.w, q[0], s[0], q[1], s[1], q[2], s[2], wformat="mxfp4")
    b = oracle.moe_decode(L.x, L.ids, L.w, swap[0], s[0], swap[1], s[1], swap[2], s[2], wformat="mxfp4")
    assert not np.allclose(a, b)


def test_fp4_top1_equals_dense_swiglu():
    B, E, H, I = 3, 4, 96, 64
    L = small(B, E, 1, H, I, seed=6)
    ids = np.array([[1], [3], [1]], np.int32)
    w = np.ones((B, 1), np.float32)
    q = [host(t) for t in (L.wg_q, L.wu_q, L.wd_q)]
    s = [host(t) for t in (L.wg_s, L.wu_s, L.wd_s)]
    got = oracle.moe_decode(L.x, ids, w, q[0], s[0], q[1], s[1], q[2], s[2], wformat="mxfp4")
    x = torch.from_numpy(L.x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    Wg, Wu, Wd = (fp4_dequant(qq, ss) for qq, ss in zip(q, s))
    for b in range(B):
        e = ids[b, 0]
        g = Wg[e] @ x[b]
        u = Wu[e] @ x[b]
        act = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
        ref = Wd[e] @ act
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_fp4_encoder_lands_on_the_grid():
    gen = torch.Generator().manual_seed(7)
    d = torch.randn((4, 8, 128), generator=gen) * 0.02
    d[0, 0, :32] = 0.0                                       # an all-zero block
    q, s = synth.encode_mxfp4(d)
    assert q.shape == (4, 8, 64) and s.shape == (4, 8, 4)
    dec = fp4_dequant(q.numpy(), s.numpy())
    scale = np.repeat(np.exp2(s.numpy().astype(np.float64) - 127.0), 32, axis=-1)
    err = np.abs(dec - d.double().numpy()) / scale
    # in scaled units the block maximum lies in [4, 8): values up to 6 round to the grid
    # (half a step, at most 1), values above 6 saturate to 6 (less than 2) -- the OCP rule
    inside = np.abs(d.double().numpy()) / scale <= 6.0
    assert err[inside].max() <= 1.0 + 1e-9
    assert err.max() < 2.0
    assert not dec[0, 0, :32].any()
    # every block's largest magnitude maps to one of the top codes 4 or 6 (times the scale)
    top = np.abs(dec).reshape(4, 8, 4, 32).max(-1) / np.exp2(s.numpy().astype(np.float64) - 127.0)
    assert set(np.unique(top[1:])) <= {4.0, 6.0}
