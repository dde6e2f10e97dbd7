"""The oracle at the decode workloads' own shapes (B=1 .. 64, H up to 7168, I up to 2048), pinned
against the brute-force matrix form: a dense routing matrix over the experts the sampled tokens
are routed to, every one of those experts evaluated densely on every sampled token with numpy
float64 matmuls, weights decoded with torch's float8 decoders.

Inputs: each workload's own activations and routing (the seeded recipe), and random MXFP8 codes
(no NaN code; scale codes 112..120) for the experts the sampled tokens are routed to, renumbered
0..U-1, so that the weights stay small enough for the CPU. The weight values do not matter for
this pin, the shapes and the routing do. Every output of the sampled tokens is compared:
2048 .. 7168 per token.
"""
import numpy as np
import pytest

import oracle
from output_centric_expert_amd import synth
from test_oracle_pins import lib_dequant, lib_x, silu

WORKLOADS = ["wide_B1_E128_k8_H2048_I768", "batch_B8_E128_k8_H2048_I768",
             "batch_B32_E128_k8_H4096_I1536", "skewed_B64_E256_k8_H7168_I2048"]


@pytest.fixture(scope="module", autouse=True)
def built():
    oracle.build(force=False)


def random_mxfp8(rng, U, N, K):
    q = rng.integers(0, 256, size=(U, N, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] ^= 0x01                       # no NaN codes (0x7F, 0xFF -> 0x7E, 0xFE)
    s = rng.integers(112, 121, size=(U, N, K // 32), dtype=np.uint8)
    return q, s


def matrix_form(x_bits, ids, w, mats, U, H):
    """out [T, H] = sum_e R[:, e] * ((SiLU(X Wg_e^T) * (X Wu_e^T)) Wd_e^T), one expert at a time."""
    T = x_bits.shape[0]
    R = np.zeros((T, U))
    for t in range(T):
        for j in range(ids.shape[1]):
            R[t, ids[t, j]] += float(w[t, j])
    X = lib_x(x_bits)
    out = np.zeros((T, H))
    (gq, gs), (uq, us), (dq, ds) = mats
    for e in range(U):
        act = silu(X @ lib_dequant(gq[e], gs[e]).T) * (X @ lib_dequant(uq[e], us[e]).T)
        out += R[:, e:e + 1] * (act @ lib_dequant(dq[e], ds[e]).T)
    return out


@pytest.mark.parametrize("name", WORKLOADS)
def test_oracle_matches_matrix_form_at_workload_shape(name):
    sh = synth.WORKLOADS[name]
    seed = synth.workload_seed(name)
    x = synth.make_activations(sh.B, sh.H, seed)
    ids, w, _ = synth.make_routing(sh.B, sh.E, sh.k, seed, sh.zipf_s)
    toks = [0] if sh.B == 1 else [0, sh.B - 1]
    ids_t = ids[toks]
    experts = sorted(set(int(e) for e in ids_t.ravel()))
    remap = {e: n for n, e in enumerate(experts)}
    ids_c = np.vectorize(remap.get)(ids_t).astype(np.int32)
    U = len(experts)
    rng = np.random.default_rng(seed)
    mats = [random_mxfp8(rng, U, sh.I, sh.H), random_mxfp8(rng, U, sh.I, sh.H), random_mxfp8(rng, U, sh.H, sh.I)]
    x_t = np.ascontiguousarray(x[toks])
    w_t = np.ascontiguousarray(w[toks])
    got = oracle.moe_decode(x_t, ids_c, w_t, mats[0][0], mats[0][1], mats[1][0], mats[1][1],
                            mats[2][0], mats[2][1])
    ref = matrix_form(x_t, ids_c, w_t, mats, U, sh.H)
    assert np.isfinite(ref).all() and np.abs(ref).max() > 0
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < 1e-12, f"{name}: {err:.3e}"
