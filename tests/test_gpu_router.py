"""GPU tests of the router front-end (moe_route) and of the layer fed by it,
with shared experts, through the C-ABI, against the float64 CPU oracle.

Expert ids (and their order) must match the oracle exactly -- both sides
compare the same float32 logits; the weights are computed in float32 on the
GPU and must agree to 1e-5 relative. The layer then runs on the GPU router's
output and is held to the usual 2e-3 * rms tolerance against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from output_centric_expert_amd import moedecode as md
from output_centric_expert_amd import synth
from test_gpu_parity import check_f32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    md.load()
    oracle.build(force=False)


def gpu_route(lg, k, n_shared=0, scale=1.0):
    ids, w = md.moe_route(torch.from_numpy(lg).cuda(), k, n_shared, scale)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def check_route(lg, k, n_shared=0, scale=1.0, label=""):
    ids, w = gpu_route(lg, k, n_shared, scale)
    rid, rw = oracle.route(lg, k, n_shared, scale)
    assert np.array_equal(ids, rid), label
    fin = np.isfinite(rw)
    assert np.array_equal(fin, np.isfinite(w)), label
    np.testing.assert_allclose(w[fin], rw[fin], rtol=1e-5, atol=0, err_msg=label)
    return ids, w


@pytest.mark.parametrize("B,E,k", [(1, 128, 8), (8, 128, 8), (64, 256, 8), (5, 8, 2), (3, 67, 5),
                                   (2, 2048, 16), (4, 130, 64), (7, 1, 1), (33, 64, 64)])
def test_route_matches_oracle(B, E, k):
    rng = np.random.default_rng(B * 7919 + E * 31 + k)
    lg = (rng.standard_normal((B, E)) * 3.0).astype(np.float32)
    check_route(lg, k, label=f"B{B} E{E} k{k}")


def test_route_workload_logits():
    """The skewed workload's router logits (log-Zipf prior), as float32."""
    lg = synth.make_router_logits(64, 256, seed=7, zipf_s=1.1).astype(np.float32)
    check_route(lg, 8, label="zipf")


def test_route_ties_nan_inf_shared_scale():
    rng = np.random.default_rng(11)
    ties = rng.integers(-3, 4, size=(16, 100)).astype(np.float32)
    ties[0, :] = 0.0
    ties[1, ::2] = -0.0                                  # +0 and -0 are equal logits
    check_route(ties, 12, label="ties")
    check_route(ties, 7, n_shared=3, scale=2.5, label="ties+shared")
    edge = np.array([[1.0, np.nan, 3.0, -np.inf, 0.5, 2.0],
                     [np.nan, np.nan, np.nan, np.nan, 2.0, np.nan],
                     [-np.inf, 0.0, -np.inf, 1.0, -np.inf, -np.inf]], np.float32)
    ids, w = check_route(edge, 4, n_shared=1, label="nan/inf")
    assert list(ids[1]) == [4, -1, -1, -1, 6]
    assert np.isnan(w[1, 1:4]).all() and w[1, 4] == 1.0


@pytest.mark.parametrize("wformat", ["mxfp8", "mxfp4"])
def test_layer_fed_by_router_with_shared_experts(wformat):
    """GPU router -> layer (E routed + 2 shared experts, k + 2 slots) vs the oracle."""
    B, E, k, ns, H, I = 6, 32, 4, 2, 256, 128
    L = synth.make_layer(synth.LayerShape("routed", B, E + ns, k + ns, H, I), seed=5, device="cuda",
                         wformat=wformat)
    lg = synth.make_router_logits(B, E, seed=5).astype(np.float32)
    ids, w = md.moe_route(torch.from_numpy(lg).cuda(), k, ns, 1.0)
    x = torch.from_numpy(L.x.view(np.int16)).cuda().view(torch.bfloat16)
    out = md.moe_decode(x, ids, w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                        out_dtype=torch.float32, wformat=wformat)
    torch.cuda.synchronize()
    rid, rw = oracle.route(lg, k, ns)
    assert np.array_equal(ids.cpu().numpy(), rid)
    ref = oracle.moe_decode(L.x, rid, w.cpu().numpy(), L.wg_q.cpu(), L.wg_s.cpu(), L.wu_q.cpu(), L.wu_s.cpu(),
                            L.wd_q.cpu(), L.wd_s.cpu(), wformat=wformat)
    check_f32(out, ref, f"routed layer {wformat}")
    # the shared experts' term alone: route with k' = 0 is not allowed, so compare against
    # the oracle with the routed weights zeroed
    w0 = w.clone()
    w0[:, :k] = 0.0
    out0 = md.moe_decode(x, ids, w0, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                         out_dtype=torch.float32, wformat=wformat)
    torch.cuda.synchronize()
    ref0 = oracle.moe_decode(L.x, rid, w0.cpu().numpy(), L.wg_q.cpu(), L.wg_s.cpu(), L.wu_q.cpu(),
                             L.wu_s.cpu(), L.wd_q.cpu(), L.wd_s.cpu(), wformat=wformat)
    check_f32(out0, ref0, f"shared term {wformat}")
    say(f"routed layer {wformat}: ok")
