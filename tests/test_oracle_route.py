"""Pins for the oracle's router front-end (softmax -> top-k -> renormalise, plus
shared-expert slots), each against something other than the oracle:

- without ties: the ids equal torch.topk of the logits (a library routine) and
  the weights equal torch's float64 softmax at those ids, renormalised;
- with ties: the ids equal Python's stable sort by (-logit, id);
- invariants: shifting all logits by a constant changes nothing, the routed
  weights sum to the routed scale, k = E returns every expert in that order;
- edge cases: NaN logits are never selected (missing slots get id -1 and a NaN
  weight), -inf logits come last with weight 0, shared slots follow the routed
  ones with ids E, E+1, ... and weight 1.
"""
import numpy as np
import pytest
import torch

import oracle


@pytest.fixture(scope="module", autouse=True)
def built():
    oracle.build(force=False)


def rand_logits(B, E, seed, scale=2.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, E)) * scale).astype(np.float32)


@pytest.mark.parametrize("B,E,k", [(4, 8, 2), (3, 128, 8), (2, 256, 8), (5, 67, 5), (1, 1, 1)])
def test_route_matches_library_topk_and_softmax(B, E, k):
    lg = rand_logits(B, E, seed=B * 1000 + E)
    ids, w = oracle.route(lg, k)
    t = torch.from_numpy(lg)
    ref_ids = torch.topk(t, k, dim=1, sorted=True).indices.numpy()
    assert np.array_equal(ids, ref_ids)
    p = torch.softmax(t.double(), dim=1).numpy()
    sel = np.take_along_axis(p, ref_ids.astype(np.int64), axis=1)
    ref_w = sel / sel.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, ref_w, rtol=2e-7, atol=0)


def test_route_ties_go_to_the_lower_id():
    rng = np.random.default_rng(3)
    lg = rng.integers(-2, 3, size=(6, 40)).astype(np.float32)   # many exact ties
    for k in (1, 3, 8, 40):
        ids, _ = oracle.route(lg, k)
        for b in range(lg.shape[0]):
            ref = sorted(range(40), key=lambda e: (-float(lg[b, e]), e))[:k]
            assert list(ids[b]) == ref


def test_route_invariants():
    lg = rand_logits(3, 64, seed=9)
    ids, w = oracle.route(lg, 6, routed_scale=2.5)
    ids2, w2 = oracle.route(lg + np.float32(4.0), 6, routed_scale=2.5)
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=2e-6)
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), 2.5, rtol=1e-6)
    full, _ = oracle.route(lg, 64)
    for b in range(3):
        assert list(full[b]) == sorted(range(64), key=lambda e: (-float(lg[b, e]), e))


def test_route_nan_inf_and_shared_slots():
    lg = np.array([[1.0, np.nan, 3.0, -np.inf, 0.5],
                   [np.nan, np.nan, np.nan, np.nan, 2.0]], np.float32)
    ids, w = oracle.route(lg, 4, n_shared=2)
    assert list(ids[0]) == [2, 0, 4, 3, 5, 6]
    assert w[0, 3] == 0.0 and w[0, 4] == 1.0 and w[0, 5] == 1.0
    np.testing.assert_allclose(w[0, :3].astype(np.float64).sum(), 1.0, rtol=1e-6)
    assert list(ids[1]) == [4, -1, -1, -1, 5, 6]
    assert w[1, 0] == 1.0 and np.isnan(w[1, 1:4]).all()


def test_route_rejects_bad_sizes():
    lg = rand_logits(1, 4, seed=1)
    for k, ns in ((0, 0), (5, 0), (2, -1)):
        with pytest.raises(ValueError):
            oracle.route(lg, k, n_shared=ns)
