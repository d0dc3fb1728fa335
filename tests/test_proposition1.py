"""Proposition 1 of [N] §3.3 (LOCKS reading notes): a scoring rule that sees a
page only through the query, its centroid and the sketches W^T k_i of a fixed
shared projection W (rank rho < d) is blind to a (d - rho)-dimensional family
of within-page changes: adding c u to one key and subtracting it from another,
u orthogonal to span(W), leaves every such score unchanged while the exact
page log-mass moves without bound as c grows. The per-page summary of
[N] §4.1 is not blind to it. CPU pins on the oracle; the GPU test runs the
library's build and score on the same pages."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import locks_oracle as O

CS = (0.0, 1.0, 2.0, 4.0, 8.0, 16.0, 32.0)


def _setup(seed=41, rho=8, n=12):
    rng = np.random.default_rng(seed)
    g = torch.Generator().manual_seed(seed)
    K = synth.page_keys(n, g).double().numpy()                       # (n, 16, 128)
    # a fixed shared basis: the top-rho principal directions of all keys
    X = K.reshape(-1, 128) - K.reshape(-1, 128).mean(axis=0)
    W = np.linalg.svd(X, full_matrices=False)[2][:rho].T           # (128, rho)
    q = rng.standard_normal((4, 128))
    # u orthogonal to span(W) with q . u > 0 for every query of the group
    u = q.mean(axis=0) - W @ (W.T @ q.mean(axis=0))
    u /= np.linalg.norm(u)
    assert (q @ u > 0).all()
    return K, W, q, u


def test_shared_sketch_is_blind_to_the_orthogonal_family():
    K, W, q, u = _setup()
    base = O.shared_sketch_scores(q, K, W)
    for c in CS[1:]:
        Kc = np.stack([O.blind_direction_pair(k, W, u, c) for k in K])
        # the centroid and every sketch are unchanged ...
        np.testing.assert_allclose(Kc.mean(axis=1), K.mean(axis=1), atol=1e-12)
        np.testing.assert_allclose(Kc @ W, K @ W, atol=1e-12)
        # ... so the shared-sketch score is unchanged for every query
        np.testing.assert_allclose(O.shared_sketch_scores(q, Kc, W), base, atol=1e-12)


def test_exact_mass_moves_without_bound():
    """For q . u > 0 the key given + c u has logit (q.k_a + c q.u)/sqrt(d), so
    the exact page LSE is at least that and grows at least linearly in c."""
    K, W, q, u = _setup()
    for c in CS[1:]:
        Kc = np.stack([O.blind_direction_pair(k, W, u, c) for k in K])
        ex = O.exact_page_lse(q, Kc)
        lower = (np.einsum("pd,gd->pg", K[:, 0], q) + c * (q @ u)[None, :]) / math.sqrt(128)
        assert (ex >= lower - 1e-12).all()
    # (convex in c, not monotone from c = 0: the key given - c u may dominate
    # at first); at c = 32 every page and query has moved by more than 7 nat
    assert (ex - O.exact_page_lse(q, K)).min() > 7.0


def test_per_page_summary_follows_the_change():
    """The per-page rank-8 summary moves with the exact LSE. At c = 32 the
    exact score of every page has moved by more than 7 nat and the shared
    sketch is off by that much; the unquantised summary stays within 0.1 nat.
    The stored summary stays within 1 nat: the coefficient rows of the two
    changed keys have one int8 scale each, set by their +-c entry, so the
    step on their other coefficients grows with c (0.04 nat at c = 0, 0.7 at
    c = 32 here)."""
    K, W, q, u = _setup()
    c = 32.0
    Kc = np.stack([O.blind_direction_pair(k, W, u, c) for k in K])
    ex = O.exact_page_lse(q, Kc)
    s = O.spectral_summary(Kc, 8)
    unq = O.page_scores(q, s["mu"], s["V"], s["C"])
    slots, _, _ = O.build_slots(Kc, 8)
    dq = O.dequantise(O.unpack_slots(slots, 8))
    qz = O.page_scores(q, dq["mu"], dq["V"], dq["C"])
    sh = O.shared_sketch_scores(q, Kc, W)
    assert np.abs(unq - ex).max() < 0.1
    assert np.abs(qz - ex).max() < 1.0
    assert np.abs(sh - ex).min() > 7.0


@pytest.mark.gpu
def test_gpu_summary_follows_the_change():
    """The library builds and scores the pages P and P' (c = 32): its scores
    stay within 1 nat of the exact page LSE of each while that moves by more
    than 7 nat, the change the shared sketch cannot see."""
    from kv_cache_page_amd import locks as L
    K, W, q, u = _setup()
    c = 32.0
    Kc = np.stack([O.blind_direction_pair(k, W, u, c) for k in K])
    n = K.shape[0]
    pages = torch.from_numpy(np.concatenate([K, Kc])).to(torch.bfloat16)   # (2n, 16, 128)
    Kb = pages.double().numpy()
    dev = "cuda"
    dims = L.Dims(1, 4, 8)
    pool = pages.view(2 * n, 1, 16, 128).contiguous().to(dev)
    summ = L.alloc_summaries(dims, 2 * n, dev)
    L.build(dims, pool, torch.arange(2 * n, dtype=torch.int32, device=dev), summ)
    qb = torch.from_numpy(q).to(torch.bfloat16)
    table = torch.arange(2 * n, dtype=torch.int32, device=dev).view(1, 2 * n)
    lens = torch.tensor([2 * n * 16], dtype=torch.int32, device=dev)
    sc = torch.empty(1, 1, 2 * n, 4, device=dev)
    L.score_pages(dims, qb.view(1, 4, 128).to(dev), summ, table, lens, sc)
    torch.cuda.synchronize()
    got = sc[0, 0].cpu().numpy()
    ex = O.exact_page_lse(qb.double().numpy(), Kb)
    assert np.abs(got - ex).max() < 1.0
    moved = got[n:] - got[:n]
    assert (moved > 5.0).all(), moved
    sh = O.shared_sketch_scores(qb.double().numpy(), Kb, W)
    np.testing.assert_allclose(sh[n:], sh[:n], atol=0.05)   # bf16 rounding of the keys only
