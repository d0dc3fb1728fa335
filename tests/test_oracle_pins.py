"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
LOCKS reading notes print (the section 5.1 toy page), closed forms, a different
library routine (SVD, torch attention), brute force over subsets, invariants
and the bounds of Theorem 1 (eq. 7, eq. 8). Pages cited: the LOCKS reading
notes (zhongzhuzhou.org, 2026-07-29), written [N] below.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import locks_oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _structured_pages(n, seed, noise=0.05, B=16, d=128):
    g = torch.Generator().manual_seed(seed)
    return synth.page_keys(n, g, B, d, noise=noise).double().numpy()


# ---------------------------------------------------------------------------
# Build ([N] §4.1 eq. 2-3, Algorithm 1)
# ---------------------------------------------------------------------------

def test_toy_page_closed_form():
    """[N] §5.1 toy page (B = 4, d = 4, r = 1). The nonzero Gram eigenvalues
    are those of the 2x2 matrix D^T D restricted to the first two axes:
    [[3.62, 0.18], [0.18, 0.02]], i.e. (3.64 +- sqrt(3.64^2 - 4*0.04)) / 2,
    with leading eigenvector at angle theta = atan(0.36 / 3.6) / 2."""
    g = json.load(open(os.path.join(GOLDEN, "toy_page_b4_d4.json")))
    delta = np.array(g["delta"])
    mu = np.array([0.5, -1.0, 2.0, 0.25])
    s = O.spectral_summary((mu + delta)[None], g["r"])
    tr, det = 3.64, 3.62 * 0.02 - 0.18 ** 2
    lam1 = (tr + math.sqrt(tr * tr - 4 * det)) / 2
    lam2 = (tr - math.sqrt(tr * tr - 4 * det)) / 2
    theta = 0.5 * math.atan(0.36 / 3.6)
    np.testing.assert_allclose(s["mu"][0], mu, atol=1e-15)
    np.testing.assert_allclose(s["lam"][0], [lam1, lam2, 0.0, 0.0], atol=1e-12)
    np.testing.assert_allclose(s["V"][0][:, 0], [math.cos(theta), math.sin(theta), 0, 0], atol=1e-12)
    c = delta @ np.array([math.cos(theta), math.sin(theta), 0, 0])
    np.testing.assert_allclose(s["C"][0][:, 0], c, atol=1e-12)
    np.testing.assert_allclose(s["tau"][0], lam2, atol=1e-12)
    # the printed magnitudes: lambda_1 ~ 3.629, tail ~ 0.011, c ~ (+-0.9988, +-0.9039)
    assert abs(lam1 - 3.628978) < 1e-6 and abs(lam2 - 0.011022) < 1e-6
    # a query along the discarded second axis: reconstructed logits coincide
    # pairwise, exact ones do not ([N] §5.1 narrative), and eq. 7 bounds the gap
    q = np.array([[0.0, 5.0, 0.0, 0.0]])
    est = O.page_scores(q, s["mu"], s["V"], s["C"])[0, 0]
    exact = O.exact_page_lse(q, (mu + delta)[None])[0, 0]
    V = s["V"][0]
    q_perp = q[0] - V @ (V.T @ q[0])
    assert abs(est - exact) <= np.linalg.norm(q_perp) * math.sqrt(s["tau"][0]) / 2.0 + 1e-12
    assert abs(est - exact) > 1e-4


def test_eigen_matches_svd():
    """Gram eigenvalues are the squared singular values of D, and the basis
    columns are D's right singular vectors up to sign (a different LAPACK
    routine, numpy.linalg.svd)."""
    keys = _structured_pages(40, 11)
    r = 8
    s = O.spectral_summary(keys, r)
    _, D = O.centre(keys)
    for p in range(keys.shape[0]):
        _, sv, Wt = np.linalg.svd(D[p], full_matrices=False)
        np.testing.assert_allclose(s["lam"][p], sv ** 2, rtol=1e-10, atol=1e-9)
        for k in range(r):
            np.testing.assert_allclose(abs(s["V"][p][:, k] @ Wt[k]), 1.0, atol=1e-9)


def test_summary_invariants():
    """Orthonormal active basis; c_i = V^T delta_i; sum_i c_i = 0; the
    rank-r residual energy equals the dropped eigenvalue mass (Eckart-Young);
    canonical sign: the largest-|v| entry of each basis vector is positive."""
    keys = _structured_pages(30, 12)
    for r in (1, 4, 8, 16):
        s = O.spectral_summary(keys, r)
        _, D = O.centre(keys)
        for p in range(keys.shape[0]):
            V, C, act = s["V"][p], s["C"][p], s["active"][p]
            Va = V[:, act]
            np.testing.assert_allclose(Va.T @ Va, np.eye(act.sum()), atol=1e-10)
            np.testing.assert_allclose(C, D[p] @ V, atol=1e-9)
            np.testing.assert_allclose(C.sum(axis=0), 0.0, atol=1e-9)
            resid = D[p] - C @ V.T
            np.testing.assert_allclose((resid ** 2).sum(), s["dropped"][p], rtol=1e-8, atol=1e-9)
            for k in np.flatnonzero(act):
                m = np.argmax(np.abs(V[:, k]))
                assert V[m, k] > 0
        if r == 16:
            # centring leaves rank <= B - 1, so the 16th component is inactive
            assert not s["active"][:, 15].any()


def test_zero_and_rank_deficient_pages():
    """All-equal keys: every component inactive, zero basis and coefficients,
    zero codes and scales (reading R6, R1). Rank-2 page: r = 8 keeps two."""
    k = np.ones((1, 16, 128)) * 0.37
    sl, s, qs = O.build_slots(k, 8)
    assert not s["active"].any()
    assert (qs["Vq"] == 0).all() and (qs["Cq"] == 0).all() and (qs["sV"] == 0).all()
    assert qs["smu"][0] == np.float16(0.37 / 127)
    rng = _rng(3)
    base = rng.standard_normal((2, 128))
    coef = rng.standard_normal((16, 2))
    s = O.spectral_summary((coef @ base)[None], 8)
    assert s["active"][0].sum() == 2


# ---------------------------------------------------------------------------
# Quantisation (readings R1-R3)
# ---------------------------------------------------------------------------

def test_quantiser_hand_values():
    # absmax 0.7 -> scale fp16(0.1) = 0.0999755859375
    codes, sc = O.quantise(np.array([[0.7, -0.35, 0.1, 0.0]]), 7, axis=1)
    assert float(sc[0]) == 0.0999755859375
    assert codes.tolist() == [[7, -4, 1, 0]]
    # exact scale 0.5: ties round half to even
    codes, sc = O.quantise(np.array([[3.5, 1.25, 1.75, -0.25, -0.75]]), 7, axis=1)
    assert float(sc[0]) == 0.5
    assert codes.tolist() == [[7, 2, 4, 0, -2]]
    # int8: absmax 127 -> scale 1
    codes, sc = O.quantise(np.array([[127.0, -63.5, 2.5]]), 127, axis=1)
    assert float(sc[0]) == 1.0 and codes.tolist() == [[127, -64, 2]]
    # zero slice
    codes, sc = O.quantise(np.zeros((1, 5)), 127, axis=1)
    assert float(sc[0]) == 0.0 and (codes == 0).all()
    # overflowing scale saturates at the largest finite fp16
    codes, sc = O.quantise(np.array([[1e6, -1e6]]), 7, axis=1)
    assert float(sc[0]) == 65504.0 and codes.tolist() == [[7, -7]]


def test_quantiser_error_bound():
    rng = _rng(5)
    x = rng.standard_normal((200, 37)) * rng.uniform(0.01, 100, (200, 1))
    for qmax in (7, 127):
        codes, sc = O.quantise(x, qmax, axis=1)
        s = sc.astype(np.float64)[:, None]
        assert (np.abs(codes) <= qmax).all()
        slack = np.abs(np.abs(x).max(axis=1, keepdims=True) - qmax * s)
        assert (np.abs(x - codes * s) <= s / 2 * (1 + 1e-6) + slack).all()


# ---------------------------------------------------------------------------
# Slot bytes (reading R4)
# ---------------------------------------------------------------------------

def test_slot_sizes():
    """768 B of payload per page at r = 8 ([N] §6, figure 1(a) caption), i.e.
    9.375% of the 8192 B of bf16 K+V for 16 tokens x 128 dims (the "9.4%" of
    [N] §4.1); with the 25 fp16 scales 818 B, about one tenth."""
    L = O.slot_layout(8)
    assert L["payload"] - 2 * (8 + 16 + 1) == 768
    assert abs(768 / 8192 - 0.094) < 0.001
    assert L["payload"] == 818 and L["stride"] == 896
    assert abs(818 / 8192 - 0.1) < 0.001
    assert O.slot_layout(4)["payload"] == 490 and O.slot_layout(16)["payload"] == 1474


def test_slot_bytes_by_hand():
    """Column 0, dims 0..7 = 1,2,3,4,5,6,7,-1: the word's bytes carry the dim
    pairs (0,1),(4,5),(2,3),(6,7), low nibble first -> 21 65 43 F7."""
    r = 8
    qs = dict(Vq=np.zeros((1, 128, r), dtype=np.int64), sV=np.zeros((1, r), np.float16),
              Cq=np.zeros((1, 16, r), dtype=np.int64), sC=np.zeros((1, 16), np.float16),
              muq=np.zeros((1, 128), dtype=np.int64), smu=np.zeros(1, np.float16))
    qs["Vq"][0, :8, 0] = [1, 2, 3, 4, 5, 6, 7, -1]
    qs["Cq"][0, 1, 2] = -2
    qs["muq"][0, 3] = -128 + 1
    qs["sV"][0, 1] = 1.0
    qs["smu"][0] = 2.0
    b = O.pack_slots(qs)[0]
    assert list(b[0:4]) == [0x21, 0x65, 0x43, 0xF7]
    assert b[512 + 1 * 8 + 2] == 0xFE
    assert b[640 + 3] == 0x81
    assert list(b[768 + 2:768 + 4]) == [0x00, 0x3C]      # fp16 1.0, little endian
    assert list(b[816:818]) == [0x00, 0x40]              # fp16 2.0
    assert (b[818:] == 0).all()
    back = O.unpack_slots(b[None], r)
    for n in qs:
        assert np.array_equal(back[n], qs[n]), n


def test_slot_roundtrip_random():
    keys = _structured_pages(25, 13)
    for r in (4, 8, 16):
        sl, _, qs = O.build_slots(keys, r)
        back = O.unpack_slots(sl, r)
        for n in qs:
            assert np.array_equal(back[n], qs[n]), (r, n)


def _exact_summary(n, r, seed, B=16, d=128):
    """A summary whose entries are integer codes times power-of-two scales,
    with one entry of every quantised slice at +-qmax: the quantiser of
    readings R1-R2 must return exactly these codes and scales. The scales
    differ from column to column of V and from row to row of C, so a scale
    applied along the wrong axis changes the values even at r = B = 16,
    where the two shapes coincide."""
    rng = _rng(seed)

    def codes(shape, qmax, axis):
        c = rng.integers(-qmax + 1, qmax, shape)
        # put +-qmax at one random position of every slice along `axis`
        moved = np.moveaxis(c, axis, -1)
        idx = rng.integers(0, moved.shape[-1], moved.shape[:-1])
        sign = rng.choice([-1, 1], moved.shape[:-1])
        np.put_along_axis(moved, idx[..., None], (sign * qmax)[..., None], axis=-1)
        return np.moveaxis(moved, -1, axis)

    Vq = codes((n, d, r), 7, axis=1)                     # absmax over d, per column
    Cq = codes((n, B, r), 127, axis=2)                   # absmax over r, per token row
    muq = codes((n, d), 127, axis=1)
    sV = 2.0 ** -(2 + (np.arange(r)[None, :] + np.arange(n)[:, None]) % 6)
    sC = 2.0 ** -(1 + (3 * np.arange(B)[None, :] + np.arange(n)[:, None]) % 9)
    smu = 2.0 ** -(3 + np.arange(n) % 4)
    summary = dict(V=Vq * sV[:, None, :], C=Cq * sC[:, :, None], mu=muq * smu[:, None])
    codes_ = dict(Vq=Vq, sV=sV.astype(np.float16), Cq=Cq, sC=sC.astype(np.float16),
                  muq=muq, smu=smu.astype(np.float16))
    return summary, codes_


def test_exactly_representable_summary_round_trips():
    """Codes times power-of-two scales, each slice reaching +-qmax: quantise,
    pack, unpack and dequantise must return the values exactly, and the score
    of eq. 4 ([N] §4.2) from the decoded slot must equal the score of the
    unquantised values (to summation-order rounding: the arrays are equal but
    laid out differently)."""
    q = _rng(20).standard_normal((4, 128)) * 1.5
    for r in (4, 8, 16):
        summ, want = _exact_summary(9, r, 30 + r)
        qs = O.quantise_summary(summ)
        for n in want:
            assert np.array_equal(qs[n], want[n]), (r, n)
        slots = O.pack_slots(qs)
        assert slots.shape[1] == O.slot_layout(r)["stride"]
        dq = O.dequantise(O.unpack_slots(slots, r))
        for n in ("V", "C", "mu"):
            assert np.array_equal(dq[n], summ[n]), (r, n)
        s_dec = O.page_scores(q, dq["mu"], dq["V"], dq["C"])
        s_raw = O.page_scores(q, summ["mu"], summ["V"], summ["C"])
        np.testing.assert_allclose(s_dec, s_raw, rtol=0, atol=1e-12)


def _quant_step_bound(x, qmax, axis):
    """A-priori elementwise bound on |decoded - x| for symmetric absmax
    quantisation with one scale per slice along `axis`, whatever the
    rounding of the stored fp16 scale: half a step plus what the fp16
    rounding of the scale can move the largest entry (reading R1)."""
    amax = np.max(np.abs(x), axis=axis, keepdims=True)
    return 0.5 * amax / qmax * (1 + 2.0 ** -9) + amax * 2.0 ** -10


def test_quantised_summary_within_quantiser_step():
    """Decoded basis, coefficients and centroid of realistic pages lie within
    half a quantiser step of the unquantised values, slice by slice: basis per
    column, coefficients per token row, centroid per page ([N] §4.1 storage
    paragraph; readings R1-R2). A scale applied along the wrong axis breaks
    this at r = 16 as well."""
    keys = _structured_pages(40, 17)
    for r in (4, 8, 16):
        slots, s, _ = O.build_slots(keys, r)
        dq = O.dequantise(O.unpack_slots(slots, r))
        for n, qmax, axis in (("V", 7, 1), ("C", 127, 2), ("mu", 127, 1)):
            bound = _quant_step_bound(s[n], qmax, axis)
            assert (np.abs(dq[n] - s[n]) <= bound + 1e-15).all(), (r, n)


def test_quantised_score_error_bound():
    """|s_hat(quantised) - s_hat(unquantised)| is bounded by the decoded
    deltas. Per token, the logit (q.mu + (V^T q).c_i)/sqrt(d) of [N] §4.2
    eq. 4 moves by q.dmu + (dV^T q).c_hat_i + (V^T q).dc_i, and the
    log-sum-exp is 1-Lipschitz in the max norm (the argument of the eq. 7
    bound), so
      |ds| sqrt(d) <= |q| |dmu| + |dV^T q| max_i |c_hat_i| + |V^T q| max_i |dc_i|.
    The deltas themselves are pinned slice by slice against the quantiser
    step (test_quantised_summary_within_quantiser_step)."""
    keys = _structured_pages(50, 18)
    q = _rng(21).standard_normal((4, 128)) * 1.2
    worst = 0.0
    for r in (4, 8, 16):
        slots, s, _ = O.build_slots(keys, r)
        dq = O.dequantise(O.unpack_slots(slots, r))
        s_q = O.page_scores(q, dq["mu"], dq["V"], dq["C"])
        s_u = O.page_scores(q, s["mu"], s["V"], s["C"])
        for p in range(keys.shape[0]):
            dmu = np.linalg.norm(dq["mu"][p] - s["mu"][p])
            dVq = np.linalg.norm(q @ (dq["V"][p] - s["V"][p]), axis=1)          # (G,)
            chat = np.linalg.norm(dq["C"][p], axis=1).max()
            dc = np.linalg.norm(dq["C"][p] - s["C"][p], axis=1).max()
            Vtq = np.linalg.norm(q @ s["V"][p], axis=1)                       # (G,)
            bound = (np.linalg.norm(q, axis=1) * dmu + dVq * chat + Vtq * dc) / math.sqrt(128)
            err = np.abs(s_q[p] - s_u[p])
            assert (err <= bound + 1e-12).all(), (r, p, err, bound)
            worst = max(worst, float((err / bound).max()))
        # quantisation does move the score, by far less than a logit
        assert 1e-6 < np.abs(s_q - s_u).max() < 0.5, r
    # the bound is tight enough to mean something: some page comes within a
    # factor of 20 of it
    assert worst > 0.05, worst


# ---------------------------------------------------------------------------
# Score, shares, select ([N] §4.2 eq. 4-5)
# ---------------------------------------------------------------------------

def test_score_hand_value():
    """d = 4, B = 2, r = 1: mu = e1, v = e2, c = (1, -1), q = (2, 3, 0, 0):
    logits (2 +- 3) / 2, so s = log(e^2.5 + e^-0.5)."""
    q = np.array([[2.0, 3.0, 0.0, 0.0]])
    mu = np.array([[1.0, 0, 0, 0]])
    V = np.array([[[0.0], [1.0], [0.0], [0.0]]])
    C = np.array([[[1.0], [-1.0]]])
    assert abs(O.page_scores(q, mu, V, C)[0, 0] - math.log(math.exp(2.5) + math.exp(-0.5))) < 1e-14


def test_full_rank_summary_is_exact_lse():
    """r = B and no quantisation: the reconstruction is exact, so eq. 4 gives
    the exact page LSE."""
    keys = _structured_pages(20, 14)
    q = _rng(1).standard_normal((4, 128))
    s = O.spectral_summary(keys, 16)
    np.testing.assert_allclose(O.page_scores(q, s["mu"], s["V"], s["C"]),
                               O.exact_page_lse(q, keys), atol=1e-10)


def test_rank8_pages_exact_at_r8():
    """Pages with exact rank-8 structure (noise off): r = 8 leaves no spectral
    tail, so eta = 0 (eq. 6-7)."""
    keys = _structured_pages(20, 15, noise=0.0)
    q = _rng(2).standard_normal((4, 128))
    s = O.spectral_summary(keys, 8)
    assert (s["dropped"] < 1e-9 * s["lam"][:, 0]).all()
    np.testing.assert_allclose(O.page_scores(q, s["mu"], s["V"], s["C"]),
                               O.exact_page_lse(q, keys), atol=1e-9)


def test_eq7_tail_bound():
    """|s_hat - s| <= |q_perp| sqrt(tail) / sqrt(d) for unquantised summaries,
    q_perp taken against the page's kept basis (eq. 7)."""
    keys = _structured_pages(60, 16)
    q = _rng(3).standard_normal((4, 128)) * 2
    for r in (1, 2, 4, 8):
        s = O.spectral_summary(keys, r)
        est = O.page_scores(q, s["mu"], s["V"], s["C"])
        ex = O.exact_page_lse(q, keys)
        for p in range(keys.shape[0]):
            V = s["V"][p]
            qp = q - (q @ V) @ V.T
            bound = np.linalg.norm(qp, axis=1) * math.sqrt(s["dropped"][p]) / math.sqrt(128)
            assert (np.abs(est[p] - ex[p]) <= bound + 1e-10).all()


def test_shares_sum_to_one():
    s = _rng(4).standard_normal((50, 4)) * 3
    key, logZ = O.share_keys(s)
    assert abs(np.exp(key).sum() - 1.0) < 1e-12
    # G = 1: the group average is the per-query share itself
    key1, _ = O.share_keys(s[:, :1])
    np.testing.assert_allclose(np.exp(key1), np.exp(s[:, 0]) / np.exp(s[:, 0]).sum(), rtol=1e-12)
    # explicit eq. 5 on one page
    m = np.exp(s) / np.exp(s).sum(axis=0, keepdims=True)
    np.testing.assert_allclose(np.exp(key), m.mean(axis=1), rtol=1e-12)


def test_select_bruteforce_coverage():
    """Corollary 3 ([N] §4.2): with shares fixed, the chosen set maximises the
    group-average coverage among all budget-sized sets that contain the sink
    and the recent page; checked by enumerating every subset."""
    rng = _rng(6)
    for trial in range(40):
        P = int(rng.integers(3, 11))
        k = int(rng.integers(2, P + 1))
        s = rng.standard_normal((P, 3)) * 2
        key, _ = O.share_keys(s)
        sel = O.select_pages(key, P, k)
        assert len(sel) == min(k, P) and 0 in sel and P - 1 in sel
        best = -1
        for comb in itertools.combinations(range(1, P - 1), min(k, P) - 2):
            best = max(best, np.exp(key[list(comb)]).sum())
        got = np.exp(key[[j for j in sel if j not in (0, P - 1)]]).sum()
        assert got >= best - 1e-12


def test_select_edges_and_ties():
    assert O.select_pages(np.zeros(0), 1, 4) == [0]
    assert O.select_pages(np.zeros(1), 1, 4) == [0]
    assert O.select_pages(np.zeros(2), 2, 2) == [0, 1]
    assert O.select_pages(np.arange(6.0), 6, 9) == [0, 1, 2, 3, 4, 5]
    # equal keys: the lower page index wins
    assert O.select_pages(np.array([0, 1, 1, 1, 1, 0.0]), 6, 4) == [0, 1, 2, 5]
    assert O.select_pages(np.array([0, 1, 2, 2, 1, 0.0]), 6, 3) == [0, 2, 5]
    assert O.select_pages(np.array([5, -1, -1, -1, -1, 5.0]), 6, 2) == [0, 5]


# ---------------------------------------------------------------------------
# Attention ([N] §3.1 eq. 1; textbook decode attention)
# ---------------------------------------------------------------------------

def test_attend_matches_torch_sdpa():
    rng = _rng(7)
    q = rng.standard_normal((4, 128))
    K = rng.standard_normal((300, 128))
    V = rng.standard_normal((300, 128))
    o, _ = O.attend(q, K, V)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None], torch.tensor(K)[None], torch.tensor(V)[None])[0].numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_identity_eq1():
    """o - o_S = (1 - gamma_S) (vbar_{S^c} - vbar_S) ([N] §3.1 eq. 1), with o
    the dense output and o_S the oracle's renormalised restriction to S."""
    rng = _rng(8)
    q = rng.standard_normal((3, 128))
    K = rng.standard_normal((64, 128))
    V = rng.standard_normal((64, 128))
    S = np.sort(rng.choice(64, 20, replace=False))
    Sc = np.setdiff1d(np.arange(64), S)
    o, _ = O.attend(q, K, V)
    oS, _ = O.attend(q, K[S], V[S])
    w = np.exp(q @ K.T / math.sqrt(128))
    w /= w.sum(axis=1, keepdims=True)
    gam = w[:, S].sum(axis=1)
    vS = (w[:, S] @ V[S]) / gam[:, None]
    vSc = (w[:, Sc] @ V[Sc]) / (1 - gam)[:, None]
    np.testing.assert_allclose(o - oS, (1 - gam)[:, None] * (vSc - vS), atol=1e-12)


def test_decode_select_all_is_dense():
    b = synth.make_decode_batch([40 * 16 + 5], 1, 4, [1000], seed=21)
    q, Kp, Vp = _head_pages(b, 0, 0)
    L = int(b.seq_lens[0])
    res = O.decode_head(q, Kp, Vp, L, 1000)
    assert res["sel"] == list(range(41))
    Kt = Kp.reshape(-1, 128)[:L]
    Vt = Vp.reshape(-1, 128)[:L]
    dense, _ = O.attend(q, Kt, Vt)
    np.testing.assert_allclose(res["out"], dense, atol=1e-12)


def _head_pages(b, s, h):
    P = (int(b.seq_lens[s]) + 15) // 16
    blocks = b.block_table[s, :P].long()
    Kp = b.k_pool[blocks, h].double().numpy()
    Vp = b.v_pool[blocks, h].double().numpy()
    q = b.q[s, h * b.G:(h + 1) * b.G].double().numpy()
    return q, Kp, Vp


# ---------------------------------------------------------------------------
# Retention (Lemma 1 selector; eq. 8)
# ---------------------------------------------------------------------------

def test_exact_selector_keeps_needles_tiny():
    b = synth.config_batch("tiny")
    q, Kp, Vp = _head_pages(b, 0, 0)
    res = O.decode_head(q, Kp, Vp, int(b.seq_lens[0]), int(b.budgets[0]), mode="exact")
    for (_, _, j, _) in b.needles:
        assert j in res["sel"]
    res_q = O.decode_head(q, Kp, Vp, int(b.seq_lens[0]), int(b.budgets[0]))
    for (_, _, j, _) in b.needles:
        assert j in res_q["sel"]


@pytest.mark.slow
def test_exact_selector_keeps_needles_32k():
    b = synth.config_batch("ctx32k")
    for h in range(b.H):
        q, Kp, Vp = _head_pages(b, 0, h)
        res = O.decode_head(q, Kp, Vp, int(b.seq_lens[0]), int(b.budgets[0]), mode="exact")
        for (_, hh, j, _) in b.needles:
            if hh == h:
                assert j in res["sel"]


def test_eq8_retention_bound():
    """Coverage of the LOCKS set under exact shares is at least e^{-4 eta}
    times that of the exact-LSE set (eq. 8), eta = max |s_hat - s| (eq. 6),
    for unquantised summaries; checked at several ranks."""
    b = synth.config_batch("tiny")
    q, Kp, Vp = _head_pages(b, 0, 0)
    L, k = int(b.seq_lens[0]), int(b.budgets[0])
    P = (L + 15) // 16
    ex = O.exact_page_lse(q, Kp[:P])
    m_exact = np.exp(ex - O.logsumexp(ex, axis=0)[None, :])   # (P, G) exact shares
    for r in (1, 2, 4, 8):
        s = O.spectral_summary(Kp[:P], r)
        est = O.page_scores(q, s["mu"], s["V"], s["C"])
        eta = np.abs(est - ex).max()
        sel = O.select_pages(O.share_keys(est)[0], P, k)
        sel_ex = O.select_pages(O.share_keys(ex)[0], P, k)
        cov = m_exact[sel].sum(axis=0).mean()
        cov_ex = m_exact[sel_ex].sum(axis=0).mean()
        assert cov >= math.exp(-4 * eta) * cov_ex - 1e-12


def test_deferred_build_scores_pages_full_before_the_token():
    """Reading R17 (the build of a filled page outside the decode critical
    path, [N] §2): the step whose token completes page P-1 scores only the F-1
    pages full before that token, with the shares of eq. 5 ([N] §4.2)
    normalised over those pages (written out here), keeps page P-1 as the
    recent page, and attends the same kind of set; on a step that completes
    no page the two readings coincide."""
    b = synth.make_decode_batch([40 * 16, 40 * 16 + 5, 2 * 16], 1, 4, [9, 9, 4], seed=31)
    for s in range(3):
        Lq = int(b.seq_lens[s])
        q, Kp, Vp = _head_pages(b, s, 0)
        normal = O.decode_head(q, Kp, Vp, Lq, int(b.budgets[s]))
        defer = O.decode_head(q, Kp, Vp, Lq, int(b.budgets[s]), deferred=True)
        if Lq % 16:
            for n in ("scores", "key", "out", "lse"):
                np.testing.assert_array_equal(defer[n], normal[n])
            assert defer["sel"] == normal["sel"]
            continue
        F = Lq // 16
        P = F
        assert defer["scores"].shape[0] == F - 1
        np.testing.assert_allclose(defer["scores"], normal["scores"][:F - 1], atol=1e-12)
        S = defer["scores"]
        m = np.exp(S) / np.exp(S).sum(axis=0, keepdims=True)      # eq. 5 over pages 0..F-2
        np.testing.assert_allclose(np.exp(defer["key"]), m.mean(axis=1), rtol=1e-12)
        assert 0 in defer["sel"] and P - 1 in defer["sel"]
        assert len(defer["sel"]) == min(int(b.budgets[s]), P)
        toks = np.concatenate([Kp[j] for j in defer["sel"]]), np.concatenate([Vp[j] for j in defer["sel"]])
        np.testing.assert_allclose(defer["out"], O.attend(q, *toks)[0], atol=1e-12)
