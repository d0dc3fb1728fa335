"""Oracle pins of the ablation variants ([N] §6, rank x precision and the GQA
merge rule; readings R18 and R19): slot sizes and bytes of the int8 and int2
bases by hand, exact round trips, the quantiser step bound, the merge rules'
special cases and inequalities, and the ablation's measured ordering on
synthetic keys."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import locks_oracle as O


@pytest.mark.parametrize("bits,payload,stride", [(2, 562, 640), (4, 818, 896), (8, 1330, 1408)])
def test_slot_sizes_by_bits(bits, payload, stride):
    L = O.slot_layout(8, basis_bits=bits)
    # basis r * d * bits / 8, coefficients 16 r, centroid 128, 25 fp16 scales
    assert L["payload"] == 8 * 128 * bits // 8 + 128 + 128 + 50 == payload
    assert L["stride"] == stride and L["c"] == 8 * 128 * bits // 8


def _one_column(codes, bits, scale=1.0):
    """Codes of a rank-1 basis column (128 dims), other fields zero."""
    qs = dict(Vq=np.asarray(codes, dtype=np.int64).reshape(1, 128, 1),
              sV=np.array([[scale]], dtype=np.float16),
              Cq=np.zeros((1, 16, 1), dtype=np.int64), sC=np.zeros((1, 16), dtype=np.float16),
              muq=np.zeros((1, 128), dtype=np.int64), smu=np.zeros(1, dtype=np.float16))
    return qs, O.pack_slots(qs, basis_bits=bits)


def test_int2_bytes_by_hand():
    codes = np.zeros(128, dtype=np.int64)
    codes[:8] = [-1, 0, 1, -1, 1, 1, 0, -1]
    codes[127] = 1
    _, buf = _one_column(codes, 2)
    # four dims per byte, lowest bits first, two's complement two-bit fields:
    # (-1, 0, 1, -1) -> 3 | 0 << 2 | 1 << 4 | 3 << 6
    assert buf[0, 0] == 3 | (0 << 2) | (1 << 4) | (3 << 6) == 211
    assert buf[0, 1] == 1 | (1 << 2) | (0 << 4) | (3 << 6) == 197
    assert buf[0, 31] == 1 << 6
    assert not buf[0, 2:31].any()
    back = O.unpack_slots(buf, 1, basis_bits=2)
    assert np.array_equal(back["Vq"][0, :, 0], codes)


def test_int8_bytes_by_hand():
    codes = np.zeros(128, dtype=np.int64)
    codes[0], codes[1], codes[77], codes[127] = -5, 127, -127, 3
    _, buf = _one_column(codes, 8)
    assert buf[0, 0] == 0xFB and buf[0, 1] == 0x7F and buf[0, 77] == 0x81 and buf[0, 127] == 3
    assert np.count_nonzero(buf[0, :128]) == 4
    assert np.array_equal(O.unpack_slots(buf, 1, basis_bits=8)["Vq"][0, :, 0], codes)


@pytest.mark.parametrize("bits", [2, 8])
def test_exactly_representable_round_trip(bits):
    """A summary whose basis entries are codes times power-of-two scales, each
    column reaching +-qmax, quantises to exactly those codes and back."""
    rng = np.random.default_rng(bits)
    qmax = O.qmax_of(bits)
    n, r = 5, 6
    codes = rng.integers(-qmax, qmax + 1, size=(n, 128, r))
    codes[:, 0, :] = qmax
    codes[:, 1, :] = -qmax
    scales = 2.0 ** rng.integers(-9, -2, size=(n, r))
    V = codes * scales[:, None, :]
    s = dict(V=V, C=np.zeros((n, 16, r)), mu=np.zeros((n, 128)))
    qs = O.quantise_summary(s, basis_bits=bits)
    assert np.array_equal(qs["Vq"], codes)
    buf = O.pack_slots(qs, basis_bits=bits)
    back = O.dequantise(O.unpack_slots(buf, r, basis_bits=bits))
    assert np.array_equal(back["V"], V)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_basis_within_half_a_step(bits):
    g = torch.Generator().manual_seed(11)
    K = synth.page_keys(64, g).to(torch.bfloat16).double().numpy()
    buf, s, qs = O.build_slots(K, 8, basis_bits=bits)
    dq = O.dequantise(O.unpack_slots(buf, 8, basis_bits=bits))
    step = qs["sV"].astype(np.float64)[:, None, :]
    qmax = O.qmax_of(bits)
    # half a step, plus the fp16 rounding of the scale times qmax at the ends
    rel = np.abs(s["V"]).max(axis=1, keepdims=True) * 2.0 ** -10
    assert (np.abs(dq["V"] - s["V"]) <= 0.5 * step + qmax * rel + 1e-15).all()
    with pytest.raises(ValueError):
        O.qmax_of(3)


def _scores(G, n=50, seed=3):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(n, G)) * 2.0 + rng.normal(size=(1, G)) * 3.0


def test_merge_rules_agree_for_one_query_head():
    s = _scores(1)
    k0, _ = O.share_keys(s, "share")
    for rule in ("max", "mass"):
        np.testing.assert_allclose(O.share_keys(s, rule)[0], k0, atol=1e-12)


def test_merge_rule_inequalities_and_sums():
    s = _scores(4)
    share, logZ = O.share_keys(s, "share")
    mx, _ = O.share_keys(s, "max")
    mass, _ = O.share_keys(s, "mass")
    # max_g m_g >= mean_g m_g >= max_g m_g / G
    assert (mx >= share - 1e-12).all() and (mx <= share + math.log(4) + 1e-12).all()
    # the shares and the pooled masses are distributions over the pages
    assert abs(np.exp(share).sum() - 1.0) < 1e-12 and abs(np.exp(mass).sum() - 1.0) < 1e-12
    assert np.exp(mx).sum() >= 1.0 - 1e-12
    # pooled mass weighs each head by its own Z_g: equal to the share average
    # exactly when every Z_g is the same (columns that are permutations)
    base = s[:, 0]
    perm = np.stack([base, base[::-1], np.roll(base, 7), np.roll(base, 19)], axis=1)
    np.testing.assert_allclose(O.share_keys(perm, "mass")[0], O.share_keys(perm, "share")[0],
                               atol=1e-12)
    assert np.abs(mass - share).max() > 1e-3          # and differs otherwise
    with pytest.raises(ValueError):
        O.share_keys(s, "vote")


def test_group_max_keeps_a_page_one_head_alone_wants():
    """A page that only query head 3 rates highly: its group-max key is that
    head's share, its share-average key a quarter of it."""
    s = np.zeros((20, 4))
    s[7, 3] = 6.0
    share, _ = O.share_keys(s, "share")
    mx, _ = O.share_keys(s, "max")
    assert np.argmax(mx) == 7 and np.argmax(share) == 7
    m3 = np.exp(6.0) / (19 + np.exp(6.0))          # head 3's share of page 7
    m0 = 1.0 / 20                                   # the other heads' (uniform)
    np.testing.assert_allclose(np.exp(mx[7]), m3, rtol=1e-12)
    np.testing.assert_allclose(np.exp(share[7]), (m3 + 3 * m0) / 4, rtol=1e-12)


def test_precision_ablation_ordering():
    """[N] §6: int8 tracks the unquantised basis, int4 loses some and stops
    improving past a moderate rank, int2 falls most of the way to the
    centroid. Median score errors on slowly decaying spectra (4096 pages)."""
    g = torch.Generator().manual_seed(5)
    K = synth.page_keys(4096, g, sigmas=synth.TAIL_SIGMAS).to(torch.bfloat16).double().numpy()
    q = torch.randn(4, 128, generator=g).double().numpy()
    ex = O.exact_page_lse(q, K)

    def err(r, bits=None):
        if bits is None:
            sm = O.spectral_summary(K, r)
            return np.median(np.abs(O.page_scores(q, sm["mu"], sm["V"], sm["C"]) - ex))
        dq = O.dequantise(O.unpack_slots(O.build_slots(K, r, basis_bits=bits)[0], r, basis_bits=bits))
        return np.median(np.abs(O.page_scores(q, dq["mu"], dq["V"], dq["C"]) - ex))

    sm = O.spectral_summary(K, 8)
    cen = np.median(np.abs(O.page_scores(q, sm["mu"], sm["V"][:, :, :0], sm["C"][:, :, :0]) - ex))
    un8, i8, i4, i2 = err(8), err(8, 8), err(8, 4), err(8, 2)
    assert un8 < i8 < 1.5 * un8 < i4
    assert 3 * i4 < i2 < cen
    assert err(16, 4) > 0.8 * i4                  # int4: little gain from r = 8 to 16
    assert err(16) < 1e-12 < err(16, 8)           # unquantised exact at full rank, int8 not


# ---------------------------------------------------------------------------
# per-head selection (reading R19: the per-head oracle of [N] §4.2 and §6)
# ---------------------------------------------------------------------------

def _small_head(G, seed, P=9, tail=5):
    rng = np.random.default_rng(seed)
    K = rng.normal(size=(P, 16, 128))
    V = rng.normal(size=(P, 16, 128))
    q = rng.normal(size=(G, 128)) * 0.4
    return q, K, V, 16 * (P - 1) + tail


def test_per_head_with_one_query_head_is_the_share_rule():
    q, K, V, ln = _small_head(1, 21)
    a = O.decode_head(q, K, V, ln, 5, merge="share")
    b = O.decode_head(q, K, V, ln, 5, merge="per_head")
    assert b["sel"] == [a["sel"]]
    np.testing.assert_array_equal(b["out"], a["out"])
    np.testing.assert_array_equal(b["lse"], a["lse"])


def test_per_head_rows_are_single_query_decodes():
    """Query head g's selection and output are those of a decode of query g
    alone: the per-head path pairs every query with its own page set."""
    q, K, V, ln = _small_head(4, 22)
    slots = O.build_slots(K[:8], 8)[0]
    ph = O.decode_head(q, K, V, ln, 4, slots=slots, merge="per_head")
    assert len(ph["sel"]) == 4 and len({tuple(s) for s in ph["sel"]}) > 1  # the heads disagree
    for g in range(4):
        one = O.decode_head(q[g:g + 1], K, V, ln, 4, slots=slots, merge="share")
        assert ph["sel"][g] == one["sel"]
        np.testing.assert_array_equal(ph["out"][g], one["out"][0])
        np.testing.assert_array_equal(ph["lse"][g], one["lse"][0])


def test_per_head_maximises_each_heads_own_coverage():
    """Brute force over every k-set with the sink and the recent page: query
    head g's own selection has the largest coverage sum_{j in S} m_g(j) that
    any such set reaches (Corollary 3 with G = 1), so it covers at least as
    much of head g as the group's shared selection does."""
    import itertools
    rng = np.random.default_rng(7)
    P, k, G = 9, 4, 4
    s = rng.normal(size=(P, G)) * 1.5
    key, logZ = O.share_keys(s, "per_head")
    m = np.exp(key)                                   # m_g(j)
    shared = O.select_pages(O.share_keys(s, "share")[0], P, k)
    best = [max(sum(m[j, g] for j in (0, P - 1) + c)
                for c in itertools.combinations(range(1, P - 1), k - 2)) for g in range(G)]
    for g in range(G):
        own = O.select_pages(key[:, g], P, k)
        cov = m[own, g].sum()
        assert abs(cov - best[g]) < 1e-12
        assert cov >= m[shared, g].sum() - 1e-12
    np.testing.assert_allclose(m.sum(axis=0), 1.0, atol=1e-12)


def test_per_head_with_identical_query_heads_matches_the_shared_set():
    q, K, V, ln = _small_head(1, 23)
    q4 = np.repeat(q, 4, axis=0)
    ph = O.decode_head(q4, K, V, ln, 5, merge="per_head")
    sh = O.decode_head(q4, K, V, ln, 5, merge="share")
    assert all(sel == sh["sel"] for sel in ph["sel"])
    np.testing.assert_allclose(ph["out"], sh["out"], atol=1e-12)
