"""Fidelity of the page summaries on synthetic KV ([N] §5: quantised error
measured, about twice the unquantised one at matched percentiles, heavy-tailed;
[N] §6 Fig. 1(b)-(c): carrier retention down to 0.5 % budgets and the error
ladder; [N] §4.2: shared selection a little below the per-head oracle's
coverage). The CPU tests pin the oracle's numbers; the GPU test takes the
quantised column from the library and prints the full tables."""
import numpy as np
import pytest
import torch

import synth
from oracle import locks_oracle as O
from tests import fidelity as F

FRACS = (0.005, 0.01, 0.02, 0.05, 0.1)


def _eta(sigmas, n=4096, seed=5):
    g = torch.Generator().manual_seed(seed)
    K = synth.page_keys(n, g, sigmas=sigmas).to(torch.bfloat16).double().numpy()
    q = torch.randn(4, 128, generator=g).double().numpy()
    ex = O.exact_page_lse(q, K)
    sm = O.spectral_summary(K, 8)
    dq = O.dequantise(O.unpack_slots(O.build_slots(K, 8)[0], 8))
    un = np.abs(O.page_scores(q, sm["mu"], sm["V"], sm["C"]) - ex).ravel()
    qz = np.abs(O.page_scores(q, dq["mu"], dq["V"], dq["C"]) - ex).ravel()
    return un, qz


def test_quantised_error_about_twice_unquantised_with_a_spectral_tail():
    """Keys with a slowly decaying spectrum (sigma_k = 3 k^-0.5 over all 15
    centred directions): the int4/int8 summary's error is 1.5-2.5x the
    unquantised rank-8 error at matched percentiles (p50 1.93 on this seed),
    and heavy-tailed: its maximum over 16384 (page, query) pairs is more than
    ten times its median."""
    un, qz = _eta(synth.TAIL_SIGMAS)
    for p in (50, 90, 99):
        ratio = np.percentile(qz, p) / np.percentile(un, p)
        assert 1.5 < ratio < 2.5, (p, ratio)
    assert qz.max() > 10 * np.median(qz)


def test_quantiser_floor_dominates_near_rank8_keys():
    """With near rank-8 pages the unquantised error is only the noise tail, so
    the quantiser's floor (about the same median as above) dominates: the
    ratio is well above 2 there. The ratio measures the tail, not the codec."""
    un, qz = _eta(synth.SIGMAS)
    _, qz_tail = _eta(synth.TAIL_SIGMAS)
    assert np.percentile(qz, 50) / np.percentile(un, 50) > 5
    assert 0.5 < np.median(qz) / np.median(qz_tail) < 2


def test_fidelity_report_small_batch():
    """Retention, coverage and the error ladder on 2 x 2 (sequence, KV head)
    pairs of 1024 pages (oracle only): the exact and summary selectors keep
    every needle from 2 % up, the centroid keeps fewer; the per-head oracle's
    coverage bounds the shared one's; rank correlations are near 1 and the
    ladder is ordered unquantised < quantised < centroid."""
    b = synth.make_decode_batch([16384] * 2, 2, 4, [32] * 2, seed=31, needles_per_head=1,
                                sigmas=synth.TAIL_SIGMAS)
    rep = F.batch_report(b, 8, (0.02, 0.05), workers=4)
    assert rep["retention"]["exact"] == [1.0, 1.0]
    assert rep["retention"]["quantised"] == [1.0, 1.0]
    assert rep["retention"]["centroid"][0] < 1.0
    for i in range(2):
        assert rep["coverage"]["per_head"][i] >= rep["coverage"]["exact"][i] - 1e-12
        assert abs(rep["coverage"]["quantised"][i] - rep["coverage"]["exact"][i]) < 2e-3
    for key in ("logit_mae", "lse_mae"):
        v = rep[key]
        assert v["unquantised"] < v["quantised"] < v["centroid"]
    assert rep["spearman"]["quantised"] > 0.999


def test_coverage_and_retention_by_hand():
    """coverage() on a hand-made score table, and the rank-0 centroid score."""
    ex = np.log(np.array([[1.0, 2.0], [3.0, 2.0], [6.0, 4.0]]))
    np.testing.assert_allclose(F.coverage(ex, [0, 2]), [0.7, 0.75], atol=1e-15)
    np.testing.assert_allclose(F.coverage(ex, []), [0.0, 0.0])
    K = np.random.default_rng(0).standard_normal((3, 16, 128))
    q = np.random.default_rng(1).standard_normal((2, 128))
    sm = O.spectral_summary(K, 8)
    cen = O.page_scores(q, sm["mu"], sm["V"][:, :, :0], sm["C"][:, :, :0])
    np.testing.assert_allclose(cen, K.mean(axis=1) @ q.T / np.sqrt(128) + np.log(16), atol=1e-12)
    assert F.budget_pages(2048, 0.005) == 11 and F.budget_pages(100, 0.005) == 3


def _gpu_quantised(b, ks, r=8):
    from kv_cache_page_amd import locks as L
    dev = "cuda"
    dims = L.Dims(b.H, b.G, r)
    S, MP = b.num_seqs, b.max_pages
    kp = b.k_pool.to(dev)
    table = b.block_table.to(dev)
    lens = b.seq_lens.to(dev)
    q = b.q.to(dev)
    summ = L.alloc_summaries(dims, b.num_blocks, dev)
    L.build(dims, kp, torch.arange(b.num_blocks, dtype=torch.int32, device=dev), summ)
    scores = torch.empty(S, b.H, MP, b.G, device=dev)
    L.score_pages(dims, q, summ, table, lens, scores)
    kmax = max(ks)
    ws = L.alloc_workspace(dims, S, MP, kmax, dev)
    sels = {}
    for k in ks:
        sel = torch.empty(S, b.H, kmax, dtype=torch.int32, device=dev)
        cnt = torch.empty(S, b.H, dtype=torch.int32, device=dev)
        budgets = torch.full((S,), k, dtype=torch.int32, device=dev)
        L.score_select(dims, q, summ, table, lens, budgets, kmax, sel, cnt, ws)
        torch.cuda.synchronize()
        assert (cnt.cpu() == k).all()
        sels[k] = sel.cpu().numpy()
    torch.cuda.synchronize()
    return scores.cpu().numpy(), sels


@pytest.mark.gpu
@pytest.mark.parametrize("family", ["near_rank8", "spectral_tail"])
def test_gpu_fidelity_tables(family):
    """The library's scores and selections (4 sequences x 8 KV heads, 32768
    tokens, one needle per head) against the exact page log-masses: prints
    the tables and checks the pages' qualitative claims."""
    sig = synth.SIGMAS if family == "near_rank8" else synth.TAIL_SIGMAS
    b = synth.make_decode_batch([32768] * 4, 8, 4, [64] * 4, seed=21, needles_per_head=1,
                                sigmas=sig)
    ks = [F.budget_pages(2048, f) for f in FRACS]
    scores, sels = _gpu_quantised(b, ks)
    rep = F.batch_report(b, 8, FRACS, gpu=(scores, sels), workers=16)
    print("\n" + F.format_report(f"{family} keys, library scores", rep), flush=True)
    e = rep["eta_pct"]
    if family == "spectral_tail":
        assert 1.4 < e["quantised"][50] / e["unquantised"][50] < 2.8
    assert e["quantised"][100] > 5 * e["quantised"][50]
    assert rep["spearman"]["quantised"] > 0.999
    r = rep["retention"]
    assert all(x == 1.0 for x in r["exact"])
    assert all(x >= 0.85 for x in r["quantised"])
    assert all(x == 1.0 for x in r["quantised"][1:])
    assert r["centroid"][0] < 0.5
    c = rep["coverage"]
    for i in range(len(FRACS)):
        assert c["per_head"][i] >= c["exact"][i] - 1e-12
        assert abs(c["quantised"][i] - c["exact"][i]) < 2e-3


def _scaled_batch(lens, H, seed, budgets=None):
    """Whole-page sequences with a spectral tail; the query heads of a group
    get norms x0.5 .. x2, so their page-mass normalisers Z_g differ."""
    b = synth.make_decode_batch(lens, H, 4, budgets or [32] * len(lens), seed=seed,
                                sigmas=synth.TAIL_SIGMAS)
    scale = torch.linspace(0.5, 2.0, 4).repeat(H)
    b.q = (b.q.float() * scale[None, :, None]).to(torch.bfloat16)
    return b


def test_merge_rule_coverage_ordering():
    """[N] §4.2 Corollary 3 and the ablation of [N] §6, on exact page masses
    (oracle): the share average's group-average coverage is at least that of
    group-max and group-mass (the corollary: it maximises the group-average
    coverage among shared rules) and at most the per-head oracle's; on these
    inputs it also leads on the worst head of each group and the 5th
    percentile, as the pages report."""
    b = _scaled_batch([8192] * 2, 4, 31)
    heads, P = F.exact_heads(b)
    ks = [F.budget_pages(P, f) for f in (0.02, 0.05, 0.1)]
    rows = {m: F.merge_row(heads, P, {sh: {k: O.select_pages(O.share_keys(ex, m)[0], P, k)
                                           for k in ks} for sh, (_, ex, _) in heads.items()}, ks)
            for m in ("share", "max", "mass")}
    per_head = F.merge_row(heads, P, None, ks)
    for i in range(len(ks)):
        sh = rows["share"][i]
        for m in ("max", "mass"):
            assert sh["mean"] >= rows[m][i]["mean"] - 1e-12
            assert sh["worst_head"] > rows[m][i]["worst_head"] and sh["p5"] > rows[m][i]["p5"]
        assert per_head[i]["mean"] >= sh["mean"] - 1e-12


@pytest.mark.gpu
def test_gpu_ablation_tables():
    """The ablation of [N] §6 through the library: rank x basis width (score
    error, carrier retention and coverage from the library's own builds,
    scores and selections) and the merge rule (coverage statistics of the
    library's selections). 2 sequences x 8 KV heads x 2048 pages."""
    from kv_cache_page_amd import locks as L
    dev = "cuda"
    b = _scaled_batch([32768] * 2, 8, 41, budgets=[64] * 2)
    heads, P = F.exact_heads(b)
    fracs = (0.005, 0.01, 0.05)
    ks = [F.budget_pages(P, f) for f in fracs]
    kmax = max(ks)
    S, H, MP = b.num_seqs, b.H, b.max_pages
    kp, table, lens, q = b.k_pool.to(dev), b.block_table.to(dev), b.seq_lens.to(dev), b.q.to(dev)
    ids = torch.arange(b.num_blocks, dtype=torch.int32, device=dev)

    def run(dims):
        summ = L.alloc_summaries(dims, b.num_blocks, dev)
        L.build(dims, kp, ids, summ)
        per_head = dims.merge_rule == L.MERGE_PER_HEAD
        scn = None
        if not per_head:
            sc = torch.empty(S, H, MP, b.G, device=dev)
            L.score_pages(dims, q, summ, table, lens, sc)
            torch.cuda.synchronize()
            scn = sc.cpu().numpy()
        ws = L.alloc_workspace(dims, S, MP, kmax, dev)
        rows = L.selection_heads(dims)
        sels = {sh: {} for sh in heads}
        for k in ks:
            sel = torch.empty(S, rows, kmax, dtype=torch.int32, device=dev)
            cnt = torch.empty(S, rows, dtype=torch.int32, device=dev)
            L.score_select(dims, q, summ, table, lens, torch.full((S,), k, dtype=torch.int32,
                                                                   device=dev), kmax, sel, cnt, ws)
            torch.cuda.synchronize()
            sl, cn = sel.cpu().numpy(), cnt.cpu().numpy()
            for (s, h) in heads:
                if per_head:   # one page list per query head
                    sels[(s, h)][k] = [[int(x) for x in sl[s, h * b.G + g, :cn[s, h * b.G + g]]]
                                       for g in range(b.G)]
                else:
                    sels[(s, h)][k] = [int(x) for x in sl[s, h, :cn[s, h]]]
        if scn is None:
            return None, sels
        return {(s, h): scn[s, h, :P].astype(np.float64) for (s, h) in heads}, sels

    lines = [f"### rank x basis width ({len(heads)} (sequence, KV head) pairs, {P} pages)", "",
             "| r | basis | eta p50 | eta p99 | retention " + " / ".join(f"{100 * f:g}%" for f in fracs)
             + " | coverage " + " / ".join(f"{100 * f:g}%" for f in fracs) + " |",
             "|---|---|---|---|---|---|"]
    prec = {}
    for r in (4, 8, 16):
        for bits in (8, 4, 2):
            sc, sels = run(L.Dims(H, 4, r, basis_bits=bits))
            row = F.precision_row(heads, P, sc, sels, ks)
            prec[(r, bits)] = row
            lines.append(f"| {r} | int{bits} | {row['eta_p50']:.2e} | {row['eta_p99']:.2e} | "
                         + " / ".join(f"{x:.3f}" for x in row["retention"]) + " | "
                         + " / ".join(f"{x:.4f}" for x in row["coverage"]) + " |")
    lines += ["", "### merge rule (r = 8, int4)", "",
              "| rule | " + " | ".join(f"{100 * f:g}%: mean / worst head / p5" for f in fracs) + " |",
              "|---|---|---|---|"]
    merge = {}
    for rule in ("share", "max", "mass"):
        _, sels = run(L.Dims(H, 4, 8, merge_rule=rule))
        merge[rule] = F.merge_row(heads, P, sels, ks)
    _, sels = run(L.Dims(H, 4, 8, merge_rule="per_head"))
    merge["per-head (library)"] = F.merge_row(heads, P, sels, ks)
    merge["per-head oracle"] = F.merge_row(heads, P, None, ks)
    for rule, rows in merge.items():
        lines.append(f"| {rule} | " + " | ".join(
            f"{x['mean']:.4f} / {x['worst_head']:.4f} / {x['p5']:.4f}" for x in rows) + " |")
    print("\n" + "\n".join(lines), flush=True)
    # int8 tracks int4 or better (at r = 4 the rank, not the width, sets the
    # error), int2 is far worse; from r = 8 the width shows
    for r in (4, 8, 16):
        assert prec[(r, 8)]["eta_p50"] < 1.05 * prec[(r, 4)]["eta_p50"]
        assert prec[(r, 2)]["eta_p50"] > 1.5 * prec[(r, 4)]["eta_p50"]
        assert min(prec[(r, 8)]["retention"]) >= min(prec[(r, 2)]["retention"])
    for r in (8, 16):
        assert prec[(r, 8)]["eta_p50"] < prec[(r, 4)]["eta_p50"]
    for i in range(len(ks)):
        for rule in ("max", "mass"):
            assert merge["share"][i]["mean"] >= merge[rule][i]["mean"] - 2e-3
        assert merge["per-head oracle"][i]["mean"] >= merge["share"][i]["mean"] - 2e-3
        # the library's per-head selection, from quantised scores, keeps up
        # with the exact per-head oracle and leads every shared rule
        assert merge["per-head (library)"][i]["mean"] >= merge["per-head oracle"][i]["mean"] - 2e-3
        assert merge["per-head (library)"][i]["mean"] >= merge["share"][i]["mean"]
