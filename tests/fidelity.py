"""Fidelity diagnostics of the page summaries on synthetic KV (test
infrastructure: exact values and the unquantised, quantised and centroid
summaries come from the oracle; the library's scores and selections can be
passed in to take the quantised column's place).

What is measured, per (sequence, KV head) of a decode batch whose pages are
all full, and pooled over them:
  - eta: |s_hat_jg - s_jg| over every page j and query g, the reconstruction
    error of the page log-mass ([N] §5 eq. 6 takes its maximum; the
    quantised error is reported there as measured, about twice the
    unquantised one at matched percentiles and heavy-tailed);
  - the error ladder of Fig. 1(c) ([N] §6): logit-MAE over tokens, LSE-MAE
    over pages and the Spearman rank correlation of s_hat with s over pages;
  - carrier retention vs per-head budget, Fig. 1(b): whether the page that
    holds the planted needle is in the selection S;
  - group coverage ([N] §4.2): gamma_g(S) = sum_{j in S} exp(s_jg - Z_g) with
    the exact page log-masses, averaged over the group, for the shared
    selection of eq. 5 and for the per-head oracle, which gives every query
    head its own exact top-(k-2) (G selections instead of one).
The centroid column is eq. 4 at rank 0: s_hat = q . mu / sqrt(d) + log B.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from scipy.stats import spearmanr
from threadpoolctl import threadpool_limits

from oracle import locks_oracle as O

B = 16
METHODS = ("exact", "quantised", "unquantised", "centroid")


def budget_pages(P, frac):
    """Per-head budget in pages for a fraction of the P pages (at least 3)."""
    return max(3, math.ceil(frac * P))


def token_logits(q, mu, V, C):
    """Reconstructed token logits (q . mu + (V^T q) . c_i) / sqrt(d): (P, G, B)."""
    a = mu @ q.T
    inner = np.einsum("pgr,pbr->pgb", np.einsum("pdr,gd->pgr", V, q), C)
    return (a[:, :, None] + inner) / math.sqrt(q.shape[1])


def coverage(ex, sel):
    """gamma_g(S) for each g from the exact page log-masses ex (P, G)."""
    logZ = O.logsumexp(ex, axis=0)
    idx = np.asarray(sorted(sel), dtype=np.int64)
    if idx.size == 0:
        return np.zeros(ex.shape[1])
    return np.exp(O.logsumexp(ex[idx], axis=0) - logZ)


def head_report(q, K, r, needle_page, ks, quantised_scores=None, quantised_sels=None):
    """Diagnostics of one (sequence, KV head). q (G, d) and K (P, B, d) in
    fp64 (all P pages full). ks: budgets in pages. quantised_scores (P, G) and
    quantised_sels {k: pages} replace the oracle's quantised column when given
    (the library's results). Returns a dict of per-head arrays."""
    P, _, d = K.shape
    ex = O.exact_page_lse(q, K)
    sm = O.spectral_summary(K, r)
    dq = O.dequantise(O.unpack_slots(O.build_slots(K, r)[0], r))
    scores = {
        "exact": ex,
        "unquantised": O.page_scores(q, sm["mu"], sm["V"], sm["C"]),
        "quantised": (O.page_scores(q, dq["mu"], dq["V"], dq["C"])
                      if quantised_scores is None else np.asarray(quantised_scores, np.float64)),
        "centroid": O.page_scores(q, sm["mu"], sm["V"][:, :, :0], sm["C"][:, :, :0]),
    }
    exact_logits = np.einsum("pbd,gd->pgb", K, q) / math.sqrt(d)
    rep = {"eta": {}, "logit_mae": {}, "lse_mae": {}, "spearman": {}}
    for name, (mu, V, C) in (("unquantised", (sm["mu"], sm["V"], sm["C"])),
                             ("quantised", (dq["mu"], dq["V"], dq["C"])),
                             ("centroid", (sm["mu"], sm["V"][:, :, :0], sm["C"][:, :, :0]))):
        rep["logit_mae"][name] = float(np.abs(token_logits(q, mu, V, C) - exact_logits).mean())
    for name in METHODS[1:]:
        err = np.abs(scores[name] - ex)
        rep["eta"][name] = err.ravel()
        rep["lse_mae"][name] = float(err.mean())
        rep["spearman"][name] = float(np.mean([spearmanr(scores[name][:, g], ex[:, g])[0]
                                               for g in range(q.shape[0])]))
    keys = {name: O.share_keys(s)[0] for name, s in scores.items()}
    rep["retained"] = {name: [] for name in METHODS}
    rep["coverage"] = {name: [] for name in METHODS + ("per_head",)}
    for k in ks:
        for name in METHODS:
            if name == "quantised" and quantised_sels is not None:
                sel = list(quantised_sels[k])
            else:
                sel = O.select_pages(keys[name], P, k)
            rep["retained"][name].append(needle_page in sel)
            rep["coverage"][name].append(float(coverage(ex, sel).mean()))
        per_head = [coverage(ex, O.select_pages(ex[:, g], P, k))[g] for g in range(q.shape[0])]
        rep["coverage"]["per_head"].append(float(np.mean(per_head)))
    return rep


def batch_report(batch, r, fracs, gpu=None, workers=8):
    """Pooled diagnostics over every (sequence, KV head) of `batch` (a
    synth.DecodeBatch whose sequences are whole pages, one needle per head).
    gpu: optional (scores [S][H][MP][G], {k: sel [S][H][max_budget]}) from the
    library. Returns (table dict, ks)."""
    lens = batch.seq_lens.cpu().tolist()
    assert all(L % B == 0 for L in lens)
    P = lens[0] // B
    assert all(L // B == P for L in lens)
    ks = [budget_pages(P, f) for f in fracs]
    needles = {(s, h): j for (s, h, j, _) in batch.needles}
    kp = batch.k_pool.detach().cpu()
    qs = batch.q.detach().cpu()
    table = batch.block_table.cpu()
    G = batch.G

    def one(sh):
        s, h = sh
        K = kp[table[s, :P].long(), h].double().numpy()
        q = qs[s, h * G:(h + 1) * G].double().numpy()
        qsc = qsel = None
        if gpu is not None:
            qsc = gpu[0][s, h, :P].astype(np.float64)
            qsel = {k: [int(x) for x in gpu[1][k][s, h] if x >= 0] for k in ks}
        with threadpool_limits(1):
            return head_report(q, K, r, needles[(s, h)], ks, qsc, qsel)

    pairs = [(s, h) for s in range(len(lens)) for h in range(batch.H)]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        reps = list(ex.map(one, pairs))
    out = {"pairs": len(reps), "P": P, "ks": ks, "fracs": list(fracs)}
    eta = {m: np.concatenate([rp["eta"][m] for rp in reps]) for m in METHODS[1:]}
    out["eta_pct"] = {m: {p: float(np.percentile(eta[m], p)) for p in (50, 90, 99, 99.9, 100)}
                      for m in METHODS[1:]}
    for key in ("logit_mae", "lse_mae", "spearman"):
        out[key] = {m: float(np.mean([rp[key][m] for rp in reps])) for m in reps[0][key]}
    out["retention"] = {m: np.mean([rp["retained"][m] for rp in reps], axis=0).tolist()
                        for m in METHODS}
    out["coverage"] = {m: np.mean([rp["coverage"][m] for rp in reps], axis=0).tolist()
                       for m in METHODS + ("per_head",)}
    return out


def format_report(title, rep):
    """Markdown tables of one batch_report."""
    L = [f"### {title} ({rep['pairs']} (sequence, KV head) pairs, {rep['P']} pages each)", "",
         "| eta = abs(s_hat - s) | p50 | p90 | p99 | p99.9 | max |", "|---|---|---|---|---|---|"]
    for m in METHODS[1:]:
        e = rep["eta_pct"][m]
        L.append(f"| {m} | " + " | ".join(f"{e[p]:.2e}" for p in (50, 90, 99, 99.9, 100)) + " |")
    q, u = rep["eta_pct"]["quantised"], rep["eta_pct"]["unquantised"]
    L.append("| quantised / unquantised | " + " | ".join(f"{q[p] / u[p]:.2f}" for p in (50, 90, 99, 99.9, 100)) + " |")
    L += ["", "| summary | logit-MAE | LSE-MAE | Spearman |", "|---|---|---|---|"]
    for m in ("quantised", "unquantised", "centroid"):
        L.append(f"| {m} | {rep['logit_mae'][m]:.4f} | {rep['lse_mae'][m]:.4f} | {rep['spearman'][m]:.4f} |")
    L += ["", "| budget | pages | retention exact | quantised | unquantised | centroid | "
          "coverage per-head oracle | shared exact | quantised | centroid |",
          "|---|---|---|---|---|---|---|---|---|---|"]
    for i, (f, k) in enumerate(zip(rep["fracs"], rep["ks"])):
        r, c = rep["retention"], rep["coverage"]
        L.append(f"| {100 * f:g} % | {k} | " + " | ".join(f"{r[m][i]:.3f}" for m in METHODS)
                 + " | " + " | ".join(f"{c[m][i]:.4f}" for m in ("per_head", "exact", "quantised", "centroid"))
                 + " |")
    return "\n".join(L)


# ---------------------------------------------------------------------------
# the ablation of [N] §6: rank x basis precision, and the GQA merge rule
# ---------------------------------------------------------------------------

def exact_heads(batch):
    """Per (sequence, KV head): (q (G, d), exact page LSE (P, G), needle page)
    for a batch of whole-page sequences of equal length."""
    lens = batch.seq_lens.cpu().tolist()
    P = lens[0] // B
    assert all(L == P * B for L in lens)
    needles = {(s, h): j for (s, h, j, _) in batch.needles}
    kp, qs, table, G = batch.k_pool.detach().cpu(), batch.q.detach().cpu(), batch.block_table.cpu(), batch.G
    out = {}
    for s in range(len(lens)):
        for h in range(batch.H):
            K = kp[table[s, :P].long(), h].double().numpy()
            q = qs[s, h * G:(h + 1) * G].double().numpy()
            out[(s, h)] = (q, O.exact_page_lse(q, K), needles.get((s, h)))
    return out, P


def precision_row(heads, P, scores, sels, ks):
    """One (rank, width) row: median and p99 |s_hat - s| over pages and query
    heads, carrier retention and mean group coverage at each budget, from the
    library's scores ((s, h) -> (P, G)) and selections ((s, h) -> {k: pages})."""
    err = np.concatenate([np.abs(scores[sh] - ex).ravel() for sh, (_, ex, _) in heads.items()])
    ret = [np.mean([nd in sels[sh][k] for sh, (_, _, nd) in heads.items()]) for k in ks]
    cov = [np.mean([coverage(ex, sels[sh][k]).mean() for sh, (_, ex, _) in heads.items()]) for k in ks]
    return dict(eta_p50=float(np.median(err)), eta_p99=float(np.percentile(err, 99)),
                retention=[float(x) for x in ret], coverage=[float(x) for x in cov])


def merge_row(heads, P, sels, ks):
    """Coverage statistics of one merge rule's selections ((s, h) -> {k:
    pages}, or {k: [pages of query head g]} for per-head selections): the
    mean over query heads, the mean of the worst head of each group, and the
    5th percentile over all query heads; None = the per-head oracle (each
    query head's own exact top-(k-2))."""
    rows = []
    for k in ks:
        per = []
        for sh, (q, ex, _) in heads.items():
            if sels is None:
                c = np.array([coverage(ex, O.select_pages(ex[:, g], P, k))[g] for g in range(ex.shape[1])])
            elif sels[sh][k] and isinstance(sels[sh][k][0], list):
                c = np.array([coverage(ex, sel)[g] for g, sel in enumerate(sels[sh][k])])
            else:
                c = coverage(ex, sels[sh][k])
            per.append(c)
        allc = np.concatenate(per)
        rows.append(dict(mean=float(allc.mean()), worst_head=float(np.mean([c.min() for c in per])),
                         p5=float(np.percentile(allc, 5))))
    return rows
