"""Test harness: maps a paged decode batch onto the oracle's per-(sequence,
KV head) logical pages and compares GPU results with the oracle's. Test
infrastructure only."""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import locks_oracle as O

B = 16


def np64(t):
    return t.detach().to("cpu").double().numpy()


def head_pages(k_pool, v_pool, table, seq_len, s, h):
    """Logical pages (P, B, d) of one (sequence, head), fp64 numpy."""
    P = (seq_len + B - 1) // B
    blocks = table[s, :P].long().cpu()
    return np64(k_pool[blocks, h]), np64(v_pool[blocks, h])


def oracle_summaries(k_pool, table, seq_lens, H, r, num_blocks):
    """Oracle-built slots for every full page of every (seq, head), written at
    their physical block positions: uint8 [num_blocks][H][stride]."""
    stride = O.slot_layout(r)["stride"]
    summ = np.zeros((num_blocks, H, stride), dtype=np.uint8)
    kp = k_pool.detach().to("cpu")
    for s, L in enumerate(seq_lens.tolist()):
        F = L // B
        if F == 0:
            continue
        blocks = table[s, :F].long().cpu()
        for h in range(H):
            keys = kp[blocks, h].double().numpy()
            slots, _, _ = O.build_slots(keys, r)
            summ[blocks.numpy(), h] = slots
    return summ


def oracle_head(q, k_pool, v_pool, table, seq_lens, budgets, summ, s, h, G, r, mode="quantised"):
    L = int(seq_lens[s])
    Kp, Vp = head_pages(k_pool, v_pool, table, L, s, h)
    qq = np64(q[s, h * G:(h + 1) * G])
    F = L // B
    slots = None
    if summ is not None and F > 0:
        blocks = table[s, :F].long().cpu().numpy()
        slots = summ[blocks, h]
    return O.decode_head(qq, Kp, Vp, L, int(budgets[s]), slots=slots, r=r, mode=mode)


def selection_mismatch(gpu_sel, ora_sel, key, P, tol=1e-5):
    """Pages on which the two selections differ. Every such page must sit
    within `tol` (log-share units) of the oracle's selection boundary, i.e.
    the difference is a near-tie. Returns the number of differing pages."""
    g, o = set(gpu_sel), set(ora_sel)
    assert 0 in g and (P - 1) in g, (gpu_sel[:4], P)
    if g == o:
        return 0
    cand = [j for j in o if 0 < j < P - 1]
    T = min(float(key[j]) for j in cand)
    for j in g ^ o:
        assert abs(float(key[j]) - T) < tol, (j, float(key[j]), T)
    return len(g ^ o)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def gap_flags(lam, r, rel=1e-4):
    """Pages whose eigenvalues 1..r+1 have a relative gap below `rel`
    (several bases are then correct, so codes are not comparable)."""
    lam = np.asarray(lam)
    top = lam[:, : min(r + 1, lam.shape[1])]
    scale = np.maximum(np.abs(lam[:, :1]), 1e-300)
    gaps = np.abs(np.diff(top, axis=1)) / scale
    return (gaps < rel).any(axis=1)


def sign_ambiguous(V, rel=1e-6):
    """(n, r) mask of basis columns whose two largest |entries| tie within
    `rel`: the canonical sign is then not decidable across precisions."""
    a = np.sort(np.abs(V), axis=1)
    return (a[:, -1, :] - a[:, -2, :]) <= rel * np.maximum(a[:, -1, :], 1e-300)
