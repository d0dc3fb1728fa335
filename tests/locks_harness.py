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


def oracle_summaries(k_pool, table, seq_lens, H, r, num_blocks, basis_bits=4):
    """Oracle-built slots for every full page of every (seq, head), written at
    their physical block positions: uint8 [num_blocks][H][stride]."""
    stride = O.slot_layout(r, basis_bits=basis_bits)["stride"]
    summ = np.zeros((num_blocks, H, stride), dtype=np.uint8)
    kp = k_pool.detach().to("cpu")
    for s, L in enumerate(seq_lens.tolist()):
        F = L // B
        if F == 0:
            continue
        blocks = table[s, :F].long().cpu()
        for h in range(H):
            keys = kp[blocks, h].double().numpy()
            slots, _, _ = O.build_slots(keys, r, basis_bits=basis_bits)
            summ[blocks.numpy(), h] = slots
    return summ


def oracle_head(q, k_pool, v_pool, table, seq_lens, budgets, summ, s, h, G, r, mode="quantised",
                deferred=False, basis_bits=4, merge="share"):
    L = int(seq_lens[s])
    Kp, Vp = head_pages(k_pool, v_pool, table, L, s, h)
    qq = np64(q[s, h * G:(h + 1) * G])
    F = (max(L - 1, 0) if deferred else L) // B
    slots = None
    if summ is not None and F > 0:
        blocks = table[s, :F].long().cpu().numpy()
        slots = summ[blocks, h]
    return O.decode_head(qq, Kp, Vp, L, int(budgets[s]), slots=slots, r=r, mode=mode,
                         deferred=deferred, basis_bits=basis_bits, merge=merge)


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


def plant_boundary(summ, block_table, q, seq_len, k, h, G, r, gap, n_side=3, rng=None):
    """Move the keys of the 2 n_side candidates ranked around the selection
    boundary of (sequence 0, KV head h) onto a ladder of spacing `gap`
    (log-share units): n_side members just above the boundary and n_side
    non-members just below, every consecutive pair `gap` apart. A page's key
    is moved by changing centroid codes (never one at +-127, so the scale
    stays), which shifts all 16 logits of the page, hence its score, by
    q_g . dmu / sqrt(d) exactly. Rewrites the slots in `summ` in place
    (uint8 [blocks][H][stride]) with the oracle's packer and returns the
    oracle's keys after planting (test infrastructure: slots in, slots out)."""
    rng = np.random.default_rng(0) if rng is None else rng
    P = (seq_len + B - 1) // B
    F = seq_len // B
    blocks = block_table[0, :F].long().cpu().numpy()
    qq = np64(q[0, h * G:(h + 1) * G])
    d = qq.shape[1]

    def keys_now():
        dq = O.dequantise(O.unpack_slots(summ[blocks, h], r))
        s = O.page_scores(qq, dq["mu"], dq["V"], dq["C"])
        key, logZ = O.share_keys(s)
        return key, s, logZ

    key, s, logZ = keys_now()
    cand = sorted(range(1, P - 1), key=lambda j: (-float(key[j]), j))
    top = cand[k - 2 - n_side:k - 2 + n_side]           # ranks around the boundary
    centre = 0.5 * (float(key[cand[k - 3]]) + float(key[cand[k - 2]]))
    # targets: members centre + gap/2 + i gap, non-members centre - gap/2 - i gap
    targets = [centre + gap * (n_side - 0.5 - i) for i in range(2 * n_side)]
    for _ in range(3):                                   # Z moves a little: refine
        for j, tgt in zip(top, targets):
            blk = int(blocks[j])
            u = O.unpack_slots(summ[blk, h][None], r)
            smu = float(u["smu"][0])
            for _step in range(8):
                kj = O.share_keys(s)[0]                  # current keys (Z of now)
                resid = tgt - float(kj[j])
                if abs(resid) < 1e-7 * max(1.0, gap / 1e-5):
                    break
                w = np.exp(s[j] - logZ)                  # d key_j / d s_jg, normalised below
                w = w / w.sum()
                eff = (w @ qq) * smu / math.sqrt(d)      # key change per +1 code, per dim
                free = np.abs(u["muq"][0]) < 126
                # single moves (+-1, +-2 on one dim) and paired moves (+1 on
                # dim a, -1 on dim b), whose net effect can be arbitrarily small
                moves = []
                for stepc in (1, -1, 2, -2):
                    e = np.where(free, eff * stepc, np.inf)
                    i = int(np.argmin(np.abs(resid - e)))
                    moves.append((abs(resid - e[i]), [(i, stepc)]))
                pair = eff[:, None] - eff[None, :]
                ok = free[:, None] & free[None, :] & ~np.eye(d, dtype=bool)
                pe = np.where(ok, np.abs(resid - pair), np.inf)
                a_, b_ = np.unravel_index(int(np.argmin(pe)), pe.shape)
                moves.append((float(pe[a_, b_]), [(int(a_), 1), (int(b_), -1)]))
                best, change = min(moves, key=lambda m: m[0])
                if best >= abs(resid):
                    break
                for i, stepc in change:
                    u["muq"][0, i] += stepc
                summ[blk, h] = O.pack_slots(u)[0]
                dq = O.dequantise(O.unpack_slots(summ[blk, h][None], r))
                s[j] = O.page_scores(qq, dq["mu"], dq["V"], dq["C"])[0]
        key, s, logZ = keys_now()
    return key, top


def bf16_bits_to_f64(u16):
    """uint16 array holding bf16 bit patterns -> float64 (exact)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def oracle_pair_job(args):
    """One (sequence, KV head) of a decode batch through the oracle, in a worker
    process: build the slots of its full pages, then score, select and attend
    (CPU only; inputs are bf16 bit patterns). Returns (slots, sel, key, out, lse)."""
    keys_u16, vals_u16, q, seq_len, budget, r = args
    Kp = bf16_bits_to_f64(keys_u16)
    Vp = bf16_bits_to_f64(vals_u16)
    F = seq_len // B
    slots = O.build_slots(Kp[:F], r)[0] if F else np.zeros((0, O.slot_layout(r)["stride"]), np.uint8)
    res = O.decode_head(q, Kp, Vp, seq_len, budget, slots=slots, r=r)
    return slots, res["sel"], res["key"], res["out"], res["lse"]


def oracle_pairs_parallel(k_pool, v_pool, q, table, seq_lens, budgets, H, G, r, workers=None):
    """oracle_pair_job for every (sequence, KV head) of a batch over a pool of
    threads (numpy releases the interpreter lock inside LAPACK and large array
    operations). k_pool / v_pool / q / table are CPU tensors.
    Returns {(s, h): result}."""
    import concurrent.futures
    import os
    if workers is None:
        try:
            workers = len(os.sched_getaffinity(0))
        except AttributeError:
            workers = os.cpu_count() or 1
        workers = max(1, min(16, workers))
    kp16 = k_pool.view(torch.int16).numpy().view(np.uint16)
    vp16 = v_pool.view(torch.int16).numpy().view(np.uint16)

    def job(s, h, L):
        P = (L + B - 1) // B
        blocks = table[s, :P].long().numpy()
        return oracle_pair_job((kp16[blocks, h], vp16[blocks, h], np64(q[s, h * G:(h + 1) * G]), L,
                                int(budgets[s]), r))

    try:  # one BLAS thread per worker thread
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except ImportError:
        limit = None
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            futs = {(s, h): ex.submit(job, s, h, L)
                    for s, L in enumerate(seq_lens.tolist()) for h in range(H)}
            return {key: f.result() for key, f in futs.items()}
    finally:
        if limit is not None:
            limit.restore_original_limits()
