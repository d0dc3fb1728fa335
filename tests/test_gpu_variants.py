"""GPU parity of the ablation variants ([N] §6; readings R18, R19): int8 and
int2 bases (built by both build kernels, scored, and through the decode step)
the group-max / group-mass merge rules (separate select kernel and the
fused decode step), and per-head selection (every query head its own pages,
through the separate entry points and the decode step), against the oracle on
the same inputs."""
import numpy as np
import pytest
import torch

import synth
from oracle import locks_oracle as O
from tests import locks_harness as Hh
from tests.test_gpu_parity import (DEV, _check_against_oracle, _check_step, _compare_codes,
                                   _run_decode, _run_step, _say, _step_state, _to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from kv_cache_page_amd import locks
    return locks


# 300 blocks x 2 heads take the one-wave-per-page build, 2100 x 2 the bulk build
@pytest.mark.parametrize("bits,r,n", [(8, 8, 300), (2, 8, 300), (8, 16, 2100), (2, 4, 2100),
                                      (8, 4, 300), (2, 16, 2100)])
def test_build_codes_by_width(L, bits, r, n):
    _say(f"[gpu] build, int{bits} basis, r={r}, {n} blocks x 2 heads")
    keys = synth.random_pages(2 * n, seed=500 + bits + r)            # bf16 [2n][16][128]
    pool = keys.view(n, 2, 16, 128).contiguous().to(DEV)
    dims = L.Dims(2, 4, r, basis_bits=bits)
    summ = L.alloc_summaries(dims, n, DEV)
    L.build(dims, pool, torch.arange(n, dtype=torch.int32, device=DEV), summ)
    torch.cuda.synchronize()
    got = summ.cpu().numpy().reshape(2 * n, -1)
    assert got.shape[1] == O.slot_layout(r, basis_bits=bits)["stride"]
    frac, nflag, namb = _compare_codes(got, keys.double().numpy(), r, basis_bits=bits)
    _say(f"    differing codes {frac:.2e}, near-degenerate pages {nflag}, sign-ambiguous {namb}")
    assert frac <= 1e-3


def _batch(seed, G=4):
    """Three sequences, 3 KV heads; the query heads of a group get different
    norms (x0.5 .. x2), so their Z_g differ and the merge rules disagree."""
    b = synth.make_decode_batch([70 * 16 + 3, 2000, 33 * 16], 3, G, [9, 40, 17], seed=seed)
    scale = torch.linspace(0.5, 2.0, G).repeat(b.H)
    b.q = (b.q.float() * scale[None, :, None]).to(torch.bfloat16)
    return b


@pytest.mark.parametrize("bits,r", [(8, 8), (2, 8), (8, 4), (2, 16), (8, 16), (2, 4)])
def test_decode_from_oracle_summaries_by_width(L, bits, r):
    _say(f"[gpu] score + select + attention, int{bits} basis, r={r}")
    b = _batch(600 + bits + r)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, r, b.num_blocks,
                               basis_bits=bits)
    dims = L.Dims(b.H, b.G, r, basis_bits=bits)
    kb = int(b.budgets.max())
    res = _run_decode(L, dims, _to_dev(b), torch.from_numpy(summ).to(DEV), kb)
    ws, nmis, wo = _check_against_oracle(b, summ, res, r, kb, basis_bits=bits)
    _say(f"    max |score err| {ws:.2e}, near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")


@pytest.mark.parametrize("rule", ["max", "mass"])
@pytest.mark.parametrize("bits", [4, 8])
def test_merge_rules_separate_select(L, rule, bits):
    _say(f"[gpu] merge rule {rule}, int{bits} basis (separate select)")
    b = _batch(700 + bits)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, 8, b.num_blocks,
                               basis_bits=bits)
    dims = L.Dims(b.H, b.G, 8, basis_bits=bits, merge_rule=rule)
    kb = int(b.budgets.max())
    res = _run_decode(L, dims, _to_dev(b), torch.from_numpy(summ).to(DEV), kb)
    ws, nmis, wo = _check_against_oracle(b, summ, res, 8, kb, basis_bits=bits, merge=rule)
    _say(f"    near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")
    # on these inputs the rule changes the selection of some head (a kernel
    # that ignored the rule would fail the comparison above)
    differs = 0
    for s in range(b.num_seqs):
        for h in range(b.H):
            sel = [Hh.oracle_head(b.q, b.k_pool, b.v_pool, b.block_table, b.seq_lens, b.budgets,
                                  summ, s, h, b.G, 8, basis_bits=bits, merge=m)["sel"]
                   for m in ("share", rule)]
            differs += sel[0] != sel[1]
    assert differs > 0


@pytest.mark.parametrize("bits,rule", [(4, "max"), (4, "mass"), (8, "share"), (2, "mass"),
                                       (8, "max")])
def test_decode_step_variants(L, bits, rule):
    """The whole step (append, build of completed pages, score, select, attend):
    int4 with the fused score part, int8 and int2 with the separate score
    launch; every merge rule in the fused selection."""
    _say(f"[gpu] decode step, int{bits} basis, merge rule {rule}")
    lens = [16, 17, 40 * 16, 40 * 16 + 1, 300 * 16 + 9, 257 * 16, 33]
    budgets = [2, 3, 2, 7, 64, 300, 2]
    b = synth.make_decode_batch(lens, 3, 4, budgets, seed=800 + bits, extra_blocks=5)
    r = 8
    kp, vp, kn, vn, summ, completed = _step_state(b, r, basis_bits=bits)
    dims = L.Dims(b.H, b.G, r, basis_bits=bits, merge_rule=rule)
    res, kpa, vpa, sa = _run_step(L, dims, b, kp, vp, kn, vn, summ, 300)
    ws, nmis, wo = _check_step(b, r, 300, res, kpa, vpa, sa, summ, completed, basis_bits=bits,
                               merge=rule)
    _say(f"    near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")


# ---------------------------------------------------------------------------
# per-head selection (LOCKS_MERGE_PER_HEAD; reading R19)
# ---------------------------------------------------------------------------

def _check_per_head(b, summ, res, r, kmax, basis_bits=4):
    """Every query head against the oracle's per-head path: row h G + g of
    the selection holds query head g's own pages (a near-tie swap at its own
    boundary allowed, as for the shared rule), its scores are its own, and its
    output attends its own pages. Returns (max score error, differing pages,
    worst attention rel-L2, query-head groups whose selections differ)."""
    G = b.G
    worst_s, nmis, worst_o, split = 0.0, 0, 0.0, 0
    for s in range(b.num_seqs):
        Lq = int(b.seq_lens[s])
        P, F = (Lq + 15) // 16, Lq // 16
        k = min(max(int(b.budgets[s]), 2), kmax)
        for h in range(b.H):
            ora = Hh.oracle_head(b.q, b.k_pool, b.v_pool, b.block_table, b.seq_lens, b.budgets,
                                 summ, s, h, G, r, basis_bits=basis_bits, merge="per_head")
            Kp, Vp = Hh.head_pages(b.k_pool, b.v_pool, b.block_table, Lq, s, h)
            sels = []
            for g in range(G):
                row = h * G + g
                if res["scores"] is not None and F:
                    d = np.abs(res["scores"][s, row, :F, 0] - ora["scores"][:, g])
                    worst_s = max(worst_s, float(d.max()))
                    assert d.max() <= 1e-3, (s, h, g, float(d.max()))
                n = int(res["cnt"][s, row])
                gsel = [int(j) for j in res["sel"][s, row, :n]]
                assert (res["sel"][s, row, n:] == -1).all()
                assert gsel == sorted(gsel) and len(set(gsel)) == n
                assert n == (min(k, P) if P else 0)
                if P:
                    nmis += Hh.selection_mismatch(gsel, ora["sel"][g], ora["key"][:, g], P)
                sels.append(tuple(gsel))
                if gsel:
                    m = [16 if j < P - 1 else Lq - 16 * (P - 1) for j in gsel]
                    toks_k = np.concatenate([Kp[j, :mm] for j, mm in zip(gsel, m)])
                    toks_v = np.concatenate([Vp[j, :mm] for j, mm in zip(gsel, m)])
                    o_ref, lse_ref = O.attend(Hh.np64(b.q[s, row:row + 1]), toks_k, toks_v)
                    e = Hh.rel_l2(res["out"][s, row], o_ref[0])
                    worst_o = max(worst_o, e)
                    assert e <= 1e-2, (s, h, g, e)
                    assert abs(float(res["lse"][s, row]) - float(lse_ref[0])) <= 1e-3
            split += len(set(sels)) > 1
    return worst_s, nmis, worst_o, split


def _per_head_arrays(L, dims, S, MP, kb):
    rows = L.selection_heads(dims)
    sel = torch.full((S, rows, kb), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((S, rows), -7, dtype=torch.int32, device=DEV)
    out = torch.full((S, dims.num_kv_heads * dims.group_size, 128), 7.0, dtype=torch.float32,
                     device=DEV)
    lse = torch.full((S, dims.num_kv_heads * dims.group_size), 7.0, dtype=torch.float32, device=DEV)
    return sel, cnt, out, lse


@pytest.mark.parametrize("bits,r", [(4, 8), (8, 8), (4, 5)])
def test_per_head_separate_entry_points(L, bits, r):
    """locks_score_select + locks_sparse_attn with every query head selecting
    its own pages (matrix-core scores at r = 8, the VALU score kernel for int8
    and for r = 5)."""
    _say(f"[gpu] per-head selection, int{bits} basis, r={r} (separate entry points)")
    b = _batch(900 + bits + r)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, r, b.num_blocks,
                               basis_bits=bits)
    dims = L.Dims(b.H, b.G, r, basis_bits=bits, merge_rule="per_head")
    kb = int(b.budgets.max())
    bd = _to_dev(b)
    S, MP = b.num_seqs, b.max_pages
    sel, cnt, out, lse = _per_head_arrays(L, dims, S, MP, kb)
    sc = torch.full((S, b.H * b.G, MP, 1), 123.0, dtype=torch.float32, device=DEV)
    ws = L.alloc_workspace(dims, S, MP, kb, DEV)
    summ_d = torch.from_numpy(summ).to(DEV)
    L.score_select(dims, bd.q, summ_d, bd.block_table, bd.seq_lens, bd.budgets, kb, sel, cnt, ws,
                   scores_out=sc)
    L.sparse_attn(dims, bd.q, bd.k_pool, bd.v_pool, bd.block_table, bd.seq_lens, sel, cnt, kb, out,
                  ws, lse_out=lse)
    torch.cuda.synchronize()
    res = dict(sel=sel.cpu().numpy(), cnt=cnt.cpu().numpy(), scores=sc.cpu().numpy(),
               out=out.cpu().numpy(), lse=lse.cpu().numpy())
    ws_, nmis, wo, split = _check_per_head(b, summ, res, r, kb, basis_bits=bits)
    _say(f"    max |score err| {ws_:.2e}, near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}, "
         f"groups whose query heads disagree {split} of {b.num_seqs * b.H}")
    assert split > 0


@pytest.mark.parametrize("bits", [4, 8])
def test_per_head_decode_step(L, bits):
    """The whole step under the per-head rule: the append and the build of the
    completed pages stay per KV head, every query head selects and attends
    its own pages (int4: the fused launch; int8: the separate launches)."""
    _say(f"[gpu] decode step, per-head selection, int{bits} basis")
    lens = [16, 17, 40 * 16, 40 * 16 + 1, 300 * 16 + 9, 257 * 16, 33]
    budgets = [2, 3, 2, 7, 64, 300, 2]
    b = synth.make_decode_batch(lens, 3, 4, budgets, seed=950 + bits, extra_blocks=5)
    scale = torch.linspace(0.5, 2.0, b.G).repeat(b.H)
    b.q = (b.q.float() * scale[None, :, None]).to(torch.bfloat16)
    r, kb = 8, 300
    kp, vp, kn, vn, summ, completed = _step_state(b, r, basis_bits=bits)
    dims = L.Dims(b.H, b.G, r, basis_bits=bits, merge_rule="per_head")
    S = b.num_seqs
    sel, cnt, out, lse = _per_head_arrays(L, dims, S, b.max_pages, kb)
    kp_d, vp_d = kp.to(DEV), vp.to(DEV)
    summ_d = torch.from_numpy(summ).to(DEV)
    ws = L.alloc_workspace(dims, S, b.max_pages, kb, DEV)
    ws.fill_(0xA5)
    L.decode_step(dims, b.q.to(DEV), kn.to(DEV), vn.to(DEV), kp_d, vp_d, summ_d,
                  b.block_table.to(DEV), b.seq_lens.to(DEV), b.budgets.to(DEV), kb, out, ws,
                  lse_out=lse, sel_pages=sel, sel_count=cnt, seq_lens_host=b.seq_lens.cpu())
    torch.cuda.synchronize()
    # the new tokens are in the pools once, the completed pages' summaries are
    # the build's (checked against the oracle's codes), nothing else moved
    assert torch.equal(kp_d.cpu(), b.k_pool) and torch.equal(vp_d.cpu(), b.v_pool)
    summ_after = summ_d.cpu().numpy()
    summ_ora = summ.copy()
    if completed:
        pairs = [(blk, h) for blk in completed for h in range(b.H)]
        keys = np.stack([Hh.np64(b.k_pool[blk, h]) for blk, h in pairs])
        frac, _, _ = _compare_codes(np.stack([summ_after[blk, h] for blk, h in pairs]), keys, r,
                                    basis_bits=bits)
        assert frac <= 1e-3, frac
        ora, _, _ = O.build_slots(keys, r, basis_bits=bits)
        for i, (blk, h) in enumerate(pairs):
            summ_ora[blk, h] = ora[i]
    for blk in range(b.num_blocks):
        if blk not in completed:
            assert np.array_equal(summ_after[blk], summ[blk]), blk
    res = dict(sel=sel.cpu().numpy(), cnt=cnt.cpu().numpy(), scores=None, out=out.cpu().numpy(),
               lse=lse.cpu().numpy())
    _, nmis, wo, split = _check_per_head(b, summ_ora, res, r, kb, basis_bits=bits)
    _say(f"    near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}, groups whose query heads "
         f"disagree {split} of {b.num_seqs * b.H}")
    assert split > 0
