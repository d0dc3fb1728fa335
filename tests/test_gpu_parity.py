"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Tolerances (scores 1e-3 abs; selections exact except near-ties with a key gap
below 1e-5 in log-share units; attention 1e-2 relative L2; GPU-built codes
within +-1 LSB on at most 0.1% of entries) are written in each test.
"""
import math
import sys

import numpy as np
import pytest
import torch

import synth
from synth.locks_inputs import NEEDLE_NORM
from oracle import locks_oracle as O
from tests import locks_harness as Hh

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from kv_cache_page_amd import locks
    return locks


def _to_dev(b):
    return synth.DecodeBatch(
        k_pool=b.k_pool.to(DEV), v_pool=b.v_pool.to(DEV), q=b.q.to(DEV),
        block_table=b.block_table.to(DEV), seq_lens=b.seq_lens.to(DEV), budgets=b.budgets.to(DEV),
        needles=b.needles, H=b.H, G=b.G)


def _run_decode(L, dims, bd, summ_dev, max_budget, scores=True):
    S, H, G = bd.num_seqs, bd.H, bd.G
    MP = bd.max_pages
    sel = torch.full((S, H, max_budget), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((S, H), -7, dtype=torch.int32, device=DEV)
    sc = torch.full((S, H, MP, G), 123.0, dtype=torch.float32, device=DEV) if scores else None
    out = torch.full((S, H * G, 128), 7.0, dtype=torch.float32, device=DEV)
    lse = torch.full((S, H * G), 7.0, dtype=torch.float32, device=DEV)
    ws = L.alloc_workspace(dims, S, MP, max_budget, DEV)
    L.score_select(dims, bd.q, summ_dev, bd.block_table, bd.seq_lens, bd.budgets, max_budget, sel,
                   cnt, ws, scores_out=sc)
    L.sparse_attn(dims, bd.q, bd.k_pool, bd.v_pool, bd.block_table, bd.seq_lens, sel, cnt,
                  max_budget, out, ws, lse_out=lse)
    torch.cuda.synchronize()
    return dict(sel=sel.cpu().numpy(), cnt=cnt.cpu().numpy(),
                scores=None if sc is None else sc.cpu().numpy(), out=out.cpu().numpy(),
                lse=lse.cpu().numpy())


def _check_against_oracle(b, summ, res, r, max_budget, heads=None, score_tol=1e-3, deferred=False,
                          basis_bits=4, merge="share"):
    """Compare one decode step (every or the listed (seq, head)) with the
    oracle fed the same summaries. Returns (max score error, mismatched pages,
    worst attention rel-L2)."""
    G = b.G
    worst_s, nmis, worst_o = 0.0, 0, 0.0
    pairs = heads if heads is not None else [(s, h) for s in range(b.num_seqs) for h in range(b.H)]
    for (s, h) in pairs:
        Lq = int(b.seq_lens[s])
        P, F = (Lq + 15) // 16, Lq // 16
        ora = Hh.oracle_head(b.q, b.k_pool, b.v_pool, b.block_table, b.seq_lens, b.budgets, summ,
                             s, h, G, r, deferred=deferred, basis_bits=basis_bits, merge=merge)
        if res["scores"] is not None and F:
            d = np.abs(res["scores"][s, h, :F] - ora["scores"])
            worst_s = max(worst_s, float(d.max()))
            assert d.max() <= score_tol, (s, h, float(d.max()))
            assert np.isnan(res["scores"][s, h, F:]).all()
        n = int(res["cnt"][s, h])
        gsel = [int(j) for j in res["sel"][s, h, :n]]
        assert (res["sel"][s, h, n:] == -1).all()
        assert gsel == sorted(gsel) and len(set(gsel)) == n
        k = min(max(int(b.budgets[s]), 2), max_budget)
        assert n == (min(k, P) if P else 0)
        if P:
            nmis += Hh.selection_mismatch(gsel, ora["sel"], ora["key"], P)
        # attention over the GPU's own selection against the oracle's softmax
        Kp, Vp = Hh.head_pages(b.k_pool, b.v_pool, b.block_table, Lq, s, h)
        qq = Hh.np64(b.q[s, h * G:(h + 1) * G])
        if gsel:
            toks_k = np.concatenate([Kp[j, :(16 if j < P - 1 else Lq - 16 * (P - 1))] for j in gsel])
            toks_v = np.concatenate([Vp[j, :(16 if j < P - 1 else Lq - 16 * (P - 1))] for j in gsel])
            o_ref, lse_ref = O.attend(qq, toks_k, toks_v)
            e = Hh.rel_l2(res["out"][s, h * G:(h + 1) * G], o_ref)
            worst_o = max(worst_o, e)
            assert e <= 1e-2, (s, h, e)
            np.testing.assert_allclose(res["lse"][s, h * G:(h + 1) * G], lse_ref, atol=1e-3)
        else:
            assert (res["out"][s, h * G:(h + 1) * G] == 0).all()
    return worst_s, nmis, worst_o


# ---------------------------------------------------------------------------
# score + select + attention from oracle-built summaries
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,r", [("tiny", 8), ("ctx32k", 8), ("tiny", 4), ("tiny", 16),
                                    ("tiny", 5), ("tiny", 12)])
def test_decode_from_oracle_summaries(L, name, r):
    """Ranks 4, 8 and 16 run the matrix-core score kernel; other ranks (5, 12
    here) the vector-ALU one."""
    _say(f"[gpu] decode from oracle summaries: {name} r={r}")
    b = synth.config_batch(name)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, r, b.num_blocks)
    dims = L.Dims(b.H, b.G, r)
    bd = _to_dev(b)
    kb = int(b.budgets.max())
    res = _run_decode(L, dims, bd, torch.from_numpy(summ).to(DEV), kb)
    ws, nmis, wo = _check_against_oracle(b, summ, res, r, kb)
    _say(f"    max |score err| {ws:.2e}, near-tie page swaps {nmis}, worst attn rel-L2 {wo:.2e}")
    # the exact-LSE selector keeps the needles; report LOCKS's own retention
    kept = sum(1 for (s, h, j, _) in b.needles if j in set(res["sel"][s, h, :res["cnt"][s, h]]))
    _say(f"    needle pages kept by the GPU selection: {kept}/{len(b.needles)}")


@pytest.mark.parametrize("G", [1, 2])
def test_group_sizes(L, G):
    _say(f"[gpu] group size {G}")
    b = synth.make_decode_batch([70 * 16 + 3, 33 * 16], 2, G, [9, 40], seed=40 + G)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, 8, b.num_blocks)
    dims = L.Dims(b.H, G, 8)
    res = _run_decode(L, dims, _to_dev(b), torch.from_numpy(summ).to(DEV), 40)
    _check_against_oracle(b, summ, res, 8, 40)


def test_ragged_edges(L):
    """Lengths around page boundaries (1, 16, 17 tokens ...), budgets 2..P+,
    shuffled blocks with spare blocks in the pool."""
    _say("[gpu] ragged edge cases")
    lens = [1, 15, 16, 17, 32, 33, 48, 40 * 16, 40 * 16 + 1, 300 * 16 + 9, 257 * 16]
    budgets = [2, 2, 3, 2, 2, 5, 2, 2, 7, 64, 1000]
    b = synth.make_decode_batch(lens, 3, 4, budgets, seed=50, extra_blocks=37)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, 8, b.num_blocks)
    dims = L.Dims(b.H, b.G, 8)
    res = _run_decode(L, dims, _to_dev(b), torch.from_numpy(summ).to(DEV), 300)
    _check_against_oracle(b, summ, res, 8, 300)


def test_select_all_is_dense(L):
    _say("[gpu] budget >= pages gives dense attention")
    b = synth.make_decode_batch([61 * 16 + 11], 2, 4, [64], seed=60)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, 8, b.num_blocks)
    res = _run_decode(L, L.Dims(2, 4, 8), _to_dev(b), torch.from_numpy(summ).to(DEV), 64)
    Lq = int(b.seq_lens[0])
    for h in range(2):
        assert list(res["sel"][0, h, :res["cnt"][0, h]]) == list(range(62))
        Kp, Vp = Hh.head_pages(b.k_pool, b.v_pool, b.block_table, Lq, 0, h)
        q = Hh.np64(b.q[0, 4 * h:4 * h + 4])
        dense, _ = O.attend(q, Kp.reshape(-1, 128)[:Lq], Vp.reshape(-1, 128)[:Lq])
        assert Hh.rel_l2(res["out"][0, 4 * h:4 * h + 4], dense) <= 1e-2


def test_long_table_global_keys(L):
    """A block table wider than the LDS key buffer takes the global-memory key
    path of the selection; results must not change."""
    _say("[gpu] wide block table (global key buffer)")
    b = synth.make_decode_batch([300 * 16 + 5, 1000 * 16], 2, 4, [20, 64], seed=75)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, 8, b.num_blocks)
    wide = torch.full((2, 13000), -1, dtype=torch.int32)
    wide[:, :b.max_pages] = b.block_table
    bw = synth.DecodeBatch(k_pool=b.k_pool, v_pool=b.v_pool, q=b.q, block_table=wide,
                           seq_lens=b.seq_lens, budgets=b.budgets, needles=b.needles, H=b.H, G=b.G)
    res = _run_decode(L, L.Dims(2, 4, 8), _to_dev(bw), torch.from_numpy(summ).to(DEV), 64)
    _check_against_oracle(bw, summ, res, 8, 64)


def test_equal_keys_take_lowest_pages(L):
    """q = 0 gives every page the same score, so all keys tie: the selection
    must be the sink, the recent page and the lowest-numbered candidates
    (this also drives the exact fallback for a crowded crossing bin)."""
    _say("[gpu] all keys equal")
    b = synth.make_decode_batch([3000 * 16 + 7, 40 * 16], 1, 4, [100, 9], seed=77)
    b.q.zero_()
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, 1, 8, b.num_blocks)
    res = _run_decode(L, L.Dims(1, 4, 8), _to_dev(b), torch.from_numpy(summ).to(DEV), 100)
    P0, P1 = 3001, 40
    assert list(res["sel"][0, 0, :100]) == [0] + list(range(1, 99)) + [P0 - 1]
    assert list(res["sel"][1, 0, :9]) == [0] + list(range(1, 8)) + [P1 - 1]
    _check_against_oracle(b, summ, res, 8, 100)


def test_invalid_block_ids_are_skipped(L):
    _say("[gpu] out-of-range block ids")
    b = synth.make_decode_batch([50 * 16], 1, 4, [10], seed=70)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, 1, 8, b.num_blocks)
    bd = _to_dev(b)
    bd.block_table[0, 7] = -1
    bd.block_table[0, 9] = b.num_blocks + 5
    res = _run_decode(L, L.Dims(1, 4, 8), bd, torch.from_numpy(summ).to(DEV), 10)
    assert res["scores"][0, 0, 7].max() == -np.inf and res["scores"][0, 0, 9].max() == -np.inf
    sel = set(res["sel"][0, 0, :res["cnt"][0, 0]].tolist())
    assert 7 not in sel and 9 not in sel


def test_deterministic(L):
    _say("[gpu] bit-identical reruns")
    b = synth.config_batch("ctx32k")
    summ = torch.from_numpy(Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, 8,
                                                b.num_blocks)).to(DEV)
    bd = _to_dev(b)
    r1 = _run_decode(L, L.Dims(8, 4, 8), bd, summ, 64)
    r2 = _run_decode(L, L.Dims(8, 4, 8), bd, summ, 64)
    for k in r1:
        assert np.array_equal(r1[k], r2[k], equal_nan=True), k


# ---------------------------------------------------------------------------
# build
# ---------------------------------------------------------------------------

def _compare_codes(gpu_slots, keys, r, basis_bits=4):
    """GPU slots vs the oracle's for the same keys. Returns (fraction of code
    entries that differ, pages excluded as near-degenerate, columns excluded
    as sign-ambiguous)."""
    ora_slots, summ, _ = O.build_slots(keys, r, basis_bits=basis_bits)
    g = O.unpack_slots(gpu_slots, r, basis_bits=basis_bits)
    o = O.unpack_slots(ora_slots, r, basis_bits=basis_bits)
    flag = Hh.gap_flags(summ["lam"], r)
    amb = Hh.sign_ambiguous(summ["V"]) & summ["active"]
    keep = ~flag
    colmask = keep[:, None] & ~amb                                  # (n, r)
    dv = np.abs(g["Vq"] - o["Vq"])[:, :, :]                         # (n, d, r)
    dv = np.where(colmask[:, None, :], dv, 0)
    dc = np.abs(g["Cq"] - o["Cq"])                                  # (n, B, r)
    dc = np.where(colmask[:, None, :], dc, 0)
    dm = np.abs(g["muq"] - o["muq"])[keep]
    assert dv.max() <= 1 and dc.max() <= 1 and (dm.max() if dm.size else 0) <= 1, \
        (dv.max(), dc.max(), dm.max() if dm.size else 0)
    n_entries = colmask.sum() * (128 + 16) + keep.sum() * 128
    frac = (np.count_nonzero(dv) + np.count_nonzero(dc) + np.count_nonzero(dm)) / max(n_entries, 1)
    # scales of comparable pages agree to fp16 rounding of the same absmax
    for nm in ("sV", "sC"):
        a = g[nm][keep].astype(np.float64)
        c = o[nm][keep].astype(np.float64)
        np.testing.assert_allclose(a, c, rtol=2e-3, atol=1e-7)
    assert np.array_equal(g["smu"], o["smu"])
    return frac, int(flag.sum()), int(amb.sum())


@pytest.mark.parametrize("r,n", [(4, 8192), (8, 8192), (16, 8192), (4, 4096), (8, 4096), (16, 4096),
                                 (7, 1000)])
def test_build_codes(L, r, n):
    """Lists of up to 4096 pages use the one-page-per-wave build, longer ones
    the four-pages-per-wave build: both against the oracle's codes."""
    _say(f"[gpu] build parity r={r} n={n}")
    keys = synth.random_pages(n, seed=100 + r)                       # bf16 [n][16][128] on CPU
    pool = keys.view(n, 1, 16, 128).contiguous().to(DEV)
    dims = L.Dims(1, 4, r)
    summ = L.alloc_summaries(dims, n, DEV)
    ids = torch.arange(n, dtype=torch.int32, device=DEV)
    L.build(dims, pool, ids, summ)
    torch.cuda.synchronize()
    frac, nflag, namb = _compare_codes(summ[:, 0].cpu().numpy(), keys.double().numpy(), r)
    _say(f"    differing code entries {frac:.2e}; near-degenerate pages {nflag}; "
         f"sign-ambiguous columns {namb}")
    assert frac <= 1e-3


@pytest.mark.parametrize("pad", [0, 4200])
def test_build_degenerate_pages(L, pad):
    """Degenerate pages, alone (one-page-per-wave build) and followed by
    `pad` random pages (four-pages-per-wave build)."""
    _say(f"[gpu] build of degenerate pages (pad {pad})")
    n = 8
    k = torch.zeros(n, 16, 128)
    k[1] = 0.375                                          # all keys equal
    k[2, :, :5] = torch.randn(16, 5)                       # rank <= 5
    k[3] = torch.randn(1, 128)                             # equal keys, random vector
    k[4, 0] = 3.0                                          # one outlier token
    k[5] = torch.randn(16, 128) * 1e-3
    k[6] = torch.randn(16, 128) * 300
    k[7, ::2] = 1.0                                        # two distinct keys
    keys = k.to(torch.bfloat16)
    allk = torch.cat([keys, synth.random_pages(pad, seed=77)]) if pad else keys
    for r in (1, 8, 16):
        dims = L.Dims(1, 4, r)
        summ = L.alloc_summaries(dims, n + pad, DEV)
        L.build(dims, allk.view(n + pad, 1, 16, 128).contiguous().to(DEV),
                torch.arange(n + pad, dtype=torch.int32, device=DEV), summ)
        torch.cuda.synchronize()
        got = summ[:n, 0].cpu().numpy()
        ora, s, _ = O.build_slots(keys.double().numpy(), r)
        for p in (0, 1, 3):                               # exactly degenerate: byte-identical
            assert np.array_equal(got[p], ora[p]), (r, p)
        g = O.unpack_slots(got, r)
        assert not np.isnan(g["sV"].astype(np.float64)).any()


def test_build_list_and_filled(L):
    """locks_build over a shuffled id list (invalid ids skipped), and
    locks_build_filled picking the page each sequence has just filled."""
    _say("[gpu] build id list / filled pages")
    b = synth.make_decode_batch([10 * 16, 7 * 16 + 3, 4 * 16], 2, 4, [4, 4, 4], seed=80,
                                extra_blocks=5)
    dims = L.Dims(2, 4, 8)
    bd = _to_dev(b)
    summ = L.alloc_summaries(dims, b.num_blocks, DEV)
    ids = torch.tensor([3, -1, 5, b.num_blocks, 0], dtype=torch.int32, device=DEV)
    L.build(dims, bd.k_pool, ids, summ)
    summ2 = L.alloc_summaries(dims, b.num_blocks, DEV)
    L.build_filled(dims, bd.k_pool, bd.block_table, bd.seq_lens, summ2)
    torch.cuda.synchronize()
    got, got2 = summ.cpu().numpy(), summ2.cpu().numpy()
    listed = [(blk, h) for blk in (3, 5, 0) for h in range(2)]
    frac, _, _ = _compare_codes(np.stack([got[blk, h] for blk, h in listed]),
                                np.stack([Hh.np64(b.k_pool[blk, h]) for blk, h in listed]), 8)
    assert frac <= 1e-3
    for blk in set(range(b.num_blocks)) - {3, 5, 0}:
        assert not got[blk].any()
    built = {int(b.block_table[0, 9]), int(b.block_table[2, 3])}   # seqs 0 and 2 just filled
    pairs = [(blk, h) for blk in sorted(built) for h in range(2)]
    frac, _, _ = _compare_codes(np.stack([got2[blk, h] for blk, h in pairs]),
                                np.stack([Hh.np64(b.k_pool[blk, h]) for blk, h in pairs]), 8)
    assert frac <= 1e-3
    for blk in range(b.num_blocks):
        if blk not in built:
            assert not got2[blk].any()


@pytest.mark.parametrize("r", [8, 13])
def test_build_filled_many(L, r):
    """Filled-page mode over 96 sequences x 8 KV heads (768 pages built at
    once, the shape of a decode step where many sequences fill a page)."""
    _say(f"[gpu] filled-page build, 96 x 8 pages, r={r}")
    S, H = 96, 8
    lens = [16 * (1 + (s * 7) % 11) for s in range(S)]
    b = synth.make_decode_batch(lens, H, 4, [4] * S, seed=120 + r, needles_per_head=0)
    dims = L.Dims(H, 4, r)
    bd = _to_dev(b)
    summ = L.alloc_summaries(dims, b.num_blocks, DEV)
    L.build_filled(dims, bd.k_pool, bd.block_table, bd.seq_lens, summ)
    torch.cuda.synchronize()
    got = summ.cpu().numpy()
    blks = [int(b.block_table[s, lens[s] // 16 - 1]) for s in range(S)]
    keys = np.stack([Hh.np64(b.k_pool[blk, h]) for blk in blks for h in range(H)])
    gpu = np.stack([got[blk, h] for blk in blks for h in range(H)])
    frac, nflag, namb = _compare_codes(gpu, keys, r)
    _say(f"    differing code entries {frac:.2e}; near-degenerate pages {nflag}; "
         f"sign-ambiguous columns {namb}")
    assert frac <= 1e-3
    built = set(blks)
    for blk in range(b.num_blocks):
        if blk not in built:
            assert not got[blk].any()


def test_append(L):
    _say("[gpu] append one token per sequence")
    b = synth.make_decode_batch([5 * 16 + 2, 3 * 16, 1], 2, 4, [4, 4, 4], seed=90)
    dims = L.Dims(2, 4, 8)
    bd = _to_dev(b)
    kn = torch.randn(3, 2, 128, device=DEV).to(torch.bfloat16)
    vn = torch.randn(3, 2, 128, device=DEV).to(torch.bfloat16)
    kp0 = bd.k_pool.clone()
    L.append_kv(dims, kn, vn, bd.k_pool, bd.v_pool, bd.block_table, bd.seq_lens)
    torch.cuda.synchronize()
    for s, Lq in enumerate(b.seq_lens.tolist()):
        blk = int(b.block_table[s, (Lq - 1) // 16])
        assert torch.equal(bd.k_pool[blk, :, (Lq - 1) % 16], kn[s])
        assert torch.equal(bd.v_pool[blk, :, (Lq - 1) % 16], vn[s])
        kp0[blk, :, (Lq - 1) % 16] = kn[s]
    assert torch.equal(kp0, bd.k_pool)


# ---------------------------------------------------------------------------
# end to end and full size
# ---------------------------------------------------------------------------

def test_end_to_end_gpu_build(L):
    """GPU build -> GPU score/select -> GPU attention, against the oracle run
    from its own summaries of the same keys."""
    _say("[gpu] end to end with GPU-built summaries (ctx32k)")
    b = synth.config_batch("ctx32k")
    dims = L.Dims(b.H, b.G, 8)
    bd = _to_dev(b)
    summ_dev = L.alloc_summaries(dims, b.num_blocks, DEV)
    F = int(b.seq_lens[0]) // 16
    L.build(dims, bd.k_pool, bd.block_table[0, :F].contiguous(), summ_dev)
    res = _run_decode(L, dims, bd, summ_dev, 64)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, 8, b.num_blocks)
    ws, nmis, wo = _check_against_oracle(b, summ, res, 8, 64)
    _say(f"    max |score err| {ws:.2e}, near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")


def test_full_size_128k_layer(L):
    """One layer of the 128K-token, 8-KV-head workload at its real shape,
    launched as the benchmark launches it: GPU build of all 65536 pages,
    score/select from oracle-built summaries of every head (full comparison),
    attention checked on every head."""
    _say("[gpu] full-size 128K layer")
    b = synth.config_batch("ctx128k", device=DEV)
    dims = L.Dims(b.H, b.G, 8)
    summ_gpu = L.alloc_summaries(dims, b.num_blocks, DEV)
    L.build(dims, b.k_pool, b.block_table[0].contiguous(), summ_gpu)
    torch.cuda.synchronize()
    bc = synth.DecodeBatch(k_pool=b.k_pool.cpu(), v_pool=b.v_pool.cpu(), q=b.q.cpu(),
                           block_table=b.block_table.cpu(), seq_lens=b.seq_lens.cpu(),
                           budgets=b.budgets.cpu(), needles=b.needles, H=b.H, G=b.G)
    _say("    oracle build of 65536 pages")
    summ = Hh.oracle_summaries(bc.k_pool, bc.block_table, bc.seq_lens, b.H, 8, b.num_blocks)
    # sampled build parity: 2 heads x 8192 pages
    for h in (0, 5):
        blocks = bc.block_table[0].long()
        frac, nflag, namb = _compare_codes(summ_gpu[blocks.to(DEV), h].cpu().numpy(),
                                           bc.k_pool[blocks, h].double().numpy(), 8)
        _say(f"    head {h}: differing codes {frac:.2e}, flagged pages {nflag}, ambiguous cols {namb}")
        assert frac <= 1e-3
    res = _run_decode(L, dims, b, torch.from_numpy(summ).to(DEV), 128)
    ws, nmis, wo = _check_against_oracle(bc, summ, res, 8, 128)
    _say(f"    max |score err| {ws:.2e}, near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")
    kept = sum(1 for (s, h, j, _) in b.needles if j in set(res["sel"][s, h, :res["cnt"][s, h]]))
    _say(f"    needle pages kept: {kept}/{len(b.needles)}")


# ---------------------------------------------------------------------------
# fused decode step (locks_decode_step)
# ---------------------------------------------------------------------------

def _step_state(b, r, basis_bits=4):
    """Split a batch into the state before its decode step: the token at
    position len - 1 of every sequence removed from the pools (overwritten with
    a constant) and returned as k_new / v_new, and oracle summaries of every
    full page except those that token completes (left zero)."""
    S, H = b.num_seqs, b.H
    kn = torch.zeros(S, H, 128, dtype=torch.bfloat16)
    vn = torch.zeros(S, H, 128, dtype=torch.bfloat16)
    kp, vp = b.k_pool.clone(), b.v_pool.clone()
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, H, r, b.num_blocks,
                               basis_bits=basis_bits)
    completed = []
    for s, Lq in enumerate(b.seq_lens.tolist()):
        if Lq < 1:
            continue
        blk, t = int(b.block_table[s, (Lq - 1) // 16]), (Lq - 1) % 16
        kn[s], vn[s] = b.k_pool[blk, :, t], b.v_pool[blk, :, t]
        kp[blk, :, t] = 3.0
        vp[blk, :, t] = -3.0
        if Lq % 16 == 0:
            summ[blk] = 0
            completed.append(blk)
    return kp, vp, kn, vn, summ, completed


def _run_step(L, dims, b, kp, vp, kn, vn, summ, max_budget, host_lens=True, with_sel=True,
              defer_build=False):
    S, H, G = b.num_seqs, b.H, b.G
    kp_d, vp_d = kp.to(DEV), vp.to(DEV)
    summ_d = torch.from_numpy(summ).to(DEV)
    sel = torch.full((S, H, max_budget), -7, dtype=torch.int32, device=DEV) if with_sel else None
    cnt = torch.full((S, H), -7, dtype=torch.int32, device=DEV) if with_sel else None
    out = torch.full((S, H * G, 128), 7.0, dtype=torch.float32, device=DEV)
    lse = torch.full((S, H * G), 7.0, dtype=torch.float32, device=DEV)
    ws = L.alloc_workspace(dims, S, b.max_pages, max_budget, DEV)
    ws.fill_(0xA5)   # stale contents must not matter
    L.decode_step(dims, b.q.to(DEV), kn.to(DEV), vn.to(DEV), kp_d, vp_d, summ_d,
                  b.block_table.to(DEV), b.seq_lens.to(DEV), b.budgets.to(DEV), max_budget, out,
                  ws, lse_out=lse, sel_pages=sel, sel_count=cnt,
                  seq_lens_host=b.seq_lens.cpu() if host_lens else None, defer_build=defer_build)
    torch.cuda.synchronize()
    res = dict(sel=None if sel is None else sel.cpu().numpy(),
               cnt=None if cnt is None else cnt.cpu().numpy(), scores=None,
               out=out.cpu().numpy(), lse=lse.cpu().numpy())
    return res, kp_d.cpu(), vp_d.cpu(), summ_d.cpu().numpy()


def _check_step(b, r, kmax, res, kp_after, vp_after, summ_after, summ_before, completed,
                basis_bits=4, merge="share"):
    # the new tokens are in the pools, nothing else moved
    assert torch.equal(kp_after, b.k_pool) and torch.equal(vp_after, b.v_pool)
    # completed pages got GPU-built summaries within the build tolerance; others untouched
    summ_ora = summ_before.copy()
    if completed:
        pairs = [(blk, h) for blk in completed for h in range(b.H)]
        keys = np.stack([Hh.np64(b.k_pool[blk, h]) for blk, h in pairs])
        frac, nflag, namb = _compare_codes(np.stack([summ_after[blk, h] for blk, h in pairs]), keys, r,
                                           basis_bits=basis_bits)
        assert frac <= 1e-3, frac
        ora, _, _ = O.build_slots(keys, r, basis_bits=basis_bits)
        for i, (blk, h) in enumerate(pairs):
            summ_ora[blk, h] = ora[i]
    for blk in range(b.num_blocks):
        if blk not in completed:
            assert np.array_equal(summ_after[blk], summ_before[blk]), blk
    # score/select/attend against the oracle fed its own summaries
    return _check_against_oracle(b, summ_ora, res, r, kmax, basis_bits=basis_bits, merge=merge)


@pytest.mark.parametrize("host_lens", [True, False])
def test_decode_step_ragged(L, host_lens):
    """Lengths that complete a page with the new token (16, 32, 640, 257*16),
    that start one (1, 17, 641), and others; budgets from 2 to above P."""
    _say(f"[gpu] decode step, ragged batch, host lengths {host_lens}")
    lens = [1, 16, 17, 32, 40 * 16, 40 * 16 + 1, 300 * 16 + 9, 257 * 16, 33]
    budgets = [2, 2, 3, 5, 2, 7, 64, 300, 2]
    b = synth.make_decode_batch(lens, 3, 4, budgets, seed=150, extra_blocks=11)
    kp, vp, kn, vn, summ, completed = _step_state(b, 8)
    dims = L.Dims(b.H, b.G, 8)
    res, kpa, vpa, sa = _run_step(L, dims, b, kp, vp, kn, vn, summ, 300, host_lens=host_lens)
    ws, nmis, wo = _check_step(b, 8, 300, res, kpa, vpa, sa, summ, completed)
    _say(f"    near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")


def test_decode_step_ragged_wide_table(L):
    """One fused launch over sequences of very different lengths in a table of
    4201 pages (16 selection workgroups per head, 128-page score tiles): an
    empty sequence, one shorter than a page, one that completes a page, and
    medium and long ones. The launch trims the score pairs and selection
    workgroups past each sequence's pages; every (sequence, head) is checked
    against the oracle."""
    _say("[gpu] decode step, ragged batch over a 4201-page table")
    lens = [0, 5, 16 * 16, 600 * 16 + 7, 4200 * 16 + 3]
    budgets = [2, 3, 9, 40, 200]
    b = synth.make_decode_batch(lens, 4, 4, budgets, seed=151, extra_blocks=5)
    kp, vp, kn, vn, summ, completed = _step_state(b, 8)
    dims = L.Dims(b.H, b.G, 8)
    res, kpa, vpa, sa = _run_step(L, dims, b, kp, vp, kn, vn, summ, 200)
    ws, nmis, wo = _check_step(b, 8, 200, res, kpa, vpa, sa, summ, completed)
    _say(f"    near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")


@pytest.mark.parametrize("G,r", [(1, 4), (2, 16), (4, 4), (4, 16)])
def test_decode_step_group_sizes(L, G, r):
    """Group sizes and ranks through the single launch over a short table
    (8 selection workgroups per head, 32-page score tiles)."""
    _say(f"[gpu] decode step G={G} r={r}")
    b = synth.make_decode_batch([70 * 16, 33 * 16 + 5, 129 * 16 + 1], 2, G, [9, 40, 17],
                                seed=160 + G)
    kp, vp, kn, vn, summ, completed = _step_state(b, r)
    res, kpa, vpa, sa = _run_step(L, L.Dims(b.H, G, r), b, kp, vp, kn, vn, summ, 40)
    _check_step(b, r, 40, res, kpa, vpa, sa, summ, completed)


def test_decode_step_without_selection_output(L):
    """sel_pages / sel_count are optional: the outputs must not change."""
    _say("[gpu] decode step without selection outputs")
    b = synth.make_decode_batch([500 * 16 + 3, 64 * 16], 2, 4, [32, 20], seed=170)
    kp, vp, kn, vn, summ, _ = _step_state(b, 8)
    dims = L.Dims(2, 4, 8)
    r1 = _run_step(L, dims, b, kp, vp, kn, vn, summ, 32)[0]
    r2 = _run_step(L, dims, b, kp, vp, kn, vn, summ, 32, with_sel=False)[0]
    assert np.array_equal(r1["out"], r2["out"]) and np.array_equal(r1["lse"], r2["lse"])


def test_decode_step_equal_keys(L):
    """q = 0: every key ties, more than 512 candidates share the crossing bin,
    so the fused kernel takes its radix path; the lowest pages must win."""
    _say("[gpu] decode step, all keys equal")
    b = synth.make_decode_batch([3000 * 16 + 7, 40 * 16], 1, 4, [100, 9], seed=177)
    b.q.zero_()
    kp, vp, kn, vn, summ, completed = _step_state(b, 8)
    res, kpa, vpa, sa = _run_step(L, L.Dims(1, 4, 8), b, kp, vp, kn, vn, summ, 100)
    assert list(res["sel"][0, 0, :100]) == [0] + list(range(1, 99)) + [3000]
    assert list(res["sel"][1, 0, :9]) == [0] + list(range(1, 8)) + [39]
    _check_step(b, 8, 100, res, kpa, vpa, sa, summ, completed)


def test_decode_step_equal_keys_mid_size_bin(L):
    """q = 0 with 68 and 298 tied candidates: the crossing bin is too large for
    the register ranking and small enough for the pairwise LDS ranking."""
    _say("[gpu] decode step, 68 / 298 equal keys")
    b = synth.make_decode_batch([300 * 16 + 7, 70 * 16], 1, 4, [100, 50], seed=178)
    b.q.zero_()
    kp, vp, kn, vn, summ, completed = _step_state(b, 8)
    res, kpa, vpa, sa = _run_step(L, L.Dims(1, 4, 8), b, kp, vp, kn, vn, summ, 100)
    assert list(res["sel"][0, 0, :100]) == [0] + list(range(1, 99)) + [300]
    assert list(res["sel"][1, 0, :50]) == [0] + list(range(1, 49)) + [69]
    _check_step(b, 8, 100, res, kpa, vpa, sa, summ, completed)


def test_decode_step_slice_with_many_top_pages(L):
    """80 needle pages inside one 250-page slice of a 2000-page sequence (8
    splits), budget 100: that slice holds more of the selected pages than the
    63 top candidates a slice publishes beside its histogram, so the crossing
    bin's candidates cannot all come with the first exchange."""
    _say("[gpu] decode step, one slice holding 80 of the 100 selected pages")
    b = synth.make_decode_batch([2000 * 16 - 3], 1, 4, [100], seed=181, needles_per_head=0)
    u = b.q[0, :b.G].float().mean(0)
    u = u / u.norm()
    for j in range(260, 340):
        b.k_pool[int(b.block_table[0, j]), 0, 5] = (NEEDLE_NORM * u).to(torch.bfloat16)
    kp, vp, kn, vn, summ, completed = _step_state(b, 8)
    ora = Hh.oracle_head(b.q, b.k_pool, b.v_pool, b.block_table, b.seq_lens, b.budgets, summ,
                         0, 0, b.G, 8)
    assert sum(1 for j in ora["sel"] if 250 <= j < 500) > 63
    res, kpa, vpa, sa = _run_step(L, L.Dims(1, b.G, 8), b, kp, vp, kn, vn, summ, 100)
    _check_step(b, 8, 100, res, kpa, vpa, sa, summ, completed)


def test_decode_step_32_splits(L):
    """A 9000-page table with budgets up to 1100 pages takes 32 splits (slices
    of 282 pages, 15 top candidates published per slice): a small budget on
    the long sequence, and a budget that selects most of a 1200-page one."""
    _say("[gpu] decode step, 32 splits (9000-page table, budgets 64 and 1100)")
    b = synth.make_decode_batch([9000 * 16 - 5, 1200 * 16 + 3], 1, 4, [64, 1100], seed=183)
    kp, vp, kn, vn, summ, completed = _step_state(b, 8)
    res, kpa, vpa, sa = _run_step(L, L.Dims(1, 4, 8), b, kp, vp, kn, vn, summ, 1100)
    _check_step(b, 8, 1100, res, kpa, vpa, sa, summ, completed)


def test_decode_step_wide_table_fallback(L):
    """A table wider than 16384 pages takes the separate select and attention
    launches inside the same entry point, with or without selection outputs
    (without them the selection goes through the workspace)."""
    _say("[gpu] decode step, 17000-page table")
    b = synth.make_decode_batch([300 * 16 + 5, 1000 * 16], 2, 4, [20, 64], seed=175)
    wide = torch.full((2, 17000), -1, dtype=torch.int32)
    wide[:, :b.max_pages] = b.block_table
    bw = synth.DecodeBatch(k_pool=b.k_pool, v_pool=b.v_pool, q=b.q, block_table=wide,
                           seq_lens=b.seq_lens, budgets=b.budgets, needles=b.needles, H=b.H, G=b.G)
    kp, vp, kn, vn, summ, completed = _step_state(bw, 8)
    res, kpa, vpa, sa = _run_step(L, L.Dims(2, 4, 8), bw, kp, vp, kn, vn, summ, 64)
    _check_step(bw, 8, 64, res, kpa, vpa, sa, summ, completed)
    res2 = _run_step(L, L.Dims(2, 4, 8), bw, kp, vp, kn, vn, summ, 64, with_sel=False)[0]
    assert np.array_equal(res["out"], res2["out"]) and np.array_equal(res["lse"], res2["lse"])


def test_decode_step_repeat_is_bitwise_stable(L):
    """Calls in a row on one workspace (arrival counters reused) give the
    same bits, whichever workgroup finishes last."""
    _say("[gpu] decode step reruns")
    b = synth.config_batch("ctx32k")
    kp, vp, kn, vn, summ, _ = _step_state(b, 8)
    dims = L.Dims(8, 4, 8)
    S, H, G = 1, 8, 4
    bd = _to_dev(b)
    ws = L.alloc_workspace(dims, S, b.max_pages, 64, DEV)
    outs = []
    for _ in range(3):
        kp_d, vp_d = kp.to(DEV), vp.to(DEV)
        summ_d = torch.from_numpy(summ).to(DEV)
        out = torch.empty(S, H * G, 128, dtype=torch.float32, device=DEV)
        lse = torch.empty(S, H * G, dtype=torch.float32, device=DEV)
        L.decode_step(dims, bd.q, kn.to(DEV), vn.to(DEV), kp_d, vp_d, summ_d, bd.block_table,
                      bd.seq_lens, bd.budgets, 64, out, ws, lse_out=lse,
                      seq_lens_host=b.seq_lens.cpu())
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])


def test_decode_step_graph_replays(L):
    """The single-launch decode step captured in a HIP graph and replayed:
    with the outputs reset by eager work and the stream synchronised between
    replays, and an eager call on the same workspace in between, every replay
    gives the eager call's outputs and selection bit for bit (the head
    epochs in the workspace advance with every launch, captured or not);
    the eager result matches the oracle. No length completes a page, so the
    step is one launch."""
    _say("[gpu] decode step captured in a HIP graph, 4 replays")
    lens = [600 * 16 + 5, 33 * 16 + 9, 2000 * 16 + 1]
    budgets = [40, 8, 64]
    b = synth.make_decode_batch(lens, 4, 4, budgets, seed=171, extra_blocks=3)
    kp, vp, kn, vn, summ, completed = _step_state(b, 8)
    assert not completed
    dims = L.Dims(b.H, b.G, 8)
    S, H, G, kb = b.num_seqs, b.H, b.G, 64
    kp_d, vp_d, summ_d = kp.to(DEV), vp.to(DEV), torch.from_numpy(summ).to(DEV)
    q_d, kn_d, vn_d = b.q.to(DEV), kn.to(DEV), vn.to(DEV)
    tab, lens_d, bud = b.block_table.to(DEV), b.seq_lens.to(DEV), b.budgets.to(DEV)
    host = b.seq_lens.cpu()
    ws = L.alloc_workspace(dims, S, b.max_pages, kb, DEV)
    ws.zero_()

    def bufs():
        return (torch.empty(S, H * G, 128, device=DEV), torch.empty(S, H * G, device=DEV),
                torch.empty(S, H, kb, dtype=torch.int32, device=DEV),
                torch.empty(S, H, dtype=torch.int32, device=DEV))

    def reset(t):
        t[0].fill_(float("nan"))
        t[1].fill_(float("nan"))
        t[2].fill_(-9)
        t[3].fill_(-9)

    def step(t):
        L.decode_step(dims, q_d, kn_d, vn_d, kp_d, vp_d, summ_d, tab, lens_d, bud, kb, t[0], ws,
                      lse_out=t[1], sel_pages=t[2], sel_count=t[3], seq_lens_host=host)

    eager = bufs()
    reset(eager)
    step(eager)
    torch.cuda.synchronize()
    res = dict(sel=eager[2].cpu().numpy(), cnt=eager[3].cpu().numpy(), scores=None,
               out=eager[0].cpu().numpy(), lse=eager[1].cpu().numpy())
    assert torch.equal(kp_d.cpu(), b.k_pool) and torch.equal(vp_d.cpu(), b.v_pool)
    _check_against_oracle(b, summ, res, 8, kb)

    static = bufs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(static)
    torch.cuda.synchronize()
    other = bufs()
    for rep in range(4):
        reset(static)
        torch.cuda.synchronize()
        if rep == 2:  # an eager step on the same workspace between replays
            reset(other)
            step(other)
            torch.cuda.synchronize()
            for a, e in zip(other, eager):
                assert torch.equal(a, e), "eager step between replays"
        g.replay()
        torch.cuda.synchronize()
        for a, e in zip(static, eager):
            assert torch.equal(a, e), f"replay {rep}"
    _say("    4 replays bit-identical to the eager step")


@pytest.mark.parametrize("H,r", [(8, 8), (3, 8), (3, 6)])
def test_decode_steps_in_sequence_see_the_appended_tokens(L, H, r):
    """Three decode steps in a row on the same device pools and workspace, each
    appending a token that differs from the placeholder the pools held, the
    first two completing no page and the third one: every step's attention
    must see the tokens appended by the steps before it (the previous step read
    the same tail page, so a stale cached copy would show), checked against
    the oracle on the true pools after each step. With 3 KV heads the score
    and attention workgroups of a head run on different XCDs; rank 6 takes
    the separate score launch."""
    _say(f"[gpu] decode steps in sequence, H={H} r={r}")
    G, kmax = 4, 64
    len3 = 40 * 16  # the third step completes page 39
    b = synth.make_decode_batch([len3], H, G, [24], seed=171, extra_blocks=5)
    dims = L.Dims(H, G, r)
    kp, vp = b.k_pool.clone(), b.v_pool.clone()
    toks = []
    for Lq in (len3 - 2, len3 - 1, len3):   # the three appended positions + 1
        blk, t = int(b.block_table[0, (Lq - 1) // 16]), (Lq - 1) % 16
        toks.append((b.k_pool[blk, :, t].clone(), b.v_pool[blk, :, t].clone()))
        kp[blk, :, t] = 3.0
        vp[blk, :, t] = -3.0
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, torch.tensor([len3 - 16]), H, r, b.num_blocks)
    kp_d, vp_d = kp.to(DEV), vp.to(DEV)
    summ_d = torch.from_numpy(summ).to(DEV)
    ws = L.alloc_workspace(dims, 1, b.max_pages, kmax, DEV)
    ws.fill_(0xA5)
    table = b.block_table.to(DEV)
    budgets = b.budgets.to(DEV)
    q = b.q.to(DEV)
    for i, Lq in enumerate((len3 - 2, len3 - 1, len3)):
        lens = torch.tensor([Lq], dtype=torch.int32)
        sel = torch.full((1, H, kmax), -7, dtype=torch.int32, device=DEV)
        cnt = torch.full((1, H), -7, dtype=torch.int32, device=DEV)
        out = torch.full((1, H * G, 128), 7.0, dtype=torch.float32, device=DEV)
        lse = torch.full((1, H * G), 7.0, dtype=torch.float32, device=DEV)
        kn = toks[i][0].reshape(1, H, 128).to(DEV)
        vn = toks[i][1].reshape(1, H, 128).to(DEV)
        L.decode_step(dims, q, kn, vn, kp_d, vp_d, summ_d, table, lens.to(DEV), budgets, kmax,
                      out, ws, lse_out=lse, sel_pages=sel, sel_count=cnt, seq_lens_host=lens)
        torch.cuda.synchronize()
        # the oracle sees the true tokens up to Lq (and, for its summaries, the
        # GPU-built slot of a page this step completes, checked first)
        bi = synth.DecodeBatch(k_pool=b.k_pool, v_pool=b.v_pool, q=b.q, block_table=b.block_table,
                               seq_lens=lens, budgets=b.budgets, needles=b.needles, H=H, G=G)
        summ_ora = summ.copy()
        if Lq % 16 == 0:
            blk = int(b.block_table[0, Lq // 16 - 1])
            got = summ_d[blk].cpu().numpy()
            keys = np.stack([Hh.np64(b.k_pool[blk, h]) for h in range(H)])
            frac, _, _ = _compare_codes(got, keys, r)
            assert frac <= 1e-3, frac
            summ_ora[blk] = O.build_slots(keys, r)[0]
        res = dict(sel=sel.cpu().numpy(), cnt=cnt.cpu().numpy(), scores=None,
                   out=out.cpu().numpy(), lse=lse.cpu().numpy())
        ws_, nmis, wo = _check_against_oracle(bi, summ_ora, res, r, kmax)
        _say(f"    step {i} (length {Lq}): near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")


@pytest.mark.parametrize("r", [8, 4, 16])
def test_decode_step_full_size_128k(L, r):
    """One layer of the 128K-token, 8-KV-head workload through the fused entry
    point at its real shape (one step after the bulk build), at the rank of
    the headline and at the two other ranks the decode step is timed at."""
    _say(f"[gpu] decode step, full-size 128K layer, r={r}")
    b = synth.config_batch("ctx128k")
    kp, vp, kn, vn, summ, completed = _step_state(b, r)
    res, kpa, vpa, sa = _run_step(L, L.Dims(b.H, b.G, r), b, kp, vp, kn, vn, summ, 128)
    ws, nmis, wo = _check_step(b, r, 128, res, kpa, vpa, sa, summ, completed)
    _say(f"    near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")


def test_decode_step_completes_768_pages(L):
    """96 sequences x 8 KV heads whose new token completes a page: 768 pages
    built inside locks_decode_step, each with its last key taken from k_new,
    checked against the oracle's codes under the +-1 LSB / <= 0.1 % rule; then
    score, select and attend against the oracle fed its own slots."""
    _say("[gpu] decode step completing 768 pages (96 sequences x 8 KV heads)")
    S, H = 96, 8
    rng = np.random.default_rng(7)
    lens = (16 * rng.integers(8, 200, S)).tolist()
    budgets = rng.integers(2, 40, S).tolist()
    b = synth.make_decode_batch(lens, H, 4, budgets, seed=190, extra_blocks=9)
    kp, vp, kn, vn, summ, completed = _step_state(b, 8)
    assert len(completed) == S
    res, kpa, vpa, sa = _run_step(L, L.Dims(H, 4, 8), b, kp, vp, kn, vn, summ, 40)
    ws, nmis, wo = _check_step(b, 8, 40, res, kpa, vpa, sa, summ, completed)
    _say(f"    near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")


BOUNDARY_GAPS = (2e-5, 3e-5, 4e-5, 6e-5, 1e-4, 2e-4, 3e-4, 5e-4)


def test_selection_boundary_planted_gaps(L):
    """Near ties at the selection boundary: for each of 8 KV heads the three
    candidates just above the boundary and the three just below are moved onto
    a ladder whose spacing is one of 2e-5 .. 5e-4 (log-share units, all above
    the 1e-5 tie allowance). The GPU selection must equal the oracle's exactly,
    through the separate entry points and through locks_decode_step."""
    _say("[gpu] planted near ties at the selection boundary")
    H, G, r, k = 8, 4, 8, 64
    b = synth.make_decode_batch([4000 * 16 - 5], H, G, [k], seed=210, needles_per_head=1)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, H, r, b.num_blocks)
    Lq = int(b.seq_lens[0])
    P = (Lq + 15) // 16
    tops = {}
    for h, gap in enumerate(BOUNDARY_GAPS):
        key, top = Hh.plant_boundary(summ, b.block_table, b.q, Lq, k, h, G, r, gap)
        tops[h] = top
        cand = sorted(range(1, P - 1), key=lambda j: (-float(key[j]), j))
        ladder = cand[k - 5:k + 1]
        assert set(ladder) == set(top)
        g = -np.diff([key[j] for j in ladder])
        assert (g > 0.8 * gap).all() and (g < 1.25 * gap).all(), (h, g)
    ora = {h: Hh.oracle_head(b.q, b.k_pool, b.v_pool, b.block_table, b.seq_lens, b.budgets, summ,
                             0, h, G, r) for h in range(H)}
    dims = L.Dims(H, G, r)
    # separate entry points (scores kept for the report)
    res = _run_decode(L, dims, _to_dev(b), torch.from_numpy(summ).to(DEV), k)
    for h in range(H):
        gsel = res["sel"][0, h, :res["cnt"][0, h]].tolist()
        err = np.abs(res["scores"][0, h, tops[h]] - ora[h]["scores"][tops[h]]).max()
        _say(f"    head {h} gap {BOUNDARY_GAPS[h]:.0e}: ladder score err {err:.1e}, "
             f"selection {'equal' if gsel == ora[h]['sel'] else 'DIFFERENT'}")
        assert gsel == ora[h]["sel"], (h, sorted(set(gsel) ^ set(ora[h]["sel"])))
    # fused decode step: the last token enters through k_new / v_new
    kp, vp = b.k_pool.clone(), b.v_pool.clone()
    blk, t = int(b.block_table[0, (Lq - 1) // 16]), (Lq - 1) % 16
    kn, vn = b.k_pool[blk, :, t].clone()[None], b.v_pool[blk, :, t].clone()[None]
    kp[blk, :, t] = 3.0
    vp[blk, :, t] = -3.0
    res2, _, _, _ = _run_step(L, dims, b, kp, vp, kn, vn, summ, k)
    for h in range(H):
        gsel = res2["sel"][0, h, :res2["cnt"][0, h]].tolist()
        assert gsel == ora[h]["sel"], (h, sorted(set(gsel) ^ set(ora[h]["sel"])))
        assert Hh.rel_l2(res2["out"][0, h * G:(h + 1) * G], ora[h]["out"]) <= 1e-2


def test_batch32_full_size(L):
    """The batch of 32 sequences (8K..128K tokens, budgets max(8, ceil(P/16)))
    at its real shape: GPU bulk build of every full page (two pairs compared
    with the oracle's codes), then every (sequence, KV head) pair scored,
    selected and attended from oracle-built slots, through the separate entry
    points and through locks_decode_step (one token earlier: every sequence's
    new token completes a page, which the step builds), each pair against the
    oracle. The oracle runs over a pool of worker processes."""
    _say("[gpu] batch of 32 sequences, full size, every (sequence, KV head)")
    b = synth.config_batch("batch32", device=DEV)
    S, H, G, r = b.num_seqs, b.H, b.G, 8
    dims = L.Dims(H, G, r)
    lens = [int(x) for x in b.seq_lens.tolist()]
    kmax = int(b.budgets.max())
    # GPU bulk build of every full page
    summ = L.alloc_summaries(dims, b.num_blocks, DEV)
    full = torch.cat([b.block_table[sq, :lens[sq] // 16] for sq in range(S)]).contiguous()
    L.build(dims, b.k_pool, full, summ)
    torch.cuda.synchronize()
    kp_c, vp_c, q_c, tb_c = b.k_pool.cpu(), b.v_pool.cpu(), b.q.cpu(), b.block_table.cpu()
    _say("    oracle over 256 (sequence, KV head) pairs (worker processes)")
    ora = Hh.oracle_pairs_parallel(kp_c, vp_c, q_c, tb_c, b.seq_lens.cpu(), b.budgets.cpu(), H, G, r)
    for (sq, h) in ((0, 0), (17, 6)):
        F = lens[sq] // 16
        blocks = tb_c[sq, :F].long()
        frac, _, _ = _compare_codes(summ[blocks.to(DEV), h].cpu().numpy(),
                                    kp_c[blocks, h].double().numpy(), r)
        assert frac <= 1e-3
    # every pair scored from the oracle's slots
    summ_np = np.zeros((b.num_blocks, H, summ.shape[2]), dtype=np.uint8)
    for (sq, h), (slots, *_rest) in ora.items():
        summ_np[tb_c[sq, :lens[sq] // 16].long().numpy(), h] = slots
    summ = torch.from_numpy(summ_np).to(DEV)

    def check(res, tag):
        worst, nmis = 0.0, 0
        for (sq, h), (_slots, osel, okey, oout, olse) in ora.items():
            Lq = lens[sq]
            P = (Lq + 15) // 16
            n = int(res["cnt"][sq, h])
            gsel = [int(j) for j in res["sel"][sq, h, :n]]
            assert gsel == sorted(gsel) and n == min(max(int(b.budgets[sq]), 2), kmax, P)
            nmis += Hh.selection_mismatch(gsel, osel, okey, P)
            if gsel == osel:
                o_ref, lse_ref = oout, olse
            else:
                blocks = tb_c[sq, :P].long()
                Kp, Vp = kp_c[blocks, h].double().numpy(), vp_c[blocks, h].double().numpy()
                nt = [16 if j < P - 1 else Lq - 16 * (P - 1) for j in gsel]
                o_ref, lse_ref = O.attend(Hh.np64(q_c[sq, h * G:(h + 1) * G]),
                                          np.concatenate([Kp[j, :m] for j, m in zip(gsel, nt)]),
                                          np.concatenate([Vp[j, :m] for j, m in zip(gsel, nt)]))
            e = Hh.rel_l2(res["out"][sq, h * G:(h + 1) * G], o_ref)
            assert e <= 1e-2, (tag, sq, h, e)
            np.testing.assert_allclose(res["lse"][sq, h * G:(h + 1) * G], lse_ref, atol=1e-3)
            worst = max(worst, e)
        _say(f"    {tag}: 256 pairs, near-tie swaps {nmis}, worst attn rel-L2 {worst:.2e}")

    check(_run_decode(L, dims, b, summ, kmax, scores=False), "separate entry points")

    # the same batch one token earlier, stepped by locks_decode_step: the
    # token at len - 1 completes a page in every sequence (lengths are page
    # multiples), which the step appends and builds
    kp, vp = b.k_pool.clone(), b.v_pool.clone()
    kn = torch.empty(S, H, 128, dtype=torch.bfloat16, device=DEV)
    vn = torch.empty_like(kn)
    last = []
    for sq in range(S):
        blk, t = int(b.block_table[sq, (lens[sq] - 1) // 16]), (lens[sq] - 1) % 16
        kn[sq], vn[sq] = b.k_pool[blk, :, t], b.v_pool[blk, :, t]
        kp[blk, :, t] = 3.0
        vp[blk, :, t] = -3.0
        summ[blk] = 0
        last.append(blk)
    out = torch.full((S, H * G, 128), 7.0, device=DEV)
    lse = torch.full((S, H * G), 7.0, device=DEV)
    sel = torch.full((S, H, kmax), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((S, H), -7, dtype=torch.int32, device=DEV)
    ws = L.alloc_workspace(dims, S, b.max_pages, kmax, DEV)
    L.decode_step(dims, b.q, kn, vn, kp, vp, summ, b.block_table, b.seq_lens, b.budgets, kmax, out,
                  ws, lse_out=lse, sel_pages=sel, sel_count=cnt, seq_lens_host=b.seq_lens.cpu())
    torch.cuda.synchronize()
    assert torch.equal(kp, b.k_pool) and torch.equal(vp, b.v_pool)
    # the 256 pages the step built, against the oracle's codes
    got = summ[torch.tensor(last, device=DEV)].cpu().numpy()             # (S, H, stride)
    keys = np.stack([kp_c[blk, h].double().numpy() for blk in last for h in range(H)])
    frac, _, _ = _compare_codes(got.reshape(S * H, -1), keys, r)
    assert frac <= 1e-3
    check(dict(sel=sel.cpu().numpy(), cnt=cnt.cpu().numpy(), out=out.cpu().numpy(),
               lse=lse.cpu().numpy()), "locks_decode_step")


@pytest.mark.parametrize("G,r", [(4, 8), (2, 6)])
def test_decode_step_deferred_build(L, G, r):
    """LOCKS_STEP_DEFER_BUILD (the build outside the decode critical path):
    the step appends every token, builds nothing and scores only the pages full
    before its token (checked against the oracle's deferred reading); then
    locks_build_filled summarises exactly the pages the tokens completed
    (code rule against the oracle), and the next step, one token later on the
    same pools (no page completes), uses them. Rank 6 takes the separate score
    launch."""
    _say(f"[gpu] decode step with the build deferred, G={G} r={r}")
    lens = [16, 17, 32, 40 * 16, 40 * 16 + 1, 300 * 16 + 9, 257 * 16, 33, 64 * 16]
    budgets = [2, 3, 5, 2, 7, 64, 300, 2, 9]
    b2 = synth.make_decode_batch([x + 1 for x in lens], 3, G, budgets, seed=260 + G, extra_blocks=11)
    b1 = synth.DecodeBatch(k_pool=b2.k_pool, v_pool=b2.v_pool, q=b2.q, block_table=b2.block_table,
                           seq_lens=torch.tensor(lens, dtype=torch.int32), budgets=b2.budgets,
                           needles=b2.needles, H=b2.H, G=G)
    kp, vp, kn, vn, summ, completed = _step_state(b1, r)
    dims = L.Dims(b1.H, G, r)
    res, kpa, vpa, sa = _run_step(L, dims, b1, kp, vp, kn, vn, summ, 300, defer_build=True)
    assert torch.equal(kpa, b2.k_pool) and torch.equal(vpa, b2.v_pool)
    assert np.array_equal(sa, summ)                       # nothing built by the step
    _, nmis, wo = _check_against_oracle(b1, summ, res, r, 300, deferred=True)
    _say(f"    deferred step: near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")
    # the caller's build of the completed pages
    summ_d = torch.from_numpy(sa).to(DEV)
    L.build_filled(dims, kpa.to(DEV), b1.block_table.to(DEV), b1.seq_lens.to(DEV), summ_d)
    torch.cuda.synchronize()
    built = summ_d.cpu().numpy()
    pairs = [(blk, h) for blk in completed for h in range(b1.H)]
    keys = np.stack([Hh.np64(b2.k_pool[blk, h]) for blk, h in pairs])
    frac, _, _ = _compare_codes(np.stack([built[blk, h] for blk, h in pairs]), keys, r)
    assert frac <= 1e-3
    for blk in range(b1.num_blocks):
        if blk not in completed:
            assert np.array_equal(built[blk], summ[blk])
    # the next step on the same pools: the token at position len, appended again
    kn2 = torch.zeros_like(kn)
    vn2 = torch.zeros_like(vn)
    for sq, Lq in enumerate(lens):
        blk, t = int(b2.block_table[sq, Lq // 16]), Lq % 16
        kn2[sq], vn2[sq] = b2.k_pool[blk, :, t], b2.v_pool[blk, :, t]
    summ_ora = summ.copy()
    ora_slots = O.build_slots(keys, r)[0]
    for i, (blk, h) in enumerate(pairs):
        summ_ora[blk, h] = ora_slots[i]
    res2, kpb, _, _ = _run_step(L, dims, b2, kpa, vpa, kn2, vn2, summ_ora, 300, defer_build=True)
    assert torch.equal(kpb, b2.k_pool)
    _, nmis2, wo2 = _check_against_oracle(b2, summ_ora, res2, r, 300, deferred=True)
    _say(f"    next step: near-tie swaps {nmis2}, worst attn rel-L2 {wo2:.2e}")
