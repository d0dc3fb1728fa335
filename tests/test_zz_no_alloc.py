"""locks_decode_step_noalloc against locks_decode_step, through the C ABI.

Two calls in a row on the built-in scratch, the second with a smaller input
(fewer pages, fewer KV heads, a different split count), each compared with
locks_decode_step on its own workspace over identical copies of the inputs:
outputs, log-sum-exps, selections, the appended pools and the summaries built
for completed pages must be identical (the two share their kernels). A shape
whose workspace exceeds the scratch is rejected before anything runs."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from kv_cache_page_amd import locks
    return locks


def _inputs(L, lens, H, budgets, seed, r=8, G=4):
    """A decode batch one token before its step: the token at len - 1 removed
    from the pools (placeholder values) and returned as k_new / v_new, every
    full page summarised by locks_build except those the token completes."""
    b = synth.make_decode_batch(lens, H, G, budgets, seed=seed, extra_blocks=3)
    dims = L.Dims(H, G, r)
    kp, vp = b.k_pool.clone(), b.v_pool.clone()
    S = len(lens)
    kn = torch.zeros(S, H, 128, dtype=torch.bfloat16)
    vn = torch.zeros_like(kn)
    before = []
    for s, Lq in enumerate(lens):
        blk, t = int(b.block_table[s, (Lq - 1) // 16]), (Lq - 1) % 16
        kn[s], vn[s] = b.k_pool[blk, :, t], b.v_pool[blk, :, t]
        kp[blk, :, t] = 3.0
        vp[blk, :, t] = -3.0
        before += b.block_table[s, :(Lq - 1) // 16].tolist()
    kp, vp, kn, vn = kp.to(DEV), vp.to(DEV), kn.to(DEV), vn.to(DEV)
    summ = L.alloc_summaries(dims, b.num_blocks, DEV)
    L.build(dims, kp, torch.tensor(before, dtype=torch.int32, device=DEV), summ)
    return dims, b, kp, vp, kn, vn, summ


def _step(L, fn, dims, b, kp, vp, kn, vn, summ, kmax, ws=None):
    S, H, G = b.num_seqs, b.H, b.G
    kp, vp, summ = kp.clone(), vp.clone(), summ.clone()
    out = torch.full((S, H * G, 128), 7.0, device=DEV)
    lse = torch.full((S, H * G), 7.0, device=DEV)
    sel = torch.full((S, H, kmax), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((S, H), -7, dtype=torch.int32, device=DEV)
    args = (dims, b.q.to(DEV), kn, vn, kp, vp, summ, b.block_table.to(DEV), b.seq_lens.to(DEV),
            b.budgets.to(DEV), kmax, out)
    kw = dict(lse_out=lse, sel_pages=sel, sel_count=cnt, seq_lens_host=b.seq_lens.cpu())
    if ws is None:
        fn(*args, **kw)
    else:
        fn(*args[:-1], out, ws, **kw)
    torch.cuda.synchronize()
    return [x.cpu() for x in (out, lse, sel, cnt, kp, vp, summ)]


def test_noalloc_matches_decode_step_twice(L):
    cases = [
        # (lengths, KV heads, budgets, seed): the first larger (2 x 8 heads, a
        # 3000-page table, one sequence completing a page), the second smaller
        ([3000 * 16 - 3, 1200 * 16], 8, [128, 64], 301),
        ([500 * 16 + 7], 3, [40], 302),
    ]
    for lens, H, budgets, seed in cases:
        print(f"[gpu] no-alloc decode step: lengths {lens}, {H} KV heads", flush=True)
        dims, b, kp, vp, kn, vn, summ = _inputs(L, lens, H, budgets, seed)
        kmax = max(budgets)
        assert L.workspace_bytes(dims, b.num_seqs, b.max_pages, kmax) <= L.NOALLOC_SCRATCH_BYTES
        ws = L.alloc_workspace(dims, b.num_seqs, b.max_pages, kmax, DEV)
        ref = _step(L, L.decode_step, dims, b, kp, vp, kn, vn, summ, kmax, ws=ws)
        got = _step(L, L.decode_step_noalloc, dims, b, kp, vp, kn, vn, summ, kmax)
        for name, a, c in zip(("out", "lse", "sel", "cnt", "k_pool", "v_pool", "summaries"), ref, got):
            assert torch.equal(a, c), name
        assert not torch.isnan(got[0]).any()


def test_noalloc_rejects_oversize_shape(L):
    """32 sequences of 8192-page tables with budgets of 512 need far more
    workspace than the scratch holds: rejected before anything is enqueued."""
    dims = L.Dims(8, 4, 8)
    assert L.workspace_bytes(dims, 32, 8192, 512) > L.NOALLOC_SCRATCH_BYTES
    kp = torch.zeros(16, 8, 16, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(L.LocksError) as e:
        L.decode_step_noalloc(dims, torch.zeros(32, 32, 128, dtype=torch.bfloat16, device=DEV),
                              torch.zeros(32, 8, 128, dtype=torch.bfloat16, device=DEV),
                              torch.zeros(32, 8, 128, dtype=torch.bfloat16, device=DEV), kp,
                              kp.clone(), L.alloc_summaries(dims, 16, DEV),
                              torch.zeros(32, 8192, dtype=torch.int32, device=DEV),
                              torch.ones(32, dtype=torch.int32, device=DEV),
                              torch.full((32,), 512, dtype=torch.int32, device=DEV), 512,
                              torch.zeros(32, 32, 128, device=DEV))
    assert e.value.status == L.ERR_WORKSPACE


def test_noalloc_graph_replays(L):
    """locks_decode_step_noalloc captured in a HIP graph (the kind of caller it
    is for) and replayed three times, with the outputs reset by eager work and
    the stream synchronised between replays: every replay equals the eager
    locks_decode_step on its own workspace, bit for bit (outputs, log-sum-exps,
    selections, pools, summaries). No length completes a page."""
    lens, H, budgets = [700 * 16 + 3, 90 * 16 + 11], 8, [64, 16]
    print(f"[gpu] no-alloc decode step in a HIP graph: lengths {lens}, {H} KV heads", flush=True)
    dims, b, kp, vp, kn, vn, summ = _inputs(L, lens, H, budgets, 303)
    kmax = max(budgets)
    ws = L.alloc_workspace(dims, b.num_seqs, b.max_pages, kmax, DEV)
    ref = _step(L, L.decode_step, dims, b, kp, vp, kn, vn, summ, kmax, ws=ws)
    S, G = b.num_seqs, b.G
    kp2, vp2, summ2 = kp.clone(), vp.clone(), summ.clone()
    q, tab = b.q.to(DEV), b.block_table.to(DEV)
    lens_d, bud = b.seq_lens.to(DEV), b.budgets.to(DEV)
    host = b.seq_lens.cpu()
    out = torch.empty(S, H * G, 128, device=DEV)
    lse = torch.empty(S, H * G, device=DEV)
    sel = torch.empty(S, H, kmax, dtype=torch.int32, device=DEV)
    cnt = torch.empty(S, H, dtype=torch.int32, device=DEV)

    def step():
        L.decode_step_noalloc(dims, q, kn, vn, kp2, vp2, summ2, tab, lens_d, bud, kmax, out,
                              lse_out=lse, sel_pages=sel, sel_count=cnt, seq_lens_host=host)

    step()  # the per-device set-up happens outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        sel.fill_(-9)
        cnt.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [x.cpu() for x in (out, lse, sel, cnt, kp2, vp2, summ2)]
        for name, a, c in zip(("out", "lse", "sel", "cnt", "k_pool", "v_pool", "summaries"), ref, got):
            assert torch.equal(a, c), (rep, name)
