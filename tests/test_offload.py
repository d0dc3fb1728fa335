"""Offload path ([N] §8: only the summaries on the accelerator, the KV cache
in host memory): K/V pools in pinned, device-mapped host memory
(locks_host_pool_alloc) give the same results, bit for bit, as pools in
device memory, through the decode step (in-step and deferred builds), the
separate attention entry point and the bulk build; the step's result is also
checked against the oracle."""
import numpy as np
import pytest
import torch

import synth
from tests.test_gpu_parity import DEV, _check_against_oracle, _say, _step_state


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from kv_cache_page_amd import locks
    return locks


def _host_copy(L, t):
    hp = L.HostPool(t.shape, t.dtype)
    hp.host.copy_(t)
    return hp


def _step(L, dims, b, kp, vp, kn, vn, summ, kmax, defer):
    S, H, G = b.num_seqs, b.H, b.G
    summ_d = torch.from_numpy(summ).to(DEV)
    sel = torch.full((S, H, kmax), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((S, H), -7, dtype=torch.int32, device=DEV)
    out = torch.full((S, H * G, 128), 7.0, device=DEV)
    lse = torch.full((S, H * G), 7.0, device=DEV)
    ws = L.alloc_workspace(dims, S, b.max_pages, kmax, DEV)
    L.decode_step(dims, b.q.to(DEV), kn.to(DEV), vn.to(DEV), kp, vp, summ_d,
                  b.block_table.to(DEV), b.seq_lens.to(DEV), b.budgets.to(DEV), kmax, out, ws,
                  lse_out=lse, sel_pages=sel, sel_count=cnt, seq_lens_host=b.seq_lens.cpu(),
                  defer_build=defer)
    torch.cuda.synchronize()
    return dict(sel=sel.cpu().numpy(), cnt=cnt.cpu().numpy(), out=out.cpu().numpy(),
                lse=lse.cpu().numpy(), scores=None), summ_d


@pytest.mark.gpu
@pytest.mark.parametrize("defer", [False, True])
def test_offload_decode_step_matches_device_pools(L, defer):
    _say(f"[gpu] offload decode step, deferred build {defer}")
    lens = [16 * 300, 16 * 512 + 7, 16 * 40 + 1, 33, 16 * 96]
    b = synth.make_decode_batch(lens, 4, 4, [24, 40, 8, 3, 96], seed=301, extra_blocks=5)
    r, kmax = 8, 96
    dims = L.Dims(b.H, b.G, r)
    kp, vp, kn, vn, summ, completed = _step_state(b, r)
    kp_d, vp_d = kp.to(DEV), vp.to(DEV)
    res_d, summ_dd = _step(L, dims, b, kp_d, vp_d, kn, vn, summ, kmax, defer)
    hk, hv = _host_copy(L, kp), _host_copy(L, vp)
    res_h, summ_hd = _step(L, dims, b, hk, hv, kn, vn, summ, kmax, defer)
    for key in ("sel", "cnt", "out", "lse"):
        assert np.array_equal(res_h[key], res_d[key]), key
    assert torch.equal(hk.host, kp_d.cpu()) and torch.equal(hv.host, vp_d.cpu())
    assert torch.equal(hk.host, b.k_pool) and torch.equal(hv.host, b.v_pool)
    assert torch.equal(summ_hd, summ_dd)
    if defer:
        ids_dev = (b.block_table.to(DEV), b.seq_lens.to(DEV))
        L.build_filled(dims, kp_d, *ids_dev, summ_dd)
        L.build_filled(dims, hk, *ids_dev, summ_hd)
        torch.cuda.synchronize()
        assert torch.equal(summ_hd, summ_dd)
    ref = summ if defer else summ_hd.cpu().numpy()
    _, nmis, wo = _check_against_oracle(b, ref, res_h, r, kmax, deferred=defer)
    _say(f"    near-tie swaps {nmis}, worst attn rel-L2 {wo:.2e}")
    hk.free()
    hv.free()


@pytest.mark.gpu
def test_offload_sparse_attn_and_bulk_build(L):
    _say("[gpu] offload sparse attention and bulk build")
    lens = [16 * 700 + 3, 16 * 64, 5]
    b = synth.make_decode_batch(lens, 8, 4, [64, 16, 2], seed=302)
    r, kmax = 8, 64
    dims = L.Dims(b.H, b.G, r)
    S = b.num_seqs
    kp_d, vp_d = b.k_pool.to(DEV), b.v_pool.to(DEV)
    hk, hv = _host_copy(L, b.k_pool), _host_copy(L, b.v_pool)
    ids = torch.arange(b.num_blocks, dtype=torch.int32, device=DEV)
    summ_d = L.alloc_summaries(dims, b.num_blocks, DEV)
    summ_h = L.alloc_summaries(dims, b.num_blocks, DEV)
    L.build(dims, kp_d, ids, summ_d)
    L.build(dims, hk, ids, summ_h)
    torch.cuda.synchronize()
    assert torch.equal(summ_h, summ_d)
    table, seq_lens, q = b.block_table.to(DEV), b.seq_lens.to(DEV), b.q.to(DEV)
    sel = torch.empty(S, b.H, kmax, dtype=torch.int32, device=DEV)
    cnt = torch.empty(S, b.H, dtype=torch.int32, device=DEV)
    ws = L.alloc_workspace(dims, S, b.max_pages, kmax, DEV)
    L.score_select(dims, q, summ_d, table, seq_lens, b.budgets.to(DEV), kmax, sel, cnt, ws)
    outs = []
    for kpool, vpool in ((kp_d, vp_d), (hk, hv)):
        out = torch.full((S, b.H * b.G, 128), 7.0, device=DEV)
        lse = torch.full((S, b.H * b.G), 7.0, device=DEV)
        L.sparse_attn(dims, q, kpool, vpool, table, seq_lens, sel, cnt, kmax, out, ws,
                      lse_out=lse)
        torch.cuda.synchronize()
        outs.append((out.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    hk.free()
    hv.free()
