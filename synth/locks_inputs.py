"""Seeded generators of paged-KV decode inputs (see the package docstring).

All generation runs with torch on the requested device from a seeded
torch.Generator, so a run is reproducible on that device. Pools use the
layout [num_blocks][H_kv][B][d] (bf16); block tables are int32
[num_seqs][max_pages] of physical block ids.
"""
from __future__ import annotations

import dataclasses
import math

import torch

SIGMAS = (3.0, 2.5, 2.0, 1.6, 1.3, 1.0, 0.8, 0.6)
# a slowly decaying spectrum over all 15 centred directions of a 16-token
# page (sigma_k = 3 k^-0.5): rank-8 summaries then leave a real tail
TAIL_SIGMAS = tuple(3.0 * k ** -0.5 for k in range(1, 16))
NOISE = 0.05
NEEDLE_NORM = 6.0
QUERY_NOISE = 0.3

__all__ = [
    "SIGMAS", "TAIL_SIGMAS", "DecodeBatch", "page_keys", "page_values", "gqa_queries",
    "make_decode_batch", "config_batch", "random_pages", "LayerStack", "make_layer_stack",
]


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _orthonormal(n, d, m, g, device):
    """n random orthonormal d x m bases by modified Gram-Schmidt (fp32)."""
    A = torch.randn(n, d, m, generator=g, device=device, dtype=torch.float32)
    cols = []
    for j in range(m):
        v = A[:, :, j]
        for u in cols:
            v = v - (u * v).sum(dim=1, keepdim=True) * u
        v = v / v.norm(dim=1, keepdim=True)
        cols.append(v)
    return torch.stack(cols, dim=2)


def page_keys(n, g, B=16, d=128, device="cpu", noise=NOISE, sigmas=SIGMAS,
              chunk=1 << 16):
    """n pages of keys with page-specific rank-len(sigmas) structure, fp32
    (n, B, d). Generated in chunks of pages to bound temporary memory."""
    out = torch.empty(n, B, d, dtype=torch.float32, device=device)
    sig = torch.tensor(sigmas, dtype=torch.float32, device=device)
    m = len(sigmas)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        mu = torch.randn(c, 1, d, generator=g, device=device)
        U = _orthonormal(c, d, m, g, device)
        z = torch.randn(c, B, m, generator=g, device=device) * sig
        eps = torch.randn(c, B, d, generator=g, device=device)
        out[s:s + c] = mu + torch.bmm(z, U.transpose(1, 2)) + noise * eps
    return out


def page_values(n, g, B=16, d=128, device="cpu"):
    return torch.randn(n, B, d, generator=g, device=device)


def gqa_queries(n_groups, G, g, d=128, device="cpu"):
    """(n_groups, G, d) queries and (n_groups, d) their shared directions."""
    q_dir = torch.randn(n_groups, d, generator=g, device=device)
    q = q_dir[:, None, :] + QUERY_NOISE * torch.randn(n_groups, G, d, generator=g, device=device)
    return q, q_dir


@dataclasses.dataclass
class DecodeBatch:
    """One layer's decode inputs. Tensors live on one device."""
    k_pool: torch.Tensor        # bf16 [num_blocks][H][B][d]
    v_pool: torch.Tensor        # bf16 [num_blocks][H][B][d]
    q: torch.Tensor             # bf16 [S][H*G][d]
    block_table: torch.Tensor   # int32 [S][max_pages]
    seq_lens: torch.Tensor      # int32 [S]
    budgets: torch.Tensor       # int32 [S]
    needles: list               # (seq, head, logical page, slot) tuples
    H: int
    G: int
    B: int = 16
    d: int = 128

    @property
    def num_seqs(self):
        return self.seq_lens.shape[0]

    @property
    def max_pages(self):
        return self.block_table.shape[1]

    @property
    def num_blocks(self):
        return self.k_pool.shape[0]


def make_decode_batch(seq_lens, H, G, budgets, seed, needles_per_head=1,
                      shuffle=True, device="cpu", extra_blocks=0, d=128, B=16,
                      sigmas=SIGMAS):
    """Ragged batch of sequences over a shared block pool.

    seq_lens: list of token counts (current token included). Blocks of all
    sequences are drawn from one pool (shuffled when `shuffle`), with
    `extra_blocks` unused blocks in the pool. Needles go to uniformly drawn
    logical pages 1..P-2 (never the sink or the recent page) and a uniform
    slot within the page. `sigmas` sets the within-page key spectrum."""
    g = _gen(seed, device)
    gc = _gen(seed + 7919, "cpu")          # host-side choices (tables, needles)
    pages = [(L + B - 1) // B for L in seq_lens]
    max_pages = max(pages)
    nblk = sum(pages) + extra_blocks
    perm = torch.randperm(nblk, generator=gc) if shuffle else torch.arange(nblk)
    table = torch.zeros(len(seq_lens), max_pages, dtype=torch.int32)
    pos = 0
    for s, P in enumerate(pages):
        table[s, :P] = perm[pos:pos + P].to(torch.int32)
        pos += P
    n_pages = nblk * H
    k = page_keys(n_pages, g, B, d, device, sigmas=sigmas).view(nblk, H, B, d)
    v = page_values(n_pages, g, B, d, device).view(nblk, H, B, d)
    q, q_dir = gqa_queries(len(seq_lens) * H, G, g, d, device)
    needles = []
    if needles_per_head:
        unit = q_dir / q_dir.norm(dim=1, keepdim=True)
        for s, P in enumerate(pages):
            if P < 3:
                continue
            for h in range(H):
                for _ in range(needles_per_head):
                    j = 1 + int(torch.randint(P - 2, (1,), generator=gc))
                    slot = int(torch.randint(B, (1,), generator=gc))
                    blk = int(table[s, j])
                    k[blk, h, slot] = NEEDLE_NORM * unit[s * H + h]
                    needles.append((s, h, j, slot))
    return DecodeBatch(
        k_pool=k.to(torch.bfloat16), v_pool=v.to(torch.bfloat16),
        q=q.view(len(seq_lens), H * G, d).to(torch.bfloat16),
        block_table=table.to(device), seq_lens=torch.tensor(seq_lens, dtype=torch.int32, device=device),
        budgets=torch.tensor(budgets, dtype=torch.int32, device=device),
        needles=needles, H=H, G=G, B=B, d=d)


def random_pages(n, seed, B=16, d=128, device="cpu", noise=NOISE):
    """n independent full pages of keys (bf16 [n][B][d]) for the build path."""
    g = _gen(seed, device)
    return page_keys(n, g, B, d, device, noise=noise).to(torch.bfloat16)


def config_batch(name, device="cpu", seed=None):
    """The decode workloads by name, at their stated sizes.

    tiny:    1 seq, 1 KV head, G = 4, 4096 tokens (256 pages), k = 16,
             1 needle.
    ctx32k:  1 seq, 8 KV heads, G = 4, 32768 tokens (2048 pages), k = 64,
             4 needles per KV head.
    ctx128k: 1 seq, 8 KV heads, G = 4, 131072 tokens (8192 pages), k = 128,
             1 needle per KV head (one layer of the 32-layer loop).
    batch32: 32 seqs, lengths uniform in 8K..128K tokens in multiples of 16,
             8 KV heads, G = 4, k_s = max(8, ceil(P_s / 16)), 2 needles per
             seq-head, blocks shuffled in one pool.
    """
    if name == "tiny":
        return make_decode_batch([4096], 1, 4, [16], 0 if seed is None else seed,
                                 needles_per_head=1, device=device)
    if name == "ctx32k":
        return make_decode_batch([32768], 8, 4, [64], 1 if seed is None else seed,
                                 needles_per_head=4, device=device)
    if name == "ctx128k":
        return make_decode_batch([131072], 8, 4, [128], 2 if seed is None else seed,
                                 needles_per_head=1, device=device)
    if name == "batch32":
        sd = 3 if seed is None else seed
        gc = _gen(sd + 104729, "cpu")
        lens = (torch.randint(8192 // 16, 131072 // 16 + 1, (32,), generator=gc) * 16).tolist()
        budgets = [max(8, math.ceil(((L + 15) // 16) / 16)) for L in lens]
        return make_decode_batch(lens, 8, 4, budgets, sd, needles_per_head=2, device=device)
    raise ValueError(name)


@dataclasses.dataclass
class LayerStack:
    """A single long sequence across `layers` layers that share one block
    table, with every layer's pools filled for `max_len` tokens and queries
    drawn for every (step, layer). Token t of the sequence lives in block
    block_table[0, t // B], slot t % B."""
    k_pools: list               # per layer bf16 [num_blocks][H][B][d]
    v_pools: list
    q: torch.Tensor             # bf16 [steps][layers][1][H*G][d]
    block_table: torch.Tensor   # int32 [1][max_pages]
    needles: list               # (layer, head, logical page, slot)
    H: int
    G: int
    max_len: int
    B: int = 16
    d: int = 128
    k_all: torch.Tensor = None  # the one allocation the layers' pools are slices of
    v_all: torch.Tensor = None


def make_layer_stack(layers, max_len, H, G, steps, seed, needle_pages, device="cpu",
                     d=128, B=16):
    """Pools for `layers` layers of one `max_len`-token sequence (blocks
    shuffled), one needle per (layer, KV head) on a logical page drawn
    uniformly from 1..needle_pages-2, and fresh query noise for each of
    `steps` decode steps (one q_dir per (layer, KV head))."""
    gc = _gen(seed + 7919, "cpu")
    P = (max_len + B - 1) // B
    table = torch.randperm(P, generator=gc).to(torch.int32).view(1, P)
    # every layer's pool is a slice of one allocation ([layers * P][H][B][d]),
    # so block id b of layer l is block l * P + b of the whole
    k_all = torch.empty(layers * P, H, B, d, dtype=torch.bfloat16, device=device)
    v_all = torch.empty_like(k_all)
    kps, vps, qs, needles = [], [], [], []
    for l in range(layers):
        g = _gen(seed * 1000 + l, device)
        k = page_keys(P * H, g, B, d, device).view(P, H, B, d)
        v = page_values(P * H, g, B, d, device).view(P, H, B, d)
        q_dir = torch.randn(H, d, generator=g, device=device)
        unit = q_dir / q_dir.norm(dim=1, keepdim=True)
        for h in range(H):
            j = 1 + int(torch.randint(max(needle_pages - 2, 1), (1,), generator=gc))
            slot = int(torch.randint(B, (1,), generator=gc))
            k[int(table[0, j]), h, slot] = NEEDLE_NORM * unit[h]
            needles.append((l, h, j, slot))
        k_all[l * P:(l + 1) * P] = k
        v_all[l * P:(l + 1) * P] = v
        kps.append(k_all[l * P:(l + 1) * P])
        vps.append(v_all[l * P:(l + 1) * P])
        noise = torch.randn(steps, H, G, d, generator=g, device=device)
        qs.append((q_dir[None, :, None, :] + QUERY_NOISE * noise).reshape(steps, 1, H * G, d))
        del k, v
    q = torch.stack(qs, dim=1).to(torch.bfloat16)        # [steps][layers][1][H*G][d]
    return LayerStack(k_pools=kps, v_pools=vps, q=q, block_table=table.to(device),
                      needles=needles, H=H, G=G, max_len=max_len, B=B, d=d, k_all=k_all,
                      v_all=v_all)
