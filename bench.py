#!/usr/bin/env python3
"""Decode-step benchmark of the LOCKS hot path on one MI355X.

Headline workload (synthetic, Llama-3.1-8B-shaped): one sequence at 128K
context, 32 layers, 8 KV heads x 4 query heads, d = 128, bf16 K/V, pages of
16 tokens, rank-8 int4/int8 page summaries, a budget of 128 pages per KV
head. The KV cache holds 131072 tokens' worth of pages; the sequence starts
W+K tokens short of 131072 and every decode step appends one token, so the
last timed step runs at exactly 131072 tokens.

One step = for every layer: append the new token's K/V, score every page that
was full before it from the summaries, select sink + recent + top-126 pages
and attend over them, through locks_decode_step (one launch per layer). The
summary of a page the token completes is built outside the decode critical
path: the layers' pools are slices of one allocation, so after the layer loop
one locks_build call over that page's block id in every layer summarises all
256 (layer, KV head) pages in one parallel launch (the step whose token
completes a page leaves that page out of the shares; it is the recent page
and always selected). The page-completing step is also timed with the build
inside each layer's step (locks_decode_step's default). Each step is captured once as
a HIP graph; W warm-up steps run, then K steps are timed between HIP events.

Throughput counts the metric's algorithmic bytes: 818 summary bytes per full
page and KV head, plus 8192 bytes per selected full page (512 per valid token
of the last page) and KV head, per layer.

Further workloads, each with its own roofline entry under "workloads":
  ctx32k_1layer   one layer at 32K context (8 KV heads, k = 64), over 32
                  replicas of the cache taken in turn, so that the step's
                  17.6 MB do not stay in the 256 MB Infinity Cache;
  batch32_ragged  one layer, 32 sequences of 8K..128K tokens in a shared
                  shuffled block pool, k = max(8, ceil(P / 16));
  bulk_build      locks_build over the 2,097,152 pages of the 32-layer
                  cache at r = 4, 8 and 16 (pages/s, bytes per page, fp64
                  ALU roofline);
  offload_ctx128k the 128K step with the K/V pools in pinned host memory
                  (summaries in HBM): the selected pages cross the host
                  link (roofline against PCIe 5.0 x16, one direction);
  rank_sweep_ctx128k  one 128K layer's decode step at r = 4, 8 and 16
                  (490 / 818 / 1474 summary bytes per page), over 8
                  replicas of the summaries taken in turn.

The final timed step's layer-0 outputs are checked against the fp64 oracle
(and every output for NaN); the run exits non-zero on a mismatch.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import concurrent.futures
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LAYERS, H, G, D, B, R, BUDGET, MAX_LEN = 32, 8, 4, 128, 16, 8, 128, 131072
PAGE_KV_BYTES = 2 * B * D * 2
HBM_PEAK_GBS = 8000.0
HOST_LINK_PEAK_GBS = 63.0     # PCIe 5.0 x16, one direction (32 GT/s x 16 lanes, 128b/130b)
FP64_VALU_PEAK_TFLOPS = 78.6
METRIC = "decode-step µs and achieved HBM GB/s (summary+selected KV) at 128K ctx, 8 KV heads"
CSRC = os.path.join(ROOT, "kv_cache_page_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
_STEP_SRC = ("locks_decode.hip", ["locks_score_tile.h", "locks_attn_core.h", "locks_select.h",
                                  "locks_step.h", "locks_device.h"])
_BUILD_SRC = ("locks_build_page.hip", ["locks_build_common.h", "locks_device.h"])
# (counter summary, source, headers) of every kernel a roofline entry reports on
KERNELS = {
    "step": (os.path.join(PROFILES, "decode_step_kernel_ctx128k_counters.txt"), *_STEP_SRC),
    "score": (os.path.join(PROFILES, "score_kernel_ctx128k_counters.txt"),
              "locks_score_mfma.hip", ["locks_score_tile.h", "locks_device.h"]),
    "step32k": (os.path.join(PROFILES, "decode_step_kernel_ctx32k_counters.txt"), *_STEP_SRC),
    "stepb32": (os.path.join(PROFILES, "decode_step_kernel_batch32_counters.txt"), *_STEP_SRC),
    "step_r4": (os.path.join(PROFILES, "decode_step_kernel_r4_ctx128k_counters.txt"), *_STEP_SRC),
    "step_r16": (os.path.join(PROFILES, "decode_step_kernel_r16_ctx128k_counters.txt"), *_STEP_SRC),
    "build4": (os.path.join(PROFILES, "build_page_kernel_bulk_r4_counters.txt"), *_BUILD_SRC),
    "build8": (os.path.join(PROFILES, "build_page_kernel_bulk_r8_counters.txt"), *_BUILD_SRC),
    "build16": (os.path.join(PROFILES, "build_page_kernel_bulk_r16_counters.txt"), *_BUILD_SRC),
}


def slot_payload(r):
    """Summary bytes of one (page, KV head): int4 basis, int8 coefficients and
    centroid, 25 fp16 scales at r = 8."""
    return r * D // 2 + B * r + D + 2 * (r + B + 1)


SLOT_PAYLOAD = slot_payload(R)


def build_flops_per_page(r, sweeps=6):
    """Algorithmic fp64 flops of one page summary (the count behind the bulk
    build's ALU roofline): Gram K K^T (2 B^2 d), centring (B d), a cyclic
    Jacobi of `sweeps` sweeps of B (B - 1) / 2 rotations, each updating two
    rows and two columns of the B x B matrix and two columns of U (3 flops
    per updated entry, 18 B) plus ~20 for its parameters, the basis D^T U_r
    (2 B d r) and its scaling (d r), and the quantisation (3 flops per code)."""
    rot = 18 * B + 20
    return (2 * B * B * D + B * D + sweeps * (B * (B - 1) // 2) * rot + 2 * B * D * r + D * r
            + 3 * (D * r + B * r + D))


def kernel_fingerprint(which):
    """sha256 over what decides a kernel's machine code: its source, the
    headers it includes and its compile flags."""
    from kv_cache_page_amd import build_lib
    _, src, hdrs = KERNELS[which]
    h = hashlib.sha256()
    for f in [src] + hdrs:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    # include paths relative to the repository, so the hash does not depend
    # on where the checkout sits
    flags = [os.path.relpath(f, ROOT) if os.path.isabs(f) else f
             for f in build_lib.FLAGS + build_lib.FILE_FLAGS.get(src, [])]
    h.update(" ".join(flags).encode())
    return h.hexdigest()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def head_bytes(seq_len, budget=BUDGET):
    """(summary bytes, selected-KV bytes) of one (layer, KV head) at seq_len."""
    F = seq_len // B
    P = (seq_len + B - 1) // B
    tail = seq_len - B * (P - 1)
    k = min(max(budget, 2), P)
    return F * SLOT_PAYLOAD, (k - 1) * PAGE_KV_BYTES + tail * (PAGE_KV_BYTES // B)


def step_bytes(seq_len):
    s, kv = head_bytes(seq_len)
    return LAYERS * H * (s + kv)


def traffic_from_counters(which):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary, or None when absent or taken on a different build of the kernel."""
    path = KERNELS[which][0]
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sha256") != kernel_fingerprint(which):
        return None
    try:
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def roofline(kernel, which, bytes_per_launch, us_per_launch):
    achieved = bytes_per_launch / (us_per_launch * 1e-6) / 1e9
    traffic = traffic_from_counters(which) if which else None
    return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "bytes_per_launch": round(bytes_per_launch), "us_per_launch": round(us_per_launch, 3)}


def host_cores():
    """Threads for CPU work: the cores this process may run on, at most 16
    (the host share of one GPU on the MI355X boxes)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

def capture(torch, fn, keys):
    graphs = {}
    for t in keys:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(t)
        graphs[t] = g
    torch.cuda.synchronize()
    return graphs


def timed(torch, graphs, keys):
    """ms for replaying graphs[k] for k in keys, between two events on the
    current stream (the stream the captured launches replay on)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for t in keys:
        graphs[t].replay()
    b.record()
    b.synchronize()
    return a.elapsed_time(b)


# ---------------------------------------------------------------------------
# 128K context, 32 layers (headline)
# ---------------------------------------------------------------------------

def run_ctx128k(torch, L, synth, dev, W, K, seed):
    n_steps = W + K
    len0 = MAX_LEN - n_steps            # tokens before the first decode step
    lens = [len0 + t + 1 for t in range(n_steps)]
    log(f"[bench] ctx128k: generating {LAYERS} layers x {MAX_LEN} tokens of KV on the GPU")
    t0 = time.time()
    stack = synth.make_layer_stack(LAYERS, MAX_LEN, H, G, n_steps, seed,
                                   needle_pages=len0 // B, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] generated in {time.time() - t0:.1f} s")
    MP = stack.block_table.shape[1]
    NB = stack.k_pools[0].shape[0]
    dims = L.Dims(H, G, R)
    table = stack.block_table

    # ---- prefill -> decode boundary: bulk build of every full page, all layers
    # (summaries, like the pools, are slices of one allocation)
    summ_all = L.alloc_summaries(dims, LAYERS * NB, dev)
    summ = [summ_all[l * NB:(l + 1) * NB] for l in range(LAYERS)]
    F0 = len0 // B
    ids0 = table[0, :F0].contiguous()
    for l in range(LAYERS):
        L.build(dims, stack.k_pools[l], ids0, summ[l])
    torch.cuda.synchronize()

    # ---- per-step inputs: lengths, appended tokens (the cache already holds
    # them; each step writes its token again), queries
    lens_dev = torch.tensor(lens, dtype=torch.int32, device=dev)
    budgets = torch.tensor([BUDGET], dtype=torch.int32, device=dev)
    kn = torch.empty(n_steps, LAYERS, 1, H, D, dtype=torch.bfloat16, device=dev)
    vn = torch.empty_like(kn)
    for t, Lt in enumerate(lens):
        blk, slot = int(table[0, (Lt - 1) // B]), (Lt - 1) % B
        for l in range(LAYERS):
            kn[t, l, 0] = stack.k_pools[l][blk, :, slot]
            vn[t, l, 0] = stack.v_pools[l][blk, :, slot]
    lens_host = [torch.tensor([Lt], dtype=torch.int32) for Lt in lens]
    scores = torch.empty(1, H, MP, G, dtype=torch.float32, device=dev)
    out = torch.empty(LAYERS, 1, H * G, D, dtype=torch.float32, device=dev)
    lse = torch.empty(LAYERS, 1, H * G, dtype=torch.float32, device=dev)
    ws = L.alloc_workspace(dims, 1, MP, BUDGET, dev)
    # block ids (in the whole allocation) of the page each step's token
    # completes, one per layer; empty when the token completes none
    ids_done = [torch.tensor([int(table[0, Lt // B - 1]) + l * NB for l in range(LAYERS)],
                             dtype=torch.int32, device=dev) if Lt % B == 0 else None for Lt in lens]

    def full_step(t):
        # one decode step of every layer: append, score, select, attend; then
        # the page the token completes (1 step in 16), every layer at once
        ln = lens_dev[t:t + 1]
        for l in range(LAYERS):
            L.decode_step(dims, stack.q[t, l], kn[t, l], vn[t, l], stack.k_pools[l],
                          stack.v_pools[l], summ[l], table, ln, budgets, BUDGET, out[l], ws,
                          lse_out=lse[l], seq_lens_host=lens_host[t], defer_build=True)
        if ids_done[t] is not None:
            L.build(dims, stack.k_all, ids_done[t], summ_all)

    def in_step_build(t):
        # the same step with the page build inside locks_decode_step
        ln = lens_dev[t:t + 1]
        for l in range(LAYERS):
            L.decode_step(dims, stack.q[t, l], kn[t, l], vn[t, l], stack.k_pools[l],
                          stack.v_pools[l], summ[l], table, ln, budgets, BUDGET, out[l], ws,
                          lse_out=lse[l], seq_lens_host=lens_host[t])

    def score_only(t):
        for l in range(LAYERS):
            L.score_pages(dims, stack.q[t, l], summ[l], table, lens_dev[t:t + 1], scores)

    full_step(0)            # eager warm-up of every kernel before capture
    first_comp = next(t for t in range(n_steps) if lens[t] % B == 0)
    in_step_build(first_comp)
    full_step(first_comp)
    torch.cuda.synchronize()
    log(f"[bench] capturing {n_steps} step graphs ({LAYERS} layers each)")
    g_full = capture(torch, full_step, range(n_steps))
    g_score = capture(torch, score_only, range(W, n_steps))

    log(f"[bench] warm-up {W} steps, then {K} timed steps")
    for t in range(W):
        g_full[t].replay()
    torch.cuda.synchronize()
    full_ms = timed(torch, g_full, range(W, n_steps))
    # the final step's outputs, for the check against the oracle
    final = dict(out=out[0, 0].cpu().numpy(), lse=lse[0, 0].cpu().numpy(),
                 any_nan=bool(torch.isnan(out).any() or torch.isnan(lse).any()))
    # steps whose token completes no page launch the decode-step kernel alone,
    # once per layer: their time per launch is that kernel's duration
    plain = [t for t in range(n_steps) if lens[t] % B != 0]
    completing = [t for t in range(n_steps) if lens[t] % B == 0]
    step_ms = timed(torch, g_full, plain)
    comp_ms = timed(torch, g_full, completing) if completing else float("nan")
    score_ms = timed(torch, g_score, range(W, n_steps))
    # the page-completing steps with the build inside the step (same results
    # up to the one page's term in the shares)
    comp_in = [t for t in completing if t >= W]
    g_in = capture(torch, in_step_build, comp_in)
    comp_in_ms = timed(torch, g_in, comp_in) if comp_in else float("nan")
    comp_in_us = comp_in_ms * 1e3 / len(comp_in) if comp_in else float("nan")
    del g_in
    timed_bytes = sum(step_bytes(lens[t]) for t in range(W, n_steps))
    ms_step = full_ms / K
    value = timed_bytes / (full_ms / 1e3) / 1e9
    steady_us = step_ms * 1e3 / len(plain)
    comp_us = comp_ms * 1e3 / len(completing) if completing else float("nan")
    amort_us = (15 * steady_us + comp_us) / 16
    log(f"[bench] decode step {ms_step * 1e3:.1f} us over the timed window ({value:.0f} GB/s); "
        f"steady {steady_us:.1f} us, page-completing {comp_us:.1f} us (build inside the step "
        f"{comp_in_us:.1f} us), 1 in 16 {amort_us:.1f} us")

    step_launches = len(plain) * LAYERS
    step_us = step_ms * 1e3 / step_launches
    step_bpl = sum(step_bytes(lens[t]) for t in plain) / step_launches
    score_launches = K * LAYERS
    score_us = score_ms * 1e3 / score_launches
    score_bpl = sum(LAYERS * (lens[t] // B) * H * SLOT_PAYLOAD for t in range(W, n_steps)) / score_launches
    res = dict(
        value=value, ms_step=ms_step, timed_bytes=timed_bytes,
        steady_us=steady_us, comp_us=comp_us, amort_us=amort_us, comp_in_us=comp_in_us,
        amort_in_us=(15 * steady_us + comp_in_us) / 16,
        page_build_us_per_layer=(comp_in_us - steady_us) / LAYERS if completing else None,
        roofline=roofline("decode_step_kernel<8,4,16> (locks_decode_step: score + select + attend)",
                          "step", step_bpl, step_us),
        score_stage=roofline("score_mfma_kernel<8,4,1> (locks_score_pages)", "score", score_bpl,
                             score_us),
        final=final, stack=stack, lens_final=lens[-1])
    log(f"[bench] decode-step kernel {step_us:.2f} us per launch, "
        f"{res['roofline']['achieved']:.0f} GB/s ({res['roofline']['frac']:.1%} of {HBM_PEAK_GBS:.0f}); "
        f"score kernel {score_us:.2f} us per launch ({res['score_stage']['frac']:.1%})")
    del g_full, g_score, summ, summ_all, ws, kn, vn
    return res


# ---------------------------------------------------------------------------
# 32K context, one layer, rotating replicas
# ---------------------------------------------------------------------------

def run_ctx32k(torch, L, synth, dev, replicas=32, reps=20):
    """One layer at 32K context: the step appends token 32769 (the first of a
    new page) and scores the 2048 full pages; 4 needles per KV head, k = 64.
    The graph steps `replicas` independent caches in turn."""
    ln = 32768 + 1
    k = 64
    dims = L.Dims(H, G, R)
    log(f"[bench] ctx32k: {replicas} replicas of a 32K-token layer")
    reps_state = []
    for i in range(replicas):
        b = synth.make_decode_batch([ln], H, G, [k], seed=1000 + i, needles_per_head=4, device=dev)
        summ = L.alloc_summaries(dims, b.num_blocks, dev)
        L.build(dims, b.k_pool, b.block_table[0, :ln // B].contiguous(), summ)
        blk, t = int(b.block_table[0, (ln - 1) // B]), (ln - 1) % B
        kn = b.k_pool[blk, :, t].clone()[None]
        vn = b.v_pool[blk, :, t].clone()[None]
        reps_state.append((b, summ, kn, vn))
    MP = reps_state[0][0].max_pages
    ws = L.alloc_workspace(dims, 1, MP, k, dev)
    out = torch.empty(1, H * G, D, device=dev)
    host = torch.tensor([ln], dtype=torch.int32)

    def rotate(_):
        for (b, summ, kn, vn) in reps_state:
            L.decode_step(dims, b.q, kn, vn, b.k_pool, b.v_pool, summ, b.block_table, b.seq_lens,
                          b.budgets, k, out, ws, seq_lens_host=host)

    rotate(0)
    torch.cuda.synchronize()
    g = capture(torch, rotate, [0])
    g[0].replay()
    ms = timed(torch, {i: g[0] for i in range(reps)}, range(reps))
    us = ms * 1e3 / (reps * replicas)
    s, kv = head_bytes(ln, k)
    bpl = H * (s + kv)
    nan = bool(torch.isnan(out).any())
    del reps_state, ws, g
    log(f"[bench] ctx32k decode step {us:.2f} us per launch ({bpl / us / 1e3:.0f} GB/s)")
    return {"workload": "1 seq, 32768 cached tokens + the new one, 1 layer, 8 KV heads x 4 q heads, "
                        f"k=64; {replicas} replicas stepped in turn",
            "us_per_step": round(us, 3), "bytes_per_step": bpl,
            "roofline": roofline("decode_step_kernel<8,4,8> (locks_decode_step)", "step32k", bpl, us),
            "any_nan": nan}


# ---------------------------------------------------------------------------
# rank sweep of the decode step at 128K context
# ---------------------------------------------------------------------------

def run_rank_sweep(torch, L, synth, dev, ranks=(4, 8, 16), replicas=8, reps=20):
    """One 128K-token layer (8191 full pages + 1 token, k = 128) through the
    fused decode step at each rank: the summaries of every rank built from the
    same keys, `replicas` copies of them stepped in turn (8 x 30..100 MB, so
    every launch streams its summaries from HBM; the K/V pool is shared)."""
    ln = 131072 - B + 1
    k = BUDGET
    log(f"[bench] rank sweep: 128K-token layer, r in {ranks}, {replicas} summary replicas each")
    b = synth.make_decode_batch([ln], H, G, [k], seed=1100, device=dev)
    blk, t = int(b.block_table[0, (ln - 1) // B]), (ln - 1) % B
    kn = b.k_pool[blk, :, t].clone()[None]
    vn = b.v_pool[blk, :, t].clone()[None]
    full = b.block_table[0, :ln // B].contiguous()
    out = torch.empty(1, H * G, D, device=dev)
    host = torch.tensor([ln], dtype=torch.int32)
    res = {}
    for r in ranks:
        dims = L.Dims(H, G, r)
        summs = []
        for _ in range(replicas):
            summ = L.alloc_summaries(dims, b.num_blocks, dev)
            L.build(dims, b.k_pool, full, summ)
            summs.append(summ)
        ws = L.alloc_workspace(dims, 1, b.max_pages, k, dev)

        def rotate(_):
            for summ in summs:
                L.decode_step(dims, b.q, kn, vn, b.k_pool, b.v_pool, summ, b.block_table,
                              b.seq_lens, b.budgets, k, out, ws, seq_lens_host=host)

        rotate(0)
        torch.cuda.synchronize()
        g = capture(torch, rotate, [0])
        g[0].replay()
        ms = timed(torch, {i: g[0] for i in range(reps)}, range(reps))
        us = ms * 1e3 / (reps * replicas)
        F = ln // B
        kv = (k - 1) * PAGE_KV_BYTES + (ln - B * (F)) * (PAGE_KV_BYTES // B)
        bpl = H * (F * slot_payload(r) + kv)
        res[f"r{r}"] = {"us_per_step": round(us, 3), "bytes_per_step": bpl,
                        "summary_bytes_per_page": slot_payload(r),
                        "roofline": roofline(f"decode_step_kernel<{r},4,16> (locks_decode_step)",
                                             "step" if r == R else f"step_r{r}", bpl, us),
                        "any_nan": bool(torch.isnan(out).any())}
        log(f"[bench] rank sweep r={r}: decode step {us:.2f} us per launch ({bpl / us / 1e3:.0f} GB/s)")
        del summs, ws, g
        torch.cuda.empty_cache()
    del b
    res["workload"] = ("1 seq, 131056 cached tokens + the new one (8191 full pages), 1 layer, 8 KV heads "
                       f"x 4 q heads, k=128; summaries at each rank, {replicas} replicas stepped in turn")
    return res


# ---------------------------------------------------------------------------
# batch of 32 ragged sequences, one layer
# ---------------------------------------------------------------------------

def run_batch32(torch, L, synth, dev, reps=20, seed=3):
    """32 sequences of 8K..128K cached tokens (page multiples, as the batched
    workload draws them) in one shuffled block pool; the step appends each
    sequence's next token (the first of a new page). k_s = max(8,
    ceil(P_s / 16)) with P_s the cached pages."""
    gc = torch.Generator(device="cpu")
    gc.manual_seed(seed + 104729)
    ctx = (torch.randint(8192 // 16, 131072 // 16 + 1, (32,), generator=gc) * 16).tolist()
    budgets = [max(8, math.ceil((c // B) / 16)) for c in ctx]
    lens = [c + 1 for c in ctx]
    log("[bench] batch32: generating 32 sequences of 8K..128K tokens")
    b = synth.make_decode_batch(lens, H, G, budgets, seed, needles_per_head=2, device=dev)
    dims = L.Dims(H, G, R)
    S = len(lens)
    summ = L.alloc_summaries(dims, b.num_blocks, dev)
    full = torch.cat([b.block_table[s, :lens[s] // B] for s in range(S)]).contiguous()
    L.build(dims, b.k_pool, full, summ)
    kn = torch.empty(S, H, D, dtype=torch.bfloat16, device=dev)
    vn = torch.empty_like(kn)
    for s in range(S):
        blk, t = int(b.block_table[s, (lens[s] - 1) // B]), (lens[s] - 1) % B
        kn[s], vn[s] = b.k_pool[blk, :, t], b.v_pool[blk, :, t]
    kmax = max(budgets)
    ws = L.alloc_workspace(dims, S, b.max_pages, kmax, dev)
    out = torch.empty(S, H * G, D, device=dev)
    host = b.seq_lens.cpu()

    def step(_):
        L.decode_step(dims, b.q, kn, vn, b.k_pool, b.v_pool, summ, b.block_table, b.seq_lens,
                      b.budgets, kmax, out, ws, seq_lens_host=host)

    step(0)
    torch.cuda.synchronize()
    g = capture(torch, step, [0])
    g[0].replay()
    ms = timed(torch, {i: g[0] for i in range(reps)}, range(reps))
    us = ms * 1e3 / reps
    bpl = sum(H * sum(head_bytes(ln, kb)) for ln, kb in zip(lens, budgets))
    nan = bool(torch.isnan(out).any())
    log(f"[bench] batch32 decode step {us:.2f} us per launch ({bpl / us / 1e3:.0f} GB/s, "
        f"{bpl / 1e9:.3f} GB)")
    del b, summ, ws, g, kn, vn, full
    return {"workload": "32 seqs of 8K..128K cached tokens (+ the new one), 1 layer, shuffled shared "
                        "block pool, 8 KV heads x 4 q heads, k = max(8, ceil(P/16))",
            "us_per_step": round(us, 3), "bytes_per_step": bpl,
            "roofline": roofline("decode_step_kernel<8,4,16> (locks_decode_step)", "stepb32", bpl, us),
            "any_nan": nan}


# ---------------------------------------------------------------------------
# offload: K/V pools in pinned host memory, summaries in HBM
# ---------------------------------------------------------------------------

def run_offload(torch, L, synth, dev, layers=4, reps=10, seed=5):
    """The 128K-context decode step of `layers` layers (independent caches of
    131072 tokens; the new token starts a page; k = 128) with each layer's K
    and V pools in pinned, device-mapped host memory: the score and the
    selection read the summaries in HBM, the attention reads the selected
    pages across the host link. Also timed: the same caches in HBM, and a
    DMA copy of one layer's K pool from pinned host memory (the link's
    practical read rate)."""
    ln = MAX_LEN + 1
    dims = L.Dims(H, G, R)
    log(f"[bench] offload: {layers} layers of a 128K-token cache in pinned host memory")
    state = []
    for i in range(layers):
        b = synth.make_decode_batch([ln], H, G, [BUDGET], seed=seed * 100 + i, needles_per_head=1,
                                    device=dev)
        summ = L.alloc_summaries(dims, b.num_blocks, dev)
        L.build(dims, b.k_pool, b.block_table[0, :ln // B].contiguous(), summ)
        blk, t = int(b.block_table[0, (ln - 1) // B]), (ln - 1) % B
        kn = b.k_pool[blk, :, t].clone()[None]
        vn = b.v_pool[blk, :, t].clone()[None]
        hk = L.HostPool(b.k_pool.shape)
        hv = L.HostPool(b.v_pool.shape)
        hk.host.copy_(b.k_pool.cpu())
        hv.host.copy_(b.v_pool.cpu())
        state.append((b, summ, kn, vn, hk, hv))
    torch.cuda.synchronize()
    MP = state[0][0].max_pages
    ws = L.alloc_workspace(dims, 1, MP, BUDGET, dev)
    outs = {m: torch.empty(layers, 1, H * G, D, device=dev) for m in ("host", "hbm")}
    host_len = torch.tensor([ln], dtype=torch.int32)

    def step(mode):
        for i, (b, summ, kn, vn, hk, hv) in enumerate(state):
            kp, vp = (hk, hv) if mode == "host" else (b.k_pool, b.v_pool)
            L.decode_step(dims, b.q, kn, vn, kp, vp, summ, b.block_table, b.seq_lens, b.budgets,
                          BUDGET, outs[mode][i], ws, seq_lens_host=host_len)

    for m in ("host", "hbm"):
        step(m)
    torch.cuda.synchronize()
    same = bool(torch.equal(outs["host"], outs["hbm"]))
    graphs = capture(torch, step, ["host", "hbm"])
    us = {}
    for m in ("host", "hbm"):
        graphs[m].replay()
        ms = timed(torch, {i: graphs[m] for i in range(reps)}, range(reps))
        us[m] = ms * 1e3 / (reps * layers)
    s_bytes, kv_bytes = head_bytes(ln, BUDGET)
    link_bytes = H * kv_bytes + H * 2 * D * 2          # selected pages read, new token written
    # DMA read rate of pinned host memory (one layer's K pool, 268 MB)
    src = torch.empty(state[0][0].k_pool.shape, dtype=torch.bfloat16, pin_memory=True)
    dst = torch.empty(src.shape, dtype=torch.bfloat16, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    e.record()
    e.synchronize()
    dma_gbs = 3 * src.numel() * 2 / (a.elapsed_time(e) * 1e-3) / 1e9
    achieved = link_bytes / (us["host"] * 1e-6) / 1e9
    nan = bool(torch.isnan(outs["host"]).any())
    log(f"[bench] offload decode step {us['host']:.1f} us per layer ({achieved:.1f} GB/s over the "
        f"host link; DMA copy {dma_gbs:.1f} GB/s), HBM pools {us['hbm']:.1f} us; identical "
        f"outputs: {same}")
    for (b, summ, kn, vn, hk, hv) in state:
        hk.free()
        hv.free()
    del state, ws, graphs, src, dst
    return {"workload": f"1 seq, 131072 cached tokens + the new one, {layers} layers (independent "
                        "caches) stepped in turn, 8 KV heads x 4 q heads, k=128; K/V pools in "
                        "pinned host memory, summaries in HBM",
            "us_per_layer_step": round(us["host"], 2), "us_per_layer_step_hbm_pools": round(us["hbm"], 2),
            "link_bytes_per_layer_step": link_bytes, "hbm_summary_bytes_per_layer_step": H * s_bytes,
            "host_resident_kv_bytes_per_layer": 2 * state_bytes(ln),
            "roofline": {"kernel": "decode_step_kernel<8,4,16> (locks_decode_step, host pools)",
                         "bound": "host link", "achieved": round(achieved, 2),
                         "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HOST_LINK_PEAK_GBS, 4), "traffic": None,
                         "dma_copy_gbs": round(dma_gbs, 2)},
            "identical_to_hbm_pools": same, "any_nan": nan or not same}


def state_bytes(ln):
    """bf16 bytes of one pool (K or V) of one layer holding ln tokens' pages."""
    return ((ln + B - 1) // B) * H * B * D * 2


# ---------------------------------------------------------------------------
# bulk build at the prefill -> decode boundary, r = 4, 8, 16
# ---------------------------------------------------------------------------

def run_bulk_build(torch, L, dev, stack):
    """locks_build over every page of the 32-layer, 131072-token cache
    (2,097,152 pages of 16 x 128 bf16 keys) at each rank."""
    NB = stack.k_pools[0].shape[0]
    ids = stack.block_table[0].contiguous()
    pages = LAYERS * ids.numel() * H
    out = {}
    for r in (4, 8, 16):
        dims = L.Dims(H, G, r)
        summ = L.alloc_summaries(dims, NB, dev)
        L.build(dims, stack.k_pools[0], ids, summ)          # warm
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for l in range(LAYERS):
            L.build(dims, stack.k_pools[l], ids, summ)
        b.record()
        b.synchronize()
        ms = a.elapsed_time(b)
        pps = pages / (ms / 1e3)
        flops = build_flops_per_page(r)
        achieved = pps * flops / 1e12
        traffic = traffic_from_counters(f"build{r}")
        out[f"r{r}"] = {
            "pages": pages, "ms": round(ms, 3), "pages_per_s": round(pps),
            "summary_bytes_per_page": slot_payload(r),
            "summary_frac_of_page_kv": round(slot_payload(r) / PAGE_KV_BYTES, 4),
            "roofline": {"kernel": f"build_page_kernel<{r}> (locks_build)", "bound": "alu",
                         "achieved": round(achieved, 3), "peak": FP64_VALU_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / FP64_VALU_PEAK_TFLOPS, 4),
                         "traffic": None if traffic is None else round(traffic),
                         "flops_per_page": flops, "us_per_launch": round(ms * 1e3 / LAYERS, 2),
                         "pages_per_launch": ids.numel() * H}}
        log(f"[bench] bulk build r={r}: {pps / 1e6:.2f} M pages/s, {achieved:.2f} TFLOP/s fp64 "
            f"({achieved / FP64_VALU_PEAK_TFLOPS:.1%}), {slot_payload(r)} B per page")
        del summ
    return out


# ---------------------------------------------------------------------------
# oracle: check of the final step and the CPU baseline
# ---------------------------------------------------------------------------

def oracle_layer0(stack, lens_final, torch):
    """Oracle inputs of layer 0 at the final step: per KV head the logical
    pages (fp64), the queries and the oracle-built slots of the full pages
    (built over a pool of threads; not timed)."""
    import numpy as np
    from oracle import locks_oracle as O
    P = (lens_final + B - 1) // B
    F = lens_final // B
    blocks = stack.block_table[0, :P].long()
    kp = stack.k_pools[0][blocks].cpu()
    vp = stack.v_pools[0][blocks].cpu()
    q = stack.q[-1, 0, 0].cpu()
    heads = []
    for h in range(H):
        heads.append(dict(K=kp[:, h].double().numpy(), V=vp[:, h].double().numpy(),
                          q=q[h * G:(h + 1) * G].double().numpy()))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(H, host_cores())) as ex:
        slots = list(ex.map(lambda hd: O.build_slots(hd["K"][:F], R)[0], heads))
    for hd, s in zip(heads, slots):
        hd["slots"] = s
    return heads, np


def check_final_step(final, heads, lens_final):
    """GPU layer-0 outputs of the final step against the oracle (fp64, its own
    slots, the deferred-build reading the loop runs): attention within 1e-2
    relative L2 per KV head, log-sum-exp within 1e-3, no NaN anywhere.
    Returns (ok, worst rel-L2, worst lse error)."""
    import numpy as np
    from oracle import locks_oracle as O
    if final["any_nan"]:
        return False, float("nan"), float("nan")
    worst, worst_l = 0.0, 0.0
    for h, hd in enumerate(heads):
        ora = O.decode_head(hd["q"], hd["K"], hd["V"], lens_final, BUDGET, slots=hd["slots"], r=R,
                            deferred=True)
        o = final["out"][h * G:(h + 1) * G]
        e = float(np.linalg.norm(o - ora["out"]) / np.linalg.norm(ora["out"]))
        el = float(np.abs(final["lse"][h * G:(h + 1) * G] - ora["lse"]).max())
        worst, worst_l = max(worst, e), max(worst_l, el)
    return worst <= 1e-2 and worst_l <= 1e-3, worst, worst_l


def cpu_baseline(heads, lens_final, seconds):
    """The fp64 oracle (score + share + select + attend per KV head) on layer 0
    of the final step, summaries prebuilt: once on one thread, once on every
    host core (one KV head per task, repeated until about `seconds` of
    wall time; numpy releases the interpreter lock in its array kernels)."""
    from oracle import locks_oracle as O
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # numpy then keeps its default thread count
        threadpool_limits = None
    s, kv = head_bytes(lens_final)
    per_head = s + kv

    def one(hd):
        O.decode_head(hd["q"], hd["K"], hd["V"], lens_final, BUDGET, slots=hd["slots"], r=R,
                      deferred=True)

    limit = threadpool_limits(1) if threadpool_limits else None
    try:
        # one thread: the 8 heads in turn, repeated to about seconds / 3
        t0, n1 = time.perf_counter(), 0
        while True:
            for hd in heads:
                one(hd)
                n1 += 1
            if time.perf_counter() - t0 >= seconds / 3:
                break
        t1 = time.perf_counter() - t0
        # every core: rounds of 2 x cores head tasks until about 2 seconds / 3
        cores = host_cores()
        ntasks = 0
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(max_workers=cores) as ex:
            while True:
                batch = [heads[(ntasks + i) % len(heads)] for i in range(2 * cores)]
                list(ex.map(one, batch))
                ntasks += len(batch)
                if time.perf_counter() - t0 >= seconds * 2 / 3:
                    break
        tn = time.perf_counter() - t0
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return dict(value=ntasks * per_head / tn / 1e9, unit="GB/s", cores=cores, kind="oracle",
                value_1thread=n1 * per_head / t1 / 1e9, cores_1thread=1,
                sample=f"layer 0 of the final 131072-token step, 8 KV heads (score + share + select + "
                       f"attend, fp64 numpy, summaries prebuilt, untimed): {ntasks} head tasks on "
                       f"{cores} threads in {tn:.1f} s; 1 thread: {n1} heads in {t1:.1f} s")


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=224)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle CPU-baseline budget (0 skips it; the final-step check still runs)")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--only", default="all",
                    help="comma list of ctx128k, ctx32k, batch32, build, offload, ranks (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed region, run one elementwise copy that reads 1 GiB "
                         "and writes 1 GiB (the reference for HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(see the sharding paragraph of DESIGN.md); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    W, K = args.warmup, args.steps
    if W < 0 or K < 1 or W + K < 2 or W + K > 256:
        print("need 0 <= warmup, 1 <= steps, 2 <= warmup + steps <= 256 decode steps",
              file=sys.stderr)
        sys.exit(2)
    only = (set(args.only.split(",")) if args.only != "all"
            else {"ctx128k", "ctx32k", "batch32", "build", "offload", "ranks"})

    import torch
    import synth
    from kv_cache_page_amd import locks as L

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    workloads = {}
    head = None
    if "ctx128k" in only or "build" in only:
        head = run_ctx128k(torch, L, synth, dev, W, K, args.seed)
    if "build" in only:
        workloads["bulk_build"] = run_bulk_build(torch, L, dev, head["stack"])
    if "ctx32k" in only:
        workloads["ctx32k_1layer"] = run_ctx32k(torch, L, synth, dev)
        torch.cuda.empty_cache()
    if "batch32" in only:
        workloads["batch32_ragged"] = run_batch32(torch, L, synth, dev)
        torch.cuda.empty_cache()
    if "ranks" in only:
        workloads["rank_sweep_ctx128k"] = run_rank_sweep(torch, L, synth, dev)
        torch.cuda.empty_cache()
    if "offload" in only:
        workloads["offload_ctx128k"] = run_offload(torch, L, synth, dev)
        torch.cuda.empty_cache()

    if args.calibrate_copy:
        x = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        torch.neg(x, out=y)   # one dispatch: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del x, y
        log("[bench] calibration copy done (1 GiB read + 1 GiB write)")

    ok = not any(w.get("any_nan") for w in workloads.values() if isinstance(w, dict))
    cpu, check = None, None
    if head is not None:
        log("[bench] oracle: layer-0 slots of the final step (not timed)")
        heads, _ = oracle_layer0(head["stack"], head["lens_final"], torch)
        good, rel, lerr = check_final_step(head["final"], heads, head["lens_final"])
        check = {"layer0_final_step_vs_oracle": "ok" if good else "MISMATCH",
                 "worst_attn_rel_l2": rel, "worst_lse_abs_err": lerr}
        log(f"[bench] final step, layer 0 vs oracle: {check}")
        ok = ok and good
        if args.cpu_seconds > 0:
            log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
            cpu = cpu_baseline(heads, head["lens_final"], args.cpu_seconds)
            log(f"[bench] oracle {cpu['value']:.3f} GB/s on {cpu['cores']} threads, "
                f"{cpu['value_1thread']:.3f} GB/s on 1")

    res = {
        "metric": METRIC,
        "value": None if head is None else round(head["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": None if head is None else round(head["ms_step"], 5),
        "us_per_step": None if head is None else round(head["ms_step"] * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": "bf16 K/V and queries; int4/int8 summaries with fp16 scales; scores on "
                        "fp16 matrix-core operands, attention on bf16 matrix-core operands (bf16 "
                        "probabilities in PV), fp32 accumulation and softmax; page build in fp64",
        "data": "synthetic",
        "config": {
            "workload": "ctx128k_32layer_decode: 1 seq, 131072 tokens at the last step, "
                        "32 layers, 8 KV heads x 4 q heads, d=128, B=16, r=8, k=128 pages",
            "seq_len": MAX_LEN, "layers": LAYERS, "kv_heads": H, "group": G, "head_dim": D,
            "page_size": B, "rank": R, "budget_pages": BUDGET, "parallelism": "none (1 GPU)",
        },
    }
    if head is not None:
        res.update({
            "bytes_per_step": round(head["timed_bytes"] / K),
            "hbm_frac": round(head["value"] / HBM_PEAK_GBS, 4),
            "us_per_step_steady": round(head["steady_us"], 2),
            "us_per_step_page_completing": round(head["comp_us"], 2),
            "us_per_step_amortised_1_in_16": round(head["amort_us"], 2),
            "us_per_step_page_completing_build_in_step": round(head["comp_in_us"], 2),
            "us_per_step_amortised_1_in_16_build_in_step": round(head["amort_in_us"], 2),
            "page_build_us_per_layer": None if head["page_build_us_per_layer"] is None
            else round(head["page_build_us_per_layer"], 2),
            "roofline": head["roofline"],
            "score_stage": head["score_stage"],
        })
    res["workloads"] = workloads
    res["check"] = check
    res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)
    if not ok:
        log("[bench] FAILED: an output is NaN or the final step does not match the oracle")
        sys.exit(1)


if __name__ == "__main__":
    main()
