#!/usr/bin/env python3
"""Decode-step benchmark of the LOCKS hot path on one MI355X.

Workload (synthetic, Llama-3.1-8B-shaped): one sequence at 128K context,
32 layers, 8 KV heads x 4 query heads, d = 128, bf16 K/V, pages of 16 tokens,
rank-8 int4/int8 page summaries, a budget of 128 pages per KV head. The KV
cache holds 131072 tokens' worth of pages; the sequence starts W+K tokens
short of 131072 and every decode step appends one token, so the last timed
step runs at exactly 131072 tokens.

One step = for every layer: append the new token's K/V, build the summary of
the page that just filled (when one did), score every full page from the
summaries, select sink + recent + top-126 pages, and attend over them, all
through locks_decode_step (one launch per layer, two on the steps whose
token completes a page). Each step is captured once as a HIP graph; W
warm-up steps run, then K steps are timed between HIP events.

Throughput counts the metric's algorithmic bytes: 818 summary bytes per full
page and KV head, plus 8192 bytes per selected full page (512 per valid token
of the last page) and KV head, per layer.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LAYERS, H, G, D, B, R, BUDGET, MAX_LEN = 32, 8, 4, 128, 16, 8, 128, 131072
SLOT_PAYLOAD = 818
PAGE_KV_BYTES = 2 * B * D * 2
HBM_PEAK_GBS = 8000.0
METRIC = "decode-step µs and achieved HBM GB/s (summary+selected KV) at 128K ctx, 8 KV heads"
CSRC = os.path.join(ROOT, "kv_cache_page_amd", "csrc")
# (counter summary, source, headers) of the two kernels bench.py reports on:
# the decode-step kernel (score + selection + attention in one launch) and the
# stand-alone page-score kernel
KERNELS = {
    "step": (os.path.join(ROOT, "profiles", "decode_step_kernel_ctx128k_counters.txt"),
             "locks_decode.hip",
             ["locks_score_tile.h", "locks_attn_core.h", "locks_select.h", "locks_step.h",
              "locks_device.h"]),
    "score": (os.path.join(ROOT, "profiles", "score_kernel_ctx128k_counters.txt"),
              "locks_score_mfma.hip", ["locks_score_tile.h", "locks_device.h"]),
}


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


def cpu_baseline(stack, lens_final, seconds):
    """The fp64 oracle, single-threaded, on layer 0 of the final step: summaries
    built by the oracle (untimed), then score + share + select + attend per KV
    head, timed until `seconds` of work or all heads are done."""
    import numpy as np
    from oracle import locks_oracle as O
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # numpy then keeps its default thread count
        threadpool_limits = None
    P = (lens_final + B - 1) // B
    F = lens_final // B
    blocks = stack.block_table[0, :P].long().cpu()
    kp = stack.k_pools[0][blocks.to(stack.k_pools[0].device)].cpu()
    vp = stack.v_pools[0][blocks.to(stack.v_pools[0].device)].cpu()
    q = stack.q[-1, 0, 0].cpu()
    done_bytes, elapsed, heads = 0, 0.0, 0
    for h in range(H):
        keys = kp[:, h].double().numpy()
        slots, _, _ = O.build_slots(keys[:F], R)
        qq = q[h * G:(h + 1) * G].double().numpy()
        vals = vp[:, h].double().numpy()
        if threadpool_limits is not None:
            with threadpool_limits(1):
                t0 = time.perf_counter()
                O.decode_head(qq, keys, vals, lens_final, BUDGET, slots=slots, r=R)
                dt = time.perf_counter() - t0
        else:
            t0 = time.perf_counter()
            O.decode_head(qq, keys, vals, lens_final, BUDGET, slots=slots, r=R)
            dt = time.perf_counter() - t0
        elapsed += dt
        s, kv = head_bytes(lens_final)
        done_bytes += s + kv
        heads += 1
        if elapsed >= seconds:
            break
    return dict(value=done_bytes / elapsed / 1e9, unit="GB/s", cores=1, kind="oracle",
                sample=f"layer 0 of the final 131072-token step, {heads} of {H} KV heads "
                       f"(score+share+select+attend, fp64 numpy, 1 thread), {elapsed:.1f} s; "
                       f"summaries built beforehand, untimed")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=224)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle CPU-baseline budget (0 skips it)")
    ap.add_argument("--seed", type=int, default=2)
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

    import torch
    import synth
    from kv_cache_page_amd import locks as L

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    n_steps = W + K
    len0 = MAX_LEN - n_steps            # tokens before the first decode step
    lens = [len0 + t + 1 for t in range(n_steps)]
    log(f"[bench] generating {LAYERS} layers x {MAX_LEN} tokens of KV on the GPU")
    t0 = time.time()
    stack = synth.make_layer_stack(LAYERS, MAX_LEN, H, G, n_steps, args.seed,
                                   needle_pages=len0 // B, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] generated in {time.time() - t0:.1f} s")
    MP = stack.block_table.shape[1]
    NB = stack.k_pools[0].shape[0]
    dims = L.Dims(H, G, R)
    table = stack.block_table

    # ---- prefill -> decode boundary: bulk build of every full page, all layers
    summ = [L.alloc_summaries(dims, NB, dev) for _ in range(LAYERS)]
    F0 = len0 // B
    ids0 = table[0, :F0].contiguous()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    L.build(dims, stack.k_pools[0], ids0, summ[0])          # warm the build kernel
    torch.cuda.synchronize()
    e0.record()
    for l in range(LAYERS):
        L.build(dims, stack.k_pools[l], ids0, summ[l])
    e1.record()
    e1.synchronize()
    build_ms = e0.elapsed_time(e1)
    build_pages = LAYERS * F0 * H
    log(f"[bench] bulk build of {build_pages} pages: {build_ms:.1f} ms "
        f"({build_pages / build_ms / 1e3:.2f} M pages/s)")

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
    out = torch.empty(1, H * G, D, dtype=torch.float32, device=dev)
    lse = torch.empty(1, H * G, dtype=torch.float32, device=dev)
    ws = L.alloc_workspace(dims, 1, MP, BUDGET, dev)

    def full_step(t):
        # one decode step of every layer: append, build of the page the token
        # completes (1 step in 16), score, select, attend
        ln = lens_dev[t:t + 1]
        for l in range(LAYERS):
            L.decode_step(dims, stack.q[t, l], kn[t, l], vn[t, l], stack.k_pools[l],
                          stack.v_pools[l], summ[l], table, ln, budgets, BUDGET, out, ws,
                          lse_out=lse, seq_lens_host=lens_host[t])

    def score_only(t):
        for l in range(LAYERS):
            L.score_pages(dims, stack.q[t, l], summ[l], table, lens_dev[t:t + 1], scores)

    # eager warm-up of every kernel before capture
    full_step(0)
    torch.cuda.synchronize()

    def capture(fn, steps):
        graphs = {}
        for t in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(t)
            graphs[t] = g
        torch.cuda.synchronize()
        return graphs

    def timed(graphs, steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for t in steps:
            graphs[t].replay()
        b.record()
        b.synchronize()
        return a.elapsed_time(b)

    log(f"[bench] capturing {n_steps} step graphs ({LAYERS} layers each)")
    g_full = capture(full_step, range(n_steps))
    g_score = capture(score_only, range(W, n_steps))

    log(f"[bench] warm-up {W} steps, then {K} timed steps")
    for t in range(W):
        g_full[t].replay()
    torch.cuda.synchronize()
    full_ms = timed(g_full, range(W, n_steps))
    # the steps whose token completes no page launch the decode-step kernel
    # alone, once per layer: their time per launch is that kernel's duration
    plain = [t for t in range(n_steps) if lens[t] % B != 0]
    step_ms = timed(g_full, plain)
    score_ms = timed(g_score, range(W, n_steps))
    timed_bytes = sum(step_bytes(lens[t]) for t in range(W, n_steps))
    ms_step = full_ms / K
    value = timed_bytes / (full_ms / 1e3) / 1e9
    log(f"[bench] decode step {ms_step * 1e3:.1f} us ({value:.0f} GB/s)")

    # dominant kernel: the decode-step kernel (score + selection + attention),
    # the metric's bytes of one layer per launch
    step_launches = len(plain) * LAYERS
    step_us = step_ms * 1e3 / step_launches
    step_bytes_per_launch = sum(step_bytes(lens[t]) for t in plain) / step_launches
    achieved = step_bytes_per_launch / (step_us * 1e-6) / 1e9
    traffic = traffic_from_counters("step")
    log(f"[bench] decode-step kernel {step_us:.2f} us per launch, {achieved:.0f} GB/s "
        f"({achieved / HBM_PEAK_GBS:.1%} of {HBM_PEAK_GBS:.0f})")
    # the score stage alone (stand-alone score kernel): F x H slots of 818 bytes
    score_launches = K * LAYERS
    score_us = score_ms * 1e3 / score_launches
    score_bytes = sum(LAYERS * (lens[t] // B) * H * SLOT_PAYLOAD for t in range(W, n_steps))
    score_bytes_per_launch = score_bytes / score_launches
    score_achieved = score_bytes_per_launch / (score_us * 1e-6) / 1e9
    score_traffic = traffic_from_counters("score")
    log(f"[bench] score kernel {score_us:.2f} us per launch, {score_achieved:.0f} GB/s "
        f"({score_achieved / HBM_PEAK_GBS:.1%} of {HBM_PEAK_GBS:.0f})")

    if args.calibrate_copy:
        x = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        torch.neg(x, out=y)   # one dispatch: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del x, y
        log("[bench] calibration copy done (1 GiB read + 1 GiB write)")

    cpu = None
    if args.cpu_seconds > 0:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(stack, lens[-1], args.cpu_seconds)
        log(f"[bench] oracle {cpu['value']:.3f} GB/s")

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "ctx128k_32layer_decode: 1 seq, 131072 tokens at the last step, "
                        "32 layers, 8 KV heads x 4 q heads, d=128, B=16, r=8, k=128 pages",
            "seq_len": MAX_LEN, "layers": LAYERS, "kv_heads": H, "group": G, "head_dim": D,
            "page_size": B, "rank": R, "budget_pages": BUDGET, "parallelism": "none (1 GPU)",
        },
        "bytes_per_step": round(timed_bytes / K),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "bulk_build_pages_per_s": round(build_pages / (build_ms / 1e3)),
        "roofline": {
            "kernel": "decode_step_kernel<8,4,16> (locks_decode_step: score + select + attend)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "bytes_per_launch": round(step_bytes_per_launch),
            "us_per_launch": round(step_us, 3),
        },
        "score_stage": {
            "kernel": "score_mfma_kernel<8,4,1> (locks_score_pages)",
            "bound": "hbm",
            "achieved": round(score_achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(score_achieved / HBM_PEAK_GBS, 4),
            "traffic": None if score_traffic is None else round(score_traffic),
            "bytes_per_launch": round(score_bytes_per_launch),
            "us_per_launch": round(score_us, 3),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
