#!/usr/bin/env python3
"""Benchmark of the streaming attention path on one MI355X.

One step = one streaming step of the workload at steady state: append the
step's F new frames of K/V to the rolling cache (uf_kvcache_append) and run
chunk attention of the step's queries over the visible window, with the
step's seeded 128x128 block mask (uf_attn_step).  Inputs (q, k, v, masks)
are resident in HBM before the timed region starts.

Prints one JSON line.  `value` is executed attention TFLOP/s over the whole
step (append included), timed over --steps steady steps (default 300, about
1 s of GPU work at the 2K chunk); `roofline` rates the attention kernel alone
from HIP events on the launch stream; `cpu_baseline` times the float64 oracle
on the host's cores (its affinity mask): a bounded sample of the same step,
and the tiny, 480P and decoder streams from their first step (each bounded).
`also` repeats the step measurement for the tiny, 1K, 480P, decoder and
FlashDecoder-XL workloads (at least --also-seconds of GPU time each, at most
20000 steps); `fp8`,
`block_order`, `mask_topk` and `mask_topk_gqa` are the FP8 cache, the (2,8,8)
block order and block-mask generation legs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import WORKLOADS, TILE, bf16_bits_to_f32, draw_step_tensors, make_block_mask  # noqa: E402

METRIC = "attention TFLOP/s (% bf16 MFMA peak) + frames/s at 1K and 2K chunk shapes"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CUs x 2.4 GHz x 4096 FLOP/clk/CU)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense FP8 MFMA (twice the bf16 rate)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_traffic.md")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_kernel_mfma_counters.md")
CSRC = os.path.join(ROOT, "windowed_attention_amd", "csrc")
# every source compiled into the bf16 attention kernel (its schedule lives in the headers)
KERNEL_SOURCES = ["uf_kernels.hip", "uf_attn_bf16.h", "uf_attn_d128.hip", "uf_attn_d64.hip", "uf_attn_walk.h",
                  "uf_device.h", "uf_internal.h"]


def kernel_sources_sha256():
    """sha256 over the bf16 attention kernel's sources, in KERNEL_SOURCES order (each file's
    name, a NUL, its bytes); the committed profiles record it."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(name.encode() + b"\0")
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _profile_text(path):
    """A committed profile summary, or None when it was taken on other kernel sources."""
    try:
        text = open(path).read()
        src = kernel_sources_sha256()
    except OSError:
        return None
    m = re.search(r"sources sha256 `([0-9a-f]{64})`", text)
    return text if m and m.group(1) == src else None


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary,
    or None when that summary was taken on different kernel sources."""
    text = _profile_text(TRAFFIC_FILE)
    t = text and re.search(r"traffic_bytes_per_launch\[%s\]: (\d+)" % re.escape(workload), text)
    return int(t.group(1)) if t else None


def profiled_clock(workload):
    """Clock (GHz) the chip held under the attention kernel in the committed MFMA counter
    summary (GRBM_GUI_ACTIVE per XCD over the dispatch time), or None when that summary was
    taken on different kernel sources."""
    text = _profile_text(COUNTERS_FILE)
    row = text and re.search(r"^\| %s \|(.*)$" % re.escape(workload), text, re.M)
    if not row:
        return None
    cells = [c.strip() for c in row.group(1).split("|")]
    return float(cells[6])  # dispatch, MFMA FLOPs, executed FLOPs, MFMA, VALU, exp, clock


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def executed_flops(n_q, n_k, n_q_heads, d, mask):
    """4*d per (query, key, head) score entry actually computed (kept tiles, valid rows/cols)."""
    if mask is None:
        return 4 * d * n_q * n_k * n_q_heads
    bm = mask != 0
    rows = np.minimum(TILE, n_q - TILE * np.arange(bm.shape[1]))
    cols = np.minimum(TILE, n_k - TILE * np.arange(bm.shape[2]))
    pairs = int((bm * rows[None, :, None] * cols[None, None, :]).sum())
    if bm.shape[0] == 1:
        pairs *= n_q_heads
    return 4 * d * pairs


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def steady_keys(cfg):
    """Visible keys once the window is full."""
    return (cfg.anchor_frames + cfg.window_frames) * cfg.tokens_per_frame


_POOLS = {}


def prepare(cfg, n_steps):
    """Device inputs of the stream's first n_steps steps (bf16 q/k/v), drawn once per workload
    and shared by every leg that runs it."""
    key = (cfg.name, n_steps)
    if key not in _POOLS:
        pool = []
        for s in range(n_steps):
            qb, kb, vb = draw_step_tensors(cfg, s)
            pool.append({"q": to_dev(qb), "k": to_dev(kb), "v": to_dev(vb), "mask": None, "mask_np": None})
        _POOLS.clear()  # one workload's inputs resident at a time
        _POOLS[key] = pool
    return _POOLS[key]


def attach_masks(cfg, pool, n_keys_per_step):
    import torch
    for s, item in enumerate(pool):
        if cfg.mask_pct is not None and item["mask_np"] is None:
            m = make_block_mask(cfg.index, s, cfg.n_q_heads, cfg.q_tokens, n_keys_per_step[s], cfg.mask_pct)
            item["mask_np"] = m
            item["mask"] = torch.from_numpy(m).to("cuda:0")


FP8_SCALES = (0.02, 0.015, 0.02)  # static q, k, v scales for N(0,1) draws (E4M3 range, no saturation)


def pool_size(cfg):
    """Steps drawn for a workload: the opening steps that fill the window plus two steady ones
    (the whole stream when it has at most 8 steps)."""
    fill = -(-(cfg.anchor_frames + cfg.window_frames) // cfg.frames_per_step)
    return fill, max(cfg.steps if cfg.steps <= 8 else fill + 2, fill + 1)


def run_workload(cfg, warmup, steps, fp8=False, block_order=False, min_seconds=0.0, cache_kw=None):
    """Stream the workload's opening steps, then time `steps` steady steps (more when
    min_seconds asks for a longer timed region: steps are then added until the estimated GPU
    time reaches it)."""
    import torch
    from windowed_attention_amd import KVCache, uf

    F, L = cfg.frames_per_step, cfg.tokens_per_frame
    fill, n_pool = pool_size(cfg)
    t0 = time.time()
    log(f"{cfg.name}: inputs of {n_pool} steps")
    pool = prepare(cfg, n_pool)
    kw = dict(cache_kw or {})
    if block_order:
        kw["block_grid"] = cfg.grid
    if fp8:
        q_s, k_s, v_s = FP8_SCALES
        kw.update(kv_dtype=uf.UF_FP8_E4M3, q_scale=q_s, k_scale=k_s, v_scale=v_s)
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, L, cfg.window_frames, cfg.anchor_frames,
                    max_q_heads=cfg.n_q_heads, max_q_tokens=cfg.q_tokens, **kw)
    # key counts per pool step follow the window bookkeeping of the library itself
    n_keys = []
    for s in range(n_pool):
        plan = cache.plan_append(F)
        n_keys.append(plan.window_after.n_keys)
        cache.append(None, None, F, flags=uf.UF_APPEND_COMMIT_ONLY)  # bookkeeping only, nothing copied
    cache.reset()
    attach_masks(cfg, pool, n_keys)
    prep_s = time.time() - t0
    log(f"{cfg.name}: inputs ready in {prep_s:.1f} s; warm-up")

    out = torch.empty_like(pool[0]["q"])
    steady = list(range(fill, n_pool)) or [n_pool - 1]

    def one_step(item, ev=None):
        if ev is not None:
            ev[0].record()
        cache.append(item["k"], item["v"], F)
        if ev is not None:
            ev[1].record()
        cache.attn_step(item["q"], out, item["mask"])
        if ev is not None:
            ev[2].record()

    # warm-up: the stream's opening steps (window filling), then steady steps
    for s in range(n_pool):
        one_step(pool[s])
    for i in range(max(0, warmup - n_pool)):
        one_step(pool[steady[i % len(steady)]])
    torch.cuda.synchronize()
    assert cache.window().n_keys == steady_keys(cfg)
    if min_seconds > 0:
        t = time.perf_counter()
        for i in range(10):
            one_step(pool[steady[i % len(steady)]])
        torch.cuda.synchronize()
        per_step = (time.perf_counter() - t) / 10
        steps = max(steps, min(20000, int(min_seconds / per_step) + 1))

    log(f"{cfg.name}: timing {steps} steps")
    seq = [steady[i % len(steady)] for i in range(steps)]
    flops = [executed_flops(cfg.q_tokens, steady_keys(cfg), cfg.n_q_heads, cfg.head_dim, pool[s]["mask_np"])
             for s in seq]
    # timed region: wall clock over exactly `steps` steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in seq:
        one_step(pool[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    # per-kernel durations from HIP events on the launch stream (separate pass, same steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in seq]
    torch.cuda.synchronize()
    for s, ev in zip(seq, evs):
        one_step(pool[s], ev)
    torch.cuda.synchronize()
    append_ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in evs]))
    attn_ms = float(np.mean([ev[1].elapsed_time(ev[2]) for ev in evs]))
    cache.close()

    total_flops = float(sum(flops))
    # K and V, each read (bf16) and written (bf16, or one byte per element for FP8)
    append_bytes = 2 * F * L * cfg.n_kv_heads * cfg.head_dim * (2 + (1 if fp8 else 2))
    return {
        "cfg": cfg,
        "steps": steps,
        "prep_s": prep_s,
        "ms_per_step": 1e3 * wall / steps,
        "tflops": total_flops / wall / 1e12,
        "frames_per_s": F * steps / wall,
        "attn_ms": attn_ms,
        "append_ms": append_ms,
        "attn_tflops": (total_flops / steps) / (attn_ms * 1e-3) / 1e12,
        "flops_per_step": total_flops / steps,
        "append_gbs": append_bytes / (append_ms * 1e-3) / 1e9,
        "append_bytes": append_bytes,
    }


def _topk_setup(cfg, cache_kw=None):
    """A cache at the workload's steady state, its step's queries, and the top_k that keeps the
    workload's mask density (less the local window of 2 + 2 tiles)."""
    from windowed_attention_amd import KVCache
    F = cfg.frames_per_step
    fill, n_pool = pool_size(cfg)
    pool = prepare(cfg, n_pool)
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames,
                    **(cache_kw or {}))
    for s in range(fill + 1):
        cache.append(pool[s]["k"], pool[s]["v"], F)
    return cache, pool[fill]["q"]


def run_topk(cfg, steps, local_blocks=1, pct=None, cache_kw=None):
    """Block-mask generation (uf_block_mask_topk) at the workload's steady state, then attention
    under the generated mask.  top_k = the mask density (the workload's, or pct) times the key
    tiles, less the local window (at least 0)."""
    import torch
    from windowed_attention_amd import uf

    cache, q = _topk_setup(cfg, cache_kw)
    n_k = cache.window().n_keys
    n_qb, n_kb = -(-cfg.q_tokens // TILE), -(-n_k // TILE)
    pct = pct or cfg.mask_pct or 100
    top_k = max(0, (pct * n_kb + 50) // 100 - (2 + 2 * local_blocks))
    mask = torch.empty((cfg.n_q_heads, n_qb, n_kb), dtype=torch.uint8, device="cuda:0")
    ws = torch.empty(uf.uf_block_mask_workspace_bytes(cache.desc, cfg.q_tokens, cfg.n_q_heads), dtype=torch.uint8,
                     device="cuda:0")
    out = torch.empty_like(q)
    for _ in range(3):
        cache.block_mask_topk(q, top_k, local_blocks, mask=mask, workspace=ws)
        cache.attn_step(q, out, mask)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        cache.block_mask_topk(q, top_k, local_blocks, mask=mask, workspace=ws)
        e[1].record()
        cache.attn_step(q, out, mask)
        e[2].record()
    torch.cuda.synchronize()
    gen_ms = [e[0].elapsed_time(e[1]) for e in ev]
    attn_ms = [e[1].elapsed_time(e[2]) for e in ev]
    cache.close()
    m = mask.cpu().numpy()
    flops = executed_flops(cfg.q_tokens, n_k, cfg.n_q_heads, cfg.head_dim, m)
    # algorithmic bytes: q and the visible K read once, the mask written once
    nbytes = 2 * cfg.head_dim * (cfg.q_tokens * cfg.n_q_heads + n_k * cfg.n_kv_heads) + m.size
    g = float(np.mean(gen_ms))
    a = float(np.mean(attn_ms))
    return {
        "top_k": top_k,
        "local_blocks": local_blocks,
        "kept_tiles_per_row": float(m.sum() / (m.shape[0] * m.shape[1])),
        "mask_gen_ms": round(g, 4),
        "mask_gen_gbs": round(nbytes / (g * 1e-3) / 1e9, 1),
        "mask_gen_frac_hbm": round(nbytes / (g * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "mask_gen_bytes": nbytes,
        "attn_ms": round(a, 4),
        "attn_tflops": round(flops / (a * 1e-3) / 1e12, 2),
        "pct_peak_attn": round(100 * flops / (a * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "pct_of_attn": round(100 * g / a, 2),
    }


def host_cores():
    """CPUs this process may run on (its affinity mask)."""
    return len(os.sched_getaffinity(0))


def _oracle_tiles(q, kk, vv, mask, tiles, n_q, cores):
    """The unchanged oracle on whole query tiles, one call per tile on `cores` threads with one
    BLAS thread each (numpy's matrix products and exponentials release the GIL)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    def one(t):
        rows = np.arange(t * TILE, min((t + 1) * TILE, n_q))
        return oracle.attend(q, kk, vv, mask, rows=rows)

    with threadpool_limits(1), ThreadPoolExecutor(cores) as ex:
        return list(ex.map(one, tiles))


def cpu_baseline(cfg, pool_step, budget_s=15.0):
    """The float64 oracle on a bounded sample of one steady step: whole query tiles, all heads,
    `cores` tiles at a time, until the budget is spent."""
    import oracle

    cores = host_cores()
    F, L, W, A = cfg.frames_per_step, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames
    win = oracle.FrameListWindow(L, W, A)
    for s in range(pool_step + 1):
        _, kb, vb = draw_step_tensors(cfg, s)
        win.append(bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), F)
    qb, _, _ = draw_step_tensors(cfg, pool_step)
    q = bf16_bits_to_f32(qb)
    kk, vv = win.keys_values()
    n_k = kk.shape[0]
    mask = None
    if cfg.mask_pct is not None:
        mask = make_block_mask(cfg.index, pool_step, cfg.n_q_heads, cfg.q_tokens, n_k, cfg.mask_pct)
    n_qt = -(-cfg.q_tokens // TILE)

    def tile_flops(t):
        return executed_flops(min(TILE, cfg.q_tokens - t * TILE), n_k, cfg.n_q_heads, cfg.head_dim,
                              None if mask is None else mask[:, t:t + 1, :])

    log(f"cpu baseline: oracle on {cfg.name} step {pool_step}, {cores} threads")
    _oracle_tiles(q, kk, vv, mask, [0], cfg.q_tokens, 1)   # warm-up: first query tile, not counted
    t_total, done_flops, tiles = 0.0, 0, []
    t = 1 if n_qt > 1 else 0
    while t < n_qt and t_total < budget_s:
        chunk = list(range(t, min(t + 2 * cores, n_qt)))
        t0 = time.perf_counter()
        _oracle_tiles(q, kk, vv, mask, chunk, cfg.q_tokens, cores)
        t_total += time.perf_counter() - t0
        done_flops += sum(tile_flops(x) for x in chunk)
        tiles += chunk
        t = chunk[-1] + 1
    step_flops = executed_flops(cfg.q_tokens, n_k, cfg.n_q_heads, cfg.head_dim, mask)
    rate = done_flops / t_total
    return {
        "value": rate / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{cfg.name} step {pool_step}: query tiles {tiles[0]}..{tiles[-1]} of {n_qt}, all {cfg.n_q_heads} "
                  f"heads ({done_flops / 1e9:.1f} GFLOP in {t_total:.1f} s; float64 numpy, one oracle call per "
                  f"query tile on {cores} threads)",
        "s_per_step": step_flops / rate,
        "frames_per_s": F * rate / step_flops,
    }


def cpu_stream(cfg, budget_s=20.0):
    """The float64 oracle streaming the workload from its first step: window bookkeeping plus
    attention of every query tile of each step, steps in order until the stream ends or the
    budget is spent.  Input drawing is not timed."""
    import oracle

    cores = host_cores()
    F = cfg.frames_per_step
    win = oracle.FrameListWindow(cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames)
    n_qt = -(-cfg.q_tokens // TILE)
    t_total, flops, steps = 0.0, 0, 0
    log(f"cpu baseline: oracle streaming {cfg.name}")
    for s in range(cfg.steps):
        qb, kb, vb = draw_step_tensors(cfg, s)
        q, k, v = bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb)
        t0 = time.perf_counter()
        win.append(k, v, F)
        kk, vv = win.keys_values()
        mask = None
        if cfg.mask_pct is not None:
            mask = make_block_mask(cfg.index, s, cfg.n_q_heads, cfg.q_tokens, kk.shape[0], cfg.mask_pct)
        _oracle_tiles(q, kk, vv, mask, list(range(n_qt)), cfg.q_tokens, cores)
        t_total += time.perf_counter() - t0
        flops += executed_flops(cfg.q_tokens, kk.shape[0], cfg.n_q_heads, cfg.head_dim, mask)
        steps += 1
        if t_total >= budget_s:
            break
    return {
        "steps": steps,
        "of_steps": cfg.steps,
        "whole_stream": steps == cfg.steps,
        "seconds": round(t_total, 3),
        "s_per_step": round(t_total / steps, 4),
        "frames_per_s": round(F * steps / t_total, 3),
        "tflops": round(flops / t_total / 1e12, 4),
        "cores": cores,
    }


def summary(r, profiled=True):
    """The leg's figures; profiled=False for legs the committed bf16 profiles do not cover (FP8,
    block order)."""
    cfg = r["cfg"]
    traffic = measured_traffic(cfg.name) if profiled else None
    return {
        "workload": f"{cfg.name} chunk: {cfg.n_q_heads}x{cfg.head_dim} heads (KV {cfg.n_kv_heads}), "
                    f"{cfg.grid[0]}x{cfg.grid[1]} tokens/frame, {cfg.frames_per_step} frames/step, "
                    f"window {cfg.window_frames} frames + anchor {cfg.anchor_frames}, "
                    + (f"{cfg.mask_pct}% block mask" if cfg.mask_pct else "dense"),
        "q_tokens": cfg.q_tokens,
        "keys": steady_keys(cfg),
        "steps": r["steps"],
        "ms_per_step": r["ms_per_step"],
        "tflops": r["tflops"],
        "pct_peak_step": 100 * r["tflops"] / PEAK_BF16_TFLOPS,
        "attn_kernel_ms": r["attn_ms"],
        "attn_kernel_tflops": r["attn_tflops"],
        "pct_peak_attn_kernel": 100 * r["attn_tflops"] / PEAK_BF16_TFLOPS,
        "frames_per_s": r["frames_per_s"],
        "append_ms": r["append_ms"],
        "append_gbs": r["append_gbs"],
        "append_frac_hbm": r["append_gbs"] / PEAK_HBM_GBS,
        "gflop_per_step": r["flops_per_step"] / 1e9,
        # bf16 legs: HBM bytes per attention launch from the committed counter profile, over the
        # algorithmic bytes (None when the profile is of other kernel sources)
        "traffic_over_algorithmic": None if traffic is None else round(traffic / algorithmic_attn_bytes(cfg), 2),
        "profiled_clock_ghz": profiled_clock(cfg.name) if profiled else None,
    }


def algorithmic_attn_bytes(cfg):
    """Q and O once plus the visible K and V once (bf16)."""
    return 2 * cfg.head_dim * (2 * cfg.q_tokens * cfg.n_q_heads + 2 * steady_keys(cfg) * cfg.n_kv_heads)


DEFAULT_ALSO = "tiny,1k,480p,decoder,decoder-xl,refine-xl"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300, help="steps timed for the main workload")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="2k", choices=[c.name for c in WORKLOADS])
    ap.add_argument("--also", default=DEFAULT_ALSO,
                    help="comma-separated extra workloads reported under 'also' ('' = none)")
    ap.add_argument("--also-seconds", type=float, default=1.0,
                    help="least GPU time timed per extra workload (steps are added to reach it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-topk", action="store_true", help="skip the block-mask generation legs")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 (E4M3) cache leg")
    ap.add_argument("--no-block-order", action="store_true", help="skip the (2,8,8) block-order leg")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work on the main step")
    ap.add_argument("--cpu-stream-budget", type=float, default=20.0,
                    help="seconds of oracle work per streamed workload (tiny, 480p, decoder)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (3 times), a known-size kernel "
                         "against which profiler byte counters are scaled")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.init()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)  # reads and writes n * 4 bytes
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {args.copy_calibration_mib} MiB")
        del src, dst
    by_name = {c.name: c for c in WORKLOADS}
    cfg = by_name[args.workload]
    main_r = run_workload(cfg, args.warmup, args.steps)
    fp8 = None
    if not args.no_fp8 and cfg.head_dim in (64, 128):
        log(f"{cfg.name}: FP8 (E4M3) cache")
        r8 = run_workload(cfg, args.warmup, args.steps, fp8=True)
        fp8 = summary(r8, profiled=False)
        fp8["scales_q_k_v"] = list(FP8_SCALES)
        fp8["peak_fp8_tflops"] = PEAK_FP8_TFLOPS
        fp8["pct_peak_fp8_attn_kernel"] = 100 * r8["attn_tflops"] / PEAK_FP8_TFLOPS
    blk = None
    if not args.no_block_order:
        log(f"{cfg.name}: (2,8,8) block order")
        blk = summary(run_workload(cfg, args.warmup, args.steps, block_order=True), profiled=False)
    topk = None
    if not args.no_topk and cfg.mask_pct is not None:
        log(f"{cfg.name}: top-k block-mask generation")
        topk = run_topk(cfg, 50)
    also = {}
    for name in [n for n in args.also.split(",") if n and n != cfg.name]:
        also[name] = summary(run_workload(by_name[name], args.warmup, 20, min_seconds=args.also_seconds))
    gqa_topk = None
    if not args.no_topk and "decoder-xl" in by_name:
        # per-head top-k masks on the GQA-8 decoder shape: one query head per work-group against
        # four heads of a KV group sharing each staged tile (the union of their rows)
        xl = by_name["decoder-xl"]
        log("decoder-xl: top-k masks, heads per work-group 1 and 4")
        gqa_topk = {f"heads_per_wg_{h}": run_topk(xl, 50, pct=25, cache_kw={"heads_per_wg": h}) for h in (1, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        fill, _ = pool_size(cfg)
        cpu = cpu_baseline(cfg, fill, args.cpu_budget)
        cpu["streams"] = {n: cpu_stream(by_name[n], args.cpu_stream_budget) for n in ("tiny", "480p", "decoder")}
        # the other chunk shape of the metric: one steady step, bounded like the main one
        if cfg.name != "1k":
            c1k = by_name["1k"]
            cpu["other_steps"] = {"1k": cpu_baseline(c1k, pool_size(c1k)[0], args.cpu_budget)}

    s = summary(main_r)
    traffic_bytes = measured_traffic(cfg.name)
    traffic_gbs = None if traffic_bytes is None else round(traffic_bytes / (main_r["attn_ms"] * 1e-3) / 1e9, 1)
    clock = profiled_clock(cfg.name)
    algo_bytes = algorithmic_attn_bytes(cfg)
    line = {
        "metric": METRIC,
        "value": round(main_r["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": main_r["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(main_r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v rounded to bf16, seeded block masks)",
        "config": {"workload": s["workload"], "q_tokens": s["q_tokens"], "keys": s["keys"],
                   "gflop_per_step": round(s["gflop_per_step"], 2)},
        "pct_peak": round(100 * main_r["tflops"] / PEAK_BF16_TFLOPS, 2),
        "frames_per_s": round(main_r["frames_per_s"], 2),
        "append_gbs": round(main_r["append_gbs"], 1),
        "roofline": {
            "bound": "mfma",
            "kernel": f"attn_kernel<{cfg.head_dim}>",
            "achieved": round(main_r["attn_tflops"], 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(main_r["attn_tflops"] / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_gbs,
            "traffic_unit": "GB/s (rocprofv3 FETCH_SIZE + WRITE_SIZE bytes per launch / launch time)",
            "traffic_bytes_per_launch": traffic_bytes,
            "algorithmic_bytes_per_launch": algo_bytes,
            "traffic_over_algorithmic": None if traffic_bytes is None else round(traffic_bytes / algo_bytes, 2),
            "launch_ms": round(main_r["attn_ms"], 4),
            "kernel_sources_sha256": kernel_sources_sha256(),
            # the spec peak assumes 2.4 GHz; the counter profile gives the clock actually held
            "profiled_clock_ghz": clock,
            "frac_at_profiled_clock": None if clock is None else
            round(main_r["attn_tflops"] / (PEAK_BF16_TFLOPS * clock / 2.4), 4),
        },
        "cpu_baseline": cpu,
        "mask_topk": topk,
        "mask_topk_gqa": gqa_topk,
        "fp8": fp8,
        "block_order": blk,
        "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
