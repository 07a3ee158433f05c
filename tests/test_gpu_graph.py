"""One streaming step captured in a HIP graph and replayed.

The library launches only on the stream it is given and issues no memset,
allocation or synchronisation, so a whole step (append, top-k mask
generation, attention) can be captured.  The graph holds the launch
arguments of the captured step, so every replay repeats that step; each
replay, with eager work and synchronisations in between, must give the eager
result bit for bit.
"""
import numpy as np
import pytest
import torch

from synth import Workload, draw_step_tensors
from tests.gpu_util import to_dev
from windowed_attention_amd import KVCache, uf

pytestmark = pytest.mark.gpu

CACHES = {
    "bf16": {},
    "fp8": dict(kv_dtype=uf.UF_FP8_E4M3, q_scale=0.02, k_scale=0.015, v_scale=0.02),
    "block-order": dict(block_grid=(10, 20)),
}


@pytest.mark.parametrize("kind", list(CACHES))
def test_captured_step_replays_bit_exact(kind):
    # anchor of one step (2 frames of 10x20 tokens), window of 4 frames, GQA 2
    cfg = Workload(50, "g-capture", "bf16", 4, 2, 128, (10, 20), 2, 4, 2, 5, None)
    F = cfg.frames_per_step
    cache = KVCache(cfg.n_kv_heads, cfg.head_dim, cfg.tokens_per_frame, cfg.window_frames, cfg.anchor_frames,
                    **CACHES[kind])
    steps = [draw_step_tensors(cfg, s) for s in range(cfg.steps)]
    dev = [(to_dev(q), to_dev(k), to_dev(v)) for q, k, v in steps]
    last = cfg.steps - 1

    # eager reference: stream every step; the last step with a generated top-k mask
    for s in range(last):
        cache.append(dev[s][1], dev[s][2], F)
    q, k, v = dev[last]
    cache.append(k, v, F)
    mask_e = cache.block_mask_topk(q, top_k=2, local_blocks=1)
    out_e = torch.empty_like(q)
    cache.attn_step(q, out_e, mask_e)
    torch.cuda.synchronize()

    # same state before the last append (storage already holds the frames), then capture
    cache.reset()
    for s in range(last):
        cache.append(None, None, F, flags=2)  # UF_APPEND_COMMIT_ONLY: bookkeeping only
    mask_g = torch.empty_like(mask_e)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda:0")
    out_g = torch.zeros_like(q)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            cache.append(k, v, F)
            cache.block_mask_topk(q, 2, 1, mask=mask_g, workspace=ws)
            cache.attn_step(q, out_g, mask_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for r in range(3):
        out_g.fill_(0)
        mask_g.fill_(7)
        torch.cuda.synchronize()
        print(f"replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(mask_g, mask_e), f"replay {r}: mask differs"
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"replay {r}: output differs"
        _ = (torch.ones(1000, device="cuda:0") * r).sum().item()  # eager work between replays
    cache.close()


@pytest.mark.parametrize("entry,pipeline", [("attn_step", 0), ("attn_step_static", 0), ("attn_step", 2)])
def test_captured_split_step_merges_on_every_replay(entry, pipeline):
    """A step whose key range is split (attention parts, then the combine kernel) captured as
    the cache's first step, replayed with eager split steps in between, through the workspace
    and through the static scratch, and with the head_dim 128 kernel's software-pipelined loop.  Every replay and every eager step must equal the eager
    result of a twin cache bit for bit."""
    cfg = Workload(51, "g-split", "bf16", 8, 2, 128, (12, 25), 1, 3, 0, 4, None)
    F = cfg.frames_per_step
    mk = lambda: KVCache(cfg.n_kv_heads, cfg.head_dim, cfg.tokens_per_frame, cfg.window_frames, 0, splits=3,
                         pipeline=pipeline)
    cache, twin = mk(), mk()
    dev = [tuple(to_dev(x) for x in draw_step_tensors(cfg, s)) for s in range(cfg.steps)]
    for s in range(cfg.steps):
        for c in (cache, twin):
            c.append(dev[s][1], dev[s][2], F)
    q = dev[-1][0]
    out_e = torch.empty_like(q)
    twin.attn_step(q, out_e)
    torch.cuda.synchronize()
    call = getattr(cache, entry)

    out_g = torch.zeros_like(q)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            call(q, out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        out_g.fill_(0)
        torch.cuda.synchronize()
        print(f"{entry}: replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"replay {r}: output differs"
        out_x = torch.full_like(q, 5.0)
        call(q, out_x)   # eager split steps between the replays
        torch.cuda.synchronize()
        assert torch.equal(out_x.view(torch.int16), out_e.view(torch.int16)), f"eager step after replay {r} differs"
    cache.close()
    twin.close()
