"""The block pass as one submission: dflash_block_noalloc captured into a HIP
graph on the handle's stream and replayed. Each replay runs after eager work
on the same handle and the same static scratch (blocks at other anchors),
its output buffers refilled with NaN and -1 first, and must reproduce the
eager call bit for bit."""
import numpy as np
import pytest
import torch

import block_drafter_settle_amd as pkg
from block_drafter_settle_amd import synth

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


@pytest.mark.parametrize("name", ["small", "t27b"])
def test_block_graph_replays_match_eager(name):
    dev = _dev()
    if name == "small":
        g = synth.small_geometry(windows=[0, 6], no_rope=[1])
        ctx, k, width = 120, 7, 1000
    else:
        g = synth.geometry("t27b")
        ctx, k, width = 2500, 15, g["vocab"]
    s = torch.cuda.Stream(dev)
    w = synth.make_weights(g, seed=31, device=dev)
    d = pkg.Drafter(g, w, max_context=ctx + 64, stream=s.cuda_stream)
    del w
    top = g["selector_top"]
    with torch.cuda.stream(s):
        taps = synth.make_taps(g, ctx, seed=32, device=dev)
        bufs = dict(logits=torch.empty(k, width, device=dev),
                    cand=torch.empty(k, top, dtype=torch.int32, device=dev),
                    unary=torch.empty(k, top, device=dev), score=torch.empty(k, top, device=dev),
                    chosen=torch.empty(k, dtype=torch.int32, device=dev))
        other = {n: torch.empty_like(t) for n, t in bufs.items()}
    ptrs = [bufs[n].data_ptr() for n in ("logits", "cand", "unary", "score", "chosen")]
    optrs = [other[n].data_ptr() for n in ("logits", "cand", "unary", "score", "chosen")]
    try:
        d.settle(0, ctx, taps.data_ptr())
        anchor, a = 17, ctx
        d.block_noalloc(anchor, a, k, width, *ptrs)
        d.sync()
        ref = {n: t.cpu().numpy() for n, t in bufs.items()}
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=s, capture_error_mode="thread_local"):
            d.block_noalloc(anchor, a, k, width, *ptrs)
        for rep in range(3):
            # eager work between replays: blocks at other anchors through both
            # entry points (the captured call's parameters, the context range
            # of each layer included, are fixed at capture: the context itself
            # must not change between replays)
            d.block_noalloc(5 + rep, a - 3, k, width, *optrs)
            d.block(9 + rep, a, k, width, *optrs)
            # the refill and the replay on the handle's stream, ordered after
            # the eager calls (a replay runs on torch's current stream)
            with torch.cuda.stream(s):
                for n, t in bufs.items():
                    t.fill_(-1 if t.dtype == torch.int32 else float("nan"))
                gr.replay()
            s.synchronize()
            for n, t in bufs.items():
                assert np.array_equal(t.cpu().numpy(), ref[n]), (name, rep, n)
            print(f"{name}: replay {rep} bit-identical to the eager call", flush=True)
    finally:
        d.close()
