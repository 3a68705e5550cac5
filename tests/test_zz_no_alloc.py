"""dflash_block_noalloc (the block pass on the library's static scratch)
against dflash_block on the same handle: bit-identical outputs on two calls
in a row, the second smaller, after a larger sidecar has left its contents in
the shared array; and the rejections of a NULL logits buffer and of a
geometry whose scratch exceeds the array."""
import numpy as np
import pytest
import torch

import block_drafter_settle_amd as pkg
from block_drafter_settle_amd import synth

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _outs(g, k, width):
    dev = _dev()
    top = g["selector_top"]
    return dict(logits=torch.full((k, width), float("nan"), device=dev),
                cand=torch.full((k, top), -1, dtype=torch.int32, device=dev),
                unary=torch.full((k, top), float("nan"), device=dev),
                score=torch.full((k, top), float("nan"), device=dev),
                chosen=torch.full((k,), -1, dtype=torch.int32, device=dev))


def _call(d, g, fn, anchor, a, k, width):
    o = _outs(g, k, width)
    fn(anchor, a, k, width, *(o[n].data_ptr() for n in ("logits", "cand", "unary", "score",
                                                          "chosen")))
    d.sync()
    return {n: t.cpu().numpy() for n, t in o.items()}


def _same(x, y, what):
    for n in x:
        assert np.array_equal(x[n], y[n]), (what, n)


def _drafter(g, seed, ctx):
    w = synth.make_weights(g, seed=seed, device=_dev())
    d = pkg.Drafter(g, w, max_context=ctx + 16, stream=torch.cuda.current_stream(_dev()).cuda_stream)
    taps = synth.make_taps(g, ctx, seed=seed, device=_dev())
    d.settle(0, ctx, taps.data_ptr())
    return d


def test_noalloc_matches_block_full_size():
    """The 27B-shaped sidecar (the scratch the static array is sized for)."""
    g = synth.geometry("t27b")
    d = _drafter(g, 0, 2500)
    try:
        for anchor, a, k, width in ((11, 2500, 15, g["vocab"]), (99, 2100, 9, 70000)):
            ref = _call(d, g, d.block, anchor, a, k, width)
            got = _call(d, g, d.block_noalloc, anchor, a, k, width)
            _same(got, ref, f"t27b a={a} k={k} width={width}")
    finally:
        d.close()


def test_noalloc_matches_block_two_calls_smaller_second():
    """Block 8 (rows past the block in the 16-row operands are stale array
    contents from the run above), then a smaller second call."""
    g = synth.small_geometry(windows=[0, 6], no_rope=[1], vocab=3000, mask_token=2999)
    d = _drafter(g, 3, 400)
    try:
        for anchor, a, k, width in ((17, 400, 7, 3000), (5, 120, 3, 700)):
            ref = _call(d, g, d.block, anchor, a, k, width)
            got = _call(d, g, d.block_noalloc, anchor, a, k, width)
            _same(got, ref, f"small a={a} k={k} width={width}")
    finally:
        d.close()


def test_noalloc_rejections():
    g = synth.small_geometry()
    d = _drafter(g, 4, 50)
    try:
        o = _outs(g, 3, 500)
        with pytest.raises(pkg.DflashError) as e:
            d.block_noalloc(1, 50, 3, 500, None, o["cand"].data_ptr(), o["unary"].data_ptr(),
                            o["score"].data_ptr(), o["chosen"].data_ptr())
        assert e.value.code == pkg.DFLASH_EINVAL
    finally:
        d.close()
    # attention states of 64 heads of 256 dims alone exceed the array
    g = synth.small_geometry(heads=64, kv_heads=8, head_dim=256, vocab=600, mask_token=599)
    d = _drafter(g, 5, 20)
    try:
        o = _outs(g, 3, 500)
        with pytest.raises(pkg.DflashError) as e:
            d.block_noalloc(1, 20, 3, 500, o["logits"].data_ptr(), o["cand"].data_ptr(),
                            o["unary"].data_ptr(), o["score"].data_ptr(), o["chosen"].data_ptr())
        assert e.value.code == pkg.DFLASH_EINVAL and "scratch" in str(e.value)
    finally:
        d.close()
