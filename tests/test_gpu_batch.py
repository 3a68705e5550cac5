"""Batched blocks (dflash_block_batch): several handles that share one set of
weights (dflash_create_context), each with its own context, drafted in one
pass. Every sequence's logits and selection are compared with the oracle's
block over that sequence's own context, and with dflash_block on the same
handle; batches of 1 to 8 sequences cover both padded row-block counts (4
and 8), contexts of different lengths, windows and starts, an empty
context, and anchors inside the context."""
import numpy as np
import pytest
import torch

import block_drafter_settle_amd as pkg
from block_drafter_settle_amd import synth
from oracle.context import Context

from test_gpu_parity import check_selection, close, run_block

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _outs(g, nseq, k, width):
    dev = _dev()
    top = g["selector_top"]
    return dict(logits=torch.full((nseq, k, width), float("nan"), device=dev),
                cand=torch.full((nseq, k, top), -1, dtype=torch.int32, device=dev),
                unary=torch.full((nseq, k, top), float("nan"), device=dev),
                score=torch.full((nseq, k, top), float("nan"), device=dev),
                chosen=torch.full((nseq, k), -1, dtype=torch.int32, device=dev))


def _batch(ds, anchors, a, k, width, g):
    o = _outs(g, len(ds), k, width)
    pkg.block_batch(ds, anchors, a, k, width, *(o[n].data_ptr() for n in
                                                ("logits", "cand", "unary", "score", "chosen")))
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in o.items()}


# (geometry overrides, [(first, length, anchor offset from the end)] per sequence, k, width)
CASES = [
    (dict(windows=[0, 6], no_rope=[1]), [(0, 50, 0), (100, 17, 0), (7, 120, -30)], 7, 1000),
    (dict(windows=[0, 0], no_rope=[], block=16), [(0, 64, 0), (3, 0, 0), (10, 90, 0),
                                                  (0, 33, -5), (50, 200, 0)], 15, 1000),
    (dict(windows=[5, 0], no_rope=[0], heads=8, kv_heads=2, head_dim=128),
     [(0, 40 + 13 * i, 0) for i in range(8)], 7, 999),
    (dict(windows=[0, 0], no_rope=[]), [(5, 70, 0)], 3, 8),
]


@pytest.mark.parametrize("case", CASES)
def test_batch_matches_oracle_per_sequence(orc, case):
    over, seqs, k, width = case
    g = synth.small_geometry(**over)
    w = synth.make_weights(g, seed=41)
    stream = torch.cuda.current_stream(_dev()).cuda_stream
    lead = pkg.Drafter(g, w, max_context=400, stream=stream)
    ds = [lead] + [pkg.Drafter.context_of(lead, 400, stream) for _ in seqs[1:]]
    m = orc.Model(g, w)
    try:
        anchors, pos, ctxs = [], [], []
        for i, (first, length, da) in enumerate(seqs):
            ctx = Context(m)
            if length:
                taps = synth.make_taps(g, length, seed=50 + i)
                ds[i].settle(first, length, taps.to(_dev()).data_ptr())
                ctx.push(first, taps.numpy())
            ctxs.append(ctx)
            anchors.append((37 * i + 11) % g["vocab"])
            pos.append(first + length + da)
        got = _batch(ds, anchors, pos, k, width, g)
        for i, ctx in enumerate(ctxs):
            tag = f"batch of {len(seqs)} {over} seq {i}"
            ref = ctx.block(anchors[i], pos[i], k, width)
            close(got["logits"][i], ref["logits"], tag + " logits")
            sel = m.select(ref["logits"], ref["hp"], anchors[i])
            check_selection({n: got[n][i] for n in ("cand", "score", "chosen")}, ref["logits"],
                            sel, tag)
            # the same block alone on the same handle
            one = run_block(ds[i], g, anchors[i], pos[i], k, width)
            close(got["logits"][i], one["logits"], tag + " vs dflash_block logits")
    finally:
        for d in ds[::-1]:
            d.close()


def test_batch_27b_two_sequences(orc):
    """The 27B-shaped sidecar: two sequences with 600- and 300-row contexts."""
    g = synth.geometry("t27b")
    dev = _dev()
    w = synth.make_weights(g, seed=0, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    lead = pkg.Drafter(g, w, max_context=1024, stream=stream)
    other = pkg.Drafter.context_of(lead, 1024, stream)
    ds = [lead, other]
    try:
        m = orc.Model(g, w)
        del w
        ctxs, pos = [], []
        for i, (first, n) in enumerate([(1000, 600), (20, 300)]):
            taps = synth.make_taps(g, n, seed=60 + i, device=dev)
            ds[i].settle(first, n, taps.data_ptr())
            ctx = Context(m)
            ctx.push(first, taps.cpu().numpy())
            ctxs.append(ctx)
            pos.append(first + n)
        anchors = [int(x) for x in synth.uniform_tokens(g, 2, seed=61)]
        k, width = 15, g["vocab"]
        got = _batch(ds, anchors, pos, k, width, g)
        for i, ctx in enumerate(ctxs):
            print(f"t27b batch: oracle block of sequence {i}", flush=True)
            ref = ctx.block(anchors[i], pos[i], k, width)
            close(got["logits"][i], ref["logits"], f"t27b batch seq {i} logits")
            sel = m.select(ref["logits"], ref["hp"], anchors[i])
            check_selection({n: got[n][i] for n in ("cand", "score", "chosen")}, ref["logits"],
                            sel, f"t27b batch seq {i}")
    finally:
        other.close()
        lead.close()


def test_batch_27b_eight_sequences(orc):
    """The 27B-shaped sidecar at eight sequences (8 row blocks, the products
    split up to 16 ways): contexts of 40 to 320 rows at different starts;
    three sequences against the oracle, all eight against dflash_block on the
    same handle."""
    g = synth.geometry("t27b")
    dev = _dev()
    w = synth.make_weights(g, seed=0, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    lead = pkg.Drafter(g, w, max_context=512, stream=stream)
    ds = [lead] + [pkg.Drafter.context_of(lead, 512, stream) for _ in range(7)]
    try:
        m = orc.Model(g, w)
        del w
        spans = [(13 * i, 40 * (i + 1)) for i in range(8)]
        taps_host, pos = [], []
        for i, (first, n) in enumerate(spans):
            taps = synth.make_taps(g, n, seed=80 + i, device=dev)
            ds[i].settle(first, n, taps.data_ptr())
            taps_host.append(taps.cpu().numpy())
            pos.append(first + n)
        anchors = [int(x) for x in synth.uniform_tokens(g, 8, seed=81)]
        k, width = 15, g["vocab"]
        got = _batch(ds, anchors, pos, k, width, g)
        again = _batch(ds, anchors, pos, k, width, g)  # the same pass twice: the same bits
        for n in got:
            assert np.array_equal(got[n], again[n]), n
        for i in range(8):
            one = run_block(ds[i], g, anchors[i], pos[i], k, width)
            close(got["logits"][i], one["logits"], f"t27b batch of 8, seq {i} against its own block")
        for i in (0, 3, 7):
            print(f"t27b batch of 8: oracle block of sequence {i}", flush=True)
            ctx = Context(m)
            ctx.push(spans[i][0], taps_host[i])
            ref = ctx.block(anchors[i], pos[i], k, width)
            close(got["logits"][i], ref["logits"], f"t27b batch of 8, seq {i} logits")
            sel = m.select(ref["logits"], ref["hp"], anchors[i])
            check_selection({n: got[n][i] for n in ("cand", "score", "chosen")}, ref["logits"],
                            sel, f"t27b batch of 8, seq {i}")
    finally:
        for d in ds[1:]:
            d.close()
        lead.close()


def test_batch_rejections():
    g = synth.small_geometry()
    w = synth.make_weights(g, seed=42)
    stream = torch.cuda.current_stream(_dev()).cuda_stream
    a = pkg.Drafter(g, w, max_context=64, stream=stream)
    b = pkg.Drafter(g, w, max_context=64, stream=stream)  # same values, its own weights
    c = pkg.Drafter.context_of(a, 64, stream)
    try:
        taps = synth.make_taps(g, 10, seed=1).to(_dev())
        for d in (a, b, c):
            d.settle(0, 10, taps.data_ptr())
        with pytest.raises(pkg.DflashError) as e:      # does not share the lead's weights
            _batch([a, b], [1, 2], [10, 10], 3, 100, g)
        assert e.value.code == pkg.DFLASH_EINVAL
        c.queue(10, 2, taps.data_ptr())                # rows wait on c
        with pytest.raises(pkg.DflashError) as e:
            _batch([a, c], [1, 2], [10, 10], 3, 100, g)
        assert e.value.code == pkg.DFLASH_EINVAL
        c.flush()
        with pytest.raises(pkg.DflashError) as e:      # nine sequences
            _batch([a] + [c] * 8, [1] * 9, [10] * 9, 3, 100, g)
        assert e.value.code == pkg.DFLASH_EINVAL
        got = _batch([a, c, c], [1, 2, 2], [12, 12, 12], 3, 100, g)  # a handle twice: fine
        assert np.array_equal(got["cand"][1], got["cand"][2])
    finally:
        c.close()
        b.close()
        a.close()
